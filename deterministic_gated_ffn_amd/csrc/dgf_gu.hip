// Fused gate/up projection and activation for few tokens (gfx950).
//
// a[m][n] = rnd( silu(g) u ) with g = T_K(x[m,:] . W_gate[n,:]) and
// u = T_K(x[m,:] . W_up[n,:]), both rounded to the stored type (the stage boundaries of
// RL-Kernel PR #325, sections "Design" and "Operator test matrix").
//
// One workgroup of 8 waves owns whole output tiles of 16 columns and all K:
// the canonical midpoint tree over the L <= 64 leaves is cut at depth 3 into
// one subtree per wave (at most 8 leaves), the wave reduces its subtree with
// the fixed post-order in registers, and after a workgroup barrier the 8
// wave roots are joined with the balanced top three levels.  Gate and up of a
// tile are reduced by the same workgroup one after the other, so the
// activation is applied right there: no partial roots, no join kernel.
//
// The activation operand stays on chip for the whole kernel: the first NR
// leaves of a wave's subtree in registers, the rest in the wave's own LDS
// region (a wave reads only what it wrote, so no barrier guards it).  It is
// brought in during the first tile, a few leaves ahead of its first use, so
// that its loads run beside the weight stream rather than before it.  Weights
// stream through the wave as whole 128-byte row segments (8 rows per load
// instruction, buffer loads on a rebased descriptor) staged through a
// swizzled LDS slab into the MFMA layout; each weight byte is read from HBM
// once per 16-token tile.
#include "dgf_device.hpp"
#include "dgf_kernels.hpp"

namespace dgf {
namespace {

constexpr int kGuWaves = 8;
constexpr int kGuMaxNL = 8;  // leaves per wave (L <= 64)
constexpr int kGuCols = 16;  // output columns per tile
constexpr int kGuRing = 4;   // ring slots of weight units: PR - 1 units in flight per wave

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int MT>
constexpr int nr_of() {
  return MT == 1 ? kGuMaxNL : 5;  // activation leaves held in registers
}

template <int MT>
struct GuLds {
  // per wave: the LDS-resident activation fragments, then the weight slab
  static constexpr int XL = kGuMaxNL - nr_of<MT>();
  static constexpr size_t x_bytes = (size_t)XL * MT * 2 * 64 * 16;
  static constexpr size_t slab_bytes = (size_t)kGuCols * 64 * 2;
  static constexpr size_t roots_bytes = (size_t)2 * 2 * kGuWaves * (MT * 2) * 64 * 4;  // [parity][b][wave][NP][lane]
  static constexpr size_t total = roots_bytes + kGuWaves * (x_bytes + slab_bytes);
};

template <class T, int MT>
struct GuWave {
  static constexpr int NP = MT * 2;  // packed pairs of stored values per lane: index 2 t + h
  static constexpr int NR = nr_of<MT>();
  struct WF {
    u32x4 v[2];  // rows 8 i2 + lane / 8 of the tile, 16-byte K chunk lane % 8 of the leaf
  };

  const GuParams &p;
  uint32_t *roots;   // LDS [2][2][waves][NP][64]
  u32x4 *xl;         // this wave's LDS activation fragments [XL][MT][2][64]
  uint16_t *slab;    // this wave's 16 x 64 staging slab
  int wave, lane, r16, g4;
  int lo;
  int64_t m0;
  int t0, ts, ntl;  // tiles t0 + i ts, i < ntl
  int64_t wbytes[2];

  __device__ __forceinline__ int64_t col0(int i) const { return (int64_t)(t0 + (i < ntl ? i : ntl - 1) * ts) * kGuCols; }

  // Weight unit (tile i, product b, leaf lo + j): 16 rows x 128 bytes.  Rows
  // past N read as zero (range check of the rebased descriptor), and so does
  // every row of a prefetch past this workgroup's last tile (an empty range:
  // no memory request at all).
  __device__ __forceinline__ void load_unit(int i, int b, int j, WF &w, const uint32_t (&voff)[2][2]) const {
    const int64_t base = (col0(i) * p.ldw[b] + (int64_t)(lo + j) * kLeaf) * 2;
    const int64_t left = i < ntl ? wbytes[b] - base : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)p.w[b] + base), (short)0,
        (int)(left > 0 ? (left < 0x7fffffff ? left : 0x7fffffff) : 0), 0x00020000);
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
      w.v[i2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff[b][i2], 0, 2));
  }

  // Leaf J of product b: the 16 weight rows through the slab (row r's chunk c
  // at r*64 + 8 (c ^ (r & 7)): conflict-free row writes and MFMA-layout
  // reads), two MFMAs per token tile from a zero accumulator, rounded and packed.
  template <int J>
  __device__ __forceinline__ void leaf(const WF &w, const typename T::frag (&xr)[NR][MT][2], uint32_t (&v)[NP]) const {
    const int wr = lane >> 3, wc = lane & 7;
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) *reinterpret_cast<u32x4 *>(&slab[(8 * i2 + wr) * 64 + 8 * (wc ^ wr)]) = w.v[i2];
    wave_lds_sync();
    const typename T::frag w0 = *reinterpret_cast<const typename T::frag *>(&slab[r16 * 64 + 8 * ((0 + g4) ^ (r16 & 7))]);
    const typename T::frag w1 = *reinterpret_cast<const typename T::frag *>(&slab[r16 * 64 + 8 * ((4 + g4) ^ (r16 & 7))]);
    typename T::frag xf[MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if constexpr (J < NR)
          xf[t][s] = xr[J][t][s];
        else
          xf[t][s] = __builtin_bit_cast(typename T::frag, xl[((J - NR) * MT + t) * 2 * 64 + s * 64 + lane]);
      }
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      acc[t] = T::mfma(w0, xf[t][0], f32x4{0.f, 0.f, 0.f, 0.f});
      acc[t] = T::mfma(w1, xf[t][1], acc[t]);
    }
    wave_lds_sync();  // slab reads done before the next unit overwrites it
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      v[2 * t + 0] = T::pack(acc[t][0], acc[t][1]);
      v[2 * t + 1] = T::pack(acc[t][2], acc[t][3]);
    }
  }

  // Activation leaf j (all token blocks): whole 128-byte row segments (lane:
  // row 8 s + lane / 8 of token block t, 16-byte chunk lane % 8 of the leaf;
  // rows past M clamped to a valid row, never stored), every row segment by
  // one instruction.  Fragment-layout loads would split every line over two.
  __device__ __forceinline__ void load_x(int j, u32x4 (&raw)[MT][2]) const {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t r = m0 + 16 * t + 8 * s + (lane >> 3);
        const uint16_t *row = p.x + (r < p.M ? r : p.M - 1) * p.ldx + 8 * (lane & 7);
        raw[t][s] = __builtin_bit_cast(u32x4, load_frag<T>(row, (int64_t)(lo + j) * kLeaf));
      }
  }

  // ... rearranged into the MFMA layout through the wave's slab, as the weight
  // units are: the first NR leaves to registers, the rest to the wave's LDS.
  template <int J>
  __device__ __forceinline__ void place_x(const u32x4 (&raw)[MT][2], typename T::frag (&xr)[NR][MT][2]) const {
    const int wr = lane >> 3, wc = lane & 7;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int s = 0; s < 2; ++s) *reinterpret_cast<u32x4 *>(&slab[(8 * s + wr) * 64 + 8 * (wc ^ wr)]) = raw[t][s];
      wave_lds_sync();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const typename T::frag f = *reinterpret_cast<const typename T::frag *>(&slab[r16 * 64 + 8 * ((4 * s + g4) ^ (r16 & 7))]);
        if constexpr (J < NR)
          xr[J][t][s] = f;
        else
          xl[((J - NR) * MT + t) * 2 * 64 + s * 64 + lane] = __builtin_bit_cast(u32x4, f);
      }
      wave_lds_sync();  // the slab's reads are done before it is rewritten
    }
  }

  // Units U.. of one tile: unit U is leaf U % NL of product U / NL, in ring
  // slot U % PR (PR divides the 2 NL units of a tile, so every tile starts in
  // slot 0); each unit first issues the loads of the unit PR - 1 ahead
  // (possibly of the next tile) into the slot the previous unit freed.  In
  // the first tile (FIRST) the gate units also bring in the activation: unit
  // J issues the loads of activation leaf J + XD and places leaf J, whose
  // loads went out XD units earlier, so that the activation arrives beside
  // the weight stream instead of before it.
  static constexpr int XD = 3;       // activation leaves in flight ahead of their first use
  static constexpr int XS = XD + 1;  // their register slots
  template <int NL, int PR, int U, bool FIRST>
  __device__ __forceinline__ void units(int i, WF (&ring)[PR], typename T::frag (&xr)[NR][MT][2], u32x4 (&raw)[XS][MT][2],
                                        uint32_t (&v)[NP], uint32_t (&st)[3][NP], uint32_t (&rg)[NP],
                                        const uint32_t (&voff)[2][2]) const {
    constexpr int UN = 2 * NL;
    if constexpr (U < UN) {
      constexpr int b = U / NL, J = U % NL;
      constexpr int nx = U + PR - 1, nu = nx % UN;
      load_unit(i + nx / UN, nu / NL, nu % NL, ring[nx % PR], voff);
      if constexpr (FIRST && U < NL) {
        if constexpr (U + XD < NL) load_x(U + XD, raw[(U + XD) % XS]);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the placement
        place_x<U>(raw[U % XS], xr);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this unit's MFMAs
      leaf<J>(ring[U % PR], xr, v);
      push_leaf<T, NP, NL, J>(v, st);
      if constexpr (J == NL - 1 && b == 0) {
#pragma unroll
        for (int q = 0; q < NP; ++q) rg[q] = v[q];
      }
      units<NL, PR, U + 1, FIRST>(i, ring, xr, raw, v, st, rg, voff);
    }
  }

  // Park the gate and up roots of tile i, then (after the barrier) join the 8
  // wave roots of each with the balanced top of the tree and apply the
  // activation: wave t < MT takes token block t.
  __device__ __forceinline__ void finish_tile(int i, const uint32_t (&rg)[NP], const uint32_t (&ru)[NP]) const {
    uint32_t *buf = roots + (size_t)(i & 1) * 2 * kGuWaves * NP * 64;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      buf[((0 * kGuWaves + wave) * NP + q) * 64 + lane] = rg[q];
      buf[((1 * kGuWaves + wave) * NP + q) * 64 + lane] = ru[q];
    }
    __syncthreads();
    if (wave >= MT) return;
    const int t = wave;
    uint32_t o[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t r[kGuWaves];
#pragma unroll
        for (int w2 = 0; w2 < kGuWaves; ++w2) r[w2] = buf[((b * kGuWaves + w2) * NP + 2 * t + h) * 64 + lane];
        o[b][h] = node2t<T>(node2t<T>(node2t<T>(r[0], r[1]), node2t<T>(r[2], r[3])), node2t<T>(node2t<T>(r[4], r[5]), node2t<T>(r[6], r[7])));
      }
    uint32_t av[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float ga = T::lo(o[0][h]), gb = T::hi(o[0][h]);
      const float ua = T::lo(o[1][h]), ub = T::hi(o[1][h]);
      const float sa = ga * sigma_f(ga), sb = gb * sigma_f(gb);
      av[h] = T::pack_prod(sa * ua, sb * ub);
    }
    const int64_t m = m0 + 16 * t + r16, n = col0(i) + 4 * g4;
    if (m >= p.M || n >= p.N) return;
    auto put = [&](uint16_t *C, int64_t ldc, uint32_t lo2, uint32_t hi2) {
      uint16_t *dst = C + m * ldc + n;
      if (n + 3 < p.N) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(lo2, hi2);
      } else {
        const uint16_t h4[4] = {(uint16_t)(lo2 & 0xffff), (uint16_t)(lo2 >> 16), (uint16_t)(hi2 & 0xffff),
                                (uint16_t)(hi2 >> 16)};
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) dst[e] = h4[e];
      }
    };
    put(p.a, p.lda, av[0], av[1]);
    if (p.g) put(p.g, p.ldgu, o[0][0], o[0][1]);
    if (p.u) put(p.u, p.ldgu, o[1][0], o[1][1]);
  }

  template <int NL>
  __device__ __forceinline__ void run() const {
    if (ntl <= 0) return;
    // the first activation leaves go out before the first weight units: all
    // workgroups start together, and a load issued behind the weight units
    // would wait for the whole chip's first units to drain
    typename T::frag xr[NR][MT][2];
    u32x4 raw[XS][MT][2];
#pragma unroll
    for (int j = 0; j < XD && j < NL; ++j) load_x(j, raw[j]);
    uint32_t voff[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
        voff[b][i2] = (uint32_t)(((8 * i2 + (lane >> 3)) * p.ldw[b] + 8 * (lane & 7)) * 2);
    constexpr int PR = (2 * NL) % kGuRing == 0 ? kGuRing : 2;
    WF ring[PR];
#pragma unroll
    for (int g = 0; g < PR - 1; ++g) load_unit(g / (2 * NL), (g % (2 * NL)) / NL, g % NL, ring[g], voff);
    {
      uint32_t v[NP], st[3][NP], rg[NP];
      units<NL, PR, 0, true>(0, ring, xr, raw, v, st, rg, voff);
      finish_tile(0, rg, v);
    }
    for (int i = 1; i < ntl; ++i) {
      uint32_t v[NP], st[3][NP], rg[NP];
      units<NL, PR, 0, false>(i, ring, xr, raw, v, st, rg, voff);
      finish_tile(i, rg, v);
    }
  }
};

template <class T, int MT>
__global__ __launch_bounds__(kGuWaves * 64) void k_gate_up_act(GuParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t gu_lds[];
  using Wv = GuWave<T, MT>;
  using Lay = GuLds<MT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lo, hi;
  subtree_range(p.L, 3, wave, lo, hi);
  const int tiles_n = (int)((p.N + kGuCols - 1) / kGuCols);
  // tiles t0, t0 + G, t0 + 2G, ... with t0 consecutive on one XCD: at each
  // step the workgroups of an XCD write neighbouring 16-column tiles, so the
  // four pieces of a 64-column output line reach one L2 at about one time
  const int G = (int)gridDim.x;
  const int t0 = xcd_tile((int)blockIdx.x, G);
  const int ntl = t0 < tiles_n ? (tiles_n - t0 + G - 1) / G : 0;
  char *base = reinterpret_cast<char *>(gu_lds) + Lay::roots_bytes + (size_t)wave * (Lay::x_bytes + Lay::slab_bytes);
  Wv w{p,
       gu_lds,
       reinterpret_cast<u32x4 *>(base),
       reinterpret_cast<uint16_t *>(base + Lay::x_bytes),
       wave,
       lane,
       lane & 15,
       lane >> 4,
       lo,
       (int64_t)blockIdx.y * 16 * MT,
       t0,
       G,
       ntl,
       {p.N * p.ldw[0] * 2, p.N * p.ldw[1] * 2}};
  switch (hi - lo) {  // 1..8 by the launch conditions (8 <= L <= 64)
    case 1: w.template run<1>(); break;
    case 2: w.template run<2>(); break;
    case 3: w.template run<3>(); break;
    case 4: w.template run<4>(); break;
    case 5: w.template run<5>(); break;
    case 6: w.template run<6>(); break;
    case 7: w.template run<7>(); break;
    default: w.template run<8>(); break;
  }
}

}  // namespace

bool gu_act_applies(int64_t M, int64_t N, int64_t K) {
  const int64_t L = K / kLeaf;
  return M >= 1 && M <= 32 && N >= 1 && K % kLeaf == 0 && L >= kGuWaves && L <= kGuWaves * kGuMaxNL;
}

template <class T>
hipError_t launch_gu_act_t(const GuParams &p, hipStream_t stream) {
  const int mt = p.M <= 16 ? 1 : 2;
  const int64_t tiles_n = (p.N + kGuCols - 1) / kGuCols;
  // one wave of workgroups over the 256 CUs (one workgroup per CU by LDS);
  // each takes ceil(tiles / groups) tiles, `groups` apart
  int64_t per = (tiles_n + 255) / 256;
  const int64_t groups = (tiles_n + per - 1) / per;
  const dim3 grid((unsigned)groups, 1u), block(kGuWaves * 64);
  if (mt == 1)
    dgf_launch(k_gate_up_act<T, 1>, grid, block, GuLds<1>::total, stream, p);
  else
    dgf_launch(k_gate_up_act<T, 2>, grid, block, GuLds<2>::total, stream, p);
  return hipGetLastError();
}

hipError_t launch_gu_act(const GuParams &p, hipStream_t stream) {
  if (p.fmt == FMT_F16) return launch_gu_act_t<F16>(p, stream);
  return launch_gu_act_t<Bf16>(p, stream);
}

}  // namespace dgf
