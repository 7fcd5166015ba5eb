// Weight-streaming tree GEMMs with stationary activations (gfx950).
//
// C_b[m][n] = T_K( A_b[m,:] . W_b[n or :, :] ) for the FFN's thin products:
// few tokens m, a large weight W_b that is read from HBM exactly once.
//
// Work split.  The canonical midpoint tree over the L = ceil(K/64) leaves is
// cut at depth kd into 2^kd K pieces (grid.z, times the batched products b),
// and each piece again at depth log2(WAVES) into one subtree of at most 4
// leaves per wave.  A wave loads the activation fragments of its leaves once
// and keeps them in registers while it walks over a contiguous range of
// output tiles (16 RT columns each): per tile it streams its leaves' weight
// rows (NT: 16 RT rows x 64 K per leaf, staged through LDS so that every load
// instruction reads whole 128-byte row segments) or weight slab (NN: 64 K
// rows x 16 RT columns per leaf, in two halves of 32 rows, transposed through
// LDS),
// reduces the leaves with the subtree's fixed shape in registers and parks
// the subtree root in LDS.  After a workgroup barrier the WAVES roots of the
// tile are joined with the balanced top of the piece's subtree, each wave
// taking one 16 x 16 block of the tile, and the piece root is stored: to the
// caller's output (kd = 0, plain store), else to a partial buffer that a
// combine kernel joins with the top kd levels of the tree and the epilogue
// (RL-Kernel PR #325, section "Design": contiguous K pieces are subtrees of
// the one canonical tree, so any cut reproduces the unsharded result).
//
// Every weight byte is read once per token tile; the activation operand is
// read once per wave instead of once per leaf and tile, which is what bounds
// a thin tree GEMM that reloads it.  An NN wave reads whole 128-byte row
// segments (64 columns); with 32 columns two CUs would each fetch half of
// every line.
#include "dgf_device.hpp"
#include "dgf_kernels.hpp"

namespace dgf {
namespace {

constexpr int kMaxNL = 4;    // leaves per wave
constexpr int kXsWaves = 8;  // waves per workgroup (at most)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-column tiles per output tile.  NT: 4 (64 columns) for one token tile, 2
// for two, which keeps a wave's registers (stationary activations, two leaves
// of weights in flight, the pending subtree values) within the 256 that let
// two waves share a SIMD.  NN: always 4, streamed in half leaves.
template <int LAYOUT, int MT>
constexpr int rt_of() {
  return LAYOUT == DGF_LAYOUT_NN ? 4 : (MT == 1 ? 4 : 2);
}

// NN slab: the leaf's 64 K rows of 64 columns, row-major in 16-byte chunks,
// chunk c of row k at c ^ nn_swz(k).  The transposing reads of one operand
// touch 16 rows k = 8 q + 4 h + r (q = lane / 16, r = lane / 4 % 4) at 32
// bytes each; this map puts the rows of any 32 lanes on distinct 4-byte banks
// of a 64-bank LDS and the rows of all 64 lanes on distinct banks of a
// 128-bank one (bank offset 32 (k mod 2) or 32 (k mod 4) plus 4 c): chunk bit
// 1 takes q's low bit, chunk bit 2 the parity of k's bit 1 and q's high bit.
__device__ __forceinline__ int nn_swz(int k) { return ((k >> 2) & 2) | ((((k >> 1) ^ (k >> 4)) & 1) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// One streaming unit of weights: NT a whole leaf, NN half a leaf.
template <int LAYOUT, int RT>
struct WFrag;
template <int RT>
struct WFrag<DGF_LAYOUT_NT, RT> {
  u32x4 v[2 * RT];  // rows 8 i + lane / 8, 16-byte K chunk lane % 8 of the leaf
};
template <int RT>
struct WFrag<DGF_LAYOUT_NN, RT> {
  u32x4 v[RT];  // slab rows 32 S + lrow + (32 / RT) i, columns 8 lcol .. 8 lcol + 7
};

template <class T, int MT>
struct XFrag {
  typename T::frag v[kMaxNL][MT][2];
};

// Static-shape post-order reduction of a wave's NL <= 4 leaves (midpoint
// tree: 3 leaves split 1 | 2, 4 leaves split 2 | 2).  v holds leaf J of the
// tile on entry and, after the last leaf, the subtree root.
template <class T, int NP, int NL, int J>
__device__ __forceinline__ void leaf_reduce(uint32_t (&v)[NP], uint32_t (&s0)[NP], uint32_t (&s1)[NP]) {
  if constexpr (NL == 2) {
    if constexpr (J == 0) {
#pragma unroll
      for (int q = 0; q < NP; ++q) s0[q] = v[q];
    } else {
#pragma unroll
      for (int q = 0; q < NP; ++q) v[q] = node2t<T>(s0[q], v[q]);
    }
  } else if constexpr (NL == 3) {
    if constexpr (J == 0) {
#pragma unroll
      for (int q = 0; q < NP; ++q) s0[q] = v[q];
    } else if constexpr (J == 1) {
#pragma unroll
      for (int q = 0; q < NP; ++q) s1[q] = v[q];
    } else {
#pragma unroll
      for (int q = 0; q < NP; ++q) v[q] = node2t<T>(s0[q], node2t<T>(s1[q], v[q]));
    }
  } else if constexpr (NL == 4) {
    if constexpr (J == 0) {
#pragma unroll
      for (int q = 0; q < NP; ++q) s0[q] = v[q];
    } else if constexpr (J == 1) {
#pragma unroll
      for (int q = 0; q < NP; ++q) s0[q] = node2t<T>(s0[q], v[q]);
    } else if constexpr (J == 2) {
#pragma unroll
      for (int q = 0; q < NP; ++q) s1[q] = v[q];
    } else {
#pragma unroll
      for (int q = 0; q < NP; ++q) v[q] = node2t<T>(s0[q], node2t<T>(s1[q], v[q]));
    }
  }
}

// PR: ring slots of weight units (prefetch distance PR - 1 units).
template <class T, int LAYOUT, int MT, int PR>
struct XsWave {
  static constexpr bool NN = LAYOUT == DGF_LAYOUT_NN;
  static constexpr int RT = rt_of<LAYOUT, MT>();
  static constexpr int NP = RT * MT * 2;  // packed pairs of stored values per lane: index (rt MT + t) 2 + h
  static constexpr int NI = 2 * RT;       // NN: lanes per slab row (16 bytes each)
  static constexpr int ROWS = 32 / RT;    // NN: slab rows per load instruction
  static constexpr int COLS = 16 * RT;    // output columns per tile
  using WF = WFrag<LAYOUT, RT>;

  const GemmParams &p;
  uint32_t *roots;   // LDS [2][waves][NP][64]
  uint16_t *slab;    // LDS, this wave's COLS x 64 staging slab
  int waves, wave, lane, r16, g4;
  int b, lo, nl;
  bool tail;
  int64_t m0;
  int tiles_n, t0, ntl;  // this workgroup's tiles: t0 .. t0 + ntl - 1
  const uint16_t *W;
  int64_t ldw;
  uint16_t *out;
  int64_t ldo;
  int64_t wbytes;  // bytes of W the loads may touch: N rows (NT) or K rows (NN) of ldw elements

  __device__ __forceinline__ int tile_at(int i) const { return t0 + (i < ntl ? i : ntl - 1); }

  // Weights of unit (tile i clamped, leaf lo + j, half s): NT the whole leaf
  // (s ignored), NN rows 32 s .. 32 s + 31 of the leaf's slab.  Buffer loads:
  // the descriptor is rebased on the unit's first byte (scalar arithmetic)
  // and every lane adds its fixed offset voff[i2], so a unit costs no vector
  // address arithmetic.  Bytes past the matrix read as zero (the range check
  // of the rebased descriptor): NT rows past N, NN rows past K, and every
  // byte of a prefetch past this workgroup's last tile (an empty range: no
  // memory request at all).
  __device__ __forceinline__ void load_unit(int i, int j, int s, WF &w, const uint32_t (&voff)[2 * RT]) const {
    const int64_t n0 = (int64_t)tile_at(i) * COLS;
    const int64_t kb = (int64_t)(lo + j) * kLeaf;
    const int64_t base = NN ? ((kb + 32 * s) * ldw + n0) * 2 : (n0 * ldw + kb) * 2;
    const int64_t left = i < ntl ? wbytes - base : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)W + base), (short)0, (int)(left > 0 ? (left < 0x7fffffff ? left : 0x7fffffff) : 0),
        0x00020000);
    constexpr int NL = NN ? RT : 2 * RT;
#pragma unroll
    for (int i2 = 0; i2 < NL; ++i2)
      w.v[i2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff[i2], 0, 2));
  }

  // per-lane byte offsets of the unit loads (relative to the unit's first byte)
  __device__ __forceinline__ void unit_offsets(uint32_t (&voff)[2 * RT]) const {
    if constexpr (!NN) {
#pragma unroll
      for (int i2 = 0; i2 < 2 * RT; ++i2) voff[i2] = (uint32_t)(((8 * i2 + (lane >> 3)) * ldw + 8 * (lane & 7)) * 2);
    } else {
      const int lrow = lane / NI, lcol = lane % NI;
#pragma unroll
      for (int i2 = 0; i2 < 2 * RT; ++i2) voff[i2] = (uint32_t)(((lrow + ROWS * i2) * ldw + 8 * lcol) * 2);
    }
  }

  // The same for the partial last leaf: zeros past K.
  __device__ __forceinline__ void load_unit_tail(int i, int j, int s, WF &w) const {
    const int64_t n0 = (int64_t)tile_at(i) * COLS;
    const int64_t kb = (int64_t)(lo + j) * kLeaf;
    if constexpr (!NN) {
#pragma unroll
      for (int i2 = 0; i2 < 2 * RT; ++i2) {
        const int64_t n = n0 + 8 * i2 + (lane >> 3) < p.N ? n0 + 8 * i2 + (lane >> 3) : p.N - 1;
        w.v[i2] = __builtin_bit_cast(u32x4, load_frag_tail<T>(W + n * ldw, kb + 8 * (lane & 7), p.K));
      }
    } else {
      // rows past K read row K-1 and are zeroed
      const int lrow = lane / NI, lcol = lane % NI;
      const int64_t c0 = n0 + 8 * lcol;
      const int64_t nlast = ((p.N + 7) & ~(int64_t)7) - 8;
      const int64_t c = c0 <= nlast ? c0 : nlast;
#pragma unroll
      for (int i2 = 0; i2 < RT; ++i2) {
        const int64_t k = kb + 32 * s + lrow + ROWS * i2;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(W + (k < p.K ? k : p.K - 1) * ldw + c);
        w.v[i2] = k < p.K ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void pack(const f32x4 (&acc)[RT][MT], uint32_t (&v)[NP]) const {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        v[(rt * MT + t) * 2 + 0] = T::pack(acc[rt][t][0], acc[rt][t][1]);
        v[(rt * MT + t) * 2 + 1] = T::pack(acc[rt][t][2], acc[rt][t][3]);
      }
  }

  // NT: both K halves of a leaf (the second unless `half1` is false: an
  // all-zero block leaves the sum unchanged), rounded and packed.  The rows pass
  // through this wave's LDS slab: row r's 16-byte chunk c at r*64 + 8 (c ^ (r&7)),
  // which keeps both the row-wise writes and the MFMA-layout reads (lane:
  // row 16 rt + r16, chunk 4 h + g4) on distinct banks.
  __device__ __forceinline__ void leaf_nt(const WF &w, const typename T::frag (&x)[MT][2], bool half1, uint32_t (&v)[NP]) const {
    const int wr = lane >> 3, wc = lane & 7;
#pragma unroll
    for (int i2 = 0; i2 < 2 * RT; ++i2)
      *reinterpret_cast<u32x4 *>(&slab[(8 * i2 + wr) * 64 + 8 * (wc ^ wr)]) = w.v[i2];
    wave_lds_sync();  // this wave's slab writes land before its lanes read them
    f32x4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = 16 * rt + r16;
      const typename T::frag w0 = *reinterpret_cast<const typename T::frag *>(&slab[r * 64 + 8 * ((0 + g4) ^ (r & 7))]);
      const typename T::frag w1 = *reinterpret_cast<const typename T::frag *>(&slab[r * 64 + 8 * ((4 + g4) ^ (r & 7))]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[rt][t] = T::mfma(w0, x[t][0], f32x4{0.f, 0.f, 0.f, 0.f});
        if (half1) acc[rt][t] = T::mfma(w1, x[t][1], acc[rt][t]);
      }
    }
    wave_lds_sync();  // slab reads done before the next leaf overwrites it
    pack(acc, v);
  }

  // NN: half S of a leaf.  The 32 slab rows go to LDS as loaded (row-major,
  // 16-byte writes), and each weight operand comes back in MFMA layout with
  // two transposing reads (ds_read_b64_tr_b16: within each 16 lanes, the
  // 4-element reads of lanes 4 r .. 4 r + 3 form row r of a 4 x 16 block and
  // lane j receives its column j).  Lane (q = lane / 16, r, c = lane % 4)
  // reads row k = 32 S + 8 q + 4 h + r, columns 16 rt + 4 c .. + 3, so that
  // lane l obtains column 16 rt + l % 16 at K rows 32 S + 8 q + 4 h .. + 3.
  template <int S>
  __device__ __forceinline__ void half_nn(const WF &w, const typename T::frag (&x)[MT][2], f32x4 (&acc)[RT][MT]) const {
    const int lrow = lane / NI, lcol = lane % NI;
#pragma unroll
    for (int i2 = 0; i2 < RT; ++i2) {
      const int k = 32 * S + lrow + ROWS * i2;
      *reinterpret_cast<u32x4 *>(&slab[k * 64 + 8 * (lcol ^ nn_swz(k))]) = w.v[i2];
    }
    wave_lds_sync();  // this wave's slab writes land before its lanes read them
    const int q = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      s16x4 hv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 32 * S + 8 * q + 4 * h + r, n = 16 * rt + 4 * c;
        hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)&slab[k * 64 + 8 * ((n >> 3) ^ nn_swz(k)) + (n & 7)]);
      }
      const typename T::frag wf = __builtin_bit_cast(typename T::frag, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[rt][t] = T::mfma(wf, x[t][S], S == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[rt][t]);
    }
    wave_lds_sync();  // slab reads done before the next unit overwrites it
  }

  // Park this wave's subtree root of tile i, then (after the barrier) join the
  // WAVES roots for one 16 x 16 block per wave and store it.
  __device__ __forceinline__ void finish_tile(int i, const uint32_t (&root)[NP]) const {
    uint32_t *buf = roots + (size_t)(i & 1) * waves * NP * 64;
#pragma unroll
    for (int q = 0; q < NP; ++q) buf[(wave * NP + q) * 64 + lane] = root[q];
    __syncthreads();
    const int64_t n0 = (int64_t)tile_at(i) * COLS;
    for (int blk = wave; blk < RT * MT; blk += waves) {
      // the balanced tree over 8 roots, level by level; with fewer waves the
      // root is the level-log2(waves) node of the first group (roots past the
      // last wave read the last wave's and are never selected)
      uint32_t r[kXsWaves][2];
#pragma unroll
      for (int w2 = 0; w2 < kXsWaves; ++w2) {
        const int src = w2 < waves ? w2 : waves - 1;
        r[w2][0] = buf[(src * NP + 2 * blk + 0) * 64 + lane];
        r[w2][1] = buf[(src * NP + 2 * blk + 1) * 64 + lane];
      }
      uint32_t l1[4][2], l2[2][2], l3[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) l1[k2][h] = node2t<T>(r[2 * k2][h], r[2 * k2 + 1][h]);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) l2[k2][h] = node2t<T>(l1[2 * k2][h], l1[2 * k2 + 1][h]);
        l3[h] = node2t<T>(l2[0][h], l2[1][h]);
      }
      uint32_t o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) o[h] = waves == 8 ? l3[h] : waves == 4 ? l2[0][h] : waves == 2 ? l1[0][h] : r[0][h];
      const int rt = blk / MT, t = blk % MT;
      const int64_t m = m0 + 16 * t + r16, n = n0 + 16 * rt + 4 * g4;
      if (m < p.M) {
        uint16_t *dst = out + m * ldo + n;
        if (n + 3 < p.N) {
          *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0], o[1]);
        } else {
          const uint16_t h4[4] = {(uint16_t)(o[0] & 0xffff), (uint16_t)(o[0] >> 16), (uint16_t)(o[1] & 0xffff),
                                  (uint16_t)(o[1] >> 16)};
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) dst[e] = h4[e];
        }
      }
    }
  }

  // Units U.. of one tile.  Unit U is leaf U (NT) or half U % 2 of leaf U / 2
  // (NN).  Tiles run in groups of PR; unit U of the group's tile Q has group
  // index g = Q UN + U and lives in ring slot g % PR, and each unit first
  // issues the loads of unit g + PR - 1 (possibly of a later tile) into its slot.
  template <int NL, int NF, int Q, int U>
  __device__ __forceinline__ void units(int i, WF (&ring)[PR], const XFrag<T, MT> &xs, f32x4 (&acc)[RT][MT],
                                        uint32_t (&v)[NP], uint32_t (&s0)[NP], uint32_t (&s1)[NP],
                                        const uint32_t (&voff)[2 * RT]) const {
    constexpr int UN = NN ? 2 * NF : NF;
    if constexpr (U < UN) {
      constexpr int J = NN ? U / 2 : U, S = NN ? U % 2 : 0;
      constexpr int g = Q * UN + U, slot = g % PR;
      constexpr int nx = U + PR - 1;  // the unit to prefetch, counted from this tile's unit 0
      constexpr int nu = nx % UN;
      load_unit(i + nx / UN, NN ? nu / 2 : nu, NN ? nu % 2 : 0, ring[(g + PR - 1) % PR], voff);
      // keep the prefetch ahead of this unit's MFMAs: the scheduler would
      // otherwise sink the loads next to their use and serialise the stream
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!NN) {
        leaf_nt(ring[slot], xs.v[J], true, v);
        leaf_reduce<T, NP, NL, J>(v, s0, s1);
      } else {
        half_nn<S>(ring[slot], xs.v[J], acc);
        if constexpr (S == 1) {
          pack(acc, v);
          leaf_reduce<T, NP, NL, J>(v, s0, s1);
        }
      }
      units<NL, NF, Q, U + 1>(i, ring, xs, acc, v, s0, s1, voff);
    }
  }

  // One tile (index i) of a wave with NL leaves, the last partial when TAIL
  // (loaded without prefetch); NF = NL - TAIL go through the ring.
  template <int NL, bool TAIL, int Q>
  __device__ __forceinline__ void tile(int i, WF (&ring)[PR], const XFrag<T, MT> &xs, const uint32_t (&voff)[2 * RT]) const {
    constexpr int NF = NL - (TAIL ? 1 : 0);
    uint32_t s0[NP], s1[NP], v[NP];
    f32x4 acc[RT][MT];
    units<NL, NF, Q, 0>(i, ring, xs, acc, v, s0, s1, voff);
    if constexpr (TAIL) {
      const int64_t kb = (int64_t)(lo + NF) * kLeaf;
      const bool half1 = kb + 32 < p.K;  // an all-zero block leaves the sum unchanged
      WF wt;
      if constexpr (!NN) {
        load_unit_tail(i, NF, 0, wt);
        leaf_nt(wt, xs.v[NF], half1, v);
      } else {
        load_unit_tail(i, NF, 0, wt);
        half_nn<0>(wt, xs.v[NF], acc);
        if (half1) {
          load_unit_tail(i, NF, 1, wt);
          half_nn<1>(wt, xs.v[NF], acc);
        }
        pack(acc, v);
      }
      leaf_reduce<T, NP, NL, NF>(v, s0, s1);
    }
    finish_tile(i, v);
  }

  template <int NL, bool TAIL>
  __device__ __forceinline__ void run() const {
    constexpr int NF = NL - (TAIL ? 1 : 0);
    if (ntl <= 0) return;  // no tile for this workgroup (the same for all its waves)
    // The activation loads go out first, then the first weight units: all
    // workgroups start together, and an activation load issued behind the
    // weight units would wait for the whole chip's first units (megabytes)
    // to drain; this way the activation is rearranged while the weights are
    // on their way.  Stationary activation fragments of this wave's leaves
    // are loaded as whole 128-byte row segments (lane: row 8 s + lane / 8 of
    // token block t, 16-byte chunk lane % 8 of the leaf; rows past M clamped,
    // never stored; zeros past K) and rearranged into the MFMA layout through
    // this wave's slab: fragment-layout loads would split every line over two
    // instructions.
    u32x4 raw[NL][MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t r = m0 + 16 * t + 8 * s + (lane >> 3);
        const uint16_t *row = p.A[b] + (r < p.M ? r : p.M - 1) * p.lda[b];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int64_t k = (int64_t)(lo + j) * kLeaf + 8 * (lane & 7);
          raw[j][t][s] = __builtin_bit_cast(u32x4, (TAIL && j == NF) ? load_frag_tail<T>(row, k, p.K) : load_frag<T>(row, k));
        }
      }
    WF ring[PR];
    uint32_t voff[2 * RT];
    unit_offsets(voff);
    if constexpr (NF > 0) {
      constexpr int UN = NN ? 2 * NF : NF;
#pragma unroll
      for (int g = 0; g < PR - 1; ++g) {
        const int u = g % UN;
        load_unit(g / UN, NN ? u / 2 : u, NN ? u % 2 : 0, ring[g], voff);
      }
    }
    XFrag<T, MT> xs;
    {
      const int wr = lane >> 3, wc = lane & 7;
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
#pragma unroll
          for (int s = 0; s < 2; ++s)
            *reinterpret_cast<u32x4 *>(&slab[(8 * s + wr) * 64 + 8 * (wc ^ wr)]) = raw[j][t][s];
          wave_lds_sync();
#pragma unroll
          for (int s = 0; s < 2; ++s)
            xs.v[j][t][s] = *reinterpret_cast<const typename T::frag *>(&slab[r16 * 64 + 8 * ((4 * s + g4) ^ (r16 & 7))]);
          wave_lds_sync();  // the slab's reads are done before it is rewritten
        }
    }
    for (int i = 0; i < ntl; i += PR) {
      tile<NL, TAIL, 0>(i, ring, xs, voff);
      if (i + 1 < ntl) tile<NL, TAIL, 1>(i + 1, ring, xs, voff);
      if constexpr (PR > 2)
        if (i + 2 < ntl) tile<NL, TAIL, 2>(i + 2, ring, xs, voff);
    }
  }
};

// NLMAX: the largest leaf count of a wave in this launch.  The midpoint cuts
// leave every wave ceil or floor of L / 2^(kd + log2 waves) leaves, so one
// launch holds the shapes NLMAX and NLMAX - 1 only, and each instantiation
// is register-allocated for those two alone.
template <class T, int LAYOUT, int MT, int NLMAX>
__global__ __launch_bounds__(kXsWaves * 64) void k_xs(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs_lds[];
  // NN units are half leaves: two of them in flight measured faster than one
  // (except with 4 leaves and two token tiles, where the third slot spills);
  // the NT kernel measured fastest with one whole leaf in flight
  constexpr int PR = LAYOUT == DGF_LAYOUT_NN && !(MT == 2 && NLMAX == 4) ? 3 : 2;
  using Wv = XsWave<T, LAYOUT, MT, PR>;
  const int waves = blockDim.x >> 6;
  const int dw = __builtin_ctz(waves);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kd = p.ksplit_depth;
  // Workgroups are dealt to the 8 XCDs round robin in launch order; with
  // xcd_slices they are renumbered so that each XCD runs whole (product,
  // K piece) slices, whose workgroups then read the slice's activation
  // through one L2.
  int vx = (int)blockIdx.x, vy = (int)blockIdx.y, vz = (int)blockIdx.z;
  const unsigned gxy = gridDim.x * gridDim.y, nwg = gxy * gridDim.z;
  if (p.xcd_slices && (nwg & 7u) == 0 && ((nwg >> 3) % gxy) == 0) {
    unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    lin = (lin & 7u) * (nwg >> 3) + (lin >> 3);
    vx = (int)(lin % gridDim.x);
    vy = (int)((lin / gridDim.x) % gridDim.y);
    vz = (int)(lin / gxy);
  }
  const int b = vz >> kd, piece = vz & ((1 << kd) - 1);
  int lo, hi;
  subtree_range(p.L, kd + dw, (piece << dw) | wave, lo, hi);
  const int tiles_n = (int)((p.N + Wv::COLS - 1) / Wv::COLS);
  // contiguous tile ranges: workgroup g takes tiles g*per .. g*per + per - 1
  const int per = (tiles_n + (int)gridDim.x - 1) / (int)gridDim.x;
  const int t0 = vx * per;
  const int ntl = t0 < tiles_n ? min(per, tiles_n - t0) : 0;
  Wv w{p,
       xs_lds,
       reinterpret_cast<uint16_t *>(xs_lds + (size_t)2 * waves * Wv::NP * 64) + (size_t)wave * Wv::COLS * 64,
       waves,
       wave,
       lane,
       lane & 15,
       lane >> 4,
       b,
       lo,
       hi - lo,
       (int64_t)hi * kLeaf > p.K,
       (int64_t)vy * 16 * MT,
       tiles_n,
       t0,
       ntl,
       p.B[b],
       p.ldb[b],
       p.to_part ? p.part + ((int64_t)b * (1 << kd) + piece) * p.part_stride : p.C[b],
       p.to_part ? p.ldp : p.ldc[b],
       (LAYOUT == DGF_LAYOUT_NN ? p.K : p.N) * p.ldb[b] * 2};
  // the wave's leaf count (NLMAX or NLMAX - 1) and whether it owns the
  // partial last leaf, as compile-time shapes
  if (w.nl == NLMAX || NLMAX == 1) {
    if (w.tail)
      w.template run<NLMAX, true>();
    else
      w.template run<NLMAX, false>();
  } else if constexpr (NLMAX > 1) {
    if (w.tail)
      w.template run<NLMAX - 1, true>();
    else
      w.template run<NLMAX - 1, false>();
  }
}

}  // namespace

int xs_tile_cols(int layout, int mt) {
  if (layout == DGF_LAYOUT_NN) return 16 * rt_of<DGF_LAYOUT_NN, 1>();
  return 16 * (mt == 1 ? rt_of<DGF_LAYOUT_NT, 1>() : rt_of<DGF_LAYOUT_NT, 2>());
}

size_t xs_lds_bytes(int layout, int mt, int waves) {
  const size_t cols = (size_t)xs_tile_cols(layout, mt);
  const size_t np = cols / 16 * mt * 2;
  return 2 * (size_t)waves * np * 64 * 4 + (size_t)waves * cols * 64 * 2;
}

template <class T, int LAYOUT, int MT>
void launch_xs_nl(int nlmax, dim3 grid, dim3 block, size_t shm, hipStream_t stream, const GemmParams &p) {
  switch (nlmax) {
    case 1: dgf_launch((k_xs<T, LAYOUT, MT, 1>), grid, block, shm, stream, p); break;
    case 2: dgf_launch((k_xs<T, LAYOUT, MT, 2>), grid, block, shm, stream, p); break;
    case 3: dgf_launch((k_xs<T, LAYOUT, MT, 3>), grid, block, shm, stream, p); break;
    default: dgf_launch((k_xs<T, LAYOUT, MT, 4>), grid, block, shm, stream, p); break;
  }
}

template <class T>
hipError_t launch_xs_t(int layout, GemmParams p, int nb, int waves, int groups, hipStream_t stream) {
  const int mt = p.M <= 16 ? 1 : 2;
  const int64_t tiles_m = (p.M + 16 * mt - 1) / (16 * mt);
  const dim3 grid((unsigned)groups, (unsigned)tiles_m, (unsigned)(nb << p.ksplit_depth));
  const dim3 block((unsigned)(64 * waves));
  const size_t shm = xs_lds_bytes(layout, mt, waves);
  const int depth = p.ksplit_depth + __builtin_ctz((unsigned)waves);
  const int nlmax = (p.L + (1 << depth) - 1) >> depth;
  if (nlmax < 1 || nlmax > kMaxNL || (p.L >> depth) < 1) return hipErrorInvalidValue;
  if (layout == DGF_LAYOUT_NT) {
    if (mt == 1)
      launch_xs_nl<T, DGF_LAYOUT_NT, 1>(nlmax, grid, block, shm, stream, p);
    else
      launch_xs_nl<T, DGF_LAYOUT_NT, 2>(nlmax, grid, block, shm, stream, p);
  } else {
    if (mt == 1)
      launch_xs_nl<T, DGF_LAYOUT_NN, 1>(nlmax, grid, block, shm, stream, p);
    else
      launch_xs_nl<T, DGF_LAYOUT_NN, 2>(nlmax, grid, block, shm, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_xs(int layout, GemmParams p, int nb, int waves, int groups, hipStream_t stream) {
  if (p.fmt == FMT_F16) return launch_xs_t<F16>(layout, p, nb, waves, groups, stream);
  return launch_xs_t<Bf16>(layout, p, nb, waves, groups, stream);
}

}  // namespace dgf
