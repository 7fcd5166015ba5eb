// All-K tree GEMM for few tokens (gfx950): the down projection.
//
// C[m][n] = T_K( A[m,:] . B[n,:] ) for M <= 18 tokens, A [M, K] and B [N, K]
// both K-contiguous, with the canonical tree of RL-Kernel PR #325, section
// "Design".  The activation operand of the down projection (a, M x I) is a
// few hundred KB, small enough to be read from L2 by every workgroup, so
// instead of cutting K into pieces (partial roots and a join launch) every
// workgroup owns one 16-column output tile and all of K: the tree is cut at
// depth 3 into one equal subtree of NW leaves per wave (L = 8 NW), each wave
// streams its leaves' weight rows (HBM, read once) and activation rows (L2)
// as whole 128-byte row segments, stages both through its own swizzled LDS
// slabs into MFMA layout, and reduces its subtree with the fixed post-order
// in registers (the whole leaf sequence is unrolled, so the ring slots and
// the pending-value slots are static).  After a workgroup barrier the 8 wave
// roots are joined with the balanced top three levels and stored.
//
// Every workgroup reads all of A: 16 M_pad x 128 bytes of activation per
// 2 KB weight leaf.  A compute unit keeps only so many cache-line misses in
// flight, so activation lines compete with weight lines for them; measured on
// the Qwen3-8B down projection (forward at 12..24 tokens against the
// split-K kernel with its join), the all-K kernel is faster up to 17 tokens
// and slower from 20 (2.6 us at 24), so it takes at most 18.
#include "dgf_device.hpp"
#include "dgf_kernels.hpp"

namespace dgf {
namespace {

constexpr int kAkWaves = 8;
constexpr int kAkCols = 16;  // output columns per workgroup
constexpr int kAkRing = 4;   // ring slots: three leaves in flight per wave
constexpr int kAkMaxD = 6;   // depth of a wave subtree of at most 32 leaves
constexpr int kAkMaxM = 18;  // tokens (two token tiles from 17)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Feed leaf J of an N-leaf subtree (N <= 32): merge it with the pending left
// siblings its position closes, then park it at its depth.
template <class T, int NP, int N, int J>
__device__ __forceinline__ void push_leaf_deep(uint32_t (&v)[NP], uint32_t (&st)[kAkMaxD][NP]) {
  constexpr LeafPos lp = leaf_pos(N, J);
  static_assert(lp.D <= kAkMaxD, "subtree too deep");
#pragma unroll
  for (int t = 0; t < lp.m; ++t)
#pragma unroll
    for (int q = 0; q < NP; ++q) v[q] = node2t<T>(st[lp.D - 1 - t][q], v[q]);
  constexpr int d = lp.D - lp.m;
  if constexpr (d > 0) {
#pragma unroll
    for (int q = 0; q < NP; ++q) st[d - 1][q] = v[q];
  }
}

template <int MT>
struct AkLds {
  static constexpr size_t slab_w = (size_t)kAkCols * 64 * 2;   // 16 weight rows x 64 K
  static constexpr size_t slab_a = (size_t)16 * MT * 64 * 2;   // 16 MT activation rows x 64 K
  static constexpr size_t roots = (size_t)kAkWaves * (MT * 2) * 64 * 4;
  static constexpr size_t total = roots + kAkWaves * (slab_w + slab_a);
};

template <class T, int MT, int NW>
struct AkWave {
  static constexpr int NP = MT * 2;  // packed pairs of stored values per lane: index 2 t + h
  static constexpr int PR = kAkRing;
  struct Unit {
    u32x4 w[2];       // weight rows 8 i + lane / 8 of the tile, 16-byte K chunk lane % 8
    u32x4 a[2 * MT];  // activation rows 16 t + 8 i + lane / 8, same chunk
  };

  const AllkParams &p;
  uint16_t *sw, *sa;  // this wave's weight and activation slabs
  uint32_t *roots;
  int wave, lane, r16, g4, lo;
  int64_t n0;
  uint32_t vw[2], va[2 * MT];  // per-lane byte offsets within a leaf's rows

  // Leaf lo + J: rebased buffer descriptors (scalar arithmetic); weight rows
  // past N and activation rows past M read as zero (outside the range).
  __device__ __forceinline__ void load(int J, Unit &u) const {
    const int64_t kb = (int64_t)(lo + J) * kLeaf;
    const int64_t bw = (n0 * p.ldb + kb) * 2, rw = p.N * p.ldb * 2 - bw;
    const int64_t ra = p.M * p.lda * 2 - kb * 2;
    const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)p.B + bw), (short)0, (int)(rw > 0 ? (rw < 0x7fffffff ? rw : 0x7fffffff) : 0),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.A + kb), (short)0, (int)(ra > 0 ? (ra < 0x7fffffff ? ra : 0x7fffffff) : 0), 0x00020000);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      u.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsw, (int)vw[i], 0, 2));
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i)
      u.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsa, (int)va[i], 0, 0));
  }

  // One leaf: both operands through the slabs (row r's chunk c at
  // r*64 + 8 (c ^ (r & 7))), two MFMAs per token tile from a zero
  // accumulator, rounded and packed.
  __device__ __forceinline__ void leaf(const Unit &u, uint32_t (&v)[NP]) const {
    const int wr = lane >> 3, wc = lane & 7;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4 *>(&sw[(8 * i + wr) * 64 + 8 * (wc ^ wr)]) = u.w[i];
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) *reinterpret_cast<u32x4 *>(&sa[(8 * i + wr) * 64 + 8 * (wc ^ wr)]) = u.a[i];
    wave_lds_sync();
    const typename T::frag w0 = *reinterpret_cast<const typename T::frag *>(&sw[r16 * 64 + 8 * ((0 + g4) ^ (r16 & 7))]);
    const typename T::frag w1 = *reinterpret_cast<const typename T::frag *>(&sw[r16 * 64 + 8 * ((4 + g4) ^ (r16 & 7))]);
    typename T::frag x[MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        x[t][h] = *reinterpret_cast<const typename T::frag *>(&sa[(16 * t + r16) * 64 + 8 * ((4 * h + g4) ^ (r16 & 7))]);
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      acc[t] = T::mfma(w0, x[t][0], f32x4{0.f, 0.f, 0.f, 0.f});
      acc[t] = T::mfma(w1, x[t][1], acc[t]);
    }
    wave_lds_sync();  // slab reads done before the next leaf overwrites them
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      v[2 * t + 0] = T::pack(acc[t][0], acc[t][1]);
      v[2 * t + 1] = T::pack(acc[t][2], acc[t][3]);
    }
  }

  // Leaves J..: leaf J in ring slot J % PR; each first issues the loads of
  // leaf J + PR - 1 (none past the wave's last leaf) into the slot leaf J - 1
  // freed.
  template <int J>
  __device__ __forceinline__ void leaves(Unit (&ring)[PR], uint32_t (&v)[NP], uint32_t (&st)[kAkMaxD][NP]) const {
    if constexpr (J < NW) {
      if constexpr (J + PR - 1 < NW) load(J + PR - 1, ring[(J + PR - 1) % PR]);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this leaf's MFMAs
      leaf(ring[J % PR], v);
      push_leaf_deep<T, NP, NW, J>(v, st);
      leaves<J + 1>(ring, v, st);
    }
  }

  __device__ __forceinline__ void run() const {
    Unit ring[PR];
#pragma unroll
    for (int j = 0; j < PR - 1; ++j)
      if (j < NW) load(j, ring[j]);
    uint32_t v[NP], st[kAkMaxD][NP];
    leaves<0>(ring, v, st);
    // the 8 wave roots: balanced top three levels, wave t < MT taking token block t
#pragma unroll
    for (int q = 0; q < NP; ++q) roots[(wave * NP + q) * 64 + lane] = v[q];
    __syncthreads();
    if (wave >= MT) return;
    const int t = wave;
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t r[kAkWaves];
#pragma unroll
      for (int w2 = 0; w2 < kAkWaves; ++w2) r[w2] = roots[(w2 * NP + 2 * t + h) * 64 + lane];
      o[h] = node2t<T>(node2t<T>(node2t<T>(r[0], r[1]), node2t<T>(r[2], r[3])), node2t<T>(node2t<T>(r[4], r[5]), node2t<T>(r[6], r[7])));
    }
    const int64_t m = 16 * t + r16, n = n0 + 4 * g4;
    if (m >= p.M || n >= p.N) return;
    uint16_t *dst = p.C + m * p.ldc + n;
    if (n + 3 < p.N) {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0], o[1]);
    } else {
      const uint16_t h4[4] = {(uint16_t)(o[0] & 0xffff), (uint16_t)(o[0] >> 16), (uint16_t)(o[1] & 0xffff),
                              (uint16_t)(o[1] >> 16)};
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) dst[e] = h4[e];
    }
  }
};

template <class T, int MT, int NW>
__global__ __launch_bounds__(kAkWaves * 64) void k_allk(AllkParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t ak_lds[];
  using Lay = AkLds<MT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char *base = reinterpret_cast<char *>(ak_lds) + Lay::roots + (size_t)wave * (Lay::slab_w + Lay::slab_a);
  AkWave<T, MT, NW> w{p,
                   reinterpret_cast<uint16_t *>(base),
                   reinterpret_cast<uint16_t *>(base + Lay::slab_w),
                   ak_lds,
                   wave,
                   lane,
                   lane & 15,
                   lane >> 4,
                   wave * NW,  // the depth-3 subtrees of L = 8 NW leaves are NW leaves each
                   (int64_t)blockIdx.x * kAkCols,
                   {0u, 0u},
                   {}};
#pragma unroll
  for (int i = 0; i < 2; ++i) w.vw[i] = (uint32_t)(((8 * i + (lane >> 3)) * p.ldb + 8 * (lane & 7)) * 2);
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i) w.va[i] = (uint32_t)(((8 * i + (lane >> 3)) * p.lda + 8 * (lane & 7)) * 2);
  w.run();
}

template <class T, int MT>
hipError_t launch_allk_mt(const AllkParams &p, int nw, hipStream_t s) {
  const dim3 grid((unsigned)((p.N + kAkCols - 1) / kAkCols)), block(kAkWaves * 64);
  const size_t shm = AkLds<MT>::total;
  switch (nw) {
    case 1: dgf_launch((k_allk<T, MT, 1>), grid, block, shm, s, p); break;
    case 2: dgf_launch((k_allk<T, MT, 2>), grid, block, shm, s, p); break;
    case 3: dgf_launch((k_allk<T, MT, 3>), grid, block, shm, s, p); break;
    case 4: dgf_launch((k_allk<T, MT, 4>), grid, block, shm, s, p); break;
    case 6: dgf_launch((k_allk<T, MT, 6>), grid, block, shm, s, p); break;
    case 8: dgf_launch((k_allk<T, MT, 8>), grid, block, shm, s, p); break;
    case 12: dgf_launch((k_allk<T, MT, 12>), grid, block, shm, s, p); break;
    case 16: dgf_launch((k_allk<T, MT, 16>), grid, block, shm, s, p); break;
    case 24: dgf_launch((k_allk<T, MT, 24>), grid, block, shm, s, p); break;
    case 32: dgf_launch((k_allk<T, MT, 32>), grid, block, shm, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool allk_applies(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kAkMaxM || N < 1 || K % kLeaf != 0) return false;
  const int64_t L = K / kLeaf;
  if (L % kAkWaves != 0) return false;
  const int64_t nw = L / kAkWaves;
  return nw == 1 || nw == 2 || nw == 3 || nw == 4 || nw == 6 || nw == 8 || nw == 12 || nw == 16 || nw == 24 ||
         nw == 32;
}

hipError_t launch_allk(const AllkParams &p, hipStream_t stream) {
  if (p.M > kAkMaxM) return hipErrorInvalidValue;
  if (p.fmt == FMT_F16) {
    if (p.M > 16) return launch_allk_mt<F16, 2>(p, p.L / kAkWaves, stream);
    return launch_allk_mt<F16, 1>(p, p.L / kAkWaves, stream);
  }
  if (p.M > 16) return launch_allk_mt<Bf16, 2>(p, p.L / kAkWaves, stream);
  return launch_allk_mt<Bf16, 1>(p, p.L / kAkWaves, stream);
}

}  // namespace dgf
