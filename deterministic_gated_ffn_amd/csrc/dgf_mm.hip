// Tiled tree GEMM for many tokens (gfx950).
//
// C_b[m][n] = T_K( A_b[m,:] . B_b[n,:] ): A_b [M, K] and B_b [N, K] both
// K-contiguous, the canonical tree over K of RL-Kernel PR #325, section
// "Design" (64-element FP32 leaves rounded to the stored type, BF16 or FP16,
// midpoint nodes adding two stored children in FP32).  This is the compute-bound shape: thousands of tokens, so
// the weights are reused across many token rows and the kernel is organised
// around MFMA throughput rather than weight streaming.
//
// Work split.  A workgroup of 8 waves owns a 128 x 128 output tile (tokens x
// outputs) for one K piece (a subtree at depth kd of the tree, as in the other
// kernels); every wave owns 32 tokens x 64 outputs of it (8 MFMA tiles) and
// runs every leaf of the piece.  Per leaf the workgroup stages the 128 x 64 A
// and B tiles in LDS (double buffered, one barrier per leaf; rows swizzled by
// chunk ^ (row & 7) so that both the row-wise writes and the MFMA-layout reads
// are conflict-free; two leaves of tiles in flight in registers), and each
// wave runs two MFMAs per tile from a zero accumulator, the leaf of the other
// kernels.
//
// Tree.  The piece's midpoint tree is cut at depth UP (<= 3): every lower
// subtree (at most 4 leaves, two compile-time sizes) is reduced in registers
// with its static post-order as its leaves arrive, the merges of one leaf
// issued while the next leaf's fragment reads drain, and the 2^UP lower roots go through
// the perfect binary top of the tree, its pending left children parked in
// the wave's own LDS region (touched once per lower subtree).  The piece root
// goes to C or, with K split or an epilogue, to the partial buffer that the
// join kernel finishes.
//
// Bound.  Per leaf every wave runs 16 MFMAs but, for BF16, about 130 other
// VALU instructions (the rounding of 32 leaf values, about 32 nodes of an add
// and a rounding each, staging), and the barrier keeps the waves in step, so
// the LDS reads, the MFMAs and the VALU work of a leaf follow each other
// instead of overlapping: about 20% of the MFMA peak at the FFN's 4096-token
// shapes.  FP16 tree values are packed pairs (two roundings per conversion,
// two nodes per packed add), which halves that VALU work.
#include <type_traits>

#include "dgf_device.hpp"
#include "dgf_kernels.hpp"

namespace dgf {
namespace {

constexpr int kMmWaves = 8;
constexpr int kMmBM = 128, kMmBN = 128;  // workgroup tile: tokens x outputs
constexpr int kMmTM = 2, kMmTN = 4;      // a wave's 16 x 16 tiles: 32 tokens x 64 outputs
constexpr int kMmNV = kMmTM * kMmTN * 4;  // tree values per lane: index (tn TM + tm) 4 + e
constexpr int kMmNP = kMmNV / 2;          // the same as packed pairs (parked levels)
constexpr size_t kMmStage = (size_t)(kMmBM + kMmBN) * 64 * 2;  // A then B tile of one leaf (bytes)
// Leaves per lower subtree, at most: their pending values stay in registers.
constexpr int kMmMaxNL = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A lane's 32 tree values (tile i = tn TM + tm, element e) in the form that
// makes a node cheapest for the stored type.
//  - BF16: 32 FP32 registers, each value in FP32 form (the BF16 rounding kept
//    as an FP32 value, low half zero: one v_cvt_pk_bf16_f32 with a zero
//    partner), so a node is one FP32 add and one rounding.
//  - FP16: 16 registers of packed FP16 pairs (elements 2k and 2k + 1 of a
//    tile), so that one v_pk_add_f16 makes two nodes.  An FP16 add rounds the
//    exact sum once; rounding it to FP32 first and then to FP16 gives the same
//    value, because FP32 carries at least 2 * 11 + 2 significant bits (the
//    double rounding of a sum is innocuous then), and the exact sum of two
//    FP16 numbers below the FP16 normal range is exact in FP32.
template <class T>
struct Tv;
template <>
struct Tv<Bf16> {
  typedef float V;
  static constexpr int N = kMmNV;
  static constexpr int kLeafValu = kMmNV, kNodeValu = 2 * kMmNV;  // VALU per leaf rounding, per merge
  static __device__ __forceinline__ void leaf(const f32x4 &a, V (&v)[N], int i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * i + e] = Bf16::rf(a[e]);
  }
  static __device__ __forceinline__ V node(V l, V r) { return Bf16::rf(l + r); }
  // packed pair k (elements 2k, 2k + 1 of the lane's values) of stored values
  static __device__ __forceinline__ uint32_t pair(const V (&v)[N], int k) { return Bf16::pack_x(v[2 * k], v[2 * k + 1]); }
  static __device__ __forceinline__ void merge_pair(uint32_t l, V (&v)[N], int k) {
    v[2 * k] = Bf16::rf(Bf16::lo(l) + v[2 * k]);
    v[2 * k + 1] = Bf16::rf(Bf16::hi(l) + v[2 * k + 1]);
  }
};
template <>
struct Tv<F16> {
  typedef uint32_t V;
  static constexpr int N = kMmNV / 2;
  static constexpr int kLeafValu = kMmNV / 2, kNodeValu = kMmNV / 2;
  static __device__ __forceinline__ void leaf(const f32x4 &a, V (&v)[N], int i) {
    v[2 * i] = F16::pack(a[0], a[1]);
    v[2 * i + 1] = F16::pack(a[2], a[3]);
  }
  static __device__ __forceinline__ V node(V l, V r) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, l) + __builtin_bit_cast(f16x2, r));
  }
  static __device__ __forceinline__ uint32_t pair(const V (&v)[N], int k) { return v[k]; }
  static __device__ __forceinline__ void merge_pair(uint32_t l, V (&v)[N], int k) { v[k] = node(l, v[k]); }
};

// Feed leaf J (values v) of an N-leaf lower subtree (N <= 4): merge it with
// the pending left siblings its position closes, then park it at its depth;
// after the last leaf v is the subtree root.
template <class T, int N, int J>
__device__ __forceinline__ void push_f(typename Tv<T>::V (&v)[Tv<T>::N], typename Tv<T>::V (&st)[2][Tv<T>::N]) {
  constexpr LeafPos lp = leaf_pos(N, J);
#pragma unroll
  for (int t = 0; t < lp.m; ++t)
#pragma unroll
    for (int q = 0; q < Tv<T>::N; ++q) v[q] = Tv<T>::node(st[lp.D - 1 - t][q], v[q]);
  constexpr int d = lp.D - lp.m;
  if constexpr (d > 0) {
#pragma unroll
    for (int q = 0; q < Tv<T>::N; ++q) st[d - 1][q] = v[q];
  }
}

// TAIL: K is not a whole number of leaves (the last leaf is partial and
// loads element by element); otherwise every leaf takes the buffer path and
// the leaf sequence has no branches.
template <class T, bool TAIL>
struct MmWg {
  const GemmParams &p;
  uint16_t *lds;  // [2 stages][A 128 x 64 | B 128 x 64], then the waves' top-level stacks
  const uint16_t *A, *B;
  int64_t lda, ldb;
  int64_t m0, n0;
  int tid, wave, lane, r16, g4;
  int wm, wn;  // this wave's 32-token row block and 64-output column block
  int plo, phi;
  uint32_t voa[2], vob[2];  // byte offsets of this thread's chunks within a leaf's A and B tiles
  // whole-leaf path: descriptors at the tile's first row (k = 0), over the
  // rows from there on (rows past M / N fall outside and read as zero)
  __amdgpu_buffer_rsrc_t sa_tile, sb_tile;

  // Global loads of leaf j's two tiles: thread t covers chunks t and t + 512
  // of each (8 threads per 128-byte row segment).  A full leaf uses buffer
  // loads on descriptors rebased at the tile's first byte of the leaf (scalar
  // arithmetic) with fixed per-thread offsets; rows past M / N fall outside
  // the descriptor's range and read as zero.  The partial last leaf reads
  // element by element with zeros past K.
  // A leaf past the piece (j >= phi) is pushed out of the descriptors'
  // range: no memory request (the register set it fills is never used).
  __device__ __forceinline__ void fetch(int j, u32x4 (&g)[4]) const {
    const int64_t kb = (int64_t)j * kLeaf;
    if (!TAIL || kb + kLeaf <= p.K) {
      const uint32_t add = j < phi ? (uint32_t)(kb * 2) : 0x80000000u;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        g[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sa_tile, (int)(voa[i] + add), 0, 0));
        g[2 + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sb_tile, (int)(vob[i] + add), 0, 0));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 512 * i, row = q >> 3, kc = q & 7;
      const int64_t k = kb + 8 * kc;
      const int64_t m = m0 + row, n = n0 + row;
      g[i] = m < p.M ? __builtin_bit_cast(u32x4, load_frag_tail<T>(A + m * lda, k, p.K)) : u32x4{0u, 0u, 0u, 0u};
      g[2 + i] = n < p.N ? __builtin_bit_cast(u32x4, load_frag_tail<T>(B + n * ldb, k, p.K)) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  __device__ __forceinline__ void stage_store(int s, const u32x4 (&g)[4]) const {
    uint16_t *sa = lds + (size_t)s * (kMmStage / 2), *sb = sa + kMmBM * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 512 * i, row = q >> 3, kc = q & 7;
      *reinterpret_cast<u32x4 *>(&sa[row * 64 + 8 * (kc ^ (row & 7))]) = g[i];
      *reinterpret_cast<u32x4 *>(&sb[row * 64 + 8 * (kc ^ (row & 7))]) = g[2 + i];
    }
  }

  // The MFMA fragments of K half H of the leaf in stage s: this wave's 2 A
  // and 4 B tiles.
  template <int H>
  __device__ __forceinline__ void frags(const uint16_t *sa, const uint16_t *sb, typename T::frag (&af)[kMmTM],
                                        typename T::frag (&bf)[kMmTN]) const {
#pragma unroll
    for (int t = 0; t < kMmTM; ++t) {
      const int row = 32 * wm + 16 * t + r16;
      af[t] = *reinterpret_cast<const typename T::frag *>(&sa[row * 64 + 8 * ((4 * H + g4) ^ (r16 & 7))]);
    }
#pragma unroll
    for (int t = 0; t < kMmTN; ++t) {
      const int row = 64 * wn + 16 * t + r16;
      bf[t] = *reinterpret_cast<const typename T::frag *>(&sb[row * 64 + 8 * ((4 * H + g4) ^ (r16 & 7))]);
    }
  }

  // The canonical leaf of the wave's 8 tiles: two MFMAs per tile from a zero
  // accumulator (K 0..31, then 32..63).
  __device__ __forceinline__ void leaf_mfma(int s, f32x4 (&acc)[kMmTN][kMmTM]) const {
    const uint16_t *sa = lds + (size_t)s * (kMmStage / 2), *sb = sa + kMmBM * 64;
    typename T::frag af0[kMmTM], bf0[kMmTN], af1[kMmTM], bf1[kMmTN];
    frags<0>(sa, sb, af0, bf0);
    frags<1>(sa, sb, af1, bf1);
#pragma unroll
    for (int tn = 0; tn < kMmTN; ++tn)
#pragma unroll
      for (int tm = 0; tm < kMmTM; ++tm) acc[tn][tm] = T::mfma(bf0[tn], af0[tm], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int tn = 0; tn < kMmTN; ++tn)
#pragma unroll
      for (int tm = 0; tm < kMmTM; ++tm) acc[tn][tm] = T::mfma(bf1[tn], af1[tm], acc[tn][tm]);
  }

  typedef typename Tv<T>::V V;
  static constexpr int NV = Tv<T>::N;

  // A leaf's accumulators rounded to the stored type, as tree values.
  __device__ __forceinline__ void round_leaf(const f32x4 (&acc)[kMmTN][kMmTM], V (&v)[NV]) const {
#pragma unroll
    for (int tn = 0; tn < kMmTN; ++tn)
#pragma unroll
      for (int tm = 0; tm < kMmTM; ++tm) Tv<T>::leaf(acc[tn][tm], v, tn * kMmTM + tm);
  }

  // Leaf j (leaf J of a lower subtree of NL leaves) from stage s into acc, in
  // one scheduling region: the fragment reads, then the MFMAs interleaved
  // with the tree step of leaf J - 1 (rounding and merges of prev:
  // independent VALU work, about seven instructions per MFMA), then leaf
  // j + 1's tiles (fetched two leaves earlier into register set `nx`) into
  // the other stage and the fetch of leaf j + 3 into that set; the barrier
  // publishes the stage just written and frees the one just read.
  // FIN: at J = 0 the tree work beside the MFMAs is the last step of the
  // previous lower subtree (of the same size, its last leaf in prev): its
  // root in v afterwards.
  template <int NL, int J, bool FIN>
  __device__ __forceinline__ void one_leaf(int j, int s, u32x4 (&nx)[4], const f32x4 (&prev)[kMmTN][kMmTM],
                                           f32x4 (&acc)[kMmTN][kMmTM], V (&v)[NV], V (&st)[2][NV]) const {
    // merges of the tree step beside the MFMAs (-1: none), and the VALU
    // instructions to put beside each MFMA (a rounding, then an add and a
    // rounding per merge, per value)
    constexpr int m = J > 0 ? leaf_pos(NL, J - 1).m : FIN ? leaf_pos(NL, NL - 1).m : -1;
    constexpr int vpm = m < 0 ? 1 : (Tv<T>::kLeafValu + m * Tv<T>::kNodeValu + 15) / 16;
    __builtin_amdgcn_sched_barrier(0);
    leaf_mfma(s, acc);
    if constexpr (J > 0) {
      round_leaf(prev, v);
      push_f<T, NL, J - 1>(v, st);
    } else if constexpr (FIN) {
      round_leaf(prev, v);
      push_f<T, NL, NL - 1>(v, st);
    }
    // past the piece's last leaf the stage store writes a stage nobody reads
    // and the fetch requests nothing, so the leaf sequence needs no branch
    if (!TAIL || j + 1 < phi) stage_store(s ^ 1, nx);
    if (!TAIL || j + 3 < phi) fetch(j + 3, nx);
    if constexpr (!TAIL) {
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // fragment reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, vpm, 0);  // a share of the tree step
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);  // stage store
      __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);  // next fetch
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // Leaves J.. of a lower subtree of NL leaves, the first being leaf j of the
  // piece, whose parity in the piece is P0: the stage and register set of
  // every leaf are compile-time, and the two accumulator sets alternate with J.
  template <int NL, int J, int P0>
  __device__ __forceinline__ void leaves(int j, u32x4 (&r0)[4], u32x4 (&r1)[4], f32x4 (&prev)[kMmTN][kMmTM],
                                         f32x4 (&acc)[kMmTN][kMmTM], V (&v)[NV], V (&st)[2][NV]) const {
    if constexpr (J < NL) {
      constexpr int S = (P0 ^ J) & 1;
      if constexpr (S == 0)
        one_leaf<NL, J, false>(j, 0, r1, prev, acc, v, st);
      else
        one_leaf<NL, J, false>(j, 1, r0, prev, acc, v, st);
      leaves<NL, J + 1, P0>(j + 1, r0, r1, acc, prev, v, st);
    } else {
      round_leaf(prev, v);
      push_f<T, NL, NL - 1>(v, st);  // the subtree's last leaf: v becomes its root
    }
  }

  template <int NL>
  __device__ __forceinline__ void lower_tree(int j, u32x4 (&r0)[4], u32x4 (&r1)[4], V (&v)[NV]) const {
    V st[2][NV];
    f32x4 a0[kMmTN][kMmTM], a1[kMmTN][kMmTM];
    if (((j - plo) & 1) == 0)
      leaves<NL, 0, 0>(j, r0, r1, a0, a1, v, st);
    else
      leaves<NL, 0, 1>(j, r0, r1, a0, a1, v, st);
  }

  // The same when every lower subtree of the piece has NL leaves: the last
  // step of a subtree (about 5 VALU instructions per value) is deferred into
  // the first leaf of the next, beside its MFMAs.  Leaf jj of the piece (jj =
  // j - plo) accumulates into set jj & 1 (a0 or a1) and reads stage jj & 1;
  // after leaf 0 of a subtree, `upper` takes the previous subtree's root.
  template <int NL, int J, int P0, class UP>
  __device__ __forceinline__ void leaves_d(int j, u32x4 (&r0)[4], u32x4 (&r1)[4], f32x4 (&a0)[kMmTN][kMmTM],
                                           f32x4 (&a1)[kMmTN][kMmTM], V (&v)[NV], V (&st)[2][NV],
                                           const UP &upper) const {
    if constexpr (J < NL) {
      constexpr int S = (P0 ^ J) & 1;
      if constexpr (S == 0)
        one_leaf<NL, J, true>(j, 0, r1, a1, a0, v, st);
      else
        one_leaf<NL, J, true>(j, 1, r0, a0, a1, v, st);
      if constexpr (J == 0) upper(v);
      leaves_d<NL, J + 1, P0>(j + 1, r0, r1, a0, a1, v, st, upper);
    }
  }

  __device__ __forceinline__ void store_root(const V (&v)[NV], uint16_t *out, int64_t ldo) const {
#pragma unroll
    for (int tn = 0; tn < kMmTN; ++tn)
#pragma unroll
      for (int tm = 0; tm < kMmTM; ++tm) {
        const int64_t m = m0 + 32 * wm + 16 * tm + r16, n = n0 + 64 * wn + 16 * tn + 4 * g4;
        if (m >= p.M || n >= p.N) continue;
        const int i = (tn * kMmTM + tm) * 2;  // the tile's two packed pairs
        const uint32_t lo2 = Tv<T>::pair(v, i), hi2 = Tv<T>::pair(v, i + 1);
        uint16_t *dst = out + m * ldo + n;
        if (n + 3 < p.N) {
          *reinterpret_cast<uint2 *>(dst) = make_uint2(lo2, hi2);
        } else {
          const uint16_t h4[4] = {(uint16_t)(lo2 & 0xffff), (uint16_t)(lo2 >> 16), (uint16_t)(hi2 & 0xffff),
                                  (uint16_t)(hi2 >> 16)};
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) dst[e] = h4[e];
        }
      }
  }
};

// Pending left subtrees of the top levels, in this wave's own LDS region as
// packed pairs of stored values: level t, pair q of lane l at base[(t kMmNP + q) 64 + l]
// (each lane reads back only what it wrote; consecutive lanes, consecutive
// dwords).
template <class T>
__device__ __forceinline__ void park(uint32_t *base, int t, const typename Tv<T>::V (&v)[Tv<T>::N]) {
#pragma unroll
  for (int q = 0; q < kMmNP; ++q) base[(t * kMmNP + q) * 64] = Tv<T>::pair(v, q);
}
template <class T>
__device__ __forceinline__ void merge(const uint32_t *base, int t, typename Tv<T>::V (&v)[Tv<T>::N]) {
#pragma unroll
  for (int q = 0; q < kMmNP; ++q) Tv<T>::merge_pair(base[(t * kMmNP + q) * 64], v, q);
}

// NLH: the larger of the two lower-subtree sizes (the smaller is NLH - 1).
template <class T, int NLH, bool TAIL>
__global__ __launch_bounds__(kMmWaves * 64) void k_mm(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t mm_lds[];
  const int kd = p.ksplit_depth, up = p.stack_slots;  // K-piece depth; upper levels cut inside the piece
  const int b = blockIdx.z >> kd, piece = blockIdx.z & ((1 << kd) - 1);
  // Row-major tile order: the workgroups in flight share the A rows of a few
  // tile rows (a banded per-XCD order measured the same).
  const int tiles_n = (int)((p.N + kMmBN - 1) / kMmBN);
  const int tile_m = (int)blockIdx.x / tiles_n, tile_n = (int)blockIdx.x % tiles_n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)tile_m * kMmBM, n0 = (int64_t)tile_n * kMmBN;
  // descriptors at the tile's first row (k = 0) over the rows from there on;
  // a tile's rows times the leading dimension stay below 2^31 bytes (ld < 2^23)
  const int64_t ra = (p.M - m0) * p.lda[b] * 2, rb = (p.N - n0) * p.ldb[b] * 2;
  const __amdgpu_buffer_rsrc_t sa_tile = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(p.A[b] + m0 * p.lda[b]), (short)0, (int)(ra < 0x7fffffff ? ra : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t sb_tile = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(p.B[b] + n0 * p.ldb[b]), (short)0, (int)(rb < 0x7fffffff ? rb : 0x7fffffff), 0x00020000);
  MmWg<T, TAIL> w{p,
         mm_lds,
         p.A[b],
         p.B[b],
         p.lda[b],
         p.ldb[b],
         (int64_t)tile_m * kMmBM,
         (int64_t)tile_n * kMmBN,
         tid,
         wave,
         lane,
         lane & 15,
         lane >> 4,
         wave & 3,
         wave >> 2,
         0,
         0,
         {0u, 0u},
         {0u, 0u},
         sa_tile,
         sb_tile};
  subtree_range(p.L, kd, piece, w.plo, w.phi);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 512 * i, row = q >> 3, kc = q & 7;
    w.voa[i] = (uint32_t)((row * w.lda + 8 * kc) * 2);
    w.vob[i] = (uint32_t)((row * w.ldb + 8 * kc) * 2);
  }

  // leaf plo into stage 0; leaves plo + 1 and plo + 2 in flight in the two register sets
  u32x4 r0[4], r1[4];
  w.fetch(w.plo, r0);
  w.stage_store(0, r0);
  w.fetch(w.plo + 1, r1);  // empty past the piece
  w.fetch(w.plo + 2, r0);
  __syncthreads();

  // lower subtrees in order; the top `up` levels over their roots
  typedef typename Tv<T>::V V;
  constexpr int NV = Tv<T>::N;
  V v[NV];
  uint32_t *upl = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(mm_lds) + 2 * kMmStage) +
                  (size_t)wave * 3 * kMmNP * 64 + lane;
  const int nsub = 1 << up;
  // (the deferred form keeps both accumulator sets and the subtree's pending
  // values live across subtrees: with a partial last leaf that no longer fits
  // the 256 registers of two waves per SIMD; with BF16 3-leaf subtrees it fits
  // at 242 but measured 2% slower than the immediate form, while FP16's packed
  // values fit at 219 and made those launches 7% faster)
  constexpr bool kDefer = (NLH != 3 || std::is_same<T, F16>::value) && !TAIL;
  bool uniform = false;
  if constexpr (kDefer) uniform = w.phi - w.plo == (NLH << up);
  if constexpr (kDefer) {
  if (uniform) {
    // every lower subtree has NLH leaves: each one's last step runs beside the
    // next one's first MFMAs (the first subtree's leaf 0 finalises zeros,
    // which are dropped)
    f32x4 a0[kMmTN][kMmTM], a1[kMmTN][kMmTM];
    V st[2][NV];
#pragma unroll
    for (int tn = 0; tn < kMmTN; ++tn)
#pragma unroll
      for (int tm = 0; tm < kMmTM; ++tm) a0[tn][tm] = a1[tn][tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NV; ++q) st[0][q] = st[1][q] = V(0);
    for (int sidx = 0; sidx < nsub; ++sidx) {
      // root of subtree sidx - 1 into the top levels: merge with the pending
      // left subtrees its position closes, then park it (it is not the last)
      auto upper = [&](V (&rv)[NV]) {
        if (sidx == 0) return;
        int t = 0;
        for (; ((sidx - 1) >> t) & 1; ++t) merge<T>(upl, t, rv);
        park<T>(upl, t, rv);
      };
      const int j = w.plo + sidx * NLH;
      if constexpr ((NLH & 1) == 0) {
        w.template leaves_d<NLH, 0, 0>(j, r0, r1, a0, a1, v, st, upper);
      } else {
        // odd subtree sizes alternate the parity of their first leaf: two
        // subtrees per iteration, each of compile-time parity
        w.template leaves_d<NLH, 0, 0>(j, r0, r1, a0, a1, v, st, upper);
        if (sidx + 1 < nsub) {
          ++sidx;
          auto upper1 = [&](V (&rv)[NV]) {
            int t = 0;
            for (; ((sidx - 1) >> t) & 1; ++t) merge<T>(upl, t, rv);
            park<T>(upl, t, rv);
          };
          w.template leaves_d<NLH, 0, 1>(j + NLH, r0, r1, a0, a1, v, st, upper1);
        }
      }
    }
    // the last subtree's last step, then the top levels over its root
    if ((((NLH << up) - 1) & 1) == 0)
      w.round_leaf(a0, v);
    else
      w.round_leaf(a1, v);
    push_f<T, NLH, NLH - 1>(v, st);
    for (int t = 0; ((nsub - 1) >> t) & 1; ++t) merge<T>(upl, t, v);
  }
  }
  if (!uniform) {
  for (int sidx = 0; sidx < nsub; ++sidx) {
    int lo, hi;
    subtree_range(w.phi - w.plo, up, sidx, lo, hi);
    const int j = w.plo + lo;
    if (hi - lo == NLH)
      w.template lower_tree<NLH>(j, r0, r1, v);
    else if constexpr (NLH > 1)
      w.template lower_tree<NLH - 1>(j, r0, r1, v);
    // root sidx of the perfect tree over nsub roots: merge with the pending
    // left subtrees its position closes (trailing ones of sidx), then park it
    // at its level unless it is the last
    int t = 0;
    for (; (sidx >> t) & 1; ++t) merge<T>(upl, t, v);
    if (sidx + 1 < nsub) park<T>(upl, t, v);
  }
  }
  if (p.to_part)
    w.store_root(v, p.part + ((int64_t)b * (1 << kd) + piece) * p.part_stride, p.ldp);
  else
    w.store_root(v, p.C[b], p.ldc[b]);
}

}  // namespace

size_t mm_lds_bytes() { return 2 * kMmStage + (size_t)kMmWaves * 3 * kMmNP * 64 * 4; }

// Upper levels (<= 3) of a piece with Lp leaves such that every lower subtree
// holds at most kMmMaxNL leaves; -1 if the piece is too large.
int mm_upper_levels(int Lp) {
  for (int up = 0; up <= 3; ++up)
    if (((Lp + (1 << up) - 1) >> up) <= kMmMaxNL && (1 << up) <= Lp) return up;
  return -1;
}

// nlh: the largest lower-subtree size of the plan (1..kMmMaxNL); the others are nlh - 1.
template <class T>
hipError_t launch_mm_t(GemmParams p, int nb, int nlh, hipStream_t stream) {
  const int64_t tiles = ((p.M + kMmBM - 1) / kMmBM) * ((p.N + kMmBN - 1) / kMmBN);
  const dim3 grid((unsigned)tiles, 1u, (unsigned)(nb << p.ksplit_depth));
  const dim3 block(kMmWaves * 64);
  const size_t shm = mm_lds_bytes();
  const bool tail = p.K % kLeaf != 0;
  switch (nlh * 2 + (tail ? 1 : 0)) {
    case 2: dgf_launch(k_mm<T, 1, false>, grid, block, shm, stream, p); break;
    case 3: dgf_launch(k_mm<T, 1, true>, grid, block, shm, stream, p); break;
    case 4: dgf_launch(k_mm<T, 2, false>, grid, block, shm, stream, p); break;
    case 5: dgf_launch(k_mm<T, 2, true>, grid, block, shm, stream, p); break;
    case 6: dgf_launch(k_mm<T, 3, false>, grid, block, shm, stream, p); break;
    case 7: dgf_launch(k_mm<T, 3, true>, grid, block, shm, stream, p); break;
    case 8: dgf_launch(k_mm<T, 4, false>, grid, block, shm, stream, p); break;
    case 9: dgf_launch(k_mm<T, 4, true>, grid, block, shm, stream, p); break;
    default: return hipErrorInvalidValue;  // lower subtrees hold at most kMmMaxNL leaves
  }
  return hipGetLastError();
}

hipError_t launch_mm(GemmParams p, int nb, int nlh, hipStream_t stream) {
  if (p.fmt == FMT_F16) return launch_mm_t<F16>(p, nb, nlh, stream);
  return launch_mm_t<Bf16>(p, nb, nlh, stream);
}

}  // namespace dgf
