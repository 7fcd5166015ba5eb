// Device-side building blocks of the deterministic tree GEMMs (gfx950, wave64).
//
// The canonical reduction (RL-Kernel PR #325, section "Design"): K is cut into
// leaves of 64 contiguous elements; a leaf is accumulated in FP32 and rounded
// to the stored type; leaves are combined by the midpoint-split tree whose
// nodes add two stored children in FP32 and round to the stored type.  The
// stored type is BF16 or FP16 (one tree for both: PR #357, section
// "Determinism and correctness").  Here a leaf is two chained
// v_mfma_f32_16x16x32_{bf16,f16} instructions (K 0..31 then 32..63 of the
// leaf, starting from a zero accumulator): the matrix core consumes each lane
// group's 8 consecutive K values as one block, blocks in ascending K order,
// one FP32 rounding per block.  Tree nodes are evaluated in post order with a
// per-wave stack of pending left children indexed by depth; the leaf schedule
// depends only on (leaf count, leaf index), so it is wave-uniform and is
// computed on the scalar unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kLeaf = 64;

// ---------------------------------------------------------------- BF16 bits

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two FP32 values rounded to BF16 (nearest even) and packed, lo in bits 0..15
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two tree nodes at once: BF16 children added in FP32, rounded to BF16.
__device__ __forceinline__ uint32_t node2(uint32_t l, uint32_t r) {
  return pack_rne(bf_lo(l) + bf_lo(r), bf_hi(l) + bf_hi(r));
}

__device__ __forceinline__ __bf16 bf_zero() { return __builtin_bit_cast(__bf16, (uint16_t)0); }

// ---------------------------------------------------------------- stored types

// A stored 16-bit type: its MFMA operand (8 consecutive K values) and the
// 16x16x32 MFMA, the exact widening of a stored value to FP32 (alone, or the
// low / high half of a packed pair), nearest-even rounding of FP32 to the type
// (one value, or two packed with the first in bits 0..15), and, for the
// FP32-form tree of the tiled kernel, rounding that keeps the result as an FP32
// value (`rf`) and the packing of two values already representable (`pack_x`).
struct Bf16 {
  typedef bf16x8 frag;
  static constexpr int code = 0;
  static __device__ __forceinline__ float f(uint16_t h) { return bf2f(h); }
  static __device__ __forceinline__ float lo(uint32_t p) { return bf_lo(p); }
  static __device__ __forceinline__ float hi(uint32_t p) { return bf_hi(p); }
  static __device__ __forceinline__ uint16_t r(float x) { return f2bf(x); }
  static __device__ __forceinline__ uint32_t pack(float l, float h) { return pack_rne(l, h); }
  static __device__ __forceinline__ uint32_t pack_prod(float l, float h) { return pack_rne(l, h); }
  static __device__ __forceinline__ f32x4 mfma(const frag &a, const frag &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // the BF16 rounding of x as an FP32 value: one v_cvt_pk_bf16_f32 with a
  // zero low half leaves bf16(x) in the high half, i.e. the FP32 bits of it
  static __device__ __forceinline__ float rf(float x) {
    const f32x2 v = {0.f, x};
    return __builtin_bit_cast(float, __builtin_convertvector(v, bf16x2));
  }
  // two BF16 values held as FP32 (low halves zero) packed: their high halves
  static __device__ __forceinline__ uint32_t pack_x(float l, float h) {
    return __builtin_amdgcn_perm(__float_as_uint(h), __float_as_uint(l), 0x07060302u);
  }
};

struct F16 {
  typedef f16x8 frag;
  static constexpr int code = 1;
  static __device__ __forceinline__ float f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
  static __device__ __forceinline__ float lo(uint32_t p) { return f((uint16_t)p); }
  static __device__ __forceinline__ float hi(uint32_t p) { return f((uint16_t)(p >> 16)); }
  // r and pack_prod round an FP32 value that an FP32 multiply produced: the
  // empty asm keeps the rounding on its own.  Without it the compiler folds
  // the multiply into v_fma_mixlo_f16, which rounds the exact product to FP16
  // once (no FP32 rounding first) and adds +0, so that a -0 product comes out
  // as +0.  pack takes MFMA accumulators and node sums, where such a fold
  // cannot change the value (nothing to fold into an accumulator; a folded
  // add of two FP16 values rounds like the FP32 add then FP16: 24 >= 2*11+2
  // bits), and keeps the registers free.
  static __device__ __forceinline__ uint16_t r(float x) {
    asm volatile("" : "+v"(x));
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ uint32_t pack(float l, float h) {
    const f32x2 v = {l, h};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ uint32_t pack_prod(float l, float h) {
    asm volatile("" : "+v"(l), "+v"(h));
    return pack(l, h);
  }
  static __device__ __forceinline__ f32x4 mfma(const frag &a, const frag &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float rf(float x) { return (float)(_Float16)x; }
  // exact for values representable in FP16, so the rounding mode cannot matter
  static __device__ __forceinline__ uint32_t pack_x(float l, float h) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(l, h));
  }
};

// Two tree nodes at once in the stored type T.
template <class T>
__device__ __forceinline__ uint32_t node2t(uint32_t l, uint32_t r) {
  return T::pack(T::lo(l) + T::lo(r), T::hi(l) + T::hi(r));
}

// ---------------------------------------------------------------- tree schedule

// Leaf range [lo, hi) of subtree `idx` at depth `depth` of the midpoint tree
// over L leaves (idx's bits, most significant first, choose right halves).
__device__ __forceinline__ void subtree_range(int L, int depth, int idx, int &lo, int &hi) {
  lo = 0;
  hi = L;
  for (int b = depth - 1; b >= 0; --b) {
    int mid = lo + ((hi - lo) >> 1);
    if ((idx >> b) & 1) lo = mid; else hi = mid;
  }
}

// For leaf j of the midpoint tree over n leaves: its depth D and the number m
// of right-child steps that end its root-to-leaf path (the merges it triggers).
__device__ __forceinline__ void leaf_position(int n, int j, int &D, int &m) {
  int lo = 0, hi = n;
  D = 0;
  m = 0;
  while (hi - lo > 1) {
    int mid = lo + ((hi - lo) >> 1);
    if (j < mid) { hi = mid; m = 0; } else { lo = mid; ++m; }
    ++D;
  }
}

// Compile-time form of leaf_position: depth D of leaf j in the midpoint tree
// over n leaves and the number m of merges it triggers.
struct LeafPos {
  int D, m;
};
constexpr LeafPos leaf_pos(int n, int j) {
  int lo = 0, hi = n, D = 0, m = 0;
  while (hi - lo > 1) {
    const int mid = lo + (hi - lo) / 2;
    if (j < mid) {
      hi = mid;
      m = 0;
    } else {
      lo = mid;
      ++m;
    }
    ++D;
  }
  return LeafPos{D, m};
}

// Feed leaf J of an N-leaf subtree (N <= 8, so depth <= 3): merge it with the
// pending left siblings its position closes, then park it at its depth; after
// the last leaf v is the subtree root.
template <class T, int NP, int N, int J>
__device__ __forceinline__ void push_leaf(uint32_t (&v)[NP], uint32_t (&st)[3][NP]) {
  constexpr LeafPos lp = leaf_pos(N, J);
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

// Pending left children of a wave's subtree, slot d-1 holding depth d, kept in
// the wave's own LDS region: slot d, pair p of lane l at base[(d*NP + p)*64 + l].
// Each lane reads back only what it wrote itself, so no cross-lane ordering is
// needed, and consecutive lanes touch consecutive dwords (no bank conflicts).
template <int NP>
struct TreeStack {
  uint32_t *base;  // this wave's region, already offset by the lane

  __device__ __forceinline__ void get(int d, uint32_t (&o)[NP]) const {
#pragma unroll
    for (int p = 0; p < NP; ++p) o[p] = base[(d * NP + p) * 64];
  }
  __device__ __forceinline__ void set(int d, const uint32_t (&v)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) base[(d * NP + p) * 64] = v[p];
  }
};

// Feed leaf j (stored values v) of an n-leaf subtree: merge it with the
// pending left siblings its position closes, then park the result at its
// depth, or make it the root.
template <class T, int NP>
__device__ __forceinline__ void tree_push(TreeStack<NP> &st, uint32_t (&v)[NP], uint32_t (&root)[NP], int n, int j) {
  int D, m;
  leaf_position(n, j, D, m);
  D = __builtin_amdgcn_readfirstlane(D);
  m = __builtin_amdgcn_readfirstlane(m);
  for (int t = 0; t < m; ++t) {
    uint32_t l[NP];
    st.get(D - 1 - t, l);
#pragma unroll
    for (int p = 0; p < NP; ++p) v[p] = node2t<T>(l[p], v[p]);
  }
  const int d = D - m;
  if (d > 0) {
    st.set(d - 1, v);
  } else {
#pragma unroll
    for (int p = 0; p < NP; ++p) root[p] = v[p];
  }
}

// Balanced combine of W (power of two) roots: the midpoint tree over W parts.
template <class T, int NP, int W>
__device__ __forceinline__ void combine_roots(uint32_t (&r)[W][NP]) {
#pragma unroll
  for (int width = W; width > 1; width >>= 1) {
#pragma unroll
    for (int i = 0; i < width / 2; ++i)
#pragma unroll
      for (int p = 0; p < NP; ++p) r[i][p] = node2t<T>(r[2 * i][p], r[2 * i + 1][p]);
  }
}

// ---------------------------------------------------------------- fragments

// 8 consecutive stored values row[k..k+8) as an MFMA operand (16-byte
// aligned: aligned base, leading dimension a multiple of 8, k a multiple of 8).
template <class T>
__device__ __forceinline__ typename T::frag load_frag(const uint16_t *row, int64_t k) {
  return *reinterpret_cast<const typename T::frag *>(row + k);
}

// The same with zeros past K (the last, partial leaf only).
template <class T>
__device__ __forceinline__ typename T::frag load_frag_tail(const uint16_t *row, int64_t k, int64_t K) {
  if (k + 8 <= K) return *reinterpret_cast<const typename T::frag *>(row + k);
  u16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (k + i < K) ? row[k + i] : (uint16_t)0;
  return __builtin_bit_cast(typename T::frag, z);
}

// ---------------------------------------------------------------- activation

// sigma(g) = 1 / (1 + e), e = exp(-g) rounded once to FP32 (evaluated in
// double, then rounded), every FP32 operation separately rounded.
__device__ __forceinline__ float sigma_f(float g) {
  float e = (float)exp(-(double)g);
  float den = 1.0f + e;
  return 1.0f / den;
}

// Orders this wave's LDS accesses (compiler and hardware) without a
// workgroup barrier: waves of a workgroup run different leaf counts.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Tile index remap so that consecutive tiles share an XCD: blocks are dealt to
// the 8 XCDs round robin, so block b runs on XCD b % 8; tile = (b % 8) * per + b / 8.
__device__ __forceinline__ int xcd_tile(int b, int ntiles) {
  const int per = (ntiles + 7) >> 3;
  const int full = ntiles - (per - 1) * 8;  // XCDs that get `per` tiles
  const int x = b & 7, q = b >> 3;
  // XCD x owns the contiguous tiles [start(x), start(x) + count(x))
  const int start = x < full ? x * per : full * per + (x - full) * (per - 1);
  return start + q;
}

}  // namespace dgf
