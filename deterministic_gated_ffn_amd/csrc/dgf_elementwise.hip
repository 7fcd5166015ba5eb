// Elementwise kernels: the activation and its derivative, the fixed balanced
// combine of S partial results, and a 16-bit transpose.  T is the stored type
// (BF16 or FP16): values are widened to FP32 exactly and each result is rounded
// to T once (nearest even).
#include "dgf_device.hpp"
#include "dgf_kernels.hpp"
#include "dgf_join.hpp"

namespace dgf {

namespace {

constexpr int kThreads = 256;

unsigned grid_for(int64_t work, int per_thread) {
  int64_t blocks = (work + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (blocks > 65536) blocks = 65536;  // grid-stride loops cover the rest
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

// a = rnd(silu(g) u), silu(g) = g * sigma(g)
template <class T>
__global__ __launch_bounds__(kThreads) void k_act_fwd(const uint16_t *g, const uint16_t *u, uint16_t *a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float gv = T::f(g[i]);
    const float s = gv * sigma_f(gv);
    a[i] = T::r(s * T::f(u[i]));
  }
}

// dU = rnd(dA silu(g)), dG = rnd((dA u) silu'(g)), silu' = sigma (1 + g (1 - sigma))
template <class T>
__global__ __launch_bounds__(kThreads) void k_act_bwd(const uint16_t *da, const uint16_t *g, const uint16_t *u,
                                                      uint16_t *dg, uint16_t *du, uint16_t *a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float gv = T::f(g[i]), uv = T::f(u[i]), dav = T::f(da[i]);
    const float sg = sigma_f(gv);
    const float s = gv * sg;
    const float one_m = 1.0f - sg;
    const float t = gv * one_m;
    const float onep = 1.0f + t;
    const float ds = sg * onep;
    du[i] = T::r(dav * s);
    const float dau = dav * uv;
    dg[i] = T::r(dau * ds);
    if (a) a[i] = T::r(s * uv);
  }
}

template <class T, int S, int EPI>
__global__ __launch_bounds__(kThreads) void k_combine_epi(GemmParams p) {
  const int64_t chunks = (p.N + 7) / 8;
  const int b = blockIdx.y;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < p.M * chunks; i += (int64_t)gridDim.x * kThreads) {
    const int64_t m = i / chunks, c = (i % chunks) * 8;
    join_epi_chunk<T, S, EPI>(p, b, m, c);
  }
}

struct Parts {
  const uint16_t *p[8];
};

// Balanced combine over S parts, 8 elements per thread with 16-byte accesses.
template <int S>
__global__ __launch_bounds__(kThreads) void k_combine_vec(Parts parts, uint16_t *out, int64_t nvec) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    uint32_t r[S][4];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint4 v = reinterpret_cast<const uint4 *>(parts.p[s])[i];
      r[s][0] = v.x; r[s][1] = v.y; r[s][2] = v.z; r[s][3] = v.w;
    }
#pragma unroll
    for (int width = S; width > 1; width >>= 1)
#pragma unroll
      for (int j = 0; j < width / 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) r[j][q] = node2(r[2 * j][q], r[2 * j + 1][q]);
    reinterpret_cast<uint4 *>(out)[i] = make_uint4(r[0][0], r[0][1], r[0][2], r[0][3]);
  }
}

// The same arithmetic one element at a time (unaligned or offset views, tails).
template <int S>
__global__ __launch_bounds__(kThreads) void k_combine_scalar(Parts parts, uint16_t *out, int64_t begin, int64_t n) {
  for (int64_t i = begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    float r[S];
#pragma unroll
    for (int s = 0; s < S; ++s) r[s] = bf2f(parts.p[s][i]);
#pragma unroll
    for (int width = S; width > 1; width >>= 1)
#pragma unroll
      for (int j = 0; j < width / 2; ++j) r[j] = bf2f(f2bf(r[2 * j] + r[2 * j + 1]));
    out[i] = f2bf(r[0]);
  }
}

// FP16 and FP32 parts: the same balanced rank tree; an FP16 node adds its two
// children in FP32 and rounds the sum to FP16 (nearest even), an FP32 node is
// one FP32 addition (PR #357, "Determinism and correctness").
template <int DT>
struct CElem;
template <>
struct CElem<DGF_COMBINE_FP16> {
  using T = uint16_t;
  static constexpr int PER16 = 8;
  static __device__ __forceinline__ float ld(T v) { return (float)__builtin_bit_cast(_Float16, v); }
  static __device__ __forceinline__ T rnd(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
};
template <>
struct CElem<DGF_COMBINE_FP32> {
  using T = float;
  static constexpr int PER16 = 4;
  static __device__ __forceinline__ float ld(T v) { return v; }
  static __device__ __forceinline__ T rnd(float f) { return f; }
};

struct PartsV {
  const void *p[8];
};

template <int S, int DT>
__device__ __forceinline__ typename CElem<DT>::T combine_el(const PartsV &parts, int64_t i) {
  using E = CElem<DT>;
  float r[S];
#pragma unroll
  for (int s = 0; s < S; ++s) r[s] = E::ld(reinterpret_cast<const typename E::T *>(parts.p[s])[i]);
#pragma unroll
  for (int width = S; width > 1; width >>= 1)
#pragma unroll
    for (int j = 0; j < width / 2; ++j) r[j] = E::ld(E::rnd(r[2 * j] + r[2 * j + 1]));
  return E::rnd(r[0]);
}

// 16 bytes per thread and part (8 FP16 or 4 FP32 elements).
template <int S, int DT>
__global__ __launch_bounds__(kThreads) void k_combine_vec_t(PartsV parts, void *out, int64_t nvec) {
  using E = CElem<DT>;
  constexpr int P = E::PER16;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    float r[S][P];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint4 v = reinterpret_cast<const uint4 *>(parts.p[s])[i];
      typename E::T el[P];
      __builtin_memcpy(el, &v, 16);
#pragma unroll
      for (int e = 0; e < P; ++e) r[s][e] = E::ld(el[e]);
    }
#pragma unroll
    for (int width = S; width > 1; width >>= 1)
#pragma unroll
      for (int j = 0; j < width / 2; ++j)
#pragma unroll
        for (int e = 0; e < P; ++e) r[j][e] = E::ld(E::rnd(r[2 * j][e] + r[2 * j + 1][e]));
    typename E::T o[P];
#pragma unroll
    for (int e = 0; e < P; ++e) o[e] = E::rnd(r[0][e]);
    uint4 v;
    __builtin_memcpy(&v, o, 16);
    reinterpret_cast<uint4 *>(out)[i] = v;
  }
}

template <int S, int DT>
__global__ __launch_bounds__(kThreads) void k_combine_scalar_t(PartsV parts, void *out, int64_t begin, int64_t n) {
  for (int64_t i = begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    reinterpret_cast<typename CElem<DT>::T *>(out)[i] = combine_el<S, DT>(parts, i);
}

// out[m][n] = balanced combine over S partial roots (the top levels of the
// tree above the workgroups' K pieces); 8 elements per thread.
template <class T, int S>
__global__ __launch_bounds__(kThreads) void k_combine_2d(const uint16_t *part, int64_t part_stride, int64_t ldp,
                                                         uint16_t *out, int64_t ldo, int64_t M, int64_t N) {
  const int64_t per_row = (N + 7) / 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < M * per_row; i += (int64_t)gridDim.x * kThreads) {
    const int64_t m = i / per_row, c = (i % per_row) * 8;
    uint16_t *o = out + m * ldo + c;
    if (c + 8 <= N) {
      uint32_t r[S][4];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint4 v = *reinterpret_cast<const uint4 *>(part + s * part_stride + m * ldp + c);
        r[s][0] = v.x; r[s][1] = v.y; r[s][2] = v.z; r[s][3] = v.w;
      }
#pragma unroll
      for (int width = S; width > 1; width >>= 1)
#pragma unroll
        for (int j = 0; j < width / 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) r[j][q] = node2t<T>(r[2 * j][q], r[2 * j + 1][q]);
      *reinterpret_cast<uint4 *>(o) = make_uint4(r[0][0], r[0][1], r[0][2], r[0][3]);
    } else {
      for (int64_t e = 0; c + e < N; ++e) {
        float r[S];
#pragma unroll
        for (int s = 0; s < S; ++s) r[s] = T::f(part[s * part_stride + m * ldp + c + e]);
#pragma unroll
        for (int width = S; width > 1; width >>= 1)
#pragma unroll
          for (int j = 0; j < width / 2; ++j) r[j] = T::f(T::r(r[2 * j] + r[2 * j + 1]));
        o[e] = T::r(r[0]);
      }
    }
  }
}

// dx = rnd(G + U), the gate contribution first (an FP32 add of two stored
// lanes, rounded to the stored type); 8 elements per thread, rows of N (a
// multiple of 8 leading dims).
template <class T>
__global__ __launch_bounds__(kThreads) void k_add_lanes(const uint16_t *G, int64_t ldg, const uint16_t *U, int64_t ldu,
                                                        uint16_t *dx, int64_t lddx, int64_t M, int64_t N) {
  const int64_t per_row = (N + 7) / 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < M * per_row; i += (int64_t)gridDim.x * kThreads) {
    const int64_t m = i / per_row, c = (i % per_row) * 8;
    const uint16_t *g = G + m * ldg + c, *u = U + m * ldu + c;
    uint16_t *o = dx + m * lddx + c;
    if (c + 8 <= N) {
      const uint4 gv = *reinterpret_cast<const uint4 *>(g), uv = *reinterpret_cast<const uint4 *>(u);
      *reinterpret_cast<uint4 *>(o) =
          make_uint4(node2t<T>(gv.x, uv.x), node2t<T>(gv.y, uv.y), node2t<T>(gv.z, uv.z), node2t<T>(gv.w, uv.w));
    } else {
      for (int64_t j = 0; c + j < N; ++j) o[j] = T::r(T::f(g[j]) + T::f(u[j]));
    }
  }
}

// dst [C, R] = src [R, C]^T through a 64 x 64 LDS tile.
// dst [C, R] = transpose of src [R, C] in 64 x 64 tiles through LDS: 16-byte
// row-segment loads and 16-byte column-segment stores (8 threads cover one
// 128-byte segment), element by element only at ragged edges.  Both leading
// dimensions are multiples of 8 elements and both bases 16-byte aligned.
__global__ __launch_bounds__(kThreads) void k_transpose(const uint16_t *src, int64_t lds_, int64_t R, int64_t C,
                                                        uint16_t *dst, int64_t ldd) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // 144-byte rows: 16-byte aligned chunks
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int t8 = threadIdx.x >> 3, cc = threadIdx.x & 7;
  for (int j = 0; j < 64; j += kThreads / 8) {
    const int r = t8 + j;
    const int64_t gr = r0 + r, gc = c0 + 8 * cc;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (gr < R && gc + 8 <= C) {
      v = *reinterpret_cast<const uint4 *>(src + gr * lds_ + gc);
    } else if (gr < R) {
      uint16_t h[8];
      for (int e = 0; e < 8; ++e) h[e] = gc + e < C ? src[gr * lds_ + gc + e] : (uint16_t)0;
      v = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16), h[4] | ((uint32_t)h[5] << 16),
                     h[6] | ((uint32_t)h[7] << 16));
    }
    *reinterpret_cast<uint4 *>(&tile[r][8 * cc]) = v;
  }
  __syncthreads();
  for (int j = 0; j < 64; j += kThreads / 8) {
    const int oc = t8 + j;  // source column = destination row within the tile
    const int64_t drow = c0 + oc, dcol = r0 + 8 * cc;
    if (drow >= C) continue;
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = tile[8 * cc + e][oc];
    if (dcol + 8 <= R) {
      *reinterpret_cast<uint4 *>(dst + drow * ldd + dcol) =
          make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16), h[4] | ((uint32_t)h[5] << 16),
                     h[6] | ((uint32_t)h[7] << 16));
    } else {
      for (int e = 0; dcol + e < R; ++e) dst[drow * ldd + dcol + e] = h[e];
    }
  }
}

}  // namespace

hipError_t launch_act_fwd(int fmt, const uint16_t *g, const uint16_t *u, uint16_t *a, int64_t n, hipStream_t s) {
  if (fmt == FMT_F16)
    dgf_launch(k_act_fwd<F16>, dim3(grid_for(n, 1)), dim3(kThreads), 0, s, g, u, a, n);
  else
    dgf_launch(k_act_fwd<Bf16>, dim3(grid_for(n, 1)), dim3(kThreads), 0, s, g, u, a, n);
  return hipGetLastError();
}

hipError_t launch_act_bwd(int fmt, const uint16_t *da, const uint16_t *g, const uint16_t *u, uint16_t *dg,
                          uint16_t *du, uint16_t *a, int64_t n, hipStream_t s) {
  if (fmt == FMT_F16)
    dgf_launch(k_act_bwd<F16>, dim3(grid_for(n, 1)), dim3(kThreads), 0, s, da, g, u, dg, du, a, n);
  else
    dgf_launch(k_act_bwd<Bf16>, dim3(grid_for(n, 1)), dim3(kThreads), 0, s, da, g, u, dg, du, a, n);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t *const *parts, int S, uint16_t *out, int64_t n, hipStream_t s) {
  Parts P{};
  bool aligned = ((uintptr_t)out & 15) == 0;
  for (int i = 0; i < S; ++i) {
    P.p[i] = parts[i];
    aligned = aligned && (((uintptr_t)parts[i] & 15) == 0);
  }
  const int64_t nvec = aligned ? n / 8 : 0;
  if (nvec > 0) {
    const dim3 g(grid_for(nvec, 1));
    switch (S) {
      case 1: dgf_launch(k_combine_vec<1>, g, dim3(kThreads), 0, s, P, out, nvec); break;
      case 2: dgf_launch(k_combine_vec<2>, g, dim3(kThreads), 0, s, P, out, nvec); break;
      case 4: dgf_launch(k_combine_vec<4>, g, dim3(kThreads), 0, s, P, out, nvec); break;
      default: dgf_launch(k_combine_vec<8>, g, dim3(kThreads), 0, s, P, out, nvec); break;
    }
  }
  const int64_t begin = nvec * 8;
  if (begin < n) {
    const dim3 g(grid_for(n - begin, 1));
    switch (S) {
      case 1: dgf_launch(k_combine_scalar<1>, g, dim3(kThreads), 0, s, P, out, begin, n); break;
      case 2: dgf_launch(k_combine_scalar<2>, g, dim3(kThreads), 0, s, P, out, begin, n); break;
      case 4: dgf_launch(k_combine_scalar<4>, g, dim3(kThreads), 0, s, P, out, begin, n); break;
      default: dgf_launch(k_combine_scalar<8>, g, dim3(kThreads), 0, s, P, out, begin, n); break;
    }
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_combine_t(const void *const *parts, int S, void *out, int64_t n, hipStream_t s) {
  constexpr int P = CElem<DT>::PER16;
  PartsV pv{};
  bool aligned = ((uintptr_t)out & 15) == 0;
  for (int i = 0; i < S; ++i) {
    pv.p[i] = parts[i];
    aligned = aligned && (((uintptr_t)parts[i] & 15) == 0);
  }
  const int64_t nvec = aligned ? n / P : 0;
  if (nvec > 0) {
    const dim3 g(grid_for(nvec, 1));
    switch (S) {
      case 1: dgf_launch((k_combine_vec_t<1, DT>), g, dim3(kThreads), 0, s, pv, out, nvec); break;
      case 2: dgf_launch((k_combine_vec_t<2, DT>), g, dim3(kThreads), 0, s, pv, out, nvec); break;
      case 4: dgf_launch((k_combine_vec_t<4, DT>), g, dim3(kThreads), 0, s, pv, out, nvec); break;
      default: dgf_launch((k_combine_vec_t<8, DT>), g, dim3(kThreads), 0, s, pv, out, nvec); break;
    }
  }
  const int64_t begin = nvec * P;
  if (begin < n) {
    const dim3 g(grid_for(n - begin, 1));
    switch (S) {
      case 1: dgf_launch((k_combine_scalar_t<1, DT>), g, dim3(kThreads), 0, s, pv, out, begin, n); break;
      case 2: dgf_launch((k_combine_scalar_t<2, DT>), g, dim3(kThreads), 0, s, pv, out, begin, n); break;
      case 4: dgf_launch((k_combine_scalar_t<4, DT>), g, dim3(kThreads), 0, s, pv, out, begin, n); break;
      default: dgf_launch((k_combine_scalar_t<8, DT>), g, dim3(kThreads), 0, s, pv, out, begin, n); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_combine_typed(const void *const *parts, int S, void *out, int64_t n, int dtype, hipStream_t s) {
  switch (dtype) {
    case DGF_COMBINE_BF16: return launch_combine((const uint16_t *const *)parts, S, (uint16_t *)out, n, s);
    case DGF_COMBINE_FP16: return launch_combine_t<DGF_COMBINE_FP16>(parts, S, out, n, s);
    case DGF_COMBINE_FP32: return launch_combine_t<DGF_COMBINE_FP32>(parts, S, out, n, s);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
hipError_t launch_combine_2d_t(const uint16_t *part, int64_t part_stride, int64_t ldp, int S, uint16_t *out,
                               int64_t ldo, int64_t M, int64_t N, hipStream_t s) {
  const dim3 g(grid_for(M * ((N + 7) / 8), 1));
  switch (S) {
    case 1: dgf_launch((k_combine_2d<T, 1>), g, dim3(kThreads), 0, s, part, part_stride, ldp, out, ldo, M, N); break;
    case 2: dgf_launch((k_combine_2d<T, 2>), g, dim3(kThreads), 0, s, part, part_stride, ldp, out, ldo, M, N); break;
    case 4: dgf_launch((k_combine_2d<T, 4>), g, dim3(kThreads), 0, s, part, part_stride, ldp, out, ldo, M, N); break;
    case 8: dgf_launch((k_combine_2d<T, 8>), g, dim3(kThreads), 0, s, part, part_stride, ldp, out, ldo, M, N); break;
    case 16: dgf_launch((k_combine_2d<T, 16>), g, dim3(kThreads), 0, s, part, part_stride, ldp, out, ldo, M, N); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine_2d(int fmt, const uint16_t *part, int64_t part_stride, int64_t ldp, int S, uint16_t *out,
                             int64_t ldo, int64_t M, int64_t N, hipStream_t s) {
  if (fmt == FMT_F16) return launch_combine_2d_t<F16>(part, part_stride, ldp, S, out, ldo, M, N, s);
  return launch_combine_2d_t<Bf16>(part, part_stride, ldp, S, out, ldo, M, N, s);
}

hipError_t launch_add_lanes(int fmt, const uint16_t *G, int64_t ldg, const uint16_t *U, int64_t ldu, uint16_t *dx,
                            int64_t lddx, int64_t M, int64_t N, hipStream_t s) {
  const dim3 g(grid_for(M * ((N + 7) / 8), 1));
  if (fmt == FMT_F16)
    dgf_launch(k_add_lanes<F16>, g, dim3(kThreads), 0, s, G, ldg, U, ldu, dx, lddx, M, N);
  else
    dgf_launch(k_add_lanes<Bf16>, g, dim3(kThreads), 0, s, G, ldg, U, ldu, dx, lddx, M, N);
  return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t *src, int64_t lds_, int64_t R, int64_t C, uint16_t *dst, int64_t ldd,
                            hipStream_t s) {
  const dim3 g((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  dgf_launch(k_transpose, g, dim3(kThreads), 0, s, src, lds_, R, C, dst, ldd);
  return hipGetLastError();
}


template <class T, int EPI>
hipError_t launch_combine_epi_s(int S, int nb, GemmParams p, hipStream_t s) {
  const dim3 g(grid_for(p.M * ((p.N + 7) / 8), 1), EPI == EPI_STORE ? nb : 1);
  switch (S) {
    case 1: dgf_launch((k_combine_epi<T, 1, EPI>), g, dim3(kThreads), 0, s, p); break;
    case 2: dgf_launch((k_combine_epi<T, 2, EPI>), g, dim3(kThreads), 0, s, p); break;
    case 4: dgf_launch((k_combine_epi<T, 4, EPI>), g, dim3(kThreads), 0, s, p); break;
    case 8: dgf_launch((k_combine_epi<T, 8, EPI>), g, dim3(kThreads), 0, s, p); break;
    case 16: dgf_launch((k_combine_epi<T, 16, EPI>), g, dim3(kThreads), 0, s, p); break;
    case 32: dgf_launch((k_combine_epi<T, 32, EPI>), g, dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class T>
hipError_t launch_combine_epi_t(int epi, int nb, GemmParams p, hipStream_t s) {
  const int S = 1 << p.ksplit_depth;
  switch (epi) {
    case EPI_STORE: return launch_combine_epi_s<T, EPI_STORE>(S, nb, p, s);
    case EPI_ACT: return launch_combine_epi_s<T, EPI_ACT>(S, nb, p, s);
    case EPI_DSILU: return launch_combine_epi_s<T, EPI_DSILU>(S, nb, p, s);
    case EPI_DX: return launch_combine_epi_s<T, EPI_DX>(S, nb, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine_epi(int epi, int nb, GemmParams p, hipStream_t s) {
  if (p.fmt == FMT_F16) return launch_combine_epi_t<F16>(epi, nb, p, s);
  return launch_combine_epi_t<Bf16>(epi, nb, p, s);
}

}  // namespace dgf
