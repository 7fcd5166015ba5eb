// Deterministic tree GEMMs for gfx950.
//
// One workgroup owns a tile of 16 output columns n (weight rows in the NT form)
// and 16*MT output rows m (tokens).  Its WAVES waves split the K leaves into
// the WAVES subtrees at depth log2(WAVES) of the canonical midpoint tree; each
// wave runs its subtree in post order, then wave 0 combines the WAVES roots
// through LDS with the balanced top of the tree (RL-Kernel PR #325, section
// "Design": contiguous K pieces are subtrees of the one canonical tree).
//
// MFMA roles: A operand = 16 weight rows x 32 K, B operand = 32 K x 16 tokens,
// so lane l ends with D[4(l/16)+r][l%16]: four consecutive output columns of
// one token, which the epilogues store as 8 contiguous bytes.
#include "dgf_device.hpp"
#include "dgf_kernels.hpp"

namespace dgf {

// ------------------------------------------------------------------ shared tail

// Every wave parks its subtree root in slot 0 of its own stack region; wave 0
// then combines the WAVES roots with the balanced top of the tree.
template <int NP, int WAVES>
__device__ __forceinline__ bool wg_combine(uint32_t (&root)[NP], uint32_t *stack_lds, int stack_words, int wave,
                                           int lane) {
  if constexpr (WAVES == 1) {
    return true;
  } else {
#pragma unroll
    for (int p = 0; p < NP; ++p) stack_lds[wave * stack_words + p * 64 + lane] = root[p];
    __syncthreads();
    if (wave != 0) return false;
    uint32_t r[WAVES][NP];
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
#pragma unroll
      for (int p = 0; p < NP; ++p) r[w][p] = stack_lds[w * stack_words + p * 64 + lane];
    combine_roots<NP, WAVES>(r);
#pragma unroll
    for (int p = 0; p < NP; ++p) root[p] = r[0][p];
    return true;
  }
}

// Store 4 consecutive BF16 (two packed pairs) at C[m][n..n+3], bounds-checked.
__device__ __forceinline__ void store4(uint16_t *C, int64_t ldc, int64_t m, int64_t n, int64_t M, int64_t N,
                                       uint32_t p0, uint32_t p1) {
  if (m >= M) return;
  uint16_t *dst = C + m * ldc + n;
  if (n + 3 < N) {
    uint2 v = make_uint2(p0, p1);
    *reinterpret_cast<uint2 *>(dst) = v;
  } else {
    const uint16_t h[4] = {(uint16_t)(p0 & 0xffff), (uint16_t)(p0 >> 16), (uint16_t)(p1 & 0xffff), (uint16_t)(p1 >> 16)};
    for (int i = 0; i < 4; ++i)
      if (n + i < N) dst[i] = h[i];
  }
}

// ------------------------------------------------------------------ NT

// C_b[m][n] = T_K( A_b[m,:] . B_b[n,:] ), b < NB; A_b [M,K] and B_b [N,K] both
// K-contiguous.
template <int NB, int MT, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_nt(GemmParams p) {
  // gate and up share the activation operand
  constexpr bool SHARED_A = (EPI == EPI_ACT);
  constexpr int NP = NB * MT * 2;
  constexpr int DEPTH = WAVES == 1 ? 0 : WAVES == 2 ? 1 : WAVES == 4 ? 2 : 3;
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
  const int stack_words = p.stack_slots * NP * 64;  // per wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * 16;
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
  const int r16 = lane & 15, g4 = lane >> 4;

  int lo, hi;
  subtree_range(p.L, DEPTH, wave, lo, hi);
  const int nl = hi - lo;

  // Rows past N and tokens past M read a valid row instead (clamped); their
  // MFMA outputs are never stored, and every output depends only on its own
  // weight row and token.
  const uint16_t *brow[NB];
  const uint16_t *arow[NB][MT];
  {
    const int64_t n = n0 + r16 < p.N ? n0 + r16 : p.N - 1;
#pragma unroll
    for (int b = 0; b < NB; ++b) brow[b] = p.B[b] + n * p.ldb[b];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + 16 * t + r16 < p.M ? m0 + 16 * t + r16 : p.M - 1;
#pragma unroll
    for (int b = 0; b < NB; ++b) arow[b][t] = p.A[b] + m * p.lda[b];
  }

  TreeStack<NP> st{dyn_lds + wave * stack_words + lane};
  uint32_t root[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) root[q] = 0;

  for (int j = 0; j < nl; ++j) {
    const int64_t kb = (int64_t)(lo + j) * kLeaf;
    f32x4 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb + kLeaf <= p.K) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t k = kb + 32 * s + 8 * g4;
        bf16x8 wf[NB], xf[NB][MT];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          wf[b] = load_frag(brow[b], k);
#pragma unroll
          for (int t = 0; t < MT; ++t) xf[b][t] = (b > 0 && SHARED_A) ? xf[0][t] : load_frag(arow[b][t], k);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[b][t] = mfma16(wf[b], xf[b][t], acc[b][t]);
      }
    } else {
      // the partial last leaf: zeros past K; an all-zero block leaves the
      // accumulator unchanged, so a half past K is skipped
      for (int s = 0; s < 2; ++s) {
        if (kb + 32 * s >= p.K) break;
        const int64_t k = kb + 32 * s + 8 * g4;
        bf16x8 wf[NB], xf[NB][MT];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          wf[b] = load_frag_tail(brow[b], k, p.K);
#pragma unroll
          for (int t = 0; t < MT; ++t) xf[b][t] = load_frag_tail(arow[b][t], k, p.K);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[b][t] = mfma16(wf[b], xf[b][t], acc[b][t]);
      }
    }
    uint32_t v[NP];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        v[(b * MT + t) * 2 + 0] = pack_rne(acc[b][t][0], acc[b][t][1]);
        v[(b * MT + t) * 2 + 1] = pack_rne(acc[b][t][2], acc[b][t][3]);
      }
    tree_push<NP>(st, v, root, nl, j);
  }

  if (!wg_combine<NP, WAVES>(root, dyn_lds, stack_words, wave, lane)) return;

  const int64_t n = n0 + 4 * g4;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + 16 * t + r16;
    if constexpr (EPI == EPI_STORE) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        store4(p.C[b], p.ldc[b], m, n, p.M, p.N, root[(b * MT + t) * 2], root[(b * MT + t) * 2 + 1]);
    } else if constexpr (EPI == EPI_ACT) {
      // gate (b = 0) and up (b = 1) of the same (m, n): a = bf16(silu(g) u)
      uint32_t ap[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t gp = root[(0 * MT + t) * 2 + h], up = root[(1 * MT + t) * 2 + h];
        float a2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float g = e ? bf_hi(gp) : bf_lo(gp);
          const float u = e ? bf_hi(up) : bf_lo(up);
          const float s = g * sigma_f(g);
          a2[e] = s * u;
        }
        ap[h] = pack_rne(a2[0], a2[1]);
      }
      store4(p.act_out, p.ld_act, m, n, p.M, p.N, ap[0], ap[1]);
      if (p.C[0]) store4(p.C[0], p.ldc[0], m, n, p.M, p.N, root[(0 * MT + t) * 2], root[(0 * MT + t) * 2 + 1]);
      if (p.C[1]) store4(p.C[1], p.ldc[1], m, n, p.M, p.N, root[(1 * MT + t) * 2], root[(1 * MT + t) * 2 + 1]);
    }
  }
}

// ------------------------------------------------------------------ NN

// C_b[m][n] = T_K( A_b[m,:] . B_b[:,n] ); A_b [M,K] K-contiguous, B_b [K,N]
// N-contiguous.  Each wave transposes its 64 x 16 weight slab of every leaf
// through its own LDS region so that the MFMA A operand is K-contiguous.
constexpr int kTStride = 72;  // padded K stride of a transposed slab (elements)

template <int NB, int MT, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_nn(GemmParams p) {
  constexpr int NP = NB * MT * 2;
  constexpr int DEPTH = WAVES == 1 ? 0 : WAVES == 2 ? 1 : WAVES == 4 ? 2 : 3;
  __shared__ __attribute__((aligned(16))) uint16_t slab[WAVES][NB][16 * kTStride];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
  const int stack_words = p.stack_slots * NP * 64;  // per wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * 16;
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
  const int r16 = lane & 15, g4 = lane >> 4;

  int lo, hi;
  subtree_range(p.L, DEPTH, wave, lo, hi);
  const int nl = hi - lo;

  const uint16_t *arow[NB][MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + 16 * t + r16 < p.M ? m0 + 16 * t + r16 : p.M - 1;  // clamped, never stored
#pragma unroll
    for (int b = 0; b < NB; ++b) arow[b][t] = p.A[b] + m * p.lda[b];
  }
  const bool full_n = n0 + 16 <= p.N;

  TreeStack<NP> st{dyn_lds + wave * stack_words + lane};
  uint32_t root[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) root[q] = 0;

  for (int j = 0; j < nl; ++j) {
    const int64_t kb = (int64_t)(lo + j) * kLeaf;
    const bool full_leaf = kb + kLeaf <= p.K;
    // lane l stages weight row kb + l, columns n0..n0+15, as slab[n][l]
    const int64_t kr = kb + lane;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint32_t q[8];
      if (full_leaf && full_n) {
        const uint16_t *src = p.B[b] + kr * p.ldb[b] + n0;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(src);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(src + 8);
        q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
        q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
      } else {
        const bool kok = kr < p.K;
        const uint16_t *src = p.B[b] + (kok ? kr : 0) * p.ldb[b] + n0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t lo16 = (kok && n0 + 2 * i < p.N) ? src[2 * i] : 0u;
          const uint32_t hi16 = (kok && n0 + 2 * i + 1 < p.N) ? src[2 * i + 1] : 0u;
          q[i] = lo16 | (hi16 << 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        slab[wave][b][(2 * i) * kTStride + lane] = (uint16_t)(q[i] & 0xffff);
        slab[wave][b][(2 * i + 1) * kTStride + lane] = (uint16_t)(q[i] >> 16);
      }
    }
    wave_lds_sync();  // this wave's slab writes land before its lanes read them

    f32x4 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (!full_leaf && kb + 32 * s >= p.K) break;  // all-zero block: accumulator unchanged
      const int64_t k = kb + 32 * s + 8 * g4;
      bf16x8 wf[NB], xf[NB][MT];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        wf[b] = *reinterpret_cast<const bf16x8 *>(&slab[wave][b][r16 * kTStride + 32 * s + 8 * g4]);
#pragma unroll
        for (int t = 0; t < MT; ++t) xf[b][t] = full_leaf ? load_frag(arow[b][t], k) : load_frag_tail(arow[b][t], k, p.K);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[b][t] = mfma16(wf[b], xf[b][t], acc[b][t]);
    }
    wave_lds_sync();  // slab reads done before the next leaf overwrites it

    uint32_t v[NP];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        v[(b * MT + t) * 2 + 0] = pack_rne(acc[b][t][0], acc[b][t][1]);
        v[(b * MT + t) * 2 + 1] = pack_rne(acc[b][t][2], acc[b][t][3]);
      }
    tree_push<NP>(st, v, root, nl, j);
  }

  if (!wg_combine<NP, WAVES>(root, dyn_lds, stack_words, wave, lane)) return;

  const int64_t n = n0 + 4 * g4;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + 16 * t + r16;
    if constexpr (EPI == EPI_STORE) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        store4(p.C[b], p.ldc[b], m, n, p.M, p.N, root[(b * MT + t) * 2], root[(b * MT + t) * 2 + 1]);
    } else if constexpr (EPI == EPI_DSILU) {
      // dA at (m, n = i) with the saved g, u: dU = bf16(dA s), dG = bf16((dA u) s'),
      // a = bf16(s u); written row-major [M, I] and transposed [I, M].
      if (m < p.M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t i = n + r;
          if (i >= p.N) break;
          const uint32_t pr = root[t * 2 + (r >> 1)];
          const float da = (r & 1) ? bf_hi(pr) : bf_lo(pr);
          const float g = bf2f(p.sg[m * p.ld_gu + i]);
          const float u = bf2f(p.su[m * p.ld_gu + i]);
          const float sg = sigma_f(g);
          const float s = g * sg;
          const float one_m = 1.0f - sg;
          const float tt = g * one_m;
          const float onep = 1.0f + tt;
          const float ds = sg * onep;
          const uint16_t du = f2bf(da * s);
          const float dau = da * u;
          const uint16_t dg = f2bf(dau * ds);
          const uint16_t a = f2bf(s * u);
          if (p.dG) p.dG[m * p.ld_d + i] = dg;
          if (p.dU) p.dU[m * p.ld_d + i] = du;
          if (p.dGT) p.dGT[i * p.ld_t + m] = dg;
          if (p.dUT) p.dUT[i * p.ld_t + m] = du;
          if (p.aT) p.aT[i * p.ld_t + m] = a;
          if (p.a_rm) p.a_rm[m * p.ld_d + i] = a;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch

#define DGF_DISPATCH_WAVES(KERNEL, NB, MT, EPI)                                                             \
  {                                                                                                         \
    const size_t shm = (size_t)waves * p.stack_slots * (NB * MT * 2) * 64 * 4;                              \
    switch (waves) {                                                                                        \
      case 1: hipLaunchKernelGGL((KERNEL<NB, MT, 1, EPI>), grid, dim3(64), shm, stream, p); break;          \
      case 2: hipLaunchKernelGGL((KERNEL<NB, MT, 2, EPI>), grid, dim3(128), shm, stream, p); break;         \
      case 4: hipLaunchKernelGGL((KERNEL<NB, MT, 4, EPI>), grid, dim3(256), shm, stream, p); break;         \
      default: hipLaunchKernelGGL((KERNEL<NB, MT, 8, EPI>), grid, dim3(512), shm, stream, p); break;        \
    }                                                                                                       \
  }

hipError_t launch_gemm(int layout, int nb, int epi, GemmParams p, int waves, hipStream_t stream) {
  const int mt = p.M <= 16 ? 1 : 2;
  const int64_t tiles_n = (p.N + 15) / 16;
  const int64_t tiles_m = (p.M + 16 * mt - 1) / (16 * mt);
  dim3 grid((unsigned)tiles_n, (unsigned)tiles_m);
  if (layout == DGF_LAYOUT_NT) {
    if (nb == 1 && epi == EPI_STORE) {
      if (mt == 1) { DGF_DISPATCH_WAVES(k_gemm_nt, 1, 1, EPI_STORE) } else { DGF_DISPATCH_WAVES(k_gemm_nt, 1, 2, EPI_STORE) }
    } else if (nb == 2 && epi == EPI_STORE) {
      if (mt == 1) { DGF_DISPATCH_WAVES(k_gemm_nt, 2, 1, EPI_STORE) } else { DGF_DISPATCH_WAVES(k_gemm_nt, 2, 2, EPI_STORE) }
    } else if (nb == 2 && epi == EPI_ACT) {
      if (mt == 1) { DGF_DISPATCH_WAVES(k_gemm_nt, 2, 1, EPI_ACT) } else { DGF_DISPATCH_WAVES(k_gemm_nt, 2, 2, EPI_ACT) }
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (nb == 1 && epi == EPI_STORE) {
      if (mt == 1) { DGF_DISPATCH_WAVES(k_gemm_nn, 1, 1, EPI_STORE) } else { DGF_DISPATCH_WAVES(k_gemm_nn, 1, 2, EPI_STORE) }
    } else if (nb == 1 && epi == EPI_DSILU) {
      if (mt == 1) { DGF_DISPATCH_WAVES(k_gemm_nn, 1, 1, EPI_DSILU) } else { DGF_DISPATCH_WAVES(k_gemm_nn, 1, 2, EPI_DSILU) }
    } else {
      return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace dgf
