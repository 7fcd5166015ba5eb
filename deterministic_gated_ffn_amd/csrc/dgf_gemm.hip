// Deterministic tree GEMMs for gfx950.
//
// One workgroup owns a tile of 16 output columns n (weight rows in the NT form)
// and 16*MT output rows m (tokens), for one of KSPLIT contiguous K pieces: the
// subtree at depth log2(KSPLIT) of the canonical midpoint tree over the K
// leaves.  Its WAVES waves split that piece further into the subtrees one
// level log2(WAVES) deeper; each wave runs its subtree in post order, then
// wave 0 combines the WAVES roots with the balanced top of the subtree.  With
// KSPLIT > 1 the workgroup roots go to a partial buffer and a combine kernel
// finishes the balanced top of the tree (RL-Kernel PR #325, section "Design":
// contiguous K pieces are subtrees of the one canonical tree).
//
// MFMA roles: A operand = 16 weight rows x 32 K, B operand = 32 K x 16 tokens,
// so lane l ends with D[4(l/16)+r][l%16]: four consecutive output columns of
// one token, which the epilogues store as 8 contiguous bytes.
#include <string.h>

#include "dgf_device.hpp"
#include "dgf_kernels.hpp"
#include "dgf_join.hpp"

namespace dgf {

// ------------------------------------------------------------------ shared tail

// Every wave parks its subtree root in slot 0 of its own stack region; wave 0
// then combines the WAVES roots with the balanced top of the tree.
template <class T, int NP, int WAVES>
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
    combine_roots<T, NP, WAVES>(r);
#pragma unroll
    for (int p = 0; p < NP; ++p) root[p] = r[0][p];
    return true;
  }
}

// Store 4 consecutive stored values (two packed pairs) at C[m][n..n+3], bounds-checked.
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

template <int W>
constexpr int log2i() {
  return W == 1 ? 0 : W == 2 ? 1 : W == 4 ? 2 : W == 8 ? 3 : 4;
}

// Streamed-once weight fragment: a non-temporal 16-byte load.
template <class T>
__device__ __forceinline__ typename T::frag load_frag_nt(const uint16_t *row, int64_t k) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename T::frag *>(row + k));
}

// ------------------------------------------------------------------ NT

// C_b[m][n] = T_K( A_b[m,:] . B_b[n,:] ), b < NB; A_b [M,K] and B_b [N,K] both
// K-contiguous.  A wave owns RT tiles of 16 weight rows per product (16 RT
// output columns n) and 16 MT tokens, so every activation fragment it loads
// feeds NB RT MFMAs.  Weight and activation fragments are loaded D leaves
// ahead of the MFMAs that use them, both at the same distance: loads complete
// in issue order, so an activation load issued after a weight load would
// otherwise make the wait for it also wait for that younger weight load.
template <class T, int NB, int RT, int MT, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_nt(GemmParams p) {
  constexpr bool SHARED_A = (EPI == EPI_ACT);  // gate and up share the activation operand
  constexpr int NA = SHARED_A ? 1 : NB;
  constexpr int NP = NB * RT * MT * 2;
  constexpr int DW = log2i<WAVES>();
  constexpr int P = NB * RT * MT >= 8 ? 2 : NB * RT * MT >= 4 ? 3 : 4, D = P - 1;  // ring slots, prefetch distance (leaves)
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
  const int stack_words = p.stack_slots * NP * 64;  // per wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * (16 * RT);
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
  const int ks = blockIdx.z;
  const int r16 = lane & 15, g4 = lane >> 4;

  int lo, hi;
  subtree_range(p.L, p.ksplit_depth + DW, (ks << DW) | wave, lo, hi);
  const int nl = hi - lo;
  const bool tail = (int64_t)hi * kLeaf > p.K;  // this wave owns the partial last leaf
  const int nfull = tail ? nl - 1 : nl;

  // Rows past N and tokens past M read a valid row instead (clamped); their
  // MFMA outputs are never stored, and every output depends only on its own
  // weight row and token.
  const uint16_t *brow[NB][RT];
  const uint16_t *arow[NA][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t n = n0 + 16 * rt + r16 < p.N ? n0 + 16 * rt + r16 : p.N - 1;
#pragma unroll
    for (int b = 0; b < NB; ++b) brow[b][rt] = p.B[b] + n * p.ldb[b] + 8 * g4;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + 16 * t + r16 < p.M ? m0 + 16 * t + r16 : p.M - 1;
#pragma unroll
    for (int a = 0; a < NA; ++a) arow[a][t] = p.A[a] + m * p.lda[a] + 8 * g4;
  }

  struct WF { typename T::frag v[NB][RT][2]; };
  struct XF { typename T::frag v[NA][MT][2]; };
  auto load_w = [&](int leaf, WF &w) {
    const int64_t k = (int64_t)leaf * kLeaf;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) w.v[b][rt][s] = load_frag_nt<T>(brow[b][rt], k + 32 * s);
  };
  auto load_x = [&](int leaf, XF &x) {
    const int64_t k = (int64_t)leaf * kLeaf;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) x.v[a][t][s] = load_frag<T>(arow[a][t], k + 32 * s);
  };

  TreeStack<NP> st{dyn_lds + wave * stack_words + lane};
  uint32_t root[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) root[q] = 0;

  // pack a leaf's accumulators (index ((b RT + rt) MT + t) 2 + h) and push them
  auto finish_leaf = [&](f32x4 (&acc)[NB][RT][MT], int j) {
    uint32_t v[NP];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int q = ((b * RT + rt) * MT + t) * 2;
          v[q + 0] = T::pack(acc[b][rt][t][0], acc[b][rt][t][1]);
          v[q + 1] = T::pack(acc[b][rt][t][2], acc[b][rt][t][3]);
        }
    tree_push<T, NP>(st, v, root, nl, j);
  };
  auto leaf_mfma = [&](const WF &w, const XF &x, int j) {
    f32x4 acc[NB][RT][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          acc[b][rt][t] = T::mfma(w.v[b][rt][0], x.v[SHARED_A ? 0 : b][t][0], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[b][rt][t] = T::mfma(w.v[b][rt][1], x.v[SHARED_A ? 0 : b][t][1], acc[b][rt][t]);
        }
    finish_leaf(acc, j);
  };

  // Ring of P fragment buffers: leaf j lives in slot j % P.  The main loop
  // issues its loads unconditionally (indices past the last full leaf are
  // clamped to it) so that every wait counts a fixed number of younger loads;
  // a conditional load would force the wait to drain the whole queue.
  WF wb[P];
  XF xb[P];
  const int last = lo + nfull - 1;
  if (nfull > 0) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      load_w(min(lo + i, last), wb[i]);
      load_x(min(lo + i, last), xb[i]);
    }
  }
  const int ngroups = nfull / P;
  for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int j = gi * P + q;
      load_w(min(lo + j + D, last), wb[(q + D) % P]);
      load_x(min(lo + j + D, last), xb[(q + D) % P]);
      leaf_mfma(wb[q], xb[q], j);
    }
  }
  // the remaining nfull % P (< P, so <= D) leaves are already in the ring
#pragma unroll
  for (int q = 0; q < P - 1; ++q) {
    const int j = ngroups * P + q;
    if (j < nfull) leaf_mfma(wb[q], xb[q], j);
  }

  if (tail) {
    // the partial last leaf: zeros past K; an all-zero block leaves the
    // accumulator unchanged, so a half past K is skipped
    const int64_t kb = (int64_t)(hi - 1) * kLeaf;
    f32x4 acc[NB][RT][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[b][rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < 2; ++s) {
      if (kb + 32 * s >= p.K) break;
      const int64_t k = kb + 32 * s;
      typename T::frag xf[NA][MT];
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int t = 0; t < MT; ++t) xf[a][t] = load_frag_tail<T>(arow[a][t], k, p.K - 8 * g4);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const typename T::frag wf = load_frag_tail<T>(brow[b][rt], k, p.K - 8 * g4);
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[b][rt][t] = T::mfma(wf, xf[SHARED_A ? 0 : b][t], acc[b][rt][t]);
        }
    }
    finish_leaf(acc, nl - 1);
  }

  if (!wg_combine<T, NP, WAVES>(root, dyn_lds, stack_words, wave, lane)) return;

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t n = n0 + 16 * rt + 4 * g4;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t m = m0 + 16 * t + r16;
      if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int q = ((b * RT + rt) * MT + t) * 2;
          if (p.ksplit_depth > 0)
            store4(p.part + ((int64_t)b * (1 << p.ksplit_depth) + ks) * p.part_stride, p.ldp, m, n, p.M, p.N,
                   root[q], root[q + 1]);
          else
            store4(p.C[b], p.ldc[b], m, n, p.M, p.N, root[q], root[q + 1]);
        }
      } else if constexpr (EPI == EPI_ACT) {
        // gate (b = 0) and up (b = 1) of the same (m, n): a = rnd(silu(g) u)
        const int qg = ((0 * RT + rt) * MT + t) * 2, qu = ((1 * RT + rt) * MT + t) * 2;
        uint32_t ap[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t gp = root[qg + h], up = root[qu + h];
          float a2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float g = e ? T::hi(gp) : T::lo(gp);
            const float u = e ? T::hi(up) : T::lo(up);
            const float s = g * sigma_f(g);
            a2[e] = s * u;
          }
          ap[h] = T::pack_prod(a2[0], a2[1]);
        }
        store4(p.act_out, p.ld_act, m, n, p.M, p.N, ap[0], ap[1]);
        if (p.C[0]) store4(p.C[0], p.ldc[0], m, n, p.M, p.N, root[qg], root[qg + 1]);
        if (p.C[1]) store4(p.C[1], p.ldc[1], m, n, p.M, p.N, root[qu], root[qu + 1]);
      }
    }
  }
}

// ------------------------------------------------------------------ NN

// C_b[m][n] = T_K( A_b[m,:] . B_b[:,n] ); A_b [M,K] K-contiguous, B_b [K,N]
// N-contiguous.  A wave owns 16 RT output columns; per leaf it loads the 64 x
// 16 RT weight slab as whole row segments (2 RT lanes of 16 bytes per row) and
// transposes it through its own LDS region so that the MFMA A operand is
// K-contiguous.  The slab keeps column n's 64 K values in one 128-byte row
// whose 16-byte chunks are permuted by XOR with swz(n), so that both the
// transposing 2-byte writes and the 16-byte operand reads spread over the
// banks.
__device__ __forceinline__ int slab_swz(int n) { return (n ^ (n >> 3)) & 7; }

template <class T, int NB, int RT, int MT, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_nn(GemmParams p) {
  constexpr int NP = NB * RT * MT * 2;
  constexpr int DW = log2i<WAVES>();
  constexpr int NI = 2 * RT;           // 16-byte loads per lane per leaf and product
  constexpr int ROWS = 32 / RT;        // slab rows per load instruction
  constexpr int P = NB * RT * MT >= 8 ? 2 : NB * RT * MT >= 4 ? 3 : 4, D = P - 1;
  __shared__ __attribute__((aligned(16))) uint16_t slab[WAVES][NB][16 * RT * 64];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
  const int stack_words = p.stack_slots * NP * 64;  // per wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * (16 * RT);
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
  const int ks = blockIdx.z;
  const int r16 = lane & 15, g4 = lane >> 4;
  // this lane's place in a load instruction: slab row lrow (+ ROWS i), columns 8 lcol .. 8 lcol + 7
  const int lrow = lane / NI, lcol = lane % NI;

  int lo, hi;
  subtree_range(p.L, p.ksplit_depth + DW, (ks << DW) | wave, lo, hi);
  const int nl = hi - lo;

  const uint16_t *arow[NB][MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + 16 * t + r16 < p.M ? m0 + 16 * t + r16 : p.M - 1;  // clamped, never stored
#pragma unroll
    for (int b = 0; b < NB; ++b) arow[b][t] = p.A[b] + m * p.lda[b];
  }
  const bool full_n = n0 + 16 * RT <= p.N;
  const bool tail = (int64_t)hi * kLeaf > p.K;  // this wave owns the partial last leaf
  const int nfull = tail ? nl - 1 : nl;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  struct QF { u32x4 v[NB][NI]; };
  // full leaf, full column tile: 16-byte row pieces
  auto fetch_fast = [&](int leaf, QF &q) {
    const int64_t kr = (int64_t)leaf * kLeaf + lrow;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        q.v[b][i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(p.B[b] + (kr + ROWS * i) * p.ldb[b] + n0 + 8 * lcol));
  };
  // element by element with zeros outside the matrix
  auto fetch_slow = [&](int leaf, QF &q) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t kr = (int64_t)leaf * kLeaf + lrow + ROWS * i;
        const bool kok = kr < p.K;
        const uint16_t *src = p.B[b] + (kok ? kr : 0) * p.ldb[b] + n0 + 8 * lcol;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = n0 + 8 * lcol + 2 * e;
          const uint32_t lo16 = (kok && n < p.N) ? src[2 * e] : 0u;
          const uint32_t hi16 = (kok && n + 1 < p.N) ? src[2 * e + 1] : 0u;
          w[e] = lo16 | (hi16 << 16);
        }
        q.v[b][i] = u32x4{w[0], w[1], w[2], w[3]};
      }
  };

  TreeStack<NP> st{dyn_lds + wave * stack_words + lane};
  uint32_t root[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) root[q] = 0;

  // activation fragments of one leaf (both K halves)
  struct XF { typename T::frag v[NB][MT][2]; };
  auto load_x = [&](int leaf, XF &x) {
    const int64_t kb = (int64_t)leaf * kLeaf;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) x.v[b][t][s] = load_frag<T>(arow[b][t], kb + 32 * s + 8 * g4);
  };
  auto load_x_tail = [&](int leaf, XF &x) {
    const int64_t kb = (int64_t)leaf * kLeaf;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) x.v[b][t][s] = load_frag_tail<T>(arow[b][t], kb + 32 * s + 8 * g4, p.K);
  };

  // stage the slab transposed, two MFMA halves per column tile, then the tree
  auto leaf_body = [&](int j, const QF &q, const XF &x, bool partial) {
    const int64_t kb = (int64_t)(lo + j) * kLeaf;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int k = lrow + ROWS * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = 8 * lcol + e;
          const uint32_t w = q.v[b][i][e >> 1];
          slab[wave][b][n * 64 + 8 * ((k >> 3) ^ slab_swz(n)) + (k & 7)] = (uint16_t)((e & 1) ? (w >> 16) : w);
        }
      }
    wave_lds_sync();  // this wave's slab writes land before its lanes read them
    f32x4 acc[NB][RT][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[b][rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (partial && kb + 32 * s >= p.K) break;  // all-zero block: accumulator unchanged
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int n = 16 * rt + r16;
          const typename T::frag wf =
              *reinterpret_cast<const typename T::frag *>(&slab[wave][b][n * 64 + 8 * ((4 * s + g4) ^ slab_swz(n))]);
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[b][rt][t] = T::mfma(wf, x.v[b][t][s], acc[b][rt][t]);
        }
    }
    wave_lds_sync();  // slab reads done before the next leaf overwrites it
    uint32_t v[NP];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int qi = ((b * RT + rt) * MT + t) * 2;
          v[qi + 0] = T::pack(acc[b][rt][t][0], acc[b][rt][t][1]);
          v[qi + 1] = T::pack(acc[b][rt][t][2], acc[b][rt][t][3]);
        }
    tree_push<T, NP>(st, v, root, nl, j);
  };

  if (full_n) {
    // Weight rows and activation fragments are fetched D leaves ahead, at the
    // same distance, into a ring where leaf j lives in slot j % P; the loop
    // issues them unconditionally (clamped indices) so that waits stay partial.
    QF qb[P];
    XF xb[P];
    const int last = lo + nfull - 1;
    if (nfull > 0) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        fetch_fast(min(lo + i, last), qb[i]);
        load_x(min(lo + i, last), xb[i]);
      }
    }
    const int ngroups = nfull / P;
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
      for (int h = 0; h < P; ++h) {
        const int j = gi * P + h;
        fetch_fast(min(lo + j + D, last), qb[(h + D) % P]);
        load_x(min(lo + j + D, last), xb[(h + D) % P]);
        leaf_body(j, qb[h], xb[h], false);
      }
    }
#pragma unroll
    for (int h = 0; h < P - 1; ++h) {
      const int j = ngroups * P + h;
      if (j < nfull) leaf_body(j, qb[h], xb[h], false);
    }
  } else {
    for (int j = 0; j < nfull; ++j) {
      QF q;
      XF x;
      fetch_slow(lo + j, q);
      load_x(lo + j, x);
      leaf_body(j, q, x, false);
    }
  }
  if (tail) {
    QF q;
    XF x;
    fetch_slow(hi - 1, q);
    load_x_tail(hi - 1, x);
    leaf_body(nl - 1, q, x, true);
  }

  if (!wg_combine<T, NP, WAVES>(root, dyn_lds, stack_words, wave, lane)) return;

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t n = n0 + 16 * rt + 4 * g4;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t m = m0 + 16 * t + r16;
      if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int q = ((b * RT + rt) * MT + t) * 2;
          if (p.ksplit_depth > 0)
            store4(p.part + ((int64_t)b * (1 << p.ksplit_depth) + ks) * p.part_stride, p.ldp, m, n, p.M, p.N,
                   root[q], root[q + 1]);
          else
            store4(p.C[b], p.ldc[b], m, n, p.M, p.N, root[q], root[q + 1]);
        }
      } else if constexpr (EPI == EPI_DSILU) {
        // dA at (m, n = i) with the saved g, u: dU = rnd(dA s), dG = rnd((dA u) s'),
        // a = rnd(s u); written row-major [M, I].
        if (m < p.M) {
          const int q = (rt * MT + t) * 2;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t i = n + r;
            if (i >= p.N) break;
            const uint32_t pr = root[q + (r >> 1)];
            const float da = (r & 1) ? T::hi(pr) : T::lo(pr);
            const float g = T::f(p.sg[m * p.ld_gu + i]);
            const float u = T::f(p.su[m * p.ld_gu + i]);
            const float sg = sigma_f(g);
            const float s = g * sg;
            const float one_m = 1.0f - sg;
            const float tt = g * one_m;
            const float onep = 1.0f + tt;
            const float ds = sg * onep;
            const uint16_t du = T::r(da * s);
            const float dau = da * u;
            const uint16_t dg = T::r(dau * ds);
            const uint16_t a = T::r(s * u);
            if (p.dG) p.dG[m * p.ld_d + i] = dg;
            if (p.dU) p.dU[m * p.ld_d + i] = du;
            if (p.a_rm) p.a_rm[m * p.ld_d + i] = a;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ one leaf

// C_b[m][n] = rnd( leaf(A_b[m,:] . B[n,:]) ) for K <= 64: a single leaf, so
// no tree node; this is the weight-gradient shape (K = tokens) and is bound by
// its output writes.  A workgroup of 4 waves owns 64 m-rows x 128 n-columns;
// wave w computes m-rows 16w..16w+15 against all 128 columns (the B fragments
// are shared by the NB products), stages each 16 x 128 result in LDS and
// stores it as whole 256-byte row segments.
constexpr int kShortN = 128, kShortStride = kShortN + 8;

template <class T, int NB>
__global__ __launch_bounds__(256) void k_gemm_short(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][16 * kShortStride];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int64_t n0 = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * kShortN;
  const int64_t m0 = (int64_t)blockIdx.y * 64 + 16 * wave;

  const int64_t mrow = m0 + r16 < p.M ? m0 + r16 : p.M - 1;  // clamped rows are never stored
  const uint16_t *arow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) arow[b] = p.A[b] + mrow * p.lda[b];
  const uint16_t *brow[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int64_t n = n0 + 16 * c + r16 < p.N ? n0 + 16 * c + r16 : p.N - 1;
    brow[c] = p.B[0] + n * p.ldb[0];
  }

  f32x4 acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < 2; ++s) {
    if (32 * s >= p.K) break;  // all-zero block: the accumulator is unchanged
    const int64_t k = 32 * s + 8 * g4;
    typename T::frag xa[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xa[b] = load_frag_tail<T>(arow[b], k, p.K);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const typename T::frag w = load_frag_tail<T>(brow[c], k, p.K);
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b][c] = T::mfma(w, xa[b], acc[b][c]);
    }
  }

  uint16_t *st = stage[wave];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    // lane holds C[m0 + r16][n0 + 16c + 4 g4 + (0..3)]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint2 v = make_uint2(T::pack(acc[b][c][0], acc[b][c][1]), T::pack(acc[b][c][2], acc[b][c][3]));
      *reinterpret_cast<uint2 *>(&st[r16 * kShortStride + 16 * c + 4 * g4]) = v;
    }
    wave_lds_sync();
    // 16 rows x 256 bytes: lane l writes row (l >> 4) + 4i, bytes 16 (l & 15) .. +16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) + 4 * i;
      const int col = 8 * (lane & 15);
      const int64_t m = m0 + row, n = n0 + col;
      if (m < p.M) {
        uint16_t *dst = p.C[b] + m * p.ldc[b] + n;
        const uint4 v = *reinterpret_cast<const uint4 *>(&st[row * kShortStride + col]);
        if (n + 8 <= p.N) {
          *reinterpret_cast<uint4 *>(dst) = v;
        } else {
          const uint32_t q[4] = {v.x, v.y, v.z, v.w};
          for (int e = 0; e < 8 && n + e < p.N; ++e) dst[e] = (uint16_t)(q[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    wave_lds_sync();  // the stage is reused by the next product
  }
}

// ------------------------------------------------------------------ one leaf, TN

// C_b[r][c] = rnd( leaf( sum_k A_b[k][r] B[k][c] ) ) for K <= 64, straight
// from row-major [k][features] operands: the weight gradients, k = tokens.
// A workgroup of 4 waves owns 64 rows r and CT consecutive tiles of 128
// columns c.  It copies the K x 64 A tile into LDS feature-major once, and
// each K x 128 B tile in turn into one of two LDS buffers, with zeros past K
// (up to the next multiple of 32: an all-zero block leaves the sum
// unchanged), past M and past N.  A B tile is transposed four operand rows
// at a time: a thread loads 8 features of rows 4i .. 4i+3 and writes, per
// feature, the 4 consecutive K values as one 8-byte store.  The next B
// tile's loads are issued into registers before the current tile's MFMAs and
// committed to the other buffer after its stores, so their latency hides
// behind the stores.  Every wave computes 16 rows x 128 columns per tile and
// stores them through its own LDS stage as whole 256-byte row segments.
constexpr int kTnTile = 128;

// 8 consecutive features f0 .. f0+7 of operand row k, packed.  A row past K
// (the zero padding of the MFMA's K) loads row 0 (K >= 1) instead, and the
// caller zeroes it when it writes the tile (tn_zero_rows), so that no value
// is needed until then; features past F read as zero.
__device__ __forceinline__ uint4 tn_load8(const uint16_t *src, int64_t ld, int k, int K, int64_t f0, int64_t F) {
  const int64_t row = k < K ? k : 0;
  if (f0 + 8 <= F) return *reinterpret_cast<const uint4 *>(src + row * ld + f0);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < 8; ++e)
    if (f0 + e < F) w[e >> 1] |= (uint32_t)src[row * ld + f0 + e] << (16 * (e & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Zeroes the rows 4 k4 + r past K of a four-row group.
__device__ __forceinline__ void tn_zero_rows(uint4 (&rows)[4], int k4, int K) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * k4 + r >= K) rows[r] = make_uint4(0u, 0u, 0u, 0u);
}

// Features f = 8 cc + e of operand rows 4 k4 .. 4 k4 + 3 land at LDS row f,
// positions (4 k4) ^ (8 (cc & km)) .. + 3, one 8-byte store per feature: the
// K chunks are permuted per feature group (the XOR moves whole 8-element
// chunks), which spreads the transposing writes over the banks and keeps
// each MFMA operand read one aligned 16-byte chunk.
__device__ __forceinline__ void tn_put4x8(uint16_t *dst, int ks, int km, int k4, int cc, const uint4 (&rows)[4]) {
  const int kk = (4 * k4) ^ (8 * (cc & km));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t w4[4] = {rows[r].x, rows[r].y, rows[r].z, rows[r].w};
      h[r] = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
    }
    *reinterpret_cast<uint2 *>(&dst[(8 * cc + e) * ks + kk]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
}

// The dX lanes' join (EPI_DX over 2^kd <= 8 K pieces) on the workgroups past
// the weight-gradient tiles (grid rows gridDim.y - jrows ..): independent
// work that fills the kernel's tail instead of a launch of its own.
template <class T, int S>
__device__ void tn_dx_join(const GemmParams &j, int jrow, int jrows) {
  const int64_t chunks = (j.N + 7) / 8;
  const int64_t nthreads = (int64_t)jrows * gridDim.x * 256;
  for (int64_t i = ((int64_t)jrow * gridDim.x + blockIdx.x) * 256 + threadIdx.x; i < j.M * chunks; i += nthreads) {
    const int64_t m = i / chunks, c = (i % chunks) * 8;
    join_epi_chunk<T, S, EPI_DX>(j, 0, m, c);
  }
}

template <class T, int NB>
__global__ __launch_bounds__(256) void k_gemm_tn1(GemmParams p, int ct, GemmParams jn, int jrows) {
  extern __shared__ __attribute__((aligned(16))) uint16_t tn_lds[];
  if (jrows > 0 && (int)blockIdx.y >= (int)gridDim.y - jrows) {
    const int jrow = (int)blockIdx.y - ((int)gridDim.y - jrows);
    switch (jn.ksplit_depth) {
      case 0: tn_dx_join<T, 1>(jn, jrow, jrows); break;
      case 1: tn_dx_join<T, 2>(jn, jrow, jrows); break;
      case 2: tn_dx_join<T, 4>(jn, jrow, jrows); break;
      default: tn_dx_join<T, 8>(jn, jrow, jrows); break;
    }
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int K = (int)p.K;
  const int KH = (K + 31) / 32;  // MFMA K halves
  const int KP = 32 * KH;
  const int ks = KP + 8;         // padded K stride of the feature-major tiles
  const int km = KP / 8 - 1;     // K-chunk swizzle mask: chunks stay inside the row's KP elements
  // B-tile items: (4-row group k4, 8-feature chunk cc), one per thread for the first KP * 4 threads
  const bool bq = tid < KP * (kTnTile / 8) / 4;
  const int k4 = tid / (kTnTile / 8), bcc = tid % (kTnTile / 8);
  uint16_t *sA = tn_lds;                            // [NB][64][ks]
  uint16_t *sB0 = sA + NB * 64 * ks;                // [2][128][ks]
  uint16_t *stage = sB0 + 2 * kTnTile * ks + wave * 16 * kShortStride;  // this wave's [16][kShortStride]
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t cbase = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * kTnTile * ct;

  // rows 4 k4 .. 4 k4 + 3, features c0 + 8 bcc .. + 8 (sixteen threads per 128-byte row segment)
  uint4 nx[4];
  auto load_b = [&](int64_t c0) {
    if (bq) {
#pragma unroll
      for (int r = 0; r < 4; ++r) nx[r] = tn_load8(p.B[0], p.ldb[0], 4 * k4 + r, K, c0 + 8 * bcc, p.N);
    }
  };
  auto put_b = [&](uint16_t *sB) {
    if (bq) {
      tn_zero_rows(nx, k4, K);
      tn_put4x8(sB, ks, km, k4, bcc, nx);
    }
  };
  load_b(cbase);
  // the A tiles: items (product b, 4-row group, 8-feature chunk of the 64 rows)
  for (int q = tid; q < NB * (KP / 4) * 8; q += 256) {
    const int b = q / (KP * 2), rem = q % (KP * 2), a4 = rem / 8, cc = rem % 8;
    uint4 rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rows[r] = tn_load8(p.A[b], p.lda[b], 4 * a4 + r, K, r0 + 8 * cc, p.M);
    tn_zero_rows(rows, a4, K);
    tn_put4x8(sA + b * 64 * ks, ks, km, a4, cc, rows);
  }
  put_b(sB0);
  __syncthreads();

  const int64_t m0 = r0 + 16 * wave;
  for (int c = 0; c < ct; ++c) {
    const int64_t c0 = cbase + (int64_t)c * kTnTile;
    if (c0 >= p.N) break;  // the same for every wave of the workgroup
    const bool more = c + 1 < ct && c0 + kTnTile < p.N;
    if (more) load_b(c0 + kTnTile);  // in flight during this tile's MFMAs and stores
    const uint16_t *sB = sB0 + (c & 1) * kTnTile * ks;
    f32x4 acc[NB][8];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < KH; ++s) {
      typename T::frag xa[NB];
      const int ra = 16 * wave + r16;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        xa[b] = *reinterpret_cast<const typename T::frag *>(&sA[(b * 64 + ra) * ks + 8 * ((4 * s + g4) ^ ((ra >> 3) & km))]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rb = 16 * t + r16;
        const typename T::frag w = *reinterpret_cast<const typename T::frag *>(&sB[rb * ks + 8 * ((4 * s + g4) ^ ((rb >> 3) & km))]);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][t] = T::mfma(w, xa[b], acc[b][t]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // lane holds C[m0 + r16][c0 + 16t + 4 g4 + (0..3)]
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint2 v = make_uint2(T::pack(acc[b][t][0], acc[b][t][1]), T::pack(acc[b][t][2], acc[b][t][3]));
        *reinterpret_cast<uint2 *>(&stage[r16 * kShortStride + 16 * t + 4 * g4]) = v;
      }
      wave_lds_sync();
      // 16 rows x 256 bytes: lane l writes row (l >> 4) + 4i, bytes 16 (l & 15) .. +16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (lane >> 4) + 4 * i;
        const int col = 8 * (lane & 15);
        const int64_t m = m0 + row, n = c0 + col;
        if (m < p.M) {
          uint16_t *dst = p.C[b] + m * p.ldc[b] + n;
          const uint4 v = *reinterpret_cast<const uint4 *>(&stage[row * kShortStride + col]);
          if (n + 8 <= p.N) {
            *reinterpret_cast<uint4 *>(dst) = v;
          } else {
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < 8 && n + e < p.N; ++e) dst[e] = (uint16_t)(q[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
      wave_lds_sync();  // the stage is reused by the next product
    }
    // the other buffer was last read in the previous tile, before the barrier that ended it
    if (more) put_b(sB0 + ((c + 1) & 1) * kTnTile * ks);
    __syncthreads();  // the next B tile is in LDS
  }
}

size_t tn1_lds_bytes(int nb, int64_t K) {
  const int64_t ks = 32 * ((K + 31) / 32) + 8;
  return (size_t)(nb * 64 + 2 * kTnTile) * ks * 2 + (size_t)4 * 16 * kShortStride * 2;
}

template <class T>
hipError_t launch_gemm_tn1_t(int nb, GemmParams p, hipStream_t stream, const GemmParams *dx_join) {
  if (p.K < 0 || p.K > 64) return hipErrorInvalidValue;
  if (dx_join && dx_join->ksplit_depth > 3) return hipErrorInvalidValue;
  // column tiles per workgroup: as many as keep at least 3 workgroups per CU busy (the LDS of the
  // one-leaf tiles holds 3 per CU, so the weight gradients of the FFN shapes run as one round)
  const int64_t tiles_c = (p.N + kTnTile - 1) / kTnTile, tiles_r = (p.M + 63) / 64;
  int ct = 1;
  while (ct < 8 && tiles_c % (2 * ct) == 0 && (tiles_c / (2 * ct)) * tiles_r >= 3 * 256) ct *= 2;
  const int64_t gx = (tiles_c + ct - 1) / ct;
  // the dX join's rows of workgroups: about 64 workgroups of one chunk per thread
  int jrows = 0;
  GemmParams jn;
  memset(&jn, 0, sizeof jn);
  if (dx_join) {
    jn = *dx_join;
    const int64_t items = jn.M * ((jn.N + 7) / 8);
    const int64_t wgs = (items + 255) / 256 < 64 ? (items + 255) / 256 : 64;
    jrows = (int)((wgs + gx - 1) / gx);
    if (jrows < 1) jrows = 1;
  }
  if (tiles_r + jrows > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)gx, (unsigned)(tiles_r + jrows));
  const size_t shm = tn1_lds_bytes(nb, p.K);
  if (nb == 1)
    dgf_launch((k_gemm_tn1<T, 1>), grid, dim3(256), shm, stream, p, ct, jn, jrows);
  else
    dgf_launch((k_gemm_tn1<T, 2>), grid, dim3(256), shm, stream, p, ct, jn, jrows);
  return hipGetLastError();
}

hipError_t launch_gemm_tn1(int nb, GemmParams p, hipStream_t stream, const GemmParams *dx_join) {
  if (dx_join && dx_join->fmt != p.fmt) return hipErrorInvalidValue;
  if (p.fmt == FMT_F16) return launch_gemm_tn1_t<F16>(nb, p, stream, dx_join);
  return launch_gemm_tn1_t<Bf16>(nb, p, stream, dx_join);
}

template <class T>
hipError_t launch_gemm_short_t(int nb, GemmParams p, hipStream_t stream) {
  dim3 grid((unsigned)((p.N + kShortN - 1) / kShortN), (unsigned)((p.M + 63) / 64));
  if (nb == 1)
    dgf_launch((k_gemm_short<T, 1>), grid, dim3(256), 0, stream, p);
  else
    dgf_launch((k_gemm_short<T, 2>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_short(int nb, GemmParams p, hipStream_t stream) {
  if (p.fmt == FMT_F16) return launch_gemm_short_t<F16>(nb, p, stream);
  return launch_gemm_short_t<Bf16>(nb, p, stream);
}

// ------------------------------------------------------------------ launch

#define DGF_DISPATCH_WAVES(KERNEL, NB, RT, MT, EPI)                                                         \
  {                                                                                                         \
    const size_t shm = (size_t)waves * p.stack_slots * (NB * RT * MT * 2) * 64 * 4;                         \
    switch (waves) {                                                                                        \
      case 1: dgf_launch((KERNEL<T, NB, RT, MT, 1, EPI>), grid, dim3(64), shm, stream, p); break;   \
      case 2: dgf_launch((KERNEL<T, NB, RT, MT, 2, EPI>), grid, dim3(128), shm, stream, p); break;  \
      default: dgf_launch((KERNEL<T, NB, RT, MT, 4, EPI>), grid, dim3(256), shm, stream, p); break; \
    }                                                                                                       \
  }

#define DGF_DISPATCH_MT(KERNEL, NB, RT, EPI)                   \
  {                                                            \
    if (mt == 1) DGF_DISPATCH_WAVES(KERNEL, NB, RT, 1, EPI)    \
    else DGF_DISPATCH_WAVES(KERNEL, NB, RT, 2, EPI)            \
  }

int gemm_row_tiles(int layout, int nb, int epi) {
  if (layout == DGF_LAYOUT_NT) return nb == 2 ? 2 : 4;
  return epi == EPI_DSILU ? 2 : 4;
}

template <class T>
hipError_t launch_gemm_t(int layout, int nb, int epi, GemmParams p, int waves, hipStream_t stream) {
  const int mt = p.M <= 16 ? 1 : 2;
  const int rt = gemm_row_tiles(layout, nb, epi);
  const int64_t tiles_n = (p.N + 16 * rt - 1) / (16 * rt);
  const int64_t tiles_m = (p.M + 16 * mt - 1) / (16 * mt);
  dim3 grid((unsigned)tiles_n, (unsigned)tiles_m, (unsigned)(1 << p.ksplit_depth));
  if (layout == DGF_LAYOUT_NT) {
    if (nb == 1 && epi == EPI_STORE) DGF_DISPATCH_MT(k_gemm_nt, 1, 4, EPI_STORE)
    else if (nb == 2 && epi == EPI_STORE) DGF_DISPATCH_MT(k_gemm_nt, 2, 2, EPI_STORE)
    else if (nb == 2 && epi == EPI_ACT) DGF_DISPATCH_MT(k_gemm_nt, 2, 2, EPI_ACT)
    else return hipErrorInvalidValue;
  } else {
    if (nb == 1 && epi == EPI_STORE) DGF_DISPATCH_MT(k_gemm_nn, 1, 4, EPI_STORE)
    else if (nb == 1 && epi == EPI_DSILU) DGF_DISPATCH_MT(k_gemm_nn, 1, 2, EPI_DSILU)
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int layout, int nb, int epi, GemmParams p, int waves, hipStream_t stream) {
  if (p.fmt == FMT_F16) return launch_gemm_t<F16>(layout, nb, epi, p, waves, stream);
  return launch_gemm_t<Bf16>(layout, nb, epi, p, waves, stream);
}

}  // namespace dgf
