// Host-visible kernel interfaces of libdgf (internal; the public ABI is include/dgf.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgf {

// Start/stop events of the timed step in progress, set by the library's
// timing hook: the step's first kernel records the start event as its own
// start timestamp and every kernel of the step records the stop event as its
// own end (hipExtLaunchKernelGGL; the last one's stands), so a timed step
// measures its kernels, without the gaps of separate event packets.
extern thread_local hipEvent_t g_launch_events[2];

template <typename F, typename... Args>
inline void dgf_launch(F kernel, dim3 grid, dim3 block, size_t shm, hipStream_t s, Args... args) {
  if (g_launch_events[1]) {
    hipEvent_t start = g_launch_events[0];
    g_launch_events[0] = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)shm, s, start, g_launch_events[1], 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  }
}

enum { DGF_LAYOUT_NT = 0, DGF_LAYOUT_NN = 1, DGF_LAYOUT_TN = 2 };
// stored type of every 16-bit tensor of a launch (the public dtype codes)
enum { FMT_BF16 = 0, FMT_F16 = 1 };
enum { EPI_STORE = 0, EPI_ACT = 1, EPI_DSILU = 2, EPI_DX = 3 };

// Arguments of one tree-GEMM launch (two products when NB = 2).
struct GemmParams {
  const uint16_t *A[2];  // [M, K] K-contiguous activations
  int64_t lda[2];
  const uint16_t *B[2];  // NT: [N, K] K-contiguous; NN: [K, N] N-contiguous
  int64_t ldb[2];
  uint16_t *C[2];        // [M, N] outputs (EPI_STORE; optional g/u or lanes otherwise)
  int64_t ldc[2];
  int64_t M, N, K;
  int fmt;               // stored type: FMT_BF16 or FMT_F16
  int L;                 // leaves = ceil(K / 64)
  int stack_slots;       // LDS tree-stack slots per wave (>= 1, >= a wave subtree's depth)
  int ksplit_depth;      // the K leaves are split over 2^ksplit_depth workgroups (grid.z)
  uint16_t *part;        // ksplit_depth > 0 (or to_part): partial roots [NB][2^ksplit_depth][M][ldp]
  int to_part;           // weight-streaming kernel: roots go to `part` (joined by the combine kernel)
  int64_t ldp, part_stride;
  int shared_a;          // NB = 2 with A[1] == A[0]
  // EPI_ACT: a = bf16(silu(C0) * C1)
  uint16_t *act_out;
  int64_t ld_act;
  // EPI_DSILU: saved g, u [M, N]; outputs dG, dU, a row-major
  const uint16_t *sg, *su;
  int64_t ld_gu;
  uint16_t *dG, *dU, *a_rm;
  int64_t ld_d;
  // EPI_DX (combine only): dx = bf16(G + U) of the two lanes; C[0], C[1] keep the lanes when set
  uint16_t *dx;
  int64_t lddx;
  // weight-streaming kernel: when set (and each XCD can take whole (product, K piece) slices),
  // run each slice's workgroups on one XCD so that its activation slice is fetched by one L2
  int xcd_slices;
};

// Weight-streaming tree GEMM with stationary activations (dgf_xs.hip):
// EPI_STORE products b < nb (grid.z = nb << ksplit_depth), each wave owning
// at most 4 leaves; roots go to C[b] (ksplit_depth = 0) or to the partials.
int xs_tile_cols(int layout, int mt);
size_t xs_lds_bytes(int layout, int mt, int waves);
hipError_t launch_xs(int layout, GemmParams p, int nb, int waves, int groups, hipStream_t stream);
// Join the 2^ksplit_depth partial roots of each product and apply the
// epilogue (STORE: C[b] for b < nb; ACT: a (and g, u in C[0], C[1]) from the
// gate and up products; DSILU: dG, dU, a from dA; DX: dx from the G and U lanes).
hipError_t launch_combine_epi(int epi, int nb, GemmParams p, hipStream_t stream);

// Fused gate/up projection and activation (dgf_gu.hip): x [M, K], W_gate and
// W_up [N, K], all K-contiguous; a = bf16(silu(g) u) [M, N], g and u kept
// when non-null.  Applies to M <= 32 and K a multiple of 64 with 8..64 leaves.
struct GuParams {
  const uint16_t *x;
  int64_t ldx;
  const uint16_t *w[2];
  int64_t ldw[2];
  uint16_t *a;
  int64_t lda;
  uint16_t *g, *u;
  int64_t ldgu;
  int64_t M, N, K;
  int fmt;
  int L;
};
bool gu_act_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_gu_act(const GuParams &p, hipStream_t stream);

// All-K tree GEMM for few tokens (dgf_dn.hip): C [M, N] = A [M, K] B [N, K]^T,
// both K-contiguous, one workgroup per 16 output columns reducing all of K
// (no partial roots, no join).  Applies to M <= 24, K a multiple of 64 and
// L / 8 leaves per wave in {1, 2, 3, 4, 6, 8, 12, 16, 24, 32}.
struct AllkParams {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;
  int64_t ldb;
  uint16_t *C;
  int64_t ldc;
  int64_t M, N, K;
  int fmt;
  int L;
};
bool allk_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_allk(const AllkParams &p, hipStream_t stream);

// Tiled tree GEMM for many tokens (dgf_mm.hip): NT, 128 x 128 output tiles
// per workgroup, grid.z = nb << ksplit_depth; stack_slots holds the number of
// top levels of each K piece's tree (<= 3) above lower subtrees of at most 4
// leaves (nlh: the larger lower-subtree size, the smaller being nlh - 1).
size_t mm_lds_bytes();
int mm_upper_levels(int Lp);
hipError_t launch_mm(GemmParams p, int nb, int nlh, hipStream_t stream);

// Output row tiles of 16 per wave of the NT / NN tree GEMM kernel variants.
int gemm_row_tiles(int layout, int nb, int epi);
hipError_t launch_gemm(int layout, int nb, int epi, GemmParams p, int waves, hipStream_t stream);
// NT, EPI_STORE, K <= 64 (one leaf), B shared by the NB products
hipError_t launch_gemm_short(int nb, GemmParams p, hipStream_t stream);
// TN, EPI_STORE, K <= 64 (one leaf): A_b [K][M] and B [K][N] row-major, B shared by the NB products.
// dx_join (optional): the dX lanes' join (EPI_DX, at most 8 K pieces) run by extra workgroups of the
// same launch; it shares no memory with the weight gradients.
hipError_t launch_gemm_tn1(int nb, GemmParams p, hipStream_t stream, const GemmParams *dx_join = nullptr);

// elementwise launches take the stored type first (FMT_BF16 or FMT_F16)
hipError_t launch_act_fwd(int fmt, const uint16_t *g, const uint16_t *u, uint16_t *a, int64_t n, hipStream_t s);
hipError_t launch_act_bwd(int fmt, const uint16_t *da, const uint16_t *g, const uint16_t *u, uint16_t *dg,
                          uint16_t *du, uint16_t *a, int64_t n, hipStream_t s);
hipError_t launch_combine(const uint16_t *const *parts, int S, uint16_t *out, int64_t n, hipStream_t s);
// the same rank tree for BF16, FP16 or FP32 parts (dtype one of DGF_COMBINE_*)
enum { DGF_COMBINE_BF16 = 0, DGF_COMBINE_FP16 = 1, DGF_COMBINE_FP32 = 2 };
hipError_t launch_combine_typed(const void *const *parts, int S, void *out, int64_t n, int dtype, hipStream_t s);
// out [M, N] (ldo) = balanced combine over S partials part[s] [M, N] (ldp),
// part[s] = part + s * part_stride
hipError_t launch_combine_2d(int fmt, const uint16_t *part, int64_t part_stride, int64_t ldp, int S, uint16_t *out,
                             int64_t ldo, int64_t M, int64_t N, hipStream_t s);
// dx [M, N] = rnd(G + U) per element (the gate lane first), row-major with leading dims
hipError_t launch_add_lanes(int fmt, const uint16_t *G, int64_t ldg, const uint16_t *U, int64_t ldu, uint16_t *dx,
                            int64_t lddx, int64_t M, int64_t N, hipStream_t s);
// dst [C, R] (ldd) = transpose of src [R, C] (lds)
hipError_t launch_transpose(const uint16_t *src, int64_t lds, int64_t R, int64_t C, uint16_t *dst, int64_t ldd,
                            hipStream_t s);

}  // namespace dgf
