/*
 * dgf.h -- C ABI of the deterministic gated FFN library (libdgf.so, AMD gfx950).
 *
 * The operation (RL-Kernel PR #325 "feat(ffn): add deterministic distributed
 * Triton FFN for ROCm", sections "Summary", "Design" and "Operator test matrix"):
 * the bias-free gated Qwen3 FFN
 *     y = W_down (silu(W_gate x) * (W_up x)),
 * weights in [out, in] layout, forward and backward (dHidden and dWeights),
 * with every K-reduction evaluated by one canonical tree: leaves of 64
 * contiguous K elements accumulated in FP32 and rounded to BF16, and
 * midpoint-split internal nodes (mid = lo + floor(n/2)) that add two BF16
 * children in FP32 and round to BF16.  BF16 stage boundaries are kept:
 * g, u, a, y forward; dA, dG, dU, the dX lanes G and U, dX and dW backward.
 * Inside a leaf the FP32 accumulation takes the K elements in ascending blocks
 * of 8 with one FP32 rounding per block, the accumulation rule of the gfx950
 * bf16 matrix cores (block grid 2^(E-24), E the largest product exponent;
 * products cut toward zero, the accumulator and the sum toward minus infinity,
 * then round to nearest even; a zero block result is +0).  Results are bitwise
 * reproducible run to run and independent of the batch size M (row m of
 * every output depends on row m of the inputs only).
 *
 * Conventions for every entry point:
 *  - Tensors are BF16 bit patterns, row-major, device pointers on the current
 *    HIP device, each with a leading dimension in elements (>= the row width).
 *    Matrix operands must have 16-byte aligned base pointers and leading
 *    dimensions that are multiples of 8; otherwise DGF_EINVAL.  Leading
 *    dimensions are below 2^23 elements and K is at most 2^23 (the kernels
 *    address a tile's rows with 32-bit byte offsets); otherwise
 *    DGF_EUNSUPPORTED.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; errors raised by a kernel while it runs
 *    surface at the caller's next synchronisation.  Calls are stream-ordered,
 *    with no asynchronous overlap between calls and no compute/communication
 *    fusion claimed (PR #357, section "Compute/communication fusion").
 *  - Ownership: the caller allocates every buffer, the workspace included.  The
 *    library allocates and frees nothing and keeps no device state; the only
 *    globals are the thread-local error message and timing-hook state, and the
 *    static scratch array of dgf_ffn_fwd_static (the one entry point without a
 *    workspace argument).  Calls on different streams may run concurrently as
 *    long as their output and workspace buffers differ.
 *  - Errors are status codes; nothing aborts or throws across the ABI.
 *    dgf_last_error() describes the last non-OK status of the calling thread.
 *    Arguments are validated before any HIP call is made.
 *  - Inputs are finite.  Products, sums and FP16 stage boundaries may still
 *    overflow, and later GEMMs then see infinite operands: the leaf's block
 *    rule makes a product of magnitude 2^128 or more, or an infinity times a
 *    nonzero value, an infinity of its sign, keeps an infinite accumulator over
 *    finite products, and gives the NaN 0xFFC00000 for infinities of both
 *    signs, NaN operands and an infinity times zero; past the leaf, infinities
 *    and NaN propagate through the FP32 operations (a NaN's sign and payload
 *    are not specified).
 */
#ifndef DGF_H
#define DGF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DGF_OK = 0,
    DGF_EINVAL = 1,       /* null required pointer, bad size, leading dim or alignment */
    DGF_EUNSUPPORTED = 2, /* a valid request the library does not implement (e.g. S=3) */
    DGF_EWORKSPACE = 3,   /* workspace missing or smaller than the size query */
    DGF_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} dgf_status;

/* Version of this ABI (incremented on any signature change). */
int dgf_abi_version(void);

/* Leaf width of the canonical tree: 64. */
int dgf_leaf_size(void);

/* Message of the calling thread's last non-OK status ("" if none).  The string
 * is owned by the library and valid until the thread's next call. */
const char *dgf_last_error(void);

/*
 * Forward.  x [M,H] (ldx), W_gate [I,H] (ld_wg), W_up [I,H] (ld_wu),
 * W_down [H,I] (ld_wd) -> y [M,H] (ldy):
 *   g = T_H(x W_gate^T), u = T_H(x W_up^T)           (tree over K = H)
 *   a = bf16(silu(g) * u)                              (one BF16 rounding)
 *   y = T_I(a W_down^T)                                (tree over K = I)
 * g_save, u_save: both NULL (inference) or both non-NULL [M,I] with leading
 * dimension ld_gu (training: the backward needs them).  Training and
 * inference produce the same y bits.
 * Contiguous K shards: calling on shard views (W_gate/W_up rows [i0, i0+Is),
 * W_down columns [i0, i0+Is) with ld_wd = I) returns the shard's partial y,
 * which is the subtree of the unsharded reduction when the shard covers an
 * aligned power-of-two fraction of the leaves; dgf_tree_combine of the S
 * partials in shard order reproduces the unsharded y bit for bit.
 * Workspace: dgf_ffn_fwd_workspace(M,H,I) bytes (may be 0; ws may then be NULL).
 * M = 0 returns DGF_OK without launching.
 */
size_t dgf_ffn_fwd_workspace(int64_t M, int64_t H, int64_t I);
dgf_status dgf_ffn_fwd(const void *x, int64_t ldx,
                       const void *w_gate, int64_t ld_wg,
                       const void *w_up, int64_t ld_wu,
                       const void *w_down, int64_t ld_wd,
                       void *y, int64_t ldy,
                       void *g_save, void *u_save, int64_t ld_gu,
                       int64_t M, int64_t H, int64_t I,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * The forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors as dgf_ffn_fwd (the same
 * kernels, the same bits); the workspace is the library's own static device
 * array of DGF_STATIC_SCRATCH_BYTES, one per GPU, kept until the process
 * ends.  A problem whose dgf_ffn_fwd_workspace(M,H,I) exceeds that size
 * returns DGF_EUNSUPPORTED before anything is enqueued (H=4096, I=12288: up
 * to 128 tokens).  The call allocates nothing and calls no allocating
 * library routine; its first call on a device resolves the array's address
 * there (hipGetSymbolAddress).  Every call on a GPU shares that GPU's array:
 * calls that may overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  Nothing in the array needs clearing
 * between calls: each call writes every scratch byte it reads.
 */
#define DGF_STATIC_SCRATCH_BYTES (16u << 20)
dgf_status dgf_ffn_fwd_static(const void *x, int64_t ldx,
                              const void *w_gate, int64_t ld_wg,
                              const void *w_up, int64_t ld_wu,
                              const void *w_down, int64_t ld_wd,
                              void *y, int64_t ldy,
                              void *g_save, void *u_save, int64_t ld_gu,
                              int64_t M, int64_t H, int64_t I, void *stream);

/*
 * Backward from dY [M,H] (lddy), the input x [M,H] (ldx) and the saved g, u
 * [M,I] (ld_gu), with the same weights as the forward:
 *   dA = T_H(dY W_down)                        (K = H, along the rows of W_down)
 *   dU = bf16(dA silu(g)),  dG = bf16(dA u silu'(g))   (a recomputed)
 *   G  = T_I(dG W_gate),    U  = T_I(dU W_up)          (the two dX lanes)
 *   dX = bf16(G + U)                           (gate contribution first, then up;
 *                                               PR #325 "Communication overlap assessment")
 *   dW_gate = T_M(dG^T x),  dW_up = T_M(dU^T x),  dW_down = T_M(dY^T a)  (K = M)
 * Outputs: dx [M,H] (lddx) or NULL; dx_gate_lane / dx_up_lane [M,H] (lddx)
 * optional (NULL to skip; for I-sharded use the lanes are combined across
 * shards separately and then added gate first, never G_r + U_r per shard);
 * dw_gate [I,H] (ld_dwg), dw_up [I,H] (ld_dwu), dw_down [H,I] (ld_dwd), each
 * non-NULL.  At least one of dx and the two lanes must be given.  dW are fresh
 * tensors (no accumulation into existing gradients).
 * Workspace: dgf_ffn_bwd_workspace(M,H,I) bytes.  M = 0: dX is empty and the
 * three dW are written as +0 (each is the tree over K = M = 0 leaves, as a
 * tree GEMM with K = 0); no workspace is needed and nothing else is launched.
 */
size_t dgf_ffn_bwd_workspace(int64_t M, int64_t H, int64_t I);
dgf_status dgf_ffn_bwd(const void *dy, int64_t lddy,
                       const void *x, int64_t ldx,
                       const void *g, const void *u, int64_t ld_gu,
                       const void *w_gate, int64_t ld_wg,
                       const void *w_up, int64_t ld_wu,
                       const void *w_down, int64_t ld_wd,
                       void *dx, void *dx_gate_lane, void *dx_up_lane, int64_t lddx,
                       void *dw_gate, int64_t ld_dwg,
                       void *dw_up, int64_t ld_dwu,
                       void *dw_down, int64_t ld_dwd,
                       int64_t M, int64_t H, int64_t I,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Fixed balanced combine of S partial results in rank order (PR #357 and
 * PR #356, section "Design"): for S = 8,
 *   out = ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)),
 * every node an FP32 add of two BF16 values rounded to BF16 (the midpoint tree
 * over the parts).  parts: HOST array of S device pointers to n BF16 values
 * each; out: n BF16 values, may alias parts[0] (in place).  S must be 1, 2, 4
 * or 8 (else DGF_EUNSUPPORTED).  n = 0 returns DGF_OK with no launch.  Any
 * alignment is accepted: aligned buffers take a 16-byte vector path, others
 * an element path with the same arithmetic.
 */
dgf_status dgf_tree_combine(const void *const *parts, int S, void *out, int64_t n, void *stream);

/*
 * The same fixed rank tree for other element types (PR #357, section
 * "Determinism and correctness": FP32, FP16 and BF16 follow one rank tree).
 * dtype DGF_BF16 is dgf_tree_combine; DGF_FP16: every node adds its two FP16
 * children in FP32 and rounds the sum to FP16 (nearest even, IEEE subnormals
 * kept, overflow to infinity); DGF_FP32: every node is one FP32 addition.
 * parts/out as for dgf_tree_combine, holding n elements of the dtype; every
 * pointer aligned to the element size (else DGF_EINVAL); 16-byte aligned
 * buffers take the vector path (PR #357, section "Design").  Unknown dtype:
 * DGF_EINVAL.
 */
enum { DGF_BF16 = 0, DGF_FP16 = 1, DGF_FP32 = 2 };
dgf_status dgf_tree_combine_typed(const void *const *parts, int S, void *out, int64_t n, int dtype, void *stream);

/*
 * The FFN in FP16 or BF16 storage (PR #357, section "Determinism and
 * correctness": FP32, FP16 and BF16 follow one tree).  Each *_typed entry
 * point is the entry point of the same name without the suffix, with every
 * 16-bit tensor (inputs, outputs, saved g/u, lanes, workspace contents) of the
 * stored type `dtype`: DGF_BF16 gives exactly the untyped call; DGF_FP16 reads
 * and writes IEEE binary16 bit patterns, computes in FP32 as before, and
 * rounds every leaf, node and stage boundary to FP16 (nearest even, IEEE
 * subnormals, overflow to infinity).  An FP16 leaf is two chained
 * v_mfma_f32_16x16x32_f16, which add their products in the same blocks of 8 as
 * the BF16 instruction (a subnormal operand counts as exponent -14).
 * Arguments, layouts, workspace sizes (the *_workspace queries), ownership
 * and errors as for the untyped call; dtype DGF_FP32 -> DGF_EUNSUPPORTED (no
 * FP32 leaf is declared), any other value -> DGF_EINVAL.  dtype comes right
 * before the stream, as in dgf_tree_combine_typed.
 */
dgf_status dgf_ffn_fwd_typed(const void *x, int64_t ldx, const void *w_gate, int64_t ld_wg, const void *w_up,
                             int64_t ld_wu, const void *w_down, int64_t ld_wd, void *y, int64_t ldy, void *g_save,
                             void *u_save, int64_t ld_gu, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes,
                             int dtype, void *stream);
dgf_status dgf_ffn_bwd_typed(const void *dy, int64_t lddy, const void *x, int64_t ldx, const void *g, const void *u,
                             int64_t ld_gu, const void *w_gate, int64_t ld_wg, const void *w_up, int64_t ld_wu,
                             const void *w_down, int64_t ld_wd, void *dx, void *dx_gate_lane, void *dx_up_lane,
                             int64_t lddx, void *dw_gate, int64_t ld_dwg, void *dw_up, int64_t ld_dwu, void *dw_down,
                             int64_t ld_dwd, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes, int dtype,
                             void *stream);
dgf_status dgf_gemm_tree_typed(int layout, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K, void *ws, size_t ws_bytes, int dtype,
                               void *stream);
dgf_status dgf_act_fwd_typed(const void *g, const void *u, void *a, int64_t n, int dtype, void *stream);
dgf_status dgf_act_bwd_typed(const void *da, const void *g, const void *u, void *dg, void *du, void *a, int64_t n,
                             int dtype, void *stream);

/*
 * Diagnostic entry points (stage isolation and shard emulation; the FFN
 * entry points above are composed of the same kernels).
 *
 * dgf_gemm_tree: C [M,N] (ldc) = canonical tree over K of
 *   layout DGF_NT: A [M,K] (lda) times B [N,K] (ldb) transposed,
 *   layout DGF_NN: A [M,K] (lda) times B [K,N] (ldb),
 *   layout DGF_TN: A [K,M] (lda) transposed times B [K,N] (ldb).
 * K = 0 writes zeros.  Workspace: dgf_gemm_tree_workspace(layout,M,N,K) bytes
 * (0 when none is needed, e.g. DGF_TN with K <= 64, which reads A and B in
 * place; a NULL ws is then accepted).
 */
enum { DGF_NT = 0, DGF_NN = 1, DGF_TN = 2 };
size_t dgf_gemm_tree_workspace(int layout, int64_t M, int64_t N, int64_t K);
dgf_status dgf_gemm_tree(int layout, const void *A, int64_t lda, const void *B, int64_t ldb,
                         void *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                         void *ws, size_t ws_bytes, void *stream);

/* a = bf16(silu(g) * u) over n contiguous elements (sigma with exp(-g)
 * rounded once to FP32, then 1/(1+e), g*sigma, *u, each an FP32 operation). */
dgf_status dgf_act_fwd(const void *g, const void *u, void *a, int64_t n, void *stream);

/* dU = bf16(dA * silu(g)), dG = bf16((dA * u) * silu'(g)) with
 * silu'(g) = sigma (1 + g (1 - sigma)); a (optional, NULL to skip) = bf16(silu(g) u). */
dgf_status dgf_act_bwd(const void *da, const void *g, const void *u,
                       void *dg, void *du, void *a, int64_t n, void *stream);

/*
 * Kernel timing (for benchmarks and profilers).  events: 2*n_pairs hipEvent_t
 * handles created by the caller.  Until dgf_profile_end(), the calling
 * thread's entry points record events[2k] and events[2k+1] as the start and
 * end of their k-th launch step (k < n_pairs; a step is one kernel, or the
 * two of a vector body and its scalar tail), taken from the kernels' own
 * dispatch timestamps, so hipEventElapsedTime gives the step's execution time,
 * on the call's stream, in launch order.  dgf_profile_end() stops recording and returns the number of launches
 * made since dgf_profile_begin (only the first n_pairs were timed);
 * dgf_profile_name(k) names launch k (the string is static; "" when k is out
 * of range) until the next dgf_profile_begin.  The state is thread-local.
 */
dgf_status dgf_profile_begin(void *const *events, int n_pairs);
int dgf_profile_end(void);
const char *dgf_profile_name(int k);

#ifdef __cplusplus
}
#endif

#endif /* DGF_H */
