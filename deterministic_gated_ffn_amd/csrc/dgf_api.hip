// C ABI of libdgf: argument validation, workspace layout and the launch
// sequence of the forward and backward passes (declarations in include/dgf.h).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "dgf.h"
#include "dgf_kernels.hpp"

using namespace dgf;

namespace {

thread_local std::string g_err;

dgf_status fail(dgf_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dgf_status ok() {
  g_err.clear();
  return DGF_OK;
}

dgf_status hip_check(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(DGF_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DGF_OK;
}

}  // namespace

thread_local hipEvent_t dgf::g_launch_events[2] = {nullptr, nullptr};

namespace {

// Kernel timing hook: caller-created events, one pair per launch step (one
// kernel, or a vector body and its scalar tail), recorded as the kernels' own
// start and end timestamps.
struct Prof {
  hipEvent_t *ev = nullptr;
  int pairs = 0;
  int used = 0;
  const char *names[4096] = {};
};
thread_local Prof g_prof;

template <class F>
hipError_t timed(hipStream_t s, const char *name, F &&launch) {
  const int k = g_prof.used;
  const bool rec = g_prof.ev && k < g_prof.pairs;
  if (rec) {  // the launches record them as their kernels' start and end
    g_launch_events[0] = g_prof.ev[2 * k];
    g_launch_events[1] = g_prof.ev[2 * k + 1];
  }
  hipError_t e = launch();
  if (rec) {
    const bool none = g_launch_events[0] != nullptr;  // no kernel took them: an empty interval
    g_launch_events[0] = g_launch_events[1] = nullptr;
    if (none && e == hipSuccess) e = hipEventRecord(g_prof.ev[2 * k], s);
    if (none && e == hipSuccess) e = hipEventRecord(g_prof.ev[2 * k + 1], s);
  }
  if (g_prof.ev) {
    if (k < 4096) g_prof.names[k] = name;
    g_prof.used = k + 1;
  }
  return e;
}

#define DGF_TRY(expr)                  \
  do {                                 \
    dgf_status st_ = (expr);           \
    if (st_ != DGF_OK) return st_;     \
  } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// A row-major BF16 matrix operand: non-null, 16-byte aligned, ld >= cols, ld % 8 == 0.
constexpr int64_t kMaxLd = (int64_t)1 << 23;

dgf_status check_mat(const char *name, const void *p, int64_t ld, int64_t rows, int64_t cols) {
  if (rows == 0 || cols == 0) return DGF_OK;
  if (!p) return fail(DGF_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(DGF_EINVAL, "%s is not 16-byte aligned", name);
  if (ld < cols) return fail(DGF_EINVAL, "%s: leading dimension %lld < row width %lld", name, (long long)ld, (long long)cols);
  if (ld % 8 != 0) return fail(DGF_EINVAL, "%s: leading dimension %lld is not a multiple of 8", name, (long long)ld);
  // a 128-row tile's byte offsets from its first row stay below 2^31
  if (ld >= kMaxLd) return fail(DGF_EUNSUPPORTED, "%s: leading dimension %lld beyond the library's limit (< 2^23)", name, (long long)ld);
  return DGF_OK;
}

dgf_status check_dims(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(DGF_EINVAL, "negative dimension (M=%lld N=%lld K=%lld)", (long long)M, (long long)N, (long long)K);
  if (M > ((int64_t)1 << 21) || N > ((int64_t)1 << 30) || K > ((int64_t)1 << 23))
    return fail(DGF_EUNSUPPORTED, "dimensions beyond the library's limits (M<=2^21, N<=2^30, K<=2^23)");
  return DGF_OK;
}

int64_t round8(int64_t v) { return (v + 7) & ~(int64_t)7; }
size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

int leaves(int64_t K) { return (int)((K + 63) / 64); }

// Depth of the midpoint tree over n leaves: ceil(log2 n).
int tree_depth(int n) {
  int d = 0;
  while ((1 << d) < n) ++d;
  return d;
}

GemmParams blank(int fmt) {
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.fmt = fmt;
  return p;
}

// Public dtype code -> stored type of the kernels: BF16 and FP16 share the
// tree; an FP32 FFN has no declared leaf rule (its MFMA differs), so it is
// rejected as unsupported.
dgf_status stored_type(int dtype, int *fmt) {
  if (dtype == DGF_BF16) { *fmt = FMT_BF16; return DGF_OK; }
  if (dtype == DGF_FP16) { *fmt = FMT_F16; return DGF_OK; }
  if (dtype == DGF_FP32) return fail(DGF_EUNSUPPORTED, "dtype FP32: only BF16 and FP16 storage is implemented here");
  return fail(DGF_EINVAL, "unknown dtype %d", dtype);
}

// Launch shape of one tree GEMM.  A wave owns 16 RT output columns (RT from
// gemm_row_tiles) and 16 MT tokens; a workgroup holds 1, 2 or 4 waves, each on
// its own subtree of the K leaves, and plain-store GEMMs may further split K
// over 2..16 workgroups (subtrees one level deeper each), whose roots a
// combine kernel joins.  A shape is scored by the waves it launches, capped
// at what 256 CUs hold at once (8 waves per CU by registers, fewer when the
// workgroup's LDS, 64 KB at most, leaves room for fewer workgroups in a CU's
// 160 KB); the best score wins, then fewer K pieces, then more waves per
// workgroup.
struct Plan {
  int waves = 1, kdepth = 0, slots = 1;
  size_t lds = 0;
};

constexpr int64_t kCUs = 256;
constexpr size_t kMaxLds = 64 * 1024;

Plan plan_gemm(int layout, int nb, int epi, int64_t M, int64_t N, int64_t K) {
  Plan best;
  if (layout == DGF_LAYOUT_NT && epi == EPI_STORE && K <= 64) return best;  // the one-leaf kernel
  const int L = leaves(K);
  const int mt = M <= 16 ? 1 : 2;
  const int rt = gemm_row_tiles(layout, nb, epi);
  const int np = nb * rt * mt * 2;
  const int64_t tiles = ((N + 16 * rt - 1) / (16 * rt)) * ((M + 16 * mt - 1) / (16 * mt));
  const size_t slab = layout == DGF_LAYOUT_NN ? (size_t)nb * 16 * rt * 64 * 2 : 0;
  const int max_kdepth = epi == EPI_STORE ? 4 : 0;
  constexpr size_t kCuLds = 160 * 1024;
  int64_t best_score = -1;
  for (int kd = 0; kd <= max_kdepth; ++kd) {
    for (int waves = 4; waves >= 1; waves >>= 1) {
      const int depth = kd + tree_depth(waves);
      if ((1 << depth) > (L > 0 ? L : 1)) continue;  // every wave keeps at least one leaf
      const int per_wave = (L + (1 << depth) - 1) >> depth;  // largest subtree at that depth
      Plan pl;
      pl.waves = waves;
      pl.kdepth = kd;
      pl.slots = tree_depth(per_wave) > 1 ? tree_depth(per_wave) : 1;
      pl.lds = (size_t)waves * ((size_t)pl.slots * np * 64 * 4 + slab);
      if (pl.lds > kMaxLds) continue;
      int64_t per_cu = (int64_t)(kCuLds / (pl.lds > 0 ? pl.lds : 1)) * waves;
      if (per_cu > 8) per_cu = 8;
      const int64_t total = tiles * ((int64_t)waves << kd);
      const int64_t score = total < per_cu * kCUs ? total : per_cu * kCUs;
      if (score > best_score) {
        best_score = score;
        best = pl;
      }
    }
  }
  if (best_score < 0) {  // nothing fits: report the smallest shape's LDS
    const int per_wave = L > 0 ? L : 1;
    best.slots = tree_depth(per_wave) > 1 ? tree_depth(per_wave) : 1;
    best.lds = (size_t)best.slots * np * 64 * 4 + slab;
  }
  return best;
}

// Launch shape of the weight-streaming kernel (dgf_xs.hip): up to 8 waves per
// workgroup, the K tree cut at the smallest depth kd that leaves every wave
// at most 4 leaves (or up to two levels deeper when that spreads the output
// tiles more evenly over 256 CUs), and G workgroups per (token tile, product,
// K piece), each looping over ceil(tiles / G) output tiles.  The cost
// compared is the weight bytes of the busiest CU plus the partial roots'
// write and read spread over all CUs.  waves = 0: not applicable (more than
// 32 K pieces would be needed).
struct XsPlan {
  int waves = 0, kd = 0, groups = 0;
  size_t lds = 0;
};

XsPlan plan_xs(int layout, int nb, int64_t M, int64_t N, int64_t K) {
  XsPlan best;
  const int L = leaves(K);
  if (L == 0 || M == 0 || N == 0) return best;
  const int mt = M <= 16 ? 1 : 2;
  int waves = 8;
  while (waves > L) waves >>= 1;
  const int dw = tree_depth(waves);
  int kd_min = 0;
  while (((L + (1 << (kd_min + dw)) - 1) >> (kd_min + dw)) > 4) ++kd_min;
  if (kd_min > 5) return best;
  const int64_t cols = xs_tile_cols(layout, mt);
  const int64_t tiles_n = (N + cols - 1) / cols, tiles_m = (M + 16 * mt - 1) / (16 * mt);
  if (tiles_m > 65535) return best;
  double best_cost = 0;
  for (int kd = kd_min; kd <= kd_min + 2 && kd <= 5 && (1 << (kd + dw)) <= L; ++kd) {
    const int64_t per_piece = tiles_m * nb * ((int64_t)1 << kd);  // (token tile, product, K piece)
    int64_t T = (tiles_n * per_piece + kCUs - 1) / kCUs;
    if (T < 1) T = 1;
    const int64_t G = (tiles_n + T - 1) / T;
    const int64_t tiles_per_wg = (tiles_n + G - 1) / G;
    const int64_t rounds = (G * per_piece + kCUs - 1) / kCUs;
    const int64_t leaves_per_wave = (L + (1 << (kd + dw)) - 1) >> (kd + dw);
    const double cost = (double)rounds * tiles_per_wg * leaves_per_wave * waves * cols * 64 * 2 +
                        (kd > 0 ? 2.0 * nb * ((int64_t)1 << kd) * M * round8(N) * 2 / kCUs : 0.0);
    if (best.waves == 0 || cost < best_cost) {
      best_cost = cost;
      best.waves = waves;
      best.kd = kd;
      best.groups = (int)G;
      best.lds = xs_lds_bytes(layout, mt, waves);
    }
  }
  return best;
}

// Launch shape of the tiled kernel (dgf_mm.hip) for many tokens: the K tree
// cut at the smallest depth kd whose pieces split into at most 8 lower
// subtrees of the kernel's maximum size.  kd = -1: not applicable.
struct MmPlan {
  int kd = -1, up = 0, nlh = 0;
};

constexpr int64_t kMmMinM = 128;  // one full 128-token tile: below it the weights stream

MmPlan plan_mm(int layout, int64_t M, int64_t K) {
  MmPlan pl;
  if (layout != DGF_LAYOUT_NT || M < kMmMinM) return pl;
  const int L = leaves(K);
  for (int kd = 0; kd <= 5 && (1 << kd) <= L; ++kd) {
    const int lmin = L >> kd, lmax = (L + (1 << kd) - 1) >> kd;  // piece sizes
    const int up = mm_upper_levels(lmax);
    if (up < 0 || (1 << up) > lmin) continue;
    pl.kd = kd;
    pl.up = up;
    pl.nlh = (lmax + (1 << up) - 1) >> up;
    return pl;
  }
  return pl;
}

// Workspace bytes for the partial roots of one GEMM (0 when it needs none).
size_t partial_bytes(int layout, int nb, int epi, int64_t M, int64_t N, int64_t K) {
  if (M == 0 || N == 0) return 0;
  if ((layout == DGF_LAYOUT_NT || layout == DGF_LAYOUT_TN) && epi == EPI_STORE && K <= 64) return 0;  // one-leaf kernels
  const MmPlan mp = plan_mm(layout, M, K);
  if (mp.kd >= 0) {
    if (mp.kd == 0 && epi == EPI_STORE) return 0;
    return round256((size_t)nb * ((size_t)1 << mp.kd) * M * round8(N) * 2);
  }
  const XsPlan xp = plan_xs(layout, nb, M, N, K);
  if (xp.waves > 0) {
    if (xp.kd == 0 && epi == EPI_STORE) return 0;
    return round256((size_t)nb * ((size_t)1 << xp.kd) * M * round8(N) * 2);
  }
  const Plan pl = plan_gemm(layout, nb, epi, M, N, K);
  if (pl.kdepth == 0) return 0;
  return round256((size_t)nb * ((size_t)1 << pl.kdepth) * M * round8(N) * 2);
}

// One tree GEMM: the MFMA kernel, then (K split) the combine of the partials.
// `partials` must hold partial_bytes() of workspace.
// defer_join (EPI_DX on the streaming kernel, at most 8 K pieces): the join
// is not launched; its arguments go to *defer_join and deferred is set, for
// the weight-gradient launch to run.  dx_join (TN): that deferred join.
dgf_status run_gemm(int layout, int nb, int epi, GemmParams p, hipStream_t s, const char *what,
                    uint16_t *partials = nullptr, const char *join_what = "K-piece join",
                    GemmParams *defer_join = nullptr, bool *deferred = nullptr, const GemmParams *dx_join = nullptr) {
  if (p.M == 0 || p.N == 0) return DGF_OK;
  if ((p.M + 31) / 32 > 65535 || (p.N + 15) / 16 > 0x7fffffff)
    return fail(DGF_EUNSUPPORTED, "%s: %lld x %lld output exceeds the launch grid", what, (long long)p.M, (long long)p.N);
  p.L = leaves(p.K);
  if (layout == DGF_LAYOUT_TN) {
    if (epi != EPI_STORE || p.K > 64 || (nb == 2 && p.B[1] != p.B[0]) || (p.M + 63) / 64 > 65535)
      return fail(DGF_EUNSUPPORTED, "%s: the TN kernel takes one leaf (K <= 64) and a shared B", what);
    return hip_check(timed(s, what, [&] { return launch_gemm_tn1(nb, p, s, dx_join); }), what);
  }
  if (layout == DGF_LAYOUT_NT && epi == EPI_STORE && p.K <= 64 && (nb == 1 || p.B[1] == p.B[0]) &&
      (p.M + 63) / 64 <= 65535)
    return hip_check(timed(s, what, [&] { return launch_gemm_short(nb, p, s); }), what);
  const MmPlan mp = plan_mm(layout, p.M, p.K);
  if (mp.kd >= 0) {
    p.ksplit_depth = mp.kd;
    p.stack_slots = mp.up;
    const bool joined = mp.kd > 0 || epi != EPI_STORE;  // roots go through the combine kernel
    p.to_part = joined ? 1 : 0;
    if (!joined)
      for (int b = 0; b < nb; ++b)
        if (!p.C[b]) return fail(DGF_EINVAL, "%s: product %d has no output", what, b);
    if (joined) {
      if (!partials) return fail(DGF_EWORKSPACE, "%s: no workspace for the partial roots", what);
      p.part = partials;
      p.ldp = round8(p.N);
      p.part_stride = p.M * p.ldp;
    }
    DGF_TRY(hip_check(timed(s, what, [&] { return launch_mm(p, nb, mp.nlh, s); }), what));
    if (joined)
      DGF_TRY(hip_check(timed(s, join_what, [&] { return launch_combine_epi(epi, nb, p, s); }), join_what));
    return DGF_OK;
  }
  const XsPlan xp = plan_xs(layout, nb, p.M, p.N, p.K);
  if (xp.waves > 0) {
    p.ksplit_depth = xp.kd;
    const bool joined = xp.kd > 0 || epi != EPI_STORE;  // roots go through the combine kernel
    p.to_part = joined ? 1 : 0;
    if (!joined)
      for (int b = 0; b < nb; ++b)
        if (!p.C[b]) return fail(DGF_EINVAL, "%s: product %d has no output", what, b);
    if (joined) {
      if (!partials) return fail(DGF_EWORKSPACE, "%s: no workspace for the partial roots", what);
      p.part = partials;
      p.ldp = round8(p.N);
      p.part_stride = p.M * p.ldp;
    }
    DGF_TRY(hip_check(timed(s, what, [&] { return launch_xs(layout, p, nb, xp.waves, xp.groups, s); }), what));
    if (joined && defer_join && epi == EPI_DX && xp.kd <= 3) {
      *defer_join = p;
      *deferred = true;
      return DGF_OK;
    }
    if (joined)
      DGF_TRY(hip_check(timed(s, join_what, [&] { return launch_combine_epi(epi, nb, p, s); }), join_what));
    return DGF_OK;
  }
  if (epi == EPI_DX) return fail(DGF_EUNSUPPORTED, "%s: K=%lld is too deep for the lane kernel", what, (long long)p.K);
  const Plan pl = plan_gemm(layout, nb, epi, p.M, p.N, p.K);
  p.stack_slots = pl.slots;
  p.ksplit_depth = pl.kdepth;
  if (pl.lds > kMaxLds)
    return fail(DGF_EUNSUPPORTED, "%s: K=%lld needs %zu bytes of LDS for the tree stack", what, (long long)p.K, pl.lds);
  if (pl.kdepth > 0) {
    if (!partials) return fail(DGF_EWORKSPACE, "%s: no workspace for the K-split partials", what);
    p.part = partials;
    p.ldp = round8(p.N);
    p.part_stride = p.M * p.ldp;
  }
  DGF_TRY(hip_check(timed(s, what, [&] { return launch_gemm(layout, nb, epi, p, pl.waves, s); }), what));
  if (pl.kdepth > 0) {
    const int S = 1 << pl.kdepth;
    for (int b = 0; b < nb; ++b)
      DGF_TRY(hip_check(timed(s, "K-split combine", [&] {
                          return launch_combine_2d(p.fmt, p.part + (int64_t)b * S * p.part_stride, p.part_stride, p.ldp, S,
                                                   p.C[b], p.ldc[b], p.M, p.N, s);
                        }),
                        "K-split combine"));
  }
  return DGF_OK;
}

// Zero-fill an [M, N] output (K = 0 products).
__global__ void k_zero2d(uint16_t *C, int64_t ldc, int64_t M, int64_t N) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M * N; i += (int64_t)gridDim.x * blockDim.x)
    C[(i / N) * ldc + (i % N)] = 0;
}

dgf_status zero_mat(uint16_t *C, int64_t ldc, int64_t M, int64_t N, hipStream_t s) {
  if (M == 0 || N == 0) return DGF_OK;
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return hip_check(timed(s, "zero fill", [&] {
                     dgf_launch(k_zero2d, dim3((unsigned)blocks), dim3(256), 0, s, C, ldc, M, N);
                     return hipGetLastError();
                   }),
                   "zero fill");
}

struct Carve {
  char *base;
  size_t used;
  uint16_t *take(size_t elems) {
    uint16_t *p = (uint16_t *)(base + used);
    used += round256(elems * 2);
    return p;
  }
};

// The dX lanes run as one two-product kernel with the ordered add in its join
// when the weight-streaming kernel applies, else as two GEMMs and an add.
bool dx_fused(int64_t M, int64_t H, int64_t I) { return plan_xs(DGF_LAYOUT_NN, 2, M, H, I).waves > 0; }

// The weight gradients (K = M tokens) read the row-major operands directly
// when the tokens fit one leaf; more tokens go through transposed copies and
// the NT tree GEMM.
bool dw_direct(int64_t M) { return M <= 64; }

// Many tokens: dA and the dX lanes run as NT tree GEMMs on the tiled kernel
// over transposed copies of the weights (the streaming kernel would re-read
// every weight once per 32-token tile).
bool nn_tiled(int64_t M) { return M >= kMmMinM; }

size_t bwd_partials(int64_t M, int64_t H, int64_t I) {
  const bool t = nn_tiled(M);
  const size_t sizes[4] = {
      partial_bytes(t ? DGF_LAYOUT_NT : DGF_LAYOUT_NN, 1, EPI_DSILU, M, I, H),                   // dA
      t                 ? partial_bytes(DGF_LAYOUT_NT, 2, EPI_DX, M, H, I)
      : dx_fused(M, H, I) ? partial_bytes(DGF_LAYOUT_NN, 2, EPI_DX, M, H, I)
                          : partial_bytes(DGF_LAYOUT_NN, 1, EPI_STORE, M, H, I),                 // dX lanes
      dw_direct(M) ? 0 : partial_bytes(DGF_LAYOUT_NT, 2, EPI_STORE, I, H, M),                    // dW_gate, dW_up
      dw_direct(M) ? 0 : partial_bytes(DGF_LAYOUT_NT, 1, EPI_STORE, H, I, M)};                   // dW_down
  size_t m = 0;
  for (size_t v : sizes) m = v > m ? v : m;
  return m;
}

size_t bwd_ws_bytes(int64_t M, int64_t H, int64_t I) {
  const int64_t Mp = round8(M);
  return round256((size_t)M * round8(I) * 2) * 3                    // dG, dU, a row-major [M, I] (ld = I rounded to 8)
         + (dw_direct(M) ? 0
                         : round256((size_t)I * Mp * 2) * 3         // dG^T, dU^T, a^T [I, Mp]
                               + round256((size_t)H * Mp * 2) * 2)  // x^T, dY^T [H, Mp]
         + round256((size_t)M * round8(H) * 2) * 2                  // the dX lanes G, U [M, H]
         + (nn_tiled(M) ? round256((size_t)I * round8(H) * 2)        // W_down^T [I, H]
                              + round256((size_t)H * round8(I) * 2) * 2  // W_gate^T, W_up^T [H, I]
                        : 0)
         + bwd_partials(M, H, I);                                   // K-split partial roots
}

size_t fwd_ws_bytes(int64_t M, int64_t H, int64_t I) {
  const size_t gu = gu_act_applies(M, I, H) ? 0 : partial_bytes(DGF_LAYOUT_NT, 2, EPI_ACT, M, I, H);  // gate/up partial roots
  const size_t dn = allk_applies(M, H, I) ? 0 : partial_bytes(DGF_LAYOUT_NT, 1, EPI_STORE, M, H, I);  // down-projection partial roots
  return round256((size_t)M * round8(I) * 2)  // a [M, I]
         + (gu > dn ? gu : dn);               // the gate/up roots are joined before the down GEMM starts
}

size_t gemm_ws_bytes(int layout, int64_t M, int64_t N, int64_t K) {
  const int lay = layout == DGF_NN ? DGF_LAYOUT_NN : DGF_LAYOUT_NT;
  size_t b = partial_bytes(lay, 1, EPI_STORE, M, N, K);
  if (layout != DGF_TN) return b;
  if (K <= 64) return 0;  // the one-leaf TN kernel reads the operands in place
  const int64_t Kp = round8(K);
  return round256((size_t)M * Kp * 2) + round256((size_t)N * Kp * 2) + b;
}

// Library-owned scratch for dgf_ffn_fwd_static: one copy of this array per
// GPU the library runs on, held until the process ends.  Host code never uses
// the array's name as an address: its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = (size_t)DGF_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (resolved on the first call on
// that device, then cached).
dgf_status static_scratch(void **out) {
  int dev = -1;
  DGF_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(DGF_EUNSUPPORTED, "device %d beyond the library's %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    DGF_TRY(hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!ptr || ((uintptr_t)ptr & 255) != 0) return fail(DGF_EHIP, "scratch: bad device address %p", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DGF_OK;
}

}  // namespace

extern "C" {

int dgf_abi_version(void) { return 2; }

int dgf_leaf_size(void) { return 64; }

const char *dgf_last_error(void) { return g_err.c_str(); }

dgf_status dgf_profile_begin(void *const *events, int n_pairs) {
  if (n_pairs < 0 || (n_pairs > 0 && !events)) return fail(DGF_EINVAL, "profile_begin: bad event array");
  for (int i = 0; i < 2 * n_pairs; ++i)
    if (!events[i]) return fail(DGF_EINVAL, "profile_begin: event %d is NULL", i);
  g_prof = Prof{};
  g_prof.ev = n_pairs > 0 ? (hipEvent_t *)events : nullptr;
  g_prof.pairs = n_pairs;
  return ok();
}

int dgf_profile_end(void) {
  const int n = g_prof.used;
  g_prof.ev = nullptr;
  g_prof.pairs = 0;
  return n;
}

const char *dgf_profile_name(int k) {
  if (k < 0 || k >= 4096 || k >= g_prof.used || !g_prof.names[k]) return "";
  return g_prof.names[k];
}

size_t dgf_ffn_fwd_workspace(int64_t M, int64_t H, int64_t I) {
  if (M <= 0 || H <= 0 || I <= 0) return 0;
  return fwd_ws_bytes(M, H, I);
}

}  // extern "C"

namespace {

dgf_status ffn_fwd_impl(int fmt, const void *x, int64_t ldx, const void *w_gate, int64_t ld_wg, const void *w_up,
                        int64_t ld_wu, const void *w_down, int64_t ld_wd, void *y, int64_t ldy, void *g_save,
                        void *u_save, int64_t ld_gu, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes,
                        void *stream) {
  DGF_TRY(check_dims(M, I, H));
  DGF_TRY(check_dims(M, H, I));
  if (H == 0 || I == 0) return fail(DGF_EINVAL, "H and I must be positive (H=%lld I=%lld)", (long long)H, (long long)I);
  if (M == 0) return ok();
  DGF_TRY(check_mat("x", x, ldx, M, H));
  DGF_TRY(check_mat("w_gate", w_gate, ld_wg, I, H));
  DGF_TRY(check_mat("w_up", w_up, ld_wu, I, H));
  DGF_TRY(check_mat("w_down", w_down, ld_wd, H, I));
  DGF_TRY(check_mat("y", y, ldy, M, H));
  if ((g_save == nullptr) != (u_save == nullptr)) return fail(DGF_EINVAL, "g_save and u_save must both be given or both be NULL");
  if (g_save) {
    DGF_TRY(check_mat("g_save", g_save, ld_gu, M, I));
    DGF_TRY(check_mat("u_save", u_save, ld_gu, M, I));
  }
  const size_t need = fwd_ws_bytes(M, H, I);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DGF_EWORKSPACE, "forward workspace: need %zu bytes (16-byte aligned), got %zu", need, ws ? ws_bytes : 0);
  hipStream_t s = (hipStream_t)stream;
  Carve cv{(char *)ws, 0};
  uint16_t *a = cv.take((size_t)M * round8(I));
  const int64_t lda_ = round8(I);
  uint16_t *partials = (uint16_t *)((char *)ws + cv.used);

  if (gu_act_applies(M, I, H)) {
    // one kernel: both projections over all of K per workgroup, then the activation
    GuParams f;
    memset(&f, 0, sizeof f);
    f.x = (const uint16_t *)x; f.ldx = ldx;
    f.w[0] = (const uint16_t *)w_gate; f.ldw[0] = ld_wg;
    f.w[1] = (const uint16_t *)w_up; f.ldw[1] = ld_wu;
    f.a = a; f.lda = lda_;
    f.g = (uint16_t *)g_save; f.u = (uint16_t *)u_save; f.ldgu = ld_gu;
    f.M = M; f.N = I; f.K = H; f.L = leaves(H); f.fmt = fmt;
    DGF_TRY(hip_check(timed(s, "gate/up + act", [&] { return launch_gu_act(f, s); }), "gate/up + act"));
  } else {
    GemmParams p = blank(fmt);
    p.A[0] = p.A[1] = (const uint16_t *)x;
    p.lda[0] = p.lda[1] = ldx;
    p.shared_a = 1;
    p.B[0] = (const uint16_t *)w_gate;
    p.ldb[0] = ld_wg;
    p.B[1] = (const uint16_t *)w_up;
    p.ldb[1] = ld_wu;
    p.C[0] = (uint16_t *)g_save;
    p.C[1] = (uint16_t *)u_save;
    p.ldc[0] = p.ldc[1] = ld_gu;
    p.act_out = a;
    p.ld_act = lda_;
    p.M = M; p.N = I; p.K = H;
    DGF_TRY(run_gemm(DGF_LAYOUT_NT, 2, EPI_ACT, p, s, "gate/up tree GEMM", partials, "gate/up join + act"));
  }

  if (allk_applies(M, H, I)) {
    // every workgroup reduces all of K for its 16 output columns: no partial roots, no join
    AllkParams d;
    memset(&d, 0, sizeof d);
    d.A = a; d.lda = lda_;
    d.B = (const uint16_t *)w_down; d.ldb = ld_wd;
    d.C = (uint16_t *)y; d.ldc = ldy;
    d.M = M; d.N = H; d.K = I; d.L = leaves(I); d.fmt = fmt;
    DGF_TRY(hip_check(timed(s, "down all-K tree GEMM", [&] { return launch_allk(d, s); }), "down all-K tree GEMM"));
    return ok();
  }
  GemmParams q = blank(fmt);
  q.A[0] = a;
  q.lda[0] = lda_;
  q.B[0] = (const uint16_t *)w_down;
  q.ldb[0] = ld_wd;
  q.C[0] = (uint16_t *)y;
  q.ldc[0] = ldy;
  q.M = M; q.N = H; q.K = I;
  DGF_TRY(run_gemm(DGF_LAYOUT_NT, 1, EPI_STORE, q, s, "down tree GEMM", partials, "down join"));
  return ok();
}

}  // namespace

extern "C" {

dgf_status dgf_ffn_fwd(const void *x, int64_t ldx, const void *w_gate, int64_t ld_wg, const void *w_up, int64_t ld_wu,
                       const void *w_down, int64_t ld_wd, void *y, int64_t ldy, void *g_save, void *u_save,
                       int64_t ld_gu, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes, void *stream) {
  return ffn_fwd_impl(FMT_BF16, x, ldx, w_gate, ld_wg, w_up, ld_wu, w_down, ld_wd, y, ldy, g_save, u_save, ld_gu, M, H,
                      I, ws, ws_bytes, stream);
}

dgf_status dgf_ffn_fwd_typed(const void *x, int64_t ldx, const void *w_gate, int64_t ld_wg, const void *w_up,
                             int64_t ld_wu, const void *w_down, int64_t ld_wd, void *y, int64_t ldy, void *g_save,
                             void *u_save, int64_t ld_gu, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes,
                             int dtype, void *stream) {
  int fmt = 0;
  DGF_TRY(stored_type(dtype, &fmt));
  return ffn_fwd_impl(fmt, x, ldx, w_gate, ld_wg, w_up, ld_wu, w_down, ld_wd, y, ldy, g_save, u_save, ld_gu, M, H, I,
                      ws, ws_bytes, stream);
}

dgf_status dgf_ffn_fwd_static(const void *x, int64_t ldx, const void *w_gate, int64_t ld_wg, const void *w_up,
                              int64_t ld_wu, const void *w_down, int64_t ld_wd, void *y, int64_t ldy, void *g_save,
                              void *u_save, int64_t ld_gu, int64_t M, int64_t H, int64_t I, void *stream) {
  DGF_TRY(check_dims(M, I, H));
  DGF_TRY(check_dims(M, H, I));
  if (H == 0 || I == 0) return fail(DGF_EINVAL, "H and I must be positive (H=%lld I=%lld)", (long long)H, (long long)I);
  if (M == 0) return ok();
  const size_t need = fwd_ws_bytes(M, H, I);
  if (need > kStaticScratchBytes)
    return fail(DGF_EUNSUPPORTED, "forward without allocation: needs %zu bytes of scratch, past the library's %zu "
                "(M=%lld, H=%lld, I=%lld); use dgf_ffn_fwd with a workspace", need, kStaticScratchBytes,
                (long long)M, (long long)H, (long long)I);
  void *ws = nullptr;
  DGF_TRY(static_scratch(&ws));
  return dgf_ffn_fwd(x, ldx, w_gate, ld_wg, w_up, ld_wu, w_down, ld_wd, y, ldy, g_save, u_save, ld_gu, M, H, I, ws,
                     kStaticScratchBytes, stream);
}

size_t dgf_ffn_bwd_workspace(int64_t M, int64_t H, int64_t I) {
  if (M <= 0 || H <= 0 || I <= 0) return 0;
  return bwd_ws_bytes(M, H, I);
}

}  // extern "C"

namespace {

dgf_status ffn_bwd_impl(int fmt, const void *dy, int64_t lddy, const void *x, int64_t ldx, const void *g,
                        const void *u, int64_t ld_gu, const void *w_gate, int64_t ld_wg, const void *w_up,
                        int64_t ld_wu, const void *w_down, int64_t ld_wd, void *dx, void *dx_gate_lane,
                        void *dx_up_lane, int64_t lddx, void *dw_gate, int64_t ld_dwg, void *dw_up, int64_t ld_dwu,
                        void *dw_down, int64_t ld_dwd, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes,
                        void *stream) {
  DGF_TRY(check_dims(M, I, H));
  DGF_TRY(check_dims(M, H, I));
  if (H == 0 || I == 0) return fail(DGF_EINVAL, "H and I must be positive (H=%lld I=%lld)", (long long)H, (long long)I);
  if (M == 0) {
    // no tokens: dX is empty, and each weight gradient is the tree over K = M = 0
    // leaves, whose value is +0 (the same as a tree GEMM with K = 0)
    DGF_TRY(check_mat("dw_gate", dw_gate, ld_dwg, I, H));
    DGF_TRY(check_mat("dw_up", dw_up, ld_dwu, I, H));
    DGF_TRY(check_mat("dw_down", dw_down, ld_dwd, H, I));
    hipStream_t s0 = (hipStream_t)stream;
    DGF_TRY(zero_mat((uint16_t *)dw_gate, ld_dwg, I, H, s0));
    DGF_TRY(zero_mat((uint16_t *)dw_up, ld_dwu, I, H, s0));
    DGF_TRY(zero_mat((uint16_t *)dw_down, ld_dwd, H, I, s0));
    return ok();
  }
  DGF_TRY(check_mat("dy", dy, lddy, M, H));
  DGF_TRY(check_mat("x", x, ldx, M, H));
  DGF_TRY(check_mat("g", g, ld_gu, M, I));
  DGF_TRY(check_mat("u", u, ld_gu, M, I));
  DGF_TRY(check_mat("w_gate", w_gate, ld_wg, I, H));
  DGF_TRY(check_mat("w_up", w_up, ld_wu, I, H));
  DGF_TRY(check_mat("w_down", w_down, ld_wd, H, I));
  if (!dx && !dx_gate_lane && !dx_up_lane) return fail(DGF_EINVAL, "no dX output given (dx and both lanes are NULL)");
  if (dx) DGF_TRY(check_mat("dx", dx, lddx, M, H));
  if (dx_gate_lane) DGF_TRY(check_mat("dx_gate_lane", dx_gate_lane, lddx, M, H));
  if (dx_up_lane) DGF_TRY(check_mat("dx_up_lane", dx_up_lane, lddx, M, H));
  DGF_TRY(check_mat("dw_gate", dw_gate, ld_dwg, I, H));
  DGF_TRY(check_mat("dw_up", dw_up, ld_dwu, I, H));
  DGF_TRY(check_mat("dw_down", dw_down, ld_dwd, H, I));
  const size_t need = bwd_ws_bytes(M, H, I);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DGF_EWORKSPACE, "backward workspace: need %zu bytes (16-byte aligned), got %zu", need, ws ? ws_bytes : 0);

  hipStream_t s = (hipStream_t)stream;
  const int64_t Mp = round8(M);
  Carve cv{(char *)ws, 0};
  const int64_t ld_d = round8(I);
  const bool direct = dw_direct(M);
  uint16_t *dG = cv.take((size_t)M * ld_d), *dU = cv.take((size_t)M * ld_d), *a_rm = cv.take((size_t)M * ld_d);
  uint16_t *dGT = nullptr, *dUT = nullptr, *aT = nullptr, *xT = nullptr, *dYT = nullptr;
  if (!direct) {
    dGT = cv.take((size_t)I * Mp); dUT = cv.take((size_t)I * Mp); aT = cv.take((size_t)I * Mp);
    xT = cv.take((size_t)H * Mp); dYT = cv.take((size_t)H * Mp);
  }
  const int64_t ld_lane = round8(H);
  uint16_t *Gw = cv.take((size_t)M * ld_lane), *Uw = cv.take((size_t)M * ld_lane);
  const bool tiled = nn_tiled(M);
  uint16_t *wdT = nullptr, *wgT = nullptr, *wuT = nullptr;
  const int64_t ld_wdT = round8(H), ld_wgT = round8(I);
  if (tiled) {
    wdT = cv.take((size_t)I * ld_wdT);
    wgT = cv.take((size_t)H * ld_wgT);
    wuT = cv.take((size_t)H * ld_wgT);
  }
  uint16_t *partials = (uint16_t *)((char *)ws + cv.used);

  if (tiled) {  // K-contiguous copies of the weights for the NT form of dA and the dX lanes
    DGF_TRY(hip_check(timed(s, "transpose W_down", [&] { return launch_transpose((const uint16_t *)w_down, ld_wd, H, I, wdT, ld_wdT, s); }),
                      "transpose W_down"));
    DGF_TRY(hip_check(timed(s, "transpose W_gate", [&] { return launch_transpose((const uint16_t *)w_gate, ld_wg, I, H, wgT, ld_wgT, s); }),
                      "transpose W_gate"));
    DGF_TRY(hip_check(timed(s, "transpose W_up", [&] { return launch_transpose((const uint16_t *)w_up, ld_wu, I, H, wuT, ld_wgT, s); }),
                      "transpose W_up"));
  }

  if (!direct) {
    DGF_TRY(hip_check(timed(s, "transpose x", [&] { return launch_transpose((const uint16_t *)x, ldx, M, H, xT, Mp, s); }),
                      "transpose x"));
    DGF_TRY(hip_check(timed(s, "transpose dY", [&] { return launch_transpose((const uint16_t *)dy, lddy, M, H, dYT, Mp, s); }),
                      "transpose dY"));
  }

  // dA = T_H(dY W_down) with the dsilu epilogue
  GemmParams p = blank(fmt);
  p.A[0] = (const uint16_t *)dy;
  p.lda[0] = lddy;
  p.B[0] = tiled ? wdT : (const uint16_t *)w_down;
  p.ldb[0] = tiled ? ld_wdT : ld_wd;
  p.M = M; p.N = I; p.K = H;
  p.sg = (const uint16_t *)g;
  p.su = (const uint16_t *)u;
  p.ld_gu = ld_gu;
  p.dG = dG; p.dU = dU; p.a_rm = a_rm; p.ld_d = ld_d;
  DGF_TRY(run_gemm(tiled ? DGF_LAYOUT_NT : DGF_LAYOUT_NN, 1, EPI_DSILU, p, s, "dA tree GEMM", partials, "dA join + dsilu"));
  if (!direct) {  // token-major copies for the weight-gradient GEMMs
    DGF_TRY(hip_check(timed(s, "transpose dG", [&] { return launch_transpose(dG, ld_d, M, I, dGT, Mp, s); }), "transpose dG"));
    DGF_TRY(hip_check(timed(s, "transpose dU", [&] { return launch_transpose(dU, ld_d, M, I, dUT, Mp, s); }), "transpose dU"));
    DGF_TRY(hip_check(timed(s, "transpose a", [&] { return launch_transpose(a_rm, ld_d, M, I, aT, Mp, s); }), "transpose a"));
  }

  // dX lanes G = T_I(dG W_gate), U = T_I(dU W_up) and dX = bf16(G + U), the
  // gate lane first: one two-product GEMM whose join does the ordered add
  // (lanes kept when the caller asks for them), or two GEMMs and an add
  GemmParams dx_join = blank(fmt);
  bool dx_deferred = false;
  if (tiled || dx_fused(M, H, I)) {
    GemmParams q = blank(fmt);
    q.A[0] = dG; q.A[1] = dU;
    q.lda[0] = q.lda[1] = ld_d;
    q.B[0] = tiled ? wgT : (const uint16_t *)w_gate; q.ldb[0] = tiled ? ld_wgT : ld_wg;
    q.B[1] = tiled ? wuT : (const uint16_t *)w_up; q.ldb[1] = tiled ? ld_wgT : ld_wu;
    q.C[0] = (uint16_t *)dx_gate_lane; q.C[1] = (uint16_t *)dx_up_lane;
    q.ldc[0] = q.ldc[1] = lddx;
    q.dx = (uint16_t *)dx; q.lddx = lddx;
    q.M = M; q.N = H; q.K = I;
    // with two token tiles the 2 x 2^kd activation slices are the largest of the
    // streaming launches: each is read by the workgroups of one XCD
    q.xcd_slices = M > 16 ? 1 : 0;
    // with the one-leaf weight gradients the join runs on extra workgroups
    // of the dW_gate/dW_up launch (it reads only the lanes' partial roots)
    DGF_TRY(run_gemm(tiled ? DGF_LAYOUT_NT : DGF_LAYOUT_NN, 2, EPI_DX, q, s, "dX lanes tree GEMM", partials,
                     "dX join + lane add", direct ? &dx_join : nullptr, &dx_deferred));
  } else {
    uint16_t *G = dx_gate_lane ? (uint16_t *)dx_gate_lane : Gw;
    uint16_t *U = dx_up_lane ? (uint16_t *)dx_up_lane : Uw;
    const int64_t ldG = dx_gate_lane ? lddx : ld_lane, ldU = dx_up_lane ? lddx : ld_lane;
    for (int lane_i = 0; lane_i < 2; ++lane_i) {
      GemmParams q = blank(fmt);
      q.A[0] = lane_i == 0 ? dG : dU;
      q.lda[0] = ld_d;
      q.B[0] = (const uint16_t *)(lane_i == 0 ? w_gate : w_up);
      q.ldb[0] = lane_i == 0 ? ld_wg : ld_wu;
      q.C[0] = lane_i == 0 ? G : U;
      q.ldc[0] = lane_i == 0 ? ldG : ldU;
      q.M = M; q.N = H; q.K = I;
      DGF_TRY(run_gemm(DGF_LAYOUT_NN, 1, EPI_STORE, q, s, lane_i == 0 ? "dX gate-lane tree GEMM" : "dX up-lane tree GEMM",
                       partials));
    }
    if (dx)
      DGF_TRY(hip_check(timed(s, "dX ordered add", [&] { return launch_add_lanes(fmt, G, ldG, U, ldU, (uint16_t *)dx, lddx, M, H, s); }),
                        "dX ordered add"));
  }

  // dW_gate = T_M(dG^T x), dW_up = T_M(dU^T x); dW_down = T_M(dY^T a): one
  // leaf over the row-major operands, or NT over the transposed copies
  GemmParams w = blank(fmt);
  w.C[0] = (uint16_t *)dw_gate; w.ldc[0] = ld_dwg;
  w.C[1] = (uint16_t *)dw_up; w.ldc[1] = ld_dwu;
  w.M = I; w.N = H; w.K = M;
  GemmParams v = blank(fmt);
  v.C[0] = (uint16_t *)dw_down; v.ldc[0] = ld_dwd;
  v.M = H; v.N = I; v.K = M;
  if (direct) {
    w.A[0] = dG; w.A[1] = dU;
    w.lda[0] = w.lda[1] = ld_d;
    w.B[0] = w.B[1] = (const uint16_t *)x;
    w.ldb[0] = w.ldb[1] = ldx;
    if (dx_deferred)
      DGF_TRY(run_gemm(DGF_LAYOUT_TN, 2, EPI_STORE, w, s, "dW_gate/dW_up + dX join", nullptr, nullptr, nullptr,
                       nullptr, &dx_join));
    else
      DGF_TRY(run_gemm(DGF_LAYOUT_TN, 2, EPI_STORE, w, s, "dW_gate/dW_up tree GEMM"));
    v.A[0] = (const uint16_t *)dy; v.lda[0] = lddy;
    v.B[0] = a_rm; v.ldb[0] = ld_d;
    if (H % 16 == 0) {
      // the two row halves of dW_down as the kernel's two products over the
      // shared B = a: every staged B tile serves twice the rows, and the
      // launch fits one round of workgroups (each element is still its own
      // one-leaf sum)
      v.M = H / 2;
      v.A[1] = (const uint16_t *)dy + H / 2; v.lda[1] = lddy;
      v.B[1] = a_rm; v.ldb[1] = ld_d;
      v.C[1] = (uint16_t *)dw_down + (H / 2) * ld_dwd; v.ldc[1] = ld_dwd;
      DGF_TRY(run_gemm(DGF_LAYOUT_TN, 2, EPI_STORE, v, s, "dW_down tree GEMM"));
    } else {
      DGF_TRY(run_gemm(DGF_LAYOUT_TN, 1, EPI_STORE, v, s, "dW_down tree GEMM"));
    }
  } else {
    w.A[0] = dGT; w.A[1] = dUT;
    w.lda[0] = w.lda[1] = Mp;
    w.B[0] = w.B[1] = xT;
    w.ldb[0] = w.ldb[1] = Mp;
    DGF_TRY(run_gemm(DGF_LAYOUT_NT, 2, EPI_STORE, w, s, "dW_gate/dW_up tree GEMM", partials));
    v.A[0] = dYT; v.lda[0] = Mp;
    v.B[0] = aT; v.ldb[0] = Mp;
    DGF_TRY(run_gemm(DGF_LAYOUT_NT, 1, EPI_STORE, v, s, "dW_down tree GEMM", partials));
  }
  return ok();
}

}  // namespace

extern "C" {

dgf_status dgf_ffn_bwd(const void *dy, int64_t lddy, const void *x, int64_t ldx, const void *g, const void *u,
                       int64_t ld_gu, const void *w_gate, int64_t ld_wg, const void *w_up, int64_t ld_wu,
                       const void *w_down, int64_t ld_wd, void *dx, void *dx_gate_lane, void *dx_up_lane,
                       int64_t lddx, void *dw_gate, int64_t ld_dwg, void *dw_up, int64_t ld_dwu, void *dw_down,
                       int64_t ld_dwd, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes, void *stream) {
  return ffn_bwd_impl(FMT_BF16, dy, lddy, x, ldx, g, u, ld_gu, w_gate, ld_wg, w_up, ld_wu, w_down, ld_wd, dx,
                      dx_gate_lane, dx_up_lane, lddx, dw_gate, ld_dwg, dw_up, ld_dwu, dw_down, ld_dwd, M, H, I, ws,
                      ws_bytes, stream);
}

dgf_status dgf_ffn_bwd_typed(const void *dy, int64_t lddy, const void *x, int64_t ldx, const void *g, const void *u,
                             int64_t ld_gu, const void *w_gate, int64_t ld_wg, const void *w_up, int64_t ld_wu,
                             const void *w_down, int64_t ld_wd, void *dx, void *dx_gate_lane, void *dx_up_lane,
                             int64_t lddx, void *dw_gate, int64_t ld_dwg, void *dw_up, int64_t ld_dwu, void *dw_down,
                             int64_t ld_dwd, int64_t M, int64_t H, int64_t I, void *ws, size_t ws_bytes, int dtype,
                             void *stream) {
  int fmt = 0;
  DGF_TRY(stored_type(dtype, &fmt));
  return ffn_bwd_impl(fmt, dy, lddy, x, ldx, g, u, ld_gu, w_gate, ld_wg, w_up, ld_wu, w_down, ld_wd, dx, dx_gate_lane,
                      dx_up_lane, lddx, dw_gate, ld_dwg, dw_up, ld_dwu, dw_down, ld_dwd, M, H, I, ws, ws_bytes, stream);
}

dgf_status dgf_tree_combine(const void *const *parts, int S, void *out, int64_t n, void *stream) {
  if (n < 0) return fail(DGF_EINVAL, "negative length %lld", (long long)n);
  if (!(S == 1 || S == 2 || S == 4 || S == 8)) return fail(DGF_EUNSUPPORTED, "S=%d: only 1, 2, 4 or 8 parts", S);
  if (n == 0) return ok();
  if (!parts) return fail(DGF_EINVAL, "parts is NULL");
  if (!out) return fail(DGF_EINVAL, "out is NULL");
  for (int i = 0; i < S; ++i)
    if (!parts[i]) return fail(DGF_EINVAL, "parts[%d] is NULL", i);
  if (((uintptr_t)out & 1) != 0) return fail(DGF_EINVAL, "out is not 2-byte aligned");
  for (int i = 0; i < S; ++i)
    if (((uintptr_t)parts[i] & 1) != 0) return fail(DGF_EINVAL, "parts[%d] is not 2-byte aligned", i);
  hipStream_t s = (hipStream_t)stream;
  DGF_TRY(hip_check(timed(s, "tree_combine", [&] { return launch_combine((const uint16_t *const *)parts, S, (uint16_t *)out, n, s); }),
                    "tree_combine"));
  return ok();
}

dgf_status dgf_tree_combine_typed(const void *const *parts, int S, void *out, int64_t n, int dtype, void *stream) {
  if (n < 0) return fail(DGF_EINVAL, "negative length %lld", (long long)n);
  if (dtype != DGF_BF16 && dtype != DGF_FP16 && dtype != DGF_FP32) return fail(DGF_EINVAL, "unknown dtype %d", dtype);
  if (!(S == 1 || S == 2 || S == 4 || S == 8)) return fail(DGF_EUNSUPPORTED, "S=%d: only 1, 2, 4 or 8 parts", S);
  if (n == 0) return ok();
  if (!parts) return fail(DGF_EINVAL, "parts is NULL");
  if (!out) return fail(DGF_EINVAL, "out is NULL");
  const uintptr_t align = dtype == DGF_FP32 ? 4 : 2;
  for (int i = 0; i < S; ++i)
    if (!parts[i]) return fail(DGF_EINVAL, "parts[%d] is NULL", i);
  if (((uintptr_t)out & (align - 1)) != 0) return fail(DGF_EINVAL, "out is not %d-byte aligned", (int)align);
  for (int i = 0; i < S; ++i)
    if (((uintptr_t)parts[i] & (align - 1)) != 0) return fail(DGF_EINVAL, "parts[%d] is not %d-byte aligned", i, (int)align);
  static_assert(DGF_BF16 == DGF_COMBINE_BF16 && DGF_FP16 == DGF_COMBINE_FP16 && DGF_FP32 == DGF_COMBINE_FP32,
                "dtype codes");
  hipStream_t s = (hipStream_t)stream;
  DGF_TRY(hip_check(timed(s, "tree_combine", [&] { return launch_combine_typed(parts, S, out, n, dtype, s); }),
                    "tree_combine"));
  return ok();
}

size_t dgf_gemm_tree_workspace(int layout, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return gemm_ws_bytes(layout, M, N, K);
}

}  // extern "C"

namespace {

dgf_status gemm_tree_impl(int fmt, int layout, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, void *ws, size_t ws_bytes, void *stream) {
  if (layout != DGF_NT && layout != DGF_NN && layout != DGF_TN) return fail(DGF_EINVAL, "unknown layout %d", layout);
  DGF_TRY(check_dims(M, N, K));
  if (M == 0 || N == 0) return ok();
  DGF_TRY(check_mat("C", C, ldc, M, N));
  hipStream_t s = (hipStream_t)stream;
  if (K == 0) return zero_mat((uint16_t *)C, ldc, M, N, s) == DGF_OK ? ok() : DGF_EHIP;
  if (layout == DGF_NT) {
    DGF_TRY(check_mat("A", A, lda, M, K));
    DGF_TRY(check_mat("B", B, ldb, N, K));
  } else if (layout == DGF_NN) {
    DGF_TRY(check_mat("A", A, lda, M, K));
    DGF_TRY(check_mat("B", B, ldb, K, N));
  } else {
    DGF_TRY(check_mat("A", A, lda, K, M));
    DGF_TRY(check_mat("B", B, ldb, K, N));
  }
  const size_t need = gemm_ws_bytes(layout, M, N, K);
  if (need && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(DGF_EWORKSPACE, "gemm_tree workspace: need %zu bytes (16-byte aligned), got %zu", need, ws ? ws_bytes : 0);

  GemmParams p = blank(fmt);
  p.M = M; p.N = N; p.K = K;
  p.C[0] = (uint16_t *)C;
  p.ldc[0] = ldc;
  if (layout == DGF_TN && K <= 64) {
    p.A[0] = (const uint16_t *)A; p.lda[0] = lda;
    p.B[0] = (const uint16_t *)B; p.ldb[0] = ldb;
    DGF_TRY(run_gemm(DGF_LAYOUT_TN, 1, EPI_STORE, p, s, "TN tree GEMM"));
  } else if (layout == DGF_TN) {
    const int64_t Kp = round8(K);
    Carve cv{(char *)ws, 0};
    uint16_t *AT = cv.take((size_t)M * Kp), *BT = cv.take((size_t)N * Kp);
    uint16_t *partials = (uint16_t *)((char *)ws + cv.used);
    DGF_TRY(hip_check(timed(s, "transpose A", [&] { return launch_transpose((const uint16_t *)A, lda, K, M, AT, Kp, s); }),
                      "transpose A"));
    DGF_TRY(hip_check(timed(s, "transpose B", [&] { return launch_transpose((const uint16_t *)B, ldb, K, N, BT, Kp, s); }),
                      "transpose B"));
    p.A[0] = AT; p.lda[0] = Kp;
    p.B[0] = BT; p.ldb[0] = Kp;
    DGF_TRY(run_gemm(DGF_LAYOUT_NT, 1, EPI_STORE, p, s, "TN tree GEMM", partials));
  } else {
    p.A[0] = (const uint16_t *)A; p.lda[0] = lda;
    p.B[0] = (const uint16_t *)B; p.ldb[0] = ldb;
    DGF_TRY(run_gemm(layout == DGF_NT ? DGF_LAYOUT_NT : DGF_LAYOUT_NN, 1, EPI_STORE, p, s, "tree GEMM", (uint16_t *)ws));
  }
  return ok();
}

dgf_status act_fwd_impl(int fmt, const void *g, const void *u, void *a, int64_t n, void *stream) {
  if (n < 0) return fail(DGF_EINVAL, "negative length");
  if (n == 0) return ok();
  if (!g || !u || !a) return fail(DGF_EINVAL, "NULL pointer");
  if (((uintptr_t)g | (uintptr_t)u | (uintptr_t)a) & 1) return fail(DGF_EINVAL, "pointers must be 2-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  DGF_TRY(hip_check(timed(s, "act_fwd", [&] { return launch_act_fwd(fmt, (const uint16_t *)g, (const uint16_t *)u, (uint16_t *)a, n, s); }),
                    "act_fwd"));
  return ok();
}

dgf_status act_bwd_impl(int fmt, const void *da, const void *g, const void *u, void *dg, void *du, void *a, int64_t n,
                        void *stream) {
  if (n < 0) return fail(DGF_EINVAL, "negative length");
  if (n == 0) return ok();
  if (!da || !g || !u || !dg || !du) return fail(DGF_EINVAL, "NULL pointer");
  if (((uintptr_t)da | (uintptr_t)g | (uintptr_t)u | (uintptr_t)dg | (uintptr_t)du | (uintptr_t)a) & 1)
    return fail(DGF_EINVAL, "pointers must be 2-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  DGF_TRY(hip_check(timed(s, "act_bwd", [&] {
                      return launch_act_bwd(fmt, (const uint16_t *)da, (const uint16_t *)g, (const uint16_t *)u,
                                            (uint16_t *)dg, (uint16_t *)du, (uint16_t *)a, n, s);
                    }),
                    "act_bwd"));
  return ok();
}

}  // namespace

extern "C" {

dgf_status dgf_gemm_tree(int layout, const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, void *ws, size_t ws_bytes, void *stream) {
  return gemm_tree_impl(FMT_BF16, layout, A, lda, B, ldb, C, ldc, M, N, K, ws, ws_bytes, stream);
}

dgf_status dgf_gemm_tree_typed(int layout, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K, void *ws, size_t ws_bytes, int dtype,
                               void *stream) {
  int fmt = 0;
  DGF_TRY(stored_type(dtype, &fmt));
  return gemm_tree_impl(fmt, layout, A, lda, B, ldb, C, ldc, M, N, K, ws, ws_bytes, stream);
}

dgf_status dgf_act_fwd(const void *g, const void *u, void *a, int64_t n, void *stream) {
  return act_fwd_impl(FMT_BF16, g, u, a, n, stream);
}

dgf_status dgf_act_fwd_typed(const void *g, const void *u, void *a, int64_t n, int dtype, void *stream) {
  int fmt = 0;
  DGF_TRY(stored_type(dtype, &fmt));
  return act_fwd_impl(fmt, g, u, a, n, stream);
}

dgf_status dgf_act_bwd(const void *da, const void *g, const void *u, void *dg, void *du, void *a, int64_t n,
                       void *stream) {
  return act_bwd_impl(FMT_BF16, da, g, u, dg, du, a, n, stream);
}

dgf_status dgf_act_bwd_typed(const void *da, const void *g, const void *u, void *dg, void *du, void *a, int64_t n,
                             int dtype, void *stream) {
  int fmt = 0;
  DGF_TRY(stored_type(dtype, &fmt));
  return act_bwd_impl(fmt, da, g, u, dg, du, a, n, stream);
}

}  // extern "C"
