/*
 * CPU oracle for the deterministic gated FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library; the product path never links, calls or
 * falls back to it.  It shares no code, header, table or helper with the HIP
 * library.  It is deliberately plain and slow: one output element is computed
 * by one thread, leaf by leaf, node by node, in the order the method defines.
 *
 * Method (RL-Kernel PR #325 "feat(ffn): add deterministic distributed Triton FFN
 * for ROCm", section "Design"): the bias-free gated Qwen3 FFN
 *     y = W_down . (silu(W_gate . x) * (W_up . x)),   weights in [out, in] layout
 * (section "Operator test matrix"), with every K-reduction evaluated by one
 * canonical tree: FP32 leaves rounded to BF16, and midpoint-split internal
 * nodes that add two BF16 children in FP32 and round to BF16; BF16 stage
 * boundaries are kept in forward and backward.  In backward the gate and up
 * contributions to dHidden stay separate until a final ordered addition, gate
 * first (section "Communication overlap assessment").
 *
 * Readings taken where the pages are silent (each is also listed in the design doc):
 *  - leaf width 64 contiguous K elements; the last leaf holds the K tail;
 *  - midpoint split mid = lo + floor((hi-lo)/2), so 3 leaves = L0 + (L1 + L2);
 *  - all roundings are round-to-nearest-even, denormals kept (no flush);
 *  - the order of FP32 accumulation inside a leaf is the matrix-core block rule
 *    of oracle_block_step() below: the leaf consumes its K elements in
 *    ascending blocks of 8, each block adding its 8 exact products to the FP32
 *    running value with one rounding (parity of this choice is unpinned by the
 *    pages; it is pinned by hand-worked cases in the tests);
 *  - FP16 (PR #357 "[PERF][distributed]: optimize deterministic ROCm
 *    collectives with HIP IPC", section "Determinism and correctness": FP32,
 *    FP16 and BF16 follow one tree): the same leaf, tree and stages with FP16
 *    storage; every rounding to the stored type is FP16 nearest even with IEEE
 *    subnormals and overflow to infinity, and the leaf uses the same block
 *    rule with FP16's exponents (a subnormal counts as exponent -14);
 *  - silu(g) = g * sigma(g), sigma(g) = 1 / (1 + e), e = exp(-g) correctly
 *    rounded to FP32, each FP32 operation rounded separately (no contraction);
 *    the activation is rounded to BF16 once: a = bf16(fl32(silu(g) * u)).
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

typedef uint16_t bf16_t;
typedef uint16_t f16_t;

/* ---------------------------------------------------------------- BF16 <-> FP32 */

static float bf16_to_f32(bf16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest-even FP32 -> BF16: add 0x7FFF plus the lowest kept bit, then
 * drop the low 16 bits (a carry into the exponent is the correct rounding up). */
static bf16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (bf16_t)((u >> 16) | 0x0040u); /* quiet NaN */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

/* One node of the tree: two BF16 children added in FP32, rounded to BF16. */
static bf16_t node_add(bf16_t l, bf16_t r)
{
    float s = bf16_to_f32(l) + bf16_to_f32(r);
    return f32_to_bf16(s);
}

/* ---------------------------------------------------------------- FP16 <-> FP32 */

/* IEEE binary16 -> FP32 (exact): sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 holds subnormals (fraction * 2^-24). */
static float f16_to_f32(f16_t h)
{
    int sign = (h >> 15) & 1, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return (float)(sign ? -v : v);
}

/* FP32 -> IEEE binary16, round to nearest even.  The magnitude is split into
 * the FP16 step q at its binade (2^(e-10) for normals, 2^-24 below 2^-14), the
 * quotient |x| / q (exact in double) is rounded to an integer with ties to
 * even, and the integer is re-encoded; 65520 and above overflow to infinity. */
static f16_t f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    f16_t sign = (f16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (f16_t)(sign | 0x7E00u);
    double a = fabs((double)x);
    if (a >= 65520.0) return (f16_t)(sign | 0x7C00u);
    int e = a > 0 ? ilogb(a) : -25;          /* binade of |x| */
    if (e < -14) e = -14;                     /* subnormal range shares the 2^-24 step */
    double q = ldexp(1.0, e - 10);
    double m = a / q;                         /* exact: a power-of-two divisor */
    double r = floor(m), frac = m - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    /* r in [0, 2048]; 2048 carries into the next binade */
    if (r >= 2048.0) { r = 1024.0; e += 1; }
    if (e == -14 && r < 1024.0) return (f16_t)(sign | (f16_t)r);        /* subnormal (or zero) */
    return (f16_t)(sign | (f16_t)((e + 15) << 10) | (f16_t)((int)r - 1024));
}

/* ---------------------------------------------------------------- stored types */

/* The stored 16-bit element types (codes as for the typed combine). */
enum { DT_BF16 = 0, DT_FP16 = 1 };

static float elem_to_f32(int dt, uint16_t h) { return dt == DT_FP16 ? f16_to_f32(h) : bf16_to_f32(h); }
static uint16_t f32_to_elem(int dt, float f) { return dt == DT_FP16 ? f32_to_f16(f) : f32_to_bf16(f); }

/* One node of the tree in either type: two children added in FP32, the sum
 * rounded to the stored type. */
static uint16_t node_add_t(int dt, uint16_t l, uint16_t r)
{
    float s = elem_to_f32(dt, l) + elem_to_f32(dt, r);
    return f32_to_elem(dt, s);
}

/* ------------------------------------------------------------ exact integer tools */

typedef __int128 i128;

static int bitlen_u128(unsigned __int128 v)
{
    int n = 0;
    while (v) { v >>= 1; ++n; }
    return n;
}

/* floor(v / 2^s) for s >= 0 (toward minus infinity). */
static i128 floor_shift(i128 v, int s)
{
    if (s <= 0) return v;
    if (s >= 126) return v < 0 ? -1 : 0;
    i128 d = (i128)1 << s;
    i128 q = v / d;              /* truncates toward zero */
    if (v < 0 && q * d != v) q -= 1;
    return q;
}

/* trunc(v / 2^s) for s >= 0 (toward zero). */
static int64_t trunc_shift(int64_t v, int s)
{
    if (s <= 0) return v;
    if (s >= 63) return 0;
    int64_t m = v < 0 ? -v : v;
    m >>= s;
    return v < 0 ? -m : m;
}

/* Round the exact value v * 2^e (v a signed integer, |v| < 2^100) to the
 * nearest FP32, ties to even, with gradual underflow and overflow to infinity. */
static float round_to_f32(i128 v, int e)
{
    if (v == 0) return 0.0f;
    int neg = v < 0;
    unsigned __int128 m = neg ? (unsigned __int128)(-v) : (unsigned __int128)v;
    int lead = bitlen_u128(m) - 1 + e;           /* exponent of the leading bit */
    int q = lead - 23;                           /* exponent of the FP32 ulp */
    if (q < -149) q = -149;
    int s = q - e;                               /* bits to drop */
    if (s > 0) {
        if (s > 101) {
            m = 0;                               /* m < 2^100 < half an ulp */
        } else {
            unsigned __int128 hi = m >> s;
            unsigned __int128 rem = m - (hi << s);
            unsigned __int128 half = (unsigned __int128)1 << (s - 1);
            if (rem > half || (rem == half && (hi & 1))) hi += 1;
            m = hi;
        }
        e = q;
    }
    /* m * 2^e is now exactly representable unless it overflowed */
    double d = ldexp((double)m, e);               /* m < 2^25: exact in double */
    if (d >= 3.4028235677973366e38) return neg ? -INFINITY : INFINITY;
    float f = (float)d;                          /* exact */
    return neg ? -f : f;
}

/* ------------------------------------------------------------ the FP32 leaf */

/* Split a finite stored value into a signed integer significand and an
 * exponent so that value = sig * 2^(ex - F), F the type's fraction width (BF16
 * 7, FP16 10); zero returns 0.  Subnormals take the smallest normal exponent
 * (BF16 -126, FP16 -14). */
static int elem_split(int dt, uint16_t h, int32_t *sig, int *ex)
{
    const int fb = dt == DT_FP16 ? 10 : 7;          /* fraction bits */
    const int eb = dt == DT_FP16 ? 5 : 8;           /* exponent bits */
    const int bias = (1 << (eb - 1)) - 1;
    int be = (h >> fb) & ((1 << eb) - 1);
    int32_t m = h & ((1 << fb) - 1);
    if (be == 0 && m == 0) return 0;
    if (be == 0) *ex = 1 - bias;
    else { *ex = be - bias; m |= 1 << fb; }
    *sig = (h & 0x8000) ? -m : m;
    return 1;
}

/* Class of a stored value: 0 finite, 1 infinity, 2 NaN. */
static int elem_special(int dt, uint16_t h)
{
    const uint16_t emask = dt == DT_FP16 ? 0x7C00 : 0x7F80;
    if ((h & emask) != emask) return 0;
    return (h & (uint16_t)~(emask | 0x8000)) ? 2 : 1;
}

/* Split a finite FP32 so that value = sig * 2^(ex - 23); zero returns 0. */
static int f32_split(float f, int64_t *sig, int *ex)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    int be = (u >> 23) & 0xFF;
    int64_t m = u & 0x7FFFFF;
    if (be == 0 && m == 0) return 0;
    if (be == 0) *ex = -126;
    else { *ex = be - 127; m |= 0x800000; }
    *sig = (u & 0x80000000u) ? -m : m;
    return 1;
}

/*
 * One block step of the FP32 leaf: acc + (a[0]*b[0] + ... + a[n-1]*b[n-1]),
 * n <= 8, evaluated with the matrix-core alignment rule:
 *   1. every product a_k*b_k is exact; its nominal exponent is ea+eb;
 *   2. the block's grid is 2^(E-24), E the largest nominal exponent among the
 *      nonzero products (a block of zero products leaves acc unchanged);
 *   3. each product is cut to the grid toward zero, the accumulator is cut to
 *      the grid toward minus infinity;
 *   4. the exact sum T of the cut terms is cut toward minus infinity to 8 bits
 *      below its own FP32 ulp (never finer than 2^-157);
 *   5. that value is rounded to FP32, nearest even.
 * A zero result is always +0: a block of zero products turns a -0 accumulator
 * into +0, and a negative sum that rounds to zero gives +0, not -0.
 * Past FP32's range: a product of magnitude 2^128 or more is an infinity of its
 * sign before any sum, and so is the product of an infinite operand and a
 * nonzero one; an infinite accumulator passes a block of finite products
 * unchanged; infinities of both signs, a NaN operand or accumulator, and an
 * infinity times zero give the NaN 0xFFC00000.
 * The rule is the same for BF16 and FP16 operands; only the split differs.
 */
static float nan_f32(void)
{
    const uint32_t u = 0xFFC00000u;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float block_step_t(int dt, float acc, const uint16_t *a, ptrdiff_t sa,
                          const uint16_t *b, ptrdiff_t sb, int n)
{
    const int fb = dt == DT_FP16 ? 10 : 7;
    int32_t psig[8];
    int pexp[8], nz[8];
    int emax = -100000, any = 0;
    int pinf = 0, ninf = 0, anynan = isnan(acc);
    for (int k = 0; k < n; ++k) {
        int32_t sa_, sb_;
        int ea, eb;
        const uint16_t ak = a[k * sa], bk = b[k * sb];
        const int ca = elem_special(dt, ak), cb = elem_special(dt, bk);
        if (ca || cb) {                         /* an infinite or NaN operand */
            nz[k] = 0;
            if (ca == 2 || cb == 2 || (ak & 0x7FFF) == 0 || (bk & 0x7FFF) == 0) anynan = 1;
            else if ((ak ^ bk) & 0x8000) ninf = 1;
            else pinf = 1;
            continue;
        }
        nz[k] = elem_split(dt, ak, &sa_, &ea) & elem_split(dt, bk, &sb_, &eb);
        if (!nz[k]) continue;
        psig[k] = sa_ * sb_;                    /* |psig| < 2^(2fb+2) */
        pexp[k] = ea + eb;                      /* product = psig * 2^(pexp-2fb) */
        if (pexp[k] > emax) emax = pexp[k];
        any = 1;
    }
    if (anynan) return nan_f32();
    /* products of magnitude >= 2^128 are infinite */
    for (int k = 0; k < n; ++k) {
        if (!nz[k]) continue;
        const uint32_t mag = (uint32_t)(psig[k] < 0 ? -psig[k] : psig[k]);
        int lead = 31 - __builtin_clz(mag) + pexp[k] - 2 * fb;
        if (lead >= 128) {
            if (psig[k] > 0) pinf = 1;
            else ninf = 1;
        }
    }
    if (pinf && ninf) return nan_f32();
    if (isinf(acc)) {
        if ((acc > 0 && ninf) || (acc < 0 && pinf)) return nan_f32();
        return acc;
    }
    if (pinf) return INFINITY;
    if (ninf) return -INFINITY;
    if (!any) return acc == 0.0f ? 0.0f : acc;  /* a -0 accumulator comes out +0 */
    const int grid = emax - 24;                 /* grid exponent */

    int64_t sp = 0;                             /* products, in grid units */
    for (int k = 0; k < n; ++k) {
        if (!nz[k]) continue;
        int sh = (pexp[k] - 2 * fb) - grid;     /* = 24 - 2fb - (emax - pexp) */
        if (sh >= 0) sp += (int64_t)psig[k] << sh;
        else sp += trunc_shift(psig[k], -sh);
    }

    int64_t csig;
    int cex;
    i128 t;
    if (f32_split(acc, &csig, &cex)) {
        int sh = (cex - 23) - grid;
        if (sh > 64) {
            /* The accumulator dominates: |sp| < 2^29 while the cut in step 4 is
             * at least 2^(sh-9) grid units, so steps 4-5 return acc itself. */
            return acc;
        }
        i128 ct = sh >= 0 ? ((i128)csig << sh) : floor_shift((i128)csig, -sh);
        t = ct + (i128)sp;
    } else {
        t = (i128)sp;
    }
    if (t == 0) return 0.0f;

    /* step 4: cut toward minus infinity to 8 bits below the FP32 ulp of T */
    unsigned __int128 mag = t < 0 ? (unsigned __int128)(-t) : (unsigned __int128)t;
    int lead = bitlen_u128(mag) - 1 + grid;
    int cut = lead - 31;
    if (cut < -157) cut = -157;
    int e = grid;
    if (cut > e) {
        t = floor_shift(t, cut - e);
        e = cut;
    }
    const float r = round_to_f32(t, e);
    return r == 0.0f ? 0.0f : r;                /* a sum that rounds to zero is +0 */
}

float oracle_block_step_t(int dt, float acc, const uint16_t *a, ptrdiff_t sa,
                          const uint16_t *b, ptrdiff_t sb, int n)
{
    return block_step_t(dt, acc, a, sa, b, sb, n);
}

float oracle_block_step(float acc, const bf16_t *a, ptrdiff_t sa,
                        const bf16_t *b, ptrdiff_t sb, int n)
{
    return block_step_t(DT_BF16, acc, a, sa, b, sb, n);
}

/* The FP32 leaf over n <= 64 consecutive K elements: ascending blocks of 8
 * starting from an accumulator of +0. */
static float leaf_f32(int dt, const uint16_t *a, ptrdiff_t sa, const uint16_t *b, ptrdiff_t sb, int64_t n)
{
    float acc = 0.0f;
    for (int64_t k = 0; k < n; k += 8) {
        int w = (int)(n - k < 8 ? n - k : 8);
        acc = block_step_t(dt, acc, a + k * sa, sa, b + k * sb, sb, w);
    }
    return acc;
}

/* Block steps of 8 in ascending k from an accumulator acc0 (the chain a
 * matrix-core instruction sequence applies to one output): row r of the
 * [n][k] arrays a and b against acc0[r], into out[r]. */
void oracle_block_chains_t(int dt, const float *acc0, const uint16_t *a, const uint16_t *b, float *out,
                           int64_t n, int k)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        float acc = acc0[r];
        for (int kb = 0; kb < k; kb += 8) {
            int w = k - kb < 8 ? k - kb : 8;
            acc = block_step_t(dt, acc, a + r * k + kb, 1, b + r * k + kb, 1, w);
        }
        out[r] = acc;
    }
}

float oracle_leaf_f32_t(int dt, const uint16_t *a, ptrdiff_t sa, const uint16_t *b, ptrdiff_t sb, int64_t n)
{
    return leaf_f32(dt, a, sa, b, sb, n);
}

float oracle_leaf_f32(const bf16_t *a, ptrdiff_t sa, const bf16_t *b, ptrdiff_t sb, int64_t n)
{
    return leaf_f32(DT_BF16, a, sa, b, sb, n);
}

/* ------------------------------------------------------------ the tree */

enum { LEAF = 64 };

/* T(lo, hi) over leaves [lo, hi): a single leaf is the FP32 leaf rounded to
 * the stored type; otherwise split at mid = lo + floor((hi - lo) / 2) and add
 * the two children in FP32, rounding to the stored type. */
static uint16_t tree(int dt, const uint16_t *a, ptrdiff_t sa, const uint16_t *b, ptrdiff_t sb,
                     int64_t K, int64_t lo, int64_t hi)
{
    if (hi - lo == 1) {
        int64_t k0 = lo * LEAF;
        int64_t n = K - k0 < LEAF ? K - k0 : LEAF;
        return f32_to_elem(dt, leaf_f32(dt, a + k0 * sa, sa, b + k0 * sb, sb, n));
    }
    int64_t mid = lo + (hi - lo) / 2;
    uint16_t l = tree(dt, a, sa, b, sb, K, lo, mid);
    uint16_t r = tree(dt, a, sa, b, sb, K, mid, hi);
    return node_add_t(dt, l, r);
}

/* One output element: the canonical tree over K of a[k*sa] * b[k*sb].
 * K = 0 gives +0. */
uint16_t oracle_dot_tree_t(int dt, const uint16_t *a, ptrdiff_t sa, const uint16_t *b, ptrdiff_t sb, int64_t K)
{
    if (K <= 0) return 0;
    int64_t L = (K + LEAF - 1) / LEAF;
    return tree(dt, a, sa, b, sb, K, 0, L);
}

bf16_t oracle_dot_tree(const bf16_t *a, ptrdiff_t sa, const bf16_t *b, ptrdiff_t sb, int64_t K)
{
    return oracle_dot_tree_t(DT_BF16, a, sa, b, sb, K);
}

/* The tree over the leaves [leaf_lo, leaf_hi) of a length-K reduction: the
 * partial a contiguous K shard contributes (a subtree when the shard is one). */
uint16_t oracle_dot_subtree_t(int dt, const uint16_t *a, ptrdiff_t sa, const uint16_t *b, ptrdiff_t sb,
                              int64_t K, int64_t leaf_lo, int64_t leaf_hi)
{
    return tree(dt, a, sa, b, sb, K, leaf_lo, leaf_hi);
}

bf16_t oracle_dot_subtree(const bf16_t *a, ptrdiff_t sa, const bf16_t *b, ptrdiff_t sb,
                          int64_t K, int64_t leaf_lo, int64_t leaf_hi)
{
    return tree(DT_BF16, a, sa, b, sb, K, leaf_lo, leaf_hi);
}

/* C[m*ldc + n] = T_K( sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn] ). */
void oracle_gemm_tree_t(int dt, const uint16_t *A, int64_t sam, int64_t sak,
                        const uint16_t *B, int64_t sbk, int64_t sbn,
                        uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            C[m * ldc + n] = oracle_dot_tree_t(dt, A + m * sam, sak, B + n * sbn, sbk, K);
}

void oracle_gemm_tree(const bf16_t *A, int64_t sam, int64_t sak,
                      const bf16_t *B, int64_t sbk, int64_t sbn,
                      bf16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K)
{
    oracle_gemm_tree_t(DT_BF16, A, sam, sak, B, sbk, sbn, C, ldc, M, N, K);
}

/* The fixed balanced combine over S in {1,2,4,8} parts, in rank order:
 * ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)), every node BF16-rounded; this is the
 * midpoint tree over the parts (PR #357 "Design"; PR #356 "Design"). */
static bf16_t combine_range(const bf16_t *const *parts, int64_t i, int lo, int hi)
{
    if (hi - lo == 1) return parts[lo][i];
    int mid = lo + (hi - lo) / 2;
    return node_add(combine_range(parts, i, lo, mid), combine_range(parts, i, mid, hi));
}

int oracle_tree_combine(const bf16_t *const *parts, int S, bf16_t *out, int64_t n)
{
    if (!(S == 1 || S == 2 || S == 4 || S == 8)) return 2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = combine_range(parts, i, 0, S);
    return 0;
}

/* ------------------------------------------------------------ FP16 and FP32 combine */


/* The same fixed rank tree in FP16 and FP32 (PR #357, "Determinism and
 * correctness": FP32, FP16 and BF16 follow one rank tree).  An FP16 node adds
 * its two children in FP32 and rounds the sum to FP16 (nearest even), as the
 * BF16 node does; an FP32 node is one FP32 addition. */

static f16_t node_add_f16(f16_t l, f16_t r)
{
    float s = f16_to_f32(l) + f16_to_f32(r);
    return f32_to_f16(s);
}

static f16_t combine_range_f16(const f16_t *const *parts, int64_t i, int lo, int hi)
{
    if (hi - lo == 1) return parts[lo][i];
    int mid = lo + (hi - lo) / 2;
    return node_add_f16(combine_range_f16(parts, i, lo, mid), combine_range_f16(parts, i, mid, hi));
}

static float combine_range_f32(const float *const *parts, int64_t i, int lo, int hi)
{
    if (hi - lo == 1) return parts[lo][i];
    int mid = lo + (hi - lo) / 2;
    return combine_range_f32(parts, i, lo, mid) + combine_range_f32(parts, i, mid, hi);
}

/* dtype 0: BF16, 1: FP16, 2: FP32 (element bit patterns in and out) */
int oracle_tree_combine_typed(const void *const *parts, int S, void *out, int64_t n, int dtype)
{
    if (!(S == 1 || S == 2 || S == 4 || S == 8)) return 2;
    if (dtype == 0) return oracle_tree_combine((const bf16_t *const *)parts, S, (bf16_t *)out, n);
    if (dtype == 1) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) ((f16_t *)out)[i] = combine_range_f16((const f16_t *const *)parts, i, 0, S);
        return 0;
    }
    if (dtype == 2) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) ((float *)out)[i] = combine_range_f32((const float *const *)parts, i, 0, S);
        return 0;
    }
    return 3;
}

float oracle_f16_to_f32(uint16_t h) { return f16_to_f32(h); }
uint16_t oracle_f32_to_f16(float x) { return f32_to_f16(x); }

/* ------------------------------------------------------------ activation */

/* e = exp(-g) rounded once to FP32 (computed in double, then rounded). */
static float exp_neg_f32(float g)
{
    return (float)exp(-(double)g);
}

float oracle_sigma(float g)
{
    float e = exp_neg_f32(g);
    float den = 1.0f + e;
    return 1.0f / den;
}

float oracle_silu(float g)
{
    float sg = oracle_sigma(g);
    return g * sg;
}

/* silu'(g) = sigma * (1 + g * (1 - sigma)), FP32 step by step. */
float oracle_dsilu(float g)
{
    float sg = oracle_sigma(g);
    float one_m = 1.0f - sg;
    float t = g * one_m;
    float onep = 1.0f + t;
    return sg * onep;
}

/* a = rnd(silu(g) * u), one rounding to the stored type. */
void oracle_act_fwd_t(int dt, const uint16_t *g, const uint16_t *u, uint16_t *a, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float s = oracle_silu(elem_to_f32(dt, g[i]));
        a[i] = f32_to_elem(dt, s * elem_to_f32(dt, u[i]));
    }
}

void oracle_act_fwd(const bf16_t *g, const bf16_t *u, bf16_t *a, int64_t n)
{
    oracle_act_fwd_t(DT_BF16, g, u, a, n);
}

/* dU = rnd(dA * silu(g)), dG = rnd((dA * u) * silu'(g)); a is recomputed. */
void oracle_act_bwd_t(int dt, const uint16_t *da, const uint16_t *g, const uint16_t *u,
                      uint16_t *dg, uint16_t *du, uint16_t *a, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float gv = elem_to_f32(dt, g[i]), uv = elem_to_f32(dt, u[i]), dav = elem_to_f32(dt, da[i]);
        float s = oracle_silu(gv);
        float ds = oracle_dsilu(gv);
        du[i] = f32_to_elem(dt, dav * s);
        float dau = dav * uv;
        dg[i] = f32_to_elem(dt, dau * ds);
        if (a) a[i] = f32_to_elem(dt, s * uv);
    }
}

void oracle_act_bwd(const bf16_t *da, const bf16_t *g, const bf16_t *u,
                    bf16_t *dg, bf16_t *du, bf16_t *a, int64_t n)
{
    oracle_act_bwd_t(DT_BF16, da, g, u, dg, du, a, n);
}

/* ------------------------------------------------------------ the FFN */

/* Forward: g = T_H(x W_gate^T), u = T_H(x W_up^T), a = rnd(silu(g) u),
 * y = T_I(a W_down^T).  Row-major, contiguous: x [M,H], W_gate/W_up [I,H],
 * W_down [H,I]; g, u, a [M,I]; y [M,H]. */
void oracle_ffn_fwd_t(int dt, const uint16_t *x, const uint16_t *wg, const uint16_t *wu, const uint16_t *wd,
                      uint16_t *g, uint16_t *u, uint16_t *a, uint16_t *y,
                      int64_t M, int64_t H, int64_t I)
{
    oracle_gemm_tree_t(dt, x, H, 1, wg, 1, H, g, I, M, I, H);
    oracle_gemm_tree_t(dt, x, H, 1, wu, 1, H, u, I, M, I, H);
    oracle_act_fwd_t(dt, g, u, a, M * I);
    oracle_gemm_tree_t(dt, a, I, 1, wd, 1, I, y, H, M, H, I);
}

void oracle_ffn_fwd(const bf16_t *x, const bf16_t *wg, const bf16_t *wu, const bf16_t *wd,
                    bf16_t *g, bf16_t *u, bf16_t *a, bf16_t *y,
                    int64_t M, int64_t H, int64_t I)
{
    oracle_ffn_fwd_t(DT_BF16, x, wg, wu, wd, g, u, a, y, M, H, I);
}

/* Backward from dY [M,H] and the saved g, u:
 *   dA = T_H(dY W_down)                 (K = H, over the rows of W_down)
 *   dU = rnd(dA silu(g)), dG = rnd(dA u silu'(g)), a recomputed
 *   G  = T_I(dG W_gate), U = T_I(dU W_up),  dX = rnd(G + U)  (gate first)
 *   dW_gate = T_M(dG^T x), dW_up = T_M(dU^T x), dW_down = T_M(dY^T a). */
void oracle_ffn_bwd_t(int dt, const uint16_t *dy, const uint16_t *x, const uint16_t *g, const uint16_t *u,
                      const uint16_t *wg, const uint16_t *wu, const uint16_t *wd,
                      uint16_t *da, uint16_t *dg, uint16_t *du, uint16_t *a,
                      uint16_t *gl, uint16_t *ul, uint16_t *dx,
                      uint16_t *dwg, uint16_t *dwu, uint16_t *dwd,
                      int64_t M, int64_t H, int64_t I)
{
    oracle_gemm_tree_t(dt, dy, H, 1, wd, I, 1, da, I, M, I, H);
    oracle_act_bwd_t(dt, da, g, u, dg, du, a, M * I);
    oracle_gemm_tree_t(dt, dg, I, 1, wg, H, 1, gl, H, M, H, I);
    oracle_gemm_tree_t(dt, du, I, 1, wu, H, 1, ul, H, M, H, I);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M * H; ++i) {
        uint16_t acc = gl[i];                /* gate contribution first */
        acc = node_add_t(dt, acc, ul[i]);    /* then the up contribution */
        dx[i] = acc;
    }
    oracle_gemm_tree_t(dt, dg, 1, I, x, H, 1, dwg, H, I, H, M);
    oracle_gemm_tree_t(dt, du, 1, I, x, H, 1, dwu, H, I, H, M);
    oracle_gemm_tree_t(dt, dy, 1, H, a, I, 1, dwd, I, H, I, M);
}

void oracle_ffn_bwd(const bf16_t *dy, const bf16_t *x, const bf16_t *g, const bf16_t *u,
                    const bf16_t *wg, const bf16_t *wu, const bf16_t *wd,
                    bf16_t *da, bf16_t *dg, bf16_t *du, bf16_t *a,
                    bf16_t *gl, bf16_t *ul, bf16_t *dx,
                    bf16_t *dwg, bf16_t *dwu, bf16_t *dwd,
                    int64_t M, int64_t H, int64_t I)
{
    oracle_ffn_bwd_t(DT_BF16, dy, x, g, u, wg, wu, wd, da, dg, du, a, gl, ul, dx, dwg, dwu, dwd, M, H, I);
}

int oracle_leaf_size(void) { return LEAF; }
