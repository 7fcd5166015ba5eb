// Join of the K-piece partial roots of a tree GEMM with its epilogue (gfx950).
//
// The 2^kd partial roots of an output element are the roots of the K pieces,
// contiguous subtrees of the canonical midpoint tree over the leaves (RL-Kernel
// PR #325, section "Design"); joining them pairwise, level by level, gives the
// top kd levels of that same tree.  The epilogue then applies the stage that
// follows the product: the activation, its derivative, or the gate-then-up
// add of the two dX lanes.  Used by the join kernel and, for the dX lanes, by
// the weight-gradient kernel's extra workgroups.
#pragma once

#include "dgf_device.hpp"
#include "dgf_kernels.hpp"

namespace dgf {

// The 2^kd partial roots of product b at row m, columns c .. c+7, joined with
// the balanced top of the tree (pairs of neighbours, level by level).  The
// partial rows are padded to a multiple of 8 columns, so the 16-byte loads
// stay inside the buffer; columns past N are never stored.
template <class T, int S>
__device__ __forceinline__ void join8(const GemmParams &p, int b, int64_t m, int64_t c, uint32_t (&r)[4]) {
  const uint16_t *base = p.part + (int64_t)b * S * p.part_stride + m * p.ldp + c;
  uint32_t v[S][4];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint4 q = *reinterpret_cast<const uint4 *>(base + s * p.part_stride);
    v[s][0] = q.x; v[s][1] = q.y; v[s][2] = q.z; v[s][3] = q.w;
  }
#pragma unroll
  for (int width = S; width > 1; width >>= 1)
#pragma unroll
    for (int j = 0; j < width / 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[j][q] = node2t<T>(v[2 * j][q], v[2 * j + 1][q]);
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = v[0][q];
}

__device__ __forceinline__ uint16_t half_of(const uint32_t (&r)[4], int e) {
  return (uint16_t)(r[e >> 1] >> (16 * (e & 1)));
}

// 8 stored values to dst[0..8), or the first N - c of them.
__device__ __forceinline__ void store8(uint16_t *dst, int64_t c, int64_t N, const uint32_t (&r)[4]) {
  if (c + 8 <= N) {
    *reinterpret_cast<uint4 *>(dst) = make_uint4(r[0], r[1], r[2], r[3]);
  } else {
    for (int e = 0; c + e < N; ++e) dst[e] = half_of(r, e);
  }
}

// One 8-column chunk (row m, columns c .. c+7) of the join and epilogue EPI:
// product b for EPI_STORE; ACT and DX read both products, DSILU the one.
template <class T, int S, int EPI>
__device__ __forceinline__ void join_epi_chunk(const GemmParams &p, int b, int64_t m, int64_t c) {
  uint32_t r0[4];
  join8<T, S>(p, EPI == EPI_STORE ? b : 0, m, c, r0);
  if constexpr (EPI == EPI_STORE) {
    store8(p.C[b] + m * p.ldc[b] + c, c, p.N, r0);
  } else if constexpr (EPI == EPI_ACT) {
    // gate product 0, up product 1: a = rnd(silu(g) u)
    uint32_t r1[4], a[4];
    join8<T, S>(p, 1, m, c, r1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float g0 = T::lo(r0[q]), g1 = T::hi(r0[q]);
      const float u0 = T::lo(r1[q]), u1 = T::hi(r1[q]);
      const float s0 = g0 * sigma_f(g0), s1 = g1 * sigma_f(g1);
      a[q] = T::pack_prod(s0 * u0, s1 * u1);
    }
    store8(p.act_out + m * p.ld_act + c, c, p.N, a);
    if (p.C[0]) store8(p.C[0] + m * p.ldc[0] + c, c, p.N, r0);
    if (p.C[1]) store8(p.C[1] + m * p.ldc[1] + c, c, p.N, r1);
  } else if constexpr (EPI == EPI_DSILU) {
    // dA with the saved g, u: dU = rnd(dA s), dG = rnd((dA u) s'), a = rnd(s u), row-major [M, N]
    uint32_t dg[4] = {0, 0, 0, 0}, du[4] = {0, 0, 0, 0}, av[4] = {0, 0, 0, 0};
    uint32_t gq[4], uq[4];
    const uint16_t *gs = p.sg + m * p.ld_gu + c, *us = p.su + m * p.ld_gu + c;
    if (c + 8 <= p.N) {  // g and u rows are 16-byte aligned (ld a multiple of 8)
      const uint4 gv = *reinterpret_cast<const uint4 *>(gs), uv = *reinterpret_cast<const uint4 *>(us);
      gq[0] = gv.x; gq[1] = gv.y; gq[2] = gv.z; gq[3] = gv.w;
      uq[0] = uv.x; uq[1] = uv.y; uq[2] = uv.z; uq[3] = uv.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t e = c + 2 * q;
        gq[q] = (e < p.N ? gs[2 * q] : 0u) | (e + 1 < p.N ? (uint32_t)gs[2 * q + 1] << 16 : 0u);
        uq[q] = (e < p.N ? us[2 * q] : 0u) | (e + 1 < p.N ? (uint32_t)us[2 * q + 1] << 16 : 0u);
      }
    }
    // all 8 lanes of the chunk are computed (columns past N are never stored)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float da = T::f(half_of(r0, e));
      const float g = T::f(half_of(gq, e));
      const float u = T::f(half_of(uq, e));
      const float sg = sigma_f(g);
      const float s = g * sg;
      const float one_m = 1.0f - sg;
      const float tt = g * one_m;
      const float onep = 1.0f + tt;
      const float ds = sg * onep;
      const uint32_t duv = T::r(da * s);
      const float dau = da * u;
      const uint32_t dgv = T::r(dau * ds);
      const uint32_t aa = T::r(s * u);
      dg[e >> 1] |= dgv << (16 * (e & 1));
      du[e >> 1] |= duv << (16 * (e & 1));
      av[e >> 1] |= aa << (16 * (e & 1));
    }
    if (p.dG) store8(p.dG + m * p.ld_d + c, c, p.N, dg);
    if (p.dU) store8(p.dU + m * p.ld_d + c, c, p.N, du);
    if (p.a_rm) store8(p.a_rm + m * p.ld_d + c, c, p.N, av);
  } else if constexpr (EPI == EPI_DX) {
    // dx = rnd(G + U), the gate lane first
    uint32_t r1[4], d[4];
    join8<T, S>(p, 1, m, c, r1);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = node2t<T>(r0[q], r1[q]);
    if (p.dx) store8(p.dx + m * p.lddx + c, c, p.N, d);
    if (p.C[0]) store8(p.C[0] + m * p.ldc[0] + c, c, p.N, r0);
    if (p.C[1]) store8(p.C[1] + m * p.ldc[1] + c, c, p.N, r1);
  }
}

}  // namespace dgf
