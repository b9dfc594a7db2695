// The steps either side of the MoE layer in a transformer block: the RMS
// normalisation that feeds the router and the experts, and the add of the
// layer's output (routed experts plus the always-on dense branch) into the
// bf16 residual stream.  dragon.c page, "Precision": norms run in bf16 and
// the dense per-sub-block branches are quantised like the routed experts;
// summary: the MoE reads sub-block 0's normed hidden state and its output is
// added to the stream at the end of sub-block 1 (the shortcut-connected MoE),
// so the add takes whichever residual tensor the caller passes.
#pragma once

#include "moe_common.h"

namespace moe {

// xn[t][i] = bf16(x[t][i] * r_t * gamma[i]), r_t = 1 / sqrt(mean_i x[t][i]^2 + eps),
// all in f32.  One wavefront per row, four rows per workgroup: lane l sums the
// squares of its 8-input chunks (chunks l, l + 64, ...) in order and the
// wavefront sums the lanes in a fixed DPP order, so every row has one
// summation order; the row's first RC chunks per lane stay in registers for
// the scaling pass (longer rows re-read the rest, cache-resident).
template <int RC>
__global__ __launch_bounds__(256) void rmsnorm_bf16(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ gamma, float eps,
                                                    uint16_t* __restrict__ xn, int T, int d) {
  const int t = blockIdx.x * 4 + wave_id(), lane = lane_id();
  if (t >= T) return;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * d);
  const u32x4* g = reinterpret_cast<const u32x4*>(gamma);
  u32x4* dst = reinterpret_cast<u32x4*>(xn + (size_t)t * d);
  const int nc = d >> 3;
  u32x4 keep[RC];
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = lane + 64 * i;
    keep[i] = c < nc ? row[c] : u32x4{0u, 0u, 0u, 0u};
  }
  float ss = 0.0f;
  auto sq = [&](const u32x4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(w[j]), b = bf16_hi(w[j]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  };
#pragma unroll
  for (int i = 0; i < RC; ++i) sq(keep[i]);
  for (int c = lane + 64 * RC; c < nc; c += 64) sq(row[c]);
  const float r = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
  auto scale = [&](const u32x4& v, int c) {
    const u32x4 gv = g[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = f32_to_bf16_rne(bf16_lo(w[j]) * r * bf16_lo(gw[j]));
      const uint32_t hi = f32_to_bf16_rne(bf16_hi(w[j]) * r * bf16_hi(gw[j]));
      o[j] = lo | (hi << 16);
    }
    dst[c] = u32x4{o[0], o[1], o[2], o[3]};
  };
#pragma unroll
  for (int i = 0; i < RC; ++i)
    if (lane + 64 * i < nc) scale(keep[i], lane + 64 * i);
  for (int c = lane + 64 * RC; c < nc; c += 64) scale(row[c], c);
}

// out[i] = bf16(residual[i] + (a[i] + b[i])) (b may be absent: + a[i] only),
// f32 adds in that order; four elements per thread.
__global__ __launch_bounds__(256) void residual_add_bf16(const uint16_t* residual,
                                                         const float* __restrict__ a,
                                                         const float* __restrict__ b,
                                                         uint16_t* out, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const u32x2 rv = reinterpret_cast<const u32x2*>(residual)[i];
  f32x4 s = reinterpret_cast<const f32x4*>(a)[i];
  if (b) {
    const f32x4 bv = reinterpret_cast<const f32x4*>(b)[i];
    s = f32x4{s.x + bv.x, s.y + bv.y, s.z + bv.z, s.w + bv.w};
  }
  const uint32_t o0 = f32_to_bf16_rne(bf16_lo(rv.x) + s.x), o1 = f32_to_bf16_rne(bf16_hi(rv.x) + s.y);
  const uint32_t o2 = f32_to_bf16_rne(bf16_lo(rv.y) + s.z), o3 = f32_to_bf16_rne(bf16_hi(rv.y) + s.w);
  reinterpret_cast<u32x2*>(out)[i] = u32x2{o0 | (o1 << 16), o2 | (o3 << 16)};
}

}  // namespace moe
