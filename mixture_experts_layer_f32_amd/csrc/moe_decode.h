// Decode variant of the expert stage: for few tokens per expert the weights
// are streamed once from HBM by coalesced 16-byte (e4m3) or 8-byte (e2m1)
// loads, one wavefront per group of RPW rows, each row dotted with every
// routed token of its expert (one weight row against several tokens, as the
// Trochilus README's "Acknowledgements" credit to ds4 describes), then
// reduced across the wavefront.  The decoded weights never leave registers
// (dragon.c page, section 8 Round 2: compute from the native-precision bytes).
#pragma once

#include "moe_common.h"

namespace moe {

enum : int { FMT_E4M3 = 0, FMT_E2M1 = 1 };

// One expert matrix family on the device: byte pointers and expert strides.
struct DMat {
  const uint8_t* q;
  const uint8_t* s;
  int64_t qs;  // bytes per expert, codes
  int64_t ss;  // bytes per expert, scales
};

// A "chunk" is 16 consecutive inputs of one weight row: 16 bytes of e4m3
// codes or 8 bytes of e2m1 codes.  These helpers return the dot product of
// one chunk with 16 activations (already f32), including the scale.
template <int FMT>
struct Chunk;

template <>
struct Chunk<FMT_E4M3> {
  typedef u32x4 raw;
  static __device__ __forceinline__ raw load(const uint8_t* row, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
  }
  // scale of the 128x128 block holding row n, inputs [16c, 16c+16)
  static __device__ __forceinline__ float scale(const uint8_t* s, int n, int c, int K) {
    return reinterpret_cast<const float*>(s)[(n >> 7) * (K >> 7) + (c >> 3)];
  }
  static __device__ __forceinline__ float dot(raw w, float sc, const float* xv) {
    float p = 0.0f;
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 a = e4m3x2_to_f32<false>(ws[i]);
      const f32x2 b = e4m3x2_to_f32<true>(ws[i]);
      p += a.x * xv[4 * i] + a.y * xv[4 * i + 1] + b.x * xv[4 * i + 2] + b.y * xv[4 * i + 3];
    }
    return p * sc;
  }
};

template <>
struct Chunk<FMT_E2M1> {
  typedef u32x2 raw;
  static __device__ __forceinline__ raw load(const uint8_t* row, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row) + c);
  }
  // UE8M0 byte of the 32-input group holding inputs [16c, 16c+16) of row n
  static __device__ __forceinline__ float scale(const uint8_t* s, int n, int c, int K) {
    return ue8m0_to_f32(s[(size_t)n * (K >> 5) + (c >> 1)]);
  }
  static __device__ __forceinline__ float dot(raw w, float sc, const float* xv) {
    float p = 0.0f;
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 a = e2m1x2_to_f32<0>(ws[i], sc);
      const f32x2 b = e2m1x2_to_f32<1>(ws[i], sc);
      const f32x2 c2 = e2m1x2_to_f32<2>(ws[i], sc);
      const f32x2 d2 = e2m1x2_to_f32<3>(ws[i], sc);
      p += a.x * xv[8 * i] + a.y * xv[8 * i + 1] + b.x * xv[8 * i + 2] + b.y * xv[8 * i + 3] +
           c2.x * xv[8 * i + 4] + c2.y * xv[8 * i + 5] + d2.x * xv[8 * i + 6] +
           d2.y * xv[8 * i + 7];
    }
    return p;  // the scale is applied exactly inside the conversion
  }
};

template <int FMT>
__device__ __forceinline__ int64_t row_bytes(int K) {
  return FMT == FMT_E4M3 ? (int64_t)K : (int64_t)K / 2;
}

// 16 bf16 activations starting at input 16c of a row -> f32.
__device__ __forceinline__ void load_act16(const uint16_t* row, int c, float* xv) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row + 16 * c);
  const u32x4 a = p[0], b = p[1];
  const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xv[2 * i] = bf16_lo(v[i]);
    xv[2 * i + 1] = bf16_hi(v[i]);
  }
}

// Gate/up + SwiGLU.  grid.x: index into the list of experts that received at
// least one slot (blocks past its length exit); grid.y: groups of 4*RPW rows
// of f.  For every slot of the expert, in sorted order, writes
// h[p][n] = bf16(silu(g[n]) * u[n]) at sorted position p.
template <int FMT, int TG, int RPW>
__global__ __launch_bounds__(256) void dec_gateup(
    const uint16_t* __restrict__ x, DMat gate, DMat up, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ h, int d, int f, int k, int T) {
  if ((int)blockIdx.x >= *n_active) return;
  const int e = active[blockIdx.x];
  const int p0 = offsets[e], cnt = counts[e];
  const int n0 = (blockIdx.y * 4 + wave_id()) * RPW;
  if (n0 >= f) return;
  const int lane = lane_id();
  const int nch = d / 16;
  const int64_t rb = row_bytes<FMT>(d);
  const uint8_t* gq = gate.q + e * gate.qs + n0 * rb;
  const uint8_t* uq = up.q + e * up.qs + n0 * rb;
  const uint8_t* gs = gate.s + e * gate.ss;
  const uint8_t* us = up.s + e * up.ss;
  for (int t0 = 0; t0 < cnt; t0 += TG) {
    const uint16_t* xr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const int r = min(t0 + t, cnt - 1);
      xr[t] = x + (size_t)min((uint32_t)perm[p0 + r] / (uint32_t)k, (uint32_t)(T - 1)) * d;
    }
    float ag[RPW][TG], au[RPW][TG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t) ag[r][t] = au[r][t] = 0.0f;
    for (int c = lane; c < nch; c += WAVE) {
      typename Chunk<FMT>::raw wg[RPW], wu[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        wg[r] = Chunk<FMT>::load(gq + r * rb, c);
        wu[r] = Chunk<FMT>::load(uq + r * rb, c);
      }
      float xv[TG][16];
#pragma unroll
      for (int t = 0; t < TG; ++t) load_act16(xr[t], c, xv[t]);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float sg = Chunk<FMT>::scale(gs, n0 + r, c, d);
        const float su = Chunk<FMT>::scale(us, n0 + r, c, d);
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          ag[r][t] += Chunk<FMT>::dot(wg[r], sg, xv[t]);
          au[r][t] += Chunk<FMT>::dot(wu[r], su, xv[t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const float g = wave_sum(ag[r][t]);
        const float u = wave_sum(au[r][t]);
        if (lane == r * TG + t && t0 + t < cnt)
          h[(size_t)(p0 + t0 + t) * f + n0 + r] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
      }
  }
}

// Down projection: y[p][m] = sum_n h[p][n] Wd[m][n] (f32) for every sorted
// position p of the expert; grid as dec_gateup with rows m of d.
template <int FMT, int TG, int RPW>
__global__ __launch_bounds__(256) void dec_down(
    const uint16_t* __restrict__ h, DMat down, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, float* __restrict__ y, int d, int f) {
  if ((int)blockIdx.x >= *n_active) return;
  const int e = active[blockIdx.x];
  const int p0 = offsets[e], cnt = counts[e];
  const int m0 = (blockIdx.y * 4 + wave_id()) * RPW;
  if (m0 >= d) return;
  const int lane = lane_id();
  const int nch = f / 16;
  const int64_t rb = row_bytes<FMT>(f);
  const uint8_t* dq = down.q + e * down.qs + m0 * rb;
  const uint8_t* ds = down.s + e * down.ss;
  for (int t0 = 0; t0 < cnt; t0 += TG) {
    const uint16_t* hr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) hr[t] = h + (size_t)(p0 + min(t0 + t, cnt - 1)) * f;
    float acc[RPW][TG];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[r][t] = 0.0f;
    for (int c = lane; c < nch; c += WAVE) {
      typename Chunk<FMT>::raw wd[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) wd[r] = Chunk<FMT>::load(dq + r * rb, c);
      float hv[TG][16];
#pragma unroll
      for (int t = 0; t < TG; ++t) load_act16(hr[t], c, hv[t]);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float sd = Chunk<FMT>::scale(ds, m0 + r, c, f);
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[r][t] += Chunk<FMT>::dot(wd[r], sd, hv[t]);
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const float v = wave_sum(acc[r][t]);
        if (lane == r * TG + t && t0 + t < cnt) y[(size_t)(p0 + t0 + t) * d + m0 + r] = v;
      }
  }
}

// out[t][m] = sum over j ascending of w[t][j] * y[inv_perm[t*k+j]][m]: a
// gather in router order, so every output has one fixed summation order
// (WARP BACKENDS.md, "Coherent memory": partials reduced in router order).
__global__ __launch_bounds__(256) void combine_fixed_order(const float* __restrict__ y,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ inv_perm,
                                                           float* __restrict__ out, int d,
                                                           int k) {
  const int t = blockIdx.x;
  const int m = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (m >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(y + (size_t)inv_perm[(size_t)t * k + j] * d + m);
    acc.x += wj * v.x;
    acc.y += wj * v.y;
    acc.z += wj * v.z;
    acc.w += wj * v.w;
  }
  *reinterpret_cast<f32x4*>(out + (size_t)t * d + m) = acc;
}

}  // namespace moe
