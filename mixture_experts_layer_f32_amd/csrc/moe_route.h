// Routing kernels: f32 router logits, softmax + top-k, and the counting-sort
// permute that groups token-slots by expert.
#pragma once

#include "moe_common.h"

namespace moe {

// ---------------------------------------------------------------- router logits

// The router output of K-slice `split` goes to part[split][t][e]; the top-k
// kernel adds the slices in order 0, 1, ... and then the bias, so every logit
// has one fixed summation order.

// Few tokens: one wavefront per (expert, K-slice), four experts per
// workgroup.  The slice is taken in chunks of up to 1024 inputs: the
// workgroup stages the chunk's activations of TG tokens in LDS once (8-byte
// pieces, all loads issued before the first store), while each wavefront's
// router weights (four 16-byte loads per lane) are in flight; each lane then
// sums its inputs in ascending order and a wave-wide sum finishes each
// partial logit.  (Each wavefront reading the activations from memory itself
// moved four times the bytes through the caches and issued 16x the loads.)
template <int TG>
__global__ __launch_bounds__(256) void router_gemv(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ wr,
                                                   float* __restrict__ part, int T, int d, int E,
                                                   int slice) {
  __shared__ u32x2 xs[TG][256];  // TG tokens x 1024 bf16 inputs
  const int e = blockIdx.x * 4 + wave_id();
  const bool has_e = e < E;  // every wavefront takes part in the staging
  const int lane = lane_id(), tid = threadIdx.x;
  const int k0 = blockIdx.y * slice, k1 = min(d, k0 + slice);
  const float* wrow = wr + (size_t)min(e, E - 1) * d;
  float* out = part + (size_t)blockIdx.y * T * E;
  for (int t0 = 0; t0 < T; t0 += TG) {
    float acc[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) acc[i] = 0.0f;
    for (int kc = k0; kc < k1; kc += 1024) {
      f32x4 wv[4];
      bool in[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int k = kc + 256 * c + 4 * lane;
        in[c] = k < k1;
        wv[c] = has_e && in[c] ? *reinterpret_cast<const f32x4*>(wrow + k) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      u32x2 st[TG];
#pragma unroll
      for (int i = 0; i < TG; ++i) {  // piece tid of token row t0 + i
        const int k = kc + 4 * tid;
        st[i] = t0 + i < T && k < k1 ? *reinterpret_cast<const u32x2*>(x + (size_t)(t0 + i) * d + k)
                                     : u32x2{0u, 0u};
      }
      __syncthreads();  // the previous chunk's reads are done
#pragma unroll
      for (int i = 0; i < TG; ++i) xs[i][tid] = st[i];
      __syncthreads();
      if (has_e) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < TG; ++i) {
            const u32x2 xv = t0 + i < T && in[c] ? xs[i][64 * c + lane] : u32x2{0u, 0u};
            acc[i] += wv[c].x * bf16_lo(xv.x) + wv[c].y * bf16_hi(xv.x) + wv[c].z * bf16_lo(xv.y) +
                      wv[c].w * bf16_hi(xv.y);
          }
      }
    }
    if (has_e) {
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        if (t0 + i < T) {
          const float sum = wave_sum(acc[i]);
          if (lane == 0) out[(size_t)(t0 + i) * E + e] = sum;
        }
      }
    }
  }
}

// Many tokens: 64-token x 64-expert tiles on MFMA.  An f32 router weight w is
// the exact sum of three bf16 values hi + mid + lo (hi keeps the top 8 of its
// 24 significand bits, mid the next 8, lo the last 8; each remainder is exact
// in f32).  A bf16 activation times a bf16 value is exact in f32, so three
// v_mfma_f32_32x32x16_bf16 per 16-deep slice give x.w with only the f32
// accumulation rounding of an f32 dot product.  4 wavefronts in a 2x2 grid
// own 32x32 patches; K advances 64 per LDS stage within this block's slice.
__device__ __forceinline__ void split3_bf16(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t u = __float_as_uint(w);
  const float fh = __uint_as_float(u & 0xFFFF0000u);
  const float r1 = w - fh;
  const uint32_t ur = __float_as_uint(r1);
  const float fm = __uint_as_float(ur & 0xFFFF0000u);
  const float r2 = r1 - fm;
  hi = (uint16_t)(u >> 16);
  mid = (uint16_t)(ur >> 16);
  lo = (uint16_t)(__float_as_uint(r2) >> 16);
}

__global__ __launch_bounds__(256) void router_mfma(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ wr,
                                                   float* __restrict__ part, int T, int d, int E,
                                                   int slice) {
  // 64-deep LDS stages; the global loads of the next D - 1 stages are in
  // flight in registers while a stage is split and multiplied
  constexpr int BK = 64, LDK = BK + 8, D = 4;
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[3][64 * LDK];
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int k0 = blockIdx.z * slice, k1 = min(d, k0 + slice);
  const int wm0 = (wv >> 1) * 32, wn0 = (wv & 1) * 32;
  const int nit = (k1 - k0 + BK - 1) / BK;
  u32x4 rx[D][2];  // activations: 64 rows x 64 bf16 = 512 16-byte chunks, 2 per thread
  f32x4 rw[D][4];  // router rows: 64 x 64 f32 = 1024 16-byte chunks, 4 per thread
  auto load = [&](int it, int set) {
    const int k = k0 + it * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, r = c >> 3, col = (c & 7) * 8;
      rx[set][i] = t0 + r < T && k + col < k1
                       ? *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + r) * d + k + col)
                       : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 4, col = (c & 15) * 4;
      rw[set][i] = e0 + r < E && k + col < k1
                       ? *reinterpret_cast<const f32x4*>(wr + (size_t)(e0 + r) * d + k + col)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // the stage's bytes into LDS, each router weight split into hi / mid / lo
  auto store = [&](int set) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, r = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(xs + r * LDK + col) = rx[set][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 4, col = (c & 15) * 4;
      const f32x4 v = rw[set][i];
      uint16_t h[4], m[4], l[4];
      split3_bf16(v.x, h[0], m[0], l[0]);
      split3_bf16(v.y, h[1], m[1], l[1]);
      split3_bf16(v.z, h[2], m[2], l[2]);
      split3_bf16(v.w, h[3], m[3], l[3]);
      *reinterpret_cast<u32x2*>(ws[0] + r * LDK + col) =
          u32x2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
      *reinterpret_cast<u32x2*>(ws[1] + r * LDK + col) =
          u32x2{(uint32_t)m[0] | ((uint32_t)m[1] << 16), (uint32_t)m[2] | ((uint32_t)m[3] << 16)};
      *reinterpret_cast<u32x2*>(ws[2] + r * LDK + col) =
          u32x2{(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
    }
  };
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  auto compute = [&]() {
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(xs + (wm0 + r) * LDK + kk + kh);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(ws[p] + (wn0 + r) * LDK + kk + kh);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
    }
  };
#pragma unroll
  for (int p = 0; p < D - 1; ++p)
    if (p < nit) load(p, p);
  for (int it0 = 0; it0 < nit; it0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int it = it0 + j;
      if (it >= nit) break;
      if (it + D - 1 < nit) load(it + D - 1, (j + D - 1) % D);
      __syncthreads();  // the previous stage's MFMAs are done with LDS
      store(j);
      __syncthreads();
      compute();
    }
  }
  float* out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + wm0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    const int e = e0 + wn0 + (lane & 31);
    if (t < T && e < E) out[(size_t)t * E + e] = acc[v];
  }
}

// w3 = the hi, mid and lo planes of the router weights, each [E][d] bf16
// (n = E d, a multiple of 4).
__global__ __launch_bounds__(256) void router_split3(const float* __restrict__ wr,
                                                     uint16_t* __restrict__ w3, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * i >= n) return;
  const f32x4 v = reinterpret_cast<const f32x4*>(wr)[i];
  uint16_t h[4], m[4], l[4];
  split3_bf16(v.x, h[0], m[0], l[0]);
  split3_bf16(v.y, h[1], m[1], l[1]);
  split3_bf16(v.z, h[2], m[2], l[2]);
  split3_bf16(v.w, h[3], m[3], l[3]);
  u32x2* o = reinterpret_cast<u32x2*>(w3);
  o[i] = u32x2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
  o[n / 4 + i] = u32x2{(uint32_t)m[0] | ((uint32_t)m[1] << 16), (uint32_t)m[2] | ((uint32_t)m[3] << 16)};
  o[n / 2 + i] = u32x2{(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
}

// Many tokens and experts: 256-token x 128-expert tiles, 8 wavefronts in a
// 2 x 4 grid (128 tokens x 32 experts each: four 32-token chunks sharing each
// B fragment), on the three bf16 planes split once per forward by
// router_split3.  Each plane is read from L2 once per 256 tokens instead of
// the 64 x 64 tiles' once per 64, which re-split and re-read it per tile.
// Same products and the same order of 16-deep steps (hi, mid, lo) within a
// K-slice as router_mfma.
__global__ __launch_bounds__(512) void router_mfma_big(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ w3,
                                                       float* __restrict__ part, int T, int d,
                                                       int E, int slice) {
  constexpr int BK = 64, LDK = BK + 8, D = 3, BT = 256, BE = 128;
  __shared__ __attribute__((aligned(16))) uint16_t xs[BT * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[3][BE * LDK];
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
  const int k0 = blockIdx.z * slice, k1 = min(d, k0 + slice);
  const int wm0 = (wv >> 2) * 128, wn0 = (wv & 3) * 32;
  const int nit = (k1 - k0 + BK - 1) / BK;
  const size_t plane = (size_t)E * d;
  u32x4 rx[D][4];     // activations: 256 rows x 8 chunks = 2048, 4 per thread
  u32x4 rw[D][3][2];  // each plane: 128 rows x 8 chunks = 1024, 2 per thread
  auto load = [&](int it, int set) {
    const int k = k0 + it * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 512 * i, r = c >> 3, col = (c & 7) * 8;
      rx[set][i] = t0 + r < T && k + col < k1
                       ? *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + r) * d + k + col)
                       : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 512 * i, r = c >> 3, col = (c & 7) * 8;
#pragma unroll
      for (int p = 0; p < 3; ++p)
        rw[set][p][i] = e0 + r < E && k + col < k1
                            ? *reinterpret_cast<const u32x4*>(w3 + p * plane + (size_t)(e0 + r) * d + k + col)
                            : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 512 * i, r = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(xs + r * LDK + col) = rx[set][i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 512 * i, r = c >> 3, col = (c & 7) * 8;
#pragma unroll
      for (int p = 0; p < 3; ++p) *reinterpret_cast<u32x4*>(ws[p] + r * LDK + col) = rw[set][p][i];
    }
  };
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  auto compute = [&]() {
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 b[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) b[p] = *reinterpret_cast<const bf16x8*>(ws[p] + (wn0 + r) * LDK + kk + kh);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(xs + (wm0 + 32 * c + r) * LDK + kk + kh);
#pragma unroll
        for (int p = 0; p < 3; ++p) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[p], acc[c], 0, 0, 0);
      }
    }
  };
#pragma unroll
  for (int p = 0; p < D - 1; ++p)
    if (p < nit) load(p, p);
  for (int it0 = 0; it0 < nit; it0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int it = it0 + j;
      if (it >= nit) break;
      if (it + D - 1 < nit) load(it + D - 1, (j + D - 1) % D);
      __syncthreads();  // the previous stage's MFMAs are done with LDS
      store(j);
      __syncthreads();
      compute();
    }
  }
  float* out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = t0 + wm0 + 32 * c + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int e = e0 + wn0 + (lane & 31);
      if (t < T && e < E) out[(size_t)t * E + e] = acc[c][v];
    }
}

// ---------------------------------------------------------------- softmax + top-k

constexpr int MAX_E = 1024;
constexpr int MAX_K = 16;
constexpr int MAX_SPLIT = 8;  // most router K-slices (partials summed in order by the top-k)

// Order-preserving map of f32 to uint32: a > b  <=>  key(a) > key(b).
// NaN (outside the contract) maps to 0, below every other value.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// (the K-slice partials summed in slice order, then the bias added).  Up to
// 128 experts the k-th largest order key is found by a radix select; above,
// the k experts are taken one at a time, each round taking the largest
// remaining logit (by its order key) and of equal logits the lowest expert
// index.  Either way the k taken are the k largest with ties going to the
// lower index.  Each
// selected expert's place in ascending id order comes from the ballot masks;
// its weight is its softmax probability over all E experts (max-subtracted),
// divided by the sum over the k when `renorm`.
template <int NG>
__device__ __forceinline__ void topk_token(int t, const float* __restrict__ part, int nsplit,
                                           const float* __restrict__ bias,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int T, int E, int k, int renorm,
                                           int32_t* ids_lds = nullptr) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
  const size_t TE = (size_t)T * E;
  size_t col[NG];
  bool valid[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int e = lane + WAVE * i;
    valid[i] = e < E;
    col[i] = (size_t)t * E + min(e, E - 1);
  }
  // every load of a group of SG slices (clamped index) is issued before the
  // in-order sum; the bias (or a dummy read) goes with the first group
  constexpr int SG = NG <= 2 ? 8 : 4;
  const float* bp = bias ? bias : part;
  float bv[NG], v[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    bv[i] = bp[col[i]];
    v[i] = 0.0f;
  }
  for (int s0 = 0; s0 < nsplit; s0 += SG) {
    float ps[SG][NG];
#pragma unroll
    for (int j = 0; j < SG; ++j)
#pragma unroll
      for (int i = 0; i < NG; ++i) ps[j][i] = part[(size_t)min(s0 + j, nsplit - 1) * TE + col[i]];
#pragma unroll
    for (int j = 0; j < SG; ++j)
#pragma unroll
      for (int i = 0; i < NG; ++i)
        v[i] = s0 + j >= nsplit ? v[i] : (s0 + j == 0 ? ps[j][i] : v[i] + ps[j][i]);
  }
  float l[NG];
  uint32_t kv[NG];  // order key + 1 of each logit (NaN: 1), 0 once taken or past E
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    float x = v[i];
    if (bias) x += bv[i];
    x = x == 0.0f ? 0.0f : x;  // one key for both signed zeros
    l[i] = valid[i] && x == x ? x : -INFINITY;
    kv[i] = valid[i] ? order_key(x) + 1u : 0u;
  }
  bool take[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) take[i] = false;
  if constexpr (NG <= 2) {
    // up to 128 experts: radix select (cheaper than k rounds at one or two
    // keys per lane): 32 ballot rounds build the k-th largest key thr (the
    // largest value with at least k keys >= it); every key above thr is
    // taken, and of those equal to thr the lowest indices fill the rest.
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int n = 0;
#pragma unroll
      for (int i = 0; i < NG; ++i) n += __popcll(__ballot(kv[i] >= cand));
      if (n >= k) thr = cand;
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < NG; ++i) above += __popcll(__ballot(kv[i] > thr));
    const int need = k - above;  // places left for keys equal to thr (>= 1: past E never ties)
    int ties_before = 0;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const uint64_t tie = __ballot(kv[i] == thr);
      take[i] = kv[i] > thr || (kv[i] == thr && ties_before + __popcll(tie & below) < need);
      ties_before += __popcll(tie);
    }
  } else {
    for (int j = 0; j < k; ++j) {  // k <= E, so every round finds a key >= 1
      uint32_t lm = kv[0];
#pragma unroll
      for (int i = 1; i < NG; ++i) lm = kv[i] > lm ? kv[i] : lm;
      const uint32_t mx = wave_max_u32(lm);
      int sel = 0;
#pragma unroll
      for (int i = NG - 1; i >= 0; --i) {  // the lowest index holding mx wins
        const uint64_t b = __ballot(kv[i] == mx);
        if (b) sel = WAVE * i + (int)__builtin_ctzll(b);
      }
#pragma unroll
      for (int i = 0; i < NG; ++i)
        if (lane + WAVE * i == sel) {
          kv[i] = 0u;
          take[i] = true;
        }
    }
  }
  int pos[NG];
  int sel_before = 0;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const uint64_t sm = __ballot(take[i]);
    pos[i] = sel_before + __popcll(sm & below);
    sel_before += __popcll(sm);
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NG; ++i) m = fmaxf(m, l[i]);
  m = wave_max(m);
  float z = 0.0f, ps = 0.0f, ex[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    ex[i] = valid[i] ? __expf(l[i] - m) : 0.0f;
    z += ex[i];
    ps += take[i] ? ex[i] : 0.0f;
  }
  z = wave_sum(z);
  ps = wave_sum(ps) / z;
#pragma unroll
  for (int i = 0; i < NG; ++i)
    if (take[i]) {
      const float p = ex[i] / z;
      ids[(size_t)t * k + pos[i]] = lane + WAVE * i;
      if (ids_lds) ids_lds[t * k + pos[i]] = lane + WAVE * i;
      w[(size_t)t * k + pos[i]] = renorm ? p / ps : p;
    }
}

template <int NG>
__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ part, int nsplit,
                                                  const float* __restrict__ bias,
                                                  int32_t* __restrict__ ids,
                                                  float* __restrict__ w, int T, int E, int k,
                                                  int renorm) {
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  topk_token<NG>(t, part, nsplit, bias, ids, w, T, E, k, renorm);
}

// ---------------------------------------------------------------- permute

// Tokens are taken in chunks of 64, one wavefront per chunk.  Lane l owns
// token 64*chunk + l.  mask[e] is the 64-bit set of lanes that chose expert e;
// the rank of slot (t, j) among the chunk's slots of the same expert is the
// number of lower lanes in that set (each token lists an expert at most once,
// so this is the stable order).  hist[chunk][e] = |mask[e]|.
__global__ __launch_bounds__(64) void permute_count(const int32_t* __restrict__ ids,
                                                    int32_t* __restrict__ rank,
                                                    int32_t* __restrict__ hist, int T, int E,
                                                    int k) {
  __shared__ unsigned long long mask[MAX_E];
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x;
  for (int e = lane; e < E; e += WAVE) mask[e] = 0ull;
  __syncthreads();
  const int t = chunk * WAVE + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = min(max(ids[(size_t)t * k + j], 0), E - 1);
      atomicOr(&mask[e], 1ull << lane);
    }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
    for (int j = 0; j < k; ++j) {
      const int e = min(max(ids[(size_t)t * k + j], 0), E - 1);
      rank[(size_t)t * k + j] = __popcll(mask[e] & below);
    }
  }
  for (int e = lane; e < E; e += WAVE) hist[(size_t)chunk * E + e] = __popcll(mask[e]);
}

// Exclusive scan over the block (blockDim.x <= 1024) of one value per thread.
__device__ inline int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = lane_id(), wv = wave_id(), nw = (blockDim.x + WAVE - 1) / WAVE;
  int inc = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int y = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += y;
  }
  if (lane == WAVE - 1) wsum[wv] = inc;
  __syncthreads();
  if (wv == 0) {
    int s = lane < nw ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o, WAVE);
      if (lane >= o) s += y;
    }
    if (lane < nw) wsum[lane] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = wv ? wsum[wv - 1] : 0;
  *total = wsum[nw - 1];
  __syncthreads();
  return before + inc - v;
}

// One block of 1024 threads, thread e per expert: base[c][e] = slots of
// expert e in chunks before c; counts, offsets (exclusive scan over e);
// slot_info[i] = (expert, first sorted position, count) for the i-th expert,
// in ascending order, that received at least one slot, and (-1, 0, 0) for
// the remaining entries up to n_slots; and the grouped-GEMM tile list: for
// every expert, ceil(count/BM) tiles of (expert, first sorted position, rows).
// A layer with a shared expert (shT = T tokens, else 0) appends that
// expert's work after the routed experts': positions S .. S + T - 1 hold
// tokens 0 .. T - 1, one record (0, S, T, 1) and ceil(T/BM) tiles whose last
// field 1 marks the shared expert's weights.
__global__ __launch_bounds__(1024) void permute_scan(const int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ base,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int4* __restrict__ slot_info,
                                                     int32_t* __restrict__ n_active, int n_slots,
                                                     int4* __restrict__ tiles,
                                                     int32_t* __restrict__ n_tiles, int nchunk,
                                                     int E, int S, int BM,
                                                     int32_t* __restrict__ tok_of, int shT) {
  const int e = threadIdx.x;
  int c_e = 0;
  if (e < E) {
    // eight chunks' histogram loads in flight, then their running sums
    for (int c0 = 0; c0 < nchunk; c0 += 8) {
      int hv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) hv[j] = c0 + j < nchunk ? hist[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < nchunk) {
          base[(size_t)(c0 + j) * E + e] = c_e;
          c_e += hv[j];
        }
    }
    counts[e] = c_e;
  }
  int tot;
  const int off = block_exclusive_scan(e < E ? c_e : 0, &tot);
  if (e < E) offsets[e] = off;
  if (e == 0) offsets[E] = S;
  const int act = block_exclusive_scan((e < E && c_e > 0) ? 1 : 0, &tot);
  if (e < E && c_e > 0) slot_info[act] = make_int4(e, off, c_e, 0);
  const int n_act = tot, sh = shT > 0 ? 1 : 0;
  if (e == 0) {
    if (sh) slot_info[n_act] = make_int4(0, S, shT, 1);
    *n_active = n_act + sh;
  }
  for (int i = n_act + sh + e; i < n_slots; i += blockDim.x) slot_info[i] = make_int4(-1, 0, 0, 0);
  const int mt = (e < E) ? (c_e + BM - 1) / BM : 0;
  const int tb = block_exclusive_scan(mt, &tot);
  for (int i = 0; i < mt; ++i) {
    const int rows = min(BM, c_e - i * BM);
    tiles[tb + i] = make_int4(e, off + i * BM, rows, 0);
  }
  const int nsh = (shT + BM - 1) / BM;
  for (int i = e; i < nsh; i += blockDim.x) tiles[tot + i] = make_int4(0, S + i * BM, min(BM, shT - i * BM), 1);
  for (int t = e; t < shT; t += blockDim.x) tok_of[S + t] = t;
  if (e == 0) *n_tiles = tot + nsh;
}

// perm[offsets[e] + base[chunk][e] + rank[s]] = s; inv_perm[s] = that
// position; tok_of[that position] = s / k, the slot's token.
__global__ __launch_bounds__(256) void permute_scatter(const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ rank,
                                                       const int32_t* __restrict__ base,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv_perm,
                                                       int32_t* __restrict__ tok_of, int S,
                                                       int E, int k) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int e = min(max(ids[s], 0), E - 1);
  const int chunk = (s / k) / WAVE;
  const int p = offsets[e] + base[(size_t)chunk * E + e] + rank[s];
  if (p >= 0 && p < S) {
    perm[p] = s;
    tok_of[p] = s / k;
  }
  inv_perm[s] = min(max(p, 0), S - 1);
}

// Few tokens (T <= 16, one per wavefront): top-k and the whole counting-sort permute in one 1024-thread
// workgroup (the same arithmetic as route_topk + permute_count/scan/scatter
// with a single 64-token chunk): 16 wavefronts take the tokens' top-k, then
// LDS lane masks give the stable ranks, one scan gives counts, offsets, the
// per-expert records and the tile list, and the scatter writes perm,
// inv_perm and the token of each sorted position.  `shared` (0 or 1): the
// shared expert's record and tiles follow, as in permute_scan.
template <int NG>
__global__ __launch_bounds__(1024) void route_small(
    const float* __restrict__ part, int nsplit, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ tok_of, int4* __restrict__ slot_info, int32_t* __restrict__ n_active,
    int n_slots, int4* __restrict__ tiles, int32_t* __restrict__ n_tiles, int T, int E, int k,
    int renorm, int BM, int shared) {
  __shared__ unsigned long long mask[MAX_E];
  __shared__ int off_s[MAX_E];
  __shared__ int ids_s[WAVE * MAX_K];  // the ids again, read back without a memory round trip
  const int tid = threadIdx.x;
  for (int t = wave_id(); t < T; t += 16)
    topk_token<NG>(t, part, nsplit, bias, ids, w, T, E, k, renorm, ids_s);
  for (int e = tid; e < E; e += 1024) mask[e] = 0ull;
  __syncthreads();
  if (tid < T)
    for (int j = 0; j < k; ++j) atomicOr(&mask[min(max(ids_s[tid * k + j], 0), E - 1)], 1ull << tid);
  __syncthreads();
  const int e = tid;
  const int c_e = e < E ? __popcll(mask[e]) : 0;
  if (e < E) counts[e] = c_e;
  // one scan of three fields: slots (offsets, 10 bits), selected experts
  // (record index, 10 bits), tiles (tile-list index, bits 20..30).  The
  // caller keeps T <= 64 and T*k <= 1023, so no partial sum of the first two
  // exceeds 1023, and the tiles (at most T*k/16 + E with BM >= 16) fit 11 bits.
  const int mt = (e < E) ? (c_e + BM - 1) / BM : 0;
  int tot;
  const int packed = block_exclusive_scan(c_e | ((c_e > 0 ? 1 : 0) << 10) | (mt << 20), &tot);
  const int off = packed & 1023, act = (packed >> 10) & 1023, tb = packed >> 20;
  if (e < E) {
    offsets[e] = off;
    off_s[e] = off;
  }
  const int S = T * k;
  if (e == 0) offsets[E] = S;
  if (e < E && c_e > 0) slot_info[act] = make_int4(e, off, c_e, 0);
  const int n_act = (tot >> 10) & 1023;
  if (e == 0) {
    if (shared) slot_info[n_act] = make_int4(0, S, T, 1);
    *n_active = n_act + shared;
  }
  for (int i = n_act + shared + e; i < n_slots; i += blockDim.x) slot_info[i] = make_int4(-1, 0, 0, 0);
  for (int i = 0; i < mt; ++i) tiles[tb + i] = make_int4(e, off + i * BM, min(BM, c_e - i * BM), 0);
  // a shared expert: its tiles after the routed ones, positions S .. S + T - 1
  const int n_rt = tot >> 20, nsh = shared ? (T + BM - 1) / BM : 0;
  if (tid < nsh) tiles[n_rt + tid] = make_int4(0, S + tid * BM, min(BM, T - tid * BM), 1);
  if (shared && tid < T) tok_of[S + tid] = tid;
  if (e == 0) *n_tiles = n_rt + nsh;
  __syncthreads();
  for (int s = tid; s < S; s += 1024) {
    const int t = s / k;
    const int ex = min(max(ids_s[s], 0), E - 1);
    const unsigned long long below = t == 0 ? 0ull : (~0ull >> (WAVE - t));
    const int p = off_s[ex] + __popcll(mask[ex] & below);
    perm[p] = s;
    inv_perm[s] = p;
    tok_of[p] = t;
  }
}

// Routing of a one-expert top-1 layer (the dense branch): every token goes
// to expert 0 with weight exactly 1 (the softmax of one logit), so the
// permutation is the identity and no logits are needed.  Writes the same
// outputs and lists as the general routing kernels.
__global__ __launch_bounds__(256) void route_dense(int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ inv_perm,
                                                   int32_t* __restrict__ tok_of,
                                                   int4* __restrict__ slot_info,
                                                   int32_t* __restrict__ n_active,
                                                   int4* __restrict__ tiles,
                                                   int32_t* __restrict__ n_tiles, int T, int BM) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < T) {
    ids[i] = 0;
    w[i] = 1.0f;
    perm[i] = i;
    inv_perm[i] = i;
    tok_of[i] = i;
  }
  const int mt = (T + BM - 1) / BM;
  if (i < mt) tiles[i] = make_int4(0, i * BM, min(BM, T - i * BM), 0);
  if (i == 0) {
    counts[0] = T;
    offsets[0] = 0;
    offsets[1] = T;
    slot_info[0] = make_int4(0, 0, T, 0);
    *n_active = 1;
    *n_tiles = mt;
  }
}

}  // namespace moe
