// Routing kernels: f32 router logits, softmax + top-k, and the counting-sort
// permute that groups token-slots by expert.
#pragma once

#include "moe_common.h"

namespace moe {

// ---------------------------------------------------------------- router logits

// Few tokens: one wavefront per expert streams its f32 router row with
// 16-byte loads and dots it with up to TG tokens at a time; a wave-wide tree
// sum finishes each logit.  logits[t][e] = sum_i W_r[e][i] x[t][i] + bias[t][e].
template <int TG>
__global__ __launch_bounds__(256) void router_gemv(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int T, int d,
                                                   int E) {
  const int e = blockIdx.x * 4 + wave_id();
  if (e >= E) return;
  const int lane = lane_id();
  const float* wrow = wr + (size_t)e * d;
  for (int t0 = 0; t0 < T; t0 += TG) {
    float acc[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) acc[i] = 0.0f;
    for (int c = lane * 4; c < d; c += WAVE * 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(wrow + c);
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        if (t0 + i < T) {
          const u32x2 xv = *reinterpret_cast<const u32x2*>(x + (size_t)(t0 + i) * d + c);
          acc[i] += w.x * bf16_lo(xv.x) + w.y * bf16_hi(xv.x) + w.z * bf16_lo(xv.y) +
                    w.w * bf16_hi(xv.y);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      const float s = wave_sum(acc[i]);
      const int t = t0 + i;
      if (lane == 0 && t < T) logits[(size_t)t * E + e] = s + (bias ? bias[(size_t)t * E + e] : 0.0f);
    }
  }
}

// Many tokens: a 64-token x 64-expert tile per 256-thread block, f32 FMAs
// from LDS, K in chunks of 32; each thread owns a 4x4 patch.
__global__ __launch_bounds__(256) void router_gemm(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int T, int d,
                                                   int E) {
  __shared__ float xs[32][64 + 4];
  __shared__ float ws[32][64 + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 32) {
    {  // x tile: 64 tokens x 32 k, one 16-byte load (8 bf16) per thread
      const int r = tid / 4, c8 = (tid % 4) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t0 + r < T) v = *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + r) * d + k0 + c8);
      xs[c8 + 0][r] = bf16_lo(v.x); xs[c8 + 1][r] = bf16_hi(v.x);
      xs[c8 + 2][r] = bf16_lo(v.y); xs[c8 + 3][r] = bf16_hi(v.y);
      xs[c8 + 4][r] = bf16_lo(v.z); xs[c8 + 5][r] = bf16_hi(v.z);
      xs[c8 + 6][r] = bf16_lo(v.w); xs[c8 + 7][r] = bf16_hi(v.w);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // router tile: 64 experts x 32 k
      const int q = tid + 256 * i;
      const int r = q / 8, c4 = (q % 8) * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (e0 + r < E) v = *reinterpret_cast<const f32x4*>(wr + (size_t)(e0 + r) * d + k0 + c4);
      ws[c4 + 0][r] = v.x; ws[c4 + 1][r] = v.y; ws[c4 + 2][r] = v.z; ws[c4 + 3][r] = v.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[(size_t)t * E + e] : 0.0f);
    }
  }
}

// ---------------------------------------------------------------- softmax + top-k

constexpr int MAX_E = 1024;
constexpr int MAX_K = 16;

// Order-preserving map of f32 to uint32: a > b  <=>  key(a) > key(b).
// NaN (outside the contract) maps to 0, below every other value.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// Selection is a radix select on the order keys: 32 rounds of wave ballots
// build the k-th largest key K bit by bit (the largest value with at least k
// keys >= it).  Every expert above K is selected, and of those equal to K the
// lowest indices fill the remaining places, so equal logits go to the lower
// index.  Each selected expert's place in ascending id order comes from the
// ballot masks; its weight is its softmax probability over all E experts
// (max-subtracted), divided by the sum over the k when `renorm`.
__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ logits,
                                                  int32_t* __restrict__ ids,
                                                  float* __restrict__ w, int T, int E, int k,
                                                  int renorm) {
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
  constexpr int NPL = MAX_E / WAVE;
  const int groups = (E + WAVE - 1) / WAVE;
  float l[NPL];
  uint32_t key[NPL];
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + WAVE * i;
    const float v = (i < groups && e < E) ? row[e] : -INFINITY;
    l[i] = (v == v) ? v : -INFINITY;
    key[i] = order_key(v);
  }
  auto valid = [&](int i) { return lane + WAVE * i < E; };
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int n = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i < groups) n += __popcll(__ballot(valid(i) && key[i] >= cand));
    if (n >= k) thr = cand;
  }
  int above = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    if (i < groups) above += __popcll(__ballot(valid(i) && key[i] > thr));
  const int need = k - above;  // places left for keys equal to the threshold
  uint32_t sel = 0;            // bit i: expert lane + 64 i is selected
  int ties_before = 0, sel_before = 0, pos[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    pos[i] = 0;
    if (i < groups) {
      const uint64_t tie = __ballot(valid(i) && key[i] == thr);
      const bool take = valid(i) && (key[i] > thr ||
                                     (key[i] == thr && ties_before + __popcll(tie & below) < need));
      const uint64_t sm = __ballot(take);
      if (take) {
        sel |= 1u << i;
        pos[i] = sel_before + __popcll(sm & below);
      }
      ties_before += __popcll(tie);
      sel_before += __popcll(sm);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) m = fmaxf(m, l[i]);
  m = wave_max(m);
  float z = 0.0f, ps = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    if (i < groups && valid(i)) {
      const float ex = __expf(l[i] - m);
      z += ex;
      if (sel >> i & 1u) ps += ex;
    }
  z = wave_sum(z);
  ps = wave_sum(ps) / z;
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    if (sel >> i & 1u) {
      const float p = __expf(l[i] - m) / z;
      ids[(size_t)t * k + pos[i]] = lane + WAVE * i;
      w[(size_t)t * k + pos[i]] = renorm ? p / ps : p;
    }
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
__global__ __launch_bounds__(1024) void permute_scan(const int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ base,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int4* __restrict__ slot_info,
                                                     int32_t* __restrict__ n_active, int n_slots,
                                                     int4* __restrict__ tiles,
                                                     int32_t* __restrict__ n_tiles, int nchunk,
                                                     int E, int S, int BM) {
  const int e = threadIdx.x;
  int c_e = 0;
  if (e < E) {
    for (int c = 0; c < nchunk; ++c) {
      base[(size_t)c * E + e] = c_e;
      c_e += hist[(size_t)c * E + e];
    }
    counts[e] = c_e;
  }
  int tot;
  const int off = block_exclusive_scan(e < E ? c_e : 0, &tot);
  if (e < E) offsets[e] = off;
  if (e == 0) offsets[E] = S;
  const int act = block_exclusive_scan((e < E && c_e > 0) ? 1 : 0, &tot);
  if (e < E && c_e > 0) slot_info[act] = make_int4(e, off, c_e, 0);
  if (e == 0) *n_active = tot;
  for (int i = tot + e; i < n_slots; i += blockDim.x) slot_info[i] = make_int4(-1, 0, 0, 0);
  const int mt = (e < E) ? (c_e + BM - 1) / BM : 0;
  const int tb = block_exclusive_scan(mt, &tot);
  for (int i = 0; i < mt; ++i) {
    const int rows = min(BM, c_e - i * BM);
    tiles[tb + i] = make_int4(e, off + i * BM, rows, 0);
  }
  if (e == 0) *n_tiles = tot;
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

}  // namespace moe
