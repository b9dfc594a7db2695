// Grouped variant of the expert stage: for many tokens per expert, each
// expert's rows (in sorted-slot order) form the M dimension of a GEMM tile.
// Weight tiles are read from HBM once per M-tile, decoded exactly to bf16 in
// LDS, and multiplied with bf16 MFMA (v_mfma_f32_32x32x16_bf16) into f32.
//   e4m3: one f32 scale per 128x128 block; every 128-deep K step is summed
//         into a fresh f32 partial, then added to the running sum times the
//         block's scale (dragon.c page, section 8 Round 3: the 128-column
//         block structure folds the scale multiply out of the inner loop).
//   e2m1: the power-of-two scale is applied exactly inside the fp4 -> bf16
//         conversion, so MFMA accumulates straight into the running sum.
// The A rows of the gate/up GEMM are gathered through the permutation (the
// token's own activation row), never copied (Trochilus README, "How it keeps
// up": gate and up read a token's row through a map instead of gathered
// copies).  SwiGLU and the bf16 rounding of h are fused into the epilogue.
#pragma once

#include "moe_common.h"
#include "moe_decode.h"

namespace moe {

// Tile geometry: 4 wavefronts in a 2 x 2 grid, each owning a
// (BM/2) x (BN/2) patch of 32x32 MFMA tiles.
template <int FMT>
struct GemmCfg {
  static constexpr int BK = FMT == FMT_E4M3 ? 128 : 64;  // K depth per LDS stage
  static constexpr int LDK = BK + 8;                      // padded LDS row (bf16)
};

// A tile: BM rows x BK bf16 from `row_ptr(r)` (nullptr -> zero row), columns
// [k0, k0+BK) clipped to K.  16-byte loads, 256 threads.
template <int BM, int BK, int LDK, typename RowPtr>
__device__ __forceinline__ void load_a_tile(uint16_t* As, RowPtr row_ptr, int k0, int K) {
  constexpr int CPR = BK / 8;  // 16-byte chunks per row
  constexpr int TOTAL = BM * CPR;
#pragma unroll
  for (int i = 0; i < (TOTAL + 255) / 256; ++i) {
    const int q = threadIdx.x + 256 * i;
    if (q < TOTAL) {
      const int r = q / CPR, c = q % CPR;
      const uint16_t* src = row_ptr(r);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src != nullptr && k0 + c * 8 < K) v = *reinterpret_cast<const u32x4*>(src + k0 + c * 8);
      *reinterpret_cast<u32x4*>(As + r * LDK + c * 8) = v;
    }
  }
}

// B tile: BN weight rows [n0, n0+BN) x inputs [k0, k0+BK) of one expert,
// decoded to bf16 into Bs[n][k].  Rows past N and inputs past K are zero.
template <int FMT, int BN, int BK, int LDK>
__device__ __forceinline__ void load_b_tile(uint16_t* Bs, const uint8_t* q, const uint8_t* s,
                                            int n0, int N, int k0, int K) {
  if (FMT == FMT_E4M3) {
    constexpr int CPR = BK / 16;  // 16 codes per chunk
    constexpr int TOTAL = BN * CPR;
#pragma unroll
    for (int i = 0; i < (TOTAL + 255) / 256; ++i) {
      const int qi = threadIdx.x + 256 * i;
      if (qi < TOTAL) {
        const int r = qi / CPR, c = qi % CPR;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (n0 + r < N)
          w = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(q + (size_t)(n0 + r) * K + k0 + c * 16));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        bf16x2 o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = e4m3x2_to_bf16<false>(ws[j]);
          o[2 * j + 1] = e4m3x2_to_bf16<true>(ws[j]);
        }
        u32x4* dst = reinterpret_cast<u32x4*>(Bs + r * LDK + c * 16);
        dst[0] = *reinterpret_cast<const u32x4*>(&o[0]);
        dst[1] = *reinterpret_cast<const u32x4*>(&o[4]);
      }
    }
  } else {
    constexpr int CPR = BK / 16;  // 16 codes (8 bytes) per chunk
    constexpr int TOTAL = BN * CPR;
#pragma unroll
    for (int i = 0; i < (TOTAL + 255) / 256; ++i) {
      const int qi = threadIdx.x + 256 * i;
      if (qi < TOTAL) {
        const int r = qi / CPR, c = qi % CPR;
        const int kk = k0 + c * 16;
        u32x2 w = {0u, 0u};
        float sc = 1.0f;
        if (n0 + r < N && kk < K) {
          w = __builtin_nontemporal_load(
              reinterpret_cast<const u32x2*>(q + (size_t)(n0 + r) * (K / 2) + kk / 2));
          sc = ue8m0_to_f32(s[(size_t)(n0 + r) * (K / 32) + kk / 32]);
        }
        bf16x2 o[8];
        o[0] = e2m1x2_to_bf16<0>(w.x, sc);
        o[1] = e2m1x2_to_bf16<1>(w.x, sc);
        o[2] = e2m1x2_to_bf16<2>(w.x, sc);
        o[3] = e2m1x2_to_bf16<3>(w.x, sc);
        o[4] = e2m1x2_to_bf16<0>(w.y, sc);
        o[5] = e2m1x2_to_bf16<1>(w.y, sc);
        o[6] = e2m1x2_to_bf16<2>(w.y, sc);
        o[7] = e2m1x2_to_bf16<3>(w.y, sc);
        u32x4* dst = reinterpret_cast<u32x4*>(Bs + r * LDK + c * 16);
        dst[0] = *reinterpret_cast<const u32x4*>(&o[0]);
        dst[1] = *reinterpret_cast<const u32x4*>(&o[4]);
      }
    }
  }
}

// acc[tm][tn] += A[wave rows] * B[wave cols]^T over one BK-deep stage.
// Operand layout of v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 and
// inputs 8*(l/32) .. 8*(l/32)+7 of the 16-deep slice, for A and for B.
template <int TM, int TN, int BK, int LDK>
__device__ __forceinline__ void mfma_stage(f32x16 (&acc)[TM][TN], const uint16_t* As,
                                           const uint16_t* Bs, int wm0, int wn0) {
  const int lane = lane_id();
  const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK; kk += 16) {
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(As + (wm0 + 32 * i + r) * LDK + kk + kh);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn0 + 32 * j + r) * LDK + kk + kh);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Row index (within the 32x32 tile) of accumulator register v for this lane;
// the column is lane % 32.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// Gate/up + SwiGLU over the tile list.  grid.x: tile index (blocks past
// *n_tiles exit); grid.y: BN-wide column block of f.
template <int FMT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_gateup(
    const uint16_t* __restrict__ x, DMat gate, DMat up, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    uint16_t* __restrict__ h, int d, int f, int T) {
  constexpr int BK = GemmCfg<FMT>::BK, LDK = GemmCfg<FMT>::LDK;
  constexpr int TM = BM / 64, TN = BN / 64;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bg[BN * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bu[BN * LDK];
  __shared__ int tok[BM];
  if ((int)blockIdx.x >= *n_tiles) return;
  const int4 tile = tiles[blockIdx.x];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = blockIdx.y * BN;
  const int lane = lane_id(), wv = wave_id();
  const int wm0 = (wv >> 1) * (BM / 2), wn0 = (wv & 1) * (BN / 2);
  for (int r = threadIdx.x; r < BM; r += 256)
    tok[r] = r < rows ? (int)min((uint32_t)tok_of[p_start + r], (uint32_t)(T - 1)) : -1;
  __syncthreads();
  const uint8_t* gq = gate.q + e * gate.qs;
  const uint8_t* uq = up.q + e * up.qs;
  const uint8_t* gs = gate.s + e * gate.ss;
  const uint8_t* us = up.s + e * up.ss;
  auto xrow = [&](int r) -> const uint16_t* {
    return tok[r] >= 0 ? x + (size_t)tok[r] * d : nullptr;
  };
  f32x16 accg[TM][TN], accu[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) accg[i][j][v] = accu[i][j][v] = 0.0f;
  for (int k0 = 0; k0 < d; k0 += BK) {
    load_a_tile<BM, BK, LDK>(As, xrow, k0, d);
    load_b_tile<FMT, BN, BK, LDK>(Bg, gq, gs, n0, f, k0, d);
    load_b_tile<FMT, BN, BK, LDK>(Bu, uq, us, n0, f, k0, d);
    __syncthreads();
    if (FMT == FMT_E4M3) {
      f32x16 pg[TM][TN], pu[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) pg[i][j][v] = pu[i][j][v] = 0.0f;
      mfma_stage<TM, TN, BK, LDK>(pg, As, Bg, wm0, wn0);
      mfma_stage<TM, TN, BK, LDK>(pu, As, Bu, wm0, wn0);
      const float* gsf = reinterpret_cast<const float*>(gs);
      const float* usf = reinterpret_cast<const float*>(us);
      const float sg = gsf[(n0 >> 7) * (d >> 7) + (k0 >> 7)];
      const float su = usf[(n0 >> 7) * (d >> 7) + (k0 >> 7)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            accg[i][j][v] += sg * pg[i][j][v];
            accu[i][j][v] += su * pu[i][j][v];
          }
    } else {
      mfma_stage<TM, TN, BK, LDK>(accg, As, Bg, wm0, wn0);
      mfma_stage<TM, TN, BK, LDK>(accu, As, Bu, wm0, wn0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm0 + 32 * i + acc_row(v, lane);
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (m < rows && n < f)
          h[(size_t)(p_start + m) * f + n] =
              (uint16_t)f32_to_bf16_rne(silu(accg[i][j][v]) * accu[i][j][v]);
      }
}

// Down projection over the tile list: y[p][m] = sum_n h[p][n] Wd[m][n], f32.
template <int FMT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_down(const uint16_t* __restrict__ h, DMat down,
                                                 const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ n_tiles,
                                                 float* __restrict__ y, int d, int f) {
  constexpr int BK = GemmCfg<FMT>::BK, LDK = GemmCfg<FMT>::LDK;
  constexpr int TM = BM / 64, TN = BN / 64;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];
  if ((int)blockIdx.x >= *n_tiles) return;
  const int4 tile = tiles[blockIdx.x];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = blockIdx.y * BN;
  const int lane = lane_id(), wv = wave_id();
  const int wm0 = (wv >> 1) * (BM / 2), wn0 = (wv & 1) * (BN / 2);
  const uint8_t* dq = down.q + e * down.qs;
  const uint8_t* ds = down.s + e * down.ss;
  auto hrow = [&](int r) -> const uint16_t* {
    return r < rows ? h + (size_t)(p_start + r) * f : nullptr;
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  for (int k0 = 0; k0 < f; k0 += BK) {
    load_a_tile<BM, BK, LDK>(As, hrow, k0, f);
    load_b_tile<FMT, BN, BK, LDK>(Bs, dq, ds, n0, d, k0, f);
    __syncthreads();
    if (FMT == FMT_E4M3) {
      f32x16 p[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) p[i][j][v] = 0.0f;
      mfma_stage<TM, TN, BK, LDK>(p, As, Bs, wm0, wn0);
      const float sd = reinterpret_cast<const float*>(ds)[(n0 >> 7) * (f >> 7) + (k0 >> 7)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] += sd * p[i][j][v];
    } else {
      mfma_stage<TM, TN, BK, LDK>(acc, As, Bs, wm0, wn0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm0 + 32 * i + acc_row(v, lane);
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (m < rows && n < d) y[(size_t)(p_start + m) * d + n] = acc[i][j][v];
      }
}

}  // namespace moe
