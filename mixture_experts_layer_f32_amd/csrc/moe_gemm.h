// Grouped variant of the expert stage: for many tokens per expert, each
// expert's rows (in sorted-slot order) form the M dimension of GEMM tiles.
// Weight tiles are read from HBM once per M-tile, decoded exactly to bf16 in
// LDS, and multiplied with bf16 MFMA (v_mfma_f32_32x32x16_bf16) into f32.
//   e4m3: one f32 scale per 128x128 block; the MFMA sums of each 128-deep K
//         block go to a fresh f32 partial that is then added to the running
//         sum times the block's scale (dragon.c page, section 8 Round 3: the
//         128-column block structure folds the scale multiply out of the
//         inner loop).
//   e2m1: the power-of-two scale is applied exactly inside the fp4 -> bf16
//         conversion, so MFMA accumulates straight into the running sum.
// The A rows of the gate/up GEMM are the tokens' own activation rows, read
// through the permutation and never copied (Trochilus README, "How it keeps
// up": gate and up read a token's row through a map instead of gathered
// copies).  Gate and up rows of the same output column sit in the same lane
// and register, so SwiGLU and the bf16 rounding of h happen in registers.
//
// Pipeline: 64-deep K stages, double-buffered in LDS; while the MFMAs of
// stage k run, each thread's global loads for stage k+1 are in flight in
// registers; they are decoded and written to the other LDS buffer after the
// MFMAs, and one barrier per stage orders the buffers.
#pragma once

#include "moe_common.h"
#include "moe_decode.h"

namespace moe {

// BM rows per tile; WM wavefronts along M and 4/WM along N; each wavefront
// owns TM x TN 32x32 tiles per weight matrix; NMAT matrices (2: gate and up
// sharing A, 1: down).
template <int FMT, int NMAT, int BM, int WM, int TN, int BK_ = 64>
struct G2 {
  static constexpr int BK = BK_, LDK = BK + 8;        // stage depth, padded LDS row (bf16)
  static constexpr int WN = 4 / WM;
  static constexpr int TM = BM / WM / 32;
  static constexpr int BNM = WN * 32 * TN;            // weight rows per matrix per block
  static constexpr int A_ELEMS = BM * LDK;
  static constexpr int STAGE = A_ELEMS + NMAT * BNM * LDK;
  static constexpr int SMEM = 2 * STAGE * 2;          // bytes, two stages
  static constexpr int A_CPR = BK / 8;                                   // 16-B chunks (8 bf16) per row
  static constexpr int A_TOTAL = BM * A_CPR;
  static constexpr int A_CHUNKS = (A_TOTAL + 255) / 256;                 // per thread (last may idle)
  static constexpr int B_CPR = FMT == FMT_E4M3 ? BK / 16 : BK / 32;     // 16-B code chunks per row
  static constexpr int B_EPC = FMT == FMT_E4M3 ? 16 : 32;               // codes per chunk
  static constexpr int B_TOTAL = NMAT * BNM * B_CPR;
  static constexpr int B_CHUNKS = (B_TOTAL + 255) / 256;
  static_assert(256 % A_CPR == 0 && (A_TOTAL % 256 == 0 || A_TOTAL < 256), "A tile / threads");
  static_assert(B_TOTAL % 256 == 0 || B_TOTAL < 256, "B tile / threads");
  static_assert(TM >= 1, "tile rows");
  static_assert(FMT != FMT_E4M3 || 128 % BK == 0, "e4m3 stages divide a scale block");
};

constexpr int MAX_KBLK = 128;  // e4m3 grouped GEMM: K <= 128 * 128 (scales held in 2 VGPRs)

__device__ __forceinline__ u32x4 pack4(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

// Row index (within the 32x32 tile) of accumulator register v for this lane;
// the column is lane % 32.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// grid.x: BNM-wide column block of N; grid.y: tile index (blocks past
// *n_tiles exit).  GATEUP: act = x [T][K], out = h bf16 [S][N] (N = f,
// K = d); otherwise act = h [S][K], out = y f32 [S][N] (N = d, K = f).
template <int FMT, bool GATEUP, int BM, int WM, int TN, int BK_, int PF>
__global__ __launch_bounds__(256, 2) void gemm_expert(
    const uint16_t* __restrict__ act, DMat W0, DMat W1, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    void* __restrict__ out, int N, int K, int T) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  using C = G2<FMT, NMAT, BM, WM, TN, BK_>;
  constexpr int BK = C::BK, LDK = C::LDK, TM = C::TM, BNM = C::BNM;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  if ((int)blockIdx.y >= *n_tiles) return;
  const int4 tile = tiles[blockIdx.y];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = blockIdx.x * BNM;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int wm0 = (wv / C::WN) * (BM / WM), wn0 = (wv % C::WN) * 32 * TN;

  // this thread's A rows (fixed over K) and column
  const uint16_t* arow[C::A_CHUNKS];
  const int acol = (tid % C::A_CPR) * 8;
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int q = tid + 256 * i;
    const int r = q / C::A_CPR;
    arow[i] = nullptr;
    if (q < C::A_TOTAL && r < rows) {
      const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + r], (uint32_t)(T - 1))
                                : (size_t)(p_start + r);
      arow[i] = act + src * K;
    }
  }
  // this thread's B chunks: matrix, row, chunk column
  const uint8_t* bq[C::B_CHUNKS];
  const uint8_t* bsr[C::B_CHUNKS];
  int bdst[C::B_CHUNKS];
  const int64_t rbytes = FMT == FMT_E4M3 ? (int64_t)K : (int64_t)K / 2;
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int q = tid + 256 * i;
    const int m = q / (BNM * C::B_CPR);
    const int rem = q % (BNM * C::B_CPR);
    const int r = rem / C::B_CPR, c = rem % C::B_CPR;
    const DMat& W = (m == 0) ? W0 : W1;
    const int n = n0 + r;
    const bool ok = q < C::B_TOTAL && n < N;
    bq[i] = ok ? W.q + e * W.qs + n * rbytes + c * 16 : nullptr;
    bsr[i] = ok ? W.s + e * W.ss + (size_t)n * (K / 32) + c : nullptr;  // e2m1 group of the chunk
    bdst[i] = q < C::B_TOTAL ? C::A_ELEMS + (m * BNM + r) * LDK + c * C::B_EPC : -1;
  }

  // e4m3: this block's scale row (one 128-row block of N) for each matrix,
  // k-block kb held by lane kb % 64 of register kb / 64, read with v_readlane
  float scv[NMAT][2];
  if (FMT == FMT_E4M3) {
    const int nb = min(n0, N - 1) >> 7, kbs = K >> 7;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const DMat& W = (m == 0) ? W0 : W1;
      const float* sf = reinterpret_cast<const float*>(W.s + e * W.ss) + (size_t)nb * kbs;
      scv[m][0] = lane < kbs ? sf[lane] : 0.0f;
      scv[m][1] = lane + 64 < kbs ? sf[lane + 64] : 0.0f;
    }
  }

  // PF register sets of global loads in flight
  u32x4 ra[PF][C::A_CHUNKS], rb[PF][C::B_CHUNKS];
  float rsc[PF][C::B_CHUNKS];
  auto gload = [&](int set, int k0) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      ra[set][i] = u32x4{0u, 0u, 0u, 0u};
      if (arow[i] != nullptr && k0 + acol < K)
        ra[set][i] = *reinterpret_cast<const u32x4*>(arow[i] + k0 + acol);
    }
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
      rb[set][i] = u32x4{0u, 0u, 0u, 0u};
      rsc[set][i] = 1.0f;
      const int c = (tid + 256 * i) % C::B_CPR;
      if (bq[i] != nullptr && k0 + c * C::B_EPC < K) {
        const int64_t off = FMT == FMT_E4M3 ? k0 : k0 / 2;
        rb[set][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bq[i] + off));
        if (FMT == FMT_E2M1) rsc[set][i] = ue8m0_to_f32(bsr[i][k0 / 32]);
      }
    }
  };
  auto lstore = [&](int set, uint16_t* st) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int q = tid + 256 * i;
      if (q < C::A_TOTAL)
        *reinterpret_cast<u32x4*>(st + (q / C::A_CPR) * LDK + acol) = ra[set][i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
      if (bdst[i] < 0) continue;
      const uint32_t w[4] = {rb[set][i].x, rb[set][i].y, rb[set][i].z, rb[set][i].w};
      u32x4* dst = reinterpret_cast<u32x4*>(st + bdst[i]);
      if (FMT == FMT_E4M3) {
        bf16x2 o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = e4m3x2_to_bf16<false>(w[j]);
          o[2 * j + 1] = e4m3x2_to_bf16<true>(w[j]);
        }
        dst[0] = pack4(o[0], o[1], o[2], o[3]);
        dst[1] = pack4(o[4], o[5], o[6], o[7]);
      } else {
        const float sc = rsc[set][i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x2 o[4];
          o[0] = e2m1x2_to_bf16<0>(w[j], sc);
          o[1] = e2m1x2_to_bf16<1>(w[j], sc);
          o[2] = e2m1x2_to_bf16<2>(w[j], sc);
          o[3] = e2m1x2_to_bf16<3>(w[j], sc);
          dst[j] = pack4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  };

  f32x16 acc[TM][NMAT * TN], part[TM][NMAT * TN];
  const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < NMAT * TN; ++j) acc[i][j] = part[i][j] = zero;

  // Stage ks lives in LDS buffer ks & 1; its global loads went to register
  // set ks % PF, issued PF stages earlier.
  constexpr int SPB = 128 / BK;  // e4m3: stages per scale block
  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < nk) gload(p, p * BK);
  lstore(0, smem);
  __syncthreads();
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  for (int ks = 0; ks < nk; ++ks) {
    const uint16_t* cur = smem + (ks & 1) * C::STAGE;
    // the register set of stage ks was stored to LDS; refill it with stage ks + PF
    if (ks + PF < nk) gload(ks % PF, (ks + PF) * BK);
    const bool first = (FMT == FMT_E4M3) && (ks % SPB == 0);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 a[TM], b[NMAT * TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(cur + (wm0 + 32 * i + r32) * LDK + kk + kh);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          b[m * TN + j] = *reinterpret_cast<const bf16x8*>(
              cur + C::A_ELEMS + (m * BNM + wn0 + 32 * j + r32) * LDK + kk + kh);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < NMAT * TN; ++j) {
          if (FMT == FMT_E4M3)  // a scale block's first product starts from zero
            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a[i], b[j], (first && kk == 0) ? zero : part[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
    if (FMT == FMT_E4M3 && ((ks % SPB) == SPB - 1 || ks == nk - 1)) {
      // end of a 128-deep scale block: acc += scale * partial
      const int kb = (ks * BK) >> 7;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const float sc = __int_as_float(__builtin_amdgcn_readlane(
            __float_as_int(kb < 64 ? scv[m][0] : scv[m][1]), kb & 63));
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][m * TN + j][v] += sc * part[i][m * TN + j][v];
      }
    }
    if (ks + 1 < nk) lstore((ks + 1) % PF, smem + ((ks + 1) & 1) * C::STAGE);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm0 + 32 * i + acc_row(v, lane);
        const int n = n0 + wn0 + 32 * j + r32;
        if (m < rows && n < N) {
          if (GATEUP)
            reinterpret_cast<uint16_t*>(out)[(size_t)(p_start + m) * N + n] =
                (uint16_t)f32_to_bf16_rne(silu(acc[i][j][v]) * acc[i][TN + j][v]);
          else
            reinterpret_cast<float*>(out)[(size_t)(p_start + m) * N + n] = acc[i][j][v];
        }
      }
}

}  // namespace moe
