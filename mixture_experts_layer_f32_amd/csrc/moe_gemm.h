// Grouped variant of the expert stage: for many tokens per expert, each
// expert's rows (in sorted-slot order) form the M dimension of GEMM tiles.
// Weight tiles are decoded exactly to bf16 in LDS and multiplied with bf16
// MFMA (v_mfma_f32_32x32x16_bf16) into f32.
//   e4m3: one f32 scale per 128x128 block; the MFMA sums of each 128-deep K
//         block go to a fresh f32 partial that is then added to the running
//         sum times the block's scale (dragon.c page, section 8 Round 3: the
//         128-column block structure folds the scale multiply out of the
//         inner loop).
//   e2m1: the power-of-two scale is applied exactly inside the fp4 -> bf16
//         conversion, so MFMA accumulates straight into the running sum.
//   NVFP4: each 16-input group's e4m3 scale multiplies the decoded values in
//         f32 (exact), so MFMA again accumulates straight into the sum.
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

#include <type_traits>

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

// Block order (1-D grid, XCD-aware).  Workgroup L is dispatched to XCD
// L % 8; XCD x takes the BNM-wide column blocks c = x (mod 8) of N and walks
// super-blocks of gt tile-list entries x gc of its column blocks (about the
// workgroups one XCD holds at once): inside a super-block the gc column
// blocks of one tile are neighbours (they share the tile's activation rows),
// and the M tiles of one expert sit next to each other in the tile list (they
// share the weight tile), so both are read from HBM about once per XCD
// through its L2.  Blocks past *n_tiles or past nb
// column blocks exit.  GATEUP: act = x [T][K], out = h bf16 [S][N] (N = f,
// K = d); otherwise act = h [S][K], out = y f32 [S][N] (N = d, K = f).
template <int FMT, bool GATEUP, int BM, int WM, int TN, int BK_, int PF>
__global__ __launch_bounds__(256, 2) void gemm_expert(
    const uint16_t* __restrict__ act, DMat W0, DMat W1, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    void* __restrict__ out, int N, int K, int T, int nb, int gc, int gt, int ntb) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  using C = G2<FMT, NMAT, BM, WM, TN, BK_>;
  constexpr int BK = C::BK, LDK = C::LDK, TM = C::TM, BNM = C::BNM;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int L = blockIdx.x, xcd = L & 7, sq = L >> 3;
  const int sbsz = gc * gt, sb = sq / sbsz, wi = sq - sb * sbsz;
  const int tb = sb % ntb, cb = sb / ntb;
  const int ti = tb * gt + wi / gc, cblk = xcd + 8 * (cb * gc + wi % gc);
  if (ti >= *n_tiles || cblk >= nb) return;
  const int4 tile = tiles[ti];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = cblk * BNM;
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
    // scale byte(s) of the chunk: one UE8M0 group (e2m1) or two e4m3 groups (NVFP4)
    bsr[i] = !ok ? nullptr
             : FMT == FMT_NVFP4 ? W.s + e * W.ss + (size_t)n * (K / 16) + 2 * c
                                : W.s + e * W.ss + (size_t)n * (K / 32) + c;
    bdst[i] = q < C::B_TOTAL ? C::A_ELEMS + (m * BNM + r) * LDK + c * C::B_EPC : -1;
  }

  // e4m3: this block's scale row (one 128-row block of N) for each matrix,
  // k-block kb held by lane kb % 64 of register kb / 64, read with v_readlane
  float scv[NMAT][2];
  if (FMT == FMT_E4M3) {
    const int nrb = min(n0, N - 1) >> 7, kbs = K >> 7;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const DMat& W = (m == 0) ? W0 : W1;
      const float* sf = reinterpret_cast<const float*>(W.s + e * W.ss) + (size_t)nrb * kbs;
      scv[m][0] = lane < kbs ? sf[lane] : 0.0f;
      scv[m][1] = lane + 64 < kbs ? sf[lane + 64] : 0.0f;
    }
  }

  // PF register sets of global loads in flight
  u32x4 ra[PF][C::A_CHUNKS], rb[PF][C::B_CHUNKS];
  float rsc[PF][C::B_CHUNKS][2];
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
      rsc[set][i][0] = rsc[set][i][1] = 1.0f;
      const int c = (tid + 256 * i) % C::B_CPR;
      if (bq[i] != nullptr && k0 + c * C::B_EPC < K) {
        const int64_t off = FMT == FMT_E4M3 ? k0 : k0 / 2;
        // a stage reads 64 (e4m3) or 32 (e2m1) bytes of a 128-byte row segment;
        // ordinary loads keep the line in L2 for the next stage's part
        rb[set][i] = *reinterpret_cast<const u32x4*>(bq[i] + off);
        if constexpr (FMT == FMT_E2M1) {
          rsc[set][i][0] = ue8m0_to_f32(bsr[i][k0 / 32]);
        } else if constexpr (FMT == FMT_NVFP4) {
          const uint32_t sb = *reinterpret_cast<const uint16_t*>(bsr[i] + k0 / 16);
          rsc[set][i][0] = e4m3_to_f32(sb & 0xFF);
          rsc[set][i][1] = e4m3_to_f32(sb >> 8);
        }
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
      if constexpr (FMT == FMT_E4M3) {
        bf16x2 o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = e4m3x2_to_bf16<false>(w[j]);
          o[2 * j + 1] = e4m3x2_to_bf16<true>(w[j]);
        }
        dst[0] = pack4(o[0], o[1], o[2], o[3]);
        dst[1] = pack4(o[4], o[5], o[6], o[7]);
      } else if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // words 0-1: first 16-input group, 2-3: second
          const float sc = rsc[set][i][j >> 1];
          bf16x2 o[4];
          o[0] = e2m1x2_times_to_bf16<0>(w[j], sc);
          o[1] = e2m1x2_times_to_bf16<1>(w[j], sc);
          o[2] = e2m1x2_times_to_bf16<2>(w[j], sc);
          o[3] = e2m1x2_times_to_bf16<3>(w[j], sc);
          dst[j] = pack4(o[0], o[1], o[2], o[3]);
        }
      } else {
        const float sc = rsc[set][i][0];
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

namespace moe {

// ---------------------------------------------------------------------------
// Register-weight grouped GEMM.  Same product as gemm_expert, with the weights
// kept out of LDS: each wavefront owns TNW 32-row weight tiles per matrix and
// loads, decodes and feeds them to the MFMA from its own registers; only the
// 64-token activation tile goes through LDS, where the four wavefronts share
// it.  Per 16-deep MFMA step a wavefront reads 2 activation fragments from
// LDS for 2 * NMAT * TNW MFMAs.
//
// v_mfma_f32_32x32x16_bf16: A = tokens (lane l: row l % 32, inputs of k-slot
// h = l / 32), B = weight rows (lane l: row l % 32, k-slot h).  A 64-input
// stage from k0: lane (r, h) loads the 32 weight inputs k0 + 32h .. k0 + 32h
// + 31 of its row (e4m3: 32 bytes; e2m1: 16 bytes and the row's ue8m0 byte
// of that 32-input group; NVFP4: 16 bytes and the two e4m3 bytes of its
// 16-input groups); MFMA step s = 0..3 takes inputs k0 + 32h + 8s ..
// + 7 from both operands.
template <int FMT, bool GATEUP, int TNW, int BM_ = 64>
struct RWCfg {
  static constexpr int NMAT = GATEUP ? 2 : 1;
  static constexpr int BM = BM_, BK = 64, LDK = BK + 8;  // tokens, stage depth, padded LDS row
  static constexpr int AC = BM * 8 / 256;               // 16-byte activation chunks per thread and stage
  static constexpr int TM = BM / 32;
  static constexpr int NW = NMAT * TNW;                 // 32-row weight tiles per wavefront
  static constexpr int BNM = 4 * 32 * TNW;              // weight rows per matrix per workgroup
  static_assert(128 % (32 * TNW) == 0, "a wavefront's rows lie in one 128-row scale block");
};

template <int FMT> struct RWRaw;
template <> struct RWRaw<FMT_E4M3> { u32x4 w[2]; };
template <> struct RWRaw<FMT_E2M1> { u32x4 w; float sc; };
template <> struct RWRaw<FMT_NVFP4> { u32x4 w; float sc[2]; };

// GATEUP: act = x [T][K], out = h bf16 [S][N] (N = f, K = d); else act = h
// [S][K], out = y f32 [S][N] (N = d, K = f).  Block order as gemm_expert.
// BM_ = 64: two workgroups per CU; BM_ = 128: one, with the 32-row token
// chunks past the tile's rows skipped.
template <int FMT, bool GATEUP, int TNW, int PD, int BM_ = 64>
__global__ __launch_bounds__(256, BM_ == 64 ? 2 : 1) void gemm_rw(
    const uint16_t* __restrict__ act, DMat W0, DMat W1, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    void* __restrict__ out, int N, int K, int T, int nb, int gc, int gt, int ntb) {
  using C = RWCfg<FMT, GATEUP, TNW, BM_>;
  constexpr int NMAT = C::NMAT, BM = C::BM, BK = C::BK, LDK = C::LDK, NW = C::NW, TM = C::TM;
  constexpr int AC = C::AC;
  __shared__ __attribute__((aligned(16))) uint16_t As[PD + 1][BM * LDK];
  const int L = blockIdx.x, xcd = L & 7, sq = L >> 3;
  const int sbsz = gc * gt, sb = sq / sbsz, wi = sq - sb * sbsz;
  const int tb = sb % ntb, cb = sb / ntb;
  const int ti = tb * gt + wi / gc, cblk = xcd + 8 * (cb * gc + wi % gc);
  if (ti >= *n_tiles || cblk >= nb) return;
  const int4 tile = tiles[ti];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = cblk * C::BNM;
  const int tid = threadIdx.x, lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int r32 = lane & 31, h = lane >> 5;
  const int nw0 = n0 + 32 * TNW * w;  // this wavefront's first weight row

  const int mt = (rows + 31) >> 5;  // 32-row token chunks holding rows
  // activation tile: BM rows x 64 inputs = 8 * BM 16-byte chunks, AC per thread
  const int acol = (tid & 7) * 8;
  const uint16_t* arow[AC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int r = (tid + 256 * i) >> 3;
    arow[i] = nullptr;
    if (r < rows) {
      const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + r], (uint32_t)(T - 1))
                                : (size_t)(p_start + r);
      arow[i] = act + src * K;
    }
  }
  // weight rows of this lane: tile idx = m * TNW + j holds row nw0 + 32j + r32 of matrix m
  const int64_t rbytes = FMT == FMT_E4M3 ? (int64_t)K : (int64_t)K / 2;
  const uint8_t* wrow[NW];
  const uint8_t* srow[NW];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const DMat& W = m == 0 ? W0 : W1;
      const int n = nw0 + 32 * j + r32;
      wrow[m * TNW + j] = n < N ? W.q + e * W.qs + n * rbytes : nullptr;
      srow[m * TNW + j] = n < N ? W.s + e * W.ss + (int64_t)n * (FMT == FMT_NVFP4 ? K >> 4 : K >> 5)
                                : nullptr;
    }
  const float* sblk[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const DMat& W = m == 0 ? W0 : W1;
    sblk[m] = reinterpret_cast<const float*>(W.s + e * W.ss) + (size_t)(min(nw0, N - 1) >> 7) * (K >> 7);
  }

  auto load_a = [&](u32x4 (&ra)[AC], int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i)
      ra[i] = arow[i] != nullptr && k0 + acol < K
                  ? *reinterpret_cast<const u32x4*>(arow[i] + k0 + acol) : u32x4{0u, 0u, 0u, 0u};
  };
  auto load_w = [&](RWRaw<FMT> (&rw)[NW], int k0) {
    const int k = k0 + 32 * h;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const bool ok = wrow[t] != nullptr && k < K;
      if constexpr (FMT == FMT_E4M3) {
        rw[t].w[0] = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + k) : u32x4{0u, 0u, 0u, 0u};
        rw[t].w[1] = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + k + 16) : u32x4{0u, 0u, 0u, 0u};
      } else if constexpr (FMT == FMT_NVFP4) {
        rw[t].w = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + k / 2) : u32x4{0u, 0u, 0u, 0u};
        const uint32_t sb = ok ? *reinterpret_cast<const uint16_t*>(srow[t] + (k >> 4)) : 0u;
        rw[t].sc[0] = e4m3_to_f32(sb & 0xFF);
        rw[t].sc[1] = e4m3_to_f32(sb >> 8);
      } else {
        rw[t].w = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + k / 2) : u32x4{0u, 0u, 0u, 0u};
        rw[t].sc = ok ? ue8m0_to_f32(srow[t][k >> 5]) : 1.0f;
      }
    }
  };
  auto store_a = [&](const u32x4 (&ra)[AC], uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < AC; ++i)
      *reinterpret_cast<u32x4*>(buf + ((tid + 256 * i) >> 3) * LDK + acol) = ra[i];
  };

  const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x16 acc[TM][NW], part[FMT == FMT_E4M3 ? TM : 1][FMT == FMT_E4M3 ? NW : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < NW; ++t) acc[i][t] = zero;
  if constexpr (FMT == FMT_E4M3) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < NW; ++t) part[i][t] = zero;
  }

  const int nk = (K + BK - 1) / BK;
  // One stage: issue the loads of stage ks + PD (clamped to the last stage, so
  // every stage issues the same loads and the wait counts stay static), run
  // the MFMAs of stage ks from LDS buffer ks % (PD + 1) and weight set `cur`,
  // then put stage ks + 1's activations (loaded PD - 1 stages ago) into LDS.
  constexpr int NB = PD + 1;  // LDS activation buffers and register sets
  // `even`: ks is even (compile-time after unrolling when NB is even): an
  // e4m3 scale block (two stages) starts there and ends on the odd stage
  auto stage = [&](int ks, bool even, const RWRaw<FMT> (&cur)[NW], RWRaw<FMT> (&pf)[NW],
                   u32x4 (&ra_pf)[AC], const u32x4 (&ra_next)[AC]) {
    const int kp = min(ks + PD, nk - 1) * BK;
    load_a(ra_pf, kp);
    load_w(pf, kp);
    const uint16_t* buf = As[ks % NB];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(buf + (32 * i + r32) * LDK + 32 * h + 8 * s);
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        bf16x8 b;
        if constexpr (FMT == FMT_E4M3) {
          const u32x4 v = cur[t].w[s >> 1];
          b = (s & 1) ? e4m3x8_to_bf16(v.z, v.w) : e4m3x8_to_bf16(v.x, v.y);
        } else if constexpr (FMT == FMT_NVFP4) {
          const u32x4 v = cur[t].w;
          b = nvfp4x8_to_bf16(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w, cur[t].sc[s >> 1]);
        } else {
          const u32x4 v = cur[t].w;
          b = e2m1x8_to_bf16(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w, cur[t].sc);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (TM > 2 && i >= mt) continue;  // chunk past the tile's rows (uniform)
          if constexpr (FMT == FMT_E4M3)
            part[i][t] = (even && s == 0)
                             ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, zero, 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, part[i][t], 0, 0, 0);
          else
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i][t], 0, 0, 0);
        }
      }
    }
    if constexpr (FMT == FMT_E4M3) {
      if (!even || ks == nk - 1) {  // end of a scale block: acc += scale * partial
        const int kb = ks >> 1;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const float sc = sblk[m][kb];
#pragma unroll
          for (int j = 0; j < TNW; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i][m * TNW + j][v] += sc * part[i][m * TNW + j][v];
        }
      }
    }
    if (ks + 1 < nk) store_a(ra_next, As[(ks + 1) % NB]);
    __syncthreads();
  };

  // prologue: stages 0 .. PD-1 loaded, stage 0's activations in LDS
  RWRaw<FMT> wr[NB][NW];
  u32x4 ra[NB][AC];
#pragma unroll
  for (int p = 0; p < PD; ++p) {
    load_a(ra[p], min(p, nk - 1) * BK);
    load_w(wr[p], min(p, nk - 1) * BK);
  }
  store_a(ra[0], As[0]);
  __syncthreads();
  for (int ks = 0; ks < nk; ks += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (ks + j < nk)
        stage(ks + j, NB % 2 == 0 ? (j % 2 == 0) : ((ks + j) % 2 == 0), wr[j], wr[(j + PD) % NB],
              ra[(j + PD) % NB], ra[(j + 1) % NB]);
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 32 * i + acc_row(v, lane);
        const int n = nw0 + 32 * j + r32;
        if (m < rows && n < N) {
          if (GATEUP)
            reinterpret_cast<uint16_t*>(out)[(size_t)(p_start + m) * N + n] =
                (uint16_t)f32_to_bf16_rne(silu(acc[i][j][v]) * acc[i][TNW + j][v]);
          else
            reinterpret_cast<float*>(out)[(size_t)(p_start + m) * N + n] = acc[i][j][v];
        }
      }
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Direct-to-LDS grouped GEMM: as gemm_rw (64 tokens x 4 wavefronts x TNW
// 32-row weight tiles per matrix), but every tile byte travels from global
// memory to LDS by global_load_lds_dwordx4 (lane l's 16 bytes land at LDS
// base + 16 l), so PD stages of loads are in flight without holding VGPRs.
// Activations: 64 rows x 128 bytes per stage, row r's 16-byte chunk c stored
// at slot c ^ (r & 7) (the MFMA fragment reads of 8 consecutive rows then hit
// 8 different bank groups).  Weights: each wavefront parks its own lanes'
// bytes and reads them back into the same lanes (no sharing, so no barrier
// for them); one barrier per stage publishes the activations and frees the
// buffer the next loads go to.  Each pipeline slot is its own LDS array, so
// a wait for one slot's loads leaves the others in flight.
template <int FMT, bool GATEUP, int TNW>
struct DmaCfg {
  static constexpr int NMAT = GATEUP ? 2 : 1;
  static constexpr int BM = 64, BK = 64, TM = 2;
  static constexpr int NW = NMAT * TNW;
  static constexpr int BNM = 4 * 32 * TNW;
  static constexpr int WLD = FMT == FMT_E4M3 ? 2 : 1;          // 16-byte weight loads per tile and stage
  static constexpr int A_V4 = BM * 8;                           // u32x4 per activation stage (8 KB)
  static constexpr int W_V4 = 4 * NW * WLD * 64;                // u32x4 per weight stage
  static constexpr int LOADS = 2 + NW * WLD + (FMT != FMT_E4M3 ? NW : 0);  // vector loads per wavefront and stage
};

// The direct-to-LDS loads and the stage barrier are issued as inline
// assembly: the compiler cannot tell the pipeline slots apart and would
// otherwise drain every outstanding load (vmcnt(0)) before each LDS read and
// each barrier.  The pipeline orders them itself: a wavefront waits until at
// most one stage of its loads is outstanding (vmcnt), then the barrier makes
// every wavefront's completed stage visible.
__device__ __forceinline__ void lds_dma16(const void* g, const u32x4* l) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) u32x4*)l);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int FMT, bool GATEUP, int TNW>
__global__ __launch_bounds__(256, 2) void gemm_dma(
    const uint16_t* __restrict__ act, DMat W0, DMat W1, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    void* __restrict__ out, int N, int K, int T, int nb, int gc, int gt, int ntb) {
  using C = DmaCfg<FMT, GATEUP, TNW>;
  constexpr int NMAT = C::NMAT, NW = C::NW, TM = C::TM, BK = C::BK, WLD = C::WLD;
  __shared__ u32x4 sA0[C::A_V4], sA1[C::A_V4], sA2[C::A_V4];
  __shared__ u32x4 sW0[C::W_V4], sW1[C::W_V4], sW2[C::W_V4];
  const int L = blockIdx.x, xcd = L & 7, sq = L >> 3;
  const int sbsz = gc * gt, sb = sq / sbsz, wi = sq - sb * sbsz;
  const int tb = sb % ntb, cb = sb / ntb;
  const int ti = tb * gt + wi / gc, cblk = xcd + 8 * (cb * gc + wi % gc);
  if (ti >= *n_tiles || cblk >= nb) return;
  const int4 tile = tiles[ti];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = cblk * C::BNM;
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int r32 = lane & 31, h = lane >> 5;
  const int nw0 = n0 + 32 * TNW * w;

  // activation loads of this lane: 2 per stage (rows (2w + i) * 8 + lane / 8,
  // LDS slot lane % 8 holding chunk slot ^ (row & 7)); rows past the tile
  // repeat its last row (their products only reach outputs that are not stored)
  const uint16_t* asrc[2];
  int achunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (2 * w + i) * 8 + (lane >> 3);
    const int rr = min(r, rows - 1);
    const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + rr], (uint32_t)(T - 1))
                              : (size_t)(p_start + rr);
    asrc[i] = act + src * K;
    achunk[i] = (lane & 7) ^ (r & 7);
  }
  // weight rows of this lane (clamped to the matrix; columns past N are not stored)
  const int64_t rbytes = FMT == FMT_E4M3 ? (int64_t)K : (int64_t)K / 2;
  const uint8_t* wrow[NW];
  const uint8_t* srow[NW];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const DMat& W = m == 0 ? W0 : W1;
      const int n = min(nw0 + 32 * j + r32, N - 1);
      wrow[m * TNW + j] = W.q + e * W.qs + n * rbytes;
      srow[m * TNW + j] = W.s + e * W.ss + (int64_t)n * (FMT == FMT_NVFP4 ? K >> 4 : K >> 5);
    }
  // e4m3: the scale row of this wavefront's 128-row block, k-block kb held by
  // lane kb % 64 of register kb / 64 (loaded before the pipeline starts)
  float scv[NMAT][2];
  if constexpr (FMT == FMT_E4M3) {
    const int kbs = K >> 7;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const DMat& W = m == 0 ? W0 : W1;
      const float* sf = reinterpret_cast<const float*>(W.s + e * W.ss) + (size_t)(min(nw0, N - 1) >> 7) * kbs;
      scv[m][0] = lane < kbs ? sf[lane] : 0.0f;
      scv[m][1] = lane + 64 < kbs ? sf[lane + 64] : 0.0f;
    }
  }

  const int nk = (K + BK - 1) / BK;
  // stage kk's loads into one pipeline slot (stages past the end repeat the
  // last one so every stage issues the same loads); e2m1 and NVFP4: the
  // lanes' scale bytes (one UE8M0 or two e4m3) go to registers
  auto issue = [&](int kk, const u32x4* sA, const u32x4* sW, float (&scs)[NW][2]) {
    const int k0 = min(kk, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kc = min(k0 + 8 * achunk[i], K - 8);
      lds_dma16(asrc[i] + kc, sA + (2 * w + i) * 64);
    }
    const int kl = min(k0 + 32 * h, K - 32);  // weight inputs of this lane (k-tail clamped; zeroed at decode)
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      if constexpr (FMT == FMT_E4M3) {
        lds_dma16(wrow[t] + kl, sW + ((w * NW + t) * 2 + 0) * 64);
        lds_dma16(wrow[t] + kl + 16, sW + ((w * NW + t) * 2 + 1) * 64);
      } else {
        lds_dma16(wrow[t] + kl / 2, sW + (w * NW + t) * 64);
        if constexpr (FMT == FMT_NVFP4) {
          const uint32_t sb = *reinterpret_cast<const uint16_t*>(srow[t] + (kl >> 4));
          scs[t][0] = e4m3_to_f32(sb & 0xFF);
          scs[t][1] = e4m3_to_f32(sb >> 8);
        } else {
          scs[t][0] = ue8m0_to_f32(srow[t][kl >> 5]);
        }
      }
    }
  };

  const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x16 acc[TM][NW], part[FMT == FMT_E4M3 ? TM : 1][FMT == FMT_E4M3 ? NW : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < NW; ++t) acc[i][t] = zero;
  if constexpr (FMT == FMT_E4M3) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < NW; ++t) part[i][t] = zero;
  }

  auto compute = [&](int ks, const u32x4* sA, const u32x4* sW, const float (&scs)[NW][2]) {
    const bool first = (ks & 1) == 0;
    const bool ktail = ks * BK + 32 * h >= K;  // e2m1: this lane's inputs past K
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = 32 * i + r32;
        a[i] = __builtin_bit_cast(bf16x8, sA[m * 8 + ((4 * h + s) ^ (m & 7))]);
      }
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        bf16x8 b;
        if constexpr (FMT == FMT_E4M3) {
          const u32x4 v = sW[((w * NW + t) * 2 + (s >> 1)) * 64 + lane];
          b = (s & 1) ? e4m3x8_to_bf16(v.z, v.w) : e4m3x8_to_bf16(v.x, v.y);
        } else {
          const u32x4 v = sW[(w * NW + t) * 64 + lane];
          const uint32_t word = ktail ? 0u : (s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w);
          if constexpr (FMT == FMT_NVFP4)
            b = nvfp4x8_to_bf16(word, scs[t][s >> 1]);
          else
            b = e2m1x8_to_bf16(word, scs[t][0]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (FMT == FMT_E4M3)
            part[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, (first && s == 0) ? zero : part[i][t], 0, 0, 0);
          else
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i][t], 0, 0, 0);
        }
      }
    }
    if constexpr (FMT == FMT_E4M3) {
      if ((ks & 1) == 1 || ks == nk - 1) {
        const int kb = ks >> 1;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const float sc = __int_as_float(__builtin_amdgcn_readlane(
              __float_as_int(kb < 64 ? scv[m][0] : scv[m][1]), kb & 63));
#pragma unroll
          for (int j = 0; j < TNW; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i][m * TNW + j][v] += sc * part[i][m * TNW + j][v];
        }
      }
    }
  };

  // three slots, two stages in flight: at stage ks wait for its loads, one
  // barrier (activations visible; slot of stage ks - 1 free), issue stage ks + 2
  // into that slot, compute stage ks
  float sc0[NW][2], sc1[NW][2], sc2[NW][2];
  constexpr int LD = C::LOADS;
  issue(0, sA0, sW0, sc0);
  issue(1, sA1, sW1, sc1);
  for (int ks = 0; ks < nk; ks += 3) {
    wait_vm<LD>();
    stage_barrier();
    issue(ks + 2, sA2, sW2, sc2);
    compute(ks, sA0, sW0, sc0);
    if (ks + 1 >= nk) break;
    wait_vm<LD>();
    stage_barrier();
    issue(ks + 3, sA0, sW0, sc0);
    compute(ks + 1, sA1, sW1, sc1);
    if (ks + 2 >= nk) break;
    wait_vm<LD>();
    stage_barrier();
    issue(ks + 4, sA1, sW1, sc1);
    compute(ks + 2, sA2, sW2, sc2);
  }
  // no load may still be writing this workgroup's LDS when it ends
  wait_vm<0>();

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 32 * i + acc_row(v, lane);
        const int n = nw0 + 32 * j + r32;
        if (m < rows && n < N) {
          if (GATEUP)
            reinterpret_cast<uint16_t*>(out)[(size_t)(p_start + m) * N + n] =
                (uint16_t)f32_to_bf16_rne(silu(acc[i][j][v]) * acc[i][TNW + j][v]);
          else
            reinterpret_cast<float*>(out)[(size_t)(p_start + m) * N + n] = acc[i][j][v];
        }
      }
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Grouped GEMM, every weight format: 8 wavefronts (2 per SIMD) in a WGM x
// (8 / WGM) grid; wavefront (wm, wn) owns TM 32-row token chunks of the tile
// (tokens 32 TM wm ..) and two 32-row weight tiles of column wn (gate and up
// rows 32 wn .. for gate/up; rows 64 wn .. for down).  A workgroup covers
// BM = 32 WGM TM tokens x 32 (8 / WGM) rows of each matrix (down: twice the
// rows), and every weight byte it loads feeds up to BM tokens: an expert with
// up to BM slots streams its weights once.  WGM = 2 with TM = 2..4 for tens
// to hundreds of slots per expert; WGM = 1 with TM = 1..2 (wide, short
// tiles) for a few.  All tile bytes move by direct-to-LDS loads into NS
// slots (as many as the 160 KB of LDS holds, at most 6; NS - 1 stages in
// flight), one workgroup per CU.
// LDS layouts (64 banks of 4 bytes; a 16-byte read serves 16 lanes per
// pass): activation row r (128 bytes per 64-input stage) holds its 16-byte
// chunk c at slot c ^ ((r >> 1) & 7), or (256 bytes per 128-input stage) at
// c ^ (r & 15); a 64-byte weight row (e4m3, or fp4 in a 128-input stage) its
// chunk c at slot c ^ ((r >> 2) & 3), a 32-byte fp4 row at c ^ ((r >> 3) & 1),
// so the fragment reads of 16 consecutive rows touch 16 different bank
// groups; each weight load instruction covers whole 64- or 32-byte row
// segments.
//
// e4m3 block scales without a second accumulator: a block scale s = 2^e * m
// (1 <= |m| < 2) is split; 2^e goes into the fp8 -> bf16 conversion (exact:
// an e4m3 value times a power of two is a bf16 value), and the running sum is
// kept in units of the current block's m: at each block boundary
// R <- R * (m_prev / m) in f32, then the block's MFMAs add into R, and the
// output is R * m_last.  This is the f32 sum of the scaled block products up
// to one f32 rounding per block of the running sum (relative 2^-24 each).
// fp4 scales are applied exactly in the conversion, so there is no rescale.
template <int FMT, bool GATEUP, int TNW, int TM_, int WGM_>
struct BigCfg {
  static constexpr bool FP4 = FMT != FMT_E4M3;
  static constexpr int NMAT = GATEUP ? 2 : 1;
  static constexpr int WGM = WGM_, WGN = 8 / WGM;      // wavefront grid
  static constexpr int TM = TM_, BM = 32 * WGM * TM;
  // fp4 tiles of 128 tokens x 128 rows per matrix take 128-input stages, so
  // each weight row is read 64 contiguous bytes at a time (32 with 64-input
  // stages); taller or wider tiles (whose LDS would then hold only 2 stages)
  // and e4m3 (64 bytes per row already) take 64-input stages
  static constexpr int BK = FP4 && WGM == 2 && BM <= 128 ? 128 : 64;
  static constexpr int ACH = BK / 8;                   // 16-byte activation chunks per row and stage
  static constexpr int NW = NMAT * TNW;                // weight tiles per wavefront (2)
  static constexpr int BNM = WGN * 32 * TNW;           // weight rows per matrix per workgroup
  static constexpr int A_V4 = BM * ACH;                // u32x4 per activation stage (BM x 2 BK bytes)
  static constexpr int AL = (A_V4 + 511) / 512;        // activation loads per lane and stage
  static constexpr int WL = FP4 ? BK / 64 : 2;         // weight loads per lane, tile and stage
  static constexpr int SL = FP4 ? BK / 64 : 0;         // fp4 scale loads per lane, tile and stage
  static constexpr int TPW = NW / WGM;                 // weight tiles each wavefront loads
  static constexpr int W_V4 = WGN * NW * WL * 64;      // u32x4 per weight stage
  static constexpr int S_V4 = WGN * NW * 16 * SL;      // fp4: SL scale dwords per lane and tile, after the weights
  static constexpr int LOADS = AL + TPW * (WL + SL);   // direct-to-LDS loads per lane and stage
  static constexpr int SLOT = 16 * (A_V4 + W_V4 + S_V4);
  static constexpr int NS = 160 * 1024 / SLOT > 6 ? 6 : 160 * 1024 / SLOT;  // slots the 160 KB of LDS holds
  static_assert(NS >= 3, "two stages in flight");
  static_assert(NW == 2 && (WGM == 1 || WGM == 2), "the wavefronts of a column share its two weight tiles");
};

// The power-of-two part (exponent bits) and the signed mantissa part (+-[1, 2))
// of a normal f32, whose product is the value.
__device__ __forceinline__ float pow2_part(float s) { return __uint_as_float(__float_as_uint(s) & 0x7F800000u); }
__device__ __forceinline__ float mant_part(float s) {
  return __uint_as_float((__float_as_uint(s) & 0x807FFFFFu) | 0x3F800000u);
}
// e4m3 pairs times a power of two -> bf16 (exact; the conversion applies the
// exponent of its scale operand)
__device__ __forceinline__ bf16x8 e4m3x8_scaled_to_bf16(uint32_t lo, uint32_t hi, float p2) {
  return pack_bf16x8(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, p2, false),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, p2, true),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, p2, false),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, p2, true));
}
// Direct-to-LDS loads of one byte / one 16-bit word per lane: lane l's value,
// zero-extended, lands in the dword at LDS base + 4 l.
__device__ __forceinline__ void lds_dma_u8(const void* g, const uint32_t* l) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint32_t*)l);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ubyte %0, off" ::"v"(g), "s"(a) : "m0");
}
__device__ __forceinline__ void lds_dma_u16(const void* g, const uint32_t* l) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint32_t*)l);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ushort %0, off" ::"v"(g), "s"(a) : "m0");
}

template <int FMT, bool GATEUP, int TNW, int TM_, int WGM_>
__global__ __launch_bounds__(512, 1) void gemm_big(
    const uint16_t* __restrict__ act, DMat W0, DMat W1, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    void* __restrict__ out, int N, int K, int T, int nb) {
  using C = BigCfg<FMT, GATEUP, TNW, TM_, WGM_>;
  constexpr bool FP4 = C::FP4;
  constexpr int NMAT = C::NMAT, NW = C::NW, TM = C::TM, BK = C::BK, NS = C::NS, AL = C::AL;
  constexpr int WGM = C::WGM, BM = C::BM, TPW = C::TPW;
  __shared__ u32x4 sA[NS][C::A_V4];
  __shared__ u32x4 sW[NS][C::W_V4 + C::S_V4];
  // fp4 scale dwords of slot s: after the slot's weight bytes
  auto sS = [&](int slot) { return reinterpret_cast<uint32_t*>(&sW[slot][C::W_V4]); };
  // Block order: workgroup L runs on XCD L % 8; XCD x takes the tile-list
  // entries x, x + 8, ... and each entry's nb column blocks in turn, so an
  // entry's activation rows are fetched into one XCD's L2 and serve all of
  // its column blocks, and each weight byte is read by one workgroup.
  const int L = blockIdx.x, xcd = L & 7, sq = L >> 3;
  const int lt = sq / nb, cblk = sq - lt * nb;
  const int ti = 8 * lt + xcd;
  if (ti >= *n_tiles) return;
  const int4 tile = tiles[ti];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const int n0 = cblk * C::BNM;
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int wm = WGM == 2 ? w >> 2 : 0, wn = WGM == 2 ? w & 3 : w;
  const int r32 = lane & 31, h = lane >> 5;
  const int nw0 = n0 + 32 * TNW * wn;  // this column's first weight row
  // 32-row token chunks of this wavefront that hold rows (uniform, 0..4)
  const int nact = min(max(((rows + 31) >> 5) - TM * wm, 0), TM);

  // activation loads of this lane: AL per stage, rows (AL w + i) * (64 / ACH)
  // + lane / ACH mod BM (a short tile's rows are loaded twice, to the same
  // place; rows past the tile repeat its last row, their outputs are not
  // stored), LDS slot lane % ACH of the row holding chunk slot ^ aswz(row):
  // 128-byte rows (8 chunks) swizzle by (row >> 1) & 7, 256-byte rows (16
  // chunks) by row & 15, so each 16-lane pass of a fragment read touches 16
  // bank groups
  auto aswz = [](int r) { return C::ACH == 8 ? ((r >> 1) & 7) : (r & 15); };
  const uint16_t* asrc[AL];
  int achunk[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int r = ((AL * w + i) * (64 / C::ACH) + lane / C::ACH) % BM;
    const int rr = min(r, rows - 1);
    const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + rr], (uint32_t)(T - 1))
                              : (size_t)(p_start + rr);
    asrc[i] = act + src * K;
    achunk[i] = (lane % C::ACH) ^ aswz(r);
  }
  // activation loads of this wavefront that hold rows of the tile (its first
  // n_a; a load of 8 rows all past `rows` is skipped: the MFMAs of rows past
  // `rows` only reach outputs that are not stored, so their LDS bytes may be
  // stale)
  int n_a = 0;
#pragma unroll
  for (int i = 0; i < AL; ++i) n_a += (((AL * w + i) * (64 / C::ACH)) % BM) < rows ? 1 : 0;
  // the weight tiles this wavefront loads: WGM = 2: tile wm of its column
  // (the other wavefront of the column loads the other); WGM = 1: both.  Tile
  // t is matrix t for gate/up, rows 32 t .. of the column for down; rows are
  // clamped to N.  64 bytes of a row per stage (e4m3, and fp4 with 128-input
  // stages): load j covers tile rows 16 j + lane / 4, slot lane % 4 holding
  // chunk slot ^ ((row >> 2) & 3).  fp4 with 64-input stages (32 bytes): one
  // load covers the 32 rows, slot lane % 2 of row lane / 2 holding chunk
  // slot ^ ((row >> 3) & 1).  The fp4 scales of lane (r, h): those of its
  // 32-input chunks c = CPL h .. CPL h + CPL - 1 of row r, one load per chunk
  // (e2m1: one UE8M0 byte; NVFP4: the two e4m3 bytes of its 16-input halves).
  constexpr int CPL = BK / 64;  // fp4: 32-input chunks per lane and stage
  const int64_t rbytes = FP4 ? (int64_t)K / 2 : (int64_t)K;
  const int sgroups = FMT == FMT_NVFP4 ? K >> 4 : K >> 5;
  int tls[TPW];
  const uint8_t* wsrc[TPW][2];
  const uint8_t* wsrc16[TPW];  // fp4 with 128-input stages: the rows of load 1 (16 further)
  int wchunk[2] = {0, 0};
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tl = WGM == 2 ? wm : u;
    tls[u] = tl;
    const int ml = GATEUP ? tl : 0, jl = GATEUP ? 0 : tl;
    const DMat& WL = ml == 0 ? W0 : W1;
    if constexpr (!FP4) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tr = 16 * j + (lane >> 2);
        wsrc[u][j] = WL.q + e * WL.qs + (int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes +
                     16 * ((lane & 3) ^ ((tr >> 2) & 3));
      }
    } else if constexpr (CPL == 1) {
      const int tr = lane >> 1;
      wchunk[0] = (lane & 1) ^ ((tr >> 3) & 1);
      wsrc[u][0] = WL.q + e * WL.qs + (int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes;
      wsrc[u][1] = WL.s + e * WL.ss + (int64_t)min(nw0 + 32 * jl + r32, N - 1) * sgroups;
    } else {
      // load j covers tile rows 16 j + lane / 4
      const int tr = lane >> 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) wchunk[j] = (lane & 3) ^ (((16 * j + tr) >> 2) & 3);
      wsrc[u][0] = WL.q + e * WL.qs + (int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes;
      wsrc16[u] = WL.q + e * WL.qs + (int64_t)min(nw0 + 32 * jl + 16 + tr, N - 1) * rbytes;
      wsrc[u][1] = WL.s + e * WL.ss + (int64_t)min(nw0 + 32 * jl + r32, N - 1) * sgroups;
    }
  }
  // e4m3 scales of this column's 128-row block, k-block kb in lane kb % 64 of register kb / 64
  float scv[NMAT][2];
  if constexpr (!FP4) {
    const int kbs = K >> 7;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const DMat& W = m == 0 ? W0 : W1;
      const float* sf = reinterpret_cast<const float*>(W.s + e * W.ss) + (size_t)(min(nw0, N - 1) >> 7) * kbs;
      scv[m][0] = lane < kbs ? sf[lane] : 1.0f;
      scv[m][1] = lane + 64 < kbs ? sf[lane + 64] : 1.0f;
    }
  }
  auto block_scale = [&](int m, int kb) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? scv[m][0] : scv[m][1]), kb & 63));
  };

  const int nk = (K + BK - 1) / BK;
  // stage kk's loads into slot `slot` (addresses clamped into the rows at a
  // k-tail; those inputs are zeroed at decode)
  auto issue = [&](int kk, int slot) {
    const int k0 = kk * BK;
#pragma unroll
    for (int i = 0; i < AL; ++i)
      if (i < n_a)
        lds_dma16(asrc[i] + min(k0 + 8 * achunk[i], K - 8), &sA[slot][((AL * w + i) * 64) % C::A_V4]);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tl = tls[u];
      if constexpr (!FP4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) lds_dma16(wsrc[u][j] + k0, &sW[slot][((wn * NW + tl) * 2 + j) * 64]);
      } else {
        const int tile = wn * NW + tl;
        if constexpr (CPL == 1) {
          lds_dma16(wsrc[u][0] + min(k0 + 32 * wchunk[0], K - 32) / 2, &sW[slot][tile * 64]);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            lds_dma16((j == 0 ? wsrc[u][0] : wsrc16[u]) + min(k0 + 32 * wchunk[j], K - 32) / 2,
                      &sW[slot][(tile * 2 + j) * 64]);
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int kl = min(k0 + 32 * (CPL * h + c), K - 32);
          if constexpr (FMT == FMT_NVFP4)
            lds_dma_u16(wsrc[u][1] + (kl >> 4), sS(slot) + (tile * CPL + c) * 64);
          else
            lds_dma_u8(wsrc[u][1] + (kl >> 5), sS(slot) + (tile * CPL + c) * 64);
        }
      }
    }
  };

  const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x16 R[TM][NW];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < NW; ++t) R[i][t] = zero;
  float p2[NMAT], mcur[NMAT];  // e4m3: power-of-two and mantissa parts of the current block's scale
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    p2[m] = FP4 ? 1.0f : pow2_part(block_scale(m, 0));
    mcur[m] = FP4 ? 1.0f : mant_part(block_scale(m, 0));
  }

  auto compute = [&](int ks, int slot) {
    // e4m3, a new 128-deep scale block: R <- R * (m_prev / m), chunk by
    // chunk just before the chunk's first MFMA of the block (the multiplies
    // of one chunk then overlap the MFMAs of the one before)
    const bool newblk = !FP4 && (ks & 1) == 0 && ks > 0;
    float ratio[NMAT];
    if (newblk) {
      const int kb = ks >> 1;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const float sc = block_scale(m, kb);
        const float mn = mant_part(sc);
        ratio[m] = mcur[m] / mn;
        p2[m] = pow2_part(sc);
        mcur[m] = mn;
      }
    }
    const u32x4* a_s = sA[slot];
    const u32x4* w_s = sW[slot];
    // this stage's weight fragments, decoded once for all token chunks
    constexpr int NSTEP = C::ACH / 2;  // 16-input MFMA steps per stage
    bf16x8 b[NW][NSTEP];
    if constexpr (!FP4) {
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int q = 0; q < 2; ++q) {  // chunk 2h + q of row r32
          const u32x4 v = w_s[(wn * NW + t) * 128 + r32 * 4 + ((2 * h + q) ^ ((r32 >> 2) & 3))];
          const float ps = p2[GATEUP ? t : 0];
          b[t][2 * q] = e4m3x8_scaled_to_bf16(v.x, v.y, ps);
          b[t][2 * q + 1] = e4m3x8_scaled_to_bf16(v.z, v.w, ps);
        }
    } else {
#pragma unroll
      for (int t = 0; t < NW; ++t) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = CPL * h + c;  // this lane's 32-input chunk of the stage
          u32x4 v = CPL == 1 ? w_s[(wn * NW + t) * 64 + r32 * 2 + (h ^ ((r32 >> 3) & 1))]
                             : w_s[(wn * NW + t) * 128 + r32 * 4 + (ch ^ ((r32 >> 2) & 3))];
          if (ks * BK + 32 * ch >= K) v = u32x4{0u, 0u, 0u, 0u};  // inputs past K
          const uint32_t sb = sS(slot)[((wn * NW + t) * CPL + c) * 64 + lane];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (FMT == FMT_NVFP4)
              b[t][4 * c + q] = nvfp4x8_to_bf16(wd[q], e4m3_to_f32(q < 2 ? (sb & 0xFF) : (sb >> 8)));
            else
              b[t][4 * c + q] = e2m1x8_to_bf16(wd[q], ue8m0_to_f32(sb));
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= nact) break;  // uniform
      if (newblk) {
#pragma unroll
        for (int t = 0; t < NW; ++t) {
          const float r = ratio[GATEUP ? t : 0];
#pragma unroll
          for (int v = 0; v < 16; ++v) R[i][t][v] *= r;
        }
      }
      const int mrow = 32 * TM * wm + 32 * i + r32;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, a_s[mrow * C::ACH + ((NSTEP * h + s) ^ aswz(mrow))]);
#pragma unroll
        for (int t = 0; t < NW; ++t) R[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[t][s], R[i][t], 0, 0, 0);
      }
    }
  };

  // NS slots, NS - 1 stages in flight: at stage ks wait for its loads (later
  // stages may stay outstanding), one barrier (its bytes visible to every
  // wavefront; the slot of stage ks - 1 free), issue stage ks + NS - 1 into
  // that slot, compute stage ks.  Past the last issue the waits drain all.
  // loads per lane and stage of this wavefront: LD minus its skipped activation loads
  constexpr int LDW = C::LOADS - AL;
  auto wait_stage = [&]() {  // all but the NS - 2 most recent stages' loads done
    switch (n_a) {
      case 0: wait_vm<(NS - 2) * LDW>(); break;
      case 1: wait_vm<(NS - 2) * (LDW + 1)>(); break;
      case 2: wait_vm<(NS - 2) * (LDW + (AL >= 2 ? 2 : 1))>(); break;
      case 3: wait_vm<(NS - 2) * (LDW + (AL >= 3 ? 3 : 1))>(); break;
      default: wait_vm<(NS - 2) * (LDW + AL)>(); break;
    }
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nk) issue(p, p);
  for (int ks0 = 0; ks0 < nk; ks0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int ks = ks0 + j;
      if (ks >= nk) break;
      if (ks + NS - 2 < nk)
        wait_stage();
      else
        wait_vm<0>();
      stage_barrier();
      if (ks + NS - 1 < nk) issue(ks + NS - 1, (j + NS - 1) % NS);
      compute(ks, j);
    }
  }
  wait_vm<0>();

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i >= nact) break;
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 32 * TM * wm + 32 * i + acc_row(v, lane);
        const int n = nw0 + 32 * j + r32;
        if (m < rows && n < N) {
          if (GATEUP) {
            const float g = R[i][j][v] * mcur[0], u = R[i][TNW + j][v] * mcur[NMAT - 1];
            reinterpret_cast<uint16_t*>(out)[(size_t)(p_start + m) * N + n] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
          } else {
            reinterpret_cast<float*>(out)[(size_t)(p_start + m) * N + n] = R[i][j][v] * mcur[0];
          }
        }
      }
  }
}

}  // namespace moe
