// Grouped variant of the expert stage: for many tokens per expert, each
// expert's rows (in sorted-slot order) form the M dimension of GEMM tiles.
// Weight tiles are decoded exactly to bf16 in registers and multiplied with
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) into f32.
//   e4m3: one f32 scale per 128x128 block, applied per 128-deep K block
//         (dragon.c page, section 8 Round 3: the 128-column block structure
//         folds the scale multiply out of the inner loop); how, below.
//   e2m1: the power-of-two scale is applied exactly inside the fp4 -> bf16
//         conversion, so MFMA accumulates straight into the running sum.
//   NVFP4: each 16-input group's e4m3 scale multiplies the decoded values in
//         f32 (exact), so MFMA again accumulates straight into the sum.
// The A rows of the gate/up GEMM are the tokens' own activation rows, read
// through the permutation and never copied (Trochilus README, "How it keeps
// up": gate and up read a token's row through a map instead of gathered
// copies).  Gate and up rows of the same output column sit in the same lane
// and register, so SwiGLU and the bf16 rounding of h happen in registers.
#pragma once

#include <type_traits>
#include <utility>

#include "moe_common.h"
#include "moe_decode.h"

namespace moe {

// e4m3 grouped GEMM: K <= 127 * 128 (one lane per 128-deep block in 2 VGPRs,
// and a lane for the block after the last one)
constexpr int MAX_KBLK = 127;

// Row index (within the 32x32 tile) of accumulator register v for this lane;
// the column is lane % 32.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// The direct-to-LDS loads and the stage barrier are issued as inline
// assembly: the compiler cannot tell the pipeline slots apart and would
// otherwise drain every outstanding load (vmcnt(0)) before each LDS read and
// each barrier.  The pipeline orders them itself: a wavefront waits until at
// most the stages it still needs in flight are outstanding (vmcnt), then the
// barrier makes every wavefront's completed stage visible.  Lane l's 16
// bytes land at LDS base + 16 l.
__device__ __forceinline__ void lds_dma16(const void* g, const u32x4* l) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) u32x4*)l);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "m0");
}
// One byte / one 16-bit word per lane: lane l's value, zero-extended, lands in
// the dword at LDS base + 4 l.
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
// The same from a uniform base (an SGPR pair) plus a 32-bit per-lane byte
// offset, to the LDS byte address `lds`: the offsets stay in registers for the
// whole K loop and only the base advances.
__device__ __forceinline__ void lds_dma16_so(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Grouped GEMM, every weight format: 8 wavefronts (2 per SIMD) in a WGM x
// (8 / WGM) grid.  Wavefront (wm, wn) owns two 32-row weight tiles of column
// wn (gate and up rows 32 wn .. for gate/up; rows 64 wn .. for down) and the
// 32-row token chunks wm, wm + WGM, wm + 2 WGM, ... of the tile (up to TM of
// them): interleaved, so the two wavefront rows of a column carry the same
// number of chunks (+-1) whatever the tile's row count.  A workgroup covers
// BM = 32 WGM TM tokens x 32 (8 / WGM) rows of each matrix (down: twice the
// rows), and every weight byte it loads feeds up to BM tokens: an expert with
// up to BM slots streams its weights once.  The K loop is instantiated per
// number of active chunks of the wavefront, so its body has no branches
// between chunks.  All tile bytes move by direct-to-LDS loads into NS slots
// (as many as the 160 KB of LDS holds, at most 6; NS - 1 stages in flight),
// one workgroup per CU.  With one wavefront row, each wavefront's weight rows
// are its own: it reloads them right after its own compute of a stage, ahead
// of the barrier that the shared activation rows need.
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
// kept in units of the current block's m: after a block's last MFMAs
// R <- R * (m / m_next) in f32, then the next block's MFMAs add into R, and
// the output is R * m_last.  This is the f32 sum of the scaled block products
// up to two f32 roundings per block (the ratio and the product; relative
// 2^-24 each).  The ratios and powers of two of all of a column's blocks are
// computed once per workgroup, one block per lane.  The rescale of a token
// chunk's accumulators follows that chunk's last MFMAs of the block, so it
// overlaps the next chunk's MFMAs; the last chunk's waits for the next
// block's first chunk.  fp4 scales are applied exactly in the conversion, so
// there is no rescale.
//
// The kernel runs at the chip's power limit (the shader clock drops to about
// 1.7 GHz on quantised-normal data, against 2.35 GHz on zeros), so work that
// does not reach an output costs time even when it hides behind loads: the
// padding rows of a tile's last chunk are zeros, not copies of a token.
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
  // stages per unrolled loop trip: a multiple of NS (slot indices are then
  // compile-time) and, for e4m3, of the 2 stages of a 128-deep scale block
  // (the block boundaries are then compile-time too)
  static constexpr int UNR = (!FP4 && NS % 2) ? 2 * NS : NS;
  static_assert(NS >= 3, "two stages in flight");
  static_assert(NW == 2 && (WGM == 1 || WGM == 2), "the wavefronts of a column share its two weight tiles");
  static_assert(FP4 || BK == 64, "e4m3: two stages per 128-deep scale block");
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

// Calls f(std::integral_constant<int, j>) for j = 0 .. N-1 in order.
template <class F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Calls f(std::integral_constant<int, n>) for a run-time n in [0, MAX].
template <int MAX, int I = 0, class F>
__device__ __forceinline__ void dispatch_count(int n, F&& f) {
  if constexpr (I > MAX) {
    return;
  } else {
    if (n == I)
      f(std::integral_constant<int, I>{});
    else
      dispatch_count<MAX, I + 1>(n, f);
  }
}

template <int FMT, bool GATEUP, int TNW, int TM_, int WGM_>
__global__ __launch_bounds__(512, 1) void gemm_big(
    const uint16_t* __restrict__ act, DMat W0, DMat W1, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const int32_t* __restrict__ tok_of,
    void* __restrict__ out, int N, int K, int T, int nb, int max_tiles) {
  using C = BigCfg<FMT, GATEUP, TNW, TM_, WGM_>;
  constexpr bool FP4 = C::FP4;
  constexpr int NMAT = C::NMAT, NW = C::NW, TM = C::TM, BK = C::BK, NS = C::NS, AL = C::AL;
  constexpr int WGM = C::WGM, BM = C::BM, TPW = C::TPW, UNR = C::UNR;
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
  // the entry is read beside the count (clamped into the list), so the two
  // loads take one memory round trip
  const int4 tile = tiles[min(ti, max_tiles - 1)];
  if (ti >= *n_tiles) return;
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const bool sh = tile.w != 0;  // the shared expert's rows
  const int n0 = cblk * C::BNM;
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int wm = WGM == 2 ? w >> 2 : 0, wn = WGM == 2 ? w & 3 : w;
  const int r32 = lane & 31, h = lane >> 5;
  const int nw0 = n0 + 32 * TNW * wn;  // this column's first weight row
  // 32-row token chunks of the tile that hold rows, and this wavefront's share
  // (chunks wm, wm + WGM, ...; uniform, 0..TM)
  const int nch = (rows + 31) >> 5;
  const int nact = min(max((nch - wm + WGM - 1) / WGM, 0), TM);

  // activation loads of this lane: AL per stage, rows (AL w + i) * (64 / ACH)
  // + lane / ACH (rows past the tile repeat its last row, their outputs are
  // not stored; a load whose first row is past the tile is not issued), LDS
  // slot lane % ACH of the row holding chunk slot ^ aswz(row):
  // 128-byte rows (8 chunks) swizzle by (row >> 1) & 7, 256-byte rows (16
  // chunks) by row & 15, so each 16-lane pass of a fragment read touches 16
  // bank groups
  auto aswz = [](int r) { return C::ACH == 8 ? ((r >> 1) & 7) : (r & 15); };
  const uint16_t* asrc[AL];
  int achunk[AL];
  uint32_t aoff[AL];  // e4m3: byte offset of the lane's chunk from act + 2 k0
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int r = min((AL * w + i) * (64 / C::ACH) + lane / C::ACH, BM - 1);
    const int rr = min(r, rows - 1);
    const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + rr], (uint32_t)(T - 1))
                              : (size_t)(p_start + rr);
    asrc[i] = act + src * K;
    achunk[i] = (lane % C::ACH) ^ aswz(r);
    aoff[i] = (uint32_t)(src * K * 2 + 16 * achunk[i]);
  }
  // LDS byte addresses of the two rings
  const uint32_t lds_a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) u32x4*)&sA[0][0];
  const uint32_t lds_w = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) u32x4*)&sW[0][0];
  // activation loads of this wavefront that hold rows of the tile (its first
  // n_a; a load of 8 rows all past `rows` is skipped: the MFMAs of rows past
  // `rows` only reach outputs that are not stored, so their LDS bytes may be
  // stale)
  int n_a = 0;
#pragma unroll
  for (int i = 0; i < AL; ++i) n_a += (AL * w + i) * (64 / C::ACH) < min(rows, BM) ? 1 : 0;
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
  const uint8_t* wbase[TPW];  // e4m3: the matrix of the tile (uniform)
  uint32_t woff[TPW][2];      // e4m3: byte offset of the lane's 16 bytes from wbase + k0
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
      wbase[u] = mat_q(WL, e, sh);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tr = 16 * j + (lane >> 2);
        woff[u][j] = (uint32_t)((int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes +
                                16 * ((lane & 3) ^ ((tr >> 2) & 3)));
        wsrc[u][j] = nullptr;
      }
      wsrc16[u] = nullptr;
    } else if constexpr (CPL == 1) {
      const int tr = lane >> 1;
      wchunk[0] = (lane & 1) ^ ((tr >> 3) & 1);
      wsrc[u][0] = mat_q(WL, e, sh) + (int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes;
      wsrc[u][1] = mat_s(WL, e, sh) + (int64_t)min(nw0 + 32 * jl + r32, N - 1) * sgroups;
      wsrc16[u] = nullptr;
    } else {
      // load j covers tile rows 16 j + lane / 4
      const int tr = lane >> 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) wchunk[j] = (lane & 3) ^ (((16 * j + tr) >> 2) & 3);
      wsrc[u][0] = mat_q(WL, e, sh) + (int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes;
      wsrc16[u] = mat_q(WL, e, sh) + (int64_t)min(nw0 + 32 * jl + 16 + tr, N - 1) * rbytes;
      wsrc[u][1] = mat_s(WL, e, sh) + (int64_t)min(nw0 + 32 * jl + r32, N - 1) * sgroups;
    }
  }
  // e4m3: for k-block kb = lane + 64 q of this column's 128-row block (lane
  // kb % 64 of register kb / 64), the power of two of its scale and the ratio
  // of the previous block's mantissa to its own (1 for block 0 and for the
  // block after the last); m_last, the last block's mantissa, scales the
  // output
  float pw[NMAT][2], rt[NMAT][2], mlast[NMAT];
  // (loaded after the prologue's loads are issued: they are first needed by
  // the first stage's compute)
  auto load_scales = [&]() {
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    pw[m][0] = pw[m][1] = rt[m][0] = rt[m][1] = mlast[m] = 1.0f;
    if constexpr (!FP4) {
      const int kbs = K >> 7;
      const DMat& W = m == 0 ? W0 : W1;
      const float* sf = reinterpret_cast<const float*>(mat_s(W, e, sh)) + (size_t)(min(nw0, N - 1) >> 7) * kbs;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int kb = lane + 64 * q;
        const float s = kb < kbs ? sf[kb] : 1.0f;
        const float sp = kb >= 1 && kb < kbs ? sf[kb - 1] : s;
        pw[m][q] = pow2_part(s);
        rt[m][q] = mant_part(sp) / mant_part(s);
      }
      mlast[m] = mant_part(sf[kbs - 1]);
    }
  }
  };
  auto lane_of = [](const float (&v)[2], int kb) {  // uniform kb
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? v[0] : v[1]), kb & 63));
  };

  const int nk = (K + BK - 1) / BK;
  // stage kk's loads into slot `slot` (addresses clamped into the rows at a
  // k-tail; those inputs are zeroed at decode)
  // e4m3 (K a multiple of 128: no chunk of a stage runs past the row): the
  // activation and the weight loads of stage kk into slot `slot`
  // lanes whose activation row is past the tile load nothing: those rows of
  // the tile's last 32-row chunk are zeroed once in every slot below, so the
  // MFMAs of the padding rows multiply zeros (their outputs are not stored;
  // zero operands only save switching power)
  bool alive[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) alive[i] = (AL * w + i) * (64 / C::ACH) + lane / C::ACH < rows;
  auto issue_act = [&](int kk, int slot) {
    const uint8_t* abase = reinterpret_cast<const uint8_t*>(act) + 2 * (size_t)(kk * BK);
#pragma unroll
    for (int i = 0; i < AL; ++i)
      if (i < n_a && alive[i]) lds_dma16_so(abase, aoff[i], lds_a + 16 * (slot * C::A_V4 + (AL * w + i) * 64));
  };
  {
    const int r1 = min(BM, 32 * ((rows + 31) >> 5));
    const int n = (r1 - rows) * C::ACH;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      for (int idx = (int)threadIdx.x; idx < n; idx += 512) sA[sl][rows * C::ACH + idx] = u32x4{0u, 0u, 0u, 0u};
  }
  auto issue_wt = [&](int kk, int slot) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        lds_dma16_so(wbase[u] + kk * BK, woff[u][j],
                     lds_w + 16 * (slot * (C::W_V4 + C::S_V4) + ((wn * NW + tls[u]) * 2 + j) * 64));
  };
  auto issue = [&](int kk, int slot) {
    const int k0 = kk * BK;
    if constexpr (!FP4) {
      issue_act(kk, slot);
      issue_wt(kk, slot);
      return;
    }
#pragma unroll
    for (int i = 0; i < AL; ++i)
      if (i < n_a && alive[i])
        lds_dma16(asrc[i] + min(k0 + 8 * achunk[i], K - 8), &sA[slot][(AL * w + i) * 64]);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tl = tls[u];
      if constexpr (!FP4) {
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

  // NS slots, NS - 1 stages in flight: at stage ks wait for its loads (later
  // stages may stay outstanding), one barrier (its bytes visible to every
  // wavefront; the slot of stage ks - 1 free), issue stage ks + NS - 1 into
  // that slot, compute stage ks.  Past the last issue the waits drain all.
  // loads per lane and stage of this wavefront: LD minus its skipped activation loads
  constexpr int LDW = C::LOADS - AL;
  // One wavefront row (e4m3): a wavefront's weight rows are its own, so it
  // refills its weight region of a slot right after its own compute of the
  // stage there (weights of stage ks + NS), before the next barrier; the
  // activations, shared by all wavefronts, follow the barrier as before.
  // Per wavefront the issue order is then ... A(ks), W(ks + 1), A(ks + 1),
  // ..., W(ks + NS - 1) when stage ks is waited for: all but the last
  // LDW + (NS - 2) (LDW + n_a) loads must be done.
  constexpr bool EARLYW = !FP4 && WGM == 1;
  auto wait_early = [&]() {
    switch (n_a) {
      case 0: wait_vm<LDW + (NS - 2) * LDW>(); break;
      case 1: wait_vm<LDW + (NS - 2) * (LDW + 1)>(); break;
      case 2: wait_vm<LDW + (NS - 2) * (LDW + (AL >= 2 ? 2 : 1))>(); break;
      case 3: wait_vm<LDW + (NS - 2) * (LDW + (AL >= 3 ? 3 : 1))>(); break;
      default: wait_vm<LDW + (NS - 2) * (LDW + AL)>(); break;
    }
  };
  auto wait_stage = [&]() {  // all but the NS - 2 most recent stages' loads done
    switch (n_a) {
      case 0: wait_vm<(NS - 2) * LDW>(); break;
      case 1: wait_vm<(NS - 2) * (LDW + 1)>(); break;
      case 2: wait_vm<(NS - 2) * (LDW + (AL >= 2 ? 2 : 1))>(); break;
      case 3: wait_vm<(NS - 2) * (LDW + (AL >= 3 ? 3 : 1))>(); break;
      default: wait_vm<(NS - 2) * (LDW + AL)>(); break;
    }
  };

  // the K loop and the epilogue for NA active chunks of this wavefront
  auto run = [&](auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    constexpr int NR = NA > 0 ? NA : 1;
    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    f32x16 R[NR][NW];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int t = 0; t < NW; ++t) R[i][t] = zero;
    float p2[NMAT];  // e4m3: the power of two of the current block's scale
    // the last chunk's rescale at a block's end waits for the next stage,
    // after that stage's first chunk's MFMAs (it then overlaps MFMAs instead
    // of ending the stage); its ratio is kept here
    constexpr bool DEFER = NA > 1 && !FP4;
    float pend[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) pend[m] = 1.0f;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) p2[m] = FP4 ? 1.0f : lane_of(pw[m], 0);

    // stage ks from LDS slot `slot`; NEWBLK (e4m3): the stage opens a 128-deep
    // scale block (its power of two goes into the conversions); otherwise it
    // closes one, and each chunk's accumulators are rescaled to the next
    // block's mantissa after the chunk's MFMAs (the block after the last has
    // ratio 1)
    auto compute = [&](int ks, int slot, auto newblk_c) {
      constexpr bool NEWBLK = decltype(newblk_c)::value;
      constexpr bool ENDBLK = !FP4 && !NEWBLK;
      if constexpr (NA > 0) {
        float ratio[NMAT];
        if constexpr (NEWBLK) {
          const int kb = ks >> 1;
#pragma unroll
          for (int m = 0; m < NMAT; ++m) p2[m] = lane_of(pw[m], kb);
        }
        if constexpr (ENDBLK) {
          const int kb = (ks >> 1) + 1;
#pragma unroll
          for (int m = 0; m < NMAT; ++m) ratio[m] = lane_of(rt[m], kb);
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
        for (int i = 0; i < NA; ++i) {
          const int mrow = 32 * (WGM * i + wm) + r32;
#pragma unroll
          for (int s = 0; s < NSTEP; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, a_s[mrow * C::ACH + ((NSTEP * h + s) ^ aswz(mrow))]);
#pragma unroll
            for (int t = 0; t < NW; ++t) R[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[t][s], R[i][t], 0, 0, 0);
          }
          if constexpr (NEWBLK && DEFER) {
            if (i == 0) {
#pragma unroll
              for (int t = 0; t < NW; ++t) {
                const float r = pend[GATEUP ? t : 0];
#pragma unroll
                for (int v = 0; v < 16; ++v) R[NA - 1][t][v] *= r;
              }
            }
          }
          if constexpr (ENDBLK) {
            if (!DEFER || i < NA - 1) {
#pragma unroll
              for (int t = 0; t < NW; ++t) {
                const float r = ratio[GATEUP ? t : 0];
#pragma unroll
                for (int v = 0; v < 16; ++v) R[i][t][v] *= r;
              }
            }
          }
        }
        if constexpr (ENDBLK && DEFER) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m) pend[m] = ratio[m];
        }
      }
    };

    for (int ks0 = 0; ks0 < nk; ks0 += UNR) {
      static_for<UNR>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        const int ks = ks0 + j;
        if (ks >= nk) return;
        if constexpr (EARLYW) {
          if (ks + NS - 1 < nk)
            wait_early();
          else
            wait_vm<0>();
          stage_barrier();
          if (ks + NS - 1 < nk) issue_act(ks + NS - 1, (j + NS - 1) % NS);
          compute(ks, j % NS, std::integral_constant<bool, !FP4 && j % 2 == 0>{});
          if (ks + NS < nk) {
            // this wavefront's reads of the slot have returned before the
            // slot's weight region is written again
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_wt(ks + NS, j % NS);
          }
          return;
        }
        if (ks + NS - 2 < nk)
          wait_stage();
        else
          wait_vm<0>();
        stage_barrier();
        if (ks + NS - 1 < nk) issue(ks + NS - 1, (j + NS - 1) % NS);
        compute(ks, j % NS, std::integral_constant<bool, !FP4 && j % 2 == 0>{});
      });
    }
    wait_vm<0>();

    // One wavefront row: the output leaves through LDS, each wavefront
    // turning its 32-row chunk into rows of 16-byte pieces (bf16 h: 64 bytes
    // of a row per wavefront; f32 y: 256), so the stores are 16 bytes per
    // lane instead of 2 or 4.  Row strides padded by 8 elements: the writes of
    // the lane halves (rows r and r + 4) fall in different banks.
    constexpr int NCW = 32 * TNW, RSW = NCW + 8;
    constexpr bool TEPI = WGM == 1 && 8 * 32 * RSW * (GATEUP ? 2 : 4) <= (int)sizeof(sW);
    if constexpr (TEPI) {
      __syncthreads();  // every wavefront's reads of the last stage are done
      if constexpr (GATEUP) {
        uint16_t* ep = reinterpret_cast<uint16_t*>(&sW[0][0]) + w * 32 * RSW;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
#pragma unroll
          for (int j = 0; j < TNW; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float g = R[i][j][v] * mlast[0], u = R[i][TNW + j][v] * mlast[NMAT - 1];
              ep[acc_row(v, lane) * RSW + 32 * j + r32] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
            }
#pragma unroll
          for (int q = 0; q < NCW / 16; ++q) {
            const int idx = lane + 64 * q, row = idx / (NCW / 8), seg = idx % (NCW / 8);
            const u32x4 val = *reinterpret_cast<const u32x4*>(ep + row * RSW + seg * 8);
            const int m = 32 * i + row, n = nw0 + seg * 8;
            if (m < rows && n < N)
              *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (size_t)(p_start + m) * N + n) = val;
          }
        }
      } else {
        float* ep = reinterpret_cast<float*>(&sW[0][0]) + w * 32 * RSW;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
#pragma unroll
          for (int j = 0; j < TNW; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) ep[acc_row(v, lane) * RSW + 32 * j + r32] = R[i][j][v] * mlast[0];
#pragma unroll
          for (int q = 0; q < NCW / 8; ++q) {
            const int idx = lane + 64 * q, row = idx / (NCW / 4), seg = idx % (NCW / 4);
            const f32x4 val = *reinterpret_cast<const f32x4*>(ep + row * RSW + seg * 4);
            const int m = 32 * i + row, n = nw0 + seg * 4;
            if (m < rows && n < N)
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)(p_start + m) * N + n) = val;
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
#pragma unroll
      for (int j = 0; j < TNW; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 32 * (WGM * i + wm) + acc_row(v, lane);
          const int n = nw0 + 32 * j + r32;
          if (m < rows && n < N) {
            if (GATEUP) {
              const float g = R[i][j][v] * mlast[0], u = R[i][TNW + j][v] * mlast[NMAT - 1];
              reinterpret_cast<uint16_t*>(out)[(size_t)(p_start + m) * N + n] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
            } else {
              reinterpret_cast<float*>(out)[(size_t)(p_start + m) * N + n] = R[i][j][v] * mlast[0];
            }
          }
        }
    }
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nk) issue(p, p);
  if constexpr (EARLYW)
    if (NS - 1 < nk) issue_wt(NS - 1, NS - 1);
  load_scales();
  dispatch_count<TM>(nact, run);
}

}  // namespace moe
