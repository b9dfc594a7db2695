// The activation-quantised variant of the expert stage (opt-in per plan).
// The expert inputs, the token rows x before gate/up and h before down, are
// cut into groups of 128 consecutive inputs; each group gets a power-of-two
// scale (a UE8M0 byte) and e4m3 codes (dev.to DeepSeek-V4.1-Flash post,
// "Three bugs on RTX 50xx that never raise an error", item 2: the model's
// activation quantiser writes fp8 with UE8M0 scales).  The GEMMs then run on
// gfx950's block-scaled fp8/fp4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4),
// whose per-32-input scale operands take the activation scale and the
// weight's power-of-two scale part, so the weight codes enter the MFMA
// undecoded.
#pragma once

#include "moe_gemm.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Quantiser: bf16 rows x [R][K] -> e4m3 codes q [R][K] and UE8M0 bytes
// s [R][ng], ng = ceil(K / 128); K % 8 == 0.  A group's scale is the
// smallest 2^E (E >= -127) with max |x| <= 448 * 2^E: for max |x| = fr * 2^ex
// (fr in [0.5, 1)) that is E = ex - 9, plus one when fr > 0.875 (448 is
// 0.875 * 2^9); an all-zero group gets byte 127.  A code is the e4m3 value
// nearest x * 2^-E (exact product; ties to the even mantissa), the sign bit
// taken from x.  16 lanes per group, 8 inputs per lane, 16 groups per
// workgroup.
// DEQ: write the quantised values themselves as bf16 (code * 2^E is a bf16
// value: at most 5 significant bits), in place allowed, for the decode
// kernels, which take bf16 activations; the same values as the codes give.
template <bool DEQ>
__device__ __forceinline__ void act_quant_rows(const uint16_t* x, uint8_t* q, uint8_t* s, uint16_t* y,
                                               int R, int K, int ng) {
  const long long gid = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool live = gid < (long long)R * ng;
  const int row = live ? (int)(gid / ng) : 0;
  const int g = live ? (int)(gid - (long long)row * ng) : 0;
  const int k = 128 * g + 8 * j;
  const bool in = live && k < K;
  const u32x4 v = in ? *reinterpret_cast<const u32x4*>(x + (size_t)row * K + k) : u32x4{0u, 0u, 0u, 0u};
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i]));
  // the 16 lanes of a group are an aligned 16-lane block of the wavefront
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 16));
  const uint32_t ab = __float_as_uint(am);
  const int fe = (int)(ab >> 23);  // biased exponent (am >= 0)
  int E;
  if (am == 0.0f)
    E = 0;
  else if (fe == 0)
    E = -127;
  else
    E = max((fe - 126) - 9 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0), -127);
  const float mul = __uint_as_float((uint32_t)(127 - E) << 23);  // 2^-E, E in [-127, 120]
  uint32_t code[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(f[i] * mul);  // below 2^-126 it rounds to a zero code either way
    const int ee = max((int)(__float_as_uint(a) >> 23) - 127, -6);
    // a / 2^(ee - 3): an integer 0..16 after rounding; codes are contiguous
    // across binade edges and from the subnormals into the normals
    const float r = __builtin_rintf(a * __uint_as_float((uint32_t)(130 - ee) << 23));
    if constexpr (DEQ)  // the value r 2^(ee - 3) 2^E, the sign of x
      code[i] = f32_to_bf16_rne(copysignf(ldexpf(r, ee - 3 + E), f[i]));
    else
      code[i] = ((__float_as_uint(f[i]) >> 31) << 7) | (uint32_t)(8 * (ee + 6) + (int)r);
  }
  if (in) {
    if constexpr (DEQ) {
      *reinterpret_cast<u32x4*>(y + (size_t)row * K + k) =
          u32x4{code[0] | code[1] << 16, code[2] | code[3] << 16, code[4] | code[5] << 16, code[6] | code[7] << 16};
    } else {
      *reinterpret_cast<u32x2*>(q + (size_t)row * K + k) =
          u32x2{code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
                code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24};
      if (j == 0) s[(size_t)row * ng + g] = (uint8_t)(E + 127);
    }
  }
}

__global__ __launch_bounds__(256) void act_quant_e4m3(const uint16_t* __restrict__ x,
                                                      uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s, int R, int K,
                                                      int ng) {
  act_quant_rows<false>(x, q, s, nullptr, R, K, ng);
}

// The quantised values as bf16 rows (x and y may be the same buffer).
__global__ __launch_bounds__(256) void act_qdq_bf16(const uint16_t* x, uint16_t* y, int R, int K, int ng) {
  act_quant_rows<true>(x, nullptr, nullptr, y, R, K, ng);
}

// ---------------------------------------------------------------------------
// Grouped GEMM on quantised activations.  8 wavefronts in a 2 x 4 grid:
// wavefront (wm, wn) owns TM 32-token chunks of the tile (tokens
// 32 TM wm ..) and two 32-row weight tiles of column wn (gate/up: gate and up
// rows 32 wn ..; down: rows 64 wn and 64 wn + 32).  A workgroup covers
// BM = 64 TM tokens x 128 rows of each matrix (down: 256 rows); 128-input
// stages (one activation scale group, one e4m3 weight block column; e2m1 on
// 64-token tiles: 256-input stages, two groups) move by direct-to-LDS loads
// into NS slots, NS - 1 stages in flight.
//
// Operands of v_mfma_scale_f32_32x32x64_f8f6f4 (checked on the device):
//   fp8 A/B: lane (r, h) holds row r's inputs 16 h .. 16 h + 15 in its first
//   four registers and 32 + 16 h .. 32 + 16 h + 15 in the next four;
//   fp4 B: lane (r, h) holds inputs 32 h .. 32 h + 31 in four registers, the
//   lower nibble first;
//   the scale of row r for inputs 32 b .. 32 b + 31 comes from lane r + 32 b
//   (its byte 0).
//   The instruction rounds its 64-product sum at about 2^-14 of the sum's
//   magnitude (fp8 x fp8; fp8 x fp4 came out exact) and adds C at f32
//   precision (measured).
// e4m3 weights: each stage's two MFMAs start from zero, with the power of two
// of the stage's block scale as their B scale, and the partial joins the f32
// running sum with one FMA by the scale's mantissa (R += m * P).  e2m1: the
// group scales are the MFMA's B scales as they are, so the MFMAs accumulate
// into R directly.
//
// LDS rows: a 128-byte row (activations, e4m3 weights, fp4 weights of a
// 256-input stage) holds its 16-byte chunk c at slot c ^ ((row >> 1) & 7), a
// 256-byte activation row at c ^ (row & 15), a 64-byte fp4 row at
// c ^ ((row >> 2) & 3), so each 16-lane pass of a fragment read touches 16
// bank groups.
template <int FMT, bool GATEUP, int TM_>
struct Q8Cfg {
  static constexpr bool FP4 = FMT != FMT_E4M3;
  static constexpr int TM = TM_, BM = 64 * TM;
  // fp4 on 64-token tiles: 256-input stages, so each weight row is read 128
  // contiguous bytes at a time (64 with 128-input stages); otherwise 128
  static constexpr int BK = FP4 && TM == 1 ? 256 : 128;
  static constexpr int NU = BK / 64;                // MFMAs per token chunk and weight tile per stage
  static constexpr int TNW = GATEUP ? 1 : 2;
  static constexpr int BNM = 4 * 32 * TNW;          // weight rows per matrix per workgroup
  static constexpr int ACH = BK / 16;               // 16-byte activation chunks per row and stage
  static constexpr int A_V4 = BM * ACH;             // u32x4 of activation codes per stage
  static constexpr int AL = (A_V4 + 511) / 512;     // activation code loads per lane and stage
  static constexpr int AS = (BM + 63) / 64;         // activation scale loads (wavefronts 0 .. AS-1)
  static constexpr int AG = BK / 128;               // activation scale groups per stage
  static constexpr int WROW = FP4 ? BK / 2 : 128;   // weight bytes per row and stage
  static constexpr int WCH = WROW / 16;             // 16-byte weight chunks per row and stage
  static constexpr int W_V4 = 8 * 32 * WROW / 16;   // 8 tiles of 32 rows
  static constexpr int WL = 32 * WROW / 1024;       // weight loads per lane, tile and stage
  static constexpr int SG = FP4 ? BK / 128 : 0;     // fp4 scale loads per lane, tile and stage
  static constexpr int S_DW = 8 * 64 * SG;          // fp4 scale dwords per stage
  static constexpr int SA_B = 16 * A_V4 + 4 * AG * BM;  // LDS bytes of a stage's activations
  static constexpr int SW_B = 16 * W_V4 + 4 * S_DW; // ... and of its weights
  static constexpr int NS = 160 * 1024 / (SA_B + SW_B) > 4 ? 4 : 160 * 1024 / (SA_B + SW_B);
  static_assert(NS >= 2, "one stage in flight at least");
  // Where a common ring has only 2 slots but 2 activation slots and 3 weight
  // slots fit, the weights (from HBM) get a stage more lead than the
  // activations (mostly L2 hits: an entry's rows serve all its column blocks)
  static constexpr bool SPLIT = NS == 2 && 2 * SA_B + 3 * SW_B <= 160 * 1024;
  static constexpr int NSA = SPLIT ? 2 : NS, NSW = SPLIT ? 3 : NS;
};

template <int FMT, bool GATEUP, int TM_>
__global__ __launch_bounds__(512, 1) void gemm_q8(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, DMat W0, DMat W1,
    const int4* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const int32_t* __restrict__ tok_of, void* __restrict__ out, int N, int K, int T, int nb) {
  using C = Q8Cfg<FMT, GATEUP, TM_>;
  constexpr bool FP4 = C::FP4;
  constexpr int TM = C::TM, BM = C::BM, BK = C::BK, NS = C::NS, AL = C::AL, WL = C::WL;
  constexpr int TNW = C::TNW, NSA = C::NSA, NSW = C::NSW, ACH = C::ACH, WCH = C::WCH, NU = C::NU;
  constexpr int AG = C::AG, SG = C::SG;
  __shared__ u32x4 sA[NSA][C::A_V4];
  __shared__ u32x4 sW[NSW][C::W_V4];
  __shared__ uint32_t sAs[NSA][AG * BM];
  __shared__ uint32_t sWs[NSW][C::S_DW > 0 ? C::S_DW : 1];
  // block order as in gemm_big: XCD x takes tile-list entries x, x + 8, ...
  const int L = blockIdx.x, xcd = L & 7, sq = L >> 3;
  const int lt = sq / nb, cblk = sq - lt * nb;
  const int ti = 8 * lt + xcd;
  if (ti >= *n_tiles) return;
  const int4 tile = tiles[ti];
  const int e = tile.x, p_start = tile.y, rows = tile.z;
  const bool sh = tile.w != 0;  // the shared expert's rows
  const int n0 = cblk * C::BNM;
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int wm = w >> 2, wn = w & 3;
  const int r32 = lane & 31, h = lane >> 5;
  const int nw0 = n0 + 32 * TNW * wn;
  const int nact = min(max(((rows + 31) >> 5) - TM * wm, 0), TM);
  const int ng = (K + 127) >> 7;  // activation scale groups per row

  // activation rows of this lane's code loads: rows (AL w + i) * (64 / ACH) +
  // lane / ACH (mod BM; rows past the tile repeat its last row and are not
  // stored); a 128-byte row holds chunk c at slot c ^ ((row >> 1) & 7), a
  // 256-byte row at c ^ (row & 15)
  auto aswz = [](int r) { return ACH == 8 ? ((r >> 1) & 7) : (r & 15); };
  auto wswz = [](int r) { return WCH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  const uint8_t* asrc[AL];
  int achunk[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int r = ((AL * w + i) * (64 / ACH) + lane / ACH) % BM;
    const int rr = min(r, rows - 1);
    const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + rr], (uint32_t)(T - 1))
                              : (size_t)(p_start + rr);
    asrc[i] = aq + src * K;
    achunk[i] = (lane % ACH) ^ aswz(r);
  }
  // activation scale of tile row 64 w + lane (wavefronts 0 .. AS-1)
  const bool sload = w < C::AS;
  const uint8_t* ssrc;
  {
    const int r = min(64 * w + lane, BM - 1);
    const int rr = min(r, rows - 1);
    const size_t src = GATEUP ? (size_t)min((uint32_t)tok_of[p_start + rr], (uint32_t)(T - 1))
                              : (size_t)(p_start + rr);
    ssrc = as + src * ng;
  }
  // this wavefront loads weight tile wm of its column: tile t = wm is matrix
  // t (gate/up) or rows 32 t .. of the column (down)
  const int ml = GATEUP ? wm : 0, jl = GATEUP ? 0 : wm;
  const DMat& WT = ml == 0 ? W0 : W1;
  const int64_t rbytes = FP4 ? (int64_t)K / 2 : (int64_t)K;
  const int sgroups = K >> 5;
  const uint8_t* wsrc[WL];
  int wchunk[WL];
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int tr = (64 / WCH) * j + lane / WCH;
    wsrc[j] = mat_q(WT, e, sh) + (int64_t)min(nw0 + 32 * jl + tr, N - 1) * rbytes;
    wchunk[j] = (lane % WCH) ^ wswz(tr);
  }
  // fp4 scales: load c of lane (r, half) brings the bytes (BK / 32) kk + 4 c +
  // 2 half .. + 1 of row r
  const uint8_t* wssrc = FP4 ? mat_s(WT, e, sh) + (int64_t)min(nw0 + 32 * jl + r32, N - 1) * sgroups
                             : nullptr;
  // e4m3 block scales of this column's 128-row block: block kb in lane kb % 64
  // of register kb / 64
  float scv[GATEUP ? 2 : 1][2];
  if constexpr (!FP4) {
    const int kbs = K >> 7;
#pragma unroll
    for (int m = 0; m < (GATEUP ? 2 : 1); ++m) {
      const DMat& W = m == 0 ? W0 : W1;
      const float* sf = reinterpret_cast<const float*>(mat_s(W, e, sh)) + (size_t)(min(nw0, N - 1) >> 7) * kbs;
      scv[m][0] = lane < kbs ? sf[lane] : 1.0f;
      scv[m][1] = lane + 64 < kbs ? sf[lane + 64] : 1.0f;
    }
  }

  const int nk = (K + BK - 1) / BK;
  const int tslot = wn * 2 + wm;  // LDS tile this wavefront loads
  // a stage's activation loads (codes, then scales), then its weight loads;
  // the pipelines below rely on this order
  auto issue_a = [&](int kk, int slot) {
    const int k0 = kk * BK;
#pragma unroll
    for (int i = 0; i < AL; ++i)
      lds_dma16(asrc[i] + min(k0 + 16 * achunk[i], K - 16), &sA[slot][((AL * w + i) * 64) % C::A_V4]);
    if (sload)
#pragma unroll
      for (int g = 0; g < AG; ++g) lds_dma_u8(ssrc + min(AG * kk + g, ng - 1), &sAs[slot][g * BM + (64 * w) % BM]);
  };
  auto issue_w = [&](int kk, int slot) {
    const int k0 = kk * BK;
#pragma unroll
    for (int j = 0; j < WL; ++j)
      lds_dma16(wsrc[j] + min((int64_t)(FP4 ? k0 / 2 : k0) + 16 * wchunk[j], rbytes - 16),
                &sW[slot][(tslot * WL + j) * 64]);
    if constexpr (FP4)
#pragma unroll
      for (int c = 0; c < SG; ++c)
        lds_dma_u16(wssrc + min((BK / 32) * kk + 4 * c + 2 * h, sgroups - 2), &sWs[slot][(tslot * SG + c) * 64]);
  };
  auto issue = [&](int kk, int slot) {
    issue_a(kk, slot);
    issue_w(kk, slot);
  };

  const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x16 R[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i) R[i][0] = R[i][1] = zero;

  auto compute = [&](int ks, int slot, int wslot) {
    const int k0 = ks * BK;
    // e4m3: this stage's block scale per weight tile, split into the power of
    // two (the MFMA's B scale byte: the f32 exponent field) and the mantissa
    int sb[2];
    float mt[2];
    if constexpr (!FP4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m = GATEUP ? t : 0;
        const float sc = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(ks < 64 ? scv[m][0] : scv[m][1]), ks & 63));
        sb[t] = (int)((__float_as_uint(sc) >> 23) & 0xFF);
        mt[t] = mant_part(sc);
      }
    }
    // weight operands of both 64-input halves u, decoded never: the codes are
    // the MFMA's B operand as they are
    i32x8 b[NU][2];
    int sbl[NU][2];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int T2 = wn * 2 + t;  // LDS tile
        if constexpr (!FP4) {
          const u32x4* row = &sW[wslot][T2 * 256 + r32 * 8];
          const u32x4 lo = row[(4 * u + h) ^ ((r32 >> 1) & 7)];
          const u32x4 hi = row[(4 * u + 2 + h) ^ ((r32 >> 1) & 7)];
          b[u][t] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sbl[u][t] = sb[t];
        } else {
          const u32x4 v = sW[wslot][T2 * 32 * WCH + r32 * WCH + ((2 * u + h) ^ wswz(r32))];
          b[u][t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sbl[u][t] = (int)((sWs[wslot][(T2 * SG + (u >> 1)) * 64 + r32 + 32 * (u & 1)] >> (8 * h)) & 0xFF);
        }
      }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= nact) break;  // uniform
      const int mrow = 32 * TM * wm + 32 * i + r32;
      const u32x4* arow = &sA[slot][mrow * ACH];
      i32x8 a[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c0 = 4 * u + h, c1 = 4 * u + 2 + h;
        u32x4 lo = arow[c0 ^ aswz(mrow)];
        u32x4 hi = arow[c1 ^ aswz(mrow)];
        // inputs past K (an fp4 layer's last, shorter group) contribute zero
        if (k0 + 16 * c0 >= K) lo = u32x4{0u, 0u, 0u, 0u};
        if (k0 + 16 * c1 >= K) hi = u32x4{0u, 0u, 0u, 0u};
        a[u] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      const int sa = (int)(sAs[slot][mrow] & 0xFF);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (!FP4) {
          f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0], b[0][t], zero, 0, 0, 0, sa, 0, sbl[0][t]);
          P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1], b[1][t], P, 0, 0, 0, sa, 0, sbl[1][t]);
#pragma unroll
          for (int v = 0; v < 16; ++v) R[i][t][v] = fmaf(mt[t], P[v], R[i][t][v]);
        } else {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            // the activation scale of the 128-input group holding these 64 inputs
            const int sau = u < 2 ? sa : (int)(sAs[slot][BM + mrow] & 0xFF);
            R[i][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u], b[u][t], R[i][t], 0, 4, 0, sau, 0,
                                                                      sbl[u][t]);
          }
        }
      }
    }
  };

  // loads per lane and stage of this wavefront
  constexpr int LW0 = AL + WL + SG;
  auto wait_after = [&](int n) {  // all but the loads of the n most recent stages done
    if (sload) {
      switch (n) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<LW0 + AG>(); break;
        default: wait_vm<2 * (LW0 + AG)>(); break;
      }
    } else {
      switch (n) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<LW0>(); break;
        default: wait_vm<2 * LW0>(); break;
      }
    }
  };
  static_assert(NS - 2 <= 2, "wait_after covers up to two later stages");
  if constexpr (C::SPLIT) {
    // activations of stage ks + 1 and weights of stage ks + 2 are issued at
    // stage ks (in that order), so at stage ks only the weights issued last
    // (stage ks + 1's) may still be in flight
    constexpr int LWW = WL + SG;
    issue_a(0, 0);
    issue_w(0, 0);
    if (nk > 1) issue_w(1, 1);
    for (int ks0 = 0; ks0 < nk; ks0 += 6) {
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int ks = ks0 + j;
        if (ks >= nk) break;
        if (ks + 1 < nk)
          wait_vm<LWW>();
        else
          wait_vm<0>();
        stage_barrier();
        if (ks + 1 < nk) issue_a(ks + 1, (j + 1) % 2);
        if (ks + 2 < nk) issue_w(ks + 2, (j + 2) % 3);
        compute(ks, j % 2, j % 3);
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
      if (p < nk) issue(p, p);
    for (int ks0 = 0; ks0 < nk; ks0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int ks = ks0 + j;
        if (ks >= nk) break;
        wait_after(min(NS - 2, nk - 1 - ks));
        stage_barrier();
        if (ks + NS - 1 < nk) issue(ks + NS - 1, (j + NS - 1) % NS);
        compute(ks, j, j);
      }
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
            const float g = R[i][0][v], u = R[i][1][v];
            reinterpret_cast<uint16_t*>(out)[(size_t)(p_start + m) * N + n] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
          } else {
            reinterpret_cast<float*>(out)[(size_t)(p_start + m) * N + n] = R[i][j][v];
          }
        }
      }
  }
}

}  // namespace moe
