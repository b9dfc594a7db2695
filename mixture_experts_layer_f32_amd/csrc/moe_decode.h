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

// Weight formats: e4m3 + f32 scale per 128x128 block; e2m1 + UE8M0 scale per
// 32 inputs of a row; NVFP4 = e2m1 + e4m3 scale per 16 inputs of a row.
enum : int { FMT_E4M3 = 0, FMT_E2M1 = 1, FMT_NVFP4 = 2 };

// One expert matrix family on the device: byte pointers and expert strides,
// and the same matrix of the shared (always-on) expert if the layer has one
// (a work item whose flag is set reads those instead of expert e's).
struct DMat {
  const uint8_t* q;
  const uint8_t* s;
  int64_t qs;  // bytes per expert, codes
  int64_t ss;  // bytes per expert, scales
  const uint8_t* shq;  // shared expert: codes
  const uint8_t* shs;  // shared expert: scales
};
__device__ __forceinline__ const uint8_t* mat_q(const DMat& m, int e, bool sh) {
  return sh ? m.shq : m.q + e * m.qs;
}
__device__ __forceinline__ const uint8_t* mat_s(const DMat& m, int e, bool sh) {
  return sh ? m.shs : m.s + e * m.ss;
}

// A "chunk" is 16 consecutive inputs of one weight row: 16 bytes of e4m3
// codes or 8 bytes of e2m1 codes.  A chunk is decoded once into 8 exact bf16
// pairs (e4m3 values are bf16 values; an e2m1 value times its power-of-two
// UE8M0 scale or its e4m3 scale is a bf16 value) and dotted with each token's 16 bf16 activations by
// v_dot2_f32_bf16, whose products are exact in f32.
template <int FMT>
struct Chunk;

template <>
struct Chunk<FMT_E4M3> {
  typedef u32x4 raw;
  static constexpr bool kPostScale = true;  // scale applied to the chunk's partial sum
  static __device__ __forceinline__ raw load(const uint8_t* row, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
  }
  // scale of the 128x128 block holding row n, inputs [16c, 16c+16)
  static __device__ __forceinline__ float scale(const uint8_t* s, int n, int c, int K) {
    return reinterpret_cast<const float*>(s)[(n >> 7) * (K >> 7) + (c >> 3)];
  }
  static __device__ __forceinline__ void decode(raw w, float, bf16x2 (&o)[8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = e4m3x2_to_bf16<false>(ws[i]);
      o[2 * i + 1] = e4m3x2_to_bf16<true>(ws[i]);
    }
  }
};

template <>
struct Chunk<FMT_E2M1> {
  typedef u32x2 raw;
  static constexpr bool kPostScale = false;  // scale applied exactly inside the conversion
  static __device__ __forceinline__ raw load(const uint8_t* row, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row) + c);
  }
  // UE8M0 byte of the 32-input group holding inputs [16c, 16c+16) of row n
  static __device__ __forceinline__ float scale(const uint8_t* s, int n, int c, int K) {
    return ue8m0_to_f32(s[(size_t)n * (K >> 5) + (c >> 1)]);
  }
  static __device__ __forceinline__ void decode(raw w, float sc, bf16x2 (&o)[8]) {
    o[0] = e2m1x2_to_bf16<0>(w.x, sc);
    o[1] = e2m1x2_to_bf16<1>(w.x, sc);
    o[2] = e2m1x2_to_bf16<2>(w.x, sc);
    o[3] = e2m1x2_to_bf16<3>(w.x, sc);
    o[4] = e2m1x2_to_bf16<0>(w.y, sc);
    o[5] = e2m1x2_to_bf16<1>(w.y, sc);
    o[6] = e2m1x2_to_bf16<2>(w.y, sc);
    o[7] = e2m1x2_to_bf16<3>(w.y, sc);
  }
};

template <>
struct Chunk<FMT_NVFP4> {
  typedef u32x2 raw;
  static constexpr bool kPostScale = false;  // scale applied exactly in the decode
  static __device__ __forceinline__ raw load(const uint8_t* row, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row) + c);
  }
  // e4m3 scale byte of the 16-input group that is chunk c of row n
  static __device__ __forceinline__ float scale(const uint8_t* s, int n, int c, int K) {
    return e4m3_to_f32(s[(size_t)n * (K >> 4) + c]);
  }
  static __device__ __forceinline__ void decode(raw w, float sc, bf16x2 (&o)[8]) {
    o[0] = e2m1x2_times_to_bf16<0>(w.x, sc);
    o[1] = e2m1x2_times_to_bf16<1>(w.x, sc);
    o[2] = e2m1x2_times_to_bf16<2>(w.x, sc);
    o[3] = e2m1x2_times_to_bf16<3>(w.x, sc);
    o[4] = e2m1x2_times_to_bf16<0>(w.y, sc);
    o[5] = e2m1x2_times_to_bf16<1>(w.y, sc);
    o[6] = e2m1x2_times_to_bf16<2>(w.y, sc);
    o[7] = e2m1x2_times_to_bf16<3>(w.y, sc);
  }
};

template <int FMT>
__device__ __forceinline__ int64_t row_bytes(int K) {
  return FMT == FMT_E4M3 ? (int64_t)K : (int64_t)K / 2;
}

// 16 bf16 activations (inputs 16c .. 16c+15 of a row) as 8 packed pairs.
__device__ __forceinline__ void load_act16(const uint16_t* row, int c, uint32_t (&v)[8]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row + 16 * c);
  const u32x4 a = p[0], b = p[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// sum over 16 inputs of w * x, f32 (exact products, v_dot2_f32_bf16 chain)
__device__ __forceinline__ float dot16(const bf16x2 (&w)[8], const uint32_t (&x)[8]) {
  float p = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    p = __builtin_amdgcn_fdot2_f32_bf16(w[q], __builtin_bit_cast(bf16x2, x[q]), p, false);
  return p;
}

// Decode matvec over the experts that received at least one slot.
// grid.x: index into that list (entries past its length hold expert -1 and
// their blocks exit at once);
// grid.y: groups of 4*RPW weight rows (one wavefront per RPW rows).
// NM weight matrices share the rows (2: gate and up, 1: down).  Each lane
// takes chunks c = lane, lane+64, ... of every row; all of a pass's chunks
// are loaded before any is used.  Token slots are handled TG at a time;
// empty slots of the last group are skipped with a wave-uniform branch.
// The per-(row, slot) sums are reduced across the wavefront at the end.
template <int FMT, int NM, int TG, int RPW, int U, typename ActRow, typename Store>
__device__ __forceinline__ void dec_matvec(const uint8_t* const (&q)[NM],
                                           const uint8_t* const (&s)[NM], int n0, int K, int cnt,
                                           ActRow act_row, Store store) {
  const int lane = lane_id();
  const int nch = K / 16;
  const int64_t rb = row_bytes<FMT>(K);
  for (int t0 = 0; t0 < cnt; t0 += TG) {
    const int ntok = min(TG, cnt - t0);
    const uint16_t* ar[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) ar[t] = act_row(t0 + min(t, ntok - 1));
    float acc[NM][RPW][TG];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[m][r][t] = 0.0f;
    if constexpr (FMT != FMT_E4M3) {
      // fp4: a lane takes two adjacent chunks (32 inputs, 16 bytes of codes:
      // one e2m1 scale group, two NVFP4 groups) per step, so a step is one
      // 16-byte code load and one scale load per row instead of two of each
      const int npair = nch >> 1;
      for (int p0 = lane; p0 < npair; p0 += WAVE * U) {
        u32x4 w[U][NM][RPW];
        uint32_t sb[U][NM][RPW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pp = p0 + WAVE * u;
          if (pp < npair) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int r = 0; r < RPW; ++r) {
                w[u][m][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q[m] + r * rb) + pp);
                if constexpr (FMT == FMT_NVFP4)
                  sb[u][m][r] = reinterpret_cast<const uint16_t*>(s[m] + (size_t)(n0 + r) * (K >> 4))[pp];
                else
                  sb[u][m][r] = s[m][(size_t)(n0 + r) * (K >> 5) + pp];
              }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pp = p0 + WAVE * u;
          if (pp < npair) {
            uint32_t xv[TG][2][8];
#pragma unroll
            for (int t = 0; t < TG; ++t)
              if (t < ntok) {
                load_act16(ar[t], 2 * pp, xv[t][0]);
                load_act16(ar[t], 2 * pp + 1, xv[t][1]);
              }
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int r = 0; r < RPW; ++r) {
                float sc0, sc1;
                if constexpr (FMT == FMT_NVFP4) {
                  const f32x2 sv = __builtin_amdgcn_cvt_pk_f32_fp8(sb[u][m][r], false);
                  sc0 = sv.x;
                  sc1 = sv.y;
                } else {
                  sc0 = sc1 = ue8m0_to_f32(sb[u][m][r]);
                }
                bf16x2 wa[8], wb[8];
                Chunk<FMT>::decode(u32x2{w[u][m][r].x, w[u][m][r].y}, sc0, wa);
                Chunk<FMT>::decode(u32x2{w[u][m][r].z, w[u][m][r].w}, sc1, wb);
#pragma unroll
                for (int t = 0; t < TG; ++t)
                  if (t < ntok) acc[m][r][t] = (acc[m][r][t] + dot16(wa, xv[t][0])) + dot16(wb, xv[t][1]);
              }
          }
        }
      }
    } else
    for (int c0 = lane; c0 < nch; c0 += WAVE * U) {
      typename Chunk<FMT>::raw w[U][NM][RPW];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + WAVE * u;
        if (c < nch) {
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int r = 0; r < RPW; ++r) w[u][m][r] = Chunk<FMT>::load(q[m] + r * rb, c);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + WAVE * u;
        if (c < nch) {
          uint32_t xv[TG][8];
#pragma unroll
          for (int t = 0; t < TG; ++t)
            if (t < ntok) load_act16(ar[t], c, xv[t]);
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            // e4m3: the RPW rows (RPW divides 128, n0 a multiple of RPW) share one 128-row block
            const float sc0 = Chunk<FMT>::scale(s[m], n0, c, K);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
              const float sc = Chunk<FMT>::kPostScale ? sc0 : Chunk<FMT>::scale(s[m], n0 + r, c, K);
              bf16x2 wb[8];
              Chunk<FMT>::decode(w[u][m][r], sc, wb);
#pragma unroll
              for (int t = 0; t < TG; ++t)
                if (t < ntok) {
                  const float p = dot16(wb, xv[t]);
                  acc[m][r][t] = Chunk<FMT>::kPostScale ? fmaf(p, sc, acc[m][r][t])
                                                        : acc[m][r][t] + p;
                }
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t)
        if (t < ntok) {
          float v[NM];
#pragma unroll
          for (int m = 0; m < NM; ++m) v[m] = wave_sum(acc[m][r][t]);
          if (lane == r * TG + t) store(t0 + t, r, v);
        }
  }
}

// Gate/up + SwiGLU: for every slot of the expert (sorted position p),
// h[p][n] = bf16(silu(g[n]) * u[n]).  grid.x: slot_info entry; grid.y:
// blocks of (blockDim / 64) wavefronts x `rpw_total` rows.
template <int FMT, int TG, int RPW>
__global__ __launch_bounds__(1024) void dec_gateup(
    const uint16_t* __restrict__ x, DMat gate, DMat up, const int4* __restrict__ slot_info,
    const int32_t* __restrict__ tok_of, uint16_t* __restrict__ h, int d, int f, int T,
    int rpw_total) {
  const int4 info = slot_info[blockIdx.x];
  if (info.x < 0) return;
  const int e = info.x, p0 = info.y, cnt = info.z;
  const int n0 = (blockIdx.y * (blockDim.x / WAVE) + wave_id()) * rpw_total;
  if (n0 >= f) return;
  const int nrows = min(rpw_total, f - n0);
  const int64_t rb = row_bytes<FMT>(d);
  const bool sh = info.w != 0;
  const uint8_t* const q[2] = {mat_q(gate, e, sh) + n0 * rb, mat_q(up, e, sh) + n0 * rb};
  const uint8_t* const s[2] = {mat_s(gate, e, sh), mat_s(up, e, sh)};
  auto act_row = [&](int i) -> const uint16_t* {
    return x + (size_t)min((uint32_t)tok_of[p0 + i], (uint32_t)(T - 1)) * d;
  };
  auto store = [&](int i, int r, const float (&v)[2]) {
    h[(size_t)(p0 + i) * f + n0 + r] = (uint16_t)f32_to_bf16_rne(silu(v[0]) * v[1]);
  };
  for (int r0 = 0; r0 < nrows; r0 += RPW) {
    const uint8_t* const qq[2] = {q[0] + r0 * rb, q[1] + r0 * rb};
    auto st2 = [&](int i, int r, const float (&v)[2]) { store(i, r0 + r, v); };
    dec_matvec<FMT, 2, TG, RPW, 2>(qq, s, n0 + r0, d, cnt, act_row, st2);
  }
}

// Down projection: y[p][m] = sum_n h[p][n] Wd[m][n] (f32) for every sorted
// position p of the expert.
template <int FMT, int TG, int RPW>
__global__ __launch_bounds__(1024) void dec_down(
    const uint16_t* __restrict__ h, DMat down, const int4* __restrict__ slot_info,
    float* __restrict__ y, int d, int f, int rpw_total) {
  const int4 info = slot_info[blockIdx.x];
  if (info.x < 0) return;
  const int e = info.x, p0 = info.y, cnt = info.z;
  const int m0 = (blockIdx.y * (blockDim.x / WAVE) + wave_id()) * rpw_total;
  if (m0 >= d) return;
  const int nrows = min(rpw_total, d - m0);
  const int64_t rb = row_bytes<FMT>(f);
  const bool sh = info.w != 0;
  const uint8_t* const q[1] = {mat_q(down, e, sh) + m0 * rb};
  const uint8_t* const s[1] = {mat_s(down, e, sh)};
  auto act_row = [&](int i) -> const uint16_t* { return h + (size_t)(p0 + i) * f; };
  auto store = [&](int i, int r, const float (&v)[1]) { y[(size_t)(p0 + i) * d + m0 + r] = v[0]; };
  for (int r0 = 0; r0 < nrows; r0 += RPW) {
    const uint8_t* const qq[1] = {q[0] + r0 * rb};
    auto st1 = [&](int i, int r, const float (&v)[1]) { store(i, r0 + r, v); };
    dec_matvec<FMT, 1, TG, RPW, 2>(qq, s, m0 + r0, f, cnt, act_row, st1);
  }
}

// ---------------------------------------------------------------------------
// MFMA decode.  The expert stage for few tokens per expert as 16 x 16 output
// tiles on v_mfma_f32_16x16x32_bf16: A = 16 weight rows decoded exactly to
// bf16, B = up to 16 token columns (activation rows; columns past the
// expert's count read as zero), f32 accumulation.  The work list is the
// routing stage's tile list built with 16 rows per entry, so every entry
// holds at most 16 sorted positions of one expert.
//
// Lane l of a wavefront owns weight row n0 + (l & 15) and k-slot q = l >> 4.
// For e4m3 and a 128-input block starting at k0 it supplies, to MFMA a = 0..3,
// the 8 inputs k0 + 32q + 8a (two adjacent 16-byte loads per row and lane:
// each load then spans the row's whole 128-byte run, which streams faster
// than two half runs); for e2m1 and 256 inputs from k0, to MFMA 4h + a,
// the inputs k0 + 64q + 32h + 8a (two adjacent 16-byte loads); token
// column (l & 15) takes the activations of the same inputs, so every MFMA sums
// products of matching (row, input) and (input, token) pairs.  e4m3: the four
// MFMAs of a block start from zero and their sum is multiplied by the block's
// scale and added to the running f32 sum (one f32 accumulation per 128 x 128
// scale block); e2m1: the ue8m0 scale of the lane's 32-input group is applied
// exactly inside the conversion (nvfp4: the e4m3 scales of its two 16-input
// halves, in f32).
//
// e2m1/nvfp4 group scales: a unit needs 8 (nvfp4: 16) scale bytes per row,
// and a per-lane byte load for each would cost as much load issue as the
// weights themselves.  Instead, every fourth unit of a tile each lane loads
// the whole scale run of one of the next four units (lane q: unit j + q) with
// one wide load, the wavefront parks them in its own LDS rows, and each unit
// reads its lane's 2 (nvfp4: 4) bytes back with one LDS read per row group.
//
// Persistent grid: workgroup b takes tiles b, b + G, b + 2G, ... (so the tiles
// in flight at any time are neighbours in HBM); its KS wavefronts split each
// tile's 128-input blocks (wave w: blocks w, w + KS, ...) and sum their
// partial tiles through LDS in wave order.  Each wavefront streams its
// (tile, block) units with D units of loads in flight.  All loads are buffer
// loads: a unit past the end, an input past K or a token column past the
// count uses an out-of-range offset and reads zeros without a memory access.
constexpr uint32_t BUF_OOB = 0x80000000u;
// Offset o if ok, else o with the sign bit set: past the extent of every
// buffer these kernels read (each is under 2 GiB, which the host checks), so
// the load returns zeros.  An OR keeps the offset in one register and the
// load a single instruction; as a select of a computed offset the compiler
// may instead branch around two copies of the load, whose shared destination
// register then makes the wavefront wait for every load it has in flight.
// OOB_SEL takes the OR for NVFP4 (measured 3-8 % faster with it) and the
// plain select for e2m1 (measured 1-3 % faster with that) and e4m3 (equal).
__device__ __forceinline__ uint32_t oob_or(bool ok, uint32_t o) {
  const uint32_t m = ok ? 0u : BUF_OOB;
  uint32_t v;
  asm("v_or_b32 %0, %1, %2" : "=v"(v) : "v"(o), "v"(m));
  return v;
}
#define OOB_SEL(ok, o) (FMT == FMT_NVFP4 ? oob_or((ok), (o)) : (ok) ? (o) : BUF_OOB)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, int imm) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, imm, 0));
}
__device__ __forceinline__ bf16x8 pack_bf16x8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  const u32x4 v = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, v);
}
// 8 e4m3 codes (two words, low byte first) -> 8 bf16
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  return pack_bf16x8(e4m3x2_to_bf16<false>(lo), e4m3x2_to_bf16<true>(lo),
                     e4m3x2_to_bf16<false>(hi), e4m3x2_to_bf16<true>(hi));
}
// 8 e2m1 codes (one word, low nibble first) times their power-of-two scale -> 8 bf16
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w, float sc) {
  return pack_bf16x8(e2m1x2_to_bf16<0>(w, sc), e2m1x2_to_bf16<1>(w, sc),
                     e2m1x2_to_bf16<2>(w, sc), e2m1x2_to_bf16<3>(w, sc));
}
// 8 e2m1 codes (one word) times an e4m3 scale value -> 8 bf16, exact
__device__ __forceinline__ bf16x8 nvfp4x8_to_bf16(uint32_t w, float sc) {
  return pack_bf16x8(e2m1x2_times_to_bf16<0>(w, sc), e2m1x2_times_to_bf16<1>(w, sc),
                     e2m1x2_times_to_bf16<2>(w, sc), e2m1x2_times_to_bf16<3>(w, sc));
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One unit = one (tile, k-range) step of a wavefront: per matrix and 16-row
// group, two 16-byte weight loads per lane (e4m3: 128 inputs, one scale
// block; e2m1: 256 inputs, the lane's two 32-input groups at k0 + 64q and
// k0 + 64q + 32), and the activations of those inputs, shared by all of the
// unit's row groups and matrices.  e2m1/nvfp4: g holds, on units j = 0 mod 4
// of a tile, the scale run of unit j + q of the lane's row.
template <int FMT> struct DecUnitW;
template <> struct DecUnitW<FMT_E4M3> { u32x4 w[2]; };
template <> struct DecUnitW<FMT_E2M1> { u32x4 w[2]; u32x2 g; };
template <> struct DecUnitW<FMT_NVFP4> { u32x4 w[2]; u32x4 g; };
// Scale bytes per row and unit, and the LDS row stride that parks four units'
// runs (strides 40 and 80 put the 16 rows' reads of one unit in distinct banks).
template <int FMT> constexpr int dec_run_bytes() { return FMT == FMT_NVFP4 ? 16 : 8; }
template <int FMT> constexpr int dec_run_stride() { return FMT == FMT_NVFP4 ? 80 : 40; }

// The scale run of one unit of row n: bytes [off, off + SB) of the row's
// scales, of which `avail` lie inside the row (fewer than SB only on the last
// unit of a row whose K is not a multiple of 256).  Past the row's end a
// wide load reads the next row's scales, which only multiply the zeros that
// stand for the inputs past K (weights and activations there read as zero),
// so every row but the matrix's last (`has_next` false) takes the wide load;
// the last row's run would reach past the buffer, so it is assembled from
// byte loads, the bytes past the row reading zero.  (Byte loads for every
// ragged run made one wavefront per tile wait for all its loads in flight.)
// Wide loads need no alignment on gfx950 (unaligned buffer access).
template <int FMT>
__device__ __forceinline__ decltype(DecUnitW<FMT>::g) load_scale_run(__amdgpu_buffer_rsrc_t sr, bool in,
                                                                     uint32_t off, int avail, bool has_next) {
  constexpr int SB = dec_run_bytes<FMT>();
  if (avail >= SB || !in || has_next) {
    const uint32_t o = OOB_SEL(in, off);
    if constexpr (FMT == FMT_NVFP4)
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, o, 0, 0));
    else
      return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(sr, o, 0, 0));
  }
  uint32_t v[SB / 4];
#pragma unroll
  for (int i = 0; i < SB / 4; ++i) v[i] = 0;
#pragma unroll
  for (int i = 0; i < SB; ++i)
    v[i >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(sr, i < avail ? off + i : BUF_OOB, 0, 0) << (8 * (i & 3));
  if constexpr (FMT == FMT_NVFP4)
    return u32x4{v[0], v[1], v[2], v[3]};
  else
    return u32x2{v[0], v[1]};
}
template <int FMT> constexpr int dec_unit_k() { return FMT == FMT_E4M3 ? 128 : 256; }
template <int FMT> constexpr int dec_unit_x() { return FMT == FMT_E4M3 ? 4 : 8; }

// GATEUP: h[p][n] = bf16(silu(g) * u) for the f rows n of gate/up (K = d,
// activations x[tok_of[p]]); else y[p][m] (f32) for the d rows of down
// (K = f, activations h[p]).  A tile is RT groups of 16 rows; D units of
// loads in flight per wavefront.  act_bytes: extent of the activation buffer.
template <int FMT, bool GATEUP, int RT, int D>
__global__ __launch_bounds__(256) void dec_mfma(
    const uint16_t* __restrict__ act, uint32_t act_bytes, DMat A, DMat B,
    const int4* __restrict__ tiles, const int32_t* __restrict__ n_tiles_p,
    const int32_t* __restrict__ tok_of, void* __restrict__ outp, int N, int K, int T) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int KU = dec_unit_k<FMT>(), NX = dec_unit_x<FMT>();
  constexpr int TR = 16 * RT;  // rows per tile
  constexpr int RS = dec_run_stride<FMT>(), SB = dec_run_bytes<FMT>();
  __shared__ f32x4 red[2][3][NM * RT][WAVE];
  // per wavefront: NM * RT row groups x 16 rows x RS bytes of parked scale runs
  __shared__ __attribute__((aligned(16))) uint8_t runs[FMT == FMT_E4M3 ? 16 : 4 * NM * RT * 16 * RS];
  const int KS = blockDim.x / WAVE;
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int r = lane & 15, q = lane >> 4;
  const int tpe = (N + TR - 1) / TR;
  const int n_tiles = *n_tiles_p * tpe;
  const int G = gridDim.x, b = blockIdx.x;
  if (b >= n_tiles) return;
  const int my_tiles = (n_tiles - b + G - 1) / G;
  const int nkb = (K + KU - 1) / KU;
  const int nu = (nkb - w + KS - 1) / KS;  // units per tile for this wavefront (>= 1)
  const int units = my_tiles * nu;
  const uint32_t rb = FMT == FMT_E4M3 ? (uint32_t)K : (uint32_t)K / 2;
  const uint32_t sgroups = FMT == FMT_NVFP4 ? (uint32_t)(K >> 4) : (uint32_t)(K >> 5);
  const uint32_t q_bytes = (uint32_t)N * rb, s_bytes = (uint32_t)N * sgroups;
  const __amdgpu_buffer_rsrc_t ar = buf_rsrc(act, act_bytes);
  const DMat M[2] = {A, B};

  struct Unit {
    DecUnitW<FMT> wv[NM][RT];
    u32x4 x[NX];
    float sc[NM];
  };
  // e2m1/nvfp4: every pipeline step issues the same loads; a unit past the
  // end takes the last unit's addresses with out-of-range offsets (no memory
  // access), so the compiler's load counting sees one pattern on every path
  // and a unit waits only for its own loads, not for those issued after it
  // (measured 2-3% faster there).  e4m3 skips the issue past the end, so its
  // units also wait for the loads issued after them (the wavefront keeps one
  // unit of loads in flight): measured 2-6 % faster than the overlapped form
  // at 8-32 tokens on the OLMoE shape, and equal at 64 tokens on the d = 7168
  // layer; three units in flight and 16 wavefronts per CU measured equal or
  // slower too.
  constexpr bool ALWAYS = FMT != FMT_E4M3;
  // The issue side walks this wavefront's units in order: (i_jt, i_j) is the
  // position of the unit last issued (tile i_jt of the workgroup, unit i_j of
  // that tile), advanced by one per live issue, and the tile's entry and,
  // for gate/up, lane r's token row are looked up only when the tile changes
  // (no integer divisions or entry loads per unit).  A unit past the end
  // keeps the last unit's tile and addresses.
  int i_jt = 0, i_j = -1;
  int t_e = 0, t_p0 = 0, t_cnt = 1, t_n0 = 0;
  bool t_sh = false;
  uint32_t tile_row = 0;
  auto issue = [&](Unit& s, int u) {
    const bool live = u < units;
    if (live && ++i_j == nu) {
      i_j = 0;
      ++i_jt;
    }
    const int j = i_j;
    const int kb = w + KS * j;
    if (live && j == 0) {  // a new tile
      const int tile = b + i_jt * G;
      const int ti = tile / tpe;
      t_n0 = (tile - ti * tpe) * TR;
      const int4 info = tiles[ti];
      t_e = info.x;
      t_p0 = info.y;
      t_cnt = info.z;
      t_sh = info.w != 0;
      if (GATEUP) {
        // the entry's (<= 16) token ids by scalar loads, written to lanes
        // 0..15 of one register and spread to lane groups 1..3 by a permute
        const int32_t* tp = tok_of + t_p0;
        int tv[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) tv[jj] = tp[min(jj, t_cnt - 1)];
        int tk = 0;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) asm("v_writelane_b32 %0, %1, %2" : "+v"(tk) : "s"(tv[jj]), "i"(jj));
        tk = __builtin_amdgcn_ds_bpermute(r << 2, tk);
        tile_row = min((uint32_t)tk, (uint32_t)(T - 1));
      }
    }
    const int e = t_e, p0 = t_p0, cnt = t_cnt, n0 = t_n0;
    const bool sh = t_sh;
    const int k0 = kb * KU;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const __amdgpu_buffer_rsrc_t wr = buf_rsrc(mat_q(M[m], e, sh), q_bytes);
      if constexpr (FMT == FMT_E4M3) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int n = n0 + 16 * t + r;
          const uint32_t off = OOB_SEL(live && n < N, (uint32_t)n * rb + k0 + 32 * q);
          s.wv[m][t].w[0] = buf_load16(wr, off, 0);
          s.wv[m][t].w[1] = buf_load16(wr, off, 16);
        }
        s.sc[m] = reinterpret_cast<const float*>(mat_s(M[m], e, sh))[(n0 >> 7) * (K >> 7) + kb];
      } else {
        const __amdgpu_buffer_rsrc_t sr = buf_rsrc(mat_s(M[m], e, sh), s_bytes);
        const int run0 = SB * (w + KS * (j + q));  // lane's scale run: unit j + q
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int n = n0 + 16 * t + r;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bool in = live && n < N && k0 + 64 * q + 32 * h < K;
            s.wv[m][t].w[h] = buf_load16(wr, OOB_SEL(in, (uint32_t)n * rb + k0 / 2 + 32 * q + 16 * h), 0);
          }
          if ((j & 3) == 0)
            s.wv[m][t].g = load_scale_run<FMT>(sr, live && n < N && j + q < nu, (uint32_t)n * sgroups + run0,
                                                (int)sgroups - run0, n + 1 < N);
        }
        s.sc[m] = 0.0f;
      }
    }
    // activation row of token column r: gate/up the entry's token r (looked
    // up above), down h[p0 + r]
    const uint32_t row = GATEUP ? tile_row : (uint32_t)(p0 + min(r, cnt - 1));
    if constexpr (FMT == FMT_E4M3) {
      const uint32_t off = OOB_SEL(live && r < cnt, (row * K + k0 + 32 * q) * 2);
      s.x[0] = buf_load16(ar, off, 0);
      s.x[1] = buf_load16(ar, off, 16);
      s.x[2] = buf_load16(ar, off, 32);
      s.x[3] = buf_load16(ar, off, 48);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = k0 + 64 * q + 32 * h;
        const uint32_t off = OOB_SEL(live && r < cnt && k < K, (row * K + k) * 2);
#pragma unroll
        for (int a = 0; a < 4; ++a) s.x[4 * h + a] = buf_load16(ar, off, 16 * a);
      }
    }
  };
  f32x4 acc[NM][RT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Unit& s, int j) {  // j: the unit's place in its tile
    // e2m1/nvfp4: park the runs of units j..j+3 (on j = 0 mod 4; the wavefront's
    // own LDS rows, so program order orders the write before the reads), then
    // read this unit's bytes: e2m1 byte h = scale of chunk h; nvfp4 bytes
    // 2h, 2h + 1 = scales of chunk h's two halves
    uint32_t sv[NM][RT];
    if constexpr (FMT != FMT_E4M3) {
      uint8_t* const base = runs + w * (NM * RT * 16 * RS);
      if ((j & 3) == 0) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int t = 0; t < RT; ++t)
            *reinterpret_cast<decltype(DecUnitW<FMT>::g)*>(base + ((m * RT + t) * 16 + r) * RS + SB * q) = s.wv[m][t].g;
      }
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const uint8_t* pr = base + ((m * RT + t) * 16 + r) * RS + SB * (j & 3) + (SB / 4) * q;
          sv[m][t] = FMT == FMT_NVFP4 ? *reinterpret_cast<const uint32_t*>(pr) : *reinterpret_cast<const uint16_t*>(pr);
        }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const DecUnitW<FMT>& wq = s.wv[m][t];
        if constexpr (FMT == FMT_E4M3) {
          f32x4 part = mfma16x16x32(e4m3x8_to_bf16(wq.w[0].x, wq.w[0].y),
                                    __builtin_bit_cast(bf16x8, s.x[0]), f32x4{0.f, 0.f, 0.f, 0.f});
          part = mfma16x16x32(e4m3x8_to_bf16(wq.w[0].z, wq.w[0].w), __builtin_bit_cast(bf16x8, s.x[1]), part);
          part = mfma16x16x32(e4m3x8_to_bf16(wq.w[1].x, wq.w[1].y), __builtin_bit_cast(bf16x8, s.x[2]), part);
          part = mfma16x16x32(e4m3x8_to_bf16(wq.w[1].z, wq.w[1].w), __builtin_bit_cast(bf16x8, s.x[3]), part);
          const float sc = s.sc[m];
          acc[m][t] = f32x4{fmaf(part.x, sc, acc[m][t].x), fmaf(part.y, sc, acc[m][t].y),
                            fmaf(part.z, sc, acc[m][t].z), fmaf(part.w, sc, acc[m][t].w)};
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 v = wq.w[h];
            bf16x8 a0, a1, a2, a3;
            if constexpr (FMT == FMT_NVFP4) {  // words x, y: first 16-input group; z, w: second
              const f32x2 s01 = h ? __builtin_amdgcn_cvt_pk_f32_fp8(sv[m][t], true) : __builtin_amdgcn_cvt_pk_f32_fp8(sv[m][t], false);
              a0 = nvfp4x8_to_bf16(v.x, s01.x);
              a1 = nvfp4x8_to_bf16(v.y, s01.x);
              a2 = nvfp4x8_to_bf16(v.z, s01.y);
              a3 = nvfp4x8_to_bf16(v.w, s01.y);
            } else {
              const float sc = ue8m0_to_f32((sv[m][t] >> (8 * h)) & 0xFFu);
              a0 = e2m1x8_to_bf16(v.x, sc);
              a1 = e2m1x8_to_bf16(v.y, sc);
              a2 = e2m1x8_to_bf16(v.z, sc);
              a3 = e2m1x8_to_bf16(v.w, sc);
            }
            acc[m][t] = mfma16x16x32(a0, __builtin_bit_cast(bf16x8, s.x[4 * h + 0]), acc[m][t]);
            acc[m][t] = mfma16x16x32(a1, __builtin_bit_cast(bf16x8, s.x[4 * h + 1]), acc[m][t]);
            acc[m][t] = mfma16x16x32(a2, __builtin_bit_cast(bf16x8, s.x[4 * h + 2]), acc[m][t]);
            acc[m][t] = mfma16x16x32(a3, __builtin_bit_cast(bf16x8, s.x[4 * h + 3]), acc[m][t]);
          }
        }
      }
  };
  // Tile done: partial tiles of waves 1..KS-1 through LDS (double-buffered by
  // tile parity, so one barrier per tile), summed by wave 0 in wave order.
  // D[i][j] of lane l: rows 4q + i (i = 0..3) of a 16-row group, token column l & 15.
  auto finish = [&](int jt) {
    const int par = jt & 1;
    if (w > 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t) red[par][w - 1][m * RT + t][lane] = acc[m][t];
    }
    __syncthreads();
    if (w == 0) {
      for (int v = 0; v < KS - 1; ++v)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            const f32x4 o = red[par][v][m * RT + t][lane];
            acc[m][t] = f32x4{acc[m][t].x + o.x, acc[m][t].y + o.y, acc[m][t].z + o.z, acc[m][t].w + o.w};
          }
      const int tile = b + jt * G;
      const int ti = tile / tpe, n0 = (tile - ti * tpe) * TR;
      const int4 info = tiles[ti];
      if (r < info.z) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int n = n0 + 16 * t + 4 * q;
          if (n < N) {
            const size_t o = (size_t)(info.y + r) * N + n;
            if (GATEUP) {
              const f32x4 g = acc[0][t], u = acc[NM - 1][t];
              const uint32_t h0 = f32_to_bf16_rne(silu(g.x) * u.x), h1 = f32_to_bf16_rne(silu(g.y) * u.y);
              const uint32_t h2 = f32_to_bf16_rne(silu(g.z) * u.z), h3 = f32_to_bf16_rne(silu(g.w) * u.w);
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(outp) + o) = u32x2{h0 | (h1 << 16), h2 | (h3 << 16)};
            } else {
              *reinterpret_cast<f32x4*>(static_cast<float*>(outp) + o) = acc[0][t];
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // Software pipeline over the unit stream (D - 1 units of loads ahead);
  // the compute side keeps its own (tile, unit) position like the issue side.
  Unit st[D];
#pragma unroll
  for (int s = 0; s < D - 1; ++s)
    if (ALWAYS || s < units) issue(st[s], s);
  int c_jt = 0, c_j = -1;
  for (int u0 = 0; u0 < units; u0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (ALWAYS || u0 + s + D - 1 < units) issue(st[(s + D - 1) % D], u0 + s + D - 1);
      if (u0 + s < units) {
        if (++c_j == nu) {
          c_j = 0;
          ++c_jt;
        }
        compute(st[s], c_j);
        if (c_j == nu - 1) finish(c_jt);
      }
    }
  }
}

#undef OOB_SEL

// Fixed-order combine: out[t] = sum over j ascending of w[t,j] * y[inv_perm[t*k+j]]
// in f32, a gather in router order, so every output has one fixed summation
// order (WARP BACKENDS.md, "Coherent memory": partials reduced in router
// order); then + the shared expert's row y_sh[t] (if y_sh), stored to out (if
// out), and out_bf16[t] = bf16(residual[t] + out[t]) (if residual), the add
// into the residual stream (dragon.c page, summary: the MoE output added to
// the stream at the end of a sub-block).  Each
// thread takes 4 columns of one token.  KM = k (the plan's top-k, 1..16) as a
// compile-time count: all k row indices and weights are loaded first
// (uniform: scalar loads), then all k rows, then summed in j order, so a
// thread waits two memory round trips, not 2k.
template <int KM>
__global__ __launch_bounds__(256) void combine_fixed_order(const float* __restrict__ y,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ inv_perm,
                                                           const float* __restrict__ y_sh,
                                                           const uint16_t* __restrict__ residual,
                                                           float* __restrict__ out,
                                                           uint16_t* __restrict__ out_bf16, int d,
                                                           int ncb) {
  // workgroup = (token, 1024-column block), the column blocks of a token
  // adjacent in launch order, so its k rows are read whole and together
  const int t = blockIdx.x / ncb;
  const int m = ((blockIdx.x - t * ncb) * 256 + threadIdx.x) * 4;
  if (m >= d) return;
  int idx[KM];
  float wv[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    idx[j] = inv_perm[(size_t)t * KM + j];
    wv[j] = w[(size_t)t * KM + j];
  }
  f32x4 v[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (size_t)idx[j] * d + m));
  f32x4 sv = {0.f, 0.f, 0.f, 0.f};
  u32x2 rv = {0u, 0u};
  if (y_sh) sv = *reinterpret_cast<const f32x4*>(y_sh + (size_t)t * d + m);
  if (residual) rv = *reinterpret_cast<const u32x2*>(residual + (size_t)t * d + m);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    acc.x += wv[j] * v[j].x;
    acc.y += wv[j] * v[j].y;
    acc.z += wv[j] * v[j].z;
    acc.w += wv[j] * v[j].w;
  }
  if (y_sh) acc = f32x4{acc.x + sv.x, acc.y + sv.y, acc.z + sv.z, acc.w + sv.w};
  if (out) __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + (size_t)t * d + m));
  if (residual) {
    const uint32_t o0 = f32_to_bf16_rne(bf16_lo(rv.x) + acc.x), o1 = f32_to_bf16_rne(bf16_hi(rv.x) + acc.y);
    const uint32_t o2 = f32_to_bf16_rne(bf16_lo(rv.y) + acc.z), o3 = f32_to_bf16_rne(bf16_hi(rv.y) + acc.w);
    *reinterpret_cast<u32x2*>(out_bf16 + (size_t)t * d + m) = u32x2{o0 | (o1 << 16), o2 | (o3 << 16)};
  }
}

}  // namespace moe
