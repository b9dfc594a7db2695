// C ABI of the gfx950 MoE FFN layer: plan, validation, workspace layout and
// the launch sequence.  All device work is enqueued on the caller's stream;
// the host never waits on the device here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_common.h"
#include "moe_block.h"
#include "moe_decode.h"
#include "moe_gemm.h"
#include "moe_route.h"
#include "moe_q8.h"

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

constexpr int GEMV_MAX_T = 16;   // router: wavefront GEMV up to this many tokens, MFMA above

struct Layout {
  size_t logits, w3, ids, w, counts, offsets, perm, inv_perm, tok_of, rank, hist, base, slot_info, n_active,
      tiles, n_tiles, h, y, xq, hq, qx, sx, qh, sh, total;
  int nchunk, max_tiles, n_slots;
};

}  // namespace

// Scratch of moe_forward_noalloc: one array per device that runs the library,
// held until the process ends and shared by every such call on that device.
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, taken once per device (with
// that device current) when the first plan is made there.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES] = {};
bool scratch_tried[MAX_DEVICES] = {};

// Records the device address of `scratch` for device `dev` (the current
// device); a failed lookup leaves it NULL, and the no-alloc entry point then
// reports MOE_ERR_HIP.
void scratch_setup(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_tried[dev]) return;
  scratch_tried[dev] = true;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess)
    scratch_dev[dev] = ptr;
  else
    (void)hipGetLastError();
}

void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  return scratch_dev[dev];
}

}  // namespace

struct moe_plan_s {
  moe_desc d;
  int device = -1;
  int cus = 0;
  std::string arch;
  int t_decode = 0;  // AUTO: decode variant for T <= t_decode
  // kernel choices a fresh plan makes from the shape; moe_plan_set overrides them
  int dec_kernel = 1;     // decode expert stage: 1 = MFMA tiles, 0 = wavefront matvec
  int dec_mfma_min_t = 2; // MFMA tiles from this many tokens (matvec below)
  int small_route_t = 0;  // top-k + permute in one workgroup up to this many tokens (<= 64), 0 = by shape
  int big_cfg = 0;        // gemm_big tile shape 10 * WGM + TM (13, 14, 15, 22, 23, 24), 0 = by shape
  int q8_tm = 0;          // gemm_q8 token chunks per wavefront (tile 64 * tm tokens), 0 = by shape
  std::string info;
  std::string last_error;
  // instrumentation (moe_timing_*)
  uint32_t timing_mask = 0;
  int timing_max = 0;
  int timing_n = 0;
  std::vector<hipEvent_t> timing_ev;  // [forward][stage][begin, end]
  std::vector<uint32_t> timing_done;  // [forward]: bit s = stage s recorded
};

namespace {

int path_for(const moe_plan_s* p, int T) {
  if (p->d.path == MOE_PATH_DECODE) return MOE_PATH_DECODE;
  if (p->d.path == MOE_PATH_GROUPED) return MOE_PATH_GROUPED;
  return T <= p->t_decode ? MOE_PATH_DECODE : MOE_PATH_GROUPED;
}

// router: 256 x 128 MFMA tiles where they alone make 32 blocks (the 64 x 64
// tiles re-read the weight planes from L2 4x as often; with fewer tiles the
// larger ones leave the chip underfilled: measured on the d = 7168 layer at
// 4096 tokens 98 -> 67 us, and slower on the 2048-token OLMoE shape and the
// 1024-token FP4 layer)
bool router_big(const moe_plan_s* p, int T) {
  return (long long)((T + 255) / 256) * ((p->d.n_experts + 127) / 128) >= 32;
}

// Router K-split: enough blocks to cover the chip, slices of >= 256 inputs
// (multiples of 32).  Returns the number of slices; *slice gets their width.
int router_split(const moe_plan_s* p, int T, int* slice) {
  const int d = p->d.d_model, E = p->d.n_experts;
  const int blocks = T <= GEMV_MAX_T    ? (E + 3) / 4
                     : router_big(p, T)  ? ((T + 255) / 256) * ((E + 127) / 128)
                                         : ((T + 63) / 64) * ((E + 63) / 64);
  const int target = T <= GEMV_MAX_T ? 2 * p->cus : router_big(p, T) ? p->cus : 4 * p->cus;
  // few tokens: at most 4 slices, so the top-k sums its slice partials in
  // one round of loads (measured 0.3-1.5 % per step against 6-8 slices)
  const int cap = T <= GEMV_MAX_T ? 4 : MAX_SPLIT;
  int n = std::max(1, std::min(std::min(d / 256, cap), (target + blocks - 1) / blocks));
  int w = (d + n - 1) / n;
  w = (w + 31) / 32 * 32;
  n = (d + w - 1) / w;
  if (slice) *slice = w;
  return n;
}

// The MFMA decode addresses activations with 32-bit buffer offsets.
bool dec_mfma_fits(const moe_plan_s* p, int T) {
  const long long lim = 1LL << 31;
  return (long long)T * p->d.d_model * 2 < lim &&
         (long long)T * (p->d.top_k + (p->d.shared_expert ? 1 : 0)) * p->d.d_ff * 2 < lim;
}

// MFMA tiles for the decode expert stage from dec_mfma_min_t tokens; for a
// single token the wavefront matvec is faster (measured, both formats): each
// expert then has one slot, 15 of the MFMA's 16 token columns are empty, and
// the matvec's single batch of loads per wavefront has the shorter latency
// chain.
bool use_dec_mfma(const moe_plan_s* p, int T) {
  if (path_for(p, T) != MOE_PATH_DECODE || p->dec_kernel != 1 || !dec_mfma_fits(p, T)) return false;
  return T >= p->dec_mfma_min_t;
}

// Wavefronts splitting a decode tile's nkb k-units: all of them up to 4,
// else 4, 3 or 2, whichever divides nkb (a wavefront with fewer units than
// its neighbours waits for them at every tile's reduction), else 4.
int dec_ks(int nkb) {
  if (nkb <= 4) return nkb;
  for (int ks = 4; ks >= 2; --ks)
    if (nkb % ks == 0) return ks;
  return 4;
}

// Shape of gemm_big's tiles, as 10 * WGM + TM (tile height 32 * WGM * TM),
// from the mean slots per expert, as measured on every grouped workload:
// 128-token tiles of two wavefront rows up to 32 slots per expert (the fp4
// layer at 16 and 1024 tokens), 192-token tiles up to 96 (the skewed OLMoE
// shape at 512 tokens, whose hot experts hold about 150), and for e4m3 the
// 160-token tiles of one wavefront row up to 160 (the d = 7168 layer at 4096
// tokens, 128 per expert: every wavefront decodes only its own weight rows
// and the activations are shared by 256 rather than 128 weight rows per
// matrix, and each refills its own weight rows before the stage barrier;
// 2.06 against 2.26 ms for the gate/up stage), else 128-token tiles of one
// row (the skewed OLMoE shape at 2048, 256 per expert: 176 against 189 us
// for 256-token tiles of two rows).  fp4 keeps two rows (its 128-input stages
// need them): 192-token tiles up to 160, else 256.
int big_cfg(const moe_plan_s* p, int T) {
  if (p->big_cfg > 0) return p->big_cfg;
  const long long S = (long long)T * p->d.top_k;
  const long long mean = S / std::max(1LL, std::min<long long>(p->d.n_experts, S));
  if (mean <= 32) return 22;
  if (p->d.wfmt == MOE_W_E4M3_B128) return mean <= 96 ? 23 : (mean <= 160 ? 15 : 14);
  return mean <= 160 ? 23 : 24;
}
int big_rows(int cfg) { return 32 * (cfg / 10) * (cfg % 10); }

// gemm_q8 tile height 64 * tm tokens (tm 1..3; 4 would spill registers), from
// the mean slots per expert, as measured on the grouped workloads: 64-token
// tiles up to 32 (the fp4 layer at 1024 tokens, 16 per expert), 192 up to
// 160 (the skewed OLMoE shape at 512 tokens, whose hot experts hold about
// 150, and the d = 7168 layer at 4096, 128 per expert), 128 above (the
// skewed OLMoE shape at 2048: 256 per expert in two full tiles)
int q8_tm(const moe_plan_s* p, int T) {
  if (p->q8_tm > 0) return p->q8_tm;
  const long long S = (long long)T * p->d.top_k;
  const long long mean = S / std::max(1LL, std::min<long long>(p->d.n_experts, S));
  return mean <= 32 ? 1 : (mean <= 160 ? 3 : 2);
}

// Rows per entry of the routing stage's tile list: 16-slot entries for the
// MFMA decode, else the grouped-GEMM tile height.
int tile_rows(const moe_plan_s* p, int T) {
  if (p->d.act_fmt == MOE_ACT_E4M3_G128 && path_for(p, T) == MOE_PATH_GROUPED) return 64 * q8_tm(p, T);
  if (use_dec_mfma(p, T)) return 16;
  if (path_for(p, T) == MOE_PATH_GROUPED) return big_rows(big_cfg(p, T));
  return 16;  // the matvec reads slot_info, not the tile list
}

// The sorted positions of a forward: T * k routed slots, then (a layer with a
// shared expert) T more for the shared expert's rows.
size_t positions(const moe_plan_s* p, int T) {
  return (size_t)T * p->d.top_k + (p->d.shared_expert ? (size_t)T : 0);
}

Layout layout(const moe_plan_s* p, int T) {
  const size_t E = p->d.n_experts, k = p->d.top_k, d = p->d.d_model, f = p->d.d_ff;
  const size_t S = (size_t)T * k, SP = positions(p, T);
  const size_t BM = tile_rows(p, T);
  const size_t sh = p->d.shared_expert ? 1 : 0;
  Layout L;
  L.nchunk = (T + WAVE - 1) / WAVE;
  L.max_tiles = (int)((S + BM - 1) / BM + std::min<size_t>(E, S) + sh * ((T + BM - 1) / BM));
  L.n_slots = (int)(std::min<size_t>(E, S) + sh);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.logits = take((size_t)router_split(p, T, nullptr) * T * E * 4);
  L.w3 = take(router_big(p, T) ? 3 * E * d * 2 : 0);  // the router weights as three bf16 planes
  L.ids = take(S * 4);
  L.w = take(S * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(S * 4);
  L.inv_perm = take(S * 4);
  L.tok_of = take(SP * 4);
  L.rank = take(S * 4);
  L.hist = take((size_t)L.nchunk * E * 4);
  L.base = take((size_t)L.nchunk * E * 4);
  L.slot_info = take((size_t)L.n_slots * 16);
  L.n_active = take(4);
  L.tiles = take((size_t)L.max_tiles * 16);
  L.n_tiles = take(4);
  L.h = take(SP * f * 2);
  L.y = take(SP * d * 4);
  const bool q8 = p->d.act_fmt == MOE_ACT_E4M3_G128;
  L.xq = take(q8 ? (size_t)T * d * 2 : 0);  // decode path: the quantised x as bf16
  L.hq = take(q8 ? SP * f * 2 : 0);          // ... and the quantised h
  L.qx = take(q8 ? (size_t)T * d : 0);
  L.sx = take(q8 ? (size_t)T * ((d + 127) / 128) : 0);
  L.qh = take(q8 ? SP * f : 0);
  L.sh = take(q8 ? SP * ((f + 127) / 128) : 0);
  L.total = o;
  return L;
}

// Records the begin (end = false) or end event of `stage` for the current
// forward when timing is on for that stage.
void mark(moe_plan_s* p, int stage, bool end, hipStream_t s) {
  if (!(p->timing_mask >> stage & 1u) || p->timing_n >= p->timing_max) return;
  (void)hipEventRecord(p->timing_ev[((size_t)p->timing_n * MOE_N_STAGES + stage) * 2 + end], s);
  if (end) p->timing_done[p->timing_n] |= 1u << stage;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_fail(moe_plan_s* p, hipError_t err, const char* what) {
  p->last_error = std::string(what) + ": " + hipGetErrorString(err);
  return MOE_ERR_HIP;
}

// Decode matvec (the wavefront matvec of dec_gateup / dec_down): one
// workgroup of 4 wavefronts per (selected expert, 8 rows), each wavefront 2
// rows; up to 4 slots of the expert per pass (1 for a single token).
template <int FMT, bool GATEUP>
void launch_dec(int T, int n_slots, int N, int K, const uint16_t* x, const uint16_t* hin, DMat A,
                DMat B, const int4* info, const int32_t* tok_of, uint16_t* hout, float* y,
                hipStream_t st) {
  constexpr int RPW = 2, WPB = 4;
  const dim3 g(n_slots, (N + WPB * RPW - 1) / (WPB * RPW));
  if (T == 1) {
    if (GATEUP)
      dec_gateup<FMT, 1, RPW><<<g, WAVE * WPB, 0, st>>>(x, A, B, info, tok_of, hout, K, N, T, RPW);
    else
      dec_down<FMT, 1, RPW><<<g, WAVE * WPB, 0, st>>>(hin, A, info, y, N, K, RPW);
  } else {
    if (GATEUP)
      dec_gateup<FMT, 4, RPW><<<g, WAVE * WPB, 0, st>>>(x, A, B, info, tok_of, hout, K, N, T, RPW);
    else
      dec_down<FMT, 4, RPW><<<g, WAVE * WPB, 0, st>>>(hin, A, info, y, N, K, RPW);
  }
}

// Grouped GEMM launch: a 1-D grid of (tile-list entry, column block) pairs
// in the XCD order gemm_big decodes.
template <int FMT, bool GATEUP, int TNW, int TM, int WGM>
void launch_big_cfg(int max_tiles, int N, int K, int T, const uint16_t* act, DMat W0, DMat W1,
                    const int4* tiles, const int32_t* n_tiles, const int32_t* tok_of, void* out,
                    hipStream_t st) {
  constexpr int BNM = BigCfg<FMT, GATEUP, TNW, TM, WGM>::BNM;
  const int nb = (N + BNM - 1) / BNM;
  const dim3 g((unsigned)(8LL * ((max_tiles + 7) / 8) * nb));
  gemm_big<FMT, GATEUP, TNW, TM, WGM><<<g, 512, 0, st>>>(act, W0, W1, tiles, n_tiles, tok_of, out, N, K, T, nb,
                                                      max_tiles);
}

template <int FMT, bool GATEUP, int TNW>
void launch_big(const moe_plan_s* p, int max_tiles, int N, int K, int T, const uint16_t* act,
                DMat W0, DMat W1, const int4* tiles, const int32_t* n_tiles, const int32_t* tok_of,
                void* out, hipStream_t st) {
#define MOE_BIG(TM, WGM) \
  launch_big_cfg<FMT, GATEUP, TNW, TM, WGM>(max_tiles, N, K, T, act, W0, W1, tiles, n_tiles, tok_of, out, st)
  switch (big_cfg(p, T)) {
    case 13: MOE_BIG(3, 1); break;
    case 14: MOE_BIG(4, 1); break;
    case 15: MOE_BIG(5, 1); break;
    case 22: MOE_BIG(2, 2); break;
    case 23: MOE_BIG(3, 2); break;
    default: MOE_BIG(4, 2); break;
  }
#undef MOE_BIG
}

// y_dst: where the down projection writes y (NULL: the workspace).
void launch_act_qdq(const uint16_t* x, uint16_t* y, long long R, int K, hipStream_t st) {
  const int ng = (K + 127) / 128;
  act_qdq_bf16<<<(unsigned)((R * ng + 15) / 16), 256, 0, st>>>(x, y, (int)R, K, ng);
}

// qdq (activation-quantised plans on the decode path): the gate/up kernels
// read x's quantised values as bf16 and the down kernels h's (act_qdq_bf16
// into workspace copies, launched inside the stages' timing events); h
// itself stays the bf16 gate/up output.
template <int FMT>
moe_status launch_expert_stage(moe_plan_s* p, int T, const uint16_t* x_in, DMat G, DMat U, DMat D,
                               const Layout& L, char* ws, float* y_dst, hipStream_t st, bool qdq = false) {
  const int d = p->d.d_model, f = p->d.d_ff;
  const long long S_all = (long long)positions(p, T);
  uint16_t* xq = reinterpret_cast<uint16_t*>(ws + L.xq);
  const uint16_t* x = qdq ? xq : x_in;
  uint16_t* hq = reinterpret_cast<uint16_t*>(ws + L.hq);
  const int4* info = reinterpret_cast<const int4*>(ws + L.slot_info);
  const int32_t* tok_of = reinterpret_cast<const int32_t*>(ws + L.tok_of);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  const uint16_t* hd = qdq ? hq : h;  // what the down projection reads
  float* y = y_dst ? y_dst : reinterpret_cast<float*>(ws + L.y);
  if (use_dec_mfma(p, T)) {
    const int4* tiles = reinterpret_cast<const int4*>(ws + L.tiles);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(ws + L.n_tiles);
    const long long S = (long long)T * p->d.top_k;
    const uint32_t x_bytes = (uint32_t)((size_t)T * d * 2);
    const uint32_t h_bytes = (uint32_t)((size_t)S_all * f * 2);
    // Tile height: 16-row groups per tile (more rows share one activation
    // operand), taken larger only while the tile list stays several times the
    // persistent grid (upper bound of the list: one entry per expert hit plus
    // one per further 16 slots).
    const long long entries = std::min<long long>(p->d.n_experts, S) + (T > 16 ? S / 16 : 0);
    auto big = [&](int N, int rows) { return entries * ((N + rows - 1) / rows) >= 4LL * 3 * p->cus; };
    auto run = [&](bool gateup) {
      const int K = gateup ? d : f;
      const int ku = FMT == FMT_E4M3 ? 128 : 256;
      const int ks = dec_ks((K + ku - 1) / ku);
      const dim3 blk(WAVE * ks);
      // about 12 (tall: 8) wavefronts per CU whatever the split
      const int g3 = p->cus * 12 / ks, g2 = p->cus * 8 / ks;
      // e2m1: an input byte holds two weights, so the activation operand
      // outweighs the weights once the tiles' token columns fill; taller tiles
      // then share it over more rows (measured: faster at 8 slots per expert,
      // slower at 4)
      const bool tall = big(gateup ? f : d, gateup ? 32 : 64) &&
                        (FMT == FMT_E4M3 || S >= 8LL * p->d.n_experts);
      if (gateup) {
        if (tall)
          dec_mfma<FMT, true, 2, FMT == FMT_E4M3 ? 3 : 2><<<g2, blk, 0, st>>>(x, x_bytes, G, U, tiles, n_tiles, tok_of, h, f, d, T);
        else
          dec_mfma<FMT, true, 1, 2><<<g3, blk, 0, st>>>(x, x_bytes, G, U, tiles, n_tiles, tok_of, h, f, d, T);
      } else {
        if (tall)
          dec_mfma<FMT, false, 4, 2><<<g2, blk, 0, st>>>(hd, h_bytes, D, D, tiles, n_tiles, tok_of, y, d, f, T);
        else
          dec_mfma<FMT, false, 2, 2><<<g3, blk, 0, st>>>(hd, h_bytes, D, D, tiles, n_tiles, tok_of, y, d, f, T);
      }
    };
    mark(p, MOE_STAGE_GATEUP, false, st);
    if (qdq) launch_act_qdq(x_in, xq, T, d, st);
    run(true);
    mark(p, MOE_STAGE_GATEUP, true, st);
    mark(p, MOE_STAGE_DOWN, false, st);
    if (qdq) launch_act_qdq(h, hq, S_all, f, st);
    run(false);
    mark(p, MOE_STAGE_DOWN, true, st);
  } else if (path_for(p, T) == MOE_PATH_DECODE) {
    mark(p, MOE_STAGE_GATEUP, false, st);
    if (qdq) launch_act_qdq(x_in, xq, T, d, st);
    launch_dec<FMT, true>(T, L.n_slots, f, d, x, nullptr, G, U, info, tok_of, h, nullptr, st);
    mark(p, MOE_STAGE_GATEUP, true, st);
    mark(p, MOE_STAGE_DOWN, false, st);
    if (qdq) launch_act_qdq(h, hq, S_all, f, st);
    launch_dec<FMT, false>(T, L.n_slots, d, f, nullptr, hd, D, D, info, tok_of, nullptr, y, st);
    mark(p, MOE_STAGE_DOWN, true, st);
  } else {
    const int4* tiles = reinterpret_cast<const int4*>(ws + L.tiles);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(ws + L.n_tiles);
    mark(p, MOE_STAGE_GATEUP, false, st);
    launch_big<FMT, true, 1>(p, L.max_tiles, f, d, T, x, G, U, tiles, n_tiles, tok_of, h, st);
    mark(p, MOE_STAGE_GATEUP, true, st);
    mark(p, MOE_STAGE_DOWN, false, st);
    launch_big<FMT, false, 2>(p, L.max_tiles, d, f, T, h, D, D, tiles, n_tiles, tok_of, y, st);
    mark(p, MOE_STAGE_DOWN, true, st);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(p, err, "expert stage launch");
  return MOE_OK;
}

template <int FMT, bool GATEUP, int TM>
void launch_q8_cfg(int max_tiles, int N, int K, int T, const uint8_t* aq, const uint8_t* as,
                   DMat W0, DMat W1, const int4* tiles, const int32_t* n_tiles,
                   const int32_t* tok_of, void* out, hipStream_t st) {
  constexpr int BNM = Q8Cfg<FMT, GATEUP, TM>::BNM;
  const int nb = (N + BNM - 1) / BNM;
  const dim3 g((unsigned)(8LL * ((max_tiles + 7) / 8) * nb));
  gemm_q8<FMT, GATEUP, TM><<<g, 512, 0, st>>>(aq, as, W0, W1, tiles, n_tiles, tok_of, out, N, K, T, nb);
}

template <int FMT, bool GATEUP>
void launch_q8(const moe_plan_s* p, int max_tiles, int N, int K, int T, const uint8_t* aq,
               const uint8_t* as, DMat W0, DMat W1, const int4* tiles, const int32_t* n_tiles,
               const int32_t* tok_of, void* out, hipStream_t st) {
  switch (q8_tm(p, T)) {
    case 1: launch_q8_cfg<FMT, GATEUP, 1>(max_tiles, N, K, T, aq, as, W0, W1, tiles, n_tiles, tok_of, out, st); break;
    case 2: launch_q8_cfg<FMT, GATEUP, 2>(max_tiles, N, K, T, aq, as, W0, W1, tiles, n_tiles, tok_of, out, st); break;
    default: launch_q8_cfg<FMT, GATEUP, 3>(max_tiles, N, K, T, aq, as, W0, W1, tiles, n_tiles, tok_of, out, st); break;
  }
}

void launch_act_quant(const uint16_t* x, uint8_t* q, uint8_t* sc, long long R, int K, hipStream_t st) {
  const int ng = (K + 127) / 128;
  act_quant_e4m3<<<(unsigned)((R * ng + 15) / 16), 256, 0, st>>>(x, q, sc, (int)R, K, ng);
}

// The activation-quantised expert stage: x quantised, gate/up + SwiGLU on
// the block-scaled MFMA -> h (bf16), h quantised, down -> y.
template <int FMT>
moe_status launch_q8_stage(moe_plan_s* p, int T, const uint16_t* x, DMat G, DMat U, DMat D,
                           const Layout& L, char* ws, float* y_dst, hipStream_t st) {
  const int d = p->d.d_model, f = p->d.d_ff;
  const long long S = (long long)positions(p, T);
  const int4* tiles = reinterpret_cast<const int4*>(ws + L.tiles);
  const int32_t* n_tiles = reinterpret_cast<const int32_t*>(ws + L.n_tiles);
  const int32_t* tok_of = reinterpret_cast<const int32_t*>(ws + L.tok_of);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  float* y = y_dst ? y_dst : reinterpret_cast<float*>(ws + L.y);
  uint8_t* qx = reinterpret_cast<uint8_t*>(ws + L.qx);
  uint8_t* sx = reinterpret_cast<uint8_t*>(ws + L.sx);
  uint8_t* qh = reinterpret_cast<uint8_t*>(ws + L.qh);
  uint8_t* sh = reinterpret_cast<uint8_t*>(ws + L.sh);
  mark(p, MOE_STAGE_GATEUP, false, st);
  launch_act_quant(x, qx, sx, T, d, st);
  launch_q8<FMT, true>(p, L.max_tiles, f, d, T, qx, sx, G, U, tiles, n_tiles, tok_of, h, st);
  mark(p, MOE_STAGE_GATEUP, true, st);
  mark(p, MOE_STAGE_DOWN, false, st);
  launch_act_quant(h, qh, sh, S, f, st);
  launch_q8<FMT, false>(p, L.max_tiles, d, f, T, qh, sh, D, D, tiles, n_tiles, tok_of, y, st);
  mark(p, MOE_STAGE_DOWN, true, st);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(p, err, "expert stage launch");
  return MOE_OK;
}

moe_status check_mat(const moe_plan_s* p, const moe_mat* m) {
  if (m == nullptr || m->q == nullptr || m->scale == nullptr) return MOE_ERR_NULL_ARG;
  if (m->q_expert_stride < 0 || m->s_expert_stride < 0) return MOE_ERR_BAD_SHAPE;
  if (!aligned(m->q, 16) || m->q_expert_stride % 16) return MOE_ERR_ALIGNMENT;
  if (p->d.wfmt == MOE_W_E4M3_B128 && (!aligned(m->scale, 4) || m->s_expert_stride % 4))
    return MOE_ERR_ALIGNMENT;
  if (p->d.wfmt == MOE_W_E2M1_E4M3_G16 && (!aligned(m->scale, 2) || m->s_expert_stride % 2))
    return MOE_ERR_ALIGNMENT;
  // the activation-quantised e2m1 GEMM reads a row's group scales two at a time
  if (p->d.act_fmt == MOE_ACT_E4M3_G128 && p->d.wfmt == MOE_W_E2M1_UE8M0_G32 &&
      (!aligned(m->scale, 2) || m->s_expert_stride % 2))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL_ARG: return "MOE_ERR_NULL_ARG";
    case MOE_ERR_BAD_SHAPE: return "MOE_ERR_BAD_SHAPE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_ALIGNMENT: return "MOE_ERR_ALIGNMENT";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_plan(const moe_desc* desc, moe_plan_t* out) {
  if (desc == nullptr || out == nullptr) return MOE_ERR_NULL_ARG;
  *out = nullptr;
  const moe_desc& d = *desc;
  if (d.d_model <= 0 || d.d_ff <= 0 || d.n_experts <= 0 || d.top_k <= 0 || d.max_tokens <= 0)
    return MOE_ERR_BAD_SHAPE;
  if (d.top_k > d.n_experts) return MOE_ERR_BAD_SHAPE;
  if (d.renorm != 0 && d.renorm != 1) return MOE_ERR_BAD_SHAPE;
  if (d.path < MOE_PATH_AUTO || d.path > MOE_PATH_GROUPED) return MOE_ERR_BAD_SHAPE;
  if (d.act_fmt != MOE_ACT_BF16 && d.act_fmt != MOE_ACT_E4M3_G128) return MOE_ERR_BAD_SHAPE;
  if (d.shared_expert != 0 && d.shared_expert != 1) return MOE_ERR_BAD_SHAPE;
  if (d.shared_expert && d.n_experts == 1 && d.top_k == 1) return MOE_ERR_UNSUPPORTED;
  if (d.act_fmt == MOE_ACT_E4M3_G128) {
    if (d.wfmt == MOE_W_E2M1_E4M3_G16) return MOE_ERR_UNSUPPORTED;
    if (d.wfmt == MOE_W_E2M1_UE8M0_G32 && (d.d_model % 64 || d.d_ff % 64)) return MOE_ERR_UNSUPPORTED;
  }
  if (d.n_experts > MAX_E || d.top_k > MAX_K) return MOE_ERR_UNSUPPORTED;
  if (d.wfmt == MOE_W_E4M3_B128) {
    if (d.d_model % 128 || d.d_ff % 128) return MOE_ERR_UNSUPPORTED;
    if (d.d_model > 128 * MAX_KBLK || d.d_ff > 128 * MAX_KBLK) return MOE_ERR_UNSUPPORTED;
  } else if (d.wfmt == MOE_W_E2M1_UE8M0_G32 || d.wfmt == MOE_W_E2M1_E4M3_G16) {
    if (d.d_model % 32 || d.d_ff % 32) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  // int32 sorted positions and 32-bit grid sizes; the grouped kernels address
  // activation rows (x, h) with 32-bit byte offsets
  if ((int64_t)d.max_tokens * d.top_k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d.max_tokens * (d.top_k + 1) * std::max(d.d_model, d.d_ff) * 2 >= (int64_t)1 << 32)
    return MOE_ERR_UNSUPPORTED;

  int dev = -1, ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;

  scratch_setup(dev);
  moe_plan_s* p = new (std::nothrow) moe_plan_s();
  if (p == nullptr) return MOE_ERR_HIP;
  p->d = d;
  p->device = dev;
  p->cus = prop.multiProcessorCount;
  p->arch = prop.gcnArchName;
  // Decode (every selected expert's weights streamed once per 16 of its slots)
  // while the slots per expert stay small; measured crossovers against the
  // grouped GEMM (gemm_big): T*k about 10*E for e4m3 (OLMoE shape: decode
  // ahead at T = 64, grouped at 96; the d = 7168 layer: decode at 256,
  // grouped at 384), 14*E for fp4 (the e2m1 and NVFP4 layers: decode ahead at
  // 768 by 6 and 4 %, grouped at 1024 by 12 and 14 %).
  p->t_decode = std::max(1, (d.wfmt == MOE_W_E4M3_B128 ? 10 : 14) * d.n_experts / d.top_k);
  char buf[512];
  std::snprintf(buf, sizeof buf,
                "device %d %s (%d CUs); d=%d f=%d E=%d k=%d fmt=%s renorm=%d; path=%s "
                "(decode for T<=%d); router: wavefront gemv up to %d tokens, else 64x64 bf16x3 MFMA tiles, split-K; "
                "decode: MFMA 16-row tiles from %d tokens, matvec below; grouped: 128/192/256-token "
                "tiles by slots per expert, direct-to-LDS, MFMA 32x32x16 bf16",
                dev, p->arch.c_str(), p->cus, d.d_model, d.d_ff, d.n_experts, d.top_k,
                d.wfmt == MOE_W_E4M3_B128 ? "e4m3/128x128"
                : d.wfmt == MOE_W_E2M1_UE8M0_G32 ? "e2m1/ue8m0x32" : "e2m1/e4m3x16", d.renorm,
                d.path == MOE_PATH_AUTO ? "auto" : (d.path == MOE_PATH_DECODE ? "decode" : "grouped"),
                p->t_decode, GEMV_MAX_T, p->dec_mfma_min_t);
  p->info = buf;
  if (d.act_fmt == MOE_ACT_E4M3_G128)
    p->info += "; activations: e4m3 per 128-input group (UE8M0 scales); grouped path: "
               "block-scaled MFMA 32x32x64 (fp8 x fp8 / fp8 x fp4); decode path: the decode "
               "kernels on the quantised values as bf16";
  *out = p;
  return MOE_OK;
}

moe_status moe_plan_set(moe_plan_t p, int32_t option, int32_t value) {
  if (p == nullptr) return MOE_ERR_NULL_ARG;
  switch (option) {
    case MOE_OPT_DEC_KERNEL:
      if (value != 0 && value != 1) return MOE_ERR_BAD_SHAPE;
      p->dec_kernel = value;
      return MOE_OK;
    case MOE_OPT_DEC_MFMA_MIN_T:
      if (value < 1) return MOE_ERR_BAD_SHAPE;
      p->dec_mfma_min_t = value;
      return MOE_OK;
    case MOE_OPT_GROUPED_TILE:
      if (value != 0 && value != 13 && value != 14 && value != 15 && value != 22 && value != 23 &&
          value != 24)
        return MOE_ERR_BAD_SHAPE;
      p->big_cfg = value;
      return MOE_OK;
    case MOE_OPT_Q8_TILE:
      if (value != 0 && value != 64 && value != 128 && value != 192) return MOE_ERR_BAD_SHAPE;
      p->q8_tm = value / 64;
      return MOE_OK;
    case MOE_OPT_SMALL_ROUTE_T:
      if (value < 0 || value > 64) return MOE_ERR_BAD_SHAPE;
      p->small_route_t = value;
      return MOE_OK;
  }
  return MOE_ERR_UNSUPPORTED;
}

moe_status moe_rmsnorm(int32_t n_tokens, int32_t d, const uint16_t* x, const uint16_t* gamma,
                       float eps, uint16_t* xn, void* stream) {
  if (n_tokens < 0 || d <= 0) return MOE_ERR_BAD_SHAPE;
  if (d % 8 || !(eps >= 0.0f) || !(eps < INFINITY)) return MOE_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !gamma || !xn) return MOE_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(xn, 16)) return MOE_ERR_ALIGNMENT;
  // rows of up to 8 chunks per lane (d <= 4096) are held in registers
  rmsnorm_bf16<8><<<(n_tokens + 3) / 4, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      x, gamma, eps, xn, n_tokens, d);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_residual_add(int32_t n_tokens, int32_t d, const uint16_t* residual, const float* a,
                            const float* b, uint16_t* out, void* stream) {
  if (n_tokens < 0 || d <= 0) return MOE_ERR_BAD_SHAPE;
  if (d % 4) return MOE_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MOE_OK;
  if (!residual || !a || !out) return MOE_ERR_NULL_ARG;
  if (!aligned(residual, 8) || !aligned(a, 16) || (b && !aligned(b, 16)) || !aligned(out, 8))
    return MOE_ERR_ALIGNMENT;
  const size_t n4 = (size_t)n_tokens * d / 4;
  residual_add_bf16<<<(unsigned)((n4 + 255) / 256), 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      residual, a, b, out, n4);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_act_quant(int32_t rows, int32_t K, const uint16_t* x, uint8_t* q, uint8_t* scales,
                         void* stream) {
  if (rows < 0 || K <= 0) return MOE_ERR_BAD_SHAPE;
  if (K % 8) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(q, 8)) return MOE_ERR_ALIGNMENT;
  launch_act_quant(x, q, scales, rows, K, reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_timing_disable(moe_plan_t p) {
  if (p == nullptr) return MOE_ERR_NULL_ARG;
  for (hipEvent_t e : p->timing_ev)
    if (e != nullptr) (void)hipEventDestroy(e);  // stages outside the mask have none
  p->timing_ev.clear();
  p->timing_done.clear();
  p->timing_mask = 0;
  p->timing_max = p->timing_n = 0;
  return MOE_OK;
}

moe_status moe_timing_enable(moe_plan_t p, uint32_t stage_mask, int32_t max_forwards) {
  if (p == nullptr) return MOE_ERR_NULL_ARG;
  if (max_forwards <= 0 || max_forwards > (1 << 16) || stage_mask >> MOE_N_STAGES)
    return MOE_ERR_BAD_SHAPE;
  moe_timing_disable(p);
  p->timing_ev.assign((size_t)max_forwards * MOE_N_STAGES * 2, nullptr);
  p->timing_done.assign((size_t)max_forwards, 0u);
  for (int f = 0; f < max_forwards; ++f)
    for (int st = 0; st < MOE_N_STAGES; ++st)
      if (stage_mask >> st & 1u)
        for (int b = 0; b < 2; ++b) {
          hipError_t err = hipEventCreate(&p->timing_ev[((size_t)f * MOE_N_STAGES + st) * 2 + b]);
          if (err != hipSuccess) {
            moe_timing_disable(p);
            return hip_fail(p, err, "hipEventCreate");
          }
        }
  p->timing_mask = stage_mask;
  p->timing_max = max_forwards;
  p->timing_n = 0;
  return MOE_OK;
}

moe_status moe_timing_collect(moe_plan_t p, float* stage_ms, int32_t* n_forwards) {
  if (p == nullptr || stage_ms == nullptr) return MOE_ERR_NULL_ARG;
  for (int st = 0; st < MOE_N_STAGES; ++st) stage_ms[st] = 0.0f;
  const int n = p->timing_n;
  if (n_forwards) *n_forwards = n;
  if (n == 0 || p->timing_mask == 0) return MOE_OK;
  const uint32_t last_done = p->timing_done[n - 1];
  if (last_done == 0u) return MOE_OK;
  int last = MOE_N_STAGES - 1;
  while (!(last_done >> last & 1u)) --last;
  hipError_t err = hipEventSynchronize(p->timing_ev[((size_t)(n - 1) * MOE_N_STAGES + last) * 2 + 1]);
  if (err != hipSuccess) return hip_fail(p, err, "hipEventSynchronize");
  for (int f = 0; f < n; ++f)
    for (int st = 0; st < MOE_N_STAGES; ++st) {
      if (!(p->timing_done[f] >> st & 1u)) continue;
      float ms = 0.0f;
      const size_t i = ((size_t)f * MOE_N_STAGES + st) * 2;
      err = hipEventElapsedTime(&ms, p->timing_ev[i], p->timing_ev[i + 1]);
      if (err != hipSuccess) return hip_fail(p, err, "hipEventElapsedTime");
      stage_ms[st] += ms;
    }
  p->timing_n = 0;
  std::fill(p->timing_done.begin(), p->timing_done.end(), 0u);
  return MOE_OK;
}

void moe_plan_free(moe_plan_t p) {
  if (p == nullptr) return;
  moe_timing_disable(p);
  delete p;
}

const char* moe_plan_info(moe_plan_t p) {
  if (p == nullptr) return "";
  if (!p->last_error.empty()) {
    static thread_local std::string s;
    s = p->info + "; last error: " + p->last_error;
    return s.c_str();
  }
  return p->info.c_str();
}

size_t moe_workspace_size(moe_plan_t p, int32_t T) {
  if (p == nullptr || T <= 0) return 0;
  return layout(p, T).total;
}

int64_t moe_workspace_h_offset(moe_plan_t p, int32_t T) {
  if (p == nullptr || T <= 0) return -1;
  return (int64_t)layout(p, T).h;
}

int32_t moe_plan_path(moe_plan_t p, int32_t T) {
  if (p == nullptr) return -1;
  return path_for(p, T);
}

}  // extern "C"

namespace {

// The layer's inputs and outputs beyond moe_forward's: the shared expert's
// matrices (NULL without one) and the residual add.
struct BlockIO {
  const moe_mat* sg = nullptr;
  const moe_mat* su = nullptr;
  const moe_mat* sd = nullptr;
  const uint16_t* residual = nullptr;
  uint16_t* out_bf16 = nullptr;
};

moe_status forward_impl(moe_plan_t p, int32_t T, const uint16_t* x, const float* w_router,
                        const float* logit_bias, const moe_mat* gate, const moe_mat* up,
                        const moe_mat* down, float* out, int32_t* topk_ids, float* topk_w,
                        int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                        size_t workspace_bytes, void* stream, const BlockIO& io = BlockIO()) {
  if (p == nullptr) return MOE_ERR_NULL_ARG;
  if (T < 0 || T > p->d.max_tokens) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || workspace == nullptr) return MOE_ERR_NULL_ARG;
  // at least one destination; a residual and its bf16 sum come together
  if ((out == nullptr && io.out_bf16 == nullptr) || ((io.residual == nullptr) != (io.out_bf16 == nullptr)))
    return MOE_ERR_NULL_ARG;
  // a plan with a shared expert needs its three matrices, a plan without none
  const bool shared = p->d.shared_expert != 0;
  if (shared != (io.sg != nullptr) || shared != (io.su != nullptr) || shared != (io.sd != nullptr))
    return MOE_ERR_NULL_ARG;
  moe_status st;
  if ((st = check_mat(p, gate)) != MOE_OK || (st = check_mat(p, up)) != MOE_OK ||
      (st = check_mat(p, down)) != MOE_OK)
    return st;
  if (shared && ((st = check_mat(p, io.sg)) != MOE_OK || (st = check_mat(p, io.su)) != MOE_OK ||
                 (st = check_mat(p, io.sd)) != MOE_OK))
    return st;
  if (!aligned(x, 16) || !aligned(w_router, 16) || (out && !aligned(out, 16)) ||
      !aligned(workspace, ALIGN) || (io.residual && !aligned(io.residual, 8)) ||
      (io.out_bf16 && !aligned(io.out_bf16, 8)))
    return MOE_ERR_ALIGNMENT;
  if ((logit_bias && !aligned(logit_bias, 4)) || (topk_ids && !aligned(topk_ids, 4)) ||
      (topk_w && !aligned(topk_w, 4)) || (counts && !aligned(counts, 4)) ||
      (offsets && !aligned(offsets, 4)) || (perm && !aligned(perm, 4)))
    return MOE_ERR_ALIGNMENT;
  const Layout L = layout(p, T);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != p->device) return MOE_ERR_DEVICE;

  const int d = p->d.d_model, E = p->d.n_experts, k = p->d.top_k;
  const int S = T * k;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w ? topk_w : reinterpret_cast<float*>(ws + L.w);
  int32_t* cnt = counts ? counts : reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* off = offsets ? offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* prm = perm ? perm : reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv_perm);
  int32_t* rank = reinterpret_cast<int32_t*>(ws + L.rank);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.hist);
  int32_t* base = reinterpret_cast<int32_t*>(ws + L.base);

  // one expert, top-1 (the dense branch): the routing is the identity with
  // weight 1, so the router, the combine and the y buffer are skipped and
  // the down projection writes out directly (out = 1 * y exactly)
  const bool dense = E == 1 && k == 1;
  if (dense && (io.residual || !out)) return MOE_ERR_UNSUPPORTED;  // the down projection writes out
  if (dense) {
    mark(p, MOE_STAGE_TOPK, false, s);
    route_dense<<<(std::max(T, L.max_tiles) + 255) / 256, 256, 0, s>>>(
        ids, w, cnt, off, prm, inv, reinterpret_cast<int32_t*>(ws + L.tok_of),
        reinterpret_cast<int4*>(ws + L.slot_info), reinterpret_cast<int32_t*>(ws + L.n_active),
        reinterpret_cast<int4*>(ws + L.tiles), reinterpret_cast<int32_t*>(ws + L.n_tiles), T,
        tile_rows(p, T));
    mark(p, MOE_STAGE_TOPK, true, s);
  } else {
  // a1: router logits (K-slice partials)
  int slice = 0;
  const int nsplit = router_split(p, T, &slice);
  mark(p, MOE_STAGE_ROUTER, false, s);
  if (T <= GEMV_MAX_T) {
    const dim3 g((E + 3) / 4, nsplit);
    if (T == 1)
      router_gemv<1><<<g, 256, 0, s>>>(x, w_router, logits, T, d, E, slice);
    else if (T <= 4)
      router_gemv<4><<<g, 256, 0, s>>>(x, w_router, logits, T, d, E, slice);
    else if (T <= 8)
      router_gemv<8><<<g, 256, 0, s>>>(x, w_router, logits, T, d, E, slice);
    else
      router_gemv<16><<<g, 256, 0, s>>>(x, w_router, logits, T, d, E, slice);
  } else {
    if (router_big(p, T)) {
      uint16_t* w3 = reinterpret_cast<uint16_t*>(ws + L.w3);
      const size_t n = (size_t)E * d;
      router_split3<<<(unsigned)((n / 4 + 255) / 256), 256, 0, s>>>(w_router, w3, n);
      const dim3 g((T + 255) / 256, (E + 127) / 128, nsplit);
      router_mfma_big<<<g, 512, 0, s>>>(x, w3, logits, T, d, E, slice);
    } else {
      const dim3 g((T + 63) / 64, (E + 63) / 64, nsplit);
      router_mfma<<<g, 256, 0, s>>>(x, w_router, logits, T, d, E, slice);
    }
  }
  mark(p, MOE_STAGE_ROUTER, true, s);
  const int ng = (E + WAVE - 1) / WAVE;
  const int ngp = ng <= 1 ? 1 : ng <= 2 ? 2 : ng <= 4 ? 4 : ng <= 8 ? 8 : 16;
  // up to 64 tokens with at most 64 experts (measured on the OLMoE shape:
  // 2-5 % faster per step at 24-48 tokens than the four routing launches;
  // no gain with 256 or 384 experts), else up to 16 tokens
  const int small_t = p->small_route_t > 0 ? p->small_route_t : (E <= 64 ? 64 : 16);
  if (T <= small_t && S <= 1023) {
    // a2 + a3 in one workgroup
    mark(p, MOE_STAGE_TOPK, false, s);
#define MOE_SMALL(NG)                                                                            \
  route_small<NG><<<1, 1024, 0, s>>>(logits, nsplit, logit_bias, ids, w, cnt, off, prm, inv,     \
                                     reinterpret_cast<int32_t*>(ws + L.tok_of),                  \
                                     reinterpret_cast<int4*>(ws + L.slot_info),                  \
                                     reinterpret_cast<int32_t*>(ws + L.n_active), L.n_slots,     \
                                     reinterpret_cast<int4*>(ws + L.tiles),                      \
                                     reinterpret_cast<int32_t*>(ws + L.n_tiles), T, E, k,        \
                                     p->d.renorm, tile_rows(p, T), shared ? 1 : 0)
    switch (ngp) {
      case 1: MOE_SMALL(1); break;
      case 2: MOE_SMALL(2); break;
      case 4: MOE_SMALL(4); break;
      case 8: MOE_SMALL(8); break;
      default: MOE_SMALL(16); break;
    }
#undef MOE_SMALL
    mark(p, MOE_STAGE_TOPK, true, s);
  } else {
  // a2: softmax + top-k
  mark(p, MOE_STAGE_TOPK, false, s);
#define MOE_TOPK(NG)                                                                          \
  route_topk<NG><<<(T + 3) / 4, 256, 0, s>>>(logits, nsplit, logit_bias, ids, w, T, E, k, \
                                             p->d.renorm)
  switch (ngp) {
    case 1: MOE_TOPK(1); break;
    case 2: MOE_TOPK(2); break;
    case 4: MOE_TOPK(4); break;
    case 8: MOE_TOPK(8); break;
    default: MOE_TOPK(16); break;
  }
#undef MOE_TOPK
  mark(p, MOE_STAGE_TOPK, true, s);
  // a3: counting-sort permute
  mark(p, MOE_STAGE_PERMUTE, false, s);
  permute_count<<<L.nchunk, WAVE, 0, s>>>(ids, rank, hist, T, E, k);
  permute_scan<<<1, 1024, 0, s>>>(hist, base, cnt, off, reinterpret_cast<int4*>(ws + L.slot_info),
                                  reinterpret_cast<int32_t*>(ws + L.n_active), L.n_slots, reinterpret_cast<int4*>(ws + L.tiles),
                                  reinterpret_cast<int32_t*>(ws + L.n_tiles), L.nchunk, E, S,
                                  tile_rows(p, T), reinterpret_cast<int32_t*>(ws + L.tok_of),
                                  shared ? T : 0);
  permute_scatter<<<(S + 255) / 256, 256, 0, s>>>(ids, rank, base, off, prm, inv,
                                                  reinterpret_cast<int32_t*>(ws + L.tok_of), S, E,
                                                  k);
  mark(p, MOE_STAGE_PERMUTE, true, s);
  }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(p, err, "routing launch");

  // a4, a5: expert stage
  auto dmat = [](const moe_mat* m, const moe_mat* shm) {
    return DMat{static_cast<const uint8_t*>(m->q), static_cast<const uint8_t*>(m->scale),
                m->q_expert_stride, m->s_expert_stride,
                shm ? static_cast<const uint8_t*>(shm->q) : nullptr,
                shm ? static_cast<const uint8_t*>(shm->scale) : nullptr};
  };
  const DMat G = dmat(gate, io.sg), U = dmat(up, io.su), D = dmat(down, io.sd);
  float* y_dst = dense ? out : nullptr;
  // activation-quantised plans: the block-scaled GEMMs on the grouped path;
  // on the decode path the decode kernels on the quantised values as bf16
  const bool q8 = p->d.act_fmt == MOE_ACT_E4M3_G128;
  if (q8 && path_for(p, T) == MOE_PATH_GROUPED)
    st = p->d.wfmt == MOE_W_E4M3_B128 ? launch_q8_stage<FMT_E4M3>(p, T, x, G, U, D, L, ws, y_dst, s)
                                      : launch_q8_stage<FMT_E2M1>(p, T, x, G, U, D, L, ws, y_dst, s);
  else
  st = p->d.wfmt == MOE_W_E4M3_B128 ? launch_expert_stage<FMT_E4M3>(p, T, x, G, U, D, L, ws, y_dst, s, q8)
       : p->d.wfmt == MOE_W_E2M1_UE8M0_G32
           ? launch_expert_stage<FMT_E2M1>(p, T, x, G, U, D, L, ws, y_dst, s, q8)
           : launch_expert_stage<FMT_NVFP4>(p, T, x, G, U, D, L, ws, y_dst, s, q8);
  if (st != MOE_OK) return st;

  // a6: fixed-order combine
  mark(p, MOE_STAGE_COMBINE, false, s);
  if (!dense) {
    const int ncb = (d / 4 + 255) / 256;
    const dim3 g((unsigned)((long long)T * ncb));
    const float* y = reinterpret_cast<const float*>(ws + L.y);
    const float* y_sh = shared ? y + (size_t)S * d : nullptr;  // the shared expert's rows
    switch (k) {
#define MOE_COMBINE(KM)                                                                          \
  case KM:                                                                                       \
    combine_fixed_order<KM><<<g, 256, 0, s>>>(y, w, inv, y_sh, io.residual, out, io.out_bf16, d, ncb); \
    break;
      MOE_COMBINE(1) MOE_COMBINE(2) MOE_COMBINE(3) MOE_COMBINE(4) MOE_COMBINE(5) MOE_COMBINE(6)
      MOE_COMBINE(7) MOE_COMBINE(8) MOE_COMBINE(9) MOE_COMBINE(10) MOE_COMBINE(11) MOE_COMBINE(12)
      MOE_COMBINE(13) MOE_COMBINE(14) MOE_COMBINE(15) default: MOE_COMBINE(16)
#undef MOE_COMBINE
    }
  }
  mark(p, MOE_STAGE_COMBINE, true, s);
  if (p->timing_mask && p->timing_n < p->timing_max) ++p->timing_n;
  err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(p, err, "combine launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(moe_plan_t p, int32_t T, const uint16_t* x, const float* w_router,
                       const float* logit_bias, const moe_mat* gate, const moe_mat* up,
                       const moe_mat* down, float* out, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (out == nullptr) return MOE_ERR_NULL_ARG;
  return forward_impl(p, T, x, w_router, logit_bias, gate, up, down, out, topk_ids, topk_w, counts,
                      offsets, perm, workspace, workspace_bytes, stream);
}

moe_status moe_forward_block(moe_plan_t p, int32_t T, const uint16_t* x, const float* w_router,
                             const float* logit_bias, const moe_mat* gate, const moe_mat* up,
                             const moe_mat* down, const moe_mat* shared_gate,
                             const moe_mat* shared_up, const moe_mat* shared_down,
                             const uint16_t* residual, uint16_t* out_bf16, float* out,
                             int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* perm, void* workspace, size_t workspace_bytes, void* stream) {
  BlockIO io;
  io.sg = shared_gate;
  io.su = shared_up;
  io.sd = shared_down;
  io.residual = residual;
  io.out_bf16 = out_bf16;
  return forward_impl(p, T, x, w_router, logit_bias, gate, up, down, out, topk_ids, topk_w, counts,
                      offsets, perm, workspace, workspace_bytes, stream, io);
}

size_t moe_noalloc_scratch_bytes(void) { return MOE_NOALLOC_SCRATCH_BYTES; }

moe_status moe_forward_noalloc(moe_plan_t p, int32_t T, const uint16_t* x, const float* w_router,
                               const float* logit_bias, const moe_mat* gate, const moe_mat* up,
                               const moe_mat* down, float* out, int32_t* topk_ids, float* topk_w,
                               int32_t* counts, int32_t* offsets, int32_t* perm, void* stream) {
  if (p == nullptr) return MOE_ERR_NULL_ARG;
  if (T < 0 || T > p->d.max_tokens) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  if (layout(p, T).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = scratch_ptr(p->device);
  if (ws == nullptr) return MOE_ERR_HIP;
  return forward_impl(p, T, x, w_router, logit_bias, gate, up, down, out, topk_ids, topk_w, counts,
                      offsets, perm, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
