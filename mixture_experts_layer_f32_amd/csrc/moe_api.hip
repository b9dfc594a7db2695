// C ABI of the gfx950 MoE FFN layer: plan, validation, workspace layout and
// the launch sequence.  All device work is enqueued on the caller's stream;
// the host never waits on the device here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "moe.h"
#include "moe_common.h"
#include "moe_decode.h"
#include "moe_gemm.h"
#include "moe_route.h"

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Tile sizes of the grouped GEMMs and the decode matvecs.
constexpr int GEMM_BM = 64;
constexpr int GEMM_BN = 64;
constexpr int DEC_RPW = 2;       // rows per wavefront in the decode matvecs
constexpr int GEMV_MAX_T = 16;   // router: one wave per expert up to this many tokens

struct Layout {
  size_t logits, ids, w, counts, offsets, perm, inv_perm, rank, hist, base, active, n_active,
      tiles, n_tiles, h, y, total;
  int nchunk, max_tiles;
};

}  // namespace

struct moe_plan_s {
  moe_desc d;
  int device = -1;
  int cus = 0;
  std::string arch;
  int t_decode = 0;  // AUTO: decode variant for T <= t_decode
  std::string info;
  std::string last_error;
};

namespace {

int path_for(const moe_plan_s* p, int T) {
  if (p->d.path == MOE_PATH_DECODE) return MOE_PATH_DECODE;
  if (p->d.path == MOE_PATH_GROUPED) return MOE_PATH_GROUPED;
  return T <= p->t_decode ? MOE_PATH_DECODE : MOE_PATH_GROUPED;
}

Layout layout(const moe_plan_s* p, int T) {
  const size_t E = p->d.n_experts, k = p->d.top_k, d = p->d.d_model, f = p->d.d_ff;
  const size_t S = (size_t)T * k;
  Layout L;
  L.nchunk = (T + WAVE - 1) / WAVE;
  L.max_tiles = (int)((S + GEMM_BM - 1) / GEMM_BM + std::min<size_t>(E, S));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.logits = take((size_t)T * E * 4);
  L.ids = take(S * 4);
  L.w = take(S * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(S * 4);
  L.inv_perm = take(S * 4);
  L.rank = take(S * 4);
  L.hist = take((size_t)L.nchunk * E * 4);
  L.base = take((size_t)L.nchunk * E * 4);
  L.active = take(E * 4);
  L.n_active = take(4);
  L.tiles = take((size_t)L.max_tiles * 16);
  L.n_tiles = take(4);
  L.h = take(S * f * 2);
  L.y = take(S * d * 4);
  L.total = o;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_fail(moe_plan_s* p, hipError_t err, const char* what) {
  p->last_error = std::string(what) + ": " + hipGetErrorString(err);
  return MOE_ERR_HIP;
}

template <int FMT>
moe_status launch_expert_stage(moe_plan_s* p, int T, const uint16_t* x, DMat G, DMat U, DMat D,
                               const Layout& L, char* ws, int32_t* counts, int32_t* offsets,
                               int32_t* perm, hipStream_t st) {
  const int d = p->d.d_model, f = p->d.d_ff, E = p->d.n_experts, k = p->d.top_k;
  const int S = T * k;
  const int32_t* active = reinterpret_cast<const int32_t*>(ws + L.active);
  const int32_t* n_active = reinterpret_cast<const int32_t*>(ws + L.n_active);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  float* y = reinterpret_cast<float*>(ws + L.y);
  if (path_for(p, T) == MOE_PATH_DECODE) {
    const int slots = std::min(S, E);
    const dim3 g1(slots, (f / DEC_RPW + 3) / 4), g2(slots, (d / DEC_RPW + 3) / 4);
    if (T == 1) {
      dec_gateup<FMT, 1, DEC_RPW><<<g1, 256, 0, st>>>(x, G, U, active, n_active, counts, offsets,
                                                      perm, h, d, f, k, T);
      dec_down<FMT, 1, DEC_RPW><<<g2, 256, 0, st>>>(h, D, active, n_active, counts, offsets, y, d,
                                                    f);
    } else if (T <= 2) {
      dec_gateup<FMT, 2, DEC_RPW><<<g1, 256, 0, st>>>(x, G, U, active, n_active, counts, offsets,
                                                      perm, h, d, f, k, T);
      dec_down<FMT, 2, DEC_RPW><<<g2, 256, 0, st>>>(h, D, active, n_active, counts, offsets, y, d,
                                                    f);
    } else {
      dec_gateup<FMT, 4, DEC_RPW><<<g1, 256, 0, st>>>(x, G, U, active, n_active, counts, offsets,
                                                      perm, h, d, f, k, T);
      dec_down<FMT, 4, DEC_RPW><<<g2, 256, 0, st>>>(h, D, active, n_active, counts, offsets, y, d,
                                                    f);
    }
  } else {
    const int4* tiles = reinterpret_cast<const int4*>(ws + L.tiles);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(ws + L.n_tiles);
    const dim3 g1(L.max_tiles, (f + GEMM_BN - 1) / GEMM_BN), g2(L.max_tiles, (d + GEMM_BN - 1) / GEMM_BN);
    gemm_gateup<FMT, GEMM_BM, GEMM_BN><<<g1, 256, 0, st>>>(x, G, U, tiles, n_tiles, perm, h, d, f,
                                                          k, T);
    gemm_down<FMT, GEMM_BM, GEMM_BN><<<g2, 256, 0, st>>>(h, D, tiles, n_tiles, y, d, f);
  }
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
  if (d.n_experts > MAX_E || d.top_k > MAX_K) return MOE_ERR_UNSUPPORTED;
  if (d.wfmt == MOE_W_E4M3_B128) {
    if (d.d_model % 128 || d.d_ff % 128) return MOE_ERR_UNSUPPORTED;
  } else if (d.wfmt == MOE_W_E2M1_UE8M0_G32) {
    if (d.d_model % 32 || d.d_ff % 32) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  // int32 sorted positions and 32-bit grid sizes
  if ((int64_t)d.max_tokens * d.top_k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;

  int dev = -1, ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;

  moe_plan_s* p = new (std::nothrow) moe_plan_s();
  if (p == nullptr) return MOE_ERR_HIP;
  p->d = d;
  p->device = dev;
  p->cus = prop.multiProcessorCount;
  p->arch = prop.gcnArchName;
  // Decode while the slots per expert stay small: T*k <= 4*E.
  p->t_decode = std::max(1, 4 * d.n_experts / d.top_k);
  char buf[512];
  std::snprintf(buf, sizeof buf,
                "device %d %s (%d CUs); d=%d f=%d E=%d k=%d fmt=%s renorm=%d; path=%s "
                "(decode for T<=%d); router gemv<=%d tokens else 64x64 f32 tiles; "
                "decode matvec rows/wave=%d; grouped MFMA 32x32x16 bf16 tiles BMxBN=%dx%d",
                dev, p->arch.c_str(), p->cus, d.d_model, d.d_ff, d.n_experts, d.top_k,
                d.wfmt == MOE_W_E4M3_B128 ? "e4m3/128x128" : "e2m1/ue8m0x32", d.renorm,
                d.path == MOE_PATH_AUTO ? "auto" : (d.path == MOE_PATH_DECODE ? "decode" : "grouped"),
                p->t_decode, GEMV_MAX_T, DEC_RPW, GEMM_BM, GEMM_BN);
  p->info = buf;
  *out = p;
  return MOE_OK;
}

void moe_plan_free(moe_plan_t p) { delete p; }

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

moe_status moe_forward(moe_plan_t p, int32_t T, const uint16_t* x, const float* w_router,
                       const float* logit_bias, const moe_mat* gate, const moe_mat* up,
                       const moe_mat* down, float* out, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (p == nullptr) return MOE_ERR_NULL_ARG;
  if (T < 0 || T > p->d.max_tokens) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || out == nullptr || workspace == nullptr)
    return MOE_ERR_NULL_ARG;
  moe_status st;
  if ((st = check_mat(p, gate)) != MOE_OK || (st = check_mat(p, up)) != MOE_OK ||
      (st = check_mat(p, down)) != MOE_OK)
    return st;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(out, 16) || !aligned(workspace, ALIGN))
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

  // a1: router logits
  if (T <= GEMV_MAX_T) {
    const dim3 g((E + 3) / 4);
    if (T == 1)
      router_gemv<1><<<g, 256, 0, s>>>(x, w_router, logit_bias, logits, T, d, E);
    else if (T <= 4)
      router_gemv<4><<<g, 256, 0, s>>>(x, w_router, logit_bias, logits, T, d, E);
    else
      router_gemv<8><<<g, 256, 0, s>>>(x, w_router, logit_bias, logits, T, d, E);
  } else {
    const dim3 g((T + 63) / 64, (E + 63) / 64);
    router_gemm<<<g, 256, 0, s>>>(x, w_router, logit_bias, logits, T, d, E);
  }
  // a2: softmax + top-k
  route_topk<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, T, E, k, p->d.renorm);
  // a3: counting-sort permute
  permute_count<<<L.nchunk, WAVE, 0, s>>>(ids, rank, hist, T, E, k);
  permute_scan<<<1, 1024, 0, s>>>(hist, base, cnt, off, reinterpret_cast<int32_t*>(ws + L.active),
                                  reinterpret_cast<int32_t*>(ws + L.n_active),
                                  reinterpret_cast<int4*>(ws + L.tiles),
                                  reinterpret_cast<int32_t*>(ws + L.n_tiles), L.nchunk, E, S,
                                  GEMM_BM);
  permute_scatter<<<(S + 255) / 256, 256, 0, s>>>(ids, rank, base, off, prm, inv, S, E, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(p, err, "routing launch");

  // a4, a5: expert stage
  const DMat G{static_cast<const uint8_t*>(gate->q), static_cast<const uint8_t*>(gate->scale),
               gate->q_expert_stride, gate->s_expert_stride};
  const DMat U{static_cast<const uint8_t*>(up->q), static_cast<const uint8_t*>(up->scale),
               up->q_expert_stride, up->s_expert_stride};
  const DMat D{static_cast<const uint8_t*>(down->q), static_cast<const uint8_t*>(down->scale),
               down->q_expert_stride, down->s_expert_stride};
  st = p->d.wfmt == MOE_W_E4M3_B128
           ? launch_expert_stage<FMT_E4M3>(p, T, x, G, U, D, L, ws, cnt, off, prm, s)
           : launch_expert_stage<FMT_E2M1>(p, T, x, G, U, D, L, ws, cnt, off, prm, s);
  if (st != MOE_OK) return st;

  // a6: fixed-order combine
  combine_fixed_order<<<dim3(T, (d / 4 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const float*>(ws + L.y), w, inv, out, d, k);
  err = hipGetLastError();
  if (err != hipSuccess) return hip_fail(p, err, "combine launch");
  return MOE_OK;
}

}  // extern "C"
