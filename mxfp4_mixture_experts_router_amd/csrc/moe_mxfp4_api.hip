// Host side of the C ABI declared in include/moe_mxfp4.h: argument checks,
// workspace carving and kernel launches on the caller's stream.
//
// Every check runs before the first launch, so an error status means nothing
// was enqueued ("MXFP4 MoE decode kernels", Limitations and pitfalls: inputs
// outside the supported shapes are refused with the reason, and unexpected
// dtypes must be rejected rather than silently re-typed).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "kernels.h"
#include "moe_mxfp4.h"

namespace {

using moe::Plan;

constexpr int kMaxGrid = 16384;

struct Layout {
  size_t plan, ids, weights, counts, offsets, touched, routes, pos, a, o, total;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

Layout make_layout(const moe_mxfp4_desc& d) {
  const size_t R = static_cast<size_t>(d.T) * d.top_k;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.plan = take(sizeof(Plan));
  L.ids = take(R * 4);
  L.weights = take(R * 4);
  L.counts = take(static_cast<size_t>(d.E_local) * 4);
  L.offsets = take((static_cast<size_t>(d.E_local) + 1) * 4);
  L.touched = take(static_cast<size_t>(d.E_local) * 4);
  L.routes = take(R * 4);
  L.pos = take(R * 4);
  L.a = take(R * d.I * 2);
  L.o = take(R * d.K * 4);
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const moe_mxfp4_desc* d) {
  if (d == nullptr) return MOE_ERR_NULL;
  if (d->T < 0) return MOE_ERR_SHAPE;
  if (d->K < 32 || d->K > moe::kMaxDim || d->K % 32 != 0) return MOE_ERR_SHAPE;
  if (d->I < 32 || d->I > moe::kMaxDim || d->I % 32 != 0) return MOE_ERR_SHAPE;
  if (d->E_global < 1) return MOE_ERR_SHAPE;
  if (d->E_local < 1 || d->E_local > moe::kMaxLocalExperts) return MOE_ERR_SHAPE;
  if (d->expert_offset < 0 || d->expert_offset > d->E_global - d->E_local) return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > moe::kMaxTopK || d->top_k > d->E_global) return MOE_ERR_SHAPE;
  if (static_cast<int64_t>(d->T) * d->top_k > (int64_t{1} << 24)) return MOE_ERR_SHAPE;
  if (d->scoring != MOE_SCORING_SOFTMAX && d->scoring != MOE_SCORING_SIGMOID) return MOE_ERR_MODE;
  if (d->activation != MOE_ACT_SILU_MUL && d->activation != MOE_ACT_SWIGLU_OAI) return MOE_ERR_MODE;
  return MOE_OK;
}

int check_workspace(const moe_mxfp4_desc& d, const void* ws, size_t ws_bytes) {
  if (ws == nullptr) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < make_layout(d).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int tokens_bound(const moe_mxfp4_desc& d) {
  // number of touched local experts is at most min(E_local, T * top_k)
  return static_cast<int>(std::min<int64_t>(d.E_local, static_cast<int64_t>(d.T) * d.top_k));
}

void enqueue_bucket(const moe_mxfp4_desc& d, const int32_t* ids, const float* w_in, void* ws, hipStream_t s,
                    int32_t* counts_out, int32_t* offsets_out, int32_t* routes_out) {
  const Layout L = make_layout(d);
  const int R = d.T * d.top_k;
  hipLaunchKernelGGL(moe::bucket_kernel, dim3(1), dim3(1024), 0, s, ids, R, d.E_local, d.expert_offset,
                     counts_out ? counts_out : at<int32_t>(ws, L.counts),
                     offsets_out ? offsets_out : at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.routes),
                     at<int32_t>(ws, L.pos), at<int32_t>(ws, L.touched), at<Plan>(ws, L.plan), routes_out, w_in,
                     at<float>(ws, L.weights));
}

// Routing (logits mode) and bucketing into the workspace.
void enqueue_plan(const moe_mxfp4_desc& d, const float* logits, const int32_t* ids, const float* wts, void* ws,
                  hipStream_t s) {
  const Layout L = make_layout(d);
  if (logits != nullptr) {
    int32_t* ids_ws = at<int32_t>(ws, L.ids);
    hipLaunchKernelGGL(moe::route_topk_kernel, dim3((d.T + 3) / 4), dim3(256), 0, s, logits, d.T, d.E_global,
                       d.top_k, d.scoring, ids_ws, at<float>(ws, L.weights));
    enqueue_bucket(d, ids_ws, nullptr, ws, s, nullptr, nullptr, nullptr);
  } else {
    enqueue_bucket(d, ids, wts, ws, s, nullptr, nullptr, nullptr);
  }
}

void enqueue_w13(const moe_mxfp4_desc& d, const uint16_t* x, const uint8_t* w13p, const uint8_t* w13s,
                 const uint16_t* b13, uint16_t* a, void* ws, hipStream_t s) {
  const Layout L = make_layout(d);
  moe::W13Args A;
  A.x = x;
  A.w13p = w13p;
  A.w13s = w13s;
  A.b13 = b13;
  A.offsets = at<int32_t>(ws, L.offsets);
  A.routes = at<int32_t>(ws, L.routes);
  A.touched = at<int32_t>(ws, L.touched);
  A.plan = at<Plan>(ws, L.plan);
  A.a = a != nullptr ? a : at<uint16_t>(ws, L.a);
  A.K = d.K;
  A.I = d.I;
  A.top_k = d.top_k;
  A.act = d.activation;
  A.alpha = d.swiglu_alpha;
  A.limit = d.swiglu_limit;
  const int64_t work = static_cast<int64_t>(tokens_bound(d)) * (d.I / moe::kRowsPerTile);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(work, kMaxGrid)));
  const size_t lds = static_cast<size_t>(moe::kGemvTokens) * d.K * 2;
  hipLaunchKernelGGL(moe::w13_gemv_kernel, dim3(grid), dim3(256), lds, s, A);
}

void enqueue_w2_combine(const moe_mxfp4_desc& d, const uint16_t* a, const uint8_t* w2p, const uint8_t* w2s,
                        const uint16_t* b2, uint16_t* out, void* ws, hipStream_t s) {
  const Layout L = make_layout(d);
  moe::W2Args A;
  A.a = a != nullptr ? a : at<uint16_t>(ws, L.a);
  A.w2p = w2p;
  A.w2s = w2s;
  A.b2 = b2;
  A.offsets = at<int32_t>(ws, L.offsets);
  A.touched = at<int32_t>(ws, L.touched);
  A.plan = at<Plan>(ws, L.plan);
  A.o = at<float>(ws, L.o);
  A.K = d.K;
  A.I = d.I;
  const int64_t work = static_cast<int64_t>(tokens_bound(d)) * (d.K / moe::kRowsPerTile);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(work, kMaxGrid)));
  const size_t lds = static_cast<size_t>(moe::kGemvTokens) * d.I * 2;
  hipLaunchKernelGGL(moe::w2_gemv_kernel, dim3(grid), dim3(256), lds, s, A);

  moe::CombineArgs C;
  C.o = at<float>(ws, L.o);
  C.pos = at<int32_t>(ws, L.pos);
  C.weights = at<float>(ws, L.weights);
  C.out = out;
  C.T = d.T;
  C.K = d.K;
  C.top_k = d.top_k;
  hipLaunchKernelGGL(moe::combine_kernel, dim3((d.K / 4 + 255) / 256, d.T), dim3(256), 0, s, C);
}

int check_routing(const moe_mxfp4_desc& d, const float* logits, const int32_t* ids, const float* wts) {
  const bool logits_mode = logits != nullptr;
  const bool ids_mode = ids != nullptr || wts != nullptr;
  if (logits_mode == ids_mode) return MOE_ERR_MODE;
  if (ids_mode && (ids == nullptr || wts == nullptr)) return MOE_ERR_MODE;
  if (logits_mode && d.E_global > moe::kMaxGlobalExpertsRouted) return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_mxfp4_workspace_bytes(const moe_mxfp4_desc* desc, size_t* bytes) {
  const int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_NULL;
  *bytes = make_layout(*desc).total;
  return MOE_OK;
}

int moe_mxfp4_decode(const moe_mxfp4_desc* desc, const uint16_t* x, const float* router_logits,
                     const int32_t* topk_ids, const float* topk_weights, const uint8_t* w13_packed,
                     const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_packed,
                     const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const moe_mxfp4_desc& d = *desc;
  if ((st = check_routing(d, router_logits, topk_ids, topk_weights)) != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  if (!x || !w13_packed || !w13_scales || !w2_packed || !w2_scales || !out) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(out)) return MOE_ERR_ALIGN;
  if ((st = check_workspace(d, workspace, workspace_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  enqueue_plan(d, router_logits, topk_ids, topk_weights, workspace, s);
  enqueue_w13(d, x, w13_packed, w13_scales, w13_bias, nullptr, workspace, s);
  enqueue_w2_combine(d, nullptr, w2_packed, w2_scales, w2_bias, out, workspace, s);
  return launch_status();
}

int moe_mxfp4_plan(const moe_mxfp4_desc* desc, const float* router_logits, const int32_t* topk_ids,
                   const float* topk_weights, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_routing(*desc, router_logits, topk_ids, topk_weights)) != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  enqueue_plan(*desc, router_logits, topk_ids, topk_weights, workspace, static_cast<hipStream_t>(stream));
  return launch_status();
}

int moe_mxfp4_gate_up(const moe_mxfp4_desc* desc, const uint16_t* x, const uint8_t* w13_packed,
                      const uint8_t* w13_scales, const uint16_t* w13_bias, uint16_t* a, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!x || !w13_packed || !w13_scales) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(a)) return MOE_ERR_ALIGN;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  enqueue_w13(*desc, x, w13_packed, w13_scales, w13_bias, a, workspace, static_cast<hipStream_t>(stream));
  return launch_status();
}

int moe_mxfp4_down(const moe_mxfp4_desc* desc, const uint16_t* a, const uint8_t* w2_packed,
                   const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!w2_packed || !w2_scales || !out) return MOE_ERR_NULL;
  if (!aligned16(a) || !aligned16(w2_packed) || !aligned16(out)) return MOE_ERR_ALIGN;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  enqueue_w2_combine(*desc, a, w2_packed, w2_scales, w2_bias, out, workspace, static_cast<hipStream_t>(stream));
  return launch_status();
}

int moe_mxfp4_route(const moe_mxfp4_desc* desc, const float* router_logits, int32_t* topk_ids,
                    float* topk_weights, void* stream) {
  const int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->E_global > moe::kMaxGlobalExpertsRouted) return MOE_ERR_SHAPE;
  if (desc->T == 0) return MOE_OK;
  if (!router_logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  hipLaunchKernelGGL(moe::route_topk_kernel, dim3((desc->T + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), router_logits, desc->T, desc->E_global, desc->top_k,
                     desc->scoring, topk_ids, topk_weights);
  return launch_status();
}

int moe_mxfp4_bucket(const moe_mxfp4_desc* desc, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                     int32_t* routes, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !routes) return MOE_ERR_NULL;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  enqueue_bucket(*desc, topk_ids, nullptr, workspace, static_cast<hipStream_t>(stream), counts, offsets, routes);
  return launch_status();
}

int moe_mxfp4_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t cols, int32_t out_dtype,
                      void* out, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return MOE_ERR_SHAPE;
  if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16) return MOE_ERR_MODE;
  const int64_t n_blocks = rows * (cols / 32);
  if (n_blocks == 0) return MOE_OK;
  if (!packed || !scales || !out) return MOE_ERR_NULL;
  if (!aligned16(packed) || !aligned16(out)) return MOE_ERR_ALIGN;
  const int64_t grid = (n_blocks + 255) / 256;
  if (grid > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(moe::dequant_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), packed, scales, n_blocks, out_dtype == MOE_DTYPE_BF16 ? 1 : 0,
                     out);
  return launch_status();
}

const char* moe_mxfp4_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is outside the supported range";
    case MOE_ERR_MODE: return "MOE_ERR_MODE: give router logits or top-k ids+weights (exactly one); valid enums";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported a launch error";
    default: return "unknown status";
  }
}

const char* moe_mxfp4_version(void) { return "moe_mxfp4 0.1.0 (gfx950)"; }

}  // extern "C"
