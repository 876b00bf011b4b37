// Host side of the C ABI declared in include/moe_mxfp4.h: argument checks,
// workspace carving and kernel launches on the caller's stream.
//
// Every check runs before the first launch, so an error status means nothing
// was enqueued ("MXFP4 MoE decode kernels", Limitations and pitfalls: inputs
// outside the supported shapes are refused with the reason, and unexpected
// dtypes must be rejected rather than silently re-typed).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <tuple>
#include <utility>

#include "kernels.h"
#include "moe_mxfp4.h"

namespace {

using moe::Plan;


bool stream_regime(const moe_mxfp4_desc& d);
bool mfma_enabled(const moe_mxfp4_desc& d);
int stream_split(const moe_mxfp4_desc& d);
int down_split(const moe_mxfp4_desc& d);
size_t self_lds_bytes(const moe_mxfp4_desc& d);

struct Layout {
  size_t plan, ids, weights, counts, offsets, gemv_list, mfma_list, passes, passes2, routes, pos, a, o;
  size_t xq, xq_scale, aq, aq_scale;  // split activations of the scaled-FP4 MFMA kernels (0 bytes otherwise)
  size_t total;
};

// Bytes of one activation row split for the scaled-FP4 MFMA kernel: a
// 256-byte chunk (hi 128 B, lo 128 B) per 128 values.
size_t split_row_bytes(int L) { return static_cast<size_t>((L + 127) / 128) * 256; }

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
  L.gemv_list = take(static_cast<size_t>(d.E_local) * sizeof(moe::WorkEntry));
  L.mfma_list = take(static_cast<size_t>(d.E_local) * sizeof(moe::WorkEntry));
  // decode regime: at most one pass per route
  L.passes = take(stream_regime(d) ? R * sizeof(moe::PassEntry) : 0);
  // the down projection's own pass list, when its reduction split differs
  L.passes2 = take(down_split(d) != stream_split(d) ? R * sizeof(moe::PassEntry) : 0);
  L.routes = take(R * 4);
  L.pos = take(R * 4);
  L.a = take(R * d.I * 2);
  L.o = take(R * d.K * 4);
  const bool split = d.mma == MOE_MMA_SCALED_FP4 && mfma_enabled(d);
  L.xq = take(split ? static_cast<size_t>(d.T) * split_row_bytes(d.K) : 0);
  L.xq_scale = take(split ? static_cast<size_t>(d.T) * 4 : 0);
  L.aq = take(split ? R * split_row_bytes(d.I) : 0);
  L.aq_scale = take(split ? R * 4 : 0);
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
  // the kernels address x [T, K] and the intermediate [T*top_k, I] (bf16)
  // with 32-bit buffer offsets, out-of-range offsets reading zeros
  if (static_cast<int64_t>(d->T) * d->K * 2 >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;
  if (static_cast<int64_t>(d->T) * d->top_k * d->I * 2 >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;
  if (d->scoring != MOE_SCORING_SOFTMAX && d->scoring != MOE_SCORING_SIGMOID) return MOE_ERR_MODE;
  if (d->activation != MOE_ACT_SILU_MUL && d->activation != MOE_ACT_SWIGLU_OAI) return MOE_ERR_MODE;
  if (d->weight_layout != MOE_LAYOUT_ROWS && d->weight_layout != MOE_LAYOUT_TILE16) return MOE_ERR_MODE;
  if (d->down_pairing != MOE_PAIRING_AUTO && d->down_pairing != MOE_PAIRING_ON && d->down_pairing != MOE_PAIRING_OFF)
    return MOE_ERR_MODE;
  if (d->w13_order != MOE_W13_GATE_UP && d->w13_order != MOE_W13_INTERLEAVED) return MOE_ERR_MODE;
  if (d->mma != MOE_MMA_BF16 && d->mma != MOE_MMA_SCALED_FP4) return MOE_ERR_MODE;
  // the split activation rows (whole 128-value chunks) obey the same bound
  if (d->mma == MOE_MMA_SCALED_FP4) {
    if (static_cast<int64_t>(d->T) * split_row_bytes(d->K) >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;
    if (static_cast<int64_t>(d->T) * d->top_k * split_row_bytes(d->I) >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

int check_workspace(const moe_mxfp4_desc& d, const void* ws, size_t ws_bytes) {
  if (ws == nullptr) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < make_layout(d).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// kernel<<<grid, block, lds, s>>>(args...) through hipLaunchKernel, which
// returns the status of this launch only (an error left by other work on the
// thread is neither reported nor cleared).
template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A&&... args) {
  std::tuple<P...> vals{std::forward<A>(args)...};
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, s);
      },
      vals);
}

// Status of a sequence of enqueues: MOE_ERR_HIP at the first failed launch
// (the launches before it stay enqueued).
int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
#define MOE_TRY(expr)                      \
  do {                                     \
    const hipError_t moe_e_ = (expr);      \
    if (moe_e_ != hipSuccess) return moe_e_; \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int tokens_bound(const moe_mxfp4_desc& d) {
  // number of touched local experts is at most min(E_local, T * top_k)
  return static_cast<int>(std::min<int64_t>(d.E_local, static_cast<int64_t>(d.T) * d.top_k));
}

// The MFMA regime is used only when an expert can hold more than
// kGemvMaxTokens routes of distinct tokens, i.e. T > kGemvMaxTokens; the plan
// kernel and the launches below apply the same rule.
bool mfma_enabled(const moe_mxfp4_desc& d) { return d.T > moe::kGemvMaxTokens; }

// The GEMV list (experts with at most kGemvMaxTokens routes) is left out,
// and every touched expert goes to the MFMA list, when uniform routing
// expects at least kMfmaOnlyRoutes routes per expert (T * top_k / E_global):
// then an expert with one or two routes is rare (E_local * e^-16 * 145 <
// 0.01 at 16 per expert and 512 experts), the MFMA kernels serve it as a
// pass of one 16-route group, and the call skips two GEMV launches that
// would find an empty list (~5 us each at the wide-K shape, T = 2048).
constexpr int kMfmaOnlyRoutes = 16;
bool gemv_list_used(const moe_mxfp4_desc& d) {
  return !mfma_enabled(d) ||
         static_cast<int64_t>(d.T) * d.top_k < static_cast<int64_t>(kMfmaOnlyRoutes) * d.E_global;
}

// Stream regime: the persistent stream kernel, whose waves split the
// reduction kSplit ways with 16/kSplit routes per pass.  It serves every call
// with T <= kStreamMaxTokens, and larger calls while the routes per local
// expert, expected under uniform routing (T * top_k / E_global), stay within
// kStreamRoutesPerExpert: each pass of 16 routes streams its expert's weights
// again, so calls with many routes per expert belong to the MFMA kernel (64
// routes per weight pass).  Measured on the wide-K slice (48 of 384 experts,
// top-8): 5 routes per expert (T = 256) run 1.4x faster here than on the
// GEMV/MFMA lists, 43 (T = 2048) 1.5x slower.  A pass entry's route index is
// 16-bit, hence T * top_k < 65536.
// The split follows T (4 up to 4 tokens, 2 up to 8, else 1) and is lowered
// until every slice of both projections has at least kStreamRing steps; a
// projection whose reduction is still too short for that uses the GEMV/MFMA
// list kernels.
constexpr int kStreamRoutesPerExpert = 16;

bool stream_regime(const moe_mxfp4_desc& d) {
  if (d.T < 1) return false;
  if (d.T <= moe::kStreamMaxTokens) return true;
  const int64_t R = static_cast<int64_t>(d.T) * d.top_k;
  return R < 65536 && R <= static_cast<int64_t>(kStreamRoutesPerExpert) * d.E_global;
}

int steps_per_slice(int red, int split) { return ((red / 32 + 3) / 4 + split - 1) / split; }
bool stream_fits(int red, int split) { return split > 0 && steps_per_slice(red, split) >= moe::kStreamRing; }

// Wide reductions (K >= kWideSplitK) at T <= 32 with at most 2 routes per
// expert expected split gate/up 4 ways too: a row tile's 128-value steps
// are long enough to cut in four, and the shorter items end the launch with
// a shorter tail (wide-K slice T = 16 / 32: 95.0 / 129.4 -> 92.0 / 122.3 us
// per call; GLM-5.x slice T = 8 / 32: 48.1 / 104.4 -> 47.0 / 95.6 us).  At
// K = 2880 splitting gate/up above 8 tokens measured slower, and above 32
// tokens the 4-way split measured slower at wide K as well.
constexpr int kWideSplitK = 4096;

int stream_split(const moe_mxfp4_desc& d) {
  if (!stream_regime(d)) return 0;
  int split = d.T <= 4 ? 4 : (d.T <= 8 ? 2 : 1);
  if (d.K >= kWideSplitK && d.T <= 32 &&
      static_cast<int64_t>(d.T) * d.top_k <= 2 * static_cast<int64_t>(d.E_global))
    split = 4;
  while (split > 1 && !(stream_fits(d.K, split) && stream_fits(d.I, split))) split /= 2;
  return split;
}

// The down projection's split.  Its items are (pass, rows) with the whole
// reduction per workgroup when unsplit, so at decode (few routes per expert,
// T <= 32) a 4-way (up to 8 tokens) or 2-way split keeps more, shorter items
// in flight and ends the launch with a shorter tail; passes then hold 4 or 8
// routes, and an expert with more local routes than that is read once per
// pass.  So it is taken only when uniform routing expects at most 2 routes
// per expert (T * top_k <= 2 * E_global): the gpt-oss-120b shape at T = 32
// (1 route per expert) gains ~1% with split 4 and ~0.6% more with split 2
// (down 62.3 -> 61.4 us), the gpt-oss-20b shape at T = 32 (4 per expert)
// lost 7% with split 4.  The plan then writes a second pass list cut at
// the down split's route count.
int down_split(const moe_mxfp4_desc& d) {
  const int split = stream_split(d);
  const int64_t R = static_cast<int64_t>(d.T) * d.top_k;
  if (split > 0 && split < 4 && d.T <= 32 && R <= 2 * static_cast<int64_t>(d.E_global) && stream_fits(d.I, 4))
    return d.T > 8 ? 2 : 4;
  return split;
}
int pass_shift_of(int split) { return split == 4 ? 2 : (split == 2 ? 3 : 4); }  // kStreamPassTokens / split routes

size_t stream_lds_bytes(int red, bool gate_up, int split) {
  const size_t nw = gate_up ? 2 : 1;
  const size_t sw = (nw * 16 * (red / 32) + nw * 32 + 15) / 16 * 16;
  return 2 * 16 * static_cast<size_t>(moe::kXRowBytes) + 2 * 4 * sw + (split > 1 ? 4 * 64 * 8 * 4 : 0) +
         moe::kStreamMaxItems * sizeof(moe::PassEntry);
}

// Resident workgroups of a kernel on the current device (cached per device
// and kernel; calls from several host threads share the cache under a lock).
template <typename K>
int resident_workgroups(K kernel, size_t lds) {
  struct Entry {
    const void* fn;
    size_t lds;
    int dev;
    int n;
  };
  static Entry cache[64];
  static int used = 0;
  static std::mutex lock;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const void* fn = reinterpret_cast<const void*>(kernel);
  const std::lock_guard<std::mutex> guard(lock);
  for (int i = 0; i < used; ++i)
    if (cache[i].fn == fn && cache[i].lds == lds && cache[i].dev == dev) return cache[i].n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess) return 0;
  const int n = std::max(1, cus * per_cu);
  if (used < 64) cache[used++] = Entry{fn, lds, dev, n};
  return n;
}

// Key of the plan a call makes: every descriptor field and regime choice
// that shapes the plan (FNV-1a; never 0, the key of "no plan").  The expert
// kernels compare it with the key the plan kernel stored in the workspace.
uint32_t plan_key(const moe_mxfp4_desc& d, bool prefill) {
  const int split = prefill ? 0 : stream_split(d);
  const int dsplit = prefill ? 0 : down_split(d);
  const int32_t f[] = {d.T, d.K, d.I, d.E_global, d.E_local, d.expert_offset, d.top_k, split, dsplit, prefill ? 1 : 0,
                       mfma_enabled(d) ? 1 : 0, static_cast<int32_t>(stream_fits(d.K, split)),
                       static_cast<int32_t>(stream_fits(d.I, dsplit))};
  uint32_t h = 2166136261u;
  for (int32_t v : f) {
    for (int b = 0; b < 4; ++b) {
      h ^= (static_cast<uint32_t>(v) >> (8 * b)) & 0xFFu;
      h *= 16777619u;
    }
  }
  return h | 1u;
}

moe::PlanArgs plan_args(const moe_mxfp4_desc& d, void* ws) {
  const Layout L = make_layout(d);
  moe::PlanArgs P{};
  P.T = d.T;
  P.top_k = d.top_k;
  P.E_global = d.E_global;
  P.E_local = d.E_local;
  P.offset = d.expert_offset;
  P.scoring = d.scoring;
  P.mfma_enabled = mfma_enabled(d) ? 1 : 0;
  P.gemv_max = gemv_list_used(d) ? moe::kGemvMaxTokens : 0;
  P.lists = 1;
  P.ids_ws = at<int32_t>(ws, L.ids);
  P.weights_ws = at<float>(ws, L.weights);
  P.counts = at<int32_t>(ws, L.counts);
  P.offsets = at<int32_t>(ws, L.offsets);
  P.routes = at<int32_t>(ws, L.routes);
  P.pos = at<int32_t>(ws, L.pos);
  P.gemv_list = at<moe::WorkEntry>(ws, L.gemv_list);
  P.mfma_list = at<moe::WorkEntry>(ws, L.mfma_list);
  P.plan = at<Plan>(ws, L.plan);
  P.key = plan_key(d, false);
  return P;
}

// Routing and bucketing into the workspace.  Small calls route inside the
// plan kernel; larger ones route with one wave per token first.  The prefill
// path puts every touched expert in the MFMA list and needs no pass list.
moe::PlanArgs full_plan_args(const moe_mxfp4_desc& d, void* ws, bool prefill) {
  moe::PlanArgs P = plan_args(d, ws);
  const int split = prefill ? 0 : stream_split(d);
  P.key = plan_key(d, prefill);
  if (prefill) {
    P.mfma_enabled = 1;
    P.gemv_max = 0;
  }
  const int dsplit = prefill ? 0 : down_split(d);
  if (split > 0) {
    P.passes = at<moe::PassEntry>(ws, make_layout(d).passes);
    P.pass_shift = pass_shift_of(split);
  }
  if (dsplit != split) {
    P.passes2 = at<moe::PassEntry>(ws, make_layout(d).passes2);
    P.pass_shift2 = pass_shift_of(dsplit);
  }
  // the GEMV / MFMA lists are needed when a projection is not served by the stream kernel
  P.lists = !(stream_fits(d.K, split) && stream_fits(d.I, dsplit));
  return P;
}

// Router logits of calls up to kFusedRouteTokens tokens are routed inside
// the plan kernel, on its one CU, where a token's top-k takes one 16-lane row
// or one wave; with more than kFusedRouteMaxExperts experts, the
// one-wave-per-token kernel spreads the tokens over the chip first, which
// measured faster despite its launch (wide-K slice, 384 experts, top-8: T =
// 32 / 64 from 137.7 / 206.0 to 128.6 / 182.5 us per call; with 256 experts
// the two were equal).
constexpr int kFusedRouteMaxExperts = 256;

hipError_t enqueue_plan(const moe_mxfp4_desc& d, const float* logits, const int32_t* ids, const float* wts, void* ws,
                        hipStream_t s, bool prefill = false) {
  moe::PlanArgs P = full_plan_args(d, ws, prefill);
  if (logits != nullptr && d.T <= moe::kFusedRouteTokens && d.E_global <= kFusedRouteMaxExperts) {
    P.logits = logits;
  } else if (logits != nullptr) {
    MOE_TRY(launch(moe::route_topk_kernel, dim3((d.T + 3) / 4), dim3(256), 0, s, logits, d.T, d.E_global, d.top_k,
                   d.scoring, P.ids_ws, P.weights_ws));
    P.ids_in = P.ids_ws;
  } else {
    P.ids_in = ids;
    P.w_in = wts;
  }
  return launch(moe::plan_kernel, dim3(1), dim3(1024), 0, s, P);
}

hipError_t enqueue_bucket_hook(const moe_mxfp4_desc& d, const int32_t* ids, void* ws, hipStream_t s, int32_t* counts,
                               int32_t* offsets, int32_t* routes_out) {
  moe::PlanArgs P = plan_args(d, ws);
  P.ids_in = ids;
  P.counts = counts;
  P.offsets = offsets;
  P.routes_out = routes_out;
  P.key = 0;  // counts and offsets go to the caller: the workspace holds no usable plan
  return launch(moe::plan_kernel, dim3(1), dim3(1024), 0, s, P);
}

// The MFMA regime with scaled-FP4 instructions: the projection's input rows
// (x by token, or the intermediate a by plan position) are split into E4M3
// hi + lo parts in the workspace, then mfma_fp4_kernel runs on the same
// work list, grid and row pairing as mfma_kernel would.
hipError_t enqueue_mfma_fp4(const moe_mxfp4_desc& d, bool gate_up, moe::ExpertArgs M, const Layout& L, void* ws,
                            int groups, size_t lds, size_t lds1, int64_t slots, hipStream_t s) {
  const int rows = M.rows;
  moe::SplitArgs P{};
  P.in = M.in;
  P.L = M.red;
  P.plan = M.plan;
  P.key = M.key;
  P.rows_from_plan = gate_up ? 0 : 1;
  P.rows = gate_up ? d.T : d.T * d.top_k;
  P.out = at<uint8_t>(ws, gate_up ? L.xq : L.aq);
  P.scales = at<int32_t>(ws, gate_up ? L.xq_scale : L.aq_scale);
  MOE_TRY(launch(moe::mx8_split_kernel, dim3(static_cast<unsigned>(P.rows)), dim3(256), 0, s, P));
  M.in = reinterpret_cast<const uint16_t*>(P.out);
  M.in_stride = static_cast<uint32_t>(split_row_bytes(M.red));
  M.in_bytes = static_cast<uint32_t>(static_cast<size_t>(P.rows) * M.in_stride);
  M.in_scale = P.scales;
  if (gate_up) {
    const dim3 g(static_cast<unsigned>(slots * ((rows + moe::kMfmaRows - 1) / moe::kMfmaRows)));
    if (groups == 1) return launch(moe::mfma_fp4_kernel<true, 1, false>, g, dim3(256), lds, s, M);
    if (groups == 2) return launch(moe::mfma_fp4_kernel<true, 2, false>, g, dim3(256), lds, s, M);
    return launch(moe::mfma_fp4_kernel<true, 4, false>, g, dim3(256), lds, s, M);
  }
  bool pair = rows % 32 == 0 && d.down_pairing != MOE_PAIRING_OFF;
  const int64_t grid2 = slots * ((rows + 2 * moe::kMfmaRows - 1) / (2 * moe::kMfmaRows));
  if (pair && d.down_pairing == MOE_PAIRING_AUTO) {
    const int resident = groups == 1   ? resident_workgroups(moe::mfma_fp4_kernel<false, 1, true>, lds)
                         : groups == 2 ? resident_workgroups(moe::mfma_fp4_kernel<false, 2, true>, lds)
                                       : resident_workgroups(moe::mfma_fp4_kernel<false, 4, true>, lds);
    pair = grid2 >= resident;
  }
  if (pair) {
    const dim3 g(static_cast<unsigned>(grid2));
    if (groups == 1) return launch(moe::mfma_fp4_kernel<false, 1, true>, g, dim3(256), lds, s, M);
    if (groups == 2) return launch(moe::mfma_fp4_kernel<false, 2, true>, g, dim3(256), lds, s, M);
    return launch(moe::mfma_fp4_kernel<false, 4, true>, g, dim3(256), lds, s, M);
  }
  const dim3 g(static_cast<unsigned>(slots * ((rows + moe::kMfmaRows - 1) / moe::kMfmaRows)));
  if (groups == 1) return launch(moe::mfma_fp4_kernel<false, 1, false>, g, dim3(256), lds1, s, M);
  if (groups == 2) return launch(moe::mfma_fp4_kernel<false, 2, false>, g, dim3(256), lds1, s, M);
  return launch(moe::mfma_fp4_kernel<false, 4, false>, g, dim3(256), lds1, s, M);
}

// The four-set down kernel takes a down projection whose reduction is a
// multiple of 128 values and whose rows fill its 256-row tiles; mfma_kernel
// the others (and every gate/up projection).
bool down4_fits(const moe_mxfp4_desc& d) { return d.I % 128 == 0 && d.K % 256 == 0; }

// Both regimes of one projection.  Grids are host-side upper bounds: at most
// min(E_local, T*top_k) experts are touched, and at most T*top_k / (G+1) of
// them have more than G = kGemvMaxTokens routes (all of them are in the MFMA
// list when the GEMV list is left out); workgroups past the lists exit.
// With T <= G every expert is in the GEMV list (the GEMV kernel loops over
// token pairs if repeated ids give an expert more routes); otherwise experts
// with more than G routes are in the MFMA list, whose token groups per pass
// follow T.
hipError_t enqueue_expert_pair(const moe_mxfp4_desc& d, bool gate_up, moe::ExpertArgs A, const Layout& L, void* ws,
                               hipStream_t s) {
  const int64_t touched = tokens_bound(d);
  const int rows = A.rows, red = A.red;
  const int lanes = red > 4096 ? 32 : 16;
  const int rows_per_wg = 256 / lanes;
  if (gemv_list_used(d)) {
    moe::ExpertArgs G = A;
    G.list = at<moe::WorkEntry>(ws, L.gemv_list);
    G.list_cap = d.E_local;
    const size_t lds = static_cast<size_t>(moe::kGemvMaxTokens) * red * 2 +
                       static_cast<size_t>(gate_up ? 2 : 1) * rows_per_wg * (red / 32);
    // the kernel takes its (entry, row tile) units grid-stride: the grid is
    // the bound on the units, capped at the resident workgroup count
    const int resident = gate_up ? (lanes == 16 ? resident_workgroups(moe::gemv_kernel<true, 16>, lds)
                                                : resident_workgroups(moe::gemv_kernel<true, 32>, lds))
                                 : (lanes == 16 ? resident_workgroups(moe::gemv_kernel<false, 16>, lds)
                                                : resident_workgroups(moe::gemv_kernel<false, 32>, lds));
    int64_t grid = std::max<int64_t>(1, touched * (rows / rows_per_wg));
    if (resident > 0) grid = std::min<int64_t>(grid, resident);
    // With the MFMA regime on, the GEMV list holds the experts with 1..2
    // routes; when uniform routing makes those rare (T * top_k / E_global
    // routes per expert expected), a smaller grid keeps the launch of an
    // empty or short list cheap (the loop is grid-stride: any grid covers
    // any list, a long one only more slowly).
    if (mfma_enabled(d)) {
      const double lam = static_cast<double>(d.T) * d.top_k / d.E_global;
      const double p12 = std::exp(-lam) * (lam + 0.5 * lam * lam);
      const double expect = d.E_local * p12;
      const int64_t want = static_cast<int64_t>(std::ceil(4.0 * expect + 2.0)) * (rows / rows_per_wg);
      grid = std::max<int64_t>(1, std::min<int64_t>(grid, std::max<int64_t>(want, 64)));
    }
    const dim3 g(static_cast<unsigned>(grid));
    if (gate_up) {
      if (lanes == 16) MOE_TRY(launch(moe::gemv_kernel<true, 16>, g, dim3(256), lds, s, G));
      else MOE_TRY(launch(moe::gemv_kernel<true, 32>, g, dim3(256), lds, s, G));
    } else {
      if (lanes == 16) MOE_TRY(launch(moe::gemv_kernel<false, 16>, g, dim3(256), lds, s, G));
      else MOE_TRY(launch(moe::gemv_kernel<false, 32>, g, dim3(256), lds, s, G));
    }
  }
  const int64_t R = static_cast<int64_t>(d.T) * d.top_k;
  const int64_t mfma_experts =
      std::min<int64_t>(d.E_local, gemv_list_used(d) ? R / (moe::kGemvMaxTokens + 1) : R);
  if (mfma_experts > 0 && mfma_enabled(d)) {
    moe::ExpertArgs M = A;
    M.list = at<moe::WorkEntry>(ws, L.mfma_list);
    M.list_cap = d.E_local;
    const int groups = d.T <= 32 ? 1 : (d.T <= 64 ? 2 : 4);
    // two weight row sets per wave: gate and up rows, or (down) a pair of
    // 16-row sets, which then halves the grid; under MOE_PAIRING_AUTO the
    // down projection pairs when the halved grid still fills every resident
    // workgroup slot
    const size_t lds = 2 * static_cast<size_t>(16 * groups) * moe::kXRowBytes +
                       static_cast<size_t>(2) * moe::kMfmaRows * (red / 32);
    const size_t lds1 = 2 * static_cast<size_t>(16 * groups) * moe::kXRowBytes +
                        static_cast<size_t>(moe::kMfmaRows) * (red / 32);
    const int64_t slots = (mfma_experts + 7) / 8 * 8;
    if (d.mma == MOE_MMA_SCALED_FP4) return enqueue_mfma_fp4(d, gate_up, M, L, ws, groups, lds, lds1, slots, s);
    if (!gate_up && down4_fits(d))
      return launch(moe::down4_kernel, dim3(static_cast<unsigned>(slots * (rows / 256))), dim3(256), moe::kD4LdsBytes,
                    s, M);
    if (gate_up) {
      const dim3 g(static_cast<unsigned>(slots * ((rows + moe::kMfmaRows - 1) / moe::kMfmaRows)));
      if (groups == 1) return launch(moe::mfma_kernel<true, 1, false, false>, g, dim3(256), lds, s, M);
      if (groups == 2) return launch(moe::mfma_kernel<true, 2, false, false>, g, dim3(256), lds, s, M);
      return launch(moe::mfma_kernel<true, 4, false, false>, g, dim3(256), lds, s, M);
    }
    bool pair = rows % 32 == 0 && d.down_pairing != MOE_PAIRING_OFF;
    const int64_t grid2 = slots * ((rows + 2 * moe::kMfmaRows - 1) / (2 * moe::kMfmaRows));
    if (pair && d.down_pairing == MOE_PAIRING_AUTO) {
      const int resident = groups == 1   ? resident_workgroups(moe::mfma_kernel<false, 1, false, true>, lds)
                           : groups == 2 ? resident_workgroups(moe::mfma_kernel<false, 2, false, true>, lds)
                                         : resident_workgroups(moe::mfma_kernel<false, 4, false, true>, lds);
      pair = grid2 >= resident;
    }
    if (pair) {
      const dim3 g(static_cast<unsigned>(grid2));
      if (groups == 1) return launch(moe::mfma_kernel<false, 1, false, true>, g, dim3(256), lds, s, M);
      if (groups == 2) return launch(moe::mfma_kernel<false, 2, false, true>, g, dim3(256), lds, s, M);
      return launch(moe::mfma_kernel<false, 4, false, true>, g, dim3(256), lds, s, M);
    }
    const dim3 g(static_cast<unsigned>(slots * ((rows + moe::kMfmaRows - 1) / moe::kMfmaRows)));
    if (groups == 1) return launch(moe::mfma_kernel<false, 1, false, false>, g, dim3(256), lds1, s, M);
    if (groups == 2) return launch(moe::mfma_kernel<false, 2, false, false>, g, dim3(256), lds1, s, M);
    return launch(moe::mfma_kernel<false, 4, false, false>, g, dim3(256), lds1, s, M);
  }
  return hipSuccess;
}

// Prefill: the touched experts' weights, unpacked to bf16 in the workspace
// past the decode layout (w13 [E_l][2I][K], then w2 [E_l][K][I]).
struct PrefillLayout {
  size_t w13, w2, total;
};
PrefillLayout prefill_layout(const moe_mxfp4_desc& d) {
  PrefillLayout P;
  P.w13 = make_layout(d).total;
  P.w2 = align_up(P.w13 + static_cast<size_t>(d.E_local) * 2 * d.I * d.K * 2, 256);
  P.total = align_up(P.w2 + static_cast<size_t>(d.E_local) * d.K * d.I * 2, 256);
  return P;
}

hipError_t enqueue_unpack(const moe_mxfp4_desc& d, const uint8_t* w13p, const uint8_t* w13s, const uint8_t* w2p,
                          const uint8_t* w2s, const int32_t* counts, uint16_t* w13_out, uint16_t* w2_out,
                          hipStream_t s) {
  const int tiled = d.weight_layout == MOE_LAYOUT_TILE16;
  const int64_t b13 = static_cast<int64_t>(2) * d.I * (d.K / 32), b2 = static_cast<int64_t>(d.K) * (d.I / 32);
  MOE_TRY(launch(moe::unpack_kernel, dim3(static_cast<unsigned>((b13 + 255) / 256), d.E_local), dim3(256), 0, s, w13p,
                 w13s, 2 * d.I, d.K, tiled, counts, w13_out));
  return launch(moe::unpack_kernel, dim3(static_cast<unsigned>((b2 + 255) / 256), d.E_local), dim3(256), 0, s, w2p,
                w2s, d.K, d.I, tiled, counts, w2_out);
}

// The MFMA kernel on the unpacked weights for every touched expert (the plan
// of the prefill path lists them all).
hipError_t enqueue_mfma_bf16(const moe_mxfp4_desc& d, bool gate_up, moe::ExpertArgs M, const Layout& L, void* ws,
                             hipStream_t s) {
  const int64_t R = static_cast<int64_t>(d.T) * d.top_k;
  const int64_t experts = std::min<int64_t>(d.E_local, R);
  M.list = at<moe::WorkEntry>(ws, L.mfma_list);
  M.list_cap = d.E_local;
  const int64_t grid = std::max<int64_t>(1, (experts + 7) / 8 * 8 * ((M.rows + moe::kMfmaRows - 1) / moe::kMfmaRows));
  const int groups = d.T <= 32 ? 1 : (d.T <= 64 ? 2 : 4);
  const size_t lds = 2 * static_cast<size_t>(16 * groups) * moe::kXRowBytes +
                     static_cast<size_t>(gate_up ? 2 : 1) * moe::kMfmaRows * (M.red / 32);
  const dim3 g(static_cast<unsigned>(grid));
  if (gate_up) {
    if (groups == 1) return launch(moe::mfma_kernel<true, 1, true, false>, g, dim3(256), lds, s, M);
    if (groups == 2) return launch(moe::mfma_kernel<true, 2, true, false>, g, dim3(256), lds, s, M);
    return launch(moe::mfma_kernel<true, 4, true, false>, g, dim3(256), lds, s, M);
  }
  if (groups == 1) return launch(moe::mfma_kernel<false, 1, true, false>, g, dim3(256), lds, s, M);
  if (groups == 2) return launch(moe::mfma_kernel<false, 2, true, false>, g, dim3(256), lds, s, M);
  return launch(moe::mfma_kernel<false, 4, true, false>, g, dim3(256), lds, s, M);
}

// One projection in the decode regime.  Items: n_passes x tiles of
// 64/split rows (128/split for a paired down projection), where an expert
// with Te routes has ceil(Te / tp) passes, so n_passes
// <= (R + min(E_local, R) * (tp - 1)) / tp.  The persistent grid is the
// resident workgroup count, raised if needed so that no workgroup has more
// than kStreamMaxItems items, and never above the item bound.
struct StreamGrid {
  size_t lds;
  int64_t bound;  // items
  int64_t passes; // host bound on the plan's pass count
  int resident;
};

template <bool kGateUp, int kSplit, bool kPair, bool kSelf = false>
StreamGrid stream_grid(const moe_mxfp4_desc& d, const moe::StreamArgs& S) {
  StreamGrid G;
  G.lds = stream_lds_bytes(S.red, kGateUp || kPair, kSplit);
  if (kSelf) G.lds = std::max(G.lds, self_lds_bytes(d));
  const int64_t R = static_cast<int64_t>(d.T) * d.top_k;
  const int64_t tp = moe::kStreamPassTokens / kSplit;
  const int64_t passes = std::min<int64_t>(R, (R + tokens_bound(d) * (tp - 1)) / tp);
  const int item_rows = (kPair ? 128 : 64) / kSplit;
  G.passes = passes;
  G.bound = passes * ((S.rows + item_rows - 1) / item_rows);
  G.resident = resident_workgroups(moe::stream_kernel<kGateUp, kSplit, kPair, kSelf>, G.lds);
  return G;
}

template <bool kGateUp, int kSplit, bool kPair, bool kSelf = false>
hipError_t launch_stream(const StreamGrid& G, moe::StreamArgs S, hipStream_t s) {
  int64_t grid = std::max<int64_t>(G.resident > 0 ? G.resident : 1024,
                                   (G.bound + moe::kStreamMaxItems - 1) / moe::kStreamMaxItems);
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, G.bound));
  S.max_passes = static_cast<int>(G.passes);
  return launch(moe::stream_kernel<kGateUp, kSplit, kPair, kSelf>, dim3(static_cast<unsigned>(grid)), dim3(256), G.lds,
                s, S);
}

// The down projection runs in pairs of 16-row sets per wave (two weight loads
// per lane and step, like gate/up) when the rows allow it and, under
// MOE_PAIRING_AUTO, the paired items still fill every resident workgroup
// slot; otherwise (few touched experts) the unpaired items keep more of the
// chip streaming.
template <bool kGateUp, int kSplit>
hipError_t launch_stream_proj(const moe_mxfp4_desc& d, const moe::StreamArgs& S, hipStream_t s) {
  if (!kGateUp && S.rows % 32 == 0 && d.down_pairing != MOE_PAIRING_OFF) {
    const StreamGrid G = stream_grid<false, kSplit, true>(d, S);
    if (d.down_pairing == MOE_PAIRING_ON || G.bound >= G.resident) return launch_stream<false, kSplit, true>(G, S, s);
  }
  return launch_stream<kGateUp, kSplit, false>(stream_grid<kGateUp, kSplit, false>(d, S), S, s);
}

template <bool kGateUp>
hipError_t enqueue_stream(const moe_mxfp4_desc& d, int split, const moe::StreamArgs& S, hipStream_t s) {
  if (split == 4) return launch_stream_proj<kGateUp, 4>(d, S, s);
  if (split == 2) return launch_stream_proj<kGateUp, 2>(d, S, s);
  return launch_stream_proj<kGateUp, 1>(d, S, s);
}

// The gate/up launch that makes its own plan (S.self filled in).
hipError_t enqueue_stream_self(const moe_mxfp4_desc& d, int split, const moe::StreamArgs& S, hipStream_t s) {
  if (split == 4) return launch_stream<true, 4, false, true>(stream_grid<true, 4, false, true>(d, S), S, s);
  if (split == 2) return launch_stream<true, 2, false, true>(stream_grid<true, 2, false, true>(d, S), S, s);
  return launch_stream<true, 1, false, true>(stream_grid<true, 1, false, true>(d, S), S, s);
}

// Calls whose gate/up launch can make the plan itself: both projections in
// the stream regime (no GEMV / MFMA lists), at most kSelfRoutes routes (one
// wave buckets them) and kSelfTokens tokens.  Every workgroup routes the
// whole call, so above 16 tokens it pays only where a top-k is cheap: with
// at most 64 experts (the gpt-oss-20b shape at T = 32: 97.5 -> 95.9 us); with
// 128 (gpt-oss-120b, T = 32) the prologue took 8.5 us, as long as the plan
// launch it replaces.
bool self_plan_ok(const moe_mxfp4_desc& d) {
  const int split = stream_split(d);
  const int64_t R = static_cast<int64_t>(d.T) * d.top_k;
  return split > 0 && stream_fits(d.K, split) && stream_fits(d.I, down_split(d)) && d.T <= moe::kSelfTokens &&
         R <= moe::kSelfRoutes && (d.T <= 16 || (d.top_k <= 16 && d.E_global <= 64));
}

// LDS of the self-planning prologue (the kernel's layout).
size_t self_lds_bytes(const moe_mxfp4_desc& d) {
  const int R = d.T * d.top_k;
  return moe::kSelfLdsBase + (R > 64 ? 2 * 4 * static_cast<size_t>(moe::self_bucket_ints(d.E_local, R)) : 0);
}

moe::StreamArgs stream_args(const moe_mxfp4_desc& d, const Layout& L, void* ws) {
  moe::StreamArgs S{};
  S.passes = at<moe::PassEntry>(ws, L.passes);
  S.plan = at<Plan>(ws, L.plan);
  S.key = plan_key(d, false);
  S.E_local = d.E_local;
  S.R = d.T * d.top_k;
  S.act_kind = d.activation;
  S.alpha = d.swiglu_alpha;
  S.limit = d.swiglu_limit;
  S.tiled = d.weight_layout == MOE_LAYOUT_TILE16;
  S.top_k = d.top_k;
  return S;
}

// Bounds and plan key of the list kernels' arguments.
void set_list_bounds(const moe_mxfp4_desc& d, moe::ExpertArgs& A, bool prefill) {
  A.key = plan_key(d, prefill);
  A.T = d.T;
  A.R = d.T * d.top_k;
  A.list_cap = d.E_local;
}

// With `self` (a call that self_plan_ok() admits), the stream launch makes
// the plan from those routing inputs instead of reading one.
hipError_t enqueue_w13(const moe_mxfp4_desc& d, const uint16_t* x, const uint8_t* w13p, const uint8_t* w13s,
                       const uint16_t* b13, uint16_t* a, void* ws, hipStream_t s,
                       const moe::PlanArgs* self = nullptr) {
  const Layout L = make_layout(d);
  moe::ExpertArgs A{};
  A.in = x;
  A.in_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.K * 2);
  A.routes = at<int32_t>(ws, L.routes);
  A.top_k = d.top_k;
  A.wp = w13p;
  A.ws = w13s;
  A.bias = b13;
  A.plan = at<Plan>(ws, L.plan);
  A.red = d.K;
  A.rows = d.I;
  A.tiled = d.weight_layout == MOE_LAYOUT_TILE16;
  A.il = d.w13_order == MOE_W13_INTERLEAVED;
  A.a_out = a != nullptr ? a : at<uint16_t>(ws, L.a);
  A.act_kind = d.activation;
  A.alpha = d.swiglu_alpha;
  A.limit = d.swiglu_limit;
  set_list_bounds(d, A, false);
  const int split = stream_split(d);
  if (stream_fits(d.K, split)) {
    moe::StreamArgs S = stream_args(d, L, ws);
    S.in = x;
    S.in_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.K * 2);
    S.wp = w13p;
    S.ws = w13s;
    S.bias = b13;
    S.red = d.K;
    S.rows = d.I;
    S.tok_from_pass = 1;
    S.il = A.il;
    S.a_out = A.a_out;
    if (self != nullptr) {
      S.self = *self;
      return enqueue_stream_self(d, split, S, s);
    }
    return enqueue_stream<true>(d, split, S, s);
  }
  return enqueue_expert_pair(d, true, A, L, ws, s);
}

// Routing, bucketing and the gate/up projection of a decode call: one
// launch that plans for itself where the call admits it, else the plan
// kernel and then the gate/up launch.
hipError_t enqueue_front(const moe_mxfp4_desc& d, const float* logits, const int32_t* ids, const float* wts,
                         const uint16_t* x, const uint8_t* w13p, const uint8_t* w13s, const uint16_t* b13, void* ws,
                         hipStream_t s) {
  if (self_plan_ok(d)) {
    moe::PlanArgs P = full_plan_args(d, ws, false);
    if (logits != nullptr) {
      P.logits = logits;
    } else {
      P.ids_in = ids;
      P.w_in = wts;
    }
    return enqueue_w13(d, x, w13p, w13s, b13, nullptr, ws, s, &P);
  }
  hipError_t e = enqueue_plan(d, logits, ids, wts, ws, s);
  if (e == hipSuccess) e = enqueue_w13(d, x, w13p, w13s, b13, nullptr, ws, s);
  return e;
}

// Token sums: 1024 columns of a token per workgroup for small calls (several
// workgroups share a token), 4096 for large ones (fewer, longer workgroups).
hipError_t launch_combine(const moe_mxfp4_desc& d, const moe::CombineArgs& C, hipStream_t s) {
  if (d.T <= moe::kStreamMaxTokens)
    return launch(moe::combine_kernel<1>, dim3(d.T, (d.K + 1023) / 1024), dim3(256), 0, s, C);
  return launch(moe::combine_kernel<4>, dim3(d.T, (d.K + 4095) / 4096), dim3(256), 0, s, C);
}

// One-token calls whose down projection would run the stream kernel's 4-way
// split take token_down_kernel instead: the same bits in one launch, without
// the per-route rows and the combine launch (gpt-oss-120b T = 1: 24.3 ->
// 23.0 us per call).  Its LDS (the four padded intermediate rows) stays within
// 64 KB: at most 15 steps per slice, I <= 7680.
constexpr int kTokenDownMaxSteps = 15;
int token_down_steps(const moe_mxfp4_desc& d) { return steps_per_slice(d.I, 4); }
bool token_down_ok(const moe_mxfp4_desc& d) {
  return d.T >= 1 && d.T <= moe::kTokenMaxTokens && d.top_k <= moe::kTokenRoutes && down_split(d) == 4 && stream_fits(d.I, 4) && d.K % 16 == 0 &&
         token_down_steps(d) <= kTokenDownMaxSteps;
}

// The down projection, then either the per-token combine into out (bf16
// [T, K]) or, with out_routes, the per-route rows (fp32 [T*top_k, K]).
hipError_t enqueue_w2(const moe_mxfp4_desc& d, const uint16_t* a, const uint8_t* w2p, const uint8_t* w2s,
                      const uint16_t* b2, uint16_t* out, float* out_routes, void* ws, hipStream_t s) {
  const Layout L = make_layout(d);
  if (out_routes == nullptr && token_down_ok(d)) {
    moe::TokenDownArgs D{};
    D.a = a != nullptr ? a : at<uint16_t>(ws, L.a);
    D.a_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.top_k * d.I * 2);
    D.wp = w2p;
    D.ws = w2s;
    D.bias = b2;
    D.plan = at<Plan>(ws, L.plan);
    D.key = plan_key(d, false);
    D.ids = at<int32_t>(ws, L.ids);
    D.pos = at<int32_t>(ws, L.pos);
    D.weights = at<float>(ws, L.weights);
    D.out = out;
    D.T = d.T;
    D.K = d.K;
    D.I = d.I;
    D.E_local = d.E_local;
    D.offset = d.expert_offset;
    D.top_k = d.top_k;
    D.tiled = d.weight_layout == MOE_LAYOUT_TILE16;
    D.steps = token_down_steps(d);
    return launch(moe::token_down_kernel, dim3(d.K / 16, d.T), dim3(1024), moe::token_down_lds_bytes(D.steps), s, D);
  }
  moe::ExpertArgs A{};
  A.in = a != nullptr ? a : at<uint16_t>(ws, L.a);
  A.in_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.top_k * d.I * 2);
  A.routes = nullptr;
  A.top_k = d.top_k;
  A.wp = w2p;
  A.ws = w2s;
  A.bias = b2;
  A.plan = at<Plan>(ws, L.plan);
  A.red = d.I;
  A.rows = d.K;
  A.tiled = d.weight_layout == MOE_LAYOUT_TILE16;
  A.o_out = at<float>(ws, L.o);
  set_list_bounds(d, A, false);
  moe::CombineArgs C;
  C.o = at<float>(ws, L.o);
  C.pos = at<int32_t>(ws, L.pos);
  C.weights = at<float>(ws, L.weights);
  C.out = out;
  C.T = d.T;
  C.K = d.K;
  C.top_k = d.top_k;
  C.by_route = 0;
  const int split = down_split(d);
  const int R = d.T * d.top_k;
  if (stream_fits(d.I, split)) {
    C.by_route = 1;
    if (out_routes != nullptr) A.o_out = out_routes;  // rows by route, straight into the caller's buffer
    moe::StreamArgs S = stream_args(d, L, ws);
    S.in = A.in;
    S.in_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.top_k * d.I * 2);
    S.wp = w2p;
    S.ws = w2s;
    S.bias = b2;
    S.red = d.I;
    S.rows = d.K;
    S.tok_from_pass = 0;
    S.o_by_route = 1;
    S.o_out = A.o_out;
    if (split != stream_split(d)) {
      S.passes = at<moe::PassEntry>(ws, L.passes2);
      S.second_list = 1;
    }
    MOE_TRY(enqueue_stream<false>(d, split, S, s));
  } else {
    MOE_TRY(enqueue_expert_pair(d, false, A, L, ws, s));
  }
  if (out_routes != nullptr)
    return launch(moe::route_rows_kernel, dim3((d.K / 4 + 255) / 256, R), dim3(256), 0, s, static_cast<const float*>(C.o),
                  static_cast<const int32_t*>(C.pos), out_routes, R, d.K, C.by_route);
  return launch_combine(d, C, s);
}

// The workspace of moe_mxfp4_decode_noalloc: one array per GPU in the code
// object's device memory, held until the process ends.  Host code never uses
// the array's name as an address (it names a host-side stand-in); the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.  No part needs clearing between calls: each call's plan kernel
// writes every field the later kernels read.
static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up on the first
// call there (nullptr if the lookup fails).
void* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  static std::mutex lock;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  const std::lock_guard<std::mutex> guard(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
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
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(out) || !aligned16(w13_scales) ||
      !aligned16(w2_scales) || !aligned16(w13_bias) || !aligned16(w2_bias))
    return MOE_ERR_ALIGN;
  if ((st = check_workspace(d, workspace, workspace_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = enqueue_front(d, router_logits, topk_ids, topk_weights, x, w13_packed, w13_scales, w13_bias,
                               workspace, s);
  if (e == hipSuccess) e = enqueue_w2(d, nullptr, w2_packed, w2_scales, w2_bias, out, nullptr, workspace, s);
  return hip_status(e);
}

int moe_mxfp4_decode_noalloc(const moe_mxfp4_desc* desc, const uint16_t* x, const float* router_logits,
                             const int32_t* topk_ids, const float* topk_weights, const uint8_t* w13_packed,
                             const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_packed,
                             const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* out, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const moe_mxfp4_desc& d = *desc;
  if ((st = check_routing(d, router_logits, topk_ids, topk_weights)) != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  if (!x || !w13_packed || !w13_scales || !w2_packed || !w2_scales || !out) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(out) || !aligned16(w13_scales) ||
      !aligned16(w2_scales) || !aligned16(w13_bias) || !aligned16(w2_bias))
    return MOE_ERR_ALIGN;
  if (make_layout(d).total > MOE_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return MOE_ERR_HIP;
  return moe_mxfp4_decode(desc, x, router_logits, topk_ids, topk_weights, w13_packed, w13_scales, w13_bias,
                          w2_packed, w2_scales, w2_bias, out, ws, MOE_SCRATCH_BYTES, stream);
}

int moe_mxfp4_decode_routes(const moe_mxfp4_desc* desc, const uint16_t* x, const float* router_logits,
                            const int32_t* topk_ids, const float* topk_weights, const uint8_t* w13_packed,
                            const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_packed,
                            const uint8_t* w2_scales, const uint16_t* w2_bias, float* out_routes, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const moe_mxfp4_desc& d = *desc;
  if ((st = check_routing(d, router_logits, topk_ids, topk_weights)) != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  if (!x || !w13_packed || !w13_scales || !w2_packed || !w2_scales || !out_routes) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(out_routes) ||
      !aligned16(w13_scales) || !aligned16(w2_scales) || !aligned16(w13_bias) || !aligned16(w2_bias))
    return MOE_ERR_ALIGN;
  if ((st = check_workspace(d, workspace, workspace_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = enqueue_front(d, router_logits, topk_ids, topk_weights, x, w13_packed, w13_scales, w13_bias,
                               workspace, s);
  if (e == hipSuccess) e = enqueue_w2(d, nullptr, w2_packed, w2_scales, w2_bias, nullptr, out_routes, workspace, s);
  return hip_status(e);
}

int moe_mxfp4_prefill_workspace_bytes(const moe_mxfp4_desc* desc, size_t* bytes) {
  const int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_NULL;
  *bytes = prefill_layout(*desc).total;
  return MOE_OK;
}

int moe_mxfp4_prefill(const moe_mxfp4_desc* desc, const uint16_t* x, const float* router_logits,
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
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(out) || !aligned16(w13_scales) ||
      !aligned16(w2_scales) || !aligned16(w13_bias) || !aligned16(w2_bias))
    return MOE_ERR_ALIGN;
  if (workspace == nullptr) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  const PrefillLayout PL = prefill_layout(d);
  if (workspace_bytes < PL.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Layout L = make_layout(d);
  uint16_t* w13u = at<uint16_t>(workspace, PL.w13);
  uint16_t* w2u = at<uint16_t>(workspace, PL.w2);
  hipError_t e = enqueue_plan(d, router_logits, topk_ids, topk_weights, workspace, s, true);
  if (e == hipSuccess)
    e = enqueue_unpack(d, w13_packed, w13_scales, w2_packed, w2_scales, at<int32_t>(workspace, L.counts), w13u, w2u, s);
  moe::ExpertArgs A{};
  A.in = x;
  A.in_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.K * 2);
  A.routes = at<int32_t>(workspace, L.routes);
  A.top_k = d.top_k;
  A.ws = w13_scales;
  A.bias = w13_bias;
  A.plan = at<Plan>(workspace, L.plan);
  A.red = d.K;
  A.rows = d.I;
  A.il = d.w13_order == MOE_W13_INTERLEAVED;
  A.wbf = w13u;
  A.a_out = at<uint16_t>(workspace, L.a);
  A.act_kind = d.activation;
  A.alpha = d.swiglu_alpha;
  A.limit = d.swiglu_limit;
  set_list_bounds(d, A, true);
  if (e == hipSuccess) e = enqueue_mfma_bf16(d, true, A, L, workspace, s);
  moe::ExpertArgs B{};
  B.in = A.a_out;
  B.in_bytes = static_cast<uint32_t>(static_cast<size_t>(d.T) * d.top_k * d.I * 2);
  B.top_k = d.top_k;
  B.ws = w2_scales;
  B.bias = w2_bias;
  B.plan = A.plan;
  B.red = d.I;
  B.rows = d.K;
  B.wbf = w2u;
  B.o_out = at<float>(workspace, L.o);
  set_list_bounds(d, B, true);
  if (e == hipSuccess) e = enqueue_mfma_bf16(d, false, B, L, workspace, s);
  moe::CombineArgs C;
  C.o = B.o_out;
  C.pos = at<int32_t>(workspace, L.pos);
  C.weights = at<float>(workspace, L.weights);
  C.out = out;
  C.T = d.T;
  C.K = d.K;
  C.top_k = d.top_k;
  C.by_route = 0;
  if (e == hipSuccess) e = launch_combine(d, C, s);
  return hip_status(e);
}

int moe_mxfp4_unpack(const moe_mxfp4_desc* desc, const uint8_t* w13_packed, const uint8_t* w13_scales,
                     const uint8_t* w2_packed, const uint8_t* w2_scales, uint16_t* w13_out, uint16_t* w2_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!w13_packed || !w13_scales || !w2_packed || !w2_scales || !w13_out || !w2_out) return MOE_ERR_NULL;
  if (!aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(w13_out) || !aligned16(w2_out))
    return MOE_ERR_ALIGN;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  return hip_status(enqueue_unpack(*desc, w13_packed, w13_scales, w2_packed, w2_scales,
                                   at<int32_t>(workspace, make_layout(*desc).counts), w13_out, w2_out,
                                   static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_plan(const moe_mxfp4_desc* desc, const float* router_logits, const int32_t* topk_ids,
                   const float* topk_weights, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_routing(*desc, router_logits, topk_ids, topk_weights)) != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  return hip_status(
      enqueue_plan(*desc, router_logits, topk_ids, topk_weights, workspace, static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_gate_up(const moe_mxfp4_desc* desc, const uint16_t* x, const uint8_t* w13_packed,
                      const uint8_t* w13_scales, const uint16_t* w13_bias, uint16_t* a, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!x || !w13_packed || !w13_scales) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_packed) || !aligned16(w13_scales) || !aligned16(w13_bias) || !aligned16(a))
    return MOE_ERR_ALIGN;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  return hip_status(
      enqueue_w13(*desc, x, w13_packed, w13_scales, w13_bias, a, workspace, static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_down(const moe_mxfp4_desc* desc, const uint16_t* a, const uint8_t* w2_packed,
                   const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!w2_packed || !w2_scales || !out) return MOE_ERR_NULL;
  if (!aligned16(a) || !aligned16(w2_packed) || !aligned16(w2_scales) || !aligned16(w2_bias) || !aligned16(out))
    return MOE_ERR_ALIGN;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  return hip_status(
      enqueue_w2(*desc, a, w2_packed, w2_scales, w2_bias, out, nullptr, workspace, static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_down_routes(const moe_mxfp4_desc* desc, const uint16_t* a, const uint8_t* w2_packed,
                          const uint8_t* w2_scales, const uint16_t* w2_bias, float* out_routes, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!w2_packed || !w2_scales || !out_routes) return MOE_ERR_NULL;
  if (!aligned16(a) || !aligned16(w2_packed) || !aligned16(w2_scales) || !aligned16(w2_bias) || !aligned16(out_routes))
    return MOE_ERR_ALIGN;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  return hip_status(enqueue_w2(*desc, a, w2_packed, w2_scales, w2_bias, nullptr, out_routes, workspace,
                              static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_route(const moe_mxfp4_desc* desc, const float* router_logits, int32_t* topk_ids,
                    float* topk_weights, void* stream) {
  const int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->E_global > moe::kMaxGlobalExpertsRouted) return MOE_ERR_SHAPE;
  if (desc->T == 0) return MOE_OK;
  if (!router_logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  return hip_status(launch(moe::route_topk_kernel, dim3((desc->T + 3) / 4), dim3(256), 0,
                           static_cast<hipStream_t>(stream), router_logits, desc->T, desc->E_global, desc->top_k,
                           desc->scoring, topk_ids, topk_weights));
}

int moe_mxfp4_bucket(const moe_mxfp4_desc* desc, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                     int32_t* routes, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !routes) return MOE_ERR_NULL;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  return hip_status(
      enqueue_bucket_hook(*desc, topk_ids, workspace, static_cast<hipStream_t>(stream), counts, offsets, routes));
}

int moe_mxfp4_plan_read(const moe_mxfp4_desc* desc, const void* workspace, size_t workspace_bytes, int32_t* topk_ids,
                        float* topk_weights, int32_t* counts, int32_t* offsets, int32_t* routes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if ((st = check_workspace(*desc, workspace, workspace_bytes)) != MOE_OK) return st;
  const moe_mxfp4_desc& d = *desc;
  const Layout L = make_layout(d);
  void* ws = const_cast<void*>(workspace);
  const int R = d.T * d.top_k;
  const int n = std::max(R, d.E_local + 1);
  return hip_status(launch(moe::plan_read_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                           at<const Plan>(ws, L.plan), at<const int32_t>(ws, L.ids), at<const float>(ws, L.weights),
                           at<const int32_t>(ws, L.counts), at<const int32_t>(ws, L.offsets),
                           at<const int32_t>(ws, L.routes), R, d.E_local, topk_ids, topk_weights, counts, offsets,
                           routes));
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
  return hip_status(launch(moe::dequant_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), packed, scales, n_blocks,
                           out_dtype == MOE_DTYPE_BF16 ? 1 : 0, out));
}

int moe_mxfp4_encode(const void* in, int32_t in_dtype, int64_t rows, int64_t cols, int32_t rule, uint8_t* packed,
                     uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return MOE_ERR_SHAPE;
  if (in_dtype != MOE_DTYPE_F32 && in_dtype != MOE_DTYPE_BF16) return MOE_ERR_MODE;
  if (rule != MOE_ENCODE_OCP && rule != MOE_ENCODE_QUARK) return MOE_ERR_MODE;
  const int64_t n_blocks = rows * (cols / 32);
  if (n_blocks == 0) return MOE_OK;
  if (!in || !packed || !scales) return MOE_ERR_NULL;
  if (!aligned16(in) || !aligned16(packed)) return MOE_ERR_ALIGN;
  const int64_t grid = (n_blocks * 4 + 256 * moe::kEncodePer - 1) / (256 * moe::kEncodePer);
  if (grid > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  const int quark = rule == MOE_ENCODE_QUARK ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (in_dtype == MOE_DTYPE_BF16)
    return hip_status(launch(moe::encode_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, in, n_blocks,
                             quark, packed, scales));
  return hip_status(launch(moe::encode_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, in, n_blocks,
                           quark, packed, scales));
}

int moe_mxfp4_tile_weights(uint8_t* packed, int64_t rows, int64_t cols, int32_t inverse, void* stream) {
  if (rows < 0 || rows % 16 != 0 || cols < 32 || cols > moe::kMaxDim || cols % 32 != 0) return MOE_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return MOE_ERR_MODE;
  const int64_t groups = rows / 16;
  if (groups == 0) return MOE_OK;
  if (packed == nullptr) return MOE_ERR_NULL;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  if (groups > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  return hip_status(launch(moe::tile_kernel, dim3(static_cast<unsigned>(groups)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), packed, groups, static_cast<int>(cols / 32), inverse));
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
