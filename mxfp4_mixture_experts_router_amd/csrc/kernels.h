// Kernel declarations, the device plan layout, and the size limits the host
// checks before launching.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

constexpr int kRouteMaxPerLane = 16;                    // E_global <= 1024 in logits mode
constexpr int kMaxGlobalExpertsRouted = 64 * kRouteMaxPerLane;
constexpr int kMaxTopK = 64;
constexpr int kPlanWaves = 16;                          // waves of the planning workgroup
constexpr int kMaxLocalExperts = 512;
constexpr int kMaxDim = 8192;                           // K and I
constexpr int kFusedRouteTokens = 64;                   // T up to this (and E_global <= 256): routing runs inside the plan kernel

// Regime per touched expert, decided on the device from its route count:
// up to kGemvMaxTokens routes -> VALU GEMV (gemv_kernel); more -> bf16 MFMA
// (mfma_kernel), 4 waves x 16 rows per work item, tokens in groups of 16.
constexpr int kGemvMaxTokens = 2;
constexpr int kMfmaRows = 64;
constexpr int kChunkBlocks = 4;                         // MX blocks (of 32 values) per MFMA step
constexpr int kXRowBytes = kChunkBlocks * 64 + 16;      // LDS row of one staged chunk, padded

// One touched local expert, written by the plan kernel into the list of its
// regime.
struct WorkEntry {
  int32_t e;        // local expert
  int32_t p0;       // first route position of the expert in plan order
  int32_t Te;       // routes of the expert
  int32_t tok[kGemvMaxTokens];  // token of the first routes (GEMV entries)
  int32_t pad[8 - 3 - kGemvMaxTokens];
};
static_assert(sizeof(WorkEntry) == 32, "WorkEntry is 32 bytes");

// Stream regime (T <= kStreamMaxTokens, or few routes per expert; the host
// decides): one persistent kernel per projection walks work items (expert
// pass x row tile).  A pass is up to kStreamPassTokens routes of one expert;
// the plan kernel lists the passes of every touched expert in expert order.
constexpr int kStreamMaxTokens = 64;
constexpr int kStreamPassTokens = 16;
// Calls of at most kSelfRoutes routes and kSelfTokens tokens whose two
// projections both run in the stream regime skip the plan kernel: the gate/up
// launch routes and buckets them itself (stream_kernel's kSelf form).  Above
// 16 tokens that needs the four-tokens-per-wave router (top_k <= 16,
// E_global <= 256).  LDS of the prologue: kSelfLdsBase bytes, then (above 64
// routes) two sets of the chunked bucketing's arrays of self_bucket_ints()
// ints each.
constexpr int kSelfRoutes = 128;
constexpr int kSelfTokens = 32;
constexpr int kSelfLdsBase = 2048 + kSelfRoutes * 64;
__host__ __device__ inline int self_bucket_ints(int E_local, int R) { return (4 * E_local + 2 * R + 1 + 3) & ~3; }

struct PassEntry {
  int32_t e;        // local expert
  int32_t nt;       // routes in this pass (1..tokens per pass)
  int32_t p;        // plan position of the pass's first route
  int32_t pad0;
  uint16_t rte[kStreamPassTokens];  // route index t*top_k + j of each route of the pass; slots >= nt unset
  int32_t pad1[4];
};
static_assert(sizeof(PassEntry) == 64, "PassEntry is 64 bytes");

// Header of the device plan, at the start of the workspace.  `key` is the
// host's key of the descriptor the plan was made for (plan_key() in the
// host code); the expert kernels leave a plan with another key alone, so a
// workspace that holds no plan for this call (never planned, or planned for
// another shape) gives no output instead of out-of-range indices.
struct Plan {
  int32_t n_touched;   // local experts with at least one route
  int32_t R_local;     // local routes
  int32_t n_gemv;      // experts in the GEMV list
  int32_t n_mfma;      // experts in the MFMA list
  int32_t n_passes;    // entries of the pass list (decode regime)
  uint32_t key;        // descriptor key of the call that wrote this plan
  int32_t n_passes2;   // entries of the second pass list (another pass size), or 0
  int32_t pad[57];
};

struct PlanArgs {
  const float* logits;     // router-logits mode, or nullptr
  const int32_t* ids_in;   // ids (caller's, or written by route_topk_kernel), used when logits == nullptr
  const float* w_in;       // caller's weights to copy into the workspace (ids mode), or nullptr
  int T, top_k, E_global, E_local, offset, scoring;
  int mfma_enabled;        // the MFMA kernels run for this call (T > kGemvMaxTokens); else all experts go to GEMV
  int gemv_max;            // with mfma_enabled: experts with more routes than this go to the MFMA list
  int lists;               // build the GEMV / MFMA work lists (some projection uses the list kernels)
  int32_t* ids_ws;         // [R] routed ids (logits mode)
  float* weights_ws;       // [R] routing weights
  int32_t* counts;         // [E_l]
  int32_t* offsets;        // [E_l + 1]
  int32_t* routes;         // [R] route index by plan position
  int32_t* pos;            // [R] plan position by route index, -1 if not local
  WorkEntry* gemv_list;    // [E_l]
  WorkEntry* mfma_list;    // [E_l]
  PassEntry* passes;       // pass list, or nullptr
  int pass_shift;          // routes per pass = 1 << pass_shift (<= kStreamPassTokens) when passes != nullptr
  PassEntry* passes2;      // a second pass list, cut at 1 << pass_shift2 routes, or nullptr
  int pass_shift2;
  Plan* plan;
  uint32_t key;            // written to plan->key
  int32_t* routes_out;     // bucket hook: copy of routes padded with -1, or nullptr
};

// Packed weight rows are in the row layout, or tiled: in each group of 16
// rows, block b of row r at byte 256*b + 16*r of the group.  Either way a
// lane's 16-byte block b of row n is at row_offset(n) + b * block_stride.
__device__ __forceinline__ uint32_t row_offset(int n, uint32_t row_bytes, int tiled) {
  return tiled ? static_cast<uint32_t>(n & ~15) * row_bytes + 16u * static_cast<uint32_t>(n & 15)
               : static_cast<uint32_t>(n) * row_bytes;
}
__device__ __forceinline__ uint32_t block_stride(int tiled) { return tiled ? 256u : 16u; }

// Stored w13 row of gate row n and of up row n (rows = I row pairs per
// expert): [gate; up] puts them at n and rows + n, the interleaved order at
// 2n and 2n + 1 ("MXFP4 MoE decode kernels", Beyond gpt-oss; scales and b13
// follow the same row order).
__device__ __forceinline__ int gate_row(int n, int il) { return il ? 2 * n : n; }
__device__ __forceinline__ int up_row(int n, int rows, int il) { return il ? 2 * n + 1 : rows + n; }

struct ExpertArgs {
  const uint16_t* in;      // gate/up: x [T, K]; down: a [R, I]  (bf16)
  uint32_t in_bytes;       // size of `in` (MFMA kernel: out-of-range loads read zeros)
  const int32_t* routes;   // gate/up: activation row of position p is routes[p] / top_k; down: nullptr (row p)
  int top_k;
  const uint8_t* wp;       // packed weights
  const uint8_t* ws;       // scales
  const uint16_t* bias;    // bf16 bias or nullptr
  const WorkEntry* list;   // the kernel's expert list
  int list_cap;            // entries the list has room for (E_local)
  const Plan* plan;
  uint32_t key;            // the plan is used only when plan->key == key
  int T, R;                // tokens, routes (T * top_k): bounds of every plan-derived index
  int red;                 // reduction length: K (gate/up) or I (down)
  int rows;                // output rows per expert: I row pairs (gate/up) or K (down)
  int tiled;               // packed weights in the tiled layout
  int il;                  // gate/up: w13 rows interleaved (gate_row / up_row)
  const uint16_t* wbf;     // prefill: the weights unpacked to bf16 [E_l][rows_e][red] (MFMA kernel), else nullptr
  const int32_t* in_scale; // scaled-FP4 MFMA kernel: per activation row, E8M0 of the hi (byte 0) and lo (byte 1) parts
  uint32_t in_stride;      // scaled-FP4 MFMA kernel: bytes per split activation row (ceil(red / 128) * 256)
  uint16_t* a_out;         // gate/up output [R, I] bf16
  float* o_out;            // down output [R, K] fp32
  int act_kind;
  float alpha, limit;
};

struct CombineArgs {
  const float* o;          // per-route down projections [R, K] fp32, row = plan position or route
  const int32_t* pos;      // plan position of each route, -1 when not local; values outside [0, T*top_k) are skipped
  const float* weights;
  uint16_t* out;
  int T, K, top_k;
  int by_route;            // o rows indexed by route: their loads need not wait for pos
};

// Persistent decode-regime kernel: workgroup b of P takes items b, b+P, ...
// of the n_passes x tiles items; item = (pass, tile of 64/kSplit rows).
struct StreamArgs {
  const uint16_t* in;        // gate/up: x [T, K]; down: a [R, I]  (bf16)
  uint32_t in_bytes;         // size of `in` (out-of-range loads read zeros)
  const uint8_t* wp;         // packed weights [E_l][rows_e][red/2]
  const uint8_t* ws;         // scales [E_l][rows_e][red/32]
  const uint16_t* bias;      // [E_l][rows_e] bf16, or nullptr
  const PassEntry* passes;
  const Plan* plan;
  uint32_t key;              // the plan is used only when plan->key == key
  int max_passes;            // host bound on the plan's pass count (entries the pass list holds)
  int second_list;           // 1: `passes` is the plan's second pass list (count n_passes2)
  int E_local, R;            // bounds of the pass entries' expert, position and route fields
  int red;                   // reduction length: K (gate/up) or I (down)
  int rows;                  // output rows per expert: I row pairs (gate/up) or K (down)
  int tok_from_pass;         // 1: activation row = token of the entry's route (gate/up); 0: row = plan position (down)
  int top_k;
  int o_by_route;            // down: o rows indexed by route (t*top_k + j) instead of plan position
  int tiled;                 // packed weights in the tiled layout
  int il;                    // gate/up: w13 rows interleaved (gate_row / up_row)
  uint16_t* a_out;           // gate/up output [R, I] bf16
  float* o_out;              // down output [R, K] fp32
  int act_kind;
  float alpha, limit;
  PlanArgs self;             // kSelf: the plan this launch makes (routing inputs, workspace outputs)
};


__global__ void route_topk_kernel(const float* logits, int T, int E, int k, int scoring, int32_t* ids,
                                  float* weights);
__global__ void plan_kernel(PlanArgs P);
// GEMV regime: kLanesPerRow lanes stream one row (or [gate; up] row pair);
// a workgroup of 256 lanes covers 256 / kLanesPerRow rows of one expert.
template <bool kGateUp, int kLanesPerRow>
__global__ void gemv_kernel(ExpertArgs A);
// MFMA regime: 64 rows of one expert per workgroup (128 with kPair, the down
// projection in pairs of 16-row sets), kGroups groups of 16 tokens per pass;
// kBf16W reads the bf16-unpacked weights (prefill) instead of decoding MXFP4.
template <bool kGateUp, int kGroups, bool kBf16W, bool kPair>
__global__ void mfma_kernel(ExpertArgs A);
// The down projection of the MFMA regime with four 16-row weight sets per
// wave (256 rows per workgroup), up to 64 routes per pass, the intermediate
// rows staged by direct buffer->LDS loads: same list, same results as
// mfma_kernel<false, ...>; for I a multiple of 128 and K of 256.
constexpr int kD4ScaleSlots = 3;                // per-wave LDS ring of step scales
constexpr int kD4LdsBytes = 3 * 64 * 256 + 4 * kD4ScaleSlots * 256;
__global__ void down4_kernel(ExpertArgs A);

// Scaled-FP4 form of the MFMA regime.  Activations are first split, row by
// row, into two E4M3 parts with one E8M0 scale each (hi = the row rounded to
// E4M3 under a scale set by its largest magnitude, lo = the remainder
// rounded the same way), stored per 128-value chunk as [hi 128 B | lo 128 B]
// (mx8_split_kernel).  mfma_fp4_kernel then feeds the packed E2M1 weight
// blocks and their E8M0 scales to v_mfma_scale_f32_16x16x128_f8f6f4 without
// decoding them, two MFMAs (hi, lo) per 16-row set, 16 tokens and 128 values.
struct SplitArgs {
  const uint16_t* in;      // bf16 rows [rows][L]
  int rows;                // rows to split (the bound when rows_from_plan)
  int L;                   // values per row, multiple of 32
  int rows_from_plan;      // 1: split only plan->R_local rows (plan order, down input)
  const Plan* plan;
  uint32_t key;
  uint8_t* out;            // [rows][ceil(L / 128)][hi 128 B | lo 128 B]
  int32_t* scales;         // [rows]: E8M0 of hi | E8M0 of lo << 8
};
__global__ void mx8_split_kernel(SplitArgs A);
template <bool kGateUp, int kGroups, bool kPair>
__global__ void mfma_fp4_kernel(ExpertArgs A);
// Prefill unpack: packed [E_l][rows][cols/2] (row or tiled layout) + scales
// -> bf16 [E_l][rows][cols] in the row layout, for the experts with
// counts[e] > 0 (all when counts is nullptr); grid (ceil(rows * cols/32 / 256), E_l).
__global__ void unpack_kernel(const uint8_t* packed, const uint8_t* scales, int rows, int cols, int tiled,
                              const int32_t* counts, uint16_t* out);
// Decode regime: kSplit waves share one 16-row sub-tile and split the
// reduction (kSplit = 4, 2 or 1 for up to 4, 8 or 16 routes per pass); with
// kPair (down projection, rows % 32 == 0) a wave's sub-tile is 32 rows; with
// kSelf (gate/up, at most kSelfRoutes routes) the launch makes the plan itself.
template <bool kGateUp, int kSplit, bool kPair, bool kSelf = false>
__global__ void stream_kernel(StreamArgs A);
constexpr int kStreamRing = 4;   // steps (4 MX blocks per lane) in flight per wave
constexpr int kStreamMaxItems = 32;  // items per workgroup (their entries live in LDS)
// Token sums of the per-route rows; a workgroup takes 1024 * kCols columns of
// one token (grid: T x column blocks).
template <int kCols>
__global__ void combine_kernel(CombineArgs A);
// Calls of T <= kTokenMaxTokens tokens with top_k <= kTokenRoutes whose down
// projection runs the stream kernel's 4-way split: the down projection of
// every local route and the token sums in one launch of K / 16 x T
// workgroups (16 output rows of one token each), 16 waves = kTokenRoutes
// route slots x 4 reduction slices.  Same MFMA sequence, slice order, bias
// add and combine arithmetic as stream_kernel<false, 4, *> followed by
// combine_kernel, so the same bits.
constexpr int kTokenRoutes = 4;
// The kernel takes any T (one token per grid row); the host uses it for one
// token only: at gpt-oss-120b T = 2 / 4 it measured 36.3 / 53.5 us per call
// against 34.1 / 50.1 us for the stream kernel and the combine (a token's
// workgroups hold one route slot per wave, so experts shared by several
// tokens are streamed once per token, and K / 16 x T workgroups of 16 waves
// fill the chip in fewer, longer rounds).
constexpr int kTokenMaxTokens = 1;
struct TokenDownArgs {
  const uint16_t* a;        // intermediate rows [R, I] bf16, row = plan position
  uint32_t a_bytes;
  const uint8_t* wp;        // w2 packed [E_l][K][I/2]
  const uint8_t* ws;        // w2 scales [E_l][K][I/32]
  const uint16_t* bias;     // b2 [E_l][K] bf16, or nullptr
  const Plan* plan;
  uint32_t key;             // the plan is used only when plan->key == key
  const int32_t* ids;       // the plan's routing: global expert id of route j
  const int32_t* pos;       // plan position of route j, -1 when not local
  const float* weights;     // routing weight of route j
  uint16_t* out;            // [T, K] bf16
  int T, K, I, E_local, offset, top_k, tiled;
  int steps;                // steps (128 reduction values) per slice: ceil(ceil(I / 128) / 4)
};
__global__ void token_down_kernel(TokenDownArgs A);
// LDS of token_down_kernel: the kTokenRoutes intermediate rows, each padded to
// 4 * steps * 256 bytes, then the 16 waves' 16 row sums.
inline size_t token_down_lds_bytes(int steps) {
  return static_cast<size_t>(kTokenRoutes) * 4 * steps * 256 + 16 * 16 * sizeof(float);
}
// Per-route output rows [R, K] fp32: rows of routes outside the slice become
// zeros; with in_place == 0 the others are copied from o (plan order) to
// their route's row.
__global__ void route_rows_kernel(const float* o, const int32_t* pos, float* out, int R, int K, int in_place);
// Copy of a plan's routing and bucketing (test hook): ids/weights [R], counts
// [E_l], offsets [E_l + 1], routes [R] padded with -1 past the local routes;
// null outputs are skipped.  One workgroup of 256 threads per 256 routes or experts.
__global__ void plan_read_kernel(const Plan* plan, const int32_t* ids_ws, const float* weights_ws,
                                 const int32_t* counts_ws, const int32_t* offsets_ws, const int32_t* routes_ws, int R,
                                 int E_l, int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                                 int32_t* routes);
// In-place row layout <-> tiled layout, one workgroup per 16-row group.
__global__ void tile_kernel(uint8_t* packed, int64_t groups, int blocks, int inverse);
// MXFP4 encoder, four lanes per 32-value block (bf16 or fp32 input); each
// thread takes kEncodePer lane slots one grid width apart.
constexpr int kEncodePer = 4;
template <bool kBf16>
__global__ void encode_kernel(const void* in, int64_t n_blocks, int quark, uint8_t* packed, uint8_t* scales);
__global__ void dequant_kernel(const uint8_t* packed, const uint8_t* scales, int64_t n_blocks, int out_bf16,
                               void* out);

}  // namespace moe
