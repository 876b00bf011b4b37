// Kernel declarations and the size limits the host checks before launching.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

constexpr int kRouteMaxPerLane = 16;                    // E_global <= 1024 in logits mode
constexpr int kMaxGlobalExpertsRouted = 64 * kRouteMaxPerLane;
constexpr int kMaxTopK = 64;
constexpr int kBucketSegments = 16;                     // waves of the bucketing workgroup
constexpr int kMaxLocalExperts = 512;
constexpr int kMaxDim = 8192;                           // K and I (4 staged rows of bf16 fit 64 KB of LDS)

// Rows per expert-kernel work item: 16 lane-groups of 16 lanes each own one
// row (w2) or one [gate; up] row pair (w13).
constexpr int kRowsPerTile = 16;
// Tokens whose activations are staged in LDS at once by the GEMV kernels.
constexpr int kGemvTokens = 4;

__global__ void route_topk_kernel(const float* logits, int T, int E, int k, int scoring, int32_t* ids,
                                  float* weights);
__global__ void bucket_kernel(const int32_t* ids, int R, int E_l, int offset, int32_t* counts,
                              int32_t* offsets, int32_t* routes, int32_t* pos, int32_t* touched,
                              Plan* plan, int32_t* routes_out, const float* w_in, float* w_out);

struct W13Args {
  const uint16_t* x;
  const uint8_t* w13p;
  const uint8_t* w13s;
  const uint16_t* b13;
  const int32_t* offsets;
  const int32_t* routes;
  const int32_t* touched;
  const Plan* plan;
  uint16_t* a;
  int K, I, top_k, act;
  float alpha, limit;
};

struct W2Args {
  const uint16_t* a;
  const uint8_t* w2p;
  const uint8_t* w2s;
  const uint16_t* b2;
  const int32_t* offsets;
  const int32_t* touched;
  const Plan* plan;
  float* o;      // [R, K] fp32 per-route output
  int K, I;
};

struct CombineArgs {
  const float* o;
  const int32_t* pos;
  const float* weights;
  uint16_t* out;
  int T, K, top_k;
};

__global__ void w13_gemv_kernel(W13Args args);
__global__ void w2_gemv_kernel(W2Args args);
__global__ void combine_kernel(CombineArgs args);
__global__ void dequant_kernel(const uint8_t* packed, const uint8_t* scales, int64_t n_blocks, int out_bf16,
                               void* out);

}  // namespace moe
