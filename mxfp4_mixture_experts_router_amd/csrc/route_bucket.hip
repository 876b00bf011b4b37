// Router top-k and token-to-expert bucketing kernels.
//
// Routing: "MXFP4 MoE decode kernels", At a glance / Parity (gpt-oss top-4
// softmax routing) and "GLM-5.3-Flash on Gaudi 2", Why (top-8 sigmoid
// scoring); ids are int32 ("GLM-5.2 and GLM-5.3 (744B) in MXFP4 on Gaudi 2",
// Why it needed a port, item 4).  Selection is on the raw logits (softmax and
// sigmoid are monotone), logit descending, ties to the lower expert id.
//
// Bucketing: "MXFP4 MoE decode kernels", Design, Routing inside the kernel:
// routes are counting-sorted by local expert and routes to other expert-
// parallel ranks are skipped.  The sort here is stable (ascending route index
// inside each expert) and uses no atomics outside LDS histograms, so the
// permutation is unique and reproducible.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// One wave per token.  Each lane keeps up to kRouteMaxPerLane logits in
// registers (E_global <= 64 * kRouteMaxPerLane), and the k winners are found
// by k rounds of a wave-wide arg-max.
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int scoring, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  const float* row = logits + static_cast<size_t>(t) * E;

  float v[kRouteMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int idx = lane + 64 * i;
    v[i] = idx < E ? row[idx] : 0.0f;
    if (idx >= E) taken |= 1u << i;
  }

  int my_id = 0;
  float my_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    float best = -__builtin_inff();
    int bid = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      const int idx = lane + 64 * i;
      const bool free = !((taken >> i) & 1u);
      if (free && (v[i] > best || (v[i] == best && idx < bid))) {
        best = v[i];
        bid = idx;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bid, off);
      if (ob > best || (ob == best && oi < bid)) {
        best = ob;
        bid = oi;
      }
    }
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
    if (lane == j) {
      my_id = bid;
      my_val = best;
    }
  }

  const float top0 = __shfl(my_val, 0);
  float p = 0.0f;
  if (lane < k) p = (scoring == 0) ? expf(my_val - top0) : 1.0f / (1.0f + expf(-my_val));
  float s = p;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = my_id;
    weights[static_cast<size_t>(t) * k + lane] = p / s;
  }
}

// Single workgroup of 1024 threads (16 waves).  The R = T*k routes are split
// into 16 contiguous segments, one per wave.
//  1. per-segment histograms of local experts (LDS);
//  2. per expert, exclusive prefix over segments, then over experts, so that
//     hist[w][e] becomes the first output slot of segment w's routes to e;
//  3. each wave walks its segment in 64-route chunks; lanes with the same
//     expert rank themselves by lane index (ballot), which keeps the sort
//     stable, and the chunk's leader advances the slot;
//  4. the touched-expert list is compacted in expert order.
// With w_in given (precomputed-routing mode) the routing weights are copied
// into the workspace so that the later steps depend on the workspace only.
__global__ __launch_bounds__(1024) void bucket_kernel(const int32_t* __restrict__ ids, int R, int E_l,
                                                      int offset, int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ routes,
                                                      int32_t* __restrict__ pos,
                                                      int32_t* __restrict__ touched, Plan* __restrict__ plan,
                                                      int32_t* __restrict__ routes_out,
                                                      const float* __restrict__ w_in, float* __restrict__ w_out) {
  __shared__ int hist[kBucketSegments][kMaxLocalExperts];
  __shared__ int base_e[kMaxLocalExperts + 1];
  __shared__ int n_touched_s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  for (int i = tid; i < kBucketSegments * E_l; i += blockDim.x) hist[i / E_l][i % E_l] = 0;
  if (w_in != nullptr) {
    for (int r = tid; r < R; r += blockDim.x) w_out[r] = w_in[r];
  }
  __syncthreads();

  const int seg = (R + kBucketSegments - 1) / kBucketSegments;
  const int s0 = min(R, wave * seg), s1 = min(R, s0 + seg);
  for (int r = s0 + lane; r < s1; r += 64) {
    const int e = ids[r] - offset;
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E_l)) {
      atomicAdd(&hist[wave][e], 1);
    } else {
      pos[r] = -1;
    }
  }
  __syncthreads();

  for (int e = tid; e < E_l; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < kBucketSegments; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    base_e[e] = run;  // count of expert e for now
  }
  __syncthreads();

  // exclusive scan of the per-expert counts by wave 0 (E_l <= 512: 8 per lane)
  if (wave == 0) {
    constexpr int per = kMaxLocalExperts / 64;
    int c[per];
    int local = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      c[i] = e < E_l ? base_e[e] : 0;
      local += c[i];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    const int total = __shfl(incl, 63);
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E_l) {
        counts[e] = c[i];
        offsets[e] = run;
        base_e[e] = run;
      }
      run += c[i];
    }
    if (lane == 0) {
      offsets[E_l] = total;
      base_e[E_l] = total;
    }
  }
  __syncthreads();

  for (int i = tid; i < kBucketSegments * E_l; i += blockDim.x) hist[i / E_l][i % E_l] += base_e[i % E_l];
  __syncthreads();

  for (int b = s0; b < s1; b += 64) {
    const int r = b + lane;
    const int e = (r < s1) ? ids[r] - offset : -1;
    const bool loc = (r < s1) && static_cast<unsigned>(e) < static_cast<unsigned>(E_l);
    uint64_t rem = __ballot(loc);
    while (rem) {
      const int leader = __ffsll(static_cast<unsigned long long>(rem)) - 1;
      const int key = __shfl(e, leader);
      const uint64_t m = __ballot(loc && e == key);
      if (loc && e == key) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        const int p = hist[wave][key] + rank;
        routes[p] = r;
        pos[r] = p;
      }
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) hist[wave][key] += __popcll(m);
      __builtin_amdgcn_wave_barrier();
      rem &= ~m;
    }
  }

  // touched experts in ascending order (wave 0)
  if (wave == 0) {
    int nt = 0;
    for (int e0 = 0; e0 < E_l; e0 += 64) {
      const int e = e0 + lane;
      const bool has = e < E_l && base_e[e + 1] > base_e[e];
      const uint64_t m = __ballot(has);
      if (has) touched[nt + __popcll(m & ((1ull << lane) - 1ull))] = e;
      nt += __popcll(m);
    }
    if (lane == 0) n_touched_s = nt;
  }
  __syncthreads();
  if (tid == 0) {
    plan->n_touched = n_touched_s;
    plan->R_local = base_e[E_l];
  }
  if (routes_out != nullptr) {
    __syncthreads();
    const int Rl = base_e[E_l];
    for (int i = tid; i < R; i += blockDim.x) routes_out[i] = i < Rl ? routes[i] : -1;
  }
}

}  // namespace moe
