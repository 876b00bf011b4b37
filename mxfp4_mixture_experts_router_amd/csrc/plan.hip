// Router top-k and the per-call plan: bucketing of routes by local expert and
// the work lists of the two expert kernels.
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
#include "route_plan.h"

namespace moe {

// One wave per token, for calls too large to route inside the plan kernel.
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int scoring, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  int my_id;
  float my_val;
  wave_topk(logits + static_cast<size_t>(t) * E, E, k, lane, my_id, my_val);
  const float w = wave_route_weight(my_val, k, scoring, lane);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = my_id;
    weights[static_cast<size_t>(t) * k + lane] = w;
  }
}

// Single workgroup of 16 waves.
//  0. (router-logits mode, T <= kFusedRouteTokens) route every token, ids to LDS;
//  1. the R = T*k routes are split into 16 contiguous segments, one per wave;
//     per-segment histograms of local experts (LDS), counted with one LDS
//     atomic add per local route;
//  2. per expert, exclusive prefix over segments (a 16-lane DPP row scan),
//     then over experts, so that entry (e, w) becomes the first output slot of
//     segment w's routes to e;
//  3. each wave walks its segment again; a route's rank among the lanes of
//     its group before it keeps the sort stable, and the group's lowest lane
//     advances the slot for the next chunk;
//  4. the touched experts, in expert order, become two work lists: experts
//     with at most kGemvMaxTokens routes (GEMV regime, with their tokens) and
//     the others (MFMA regime);
//  5. (decode regime) each expert's routes, in plan order, are cut into
//     passes of 2^pass_shift routes; every route writes its index into its
//     pass entry as it is placed, and the pass's first route the header.
constexpr int kIdBatch = 8;  // 64-route chunks whose ids a wave requests at once

__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs P) {
  __shared__ int hist[kMaxLocalExperts * kPlanWaves];  // [expert][segment]
  __shared__ int base_e[kMaxLocalExperts + 1];
  __shared__ int ids_s[kFusedRouteTokens * kMaxTopK];
  __shared__ int pass_base[kMaxLocalExperts];
  __shared__ int pass_base2[kMaxLocalExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = P.T * P.top_k, E_l = P.E_local, offset = P.offset;
  const bool fused = P.logits != nullptr;

  if (fused) {
    // a wave routes tokens wave, wave + 16, ... (at most kFusedRouteTokens / 16);
    // all of their logits are requested before the first top-k
    route_call<kPlanWaves, kFusedRouteTokens / kPlanWaves>(P, ids_s, wave, lane, true);
  } else if (P.w_in != nullptr) {
    // ids mode: the plan keeps its own copy of the caller's routing
    for (int r = tid; r < R; r += blockDim.x) {
      P.weights_ws[r] = P.w_in[r];
      P.ids_ws[r] = P.ids_in[r];
    }
  }
  for (int i = tid; i < kPlanWaves * E_l; i += blockDim.x) hist[i] = 0;
  __syncthreads();

  if (R <= 64) {
    // at most 64 routes: one wave buckets them, with the same results as the
    // general path below and no workgroup barrier
    if (wave == 0) bucket_one_wave(P, fused ? ids_s : P.ids_in, R, lane, hist);
    return;
  }
  if (R <= kChunkedRoutes) {
    // up to kChunkedRoutes routes: one wave, no further workgroup barrier
    static_assert(3 * kChunkedRoutes <= kMaxLocalExperts * kPlanWaves, "LDS of the chunked path");
    if (wave == 0)
      bucket_chunks<true>(P, fused ? ids_s : P.ids_in, R, lane, hist, hist + kMaxLocalExperts,
                    hist + kMaxLocalExperts + kChunkedRoutes, base_e, pass_base, pass_base2);
    return;
  }

  // the R routes in 16 contiguous segments, one per wave, 64 at a time
  const int seg = (R + kPlanWaves - 1) / kPlanWaves;
  const int s0 = min(R, wave * seg), s1 = min(R, s0 + seg);
  constexpr int bits = kExpertIdBits;
  const uint64_t lt = (1ull << lane) - 1ull;
  // the ids of kIdBatch chunks are requested together, then the chunks are
  // processed in order (one memory latency per batch instead of per chunk);
  // the two sources are read in separate branches, unconditionally at a
  // clamped index, so that each is a plain LDS or global load with no exec
  // mask and no wait of its own (a pointer select between them would make
  // them flat loads; a conditional use would sink each load into a branch)
  auto load_ids = [&](int b0, int (&ev)[kIdBatch]) {
    if (fused) {
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u) {
        const int r = b0 + 64 * u + lane;
        ev[u] = ids_s[min(r, R - 1)] - offset;  // lanes past the segment are masked by r < s1
      }
    } else {
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u) {
        const int r = b0 + 64 * u + lane;
        ev[u] = P.ids_in[min(r, R - 1)] - offset;
      }
    }
  };
  for (int b0 = s0; b0 < s1; b0 += 64 * kIdBatch) {
    int ev[kIdBatch];
    load_ids(b0, ev);
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int r = b0 + 64 * u + lane;
      if (b0 + 64 * u >= s1) break;  // wave-uniform
      const int e = ev[u];
      const bool loc = (r < s1) && static_cast<unsigned>(e) < static_cast<unsigned>(E_l);
      if (r < s1 && !loc) P.pos[r] = -1;
      // counts only: an LDS atomic per local route (integer adds, any order)
      if (loc) atomicAdd(&hist[e * kPlanWaves + wave], 1);
    }
  }
  __syncthreads();

  // per expert, exclusive prefix over the 16 segments: one row of 16 lanes
  // per expert (lane = segment), DPP row shifts; the row's last lane has the total
  for (int i0 = 0; i0 < kPlanWaves * E_l; i0 += blockDim.x) {  // whole rows of 16 stay together
    const int i = i0 + tid;
    const int e = i >> 4, w = i & 15;
    const int v = e < E_l ? hist[i] : 0;
    int x = v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    if (e < E_l) {
      hist[i] = x - v;
      if (w == 15) base_e[e] = x;  // count of expert e for now
    }
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
    int total;
    int run = wave_exclusive_scan_dpp(local, total);
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E_l) {
        P.counts[e] = c[i];
        P.offsets[e] = run;
        base_e[e] = run;
      }
      run += c[i];
    }
    int nz = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) nz += c[i] > 0;
    int n_touched;
    (void)wave_exclusive_scan_dpp(nz, n_touched);
    if (lane == 0) {
      P.offsets[E_l] = total;
      base_e[E_l] = total;
      P.plan->n_touched = n_touched;
      P.plan->R_local = total;
      P.plan->key = P.key;
    }
    auto pass_bases = [&](int sh, int* base, int32_t* count) {
      const int tp1 = (1 << sh) - 1;
      int np = 0;
#pragma unroll
      for (int i = 0; i < per; ++i) np += (c[i] + tp1) >> sh;
      int np_total;
      int prun = wave_exclusive_scan_dpp(np, np_total);
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int e = lane * per + i;
        if (e < E_l) base[e] = prun;
        prun += (c[i] + tp1) >> sh;
      }
      if (lane == 0) *count = np_total;
    };
    if (P.passes != nullptr) pass_bases(P.pass_shift, pass_base, &P.plan->n_passes);
    if (P.passes2 != nullptr) pass_bases(P.pass_shift2, pass_base2, &P.plan->n_passes2);
  }
  __syncthreads();

  for (int i = tid; i < kPlanWaves * E_l; i += blockDim.x) hist[i] += base_e[i >> 4];
  __syncthreads();

  // placement: a route's slot is its expert's segment base plus its rank
  // among the same-expert routes before it in the segment (stable); one
  // 64-lane chunk of local routes at a time
  auto place = [&](bool loc, int r, int e) {
    const uint64_t m = same_expert_lanes(loc, e, bits);
    if (loc) {
      const int p = hist[e * kPlanWaves + wave] + __popcll(m & lt);
      P.routes[p] = r;
      P.pos[r] = p;
      if (P.passes != nullptr) place_in_pass(P.passes, P.pass_shift, pass_base[e], e, p - base_e[e], p, r, base_e);
      if (P.passes2 != nullptr) place_in_pass(P.passes2, P.pass_shift2, pass_base2[e], e, p - base_e[e], p, r, base_e);
    }
    __builtin_amdgcn_wave_barrier();
    if (loc && (m & lt) == 0) hist[e * kPlanWaves + wave] += __popcll(m);  // next chunk of the segment
    __builtin_amdgcn_wave_barrier();
  };
  if (!fused && R < (1 << 23)) {
    // The routing buffer is free: each wave first packs the local routes of
    // 4 chunks (route << 9 | expert, in segment order) into its 256 entries
    // of it, then ranks only those, so a slice with few local routes (an
    // expert-parallel shard) ranks a fraction of the chunks.
    static_assert(kFusedRouteTokens * kMaxTopK >= kPlanWaves * 256, "256 entries per wave");
    static_assert(kMaxLocalExperts <= 512, "9 bits of expert id");
    uint32_t* cbuf = reinterpret_cast<uint32_t*>(ids_s) + wave * 256;
    for (int b0 = s0; b0 < s1; b0 += 64 * kIdBatch) {
      int ev[kIdBatch];
      load_ids(b0, ev);
#pragma unroll
      for (int h = 0; h < kIdBatch; h += 4) {
        int n = 0;
#pragma unroll
        for (int u = h; u < h + 4; ++u) {
          const int r = b0 + 64 * u + lane;
          const bool loc = (r < s1) && static_cast<unsigned>(ev[u]) < static_cast<unsigned>(E_l);
          const uint64_t m = __ballot(loc);
          if (loc) cbuf[n + __popcll(m & lt)] = (static_cast<uint32_t>(r) << 9) | static_cast<uint32_t>(ev[u]);
          n += __popcll(m);
        }
        __builtin_amdgcn_wave_barrier();
        for (int c = 0; c < n; c += 64) {
          const bool loc = c + lane < n;
          const uint32_t v = loc ? cbuf[c + lane] : 0u;
          place(loc, static_cast<int>(v >> 9), static_cast<int>(v & 511u));
        }
      }
    }
  } else {
    for (int b0 = s0; b0 < s1; b0 += 64 * kIdBatch) {
      int ev[kIdBatch];
      load_ids(b0, ev);
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u) {
        if (b0 + 64 * u >= s1) break;  // wave-uniform
        const int r = b0 + 64 * u + lane;
        const int e = ev[u];
        place((r < s1) && static_cast<unsigned>(e) < static_cast<unsigned>(E_l), r, e);
      }
    }
  }

  __syncthreads();  // routes[] complete

  // work lists: touched experts in ascending order, split by regime (wave 0);
  // calls served by the stream kernel alone need only the counts
  if (wave == 0 && P.lists) build_lists(P, base_e, P.routes, lane);
  if (P.routes_out != nullptr) {
    const int Rl = base_e[E_l];
    for (int i = tid; i < R; i += blockDim.x) P.routes_out[i] = i < Rl ? P.routes[i] : -1;
  }
}

}  // namespace moe
