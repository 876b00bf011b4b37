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

namespace moe {

namespace {

// One step of a wave-wide arg-max on (value desc, id asc) pairs, exchanging
// with a DPP-permuted partner inside each row of 16 lanes.
#define MOE_ARGMAX_DPP(v, id, ctrl)                                                                     \
  do {                                                                                                  \
    const float ov_ = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),   \
                                                                         ctrl, 0xF, 0xF, false));       \
    const int oi_ = __builtin_amdgcn_mov_dpp(id, ctrl, 0xF, 0xF, false);                                \
    if (ov_ > v || (ov_ == v && oi_ < id)) {                                                            \
      v = ov_;                                                                                          \
      id = oi_;                                                                                         \
    }                                                                                                   \
  } while (0)

__device__ __forceinline__ void argmax_xor(float& v, int& id, int mask) {
  const float ov = __shfl_xor(v, mask);
  const int oi = __shfl_xor(id, mask);
  if (ov > v || (ov == v && oi < id)) {
    v = ov;
    id = oi;
  }
}

// Top-k of one token's logits by one wave: k rounds of a wave-wide arg-max
// over the not-yet-taken experts (value descending, id ascending).  Lane j < k
// returns the j-th winner.  Each lane holds kPer logits (E <= 64 * kPer).
template <int kPer>
__device__ __forceinline__ void wave_topk_n(const float* __restrict__ row, int E, int k, int lane, int& my_id,
                                            float& my_val) {
  float v[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = lane + 64 * i;
    v[i] = idx < E ? row[idx] : 0.0f;
    if (idx >= E) taken |= 1u << i;
  }
  my_id = 0;
  my_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    float best = -__builtin_inff();
    int bid = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = lane + 64 * i;
      const bool free = !((taken >> i) & 1u);
      if (free && (v[i] > best || (v[i] == best && idx < bid))) {
        best = v[i];
        bid = idx;
      }
    }
    MOE_ARGMAX_DPP(best, bid, 0xB1);   // quad_perm [1,0,3,2]
    MOE_ARGMAX_DPP(best, bid, 0x4E);   // quad_perm [2,3,0,1]
    MOE_ARGMAX_DPP(best, bid, 0x124);  // row_ror:4
    MOE_ARGMAX_DPP(best, bid, 0x128);  // row_ror:8
    argmax_xor(best, bid, 16);
    argmax_xor(best, bid, 32);
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
    if (lane == j) {
      my_id = bid;
      my_val = best;
    }
  }
}

__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int lane, int& my_id,
                                          float& my_val) {
  if (E <= 64) {
    wave_topk_n<1>(row, E, k, lane, my_id, my_val);
  } else if (E <= 128) {
    wave_topk_n<2>(row, E, k, lane, my_id, my_val);
  } else if (E <= 256) {
    wave_topk_n<4>(row, E, k, lane, my_id, my_val);
  } else if (E <= 512) {
    wave_topk_n<8>(row, E, k, lane, my_id, my_val);
  } else {
    wave_topk_n<16>(row, E, k, lane, my_id, my_val);
  }
}

// Routing weight of lane j's winner: softmax over the k selected logits, or
// sigmoid renormalised over the k selected.
__device__ __forceinline__ float wave_route_weight(float my_val, int k, int scoring, int lane) {
  const float top0 = __shfl(my_val, 0);
  float p = 0.0f;
  if (lane < k) p = (scoring == 0) ? expf(my_val - top0) : 1.0f / (1.0f + expf(-my_val));
  float s = p;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  return p / s;
}

__device__ __forceinline__ int wave_exclusive_scan(int v, int lane, int& total) {
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  total = __shfl(incl, 63);
  return incl - v;
}

}  // namespace

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
//     per-segment histograms of local experts (LDS);
//  2. per expert, exclusive prefix over segments, then over experts, so that
//     hist[w][e] becomes the first output slot of segment w's routes to e;
//  3. each wave walks its segment in 64-route chunks; lanes with the same
//     expert rank themselves by lane index (ballot), which keeps the sort
//     stable, and the chunk's leader advances the slot;
//  4. the touched experts, in expert order, become two work lists: experts
//     with at most kGemvMaxTokens routes (GEMV regime, with their tokens) and
//     the others (MFMA regime);
//  5. (decode regime) each expert's routes, in plan order, are cut into
//     passes of pass_tokens routes; every route writes its token into its
//     pass entry as it is placed, and the pass's first route the header.
__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs P) {
  __shared__ int hist[kPlanWaves][kMaxLocalExperts];
  __shared__ int base_e[kMaxLocalExperts + 1];
  __shared__ int ids_s[kFusedRouteTokens * kMaxTopK];
  __shared__ int pass_base[kMaxLocalExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = P.T * P.top_k, E_l = P.E_local, offset = P.offset;
  const bool fused = P.logits != nullptr;

  if (fused) {
    for (int t = wave; t < P.T; t += kPlanWaves) {
      int my_id;
      float my_val;
      wave_topk(P.logits + static_cast<size_t>(t) * P.E_global, P.E_global, P.top_k, lane, my_id, my_val);
      const float w = wave_route_weight(my_val, P.top_k, P.scoring, lane);
      if (lane < P.top_k) {
        ids_s[t * P.top_k + lane] = my_id;
        P.weights_ws[t * P.top_k + lane] = w;
        P.ids_ws[t * P.top_k + lane] = my_id;
      }
    }
  } else if (P.w_in != nullptr) {
    for (int r = tid; r < R; r += blockDim.x) P.weights_ws[r] = P.w_in[r];
  }
  for (int i = tid; i < kPlanWaves * E_l; i += blockDim.x) hist[i / E_l][i % E_l] = 0;
  __syncthreads();

  const int seg = (R + kPlanWaves - 1) / kPlanWaves;
  const int s0 = min(R, wave * seg), s1 = min(R, s0 + seg);
  for (int r = s0 + lane; r < s1; r += 64) {
    const int e = (fused ? ids_s[r] : P.ids_in[r]) - offset;
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E_l)) {
      atomicAdd(&hist[wave][e], 1);
    } else {
      P.pos[r] = -1;
    }
  }
  __syncthreads();

  for (int e = tid; e < E_l; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
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
    int total;
    int run = wave_exclusive_scan(local, lane, total);
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
    if (lane == 0) {
      P.offsets[E_l] = total;
      base_e[E_l] = total;
    }
    if (P.passes != nullptr) {
      const int tp = P.pass_tokens;
      int np = 0;
#pragma unroll
      for (int i = 0; i < per; ++i) np += (c[i] + tp - 1) / tp;
      int np_total;
      int prun = wave_exclusive_scan(np, lane, np_total);
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int e = lane * per + i;
        if (e < E_l) pass_base[e] = prun;
        prun += (c[i] + tp - 1) / tp;
      }
      if (lane == 0) P.plan->n_passes = np_total;
    }
  }
  __syncthreads();

  for (int i = tid; i < kPlanWaves * E_l; i += blockDim.x) hist[i / E_l][i % E_l] += base_e[i % E_l];
  __syncthreads();

  for (int b = s0; b < s1; b += 64) {
    const int r = b + lane;
    const int e = (r < s1) ? (fused ? ids_s[r] : P.ids_in[r]) - offset : -1;
    const bool loc = (r < s1) && static_cast<unsigned>(e) < static_cast<unsigned>(E_l);
    uint64_t rem = __ballot(loc);
    while (rem) {
      const int leader = __ffsll(static_cast<unsigned long long>(rem)) - 1;
      const int key = __shfl(e, leader);
      const uint64_t m = __ballot(loc && e == key);
      if (loc && e == key) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        const int p = hist[wave][key] + rank;
        P.routes[p] = r;
        P.pos[r] = p;
        if (P.passes != nullptr) {
          const int tp = P.pass_tokens;
          const int j = p - base_e[key];
          const int pass = j / tp, slot = j - pass * tp;
          PassEntry* pe = P.passes + pass_base[key] + pass;
          pe->tok[slot] = static_cast<uint16_t>(r / P.top_k);
          if (slot == 0) {
            pe->e = key;
            pe->nt = min(tp, base_e[key + 1] - base_e[key] - pass * tp);
            pe->p = p;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) hist[wave][key] += __popcll(m);
      __builtin_amdgcn_wave_barrier();
      rem &= ~m;
    }
  }

  __syncthreads();  // routes[] complete

  // work lists: touched experts in ascending order, split by regime (wave 0)
  if (wave == 0) {
    int ng = 0, nm = 0;
    for (int e0 = 0; e0 < E_l; e0 += 64) {
      const int e = e0 + lane;
      const int cnt = e < E_l ? base_e[e + 1] - base_e[e] : 0;
      const bool hm = P.mfma_enabled && cnt > kGemvMaxTokens;
      const bool hg = cnt > 0 && !hm;
      const uint64_t lt = (1ull << lane) - 1ull;
      const uint64_t mg = __ballot(hg);
      const uint64_t mm = __ballot(hm);
      if (hg || hm) {
        WorkEntry we;
        we.e = e;
        we.p0 = base_e[e];
        we.Te = cnt;
#pragma unroll
        for (int j = 0; j < kGemvMaxTokens; ++j) we.tok[j] = j < cnt ? P.routes[we.p0 + j] / P.top_k : 0;
#pragma unroll
        for (int j = 0; j < 8 - 3 - kGemvMaxTokens; ++j) we.pad[j] = 0;
        if (hg) {
          P.gemv_list[ng + __popcll(mg & lt)] = we;
        } else {
          P.mfma_list[nm + __popcll(mm & lt)] = we;
        }
      }
      ng += __popcll(mg);
      nm += __popcll(mm);
    }
    if (lane == 0) {
      P.plan->n_touched = ng + nm;
      P.plan->R_local = base_e[E_l];
      P.plan->n_gemv = ng;
      P.plan->n_mfma = nm;
    }
  }
  if (P.routes_out != nullptr) {
    const int Rl = base_e[E_l];
    for (int i = tid; i < R; i += blockDim.x) P.routes_out[i] = i < Rl ? P.routes[i] : -1;
  }
}

}  // namespace moe
