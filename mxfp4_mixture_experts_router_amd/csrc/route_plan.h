// Routing and the bucketing of small calls, by single waves: shared by the
// plan kernel and by the gate/up stream kernel's self-planning form (calls
// of at most 64 routes, where every gate/up workgroup routes and buckets the
// call itself instead of reading a plan).  Both use these functions, so the
// two make the same plan bit for bit.
//
// Routing: "MXFP4 MoE decode kernels", At a glance / Parity (gpt-oss top-4
// softmax routing) and "GLM-5.3-Flash on Gaudi 2", Why (top-8 sigmoid
// scoring).  Bucketing: "MXFP4 MoE decode kernels", Design, Routing inside
// the kernel (counting sort by local expert, routes of other ranks skipped).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {

// Top-k of one token's logits by one wave: k rounds of a wave-wide arg-max
// over the not-yet-taken experts (value descending, id ascending).  Lane j < k
// returns the j-th winner.  Each lane holds kPer logits v[i] of experts
// lane + 64 i (E <= 64 * kPer; entries past E are never taken).
template <int kPer>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, int lane, float (&v)[kPer]) {
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = lane + 64 * i;
    v[i] = idx < E ? row[idx] : 0.0f;
  }
}

// Wave-wide sum without LDS: DPP inside rows of 16 lanes, then the four row
// results read as scalars and added in a fixed order.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float rows_of_four(float v, int which) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), which));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  return (rows_of_four(v, 0) + rows_of_four(v, 16)) + (rows_of_four(v, 32) + rows_of_four(v, 48));
}

// Exclusive prefix sum over the 64 lanes (DPP row shifts, then the row
// broadcasts of lanes 15 and 31); total = sum over all lanes.
__device__ __forceinline__ int wave_exclusive_scan_dpp(int v, int& total) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Order-preserving key of a logit: a larger logit has a larger key; -0 and
// +0 share one key (they compare equal); every NaN takes key 1, below every
// number (-inf is 0x007FFFFF); key 0 marks an entry that is taken or past E.
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  if (v != v) return 1u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t m) {
  if (m == 1u) return __builtin_nanf("");
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

// Wave-wide maximum of a key: DPP inside rows of 16 lanes, then the four
// row results as scalars.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Top-k of one token by one wave, k rounds on order-preserving keys: the
// largest free key (wave max), then the lowest expert id holding it (one
// ballot per slot; slot i holds ids 64 i .. 64 i + 63, so the first slot
// with a match has the lowest id), whose key is then cleared.  Ranking:
// logit descending, equal logits (-0 and +0 included) to the lower id, NaN
// below every number and NaNs by id.  Finite logits are the precondition of
// the layer; the NaN rule only keeps the ids distinct and in range when it
// is broken.  top_k <= E, so every round finds a free entry (key >= 1).
template <int kPer>
__device__ __forceinline__ void topk_of(const float (&v)[kPer], int E, int k, int lane, int& my_id, float& my_val) {
  uint32_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) key[i] = lane + 64 * i < E ? logit_key(v[i]) : 0u;
  my_id = 0;
  my_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) lm = max(lm, key[i]);
    const uint32_t m = wave_max_key(lm);
    int win = -1;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint64_t b = __ballot(key[i] == m);
      if (win < 0 && b != 0) win = 64 * i + __ffsll(static_cast<unsigned long long>(b)) - 1;
    }
    const uint32_t keep = (win & 63) == lane ? 0u : ~0u;  // this lane holds the winner: clear its slot
#pragma unroll
    for (int i = 0; i < kPer; ++i) key[i] &= (win >> 6) == i ? keep : ~0u;
    if (lane == j) {
      my_id = win;
      my_val = key_logit(m);
    }
  }
}

template <int kPer>
__device__ __forceinline__ void wave_topk_n(const float* __restrict__ row, int E, int k, int lane, int& my_id,
                                            float& my_val) {
  float v[kPer];
  load_logits<kPer>(row, E, lane, v);
  topk_of<kPer>(v, E, k, lane, my_id, my_val);
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

__device__ __forceinline__ float wave_route_weight(float my_val, int k, int scoring, int lane) {
  const float top0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
  float p = 0.0f;
  if (lane < k) p = (scoring == 0) ? expf(my_val - top0) : 1.0f / (1.0f + expf(-my_val));
  return p / wave_sum(p);
}

// Maximum / minimum inside each row of 16 lanes, by DPP alone: every lane
// of a row ends with its row's result.
__device__ __forceinline__ uint32_t row_max_key(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  return max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
}
__device__ __forceinline__ int row_min(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  return min(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
}

// Top-k of four tokens at once, one per 16-lane row (k <= 16, E <= 16 kPer):
// lane c of a row holds the keys of experts c + 16 i.  The ranking is
// topk_of's (key descending, then the lowest id: the lowest slot i with a
// match in a lane, then the row minimum over lanes).  Lane c < k of each row
// returns its token's c-th winner; every lane gets its row's largest logit.
template <int kPer>
__device__ __forceinline__ void topk_rows(const float (&v)[kPer], int E, int k, int lane, int& my_id, float& my_val,
                                          float& top0) {
  const int c = lane & 15;
  uint32_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) key[i] = c + 16 * i < E ? logit_key(v[i]) : 0u;
  my_id = 0;
  my_val = 0.0f;
  top0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) lm = max(lm, key[i]);
    const uint32_t m = row_max_key(lm);
    int cand = 0x7FFFFFFF;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) cand = key[i] == m ? c + 16 * i : cand;
    const int win = row_min(cand);
    const uint32_t keep = (win & 15) == c ? 0u : ~0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) key[i] &= (win >> 4) == i ? keep : ~0u;
    const float val = key_logit(m);
    if (j == 0) top0 = val;
    if (c == j) {
      my_id = win;
      my_val = val;
    }
  }
}

// The routing weight of topk_rows' lane c < k.  Bit-identical to
// wave_route_weight for a token held by a whole wave: that token's weights
// are nonzero in lanes 0 .. k - 1 of row 0 only, so wave_sum's result is
// lane 0's value after four in-row DPP adds, plus zeros; here the same adds
// run inside each row and the row's first lane is read.
__device__ __forceinline__ float row_route_weight(float my_val, float top0, int k, int scoring, int lane) {
  float p = 0.0f;
  if ((lane & 15) < k) p = (scoring == 0) ? expf(my_val - top0) : 1.0f / (1.0f + expf(-my_val));
  float s = p;
  s += dpp_f<0xB1>(s);
  s += dpp_f<0x4E>(s);
  s += dpp_f<0x124>(s);
  s += dpp_f<0x128>(s);
  const float r0 = rows_of_four(s, 0), r1 = rows_of_four(s, 16), r2 = rows_of_four(s, 32), r3 = rows_of_four(s, 48);
  const int rho = lane >> 4;
  const float r = rho == 0 ? r0 : (rho == 1 ? r1 : (rho == 2 ? r2 : r3));
  return p / ((r + 0.0f) + (0.0f + 0.0f));
}

// Routing of up to 4 * kWaves * kBatches tokens, four per wave and batch:
// wave w routes tokens 4 (w + kWaves b) + row, b < kBatches, and requests
// all of their logits before the first top-k.  Same outputs as route_tokens.
template <int kPer, int kWaves, int kBatches>
__device__ __forceinline__ void route_tokens_rows(const PlanArgs& P, int* ids_s, int wave, int lane, bool write_ws) {
  const int rho = lane >> 4, c = lane & 15;
  float v[kBatches][kPer];
#pragma unroll
  for (int b = 0; b < kBatches; ++b) {
    const int t = 4 * (wave + kWaves * b) + rho;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = c + 16 * i;
      v[b][i] = (t < P.T && e < P.E_global) ? P.logits[static_cast<size_t>(t) * P.E_global + e] : 0.0f;
    }
  }
#pragma unroll
  for (int b = 0; b < kBatches; ++b) {
    const int t0 = 4 * (wave + kWaves * b);
    if (t0 < P.T) {  // wave-uniform; rows past T route zeros and store nothing
      int my_id;
      float my_val, top0;
      topk_rows<kPer>(v[b], P.E_global, P.top_k, lane, my_id, my_val, top0);
      const int t = t0 + rho;
      const bool st = t < P.T && c < P.top_k;
      if (st) ids_s[t * P.top_k + c] = my_id;
      if (write_ws) {  // uniform: the weights are computed only where they are stored
        const float w = row_route_weight(my_val, top0, P.top_k, P.scoring, lane);
        if (st) {
          P.weights_ws[t * P.top_k + c] = w;
          P.ids_ws[t * P.top_k + c] = my_id;
        }
      }
    }
  }
}

// Routing of up to kWaves * kPerWave tokens by kWaves waves: wave w routes
// tokens w, w + kWaves, ..., and requests all of their logits before the
// first top-k.  The ids go to LDS (ids_s[t * top_k + j]); with write_ws
// (uniform over the workgroup) the ids and weights also go to the workspace.
template <int kPer, int kWaves, int kPerWave>
__device__ __forceinline__ void route_tokens(const PlanArgs& P, int* ids_s, int wave, int lane, bool write_ws) {
  float v[kPerWave][kPer];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int t = wave + kWaves * j;
    if (t < P.T) load_logits<kPer>(P.logits + static_cast<size_t>(t) * P.E_global, P.E_global, lane, v[j]);
  }
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int t = wave + kWaves * j;
    if (t < P.T) {
      int my_id;
      float my_val;
      topk_of<kPer>(v[j], P.E_global, P.top_k, lane, my_id, my_val);
      if (lane < P.top_k) ids_s[t * P.top_k + lane] = my_id;
      if (write_ws) {  // uniform: the weights are computed only where they are stored
        const float w = wave_route_weight(my_val, P.top_k, P.scoring, lane);
        if (lane < P.top_k) {
          P.weights_ws[t * P.top_k + lane] = w;
          P.ids_ws[t * P.top_k + lane] = my_id;
        }
      }
    }
  }
}

// route_tokens with the per-lane logit count chosen from E_global.
// Where a wave would route more than one token and a token's top-k fits a
// 16-lane row (top_k <= 16, E_global <= 256), four tokens share each wave.
// Otherwise one token per wave, for at most kWaves * min(kPerWave, 4) tokens
// (callers keep T within that where the row form does not apply, which
// bounds the registers the logits take).
template <int kWaves, int kPerWave>
__device__ __forceinline__ void route_call(const PlanArgs& P, int* ids_s, int wave, int lane, bool write_ws) {
  if (P.T > kWaves && P.top_k <= 16 && P.E_global <= 256) {
    constexpr int kB = (kPerWave + 3) / 4;
    if (P.E_global <= 64) route_tokens_rows<4, kWaves, kB>(P, ids_s, wave, lane, write_ws);
    else if (P.E_global <= 128) route_tokens_rows<8, kWaves, kB>(P, ids_s, wave, lane, write_ws);
    else route_tokens_rows<16, kWaves, kB>(P, ids_s, wave, lane, write_ws);
    return;
  }
  constexpr int kPW = kPerWave < 4 ? kPerWave : 4;
  if (P.E_global <= 64) route_tokens<1, kWaves, kPW>(P, ids_s, wave, lane, write_ws);
  else if (P.E_global <= 128) route_tokens<2, kWaves, kPW>(P, ids_s, wave, lane, write_ws);
  else if (P.E_global <= 256) route_tokens<4, kWaves, kPW>(P, ids_s, wave, lane, write_ws);
  else if (P.E_global <= 512) route_tokens<8, kWaves, kPW>(P, ids_s, wave, lane, write_ws);
  else route_tokens<16, kWaves, kPW>(P, ids_s, wave, lane, write_ws);
}

// Bits of a local expert id (E_local <= 512).  The ballot-per-bit sorts
// always walk all of them: the bits above an id's width are zero in every
// lane and change no comparison, and a fixed count unrolls into straight-line
// code (a runtime count put every ballot behind a branch of its own).
constexpr int kExpertIdBits = 9;
static_assert((1 << kExpertIdBits) >= kMaxLocalExperts, "expert ids fit kExpertIdBits");

// Local routes of lanes in `loc` whose expert compares below / equal to this
// lane's key: one ballot per expert-id bit, most significant first (bit b
// splits the lanes still equal above b).
struct KeyCompare {
  uint64_t less, equal;
};
__device__ __forceinline__ KeyCompare compare_keys(uint64_t loc, const uint64_t (&bit_ballots)[10], int bits, int key) {
  uint64_t less = 0, eq = loc;
#pragma unroll
  for (int b = 9; b >= 0; --b) {  // unrolled: the ballots stay in registers
    if (b < bits) {
      const uint64_t one = bit_ballots[b];
      if ((key >> b) & 1) {
        less |= eq & ~one;
        eq &= one;
      } else {
        eq &= ~one;
      }
    }
  }
  return KeyCompare{less, eq};
}

// Bucketing of R <= 64 routes by one wave: the counting sort of the general
// path, written out with ballots.  Lane r holds route r; its plan position is
// the number of local routes to lower experts plus its rank among the routes
// to its own expert (stable).  The sorted order is staged in LDS (scratch,
// 128 ints), from which lane j reads the route at position j.
struct SmallBuckets {
  int p;           // plan position of this lane's route (lanes < R), -1 when not local
  int Rl;          // local routes
  int bits;        // expert-id bits
  bool jin;        // position j = lane holds a local route:
  int rj, ej;      //   its route and local expert,
  bool first;      //   whether it is its expert's first position,
  int rank, cnt;   //   its rank among its expert's routes and their count
  uint64_t fm;     // positions that start an expert
};

__device__ __forceinline__ SmallBuckets sort_small(const int32_t* ids, int R, int E_l, int offset, int lane,
                                                   int* scratch) {
  SmallBuckets b;
  const bool in = lane < R;
  const int e = in ? ids[lane] - offset : -1;
  const bool loc = in && static_cast<unsigned>(e) < static_cast<unsigned>(E_l);
  b.bits = kExpertIdBits;
  const uint64_t lt = (1ull << lane) - 1ull, le = lt | (1ull << lane);
  const uint64_t locm = __ballot(loc);
  uint64_t bb[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) bb[i] = i < b.bits ? __ballot(loc && ((e >> i) & 1)) : 0ull;
  const KeyCompare c = compare_keys(locm, bb, b.bits, e);
  const int p = __popcll(c.less) + __popcll(c.equal & lt);
  b.p = loc ? p : -1;
  b.Rl = __popcll(locm);
  if (loc) {
    scratch[p] = lane;
    scratch[64 + p] = e;
  }
  __builtin_amdgcn_wave_barrier();

  // the sorted view: position j = lane
  const int j = lane;
  b.jin = j < b.Rl;
  b.rj = b.jin ? scratch[j] : 0;
  b.ej = b.jin ? scratch[64 + j] : -1;
  const int eprev = (b.jin && j > 0) ? scratch[64 + j - 1] : -1;
  b.first = b.jin && b.ej != eprev;
  b.fm = __ballot(b.first);
  const uint64_t upto = b.fm & le, after = b.fm & ~le;
  const int start = upto ? 63 - __clzll(upto) : 0;  // first position of this expert
  const int end = after ? __ffsll(static_cast<unsigned long long>(after)) - 1 : b.Rl;
  b.rank = j - start;
  b.cnt = end - start;
  return b;
}

// A pass list of the sorted routes: each expert's routes in plan order, cut
// every 2^sh routes, into `list` (global memory or LDS); *count = passes.
__device__ __forceinline__ void small_pass_list(const SmallBuckets& b, PassEntry* list, int sh, int lane,
                                                int32_t* count) {
  const int tp = 1 << sh;
  const uint64_t le = (2ull << lane) - 1ull;
  const uint64_t psm = __ballot(b.jin && (b.rank & (tp - 1)) == 0);
  if (b.jin) {
    PassEntry* pe = list + (__popcll(psm & le) - 1);
    pe->rte[b.rank & (tp - 1)] = static_cast<uint16_t>(b.rj);
    if ((b.rank & (tp - 1)) == 0) {
      pe->e = b.ej;
      pe->nt = min(tp, b.cnt - b.rank);
      pe->p = lane;
    }
  }
  if (lane == 0) *count = __popcll(psm);
}

// The whole plan of R <= 64 routes by one wave, into the workspace:
// positions, routes, counts and offsets of every local expert, the header,
// the pass lists and (when a projection needs them) the GEMV / MFMA lists.
__device__ __forceinline__ void bucket_one_wave(const PlanArgs& P, const int32_t* ids, int R, int lane,
                                                int* scratch) {
  const int E_l = P.E_local;
  const SmallBuckets b = sort_small(ids, R, E_l, P.offset, lane, scratch);
  const uint64_t lt = (1ull << lane) - 1ull;
  if (lane < R) P.pos[lane] = b.p;
  if (b.p >= 0) P.routes[b.p] = lane;
  const int Rl = b.Rl, bits = b.bits;

  // counts and offsets of every local expert: a touched one from its first
  // position, an untouched one from the next touched expert
  const int fk = b.first ? b.ej : 0;
  uint64_t lb[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) lb[i] = i < bits ? __ballot((fk >> i) & 1) : 0ull;
  for (int e0 = 0; e0 < E_l; e0 += 64) {
    const int ee = e0 + lane;
    if (ee < E_l) {
      const KeyCompare k = compare_keys(b.fm, lb, bits, ee);
      const uint64_t ge = b.fm & ~k.less;  // leaders of experts >= ee (a suffix of the positions)
      const int at = ge ? __ffsll(static_cast<unsigned long long>(ge)) - 1 : Rl;
      int n = 0;
      if (k.equal) {
        const uint64_t nxt = b.fm & ~((k.equal << 1) - 1ull);
        n = (nxt ? __ffsll(static_cast<unsigned long long>(nxt)) - 1 : Rl) - at;
      }
      P.counts[ee] = n;
      P.offsets[ee] = at;
    }
  }
  if (lane == 0) {
    P.offsets[E_l] = Rl;
    P.plan->n_touched = __popcll(b.fm);
    P.plan->R_local = Rl;
    P.plan->key = P.key;
  }
  if (P.passes != nullptr) small_pass_list(b, P.passes, P.pass_shift, lane, &P.plan->n_passes);
  if (P.passes2 != nullptr) small_pass_list(b, P.passes2, P.pass_shift2, lane, &P.plan->n_passes2);

  if (P.lists) {
    const bool hm = b.first && P.mfma_enabled && b.cnt > P.gemv_max;
    const bool hg = b.first && !hm;
    const uint64_t mg = __ballot(hg), mm = __ballot(hm);
    if (hg || hm) {
      WorkEntry we;
      we.e = b.ej;
      we.p0 = lane;
      we.Te = b.cnt;
#pragma unroll
      for (int t = 0; t < kGemvMaxTokens; ++t) we.tok[t] = t < b.cnt ? scratch[lane + t] / P.top_k : 0;
#pragma unroll
      for (int t = 0; t < 8 - 3 - kGemvMaxTokens; ++t) we.pad[t] = 0;
      if (hg) P.gemv_list[__popcll(mg & lt)] = we;
      else P.mfma_list[__popcll(mm & lt)] = we;
    }
    if (lane == 0) {
      P.plan->n_gemv = __popcll(mg);
      P.plan->n_mfma = __popcll(mm);
    }
  }
  if (P.routes_out != nullptr && lane < R) P.routes_out[lane] = b.jin ? b.rj : -1;
}

// Lanes of the wave whose `loc` routes go to the same local expert as this
// lane: the expert's bits compared lane against lane with one ballot per bit
// (E_l <= 512: at most 9), no loop over the distinct experts.
__device__ __forceinline__ uint64_t same_expert_lanes(bool loc, int e, int bits) {
  const uint64_t locm = __ballot(loc);
  const int ek = loc ? e : 0;
  uint64_t m = locm;
#pragma unroll
  for (int b = 0; b < bits; ++b) {
    const uint64_t one = __ballot((ek >> b) & 1) & locm;
    m &= ((ek >> b) & 1) ? one : ~one;
  }
  return m;
}

// Route r, the j-th route of local expert e (plan position p), into its pass
// entry of a list cut every 2^sh routes; the pass's first route writes the
// entry's header.  `first` is the expert's first pass in the list.
__device__ __forceinline__ void place_in_pass(PassEntry* list, int sh, int first, int e, int j, int p, int r,
                                              const int* base_e) {
  const int tp = 1 << sh;
  const int pass = j >> sh, slot = j & (tp - 1);
  PassEntry* pe = list + first + pass;
  pe->rte[slot] = static_cast<uint16_t>(r);
  if (slot == 0) {
    pe->e = e;
    pe->nt = min(tp, base_e[e + 1] - base_e[e] - pass * tp);
    pe->p = p;
  }
}

// Work lists of the touched experts in ascending order, split by regime (one
// wave): experts with at most gemv_max routes (with the tokens of their first
// routes) go to the GEMV list, the others to the MFMA list.  base_e holds the
// exclusive offsets [E_l + 1]; routes_src the route of each plan position.
__device__ __forceinline__ void build_lists(const PlanArgs& P, const int* base_e, const int32_t* routes_src, int lane) {
  const int E_l = P.E_local;
  const uint64_t lt = (1ull << lane) - 1ull;
  int ng = 0, nm = 0;
  for (int e0 = 0; e0 < E_l; e0 += 64) {
    const int e = e0 + lane;
    const int cnt = e < E_l ? base_e[e + 1] - base_e[e] : 0;
    const bool hm = P.mfma_enabled && cnt > P.gemv_max;
    const bool hg = cnt > 0 && !hm;
    const uint64_t mg = __ballot(hg);
    const uint64_t mm = __ballot(hm);
    if (hg || hm) {
      WorkEntry we;
      we.e = e;
      we.p0 = base_e[e];
      we.Te = cnt;
#pragma unroll
      for (int j = 0; j < kGemvMaxTokens; ++j) we.tok[j] = j < cnt ? routes_src[we.p0 + j] / P.top_k : 0;
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
    P.plan->n_gemv = ng;
    P.plan->n_mfma = nm;
  }
}

// Bucketing of 64 < R <= kChunkedRoutes routes by one wave: the stable
// counting sort of the general path without its workgroup barriers.  Pass 1
// walks the routes in 64-route chunks, in route order: the lanes of a chunk
// that go to one expert find each other with one ballot per expert-id bit,
// rank after the expert's running count (ranks follow route order, so the
// sort is stable) and the group's lowest lane advances the count.  The
// counts are scanned into offsets and pass bases; pass 2 places every route
// at its expert's offset plus its rank.  LDS: cnt [E_l] (zeroed by the
// caller), rank_s and routes_s [R], base_e [E_l + 1], pass_base [E_l].
// kGlobal writes the plan into the workspace (the plan kernel, and workgroup 0
// of a self-planned gate/up launch); otherwise only one pass list, cut every
// 2^sh_l routes, goes to list_l with its count in *np_l (LDS of the other
// workgroups of that launch).
constexpr int kChunkedRoutes = 512;

template <bool kGlobal>
__device__ __forceinline__ void bucket_chunks(const PlanArgs& P, const int32_t* ids, int R, int lane, int* cnt, int* rank_s,
                                              int32_t* routes_s, int* base_e, int* pass_base, int* pass_base2,
                                              PassEntry* list_l = nullptr, int sh_l = 0, int* np_l = nullptr) {
  const int E_l = P.E_local;
  constexpr int bits = kExpertIdBits;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int c = 0; c < R; c += 64) {
    const int r = c + lane;
    const bool in = r < R;
    const int e = in ? ids[r] - P.offset : -1;
    const bool loc = in && static_cast<unsigned>(e) < static_cast<unsigned>(E_l);
    const uint64_t m = same_expert_lanes(loc, e, bits);
    if (loc) rank_s[r] = cnt[e] + __popcll(m & lt);
    __builtin_amdgcn_wave_barrier();
    if (loc && (m & lt) == 0) cnt[e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
    if (kGlobal && in && !loc) P.pos[r] = -1;
  }
  // counts -> offsets (and pass bases): 8 experts per lane, DPP wave scans
  constexpr int per = kMaxLocalExperts / 64;
  int cc[per];
  int local = 0, nz = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    cc[i] = e < E_l ? cnt[e] : 0;
    local += cc[i];
    nz += cc[i] > 0;
  }
  int total, n_touched;
  int run = wave_exclusive_scan_dpp(local, total);
  (void)wave_exclusive_scan_dpp(nz, n_touched);
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E_l) {
      if (kGlobal) {
        P.counts[e] = cc[i];
        P.offsets[e] = run;
      }
      base_e[e] = run;
    }
    run += cc[i];
  }
  if (lane == 0) {
    base_e[E_l] = total;
    if (kGlobal) {
      P.offsets[E_l] = total;
      P.plan->n_touched = n_touched;
      P.plan->R_local = total;
      P.plan->key = P.key;
    }
  }
  // first pass of each expert in each pass list (exclusive scan of its pass counts)
  auto pass_bases = [&](int sh, int* base, int32_t* count) {
    const int tp1 = (1 << sh) - 1;
    int np = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) np += (cc[i] + tp1) >> sh;
    int np_total;
    int prun = wave_exclusive_scan_dpp(np, np_total);
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E_l) base[e] = prun;
      prun += (cc[i] + tp1) >> sh;
    }
    if (lane == 0) *count = np_total;
  };
  if (!kGlobal) {
    pass_bases(sh_l, pass_base, np_l);
  } else {
    if (P.passes != nullptr) pass_bases(P.pass_shift, pass_base, &P.plan->n_passes);
    if (P.passes2 != nullptr) pass_bases(P.pass_shift2, pass_base2, &P.plan->n_passes2);
  }
  __builtin_amdgcn_wave_barrier();
  for (int c = 0; c < R; c += 64) {
    const int r = c + lane;
    const bool in = r < R;
    const int e = in ? ids[r] - P.offset : -1;
    const bool loc = in && static_cast<unsigned>(e) < static_cast<unsigned>(E_l);
    if (loc) {
      const int j = rank_s[r];
      const int p = base_e[e] + j;
      if (!kGlobal) {
        place_in_pass(list_l, sh_l, pass_base[e], e, j, p, r, base_e);
      } else {
        P.routes[p] = r;
        routes_s[p] = r;
        P.pos[r] = p;
        if (P.passes != nullptr) place_in_pass(P.passes, P.pass_shift, pass_base[e], e, j, p, r, base_e);
        if (P.passes2 != nullptr) place_in_pass(P.passes2, P.pass_shift2, pass_base2[e], e, j, p, r, base_e);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (!kGlobal) return;
  if (P.lists) build_lists(P, base_e, routes_s, lane);
  if (P.routes_out != nullptr) {
    for (int i = lane; i < R; i += 64) P.routes_out[i] = i < total ? routes_s[i] : -1;
  }
}

}  // namespace moe
