// Decode-regime expert projection: one persistent launch per projection.
//
// "MXFP4 MoE decode kernels" (The bottleneck; Design) makes decode a weight
// stream: every touched expert's packed rows are read once, E2M1 codes are
// decoded with their E8M0 block scale in registers and multiplied with the
// few activation rows routed to that expert.  This kernel is that stream laid
// out for gfx950:
//
//  * work item = (pass, row tile): a pass is up to 16/kSplit routes of one
//    expert (PassEntry, written by the plan kernel), a tile is 64/kSplit
//    output rows (row pairs [gate; up] for the gate/up projection);
//  * the grid is persistent: workgroup b takes items b, b+P, b+2P, ...; a
//    wave's step sequence runs across item boundaries, so the register ring
//    of kStreamRing steps keeps loading the next item's weights while the
//    current item finishes (no per-item ramp);
//  * a wave owns a 16-row sub-tile and one of kSplit slices of the reduction
//    (down projection, kPair: two 16-row sets 16 rows apart, so that, like the
//    gate/up rows, every step loads two weight blocks per lane);
//    one step = 4 MX blocks per lane (lane (r, q) holds block q of row r), so
//    a step is 4 v_mfma_f32_16x16x32_bf16 per row set, the 4 dwords of a
//    lane's 16-byte block giving the k-slots of the 4 MFMAs (the activation
//    operand is permuted the same way);
//  * activations of the step's tokens are staged in LDS by the workgroup
//    (each thread one 16-byte piece per step, out-of-range pieces read zeros);
//  * each wave copies its rows' scale strip (and bias) into LDS with one
//    global_load_lds per 1 KB when its load cursor enters an item;
//  * with kSplit > 1 the partial accumulators of the kSplit waves of a
//    sub-tile are summed in LDS in slice order (fixed, so reproducible).
// The epilogue applies bias and (gate/up) the activation of
// device_common.h's activate(), rounding the activation to bf16.
//
// kSelf (gate/up of calls with at most kSelfRoutes routes, T <= kSelfTokens):
// no plan kernel runs before this launch.  Every workgroup routes the call's
// tokens and buckets its routes itself (route_plan.h: the plan kernel's own
// functions, so the same plan), keeping the pass list in LDS, and workgroup 0
// also writes the whole plan into the workspace for the down projection and
// the combine.  That takes one dependent launch, and its memory round trips,
// off a small call.
#include "kernels.h"
#include "route_plan.h"

namespace moe {

namespace {

constexpr int kXBufBytes = 16 * kXRowBytes;  // one staged step: 16 token slots x 4 blocks

// 64 lanes x 16 bytes from global memory into LDS at lds_off + 16*lane (lanes
// active in exec only).  M0 carries the LDS base; it is saved and restored.
// Used for the scale strips and biases, which a launch reads once per item:
// non-temporal like the weights (the sweep ~1% faster than cached).
__device__ __forceinline__ void lds_dma16(uint32_t lds_off, const void* gptr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_off)), "v"(gptr)
      : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bf16x8 decode8(uint32_t d, float s) {
  bf16x8 v;
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
  return v;
}

__device__ __forceinline__ uint4 as_uint4(const __attribute__((ext_vector_type(4))) uint32_t v) {
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every range: the load returns zeros
constexpr int kNonTemporal = 2;         // cache-policy operand of a buffer load: the "nt" bit

// Wave priority (0..3) from the items a workgroup still has to finish.  At
// equal priority a CU issues for its oldest waves first, so the workgroups
// dispatched last onto a CU stream slower; ranking by remaining work lets
// the ones that fell behind catch up, which shortens the launch's tail.  In
// its last item a workgroup also adds its dispatch rank on the CU (bid / 256
// under round-robin dispatch over 256 CUs), so that the workgroups dispatched
// last finish with the others: calls of one or two items per workgroup
// (T <= 4) end ~0.7 us sooner, the sweep ~0.7% faster.
__device__ __forceinline__ void set_priority(int remaining_items) {
  if (remaining_items >= 3) __builtin_amdgcn_s_setprio(3);
  else if (remaining_items == 2) __builtin_amdgcn_s_setprio(2);
  else if (remaining_items == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

}  // namespace

template <bool kGateUp, int kSplit, bool kPair, bool kSelf>
__global__ __launch_bounds__(256, 2) void stream_kernel(StreamArgs A) {
  static_assert(!(kGateUp && kPair), "pairing is for the down projection");
  static_assert(kGateUp || !kSelf, "only the gate/up launch plans the call");
  constexpr int kR = kStreamRing;
  constexpr int kTp = 16 / kSplit;         // routes per pass
  constexpr int kSub = 4 / kSplit;         // wave sub-tiles per item
  constexpr int kWaveRows = kPair ? 32 : 16;  // output rows per wave
  constexpr int kItemRows = kWaveRows * kSub;
  constexpr int kNW = (kGateUp || kPair) ? 2 : 1;  // weight row sets per wave
  extern __shared__ __align__(16) unsigned char lds[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int st = wave / kSplit, kp = wave - st * kSplit;  // sub-tile, reduction slice

  const int rows = A.rows, red = A.red;
  const int RB = red >> 5;                 // MX blocks per row
  const int NC = (RB + 3) >> 2;            // steps per row
  const int NCp = (NC + kSplit - 1) / kSplit;  // steps per slice (host guarantees >= kR)
  const int tiles = rows / kItemRows + (rows % kItemRows != 0);
  const int rows_e = (kGateUp ? 2 : 1) * rows;
  // second weight row set of a wave, in rows past the first: the up rows of
  // gate/up, the next 16 output rows of a paired down wave (in both weight
  // layouts row n + 16 sits 16 row lengths after row n)
  const int set1 = kGateUp ? rows : 16;
  // interleaved w13 (gate/up only): the wave's 16 gate rows and 16 up rows
  // are 32 consecutive stored rows, staged as one strip; scale of set j of
  // lane row r at strip[sub * j + srs * r + block]
  const int il = kGateUp ? A.il : 0;
  const int srs = il ? 2 * RB : RB;
  const int sub = il ? RB : 16 * RB;
  const uint32_t row_bytes = static_cast<uint32_t>(red >> 1);
  const uint32_t expert_bytes = static_cast<uint32_t>(rows_e) * row_bytes;
  const uint32_t bstride = block_stride(A.tiled);

  const int P = gridDim.x;
  const int bid = static_cast<int>(blockIdx.x);
  int N, n_my, e_idx, e_pass;
  uint4 ent = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (kSelf) {
    // the call's routing and pass list, in the staging buffers and strips
    // (unused until the first item is entered): ids [kSelfRoutes] | two sort
    // scratches of 128 ints | pass count | pass list [kSelfRoutes] at byte
    // 2048 | above 64 routes, the chunked bucketing's arrays from
    // kSelfLdsBase (the host sizes the launch's LDS for them; the pass list
    // ends below the item table, which is filled only after the last barrier)
    const PlanArgs& Q = A.self;
    int* ids_l = reinterpret_cast<int*>(lds);
    int* sort0 = ids_l + kSelfRoutes;
    int* sort1 = sort0 + 128;
    int* np_l = sort1 + 128;
    PassEntry* ptab = reinterpret_cast<PassEntry*>(lds + 2048);
    const int R = Q.T * Q.top_k;
    // the workgroups sharing a CU (bids 256 apart under the usual dispatch
    // order) give their single-wave jobs (a lone token's routing, the sort)
    // to different SIMDs: virtual wave vw = 0 is a different wave in each
    const int vw = (wave - (bid >> 8)) & 3;
    if (Q.logits != nullptr) {
      route_call<4, kSelfTokens / 4>(Q, ids_l, vw, lane, bid == 0);
    } else if (tid < R) {
      ids_l[tid] = Q.ids_in[tid];
      if (bid == 0 && Q.w_in != nullptr) {  // the plan keeps its own copy of the caller's routing
        Q.weights_ws[tid] = Q.w_in[tid];
        Q.ids_ws[tid] = Q.ids_in[tid];
      }
    }
    __syncthreads();
    if (R <= 64) {
      if (vw == 0) {
        const SmallBuckets b = sort_small(ids_l, R, Q.E_local, Q.offset, lane, sort0);
        small_pass_list(b, ptab, Q.pass_shift, lane, np_l);
      } else if (vw == 1 && bid == 0) {
        bucket_one_wave(Q, ids_l, R, lane, sort1);
      }
    } else if (vw == 0 || (vw == 1 && bid == 0)) {
      // the plan kernel's chunked bucketing: the pass list into LDS, and in
      // workgroup 0 a second wave writes the whole plan
      const int E_l = Q.E_local;
      int* cnt = reinterpret_cast<int*>(lds + kSelfLdsBase) + (vw == 0 ? 0 : self_bucket_ints(E_l, R));
      int* rank_s = cnt + E_l;
      int* routes_s = rank_s + R;
      int* base_e = routes_s + R;
      int* pass_base = base_e + E_l + 1;
      int* pass_base2 = pass_base + E_l;
      for (int e = lane; e < E_l; e += 64) cnt[e] = 0;
      __builtin_amdgcn_wave_barrier();
      if (vw == 0)
        bucket_chunks<false>(Q, ids_l, R, lane, cnt, rank_s, routes_s, base_e, pass_base, pass_base2, ptab,
                             Q.pass_shift, np_l);
      else
        bucket_chunks<true>(Q, ids_l, R, lane, cnt, rank_s, routes_s, base_e, pass_base, pass_base2);
    }
    __syncthreads();
    N = min(max(*np_l, 0), A.max_passes) * tiles;
    if (bid >= N) return;  // whole workgroup
    n_my = min((N - 1 - bid) / P + 1, kStreamMaxItems);
    e_idx = bid + (tid >> 2) * P;
    e_pass = e_idx / tiles;
    if (tid < 4 * n_my) ent = reinterpret_cast<const uint4*>(ptab + e_pass)[tid & 3];
  } else {
    // The pass entries this workgroup may hold are requested before the plan
    // header is read, bounded by the host's pass bound (so always inside the
    // pass list; entries past the plan's count are dropped below): the two
    // requests share one memory round trip.
    const int n_bound = A.max_passes * tiles;
    const int n_req = bid < n_bound ? min((n_bound - 1 - bid) / P + 1, kStreamMaxItems) : 0;
    e_idx = bid + (tid >> 2) * P;  // item of this thread's entry part
    e_pass = e_idx / tiles;
    if (tid < 4 * n_req) ent = reinterpret_cast<const uint4*>(A.passes + e_pass)[tid & 3];
    // (the header's address depends on the pass bound, 0 for any valid one, so
    // that its request does not come before the bound's and the wait for the
    // bound does not also wait for it; both values are taken before the checks
    // so that neither request sinks below them)
    const Plan* plan = A.plan + ((A.max_passes >> 31) & 1);
    const uint32_t plan_key = plan->key;
    const int plan_passes = A.second_list ? plan->n_passes2 : plan->n_passes;
    asm volatile("" ::"v"(ent.x), "v"(ent.y), "v"(ent.z), "v"(ent.w), "s"(plan_key), "s"(plan_passes));
    // a workspace without this call's plan gives no output; pass entries are
    // clamped to the host's bounds, so no plan value reaches outside a buffer
    if (plan_key != A.key) return;
    N = min(max(plan_passes, 0), A.max_passes) * tiles;
    if (bid >= N) return;  // whole workgroup
    // items of this workgroup (the host's grid keeps this <= kStreamMaxItems; the
    // min only guards the LDS table)
    n_my = min((N - 1 - bid) / P + 1, kStreamMaxItems);
  }
  const int total = n_my * NCp;

  // LDS: [2][kXBufBytes] staged activations | per (buffer, wave) scale strips
  // and bias | kSplit > 1: partial sums [4 waves][64 lanes][8] | item table
  const int strip_bytes = 16 * RB;  // 16 rows x RB scale bytes, one weight row set
  const int sw = kNW * strip_bytes + kNW * 32;  // + bias of 16 rows (bf16) per row set
  const int sw16 = (sw + 15) & ~15;
  unsigned char* xbuf = lds;
  unsigned char* sbuf = lds + 2 * kXBufBytes;
  float* redbuf = reinterpret_cast<float*>(sbuf + 2 * 4 * sw16);
  const uint32_t sbuf_off = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sbuf));

  // staging role: thread u stages piece (u & 15) of token slot u >> 4, which is
  // route tt of slice `spart` of the pass
  const int ts = tid >> 4, piece = tid & 15;
  const int spart = ts / kTp, stt = ts - spart * kTp;
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.in), 0, A.in_bytes, 0x00020000);

  // ---- this workgroup's items: pass entries copied to LDS once -------------
  // item i is b + i*P; its entry is the pass (b + i*P) / tiles, and the copy's
  // pad0 field holds the tile.  The host sizes the grid so that n_my <= kStreamMaxItems.
  PassEntry* etab = reinterpret_cast<PassEntry*>(redbuf + (kSplit > 1 ? 4 * 64 * 8 : 0));
  if (tid < 4 * n_my) {
    if ((tid & 3) == 0) ent.w = static_cast<uint32_t>(e_idx - e_pass * tiles);
    reinterpret_cast<uint4*>(etab + (tid >> 2))[tid & 3] = ent;
  }
  __syncthreads();

  // load cursor (item li, step ls) and what it needs of item li
  int li = 0, ls = 0;
  int l_e = 0, l_nt = 0, l_p = 0, l_row0 = 0;  // uniform
  uint32_t l_wo = 0, l_wo1 = 0;                // this lane's row offsets (set 0, set 1) in the expert
  uint32_t l_xoff = 0;                         // staging thread's activation row (bytes)
  __amdgpu_buffer_rsrc_t wrs;                  // weights of expert l_e

  // enter item li: weights, staging row, strip DMA
  auto enter_load_item = [&]() {
    const PassEntry* pe = etab + li;
    l_e = min(max(__builtin_amdgcn_readfirstlane(pe->e), 0), A.E_local - 1);
    l_p = min(max(__builtin_amdgcn_readfirstlane(pe->p), 0), A.R - 1);
    l_nt = min(max(__builtin_amdgcn_readfirstlane(pe->nt), 0), min(kTp, A.R - l_p));
    l_row0 = __builtin_amdgcn_readfirstlane(pe->pad0) * kItemRows;
    const int tt = stt < l_nt ? stt : 0;
    const int xrow = A.tok_from_pass ? static_cast<int>(pe->rte[tt]) / A.top_k : l_p + tt;
    l_xoff = static_cast<uint32_t>(xrow) * static_cast<uint32_t>(red) * 2u;
    // this wave's sub-tile: rows are a multiple of kWaveRows, so a sub-tile is
    // all in or all out; an out sub-tile re-reads the expert's last rows (results dropped)
    const int row0w = min(l_row0 + st * kWaveRows, rows - kWaveRows);
    const int n = row0w + r;
    l_wo = row_offset(kGateUp ? gate_row(n, il) : n, row_bytes, A.tiled);
    l_wo1 = row_offset(kGateUp ? up_row(n, rows, il) : n + set1, row_bytes, A.tiled);
    wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A.wp) + static_cast<size_t>(l_e) * expert_bytes, 0,
                                            expert_bytes, 0x00020000);
    // scale strip(s) and bias of rows row0w..row0w+15 into this wave's slot
    const uint32_t dst = sbuf_off + static_cast<uint32_t>(((li & 1) * 4 + wave) * sw16);
    const uint8_t* s0 = A.ws + (static_cast<size_t>(l_e) * rows_e + (il ? 2 * row0w : row0w)) * RB;
    const int pieces0 = il ? 2 * RB : RB;  // 16 B pieces: 16 rows, or 32 interleaved rows
    for (int m = 0; m * 64 < pieces0; ++m) {
      if (m * 64 + lane < pieces0) lds_dma16(dst + m * 1024, s0 + (m * 64 + lane) * 16);
    }
    if (kNW == 2 && !il) {
      const uint8_t* s1 = s0 + static_cast<size_t>(set1) * RB;
      for (int m = 0; m * 64 < RB; ++m) {
        if (m * 64 + lane < RB) lds_dma16(dst + strip_bytes + m * 1024, s1 + (m * 64 + lane) * 16);
      }
    }
    if (A.bias != nullptr && il && lane < 4) {
      // 16 interleaved (gate, up) bias pairs
      lds_dma16(dst + kNW * strip_bytes, A.bias + static_cast<size_t>(l_e) * rows_e + 2 * row0w + lane * 8);
    } else if (A.bias != nullptr && lane < 2) {
      const uint16_t* b0 = A.bias + static_cast<size_t>(l_e) * rows_e + row0w;
      lds_dma16(dst + kNW * strip_bytes, b0 + lane * 8);
      if (kNW == 2) lds_dma16(dst + kNW * strip_bytes + 32, b0 + set1 + lane * 8);
    }
  };

  // ---- register ring ------------------------------------------------------
  uint4 rw0[kR], rw1[kR], rx[kR];
  auto load_step = [&](int slot) {
    // weights of step (li, ls) for this lane; out-of-range blocks and steps
    // past this workgroup's items read zeros.  Every weight byte is read
    // once per launch, so the loads are non-temporal (aux bit 1, "nt"):
    // gpt-oss-120b T = 32 gate/up 125 -> 112.5 us, down 69 -> 62 us.
    const int b = (kp * NCp + ls) * 4 + q;
    const bool ok = li < n_my && b < RB;
    const uint32_t o0 = ok ? l_wo + bstride * b : kOob;
    rw0[slot] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(wrs, o0, 0, kNonTemporal));
    if (kNW == 2) {
      const uint32_t o1 = ok ? l_wo1 + bstride * b : kOob;
      rw1[slot] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(wrs, o1, 0, kNonTemporal));
    }
    // activation piece of the staging thread
    const int xb = (spart * NCp + ls) * 4 + (piece >> 2);
    const bool xok = li < n_my && stt < l_nt && xb < RB;
    const uint32_t xo = xok ? l_xoff + static_cast<uint32_t>(((spart * NCp + ls) * 16 + piece) * 16) : kOob;
    rx[slot] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(xrs, xo, 0, 0));
  };
  auto advance_load = [&]() {
    if (++ls == NCp) {
      ls = 0;
      ++li;
      if (li < n_my) enter_load_item();
    }
  };
  auto xstore = [&](int step, const uint4& v) {
    *reinterpret_cast<uint4*>(xbuf + (step & 1) * kXBufBytes + ts * kXRowBytes + piece * 16) = v;
  };

  // ---- prologue: item 0 entered, steps 0..kR-1 in flight, step 0 staged ----
  enter_load_item();
  // compute cursor (item ci, step cs) and what the epilogue needs of item ci
  int ci = 0, cs = 0;
  int c_nt = l_nt, c_p = l_p, c_row0 = l_row0;
#pragma unroll
  for (int s = 0; s < kR; ++s) {
    load_step(s);
    advance_load();
  }
  xstore(0, rx[0]);
  lds_barrier();

  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  // the staged column of token c of this lane's B operand
  const int bts = kp * kTp + (r % kTp);

  // one step of the compute cursor, ring slot s (a compile-time constant)
  auto step = [&](const int g, const int s) {
    if (cs == 0) {
      set_priority(n_my - ci + (n_my - ci == 1 ? ((bid >> 8) & 3) : 0));
      // strip of item ci: its DMA was issued before this step's weight
      // loads, so once they have arrived (in-order completion) the strip has
      asm volatile("" ::"v"(rw0[s].x), "v"(rw0[s].y), "v"(rw0[s].z), "v"(rw0[s].w) : "memory");
    }
    const unsigned char* strip = sbuf + ((ci & 1) * 4 + wave) * sw16;
    // blocks past the row were loaded as zeros, which any finite scale keeps
    // zero: the scales are read unconditionally at a clamped index, so no
    // exec-masked branch (and its own LDS wait) opens the step
    const int bs = min((kp * NCp + cs) * 4 + q, RB - 1);
    const float sc0 = e8m0_to_f32(strip[r * srs + bs]);
    const float sc1 = kNW == 2 ? e8m0_to_f32(strip[sub + r * srs + bs]) : 0.0f;
    const unsigned char* xb = xbuf + (g & 1) * kXBufBytes + bts * kXRowBytes + q * 64;
    const uint32_t d0[4] = {rw0[s].x, rw0[s].y, rw0[s].z, rw0[s].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x8 bx = *reinterpret_cast<const bf16x8*>(xb + k * 16);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8(d0[k], sc0), bx, acc0, 0, 0, 0);
      if (kNW == 2) {
        const uint32_t d1 = k == 0 ? rw1[s].x : k == 1 ? rw1[s].y : k == 2 ? rw1[s].z : rw1[s].w;
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8(d1, sc1), bx, acc1, 0, 0, 0);
      }
    }
    const bool last = cs == NCp - 1;
    // At the last step of item ci the load cursor is in item ci + 1 (it
    // entered it kR steps ago and enters ci + 2 no earlier than this
    // step's refill, as NCp >= kR): take ci + 1's epilogue data, and ci's
    // bias, before the refill may reuse ci's strip slot.
    int nx_nt = 0, nx_p = 0, nx_row0 = 0;
    float b0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, b1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (last) {
      nx_nt = l_nt;
      nx_p = l_p;
      nx_row0 = l_row0;
      if (A.bias != nullptr) {
        const uint16_t* bb = reinterpret_cast<const uint16_t*>(strip + kNW * strip_bytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b0[i] = bf16_bits_to_f32(bb[il ? 2 * (4 * q + i) : 4 * q + i]);
          if (kNW == 2) b1[i] = bf16_bits_to_f32(bb[il ? 2 * (4 * q + i) + 1 : 16 + 4 * q + i]);
        }
      }
      if (kSplit > 1) {
        float* my = redbuf + (wave * 64 + lane) * 8;
        *reinterpret_cast<f32x4*>(my) = acc0;
        if (kNW == 2) *reinterpret_cast<f32x4*>(my + 4) = acc1;
      }
    }
    // refill this slot with step g + kR, stage step g + 1
    load_step(s);
    advance_load();
    xstore(g + 1, rx[(s + 1) % kR]);  // past the last step: an unread buffer
    lds_barrier();

    if (last) {
      if (kSplit > 1 && kp == 0) {
#pragma unroll
        for (int j = 1; j < kSplit; ++j) {
          const float* o = redbuf + ((wave + j) * 64 + lane) * 8;
          acc0 += *reinterpret_cast<const f32x4*>(o);
          if (kNW == 2) acc1 += *reinterpret_cast<const f32x4*>(o + 4);
        }
      }
      // lane holds rows row0w + 4q + i (i < 4) of route r of the pass
      const int row0w = c_row0 + st * kWaveRows;
      if (kp == 0 && row0w < rows && r < c_nt && r < kTp) {
        const int rl = 4 * q;
        const size_t p = static_cast<size_t>(c_p + r);
        if (kGateUp) {
          uint16_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            h[i] = f32_to_bf16_rne(activate(acc0[i] + b0[i], acc1[i] + b1[i], A.act_kind, A.alpha, A.limit));
          uint2 pk;
          pk.x = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
          pk.y = static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16);
          *reinterpret_cast<uint2*>(A.a_out + p * rows + row0w + rl) = pk;
        } else {
          const size_t orow = A.o_by_route ? static_cast<size_t>(min(static_cast<int>(etab[ci].rte[r]), A.R - 1)) : p;
          *reinterpret_cast<float4*>(A.o_out + orow * rows + row0w + rl) =
              make_float4(acc0[0] + b0[0], acc0[1] + b0[1], acc0[2] + b0[2], acc0[3] + b0[3]);
          if (kPair)
            *reinterpret_cast<float4*>(A.o_out + orow * rows + row0w + 16 + rl) =
                make_float4(acc1[0] + b1[0], acc1[1] + b1[1], acc1[2] + b1[2], acc1[3] + b1[3]);
        }
      }
      acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      acc1 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      ++ci;
      cs = 0;
      c_nt = nx_nt;
      c_p = nx_p;
      c_row0 = nx_row0;
    } else {
      ++cs;
    }
  };

  // full rounds of kR steps, then the remainder; the split keeps every
  // round's path free of skipped steps, so the ring's waits stay partial
  int g0 = 0;
  for (; g0 + kR <= total; g0 += kR) {
#pragma unroll
    for (int s = 0; s < kR; ++s) step(g0 + s, s);
  }
#pragma unroll
  for (int s = 0; s < kR - 1; ++s)
    if (g0 + s < total) step(g0 + s, s);
}

template __global__ void stream_kernel<true, 1, false, false>(StreamArgs);
template __global__ void stream_kernel<true, 2, false, false>(StreamArgs);
template __global__ void stream_kernel<true, 4, false, false>(StreamArgs);
template __global__ void stream_kernel<false, 1, false, false>(StreamArgs);
template __global__ void stream_kernel<false, 2, false, false>(StreamArgs);
template __global__ void stream_kernel<false, 4, false, false>(StreamArgs);
template __global__ void stream_kernel<false, 1, true, false>(StreamArgs);
template __global__ void stream_kernel<false, 2, true, false>(StreamArgs);
template __global__ void stream_kernel<false, 4, true, false>(StreamArgs);
template __global__ void stream_kernel<true, 1, false, true>(StreamArgs);
template __global__ void stream_kernel<true, 2, false, true>(StreamArgs);
template __global__ void stream_kernel<true, 4, false, true>(StreamArgs);

}  // namespace moe
