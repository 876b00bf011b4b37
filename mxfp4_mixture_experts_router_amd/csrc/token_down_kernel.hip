// One-token decode calls: the down projection of every local route and the
// token sum in one launch.
//
// "MXFP4 MoE decode kernels" (Design; Fused epilogues): a decode call streams
// each touched expert's w2 once, adds the bias per route, and sums a token's
// routes with their routing weights.  With one token the call's routes are
// that token's (at most top_k experts), so one workgroup can hold every
// route's share of a 16-row output tile.  Wave (j, s) computes route slot j
// over reduction slice s exactly as stream_kernel<false, 4, *> computes the
// same rows: the same 16-byte weight loads (tiled or row layout, blocks past
// the row read as zeros), the same scale byte (at a clamped block index), the
// same decode and v_mfma_f32_16x16x32_bf16 sequence, so the same partial sums.
// The partial sums meet in LDS; one wave adds the four slices in slice order
// and the bias, as the stream kernel's epilogue does, then the routing-
// weighted route values in route order with combine_kernel's roundings.  That
// takes the per-route fp32 rows, their round trip through memory and the
// combine launch off the smallest calls.
//
// Layout: K / 16 workgroups of 16 waves per token (grid row = token; the
// host launches it for one-token calls, where it measured faster than the
// separate launches, and not above); every column of a wave's MFMAs
// carries the same intermediate row (its route's), staged once in LDS with
// each row padded to the four slices' steps (zeros past I).  A route slot
// without a local route reads its weights through an empty buffer range
// (zeros, no traffic) and is skipped by the sum.
#include "kernels.h"

namespace moe {

namespace {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every range: the load returns zeros
constexpr int kNonTemporal = 2;         // cache-policy operand of a buffer load: the "nt" bit
constexpr int kRing = 8;                // steps in flight per wave: every step of a slice up to I = 4096
constexpr int kXPer = 4;                // staged 16-byte pieces per thread (host: steps <= 15)

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

// A workgroup barrier that orders LDS only, so that it does not also wait for
// the weight loads still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace

__global__ __launch_bounds__(1024) void token_down_kernel(TokenDownArgs A) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int j = wave >> 2, kp = wave & 3;  // route slot, reduction slice
  const int n0 = static_cast<int>(blockIdx.x) * 16;
  const int t = static_cast<int>(blockIdx.y);  // token
  const int k = A.top_k, R = A.T * A.top_k;

  // the token's route slots (plan position, expert id, weight) are requested
  // together with the plan's key, at indices valid for any plan, so that one
  // memory round trip brings all of them; the empty asm takes every value
  // before the key check, so no request sinks below it
  int pr_[kTokenRoutes], id_[kTokenRoutes];
  float w_[kTokenRoutes];
#pragma unroll
  for (int i = 0; i < kTokenRoutes; ++i) {
    const int ii = t * k + min(i, k - 1);
    pr_[i] = A.pos[ii];
    id_[i] = A.ids[ii];
    w_[i] = A.weights[ii];
  }
  const uint32_t plan_key = A.plan->key;
  asm volatile("" ::"s"(plan_key), "s"(pr_[0]), "s"(pr_[1]), "s"(pr_[2]), "s"(pr_[3]), "s"(id_[0]), "s"(id_[1]),
               "s"(id_[2]), "s"(id_[3]), "s"(w_[0]), "s"(w_[1]), "s"(w_[2]), "s"(w_[3]));
  if (plan_key != A.key) return;  // no plan of this call in the workspace (whole workgroup)

  const int K = A.K, I = A.I, RB = I >> 5, NCp = A.steps;
  const int xrow_bytes = 4 * NCp * 256;  // one staged intermediate row

  // slot i: plan position (-1: not local), expert, weight; a position
  // outside [0, T * top_k) counts as not local, as in the combine
  int pv[kTokenRoutes], ev[kTokenRoutes];
  float wv[kTokenRoutes];
#pragma unroll
  for (int i = 0; i < kTokenRoutes; ++i) {
    const bool in = i < k;
    pv[i] = (in && pr_[i] >= 0 && pr_[i] < R) ? pr_[i] : -1;
    ev[i] = in ? min(max(id_[i] - A.offset, 0), A.E_local - 1) : 0;
    wv[i] = in ? w_[i] : 0.0f;
  }
  int pj = pv[0], e = ev[0];
#pragma unroll
  for (int i = 1; i < kTokenRoutes; ++i) {
    pj = j == i ? pv[i] : pj;
    e = j == i ? ev[i] : e;
  }

  // the sum's bias values (wave 0, lane m < 16 sums row n0 + m), requested
  // before the rows and weights so that they are in when the sum starts
  uint16_t bv[kTokenRoutes] = {0, 0, 0, 0};
  if (wave == 0 && A.bias != nullptr) {
#pragma unroll
    for (int i = 0; i < kTokenRoutes; ++i) bv[i] = A.bias[static_cast<size_t>(ev[i]) * K + n0 + (lane & 15)];
  }

  // this lane's weight row n0 + r of expert e; an empty range for a slot
  // without a local route
  const uint32_t row_bytes = static_cast<uint32_t>(I >> 1);
  const uint32_t expert_bytes = static_cast<uint32_t>(K) * row_bytes;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A.wp) + static_cast<size_t>(e) * expert_bytes, 0, pj >= 0 ? expert_bytes : 0u, 0x00020000);
  const uint32_t wo = row_offset(n0 + r, row_bytes, A.tiled);
  const uint32_t bstride = block_stride(A.tiled);
  const uint8_t* __restrict__ srow = A.ws + (static_cast<size_t>(e) * K + n0 + r) * RB;

  uint4 rw[kRing];
  uint32_t rsc[kRing];
  auto load = [&](int ls, int slot) {
    const int b = (kp * NCp + ls) * 4 + q;
    const bool ok = ls < NCp && b < RB;
    const __attribute__((ext_vector_type(4))) uint32_t v =
        __builtin_amdgcn_raw_buffer_load_b128(wrs, ok ? wo + bstride * b : kOob, 0, kNonTemporal);
    rw[slot] = make_uint4(v[0], v[1], v[2], v[3]);
    rsc[slot] = srow[min(b, RB - 1)];  // the stream kernel's clamped scale index
  };

  // the intermediate rows' pieces are requested first, then the weights of
  // the first kRing steps, so that staging the rows in LDS waits only for
  // the rows; pieces past I (and of slots without a local route) are zeros
  const int XP = xrow_bytes / 16;  // 16-byte pieces per staged row
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.a), 0, A.a_bytes, 0x00020000);
  uint4 xv[kXPer];
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int u = tid + 1024 * m;
    const int js = u / XP, pp = u - js * XP;
    int pr = -1;
#pragma unroll
    for (int i = 0; i < kTokenRoutes; ++i) pr = js == i ? pv[i] : pr;
    const uint32_t off = (pr >= 0 && pp * 16 < I * 2)
                             ? static_cast<uint32_t>(pr) * static_cast<uint32_t>(I) * 2u + static_cast<uint32_t>(pp) * 16u
                             : kOob;
    const __attribute__((ext_vector_type(4))) uint32_t v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    xv[m] = make_uint4(v[0], v[1], v[2], v[3]);
  }
#pragma unroll
  for (int s = 0; s < kRing; ++s) load(s, s);
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int u = tid + 1024 * m;
    if (u < kTokenRoutes * XP) *reinterpret_cast<uint4*>(lds + u * 16) = xv[m];
  }
  lds_barrier();

  // the slice's steps: lane (r, q) holds block 4c + q of row r, and reads the
  // same block of its route's intermediate row for each of the 4 MFMAs
  const unsigned char* xrow = lds + j * xrow_bytes + kp * NCp * 256 + q * 64;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto step = [&](int g, int s) {
    const float sc = e8m0_to_f32(rsc[s]);
    const uint32_t d[4] = {rw[s].x, rw[s].y, rw[s].z, rw[s].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x8 bx = *reinterpret_cast<const bf16x8*>(xrow + g * 256 + k * 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode8(d[k], sc), bx, acc, 0, 0, 0);
    }
  };
  int g0 = 0;
  for (; g0 + kRing <= NCp; g0 += kRing) {
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      step(g0 + s, s);
      load(g0 + s + kRing, s);
    }
  }
#pragma unroll
  for (int s = 0; s < kRing - 1; ++s)
    if (g0 + s < NCp) step(g0 + s, s);

  // lane (0, q) holds rows n0 + 4q + i of its route slot and slice
  float* red = reinterpret_cast<float*>(lds + kTokenRoutes * xrow_bytes);  // [16 waves][16 rows]
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * 16 + 4 * q + i] = acc[i];
  }
  lds_barrier();
  if (wave == 0 && lane < 16) {
    const int n = n0 + lane;
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < kTokenRoutes; ++i) {
      if (pv[i] < 0) continue;
      // the slices in order, then the bias (0 without one), as the stream kernel's epilogue
      float o = red[(4 * i) * 16 + lane];
      o += red[(4 * i + 1) * 16 + lane];
      o += red[(4 * i + 2) * 16 + lane];
      o += red[(4 * i + 3) * 16 + lane];
      const float b = bf16_bits_to_f32(bv[i]);  // +0 without a bias
      o = o + b;
      y = __fadd_rn(y, __fmul_rn(wv[i], o));
    }
    A.out[static_cast<size_t>(t) * K + n] = f32_to_bf16_rne(y);
  }
}

}  // namespace moe
