// Grouped expert kernels of the decode regime (few tokens per expert):
// the gate/up projection with its activation, the down projection, the
// routing-weighted combine, and the dequantisation hook.
//
// What they compute: "MXFP4 MoE decode kernels", Design (x -> gate/up GEMV +
// bias + activation -> bf16 intermediate; intermediate -> down GEMV +
// routing-weighted bias + weighted sum per token) and Design, Fused
// epilogues.  Weights are read once, straight from the packed layout (Design,
// Read the served layout), and decoded in registers.
//
// Mapping on CDNA4: a workgroup of 256 lanes owns one work item, 16 rows of
// one touched expert (16 lane-groups x 16 lanes).  Lane q of a group loads the
// 16-byte MX blocks q, q+16, q+32, ... of its row (256 contiguous bytes per
// group per step, coalesced), decodes them with the scaled FP4 converts and
// multiplies with v_dot2_f32_bf16 against activations staged in LDS.  The 16
// partial sums of a row are combined with DPP row operations.  Work items are
// (touched expert, row tile) pairs taken from the bucketing plan, so the grid
// never depends on host knowledge of the routing.
#include "device_common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void w13_gemv_kernel(W13Args A) {
  extern __shared__ uint4 xs[];  // [kGemvTokens][K/8] bf16 activations
  const int K = A.K, I = A.I;
  const int KB = K >> 5;
  const int KV = K >> 3;
  const int tiles = I / kRowsPerTile;
  const int n_work = A.plan->n_touched * tiles;
  const int g = threadIdx.x >> 4, q = threadIdx.x & 15;

  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int e = A.touched[w / tiles];
    const int n = (w % tiles) * kRowsPerTile + g;
    const int p0 = A.offsets[e];
    const int Te = A.offsets[e + 1] - p0;
    const size_t grow = static_cast<size_t>(e) * 2 * I + n;
    const size_t urow = grow + I;
    const uint4* gq = reinterpret_cast<const uint4*>(A.w13p + grow * (K >> 1));
    const uint4* uq = reinterpret_cast<const uint4*>(A.w13p + urow * (K >> 1));
    const uint8_t* gs = A.w13s + grow * KB;
    const uint8_t* us = A.w13s + urow * KB;
    float bg = 0.0f, bu = 0.0f;
    if (A.b13 != nullptr) {
      bg = bf16_bits_to_f32(A.b13[grow]);
      bu = bf16_bits_to_f32(A.b13[urow]);
    }
    for (int t0 = 0; t0 < Te; t0 += kGemvTokens) {
      const int nt = min(kGemvTokens, Te - t0);
      __syncthreads();
      for (int i = threadIdx.x; i < nt * KV; i += blockDim.x) {
        const int tt = i / KV, c = i - tt * KV;
        const int tok = A.routes[p0 + t0 + tt] / A.top_k;
        xs[tt * KV + c] = reinterpret_cast<const uint4*>(A.x + static_cast<size_t>(tok) * K)[c];
      }
      __syncthreads();
      float ag[kGemvTokens], au[kGemvTokens];
#pragma unroll
      for (int tt = 0; tt < kGemvTokens; ++tt) ag[tt] = au[tt] = 0.0f;
      for (int b = q; b < KB; b += 16) {
        const uint4 gw4 = gq[b];
        const uint4 uw4 = uq[b];
        bf16x2 gw[16], uw[16];
        decode_block_bf16(gw4, e8m0_to_f32(gs[b]), gw);
        decode_block_bf16(uw4, e8m0_to_f32(us[b]), uw);
#pragma unroll
        for (int tt = 0; tt < kGemvTokens; ++tt) {
          if (tt < nt) {
            const uint4* xp = xs + tt * KV + b * 4;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint4 xv = xp[c];
              ag[tt] = dot2(gw[4 * c + 0], xv.x, ag[tt]);
              ag[tt] = dot2(gw[4 * c + 1], xv.y, ag[tt]);
              ag[tt] = dot2(gw[4 * c + 2], xv.z, ag[tt]);
              ag[tt] = dot2(gw[4 * c + 3], xv.w, ag[tt]);
              au[tt] = dot2(uw[4 * c + 0], xv.x, au[tt]);
              au[tt] = dot2(uw[4 * c + 1], xv.y, au[tt]);
              au[tt] = dot2(uw[4 * c + 2], xv.z, au[tt]);
              au[tt] = dot2(uw[4 * c + 3], xv.w, au[tt]);
            }
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < kGemvTokens; ++tt) {
        ag[tt] = row16_sum(ag[tt]);
        au[tt] = row16_sum(au[tt]);
      }
      if (q == 0) {
#pragma unroll
        for (int tt = 0; tt < kGemvTokens; ++tt) {
          if (tt < nt) {
            const float act = activate(ag[tt] + bg, au[tt] + bu, A.act, A.alpha, A.limit);
            A.a[static_cast<size_t>(p0 + t0 + tt) * I + n] = f32_to_bf16_rne(act);
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void w2_gemv_kernel(W2Args A) {
  extern __shared__ uint4 as_[];  // [kGemvTokens][I/8] bf16 intermediate rows
  const int K = A.K, I = A.I;
  const int IB = I >> 5;
  const int IV = I >> 3;
  const int tiles = K / kRowsPerTile;
  const int n_work = A.plan->n_touched * tiles;
  const int g = threadIdx.x >> 4, q = threadIdx.x & 15;

  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int e = A.touched[w / tiles];
    const int kk = (w % tiles) * kRowsPerTile + g;
    const int p0 = A.offsets[e];
    const int Te = A.offsets[e + 1] - p0;
    const size_t row = static_cast<size_t>(e) * K + kk;
    const uint4* wq = reinterpret_cast<const uint4*>(A.w2p + row * (I >> 1));
    const uint8_t* ws = A.w2s + row * IB;
    const float bias = A.b2 != nullptr ? bf16_bits_to_f32(A.b2[row]) : 0.0f;
    for (int t0 = 0; t0 < Te; t0 += kGemvTokens) {
      const int nt = min(kGemvTokens, Te - t0);
      __syncthreads();
      for (int i = threadIdx.x; i < nt * IV; i += blockDim.x) {
        const int tt = i / IV, c = i - tt * IV;
        as_[tt * IV + c] = reinterpret_cast<const uint4*>(A.a + static_cast<size_t>(p0 + t0 + tt) * I)[c];
      }
      __syncthreads();
      float acc[kGemvTokens];
#pragma unroll
      for (int tt = 0; tt < kGemvTokens; ++tt) acc[tt] = 0.0f;
      for (int b = q; b < IB; b += 16) {
        const uint4 w4 = wq[b];
        bf16x2 wv[16];
        decode_block_bf16(w4, e8m0_to_f32(ws[b]), wv);
#pragma unroll
        for (int tt = 0; tt < kGemvTokens; ++tt) {
          if (tt < nt) {
            const uint4* ap = as_ + tt * IV + b * 4;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint4 av = ap[c];
              acc[tt] = dot2(wv[4 * c + 0], av.x, acc[tt]);
              acc[tt] = dot2(wv[4 * c + 1], av.y, acc[tt]);
              acc[tt] = dot2(wv[4 * c + 2], av.z, acc[tt]);
              acc[tt] = dot2(wv[4 * c + 3], av.w, acc[tt]);
            }
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < kGemvTokens; ++tt) acc[tt] = row16_sum(acc[tt]);
      if (q == 0) {
#pragma unroll
        for (int tt = 0; tt < kGemvTokens; ++tt) {
          if (tt < nt) A.o[static_cast<size_t>(p0 + t0 + tt) * K + kk] = acc[tt] + bias;
        }
      }
    }
  }
}

// y[t, :] = sum over j (ascending) of w[t, j] * o[pos(t, j), :] for the
// token's local routes; zeros for a token without one.  Fixed order, no
// atomics, so the result is reproducible bit for bit.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs A) {
  const int t = blockIdx.y;
  const int k4 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (k4 >= A.K) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < A.top_k; ++j) {
    const int r = t * A.top_k + j;
    const int p = A.pos[r];
    if (p < 0) continue;
    const float wt = A.weights[r];
    const float4 o = *reinterpret_cast<const float4*>(A.o + static_cast<size_t>(p) * A.K + k4);
    acc.x = __fadd_rn(acc.x, __fmul_rn(wt, o.x));
    acc.y = __fadd_rn(acc.y, __fmul_rn(wt, o.y));
    acc.z = __fadd_rn(acc.z, __fmul_rn(wt, o.z));
    acc.w = __fadd_rn(acc.w, __fmul_rn(wt, o.w));
  }
  uint2 packed;
  packed.x = static_cast<uint32_t>(f32_to_bf16_rne(acc.x)) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.y)) << 16);
  packed.y = static_cast<uint32_t>(f32_to_bf16_rne(acc.z)) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.w)) << 16);
  *reinterpret_cast<uint2*>(A.out + static_cast<size_t>(t) * A.K + k4) = packed;
}

// One thread per 32-value MX block: 16 packed bytes + 1 scale byte.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ scales, int64_t n_blocks,
                                                      int out_bf16, void* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_blocks) return;
  const uint4 q = reinterpret_cast<const uint4*>(packed)[i];
  const float s = e8m0_to_f32(scales[i]);
  if (out_bf16) {
    bf16x2 v[16];
    decode_block_bf16(q, s, v);
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + i * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 u;
      u.x = __builtin_bit_cast(uint32_t, v[4 * c + 0]);
      u.y = __builtin_bit_cast(uint32_t, v[4 * c + 1]);
      u.z = __builtin_bit_cast(uint32_t, v[4 * c + 2]);
      u.w = __builtin_bit_cast(uint32_t, v[4 * c + 3]);
      o[c] = u;
    }
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + i * 32);
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x2 v[4];
      decode_dword_f32(d[c], s, v);
      o[2 * c + 0] = make_float4(v[0][0], v[0][1], v[1][0], v[1][1]);
      o[2 * c + 1] = make_float4(v[2][0], v[2][1], v[3][0], v[3][1]);
    }
  }
}

}  // namespace moe
