// Scaled-FP4 form of the MFMA regime (experts with many routes).
//
// "MXFP4 MoE decode kernels" (Design) computes each touched expert's product
// from the packed weights, unpacking E2M1 with its E8M0 block scale on the
// fly.  gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes the packed E2M1
// blocks and their E8M0 scales as they are stored, with no unpack at all, but
// wants the other operand in an 8-bit MX format.  The activations therefore
// go through mx8_split_kernel first: each bf16 row becomes hi + lo, two E4M3
// parts under one E8M0 scale each (hi: the row rounded to E4M3 under the
// scale its largest magnitude sets; lo: the exact remainder rounded the same
// way), which carries about as many significant bits as the bf16 row does.
// mfma_fp4_kernel is then mfma_kernel with the decode and the four bf16
// MFMAs of a 128-value chunk replaced by two scaled MFMAs (hi, lo).
//
// Operand layouts of the 16x16x128 scaled MFMA (A = E2M1, B = E4M3), as
// measured on the device:
//   A: lane l holds row l % 16, the 32 values of K-block l / 16 (16 bytes,
//      element j in nibble j, low nibble first), and that block's scale;
//   B: lane l holds column l % 16, values 16g .. 16g + 15 in bytes 0..15 and
//      64 + 16g .. 64 + 16g + 15 in bytes 16..31 (g = l / 16); the scale of
//      K-block b is taken from lane group b;
//   D: lane l, element i is row 4 (l / 16) + i, column l % 16.
// The A layout is the stream of a packed MXFP4 row as stored: lane (r, q)
// loads block q of row r, as in mfma_kernel.
#include "kernels.h"
#include "list_common.h"

#include <type_traits>

namespace moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t bf16_lo(uint32_t w) { return w << 16; }
__device__ __forceinline__ uint32_t bf16_hi(uint32_t w) { return w & 0xffff0000u; }

// Largest value over the workgroup (256 threads), every thread gets it.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();  // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// E8M0 exponent s of the scale 2^(s - 127) under which |x| <= amax maps below
// 2^8 (E4M3 holds up to 448, so no value overflows), kept in [1, 254].
__device__ __forceinline__ int split_scale(float amax) {
  if (!(amax > 0.0f)) return 127;
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 127;  // floor(log2(amax)) (>= -126 here)
  return min(max(e - 7 + 127, 1), 254);
}

__device__ __forceinline__ float pow2(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }

// Eight values to E4M3 (round to nearest even), bytes in value order.
__device__ __forceinline__ uint2 to_e4m3x8(const float (&v)[8], float mul) {
  uint32_t a = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * mul, v[1] * mul, 0u, false);
  a = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * mul, v[3] * mul, a, true);
  uint32_t b = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * mul, v[5] * mul, 0u, false);
  b = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * mul, v[7] * mul, b, true);
  return make_uint2(a, b);
}

__device__ __forceinline__ float e4m3_at(uint2 w, int j) {
  const uint32_t d = j < 4 ? w.x : w.y;
  switch (j & 3) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(d), 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(d), 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(d), 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(d), 3);
  }
}

constexpr int kSplitPieces = 4;  // pieces of 8 values per thread: rows of up to 4 * 256 * 8 = 8192 values

}  // namespace

// One workgroup per row.  Thread u owns pieces u, u + 256, ... of 8 values;
// piece p is values 8p .. 8p + 7 of the row, which land at bytes 8 (p % 16)
// of chunk p / 16 (hi) and 128 bytes further (lo).  Pieces of the last
// chunk past the row's end are written as zeros, so that the MFMA kernel
// can stage whole chunks.
__global__ __launch_bounds__(256) void mx8_split_kernel(SplitArgs A) {
  __shared__ float red[4];
  const int row = static_cast<int>(blockIdx.x);
  int rows = A.rows;
  if (A.rows_from_plan) {
    if (A.plan->key != A.key) return;  // no plan for this call (whole workgroup)
    rows = min(max(A.plan->R_local, 0), A.rows);
  }
  if (row >= rows) return;
  const int tid = threadIdx.x;
  const int np = A.L >> 3;                  // pieces of the row
  const int nc = (A.L + 127) >> 7;          // chunks
  const int npad = nc * 16;                 // pieces including the last chunk's padding
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(A.in + static_cast<size_t>(row) * A.L);
  uint8_t* __restrict__ dst = A.out + static_cast<size_t>(row) * nc * 256;

  float v[kSplitPieces][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kSplitPieces; ++i) {
    const int p = tid + 256 * i;
    const uint4 u = p < np ? src[p] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[i][2 * j] = __uint_as_float(bf16_lo(w[j]));
      v[i][2 * j + 1] = __uint_as_float(bf16_hi(w[j]));
      amax = fmaxf(amax, fmaxf(fabsf(v[i][2 * j]), fabsf(v[i][2 * j + 1])));
    }
  }
  const int s_hi = split_scale(block_max(amax, red));
  const float mul_hi = pow2(127 - s_hi), scl_hi = pow2(s_hi - 127);
  float ramax = 0.0f;
#pragma unroll
  for (int i = 0; i < kSplitPieces; ++i) {
    const int p = tid + 256 * i;
    if (p < npad) {
      const uint2 h = to_e4m3x8(v[i], mul_hi);
      *reinterpret_cast<uint2*>(dst + (p >> 4) * 256 + (p & 15) * 8) = h;
      // the remainder is exact: both terms are multiples of a power of two
      // that fp32 resolves within 24 bits
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[i][j] -= e4m3_at(h, j) * scl_hi;
        ramax = fmaxf(ramax, fabsf(v[i][j]));
      }
    }
  }
  const int s_lo = split_scale(block_max(ramax, red));
  const float mul_lo = pow2(127 - s_lo);
#pragma unroll
  for (int i = 0; i < kSplitPieces; ++i) {
    const int p = tid + 256 * i;
    if (p < npad) *reinterpret_cast<uint2*>(dst + (p >> 4) * 256 + 128 + (p & 15) * 8) = to_e4m3x8(v[i], mul_lo);
  }
  if (tid == 0) A.scales[row] = s_hi | (s_lo << 8);
}

// mfma_kernel's work items, staging and weight ring, on split activations:
// A.in is the split rows (A.in_stride bytes each, one 256-byte chunk per 128
// values: the same size per chunk as bf16, so the staging is unchanged) and
// A.in_scale their scales.  Per chunk and 16-token group a wave issues one
// scaled MFMA per weight row set and part (hi, lo); the weight block of lane
// (r, q) is its A operand as loaded and the strip byte its scale.
template <bool kGateUp, int kGroups, bool kPair>
__global__ __launch_bounds__(256, kGroups == 1 ? 3 : 2) void mfma_fp4_kernel(ExpertArgs A) {
  static_assert(!(kGateUp && kPair), "pairing is for the down projection");
  constexpr bool kTwo = kGateUp || kPair;
  constexpr int kWaveRows = kPair ? 32 : 16;
  constexpr int kTileRows = 4 * kWaveRows;
  constexpr int kTokens = 16 * kGroups;
  constexpr int kBuf = kTokens * kXRowBytes;
  constexpr int kRing = 4;
  extern __shared__ __align__(16) unsigned char lds[];  // [2][kTokens][kXRowBytes], then the scale strips

  const int tiles = (A.rows + kTileRows - 1) / kTileRows;
  // XCD-aware order, as in mfma_kernel
  const int xcd = static_cast<int>(blockIdx.x) & 7, kx = static_cast<int>(blockIdx.x) >> 3;
  const int item = xcd + 8 * (kx / tiles);
  const int tile = kx - (kx / tiles) * tiles;
  if (A.plan->key != A.key) return;
  const int n_items = min(max(A.plan->n_mfma, 0), A.list_cap);
  const WorkEntry we = clamp_entry(A.list[min(item, A.list_cap - 1)], A);
  if (item >= n_items) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int wrow0 = tile * kTileRows + wave * kWaveRows;
  const bool wave_ok = wrow0 < A.rows;
  const int wrow = min(wrow0 + r, A.rows - 1);
  const int red = A.red, RB = red >> 5;
  const int NC = (RB + kChunkBlocks - 1) / kChunkBlocks;
  const int rows_e = kGateUp ? 2 * A.rows : A.rows;
  const uint32_t expert_bytes = static_cast<uint32_t>(rows_e) * static_cast<uint32_t>(red >> 1);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A.wp + static_cast<size_t>(we.e) * expert_bytes), 0, expert_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.in), 0, A.in_bytes, 0x00020000);
  const uint8_t* __restrict__ sbase = A.ws + static_cast<size_t>(we.e) * rows_e * RB;
  const int il = kGateUp ? A.il : 0;
  const int wr0 = kGateUp ? gate_row(wrow, il) : wrow;
  const int wr1 = kGateUp ? up_row(wrow, A.rows, il) : min(wrow0 + 16 + r, A.rows - 1);
  const uint32_t wo0 = row_offset(wr0, red >> 1, A.tiled);
  const uint32_t wo1 = row_offset(wr1, red >> 1, A.tiled);
  const uint32_t bstride = block_stride(A.tiled);
  const int srows = min(kTileRows, A.rows - tile * kTileRows);
  unsigned char* sstrip = lds + 2 * kBuf;
  const int strip = kTileRows * RB;
  if (il) {
    dma_strip(sbase + static_cast<size_t>(2 * tile * kTileRows) * RB, sstrip, 2 * srows * RB);
  } else {
    dma_strip(sbase + static_cast<size_t>(tile * kTileRows) * RB, sstrip, srows * RB);
    if (kGateUp) dma_strip(sbase + static_cast<size_t>(tile * kTileRows + A.rows) * RB, sstrip + strip, srows * RB);
  }
  const int s0i = il ? 2 * RB : RB, s1b = il ? RB : (kPair ? 16 * RB : strip);
  const int srow_l = min(wave * kWaveRows + r, srows - 1);

  for (int tp0 = 0; tp0 < we.Te; tp0 += kTokens) {
    const int nt = min(kTokens, we.Te - tp0);
    const int NG = (nt + 15) >> 4;

    // staging role as in mfma_kernel; a split row has no partial chunk
    // (the split kernel zero-fills it), so only chunks past the row and
    // tokens past the pass read zeros
    uint32_t sxoff[kGroups];
    const int spiece = tid & 15;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const int st = (tid + 256 * k) >> 4;
      const int p = we.p0 + tp0 + (st < nt ? st : 0);
      const int row = A.routes != nullptr ? A.routes[p] / A.top_k : p;
      sxoff[k] = st < nt ? static_cast<uint32_t>(row) * A.in_stride : kOob;
    }
    // this lane's B scales: token tg * 16 + r of the pass (hi in byte 0, lo in byte 1)
    int xsc[kGroups];
#pragma unroll
    for (int tg = 0; tg < kGroups; ++tg) {
      const int tt = tg * 16 + r;
      const int p = we.p0 + tp0 + (tt < nt ? tt : 0);
      // (clamped: a stale plan gives wrong numbers, not an out-of-range load)
      const int row = min(max(A.routes != nullptr ? A.routes[p] / A.top_k : p, 0), (A.routes != nullptr ? A.T : A.R) - 1);
      xsc[tg] = tt < nt ? A.in_scale[row] : 127 | (127 << 8);
    }
    auto pass = [&](auto ng) {
      constexpr int kNG = decltype(ng)::value;
      auto xload = [&](int c, uint4 (&dst)[kGroups]) {
        const bool cok = c < NC;
        const uint32_t po = static_cast<uint32_t>((c * 16 + spiece) * 16);
#pragma unroll
        for (int k = 0; k < kGroups; ++k)
          if (k < kNG) dst[k] = buffer_load16(xrs, cok && sxoff[k] != kOob ? sxoff[k] + po : kOob);
      };
      auto xstore = [&](int c, const uint4 (&src)[kGroups]) {
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
          const int u = tid + 256 * k;
          if (k < kNG) *reinterpret_cast<uint4*>(lds + (c & 1) * kBuf + (u >> 4) * kXRowBytes + (u & 15) * 16) = src[k];
        }
      };

      f32x4 acc0[kGroups], acc1[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        acc0[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        acc1[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }

      uint4 rw0[kRing], rw1[kRing], rx[kRing][kGroups];
      auto wload = [&](int c, int slot) {
        const int b = c * kChunkBlocks + q;
        const bool ok = b < RB;
        rw0[slot] = buffer_load16(wrs, ok ? wo0 + bstride * b : kOob);
        if (kTwo) rw1[slot] = buffer_load16(wrs, ok ? wo1 + bstride * b : kOob);
      };

#pragma unroll
      for (int s = 0; s < kRing; ++s) {
        wload(s, s);
        xload(s, rx[s]);
      }
      xstore(0, rx[0]);
      xload(kRing, rx[0]);
      lds_barrier();

      const int rounds = (NC + kRing - 1) / kRing;
      for (int c0 = 0; c0 < rounds * kRing; c0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
          const int c = c0 + s;
          // blocks past the row were loaded as zeros; the scale is read at a
          // clamped index so that no branch splits the chunk
          const int bs = min(c * kChunkBlocks + q, RB - 1);
          const int sa0 = sstrip[srow_l * s0i + bs];
          const int sa1 = kTwo ? static_cast<int>(sstrip[s1b + srow_l * s0i + bs]) : 0;
          const i32x8 a0 = {static_cast<int>(rw0[s].x), static_cast<int>(rw0[s].y), static_cast<int>(rw0[s].z),
                            static_cast<int>(rw0[s].w), 0, 0, 0, 0};
          i32x8 a1 = {0, 0, 0, 0, 0, 0, 0, 0};
          if (kTwo)
            a1 = i32x8{static_cast<int>(rw1[s].x), static_cast<int>(rw1[s].y), static_cast<int>(rw1[s].z),
                       static_cast<int>(rw1[s].w), 0, 0, 0, 0};
          wload(c + kRing, s);
          const unsigned char* xb = lds + (c & 1) * kBuf;
#pragma unroll
          for (int tg = 0; tg < kGroups; ++tg) {
            if (tg < kNG) {
              const unsigned char* row = xb + (tg * 16 + r) * kXRowBytes;
              const uint4 h0 = *reinterpret_cast<const uint4*>(row + 16 * q);
              const uint4 h1 = *reinterpret_cast<const uint4*>(row + 64 + 16 * q);
              const uint4 l0 = *reinterpret_cast<const uint4*>(row + 128 + 16 * q);
              const uint4 l1 = *reinterpret_cast<const uint4*>(row + 192 + 16 * q);
              const i32x8 bh = {static_cast<int>(h0.x), static_cast<int>(h0.y), static_cast<int>(h0.z),
                                static_cast<int>(h0.w), static_cast<int>(h1.x), static_cast<int>(h1.y),
                                static_cast<int>(h1.z), static_cast<int>(h1.w)};
              const i32x8 bl = {static_cast<int>(l0.x), static_cast<int>(l0.y), static_cast<int>(l0.z),
                                static_cast<int>(l0.w), static_cast<int>(l1.x), static_cast<int>(l1.y),
                                static_cast<int>(l1.z), static_cast<int>(l1.w)};
              // format codes: A = E2M1 (4), B = E4M3 (0); B's scale byte 0 = hi, 1 = lo
              acc0[tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, bh, acc0[tg], 4, 0, 0, sa0, 0, xsc[tg]);
              acc0[tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, bl, acc0[tg], 4, 0, 0, sa0, 1, xsc[tg]);
              if (kTwo) {
                acc1[tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, bh, acc1[tg], 4, 0, 0, sa1, 0, xsc[tg]);
                acc1[tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, bl, acc1[tg], 4, 0, 0, sa1, 1, xsc[tg]);
              }
            }
          }
          const int sn = (s + 1) % kRing;
          xstore(c + 1, rx[sn]);
          xload(c + 1 + kRing, rx[sn]);
          lds_barrier();
        }
      }

      // epilogue, as in mfma_kernel: lane holds rows wrow0 + 4q + i of token tg*16 + r
      if (wave_ok) {
        const int rowbase = wrow0 + 4 * q;
        float b0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, b1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (A.bias != nullptr) {
          const size_t bb = static_cast<size_t>(we.e) * rows_e;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            b0[i] = bf16_bits_to_f32(A.bias[bb + (kGateUp ? gate_row(rowbase + i, il) : rowbase + i)]);
            if (kGateUp) b1[i] = bf16_bits_to_f32(A.bias[bb + up_row(rowbase + i, A.rows, il)]);
            if (kPair) b1[i] = bf16_bits_to_f32(A.bias[bb + rowbase + 16 + i]);
          }
        }
#pragma unroll
        for (int tg = 0; tg < kGroups; ++tg) {
          const int tt = tg * 16 + r;
          if (tg < kNG && tt < nt) {
            const size_t p = static_cast<size_t>(we.p0 + tp0 + tt);
            if (kGateUp) {
              uint16_t h[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                h[i] = f32_to_bf16_rne(
                    activate(acc0[tg][i] + b0[i], acc1[tg][i] + b1[i], A.act_kind, A.alpha, A.limit));
              uint2 pk;
              pk.x = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
              pk.y = static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16);
              *reinterpret_cast<uint2*>(A.a_out + p * A.rows + rowbase) = pk;
            } else {
              *reinterpret_cast<float4*>(A.o_out + p * A.rows + rowbase) =
                  make_float4(acc0[tg][0] + b0[0], acc0[tg][1] + b0[1], acc0[tg][2] + b0[2], acc0[tg][3] + b0[3]);
              if (kPair)
                *reinterpret_cast<float4*>(A.o_out + p * A.rows + rowbase + 16) =
                    make_float4(acc1[tg][0] + b1[0], acc1[tg][1] + b1[1], acc1[tg][2] + b1[2], acc1[tg][3] + b1[3]);
            }
          }
        }
      }
    };
    if (NG >= kGroups) {
      pass(std::integral_constant<int, kGroups>{});
    } else if constexpr (kGroups == 4) {
      if (NG == 3) pass(std::integral_constant<int, 3>{});
      else if (NG == 2) pass(std::integral_constant<int, 2>{});
      else pass(std::integral_constant<int, 1>{});
    } else if constexpr (kGroups == 2) {
      pass(std::integral_constant<int, 1>{});
    }
    if (tp0 + kTokens < we.Te) lds_barrier();
  }
}

template __global__ void mfma_fp4_kernel<true, 1, false>(ExpertArgs);
template __global__ void mfma_fp4_kernel<true, 2, false>(ExpertArgs);
template __global__ void mfma_fp4_kernel<true, 4, false>(ExpertArgs);
template __global__ void mfma_fp4_kernel<false, 1, false>(ExpertArgs);
template __global__ void mfma_fp4_kernel<false, 2, false>(ExpertArgs);
template __global__ void mfma_fp4_kernel<false, 4, false>(ExpertArgs);
template __global__ void mfma_fp4_kernel<false, 1, true>(ExpertArgs);
template __global__ void mfma_fp4_kernel<false, 2, true>(ExpertArgs);
template __global__ void mfma_fp4_kernel<false, 4, true>(ExpertArgs);

}  // namespace moe
