// Grouped expert kernels: the gate/up projection with its activation, the
// down projection, the routing-weighted combine, and the dequantisation hook.
//
// What they compute: "MXFP4 MoE decode kernels", Design (x -> gate/up GEMV +
// bias + activation -> bf16 intermediate; intermediate -> down GEMV +
// routing-weighted bias + weighted sum per token) and Design, Fused
// epilogues.  Weights are read once, straight from the packed layout (Design,
// Read the served layout), and decoded in registers with gfx950's scaled FP4
// converts; one 16-byte load of a packed row is exactly one 32-value MX block
// and needs one scale byte.
//
// Two regimes, two kernels, each serving both projections (a template flag
// selects [gate; up] row pairs with the activation, or single rows):
//  * GEMV (experts with Te <= kGemvMaxTokens routes): kLanesPerRow lanes
//    stream one row (pair); lane q loads MX blocks q, q + kLanesPerRow, ...
//    with 128-bit loads through a register ring so that several blocks per
//    row are in flight, multiplies with v_dot2_f32_bf16 against the
//    activations staged once in LDS, and the partial sums are combined with
//    DPP row operations.
//  * MFMA (Te > kGemvMaxTokens): 4 waves x 16 rows, tokens in groups of 16.
//    Each lane decodes one MX block of its row per step into four 8-value
//    bf16 operands of v_mfma_f32_16x16x32_bf16; the activation chunk of the
//    tokens is shared by the 4 waves through LDS.  The reduction index inside
//    one MFMA is permuted (lane group q carries block q of the chunk),
//    identically for both operands.
// A work item (one workgroup) is a tile of rows of one expert from the
// plan's list for its regime; blocks past the list exit at once, so the grid
// only needs a host-side upper bound.
#include "device_common.h"
#include "kernels.h"
#include "list_common.h"

#include <type_traits>

namespace moe {

namespace {

__device__ __forceinline__ bf16x8 decode_dword_bf16x8(uint32_t d, float s) {
  const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
  const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
  const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
  const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
  bf16x8 r;
  r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
  r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
  return r;
}

__device__ __forceinline__ float dot_block(const bf16x2 (&w)[16], const uint4* __restrict__ xp, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 xv = xp[c];
    acc = dot2(w[4 * c + 0], xv.x, acc);
    acc = dot2(w[4 * c + 1], xv.y, acc);
    acc = dot2(w[4 * c + 2], xv.z, acc);
    acc = dot2(w[4 * c + 3], xv.w, acc);
  }
  return acc;
}

template <int kLanesPerRow>
__device__ __forceinline__ float row_sum(float v) {
  v = row16_sum(v);
  if (kLanesPerRow == 32) v += __shfl_xor(v, 16);
  return v;
}

}  // namespace

// ---------------------------------------------------------------------------
// GEMV regime
// ---------------------------------------------------------------------------
// The hot loop is branch-free so that the compiler keeps the register ring of
// weight loads in flight: block indices are clamped to the row (the surplus
// loads of the ragged tail hit the same row) and tail contributions are
// dropped with selects.
template <bool kGateUp, int kLanesPerRow>
__global__ __launch_bounds__(256, 4) void gemv_kernel(ExpertArgs A) {
  constexpr int kRowsPerWG = 256 / kLanesPerRow;
  constexpr int kRing = kGateUp ? 4 : (kLanesPerRow == 16 ? 6 : 4);
  extern __shared__ uint4 xs[];  // [kGemvMaxTokens][red / 8], then the scale strips

  const int tiles = A.rows / kRowsPerWG;
  // work units (list entry, row tile) of the plan's list, taken grid-stride:
  // the host's grid is a bound on the units, capped near the resident count,
  // so that a call whose list is short or empty launches few workgroups
  if (A.plan->key != A.key) return;  // no plan for this call in the workspace
  const int n_units = min(max(A.plan->n_gemv, 0), A.list_cap) * tiles;
  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    if (unit != static_cast<int>(blockIdx.x)) __syncthreads();  // LDS restaged for this unit
    const int item = unit / tiles;               // < n_gemv <= E_local
    const WorkEntry we = clamp_entry(A.list[item], A);
    const int tile = unit - item * tiles;
    const int tid = threadIdx.x, g = tid / kLanesPerRow, q = tid % kLanesPerRow;
    const int red = A.red, RB = red >> 5, RV = red >> 3;
    const int n = tile * kRowsPerWG + g;
    // wave-uniform expert base pointers + 32-bit per-lane row offsets
    const int rows_e = kGateUp ? 2 * A.rows : A.rows;
    const uint8_t* __restrict__ wbase = A.wp + static_cast<size_t>(we.e) * rows_e * (red >> 1);
    const uint8_t* __restrict__ sbase = A.ws + static_cast<size_t>(we.e) * rows_e * RB;
    const int il = kGateUp ? A.il : 0;                             // interleaved w13 rows
    const int nr0 = kGateUp ? gate_row(n, il) : n, nr1 = up_row(n, A.rows, il);
    const uint32_t wo0 = row_offset(nr0, red >> 1, A.tiled), wo1 = row_offset(nr1, red >> 1, A.tiled);
    const uint32_t bstride = block_stride(A.tiled);
    const size_t row0 = static_cast<size_t>(we.e) * rows_e + nr0;  // bias index of the gate (or single) row
    const size_t row1 = static_cast<size_t>(we.e) * rows_e + nr1;  // bias index of the up row
    auto ldw = [&](uint32_t off, int b) { return *reinterpret_cast<const uint4*>(wbase + off + bstride * b); };
    // scale strips of the tile's rows, staged in LDS: [kRowsPerWG][RB] (gate/single), then up;
    // interleaved w13: the tile's 2 * kRowsPerWG stored rows in one strip
    unsigned char* sstrip = reinterpret_cast<unsigned char*>(xs) + kGemvMaxTokens * red * 2;
    const int strip = kRowsPerWG * RB;
    const uint8_t* ss0 = sbase + static_cast<size_t>(tile * kRowsPerWG) * (il ? 2 : 1) * RB;
    const uint8_t* ss1 = sbase + static_cast<size_t>(tile * kRowsPerWG + A.rows) * RB;
    auto lds_scale = [&](int which, int b) -> uint32_t {
      return il ? sstrip[(2 * g + which) * RB + b] : sstrip[which * strip + g * RB + b];
    };
    const int nmax = (RB + kLanesPerRow - 1) / kLanesPerRow;  // ring steps (uniform)
    const int Te = we.Te;

    // Token passes of up to kGemvMaxTokens routes; one pass unless repeated ids
    // gave the expert more routes while the MFMA regime is off.
    for (int t0 = 0; t0 < Te; t0 += kGemvMaxTokens) {
      const int nt = min(kGemvMaxTokens, Te - t0);
      const int n_stage = nt * RV;

      // 1. activation rows of the pass: direct global -> LDS copies (16 B per
      //    lane; a wave's copy fills 1 KB of LDS contiguously), no registers
      // activation row of each token of the pass (uniform)
      const uint4* src_row[kGemvMaxTokens];
#pragma unroll
      for (int t = 0; t < kGemvMaxTokens; ++t) {
        const int tt = min(t0 + t, Te - 1);
        int row = we.p0 + tt;  // down projection: row of the intermediate
        if (kGateUp) {
          int tok = we.tok[0];
#pragma unroll
          for (int u = 1; u < kGemvMaxTokens; ++u) tok = tt == u ? we.tok[u] : tok;
          row = tt < kGemvMaxTokens ? tok : min(max(A.routes[we.p0 + tt] / A.top_k, 0), A.T - 1);
        }
        src_row[t] = reinterpret_cast<const uint4*>(A.in + static_cast<size_t>(row) * red);
      }
#pragma unroll 1
      for (int i = tid; i < n_stage; i += 256) {
        {
          int t = 0, c = i;
#pragma unroll
          for (int u = 1; u < kGemvMaxTokens; ++u) {
            const bool next = c >= RV;
            t = next ? u : t;
            c = next ? c - RV : c;
          }
          const uint4* src = src_row[0];
#pragma unroll
          for (int u = 1; u < kGemvMaxTokens; ++u) src = t == u ? src_row[u] : src;
          __builtin_amdgcn_global_load_lds(src + c,
                                           reinterpret_cast<__attribute__((address_space(3))) void*>(
                                               reinterpret_cast<uintptr_t>(xs + (i & ~63))),
                                           16, 0, 0);
        }
      }
      if (t0 == 0) {
        if (il) {
          dma_strip(ss0, sstrip, 2 * strip);
        } else {
          dma_strip(ss0, sstrip, strip);
          if (kGateUp) dma_strip(ss1, sstrip + strip, strip);
        }
      }
      // 2. weight ring, unconditional (indices clamped to the row)
      uint4 r0[kRing], r1[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        const int b = min(q + kLanesPerRow * j, RB - 1);
        r0[j] = ldw(wo0, b);
        if (kGateUp) r1[j] = ldw(wo1, b);
      }
      __syncthreads();

      float acc0[kGemvMaxTokens], acc1[kGemvMaxTokens];
#pragma unroll
      for (int t = 0; t < kGemvMaxTokens; ++t) acc0[t] = acc1[t] = 0.0f;

      for (int j0 = 0; j0 < nmax; j0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
          const int b = q + kLanesPerRow * (j0 + s);
          const bool valid = b < RB;             // also false past the last ring step
          const int bc = min(b, RB - 1);
          // a zero scale turns a ragged-tail block into zeros
          const float sc0 = valid ? e8m0_to_f32(lds_scale(0, bc)) : 0.0f;
          const float sc1 = kGateUp && valid ? e8m0_to_f32(lds_scale(1, bc)) : 0.0f;
          const uint32_t d0[4] = {r0[s].x, r0[s].y, r0[s].z, r0[s].w};
          uint32_t d1[4] = {0, 0, 0, 0};
          if (kGateUp) {
            d1[0] = r1[s].x;
            d1[1] = r1[s].y;
            d1[2] = r1[s].z;
            d1[3] = r1[s].w;
          }
          const int bn = min(b + kLanesPerRow * kRing, RB - 1);
          r0[s] = ldw(wo0, bn);
          if (kGateUp) r1[s] = ldw(wo1, bn);
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const bf16x2 g0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d0[dw], sc0, 0);
            const bf16x2 g1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d0[dw], sc0, 1);
            const bf16x2 g2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d0[dw], sc0, 2);
            const bf16x2 g3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d0[dw], sc0, 3);
            bf16x2 u0, u1, u2, u3;
            if (kGateUp) {
              u0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d1[dw], sc1, 0);
              u1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d1[dw], sc1, 1);
              u2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d1[dw], sc1, 2);
              u3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d1[dw], sc1, 3);
            }
#pragma unroll
            for (int t = 0; t < kGemvMaxTokens; ++t) {
              if (t < nt) {
                const uint4 xv = xs[t * RV + bc * 4 + dw];
                acc0[t] = dot2(g3, xv.w, dot2(g2, xv.z, dot2(g1, xv.y, dot2(g0, xv.x, acc0[t]))));
                if (kGateUp) acc1[t] = dot2(u3, xv.w, dot2(u2, xv.z, dot2(u1, xv.y, dot2(u0, xv.x, acc1[t]))));
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);  // keep live ranges per ring slot
        }
      }

#pragma unroll
      for (int t = 0; t < kGemvMaxTokens; ++t) {
        acc0[t] = row_sum<kLanesPerRow>(acc0[t]);
        if (kGateUp) acc1[t] = row_sum<kLanesPerRow>(acc1[t]);
      }
      if (q == 0) {
        const float b0 = A.bias != nullptr ? bf16_bits_to_f32(A.bias[row0]) : 0.0f;
        const float b1 = (kGateUp && A.bias != nullptr) ? bf16_bits_to_f32(A.bias[row1]) : 0.0f;
#pragma unroll
        for (int t = 0; t < kGemvMaxTokens; ++t) {
          if (t < nt) {
            const size_t p = static_cast<size_t>(we.p0 + t0 + t);
            if (kGateUp) {
              A.a_out[p * A.rows + n] =
                  f32_to_bf16_rne(activate(acc0[t] + b0, acc1[t] + b1, A.act_kind, A.alpha, A.limit));
            } else {
              A.o_out[p * A.rows + n] = acc0[t] + b0;
            }
          }
        }
      }
      if (t0 + kGemvMaxTokens < Te) __syncthreads();  // xs is restaged by the next pass
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA regime
// ---------------------------------------------------------------------------
// Work item: 64 rows (row pairs) of one expert, 4 waves x 16 rows.  The
// reduction runs in chunks of 4 MX blocks (128 values).  Per chunk, lane
// (r, q) of a wave decodes block q of its row r (A operand) and reads 64 bytes
// of token r's activations for the same block from LDS (B operand).  The
// activation chunk of the pass's tokens is shared by the 4 waves through an
// LDS double buffer; both it and the weights stream through register rings
// kRing chunks deep, with the loop unrolled by the ring depth so every slot
// stays in its own registers and the compiler can count outstanding loads
// exactly.  One LDS-only barrier per chunk; no branches inside the ring.
//
// kBf16W (prefill): the weights come unpacked to bf16 (row layout, A.wbf);
// lane (r, q) loads the 64 bytes of block q of its row per chunk and feeds
// its g-th 16 bytes to MFMA g: the operands the MXFP4 path decodes, in the
// same order, so both give the same bits.
//
// kPair (down projection, rows % 32 == 0): a wave computes two 16-row sets
// 16 rows apart (a workgroup 128 rows), so each activation operand read from
// LDS feeds two MFMAs, as the gate and up rows of the gate/up projection do.
template <bool kGateUp, int kGroups, bool kBf16W, bool kPair>
__global__ __launch_bounds__(256, (kGroups == 1 && !kBf16W) ? 3 : 2) void mfma_kernel(ExpertArgs A) {
  static_assert(!(kGateUp && kPair), "pairing is for the down projection");
  constexpr bool kTwo = kGateUp || kPair;           // two weight row sets per wave
  constexpr int kWaveRows = kPair ? 32 : 16;
  constexpr int kTileRows = 4 * kWaveRows;          // rows of a work item
  constexpr int kTokens = 16 * kGroups;
  constexpr int kBuf = kTokens * kXRowBytes;
  constexpr int kRing = kBf16W ? 2 : 4;  // chunks in flight per wave
  constexpr int kWv = kBf16W ? 4 : 1;                         // 16-byte weight loads per lane and chunk
  extern __shared__ __align__(16) unsigned char lds[];  // [2][kTokens][kXRowBytes], then the scale strips

  const int tiles = (A.rows + kTileRows - 1) / kTileRows;
  // XCD-aware order: block b runs on XCD b % 8, so XCD x takes list entries
  // x, x + 8, ..., each with all of its row tiles in dispatch order.  The
  // tiles of one expert then stage the same activation rows through one L2
  // (a few experts at a time per XCD), instead of every XCD reading every
  // expert's rows.  The host pads the grid to 8 * tiles * ceil(experts / 8).
  const int xcd = static_cast<int>(blockIdx.x) & 7, kx = static_cast<int>(blockIdx.x) >> 3;
  const int item = xcd + 8 * (kx / tiles);
  const int tile = kx - (kx / tiles) * tiles;
  if (A.plan->key != A.key) return;  // no plan for this call in the workspace (whole workgroup)
  const int n_items = min(max(A.plan->n_mfma, 0), A.list_cap);
  const WorkEntry we = clamp_entry(A.list[min(item, A.list_cap - 1)], A);  // in bounds; used only when item < n_items
  if (item >= n_items) return;  // whole workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int wrow0 = tile * kTileRows + wave * kWaveRows;
  const bool wave_ok = wrow0 < A.rows;              // rows past the end: staging and barriers only
  const int wrow = min(wrow0 + r, A.rows - 1);      // clamped so that every load stays in the expert
  const int red = A.red, RB = red >> 5;
  const int NC = (RB + kChunkBlocks - 1) / kChunkBlocks;
  const int rows_e = kGateUp ? 2 * A.rows : A.rows;
  // weights of expert we.e and the activation rows through buffer resources:
  // blocks past a row and pieces of tokens past the pass use an out-of-range
  // offset and read zeros (no clamping, no masks)
  const uint32_t expert_bytes = static_cast<uint32_t>(rows_e) * static_cast<uint32_t>(kBf16W ? red * 2 : red >> 1);
  const uint8_t* __restrict__ wbase =
      kBf16W ? reinterpret_cast<const uint8_t*>(A.wbf) + static_cast<size_t>(we.e) * expert_bytes
             : A.wp + static_cast<size_t>(we.e) * expert_bytes;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wbase), 0, expert_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.in), 0, A.in_bytes, 0x00020000);
  const uint8_t* __restrict__ sbase = A.ws + static_cast<size_t>(we.e) * rows_e * RB;
  const int il = kGateUp ? A.il : 0;                // interleaved w13 rows
  const int wr0 = kGateUp ? gate_row(wrow, il) : wrow;
  const int wr1 = kGateUp ? up_row(wrow, A.rows, il) : min(wrow0 + 16 + r, A.rows - 1);
  const uint32_t wo0 = kBf16W ? static_cast<uint32_t>(wr0) * red * 2 : row_offset(wr0, red >> 1, A.tiled);
  const uint32_t wo1 = kBf16W ? static_cast<uint32_t>(wr1) * red * 2 : row_offset(wr1, red >> 1, A.tiled);
  const uint32_t bstride = kBf16W ? 64u : block_stride(A.tiled);
  // scale strips of the tile's rows (clamped to the expert), staged in LDS once:
  // [kTileRows][RB] (gate/single, both sets of a paired wave), then up;
  // interleaved w13: the tile's stored rows (gate, up alternating) in one strip
  const int srows = min(kTileRows, A.rows - tile * kTileRows);
  unsigned char* sstrip = lds + 2 * kBuf;
  const int strip = kTileRows * RB;
  if (kBf16W) {
    // unpacked weights carry their scales
  } else if (il) {
    dma_strip(sbase + static_cast<size_t>(2 * tile * kTileRows) * RB, sstrip, 2 * srows * RB);
  } else {
    dma_strip(sbase + static_cast<size_t>(tile * kTileRows) * RB, sstrip, srows * RB);
    if (kGateUp) dma_strip(sbase + static_cast<size_t>(tile * kTileRows + A.rows) * RB, sstrip + strip, srows * RB);
  }
  // scale of set j, strip row l: [j * s1b + l * s0i]; a paired wave's second
  // set is 16 strip rows below its first
  const int s0i = il ? 2 * RB : RB, s1b = il ? RB : (kPair ? 16 * RB : strip);
  const int srow_l = min(wave * kWaveRows + r, srows - 1);  // this lane's (first) row in the strips

  for (int tp0 = 0; tp0 < we.Te; tp0 += kTokens) {
    const int nt = min(kTokens, we.Te - tp0);
    const int NG = (nt + 15) >> 4;

    // staging role: uint4 piece u = tid + 256*k of the chunk's [kTokens][16]
    // pieces (group k < NG only: the MFMAs read no column group past the
    // pass).  Pieces of tokens past the pass and of blocks past the row read
    // zeros through an out-of-range offset.
    uint32_t sxoff[kGroups];
    const int spiece = tid & 15;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const int st = (tid + 256 * k) >> 4;
      const int p = we.p0 + tp0 + (st < nt ? st : 0);
      const int row = A.routes != nullptr ? A.routes[p] / A.top_k : p;
      sxoff[k] = st < nt ? static_cast<uint32_t>(row) * static_cast<uint32_t>(red) * 2u : kOob;
    }
    // The chunk loop is instantiated per column-group count, so that no
    // branch separates the MFMAs of one chunk: the compiler then batches
    // the LDS reads of the activation operands instead of waiting for
    // each one before its two MFMAs.
    auto pass = [&](auto ng) {
      constexpr int kNG = decltype(ng)::value;
      auto xload = [&](int c, uint4 (&dst)[kGroups]) {
        const bool bok = c * kChunkBlocks + (spiece >> 2) < RB;
        const uint32_t po = static_cast<uint32_t>((c * 16 + spiece) * 16);
  #pragma unroll
        for (int k = 0; k < kGroups; ++k)
          if (k < kNG) dst[k] = buffer_load16(xrs, bok && sxoff[k] != kOob ? sxoff[k] + po : kOob);
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

      uint4 rw0[kRing][kWv], rw1[kRing][kWv], rx[kRing][kGroups];
      auto wload = [&](int c, int slot) {
        const int b = c * kChunkBlocks + q;
        const bool ok = b < RB;
  #pragma unroll
        for (int v = 0; v < kWv; ++v) {
          rw0[slot][v] = buffer_load16(wrs, ok ? wo0 + bstride * b + 16 * v : kOob);
          if (kTwo) rw1[slot][v] = buffer_load16(wrs, ok ? wo1 + bstride * b + 16 * v : kOob);
        }
      };

      // prologue: chunks 0..kRing-1 in flight, chunk 0 staged in LDS
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
          const bool valid = c * kChunkBlocks + q < RB;  // false past the row and past the last chunk
          // blocks past the row were loaded as zeros, which any finite scale
          // keeps zero: the scale is read unconditionally (clamped index), so
          // that no exec-masked branch splits the chunk
          const int bs = min(c * kChunkBlocks + q, RB - 1);
          const float sc0 = kBf16W ? 0.0f : e8m0_to_f32(sstrip[srow_l * s0i + bs]);
          const float sc1 = (!kBf16W && kTwo) ? e8m0_to_f32(sstrip[s1b + srow_l * s0i + bs]) : 0.0f;
          const uint32_t d0[4] = {rw0[s][0].x, rw0[s][0].y, rw0[s][0].z, rw0[s][0].w};
          uint32_t d1[4] = {0, 0, 0, 0};
          if (kTwo) {
            d1[0] = rw1[s][0].x;
            d1[1] = rw1[s][0].y;
            d1[2] = rw1[s][0].z;
            d1[3] = rw1[s][0].w;
          }
          uint4 u0[kWv], u1[kWv];
  #pragma unroll
          for (int v = 0; v < kWv; ++v) {
            u0[v] = rw0[s][v];
            u1[v] = kTwo ? rw1[s][v] : make_uint4(0, 0, 0, 0);
          }
          wload(c + kRing, s);
          const unsigned char* xb = lds + (c & 1) * kBuf + q * 64;
          // decode each 8-value operand right before its MFMAs (keeps few registers live)
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x8 a0, a1;
            if constexpr (kBf16W) {
              // the unpacked values of elements 8g..8g+7 of the block; a block past
              // the row (clamped load) contributes zeros, as a zero scale does
              const uint4 z = make_uint4(0, 0, 0, 0);
              a0 = __builtin_bit_cast(bf16x8, valid ? u0[g] : z);
              if (kTwo) a1 = __builtin_bit_cast(bf16x8, valid ? u1[g] : z);
            } else {
              a0 = decode_dword_bf16x8(d0[g], sc0);
              if (kTwo) a1 = decode_dword_bf16x8(d1[g], sc1);
            }
  #pragma unroll
            for (int tg = 0; tg < kGroups; ++tg) {
              if (tg < kNG) {
                const bf16x8 bx = *reinterpret_cast<const bf16x8*>(xb + (tg * 16 + r) * kXRowBytes + g * 16);
                acc0[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bx, acc0[tg], 0, 0, 0);
                if (kTwo) acc1[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bx, acc1[tg], 0, 0, 0);
              }
            }
          }
          // stage chunk c+1 (loaded kRing-1 chunks ago) and refill its register slot
          const int sn = (s + 1) % kRing;  // compile-time after unrolling
          xstore(c + 1, rx[sn]);
          xload(c + 1 + kRing, rx[sn]);
          lds_barrier();
        }
      }

      // epilogue: lane holds rows wrow0 + 4q + i (i < 4) of token tg*16 + r
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
    if (NG >= kGroups || kBf16W) {
      // (the bf16-weight prefill kernels keep one instantiation: groups past
      // the pass load zeros and are not stored)
      pass(std::integral_constant<int, kGroups>{});
    } else if constexpr (kGroups == 4) {
      if (NG == 3) pass(std::integral_constant<int, 3>{});
      else if (NG == 2) pass(std::integral_constant<int, 2>{});
      else pass(std::integral_constant<int, 1>{});
    } else if constexpr (kGroups == 2) {
      pass(std::integral_constant<int, 1>{});
    }
    if (tp0 + kTokens < we.Te) lds_barrier();  // the next pass restages the buffers
  }
}

template __global__ void gemv_kernel<true, 16>(ExpertArgs);
template __global__ void gemv_kernel<true, 32>(ExpertArgs);
template __global__ void gemv_kernel<false, 16>(ExpertArgs);
template __global__ void gemv_kernel<false, 32>(ExpertArgs);
template __global__ void mfma_kernel<true, 1, false, false>(ExpertArgs);
template __global__ void mfma_kernel<true, 1, true, false>(ExpertArgs);
template __global__ void mfma_kernel<true, 2, false, false>(ExpertArgs);
template __global__ void mfma_kernel<true, 2, true, false>(ExpertArgs);
template __global__ void mfma_kernel<true, 4, false, false>(ExpertArgs);
template __global__ void mfma_kernel<true, 4, true, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 1, false, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 1, true, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 2, false, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 2, true, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 4, false, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 4, true, false>(ExpertArgs);
template __global__ void mfma_kernel<false, 1, false, true>(ExpertArgs);
template __global__ void mfma_kernel<false, 2, false, true>(ExpertArgs);
template __global__ void mfma_kernel<false, 4, false, true>(ExpertArgs);

// out[t, :] = sum over j (ascending) of w[t, j] * o[route (t, j), :] over the
// token's local routes (zeros without one), rounded to bf16.  Fixed order and
// explicit roundings: the same bits wherever it runs.
//
// Workgroup (t, y) takes columns [W y, W y + W), W = 1024 kCols, of token t
// (tokens on x, whose grid limit is the large one; small calls use kCols = 1
// so that a token spreads over several workgroups).  One wave lists the
// token's local routes (o row and weight, in j order) in LDS; each thread
// then requests the rows of 4 listed routes for its kCols float4 column
// groups (1024 columns apart) before adding them: one memory latency per 4
// local routes after the list.  Rows by route with top_k <= 4 (the decode
// path) skip the list: their rows are known without the positions, so both
// are requested at once (one latency in all).
template <int kCols>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs A) {
  __shared__ size_t s_row[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ int s_n;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int k = A.top_k;
  const int c0 = blockIdx.y * (1024 * kCols) + tid * 4;
  float4 acc[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) acc[c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto store = [&]() {
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      const int col = c0 + 1024 * c;
      if (col < A.K) {
        uint2 packed;
        packed.x = static_cast<uint32_t>(f32_to_bf16_rne(acc[c].x)) |
                   (static_cast<uint32_t>(f32_to_bf16_rne(acc[c].y)) << 16);
        packed.y = static_cast<uint32_t>(f32_to_bf16_rne(acc[c].z)) |
                   (static_cast<uint32_t>(f32_to_bf16_rne(acc[c].w)) << 16);
        *reinterpret_cast<uint2*>(A.out + static_cast<size_t>(t) * A.K + col) = packed;
      }
    }
  };
  auto add = [&](float wt, const float4 (&o)[kCols]) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      acc[c].x = __fadd_rn(acc[c].x, __fmul_rn(wt, o[c].x));
      acc[c].y = __fadd_rn(acc[c].y, __fmul_rn(wt, o[c].y));
      acc[c].z = __fadd_rn(acc[c].z, __fmul_rn(wt, o[c].z));
      acc[c].w = __fadd_rn(acc[c].w, __fmul_rn(wt, o[c].w));
    }
  };
  if (A.by_route && k <= 4) {
    int p[4];
    float wt[4];
    float4 o[4][kCols];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t * k + min(i, k - 1);
      const int pr = A.pos[r];
      p[i] = (i < k && pr >= 0 && pr < A.T * k) ? pr : -1;
      wt[i] = A.weights[r];
#pragma unroll
      for (int c = 0; c < kCols; ++c)
        o[i][c] = *reinterpret_cast<const float4*>(A.o + static_cast<size_t>(r) * A.K + min(c0 + 1024 * c, A.K - 4));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p[i] >= 0) add(wt[i], o[i]);
    store();
    return;
  }
  if (tid < 64) {
    // k <= 64: lane j holds route j of the token
    int p = tid < k ? A.pos[t * k + tid] : -1;
    p = p < A.T * k ? p : -1;  // a position outside the routes (stale workspace) is skipped
    const uint64_t m = __ballot(p >= 0);
    if (p >= 0) {
      const int i = __popcll(m & ((1ull << tid) - 1ull));
      // row of the route's down projection: by route index or by plan position
      s_row[i] = static_cast<size_t>(A.by_route ? t * k + tid : p) * A.K;
      s_w[i] = A.weights[t * k + tid];
    }
    if (tid == 0) s_n = __popcll(m);
  }
  __syncthreads();
  const int n = s_n;
  for (int j0 = 0; j0 < n; j0 += 4) {
    float4 o[4][kCols];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t row = s_row[min(j0 + i, n - 1)];  // listed rows only; extra slots repeat the last
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const int col = min(c0 + 1024 * c, A.K - 4);  // in bounds; columns past K are not stored
        o[i][c] = *reinterpret_cast<const float4*>(A.o + row + col);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (j0 + i >= n) break;
      add(s_w[j0 + i], o[i]);
    }
  }
  store();
}

template __global__ void combine_kernel<1>(CombineArgs);
template __global__ void combine_kernel<4>(CombineArgs);

// One thread per 32-value MX block: 16 packed bytes + 1 scale byte.
// In place: the group's 16 * blocks pieces of 16 bytes are all read into
// registers before any is written (blocks <= kMaxDim / 32, so at most 16 per
// thread).  Forward: piece (r, b) at r * blocks + b moves to b * 16 + r.
__global__ __launch_bounds__(256) void tile_kernel(uint8_t* packed, int64_t groups, int blocks, int inverse) {
  constexpr int kPer = 16 * (kMaxDim / 32) / 256;
  const int64_t g = blockIdx.x;
  if (g >= groups) return;
  uint4* base = reinterpret_cast<uint4*>(packed + g * 16 * static_cast<int64_t>(blocks) * 16);
  const int n = 16 * blocks;
  uint4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = threadIdx.x + 256 * i;
    if (s < n) v[i] = base[s];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = threadIdx.x + 256 * i;
    if (s < n) {
      // forward: source is row-major (r, b); inverse: source is block-major (b, r)
      const int d = inverse ? (s & 15) * blocks + (s >> 4) : (s % blocks) * 16 + s / blocks;
      base[d] = v[i];
    }
  }
}

// MXFP4 encoder ("GLM-5.2 and GLM-5.3 (744B) in MXFP4 on Gaudi 2", What was
// built, MXFP4 encoder): per 32-value block X = floor(log2(amax)) - 2, plus
// one under the Quark rule when amax / 2^X >= 7; elements v / 2^X rounded to
// the E2M1 grid with ties to the even code, saturating at 6; sign from the
// sign bit.  Four lanes per block, eight values per lane; every step is exact
// (power-of-two scaling, a correctly rounded convert), so the bytes are unique.
namespace {

// floor(log2(a)) for a finite a > 0, from the bits (subnormals included)
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t b = __float_as_uint(a);
  const int e = static_cast<int>(b >> 23);
  return e > 0 ? e - 127 : (31 - __clz(static_cast<int>(b & 0x7FFFFFu))) - 149;
}

}  // namespace

template <bool kBf16>
__global__ __launch_bounds__(256) void encode_kernel(const void* __restrict__ in, int64_t n_blocks, int quark,
                                                     uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  // lane slot g covers eight values of block g >> 2; a thread takes kEncodePer
  // slots one grid width apart, loading all of them before any compute.  The
  // grid width is a multiple of 4, so the four lanes of a block stay a quad.
  const int64_t slots = n_blocks * 4, width = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  float v[kEncodePer][8];
#pragma unroll
  for (int j = 0; j < kEncodePer; ++j) {
    const int64_t g = min(g0 + j * width, slots - 1);  // surplus slots re-read the last one (not stored)
    if (kBf16) {
      const uint4 w = reinterpret_cast<const uint4*>(in)[g];
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][2 * i] = __uint_as_float(d[i] << 16);
        v[j][2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
      }
    } else {
      const float4 a = reinterpret_cast<const float4*>(in)[2 * g];
      const float4 b = reinterpret_cast<const float4*>(in)[2 * g + 1];
      v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
      v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
    }
  }
#pragma unroll
  for (int j = 0; j < kEncodePer; ++j) {
    const int64_t g = g0 + j * width;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0xB1, 0xF, 0xF, false)));
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0x4E, 0xF, 0xF, false)));
    int x = -127;
    if (m > 0.0f) {
      x = floor_log2(m) - 2;
      if (quark && ldexpf(m, -x) >= 7.0f) ++x;
      x = min(max(x, -127), 127);
    }
    // y = v * 2^-x is exact (a power-of-two step); the hardware convert at
    // unit scale rounds |y| to the nearest E2M1 magnitude, a tie to the even
    // code, saturating at 6, and keeps the sign bit (also of -0); the first
    // operand of a pair lands in the low nibble
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = ldexpf(v[j][i], -x);
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[0], y[1], 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[2], y[3], 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[4], y[5], 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[6], y[7], 1.0f, 3);
    if (g < slots) {
      reinterpret_cast<uint32_t*>(packed)[g] = word;
      if ((g & 3) == 0) scales[g >> 2] = static_cast<uint8_t>(x + 127);
    }
  }
}

template __global__ void encode_kernel<true>(const void*, int64_t, int, uint8_t*, uint8_t*);
template __global__ void encode_kernel<false>(const void*, int64_t, int, uint8_t*, uint8_t*);

// Per-route output rows: grid (ceil(K / 1024), R); each thread four columns.
__global__ __launch_bounds__(256) void route_rows_kernel(const float* __restrict__ o, const int32_t* __restrict__ pos,
                                                         float* __restrict__ out, int R, int K, int in_place) {
  const int r = blockIdx.y;
  const int k4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (r >= R || k4 >= K) return;
  const int p = pos[r];
  float4* dst = reinterpret_cast<float4*>(out + static_cast<size_t>(r) * K + k4);
  if (p < 0 || p >= R) {
    *dst = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  } else if (!in_place) {
    *dst = *reinterpret_cast<const float4*>(o + static_cast<size_t>(p) * K + k4);
  }
}

// Prefill unpack ("MXFP4 MoE decode kernels", Prefill: unpack once): one
// thread per 32-value block of one expert.  Row layout: consecutive threads
// take consecutive blocks of a row; tiled layout: consecutive threads take the
// 16 rows of one block of a 16-row group, so the packed reads stay contiguous
// either way.  The output is always the row layout, in the stored row order.
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                     const uint8_t* __restrict__ scales, int rows, int cols,
                                                     int tiled, const int32_t* __restrict__ counts,
                                                     uint16_t* __restrict__ out) {
  const int e = blockIdx.y;
  if (counts != nullptr && counts[e] == 0) return;  // an untouched expert: nothing written
  const int RB = cols >> 5;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(rows) * RB) return;
  int n, b;
  if (tiled) {
    const int64_t gb = i >> 4;  // (group, block) pair
    n = static_cast<int>(gb / RB) * 16 + static_cast<int>(i & 15);
    b = static_cast<int>(gb % RB);
  } else {
    n = static_cast<int>(i / RB);
    b = static_cast<int>(i % RB);
  }
  const uint32_t row_bytes = static_cast<uint32_t>(cols >> 1);
  const uint8_t* pe = packed + static_cast<size_t>(e) * rows * row_bytes;
  const uint4 q = *reinterpret_cast<const uint4*>(pe + row_offset(n, row_bytes, tiled) + block_stride(tiled) * b);
  const size_t row = static_cast<size_t>(e) * rows + n;
  const float s = e8m0_to_f32(scales[row * RB + b]);
  bf16x2 v[16];
  decode_block_bf16(q, s, v);
  uint4* o = reinterpret_cast<uint4*>(out + row * cols + 32 * static_cast<size_t>(b));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 u;
    u.x = __builtin_bit_cast(uint32_t, v[4 * c + 0]);
    u.y = __builtin_bit_cast(uint32_t, v[4 * c + 1]);
    u.z = __builtin_bit_cast(uint32_t, v[4 * c + 2]);
    u.w = __builtin_bit_cast(uint32_t, v[4 * c + 3]);
    o[c] = u;
  }
}

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

// Copy of the plan's routing and bucketing (test hook).  Thread i < R
// copies route i (ids, weights, routes padded with -1 past the local routes);
// thread i <= E_l copies expert i's count and offset.
__global__ __launch_bounds__(256) void plan_read_kernel(const Plan* plan, const int32_t* __restrict__ ids_ws,
                                                        const float* __restrict__ weights_ws,
                                                        const int32_t* __restrict__ counts_ws,
                                                        const int32_t* __restrict__ offsets_ws,
                                                        const int32_t* __restrict__ routes_ws, int R, int E_l,
                                                        int32_t* ids, float* weights, int32_t* counts,
                                                        int32_t* offsets, int32_t* routes) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int Rl = min(max(plan->R_local, 0), R);
  if (i < R) {
    if (ids != nullptr) ids[i] = ids_ws[i];
    if (weights != nullptr) weights[i] = weights_ws[i];
    if (routes != nullptr) routes[i] = i < Rl ? routes_ws[i] : -1;
  }
  if (i < E_l && counts != nullptr) counts[i] = counts_ws[i];
  if (i <= E_l && offsets != nullptr) offsets[i] = offsets_ws[i];
}

}  // namespace moe
