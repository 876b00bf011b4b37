// Down projection of the many-routes regime (list path): a grouped GEMM per
// touched expert, weights streamed once from packed MXFP4, four 16-row
// weight sets per wave.
//
// What it computes is mfma_kernel's down projection ("MXFP4 MoE decode
// kernels", Design: intermediate -> down + bias per route, the token sum
// following in the combine), for experts with many routes, where every
// weight value meets tens of intermediate rows and the product is a real
// dense contraction.  The layout differs where that regime needs it on
// gfx950:
//
//  * a wave owns four 16-row weight sets (64 output rows), so each
//    intermediate operand read from LDS feeds four v_mfma_f32_16x16x32_bf16,
//    half the LDS traffic per weight byte of mfma_kernel's two; a workgroup
//    of four waves covers 256 output rows;
//  * the intermediate rows of the pass's routes (up to 64, four groups of
//    16) reach LDS by direct buffer->LDS loads, one 128-value chunk per step
//    in a 3-buffer ring, two steps ahead, with no register staging; a row is
//    256 bytes, its 16-byte pieces XOR-swizzled by the row's low three bits
//    so that the operand reads of eight consecutive lanes hit eight
//    different bank groups without padding (a direct load fills 1 KB of LDS
//    contiguously);
//  * weights stream through a register ring of buffer loads (3 steps, 2
//    with four token groups, whose 64 accumulators leave no room for a
//    third) whose offsets differ only by wave-uniform amounts (one VGPR
//    offset for all four sets); each step's scale bytes of the wave's 64
//    rows (one dword per row) reach a per-wave LDS ring by one direct dword
//    load; steps past the reduction load with an out-of-range offset, so
//    every step issues the same loads and the compiler's wait counts stay
//    exact;
//  * the operand and scale reads are asm blocks that wait for themselves
//    (the compiler sees no LDS read to pair with the in-flight direct loads,
//    so it adds no wait for them); each step's own direct loads are waited
//    for explicitly before the one barrier of the step.
// At 168 VGPRs three workgroups share a CU (three waves per SIMD).
//
// The reduction order is mfma_kernel's: per (row set, token group) one
// accumulator, chunks in order, the four MFMAs of a chunk in order, lane
// group q carrying block 4c + q of chunk c; so both kernels give the same
// bits on the same work.  Requires I a multiple of 128 (whole steps) and K
// a multiple of 256 (whole tiles); the host takes mfma_kernel otherwise.
// (The same structure for the gate/up projection, 128 intermediate columns
// per workgroup, measured slower than mfma_kernel there and is not built.)
#include "kernels.h"
#include "list_common.h"

#include <numeric>
#include <type_traits>

namespace moe {

namespace {

constexpr int kD4XRing = 3;                // staged activation steps (two ahead of the one in use)
constexpr int kD4Row = 256;                // LDS bytes of one token's 128-value chunk
constexpr int kD4Buf = 64 * kD4Row;        // one staged step for 64 tokens
constexpr int kD4ScaleSlot = 256;          // one step's scale dwords of a wave's 64 rows
static_assert(kD4LdsBytes == kD4XRing * kD4Buf + 4 * kD4ScaleSlots * kD4ScaleSlot, "LDS layout");
// Cache policy of the weight loads: non-temporal (each byte is read once),
// so that the weight stream does not evict from L2 the intermediate rows the
// expert's other row tiles still read, nor the scale lines of later steps.
constexpr int kNt = 2;

__device__ __forceinline__ bf16x8 decode8(uint32_t d, float s) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
  bf16x8 v;
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
  return v;
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// The activation operands of one sub-step for kNG token groups, read from LDS
// and waited for in the same asm block (addresses: tg * 16 rows apart).
template <int kNG>
__device__ __forceinline__ void read_operands(uint32_t addr, bf16x8 (&b)[4]) {
  u32x4 v0, v1, v2, v3;
  if constexpr (kNG == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v0) : "v"(addr) : "memory");
  } else if constexpr (kNG == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:4096\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v0), "=v"(v1) : "v"(addr) : "memory");
  } else if constexpr (kNG == 3) {
    asm volatile(
        "ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:4096\n\tds_read_b128 %2, %3 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(v0), "=v"(v1), "=v"(v2) : "v"(addr) : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:4096\n\tds_read_b128 %2, %4 offset:8192\n\t"
        "ds_read_b128 %3, %4 offset:12288\n\ts_waitcnt lgkmcnt(0)"
        : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3) : "v"(addr) : "memory");
  }
  b[0] = __builtin_bit_cast(bf16x8, v0);
  if constexpr (kNG > 1) b[1] = __builtin_bit_cast(bf16x8, v1);
  if constexpr (kNG > 2) b[2] = __builtin_bit_cast(bf16x8, v2);
  if constexpr (kNG > 3) b[3] = __builtin_bit_cast(bf16x8, v3);
}

// The scale bytes of a lane's four row sets for its block: byte q of row
// (set s, r), stored at 4 (16 s + r) of the wave's slot (addr = slot + 4r + q).
__device__ __forceinline__ void read_scales(uint32_t addr, uint32_t (&sb)[4]) {
  asm volatile(
      "ds_read_u8 %0, %4\n\tds_read_u8 %1, %4 offset:64\n\tds_read_u8 %2, %4 offset:128\n\t"
      "ds_read_u8 %3, %4 offset:192\n\ts_waitcnt lgkmcnt(0)"
      : "=v"(sb[0]), "=v"(sb[1]), "=v"(sb[2]), "=v"(sb[3]) : "v"(addr) : "memory");
}

// f(integral_constant<J>) for J = 0 .. kN - 1, in order.
template <int kN, int kJ = 0, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (kJ < kN) {
    f(std::integral_constant<int, kJ>{});
    unroll<kN, kJ + 1>(f);
  }
}

// s_waitcnt with only the vector-memory count set.
template <int kN>
__device__ __forceinline__ void wait_vm() {
  static_assert(kN >= 0 && kN < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace

__global__ __launch_bounds__(256, 3) void down4_kernel(ExpertArgs A) {
  // [kD4XRing][64 intermediate rows][kD4Row] (swizzled), then per wave [kD4ScaleSlots][kD4ScaleSlot]
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int kTileRows = 256;  // output rows of a work item

  const int tiles = A.rows / kTileRows;
  // XCD-aware order (block b runs on XCD b % 8): XCD x takes list entries
  // x, x + 8, ..., each with all of its row tiles, so the tiles of one
  // expert stage the same intermediate rows through one L2.  The host pads
  // the grid to 8 * tiles * ceil(experts / 8).
  const int xcd = static_cast<int>(blockIdx.x) & 7, kx = static_cast<int>(blockIdx.x) >> 3;
  const int item = xcd + 8 * (kx / tiles);
  const int tile = kx - (kx / tiles) * tiles;
  if (A.plan->key != A.key) return;  // no plan for this call in the workspace (whole workgroup)
  const int n_items = min(max(A.plan->n_mfma, 0), A.list_cap);
  const WorkEntry we = clamp_entry(A.list[min(item, A.list_cap - 1)], A);
  if (item >= n_items) return;  // whole workgroup

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int red = A.red, RB = red >> 5, NC = RB >> 2;  // steps of 128 values
  const int rows = A.rows;
  const uint32_t row_bytes = static_cast<uint32_t>(red) >> 1;

  // Row sets of this wave: rows n0 + 16 s + r, n0 = tile*256 + 64*wave.
  const int n0 = tile * kTileRows + wave * 64;

  const uint32_t expert_bytes = static_cast<uint32_t>(rows) * row_bytes;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A.wp + static_cast<size_t>(we.e) * expert_bytes), 0, expert_bytes, 0x00020000);
  const uint32_t scale_bytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(RB);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A.ws + static_cast<size_t>(we.e) * scale_bytes), 0, scale_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.in), 0, A.in_bytes, 0x00020000);

  // Lane (r, q) loads block 4c + q of row n0 + 16 s + r at step c: one VGPR
  // offset, the set and the step in the (uniform) scalar offset.
  //   tiled: (row & ~15) * row_bytes + 16 (row & 15) + 256 b = set base + 16 lane + 1024 c
  //   rows:  row * row_bytes + 16 b = set base + r * row_bytes + 16 q + 64 c
  const bool tiled = A.tiled != 0;
  const uint32_t wv = tiled ? 16u * static_cast<uint32_t>(lane) : static_cast<uint32_t>(r) * row_bytes + 16u * q;
  const uint32_t wstep = tiled ? 1024u : 64u;
  uint32_t wset[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) wset[s] = static_cast<uint32_t>(n0 + 16 * s) * row_bytes;
  // scale dword of step c for row n0 + lane (set lane / 16, row lane % 16): sv + 4c
  const uint32_t sv = static_cast<uint32_t>(n0 + lane) * static_cast<uint32_t>(RB);
  unsigned char* const scale_ring = lds + kD4XRing * kD4Buf + wave * (kD4ScaleSlots * kD4ScaleSlot);
  const uint32_t sc_rd = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(scale_ring)) + 4u * r + q;

  // Direct-load role: wave w fills rows 16j + 4w .. 16j + 4w + 3 of group j;
  // lane L the 16-byte slot L & 15 of row 16j + 4w + L / 16, which holds the
  // row's logical piece (L & 15) ^ (row & 7).
  const int dt = 4 * wave + (lane >> 4);  // row within a group
  const uint32_t dpiece = static_cast<uint32_t>((lane & 15) ^ (dt & 7));
  const uint32_t xrow_bytes = static_cast<uint32_t>(red) * 2u;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  // operand reads: lane (r, q) of sub-step g reads row 16 tg + r, logical
  // piece 4q + g
  const uint32_t rd_row = lds_base + static_cast<uint32_t>(r) * kD4Row;

  for (int tp0 = 0; tp0 < we.Te; tp0 += 64) {
    const int nt = min(64, we.Te - tp0);
    const int NG = (nt + 15) >> 4;
    uint32_t xoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * j + dt;
      const int p = we.p0 + tp0 + (t < nt ? t : 0);  // the intermediate row of plan position p
      xoff[j] = t < nt ? static_cast<uint32_t>(p) * xrow_bytes + 16u * dpiece : kOob;
    }

    // kR: weight steps in flight
    auto pass = [&](auto ng, auto ring) {
      constexpr int kNG = decltype(ng)::value;
      constexpr int kR = decltype(ring)::value;
      // direct loads of step c into ring buffer c % 3 (out of range past the
      // reduction: they fill that buffer with zeros, which nothing reads)
      auto stage = [&](int c, int buf) {
        const bool in = c < NC;
#pragma unroll
        for (int j = 0; j < kNG; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xrs,
              reinterpret_cast<__attribute__((address_space(3))) void*>(
                  reinterpret_cast<uintptr_t>(lds + buf * kD4Buf + (16 * j + 4 * wave) * kD4Row)),
              16, in ? xoff[j] : kOob, static_cast<uint32_t>(c) * kD4Row, 0, 0);
      };
      u32x4 wr[kR][4];
      auto wload = [&](int c, int slot, int sslot) {
        const bool in = c < NC;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          wr[slot][s] = __builtin_amdgcn_raw_buffer_load_b128(wrs, in ? wv : kOob, wset[s] + wstep * c, kNt);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            srs,
            reinterpret_cast<__attribute__((address_space(3))) void*>(
                reinterpret_cast<uintptr_t>(scale_ring + sslot * kD4ScaleSlot)),
            4, in ? sv : kOob, 4u * static_cast<uint32_t>(c), 0, 0);
      };

      f32x4 acc[4][kNG];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int g = 0; g < kNG; ++g) acc[s][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

      static_assert(kR <= kD4ScaleSlots, "a step's scales land after the scale slot's last read");
      // prologue: steps 0 and 1 staged, weights of steps 0 .. kR - 1 in flight
      stage(0, 0);
      wload(0, 0, 0);
      stage(1, 1);
#pragma unroll
      for (int j = 1; j < kR; ++j) wload(j, j, j);

      // step c: (1) its direct loads and scales done: the intermediate rows
      // were requested at step c - 2, and after them this wave issued 5
      // weight/scale loads at the end of step c - 2, kNG direct loads at step
      // c - 1 and 5 at its end; the scales came with step c's weights, at the
      // end of step c - kR, before the rows when kR > 2 and else followed by
      // kNG + 5 loads; (2) the barrier (every wave's loads of step c landed,
      // every wave done reading step c - 1's buffer), (3) stage step c + 2
      // into that buffer, (4) the MFMAs, (5) refill this weight slot with
      // step c + kR.  x0 = c % 3 (row buffer), s0 = c % kR (weight slot), ss
      // = c % kD4ScaleSlots (scale slot).
      auto step = [&](int c, auto xslot, auto wslot, auto sslot) {
        constexpr int x0 = decltype(xslot)::value;
        constexpr int s0 = decltype(wslot)::value;
        constexpr int ss = decltype(sslot)::value;
        wait_vm<(kR > 2 ? 10 : 5) + kNG>();
        __builtin_amdgcn_s_barrier();
        stage(c + 2, (x0 + 2) % kD4XRing);
        if (c < NC) {
          const uint32_t buf = rd_row + x0 * kD4Buf;
          // lane group q takes block 4c + q: byte q of its row's scale dword
          uint32_t sb[4];
          read_scales(sc_rd + ss * kD4ScaleSlot, sb);
          float sc[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) sc[s] = e8m0_to_f32(sb[s]);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x8 b[4];
            // logical piece 4q + g of row r (swizzled by r & 7; rows 16 tg + r
            // share r & 7)
            read_operands<kNG>(buf + 16u * static_cast<uint32_t>((4 * q + g) ^ (r & 7)), b);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const bf16x8 a = decode8(wr[s0][s][g], sc[s]);
#pragma unroll
              for (int tg = 0; tg < kNG; ++tg)
                acc[s][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[tg], acc[s][tg], 0, 0, 0);
            }
          }
        }
        wload(c + kR, s0, (ss + kR) % kD4ScaleSlots);
      };
      // unrolled by lcm(3, kR, kD4ScaleSlots) steps, so that every ring slot
      // is a constant
      constexpr int kU = std::lcm(std::lcm(3, kR), kD4ScaleSlots);
      for (int c0 = 0; c0 < NC; c0 += kU) {
        unroll<kU>([&](auto j) {
          constexpr int J = decltype(j)::value;
          step(c0 + J, std::integral_constant<int, J % 3>{}, std::integral_constant<int, J % kR>{},
               std::integral_constant<int, J % kD4ScaleSlots>{});
        });
      }

      // epilogue: lane holds rows 4q + i (i < 4) of each set, route tg*16 + r
      const size_t bb = static_cast<size_t>(we.e) * rows;
#pragma unroll
      for (int tg = 0; tg < kNG; ++tg) {
        const int tt = tg * 16 + r;
        if (tt >= nt) continue;
        const size_t p = static_cast<size_t>(we.p0 + tp0 + tt);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int n = n0 + 16 * s + 4 * q;
          float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (A.bias != nullptr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i] = bf16_bits_to_f32(A.bias[bb + n + i]);
          }
          *reinterpret_cast<float4*>(A.o_out + p * rows + n) =
              make_float4(acc[s][tg][0] + b[0], acc[s][tg][1] + b[1], acc[s][tg][2] + b[2], acc[s][tg][3] + b[3]);
        }
      }
    };
    using R2 = std::integral_constant<int, 2>;
    using R3 = std::integral_constant<int, 3>;
    if (NG >= 4) pass(std::integral_constant<int, 4>{}, R2{});
    else if (NG == 3) pass(std::integral_constant<int, 3>{}, R3{});
    else if (NG == 2) pass(std::integral_constant<int, 2>{}, R3{});
    else pass(std::integral_constant<int, 1>{}, R3{});
    // the next pass restages the buffers: every wave must be done with them,
    // and this wave's direct loads past the reduction must have landed
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
  }
}

}  // namespace moe
