// Device helpers shared by the list-path kernels (expert_kernels.hip,
// scaled_kernels.hip).  Internal linkage: each translation unit gets its own.
#pragma once
#include "kernels.h"

namespace moe {
namespace list {

// Copy nbytes (a multiple of 4, 4-byte aligned source) from global memory to
// LDS with direct global->LDS loads of one dword per lane; every thread of the
// 256-lane workgroup takes part.  A wave's copy fills 256 contiguous LDS bytes.
__device__ __forceinline__ void dma_strip(const uint8_t* __restrict__ src, unsigned char* dst, int nbytes) {
  const int n = nbytes >> 2;
  for (int i = threadIdx.x; i < n; i += 256) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(src) + i,
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(dst + 4 * (i & ~63))),
                                     4, 0, 0);
  }
}

static constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every range: the load returns zeros

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const __attribute__((ext_vector_type(4))) uint32_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A list entry with every field inside the call's bounds: expert < E_local,
// positions p0 .. p0 + Te - 1 inside [0, R), tokens inside [0, T).  The plan
// kernel writes entries that satisfy this already; the clamp keeps a stale
// or foreign workspace from turning into out-of-range accesses.
__device__ __forceinline__ WorkEntry clamp_entry(WorkEntry we, const ExpertArgs& A) {
  we.e = min(max(we.e, 0), A.list_cap - 1);
  we.p0 = min(max(we.p0, 0), A.R - 1);
  we.Te = min(max(we.Te, 0), A.R - we.p0);
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) we.tok[t] = min(max(we.tok[t], 0), A.T - 1);
  return we;
}

}  // namespace list
using namespace list;
}  // namespace moe
