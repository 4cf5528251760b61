// Chunked-prefill kernel on the matrix cores: one workgroup per (query tile,
// head group, sequence); the work itself is pf::prefill_block.  The cascade
// prefix pass uses the same body over (query tile of the whole batch, head
// group, prefix key partition).  FP8 selects the e4m3-cache form.
#include "attn_mfma_prefill.h"

namespace pkv {
namespace {

template <int BS, bool FP8>
__global__ void __launch_bounds__(pf::kThreads, 2) attn_mfma_prefill_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[pf::kLdsBytes];
  pf::prefill_block<BS, false, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z + a.z_base, s_lds);
}

template <int BS, bool FP8>
__global__ void __launch_bounds__(pf::kThreads, 2) attn_mfma_prefix_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[pf::kLdsBytes];
  pf::prefill_block<BS, true, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z, s_lds);
}

#define PKV_LAUNCH_BS_FP8(KERNEL)                                                                 \
  switch (block_size * 2 + (fp8 ? 1 : 0)) {                                                       \
    case 16: hipLaunchKernelGGL((KERNEL<8, false>), grid, dim3(pf::kThreads), 0, stream, a); break;  \
    case 17: hipLaunchKernelGGL((KERNEL<8, true>), grid, dim3(pf::kThreads), 0, stream, a); break;   \
    case 32: hipLaunchKernelGGL((KERNEL<16, false>), grid, dim3(pf::kThreads), 0, stream, a); break; \
    case 33: hipLaunchKernelGGL((KERNEL<16, true>), grid, dim3(pf::kThreads), 0, stream, a); break;  \
    case 64: hipLaunchKernelGGL((KERNEL<32, false>), grid, dim3(pf::kThreads), 0, stream, a); break; \
    case 65: hipLaunchKernelGGL((KERNEL<32, true>), grid, dim3(pf::kThreads), 0, stream, a); break;  \
    default: return hipErrorInvalidValue;                                                         \
  }

}  // namespace

hipError_t launch_attn_mfma_prefix(const AttnArgs& a, int block_size, bool fp8, dim3 grid,
                                   hipStream_t stream) {
  PKV_LAUNCH_BS_FP8(attn_mfma_prefix_kernel)
  return hipGetLastError();
}

hipError_t launch_attn_mfma_prefill(const AttnArgs& a, int block_size, bool fp8, dim3 grid,
                                    hipStream_t stream) {
  PKV_LAUNCH_BS_FP8(attn_mfma_prefill_kernel)
  return hipGetLastError();
}

}  // namespace pkv
