// Chunked-prefill kernel on the matrix cores: one workgroup per (query tile,
// head group, sequence); the work itself is pf::prefill_block.  The cascade
// prefix pass uses the same body over (query tile of the whole batch, head
// group, prefix key partition).
#include "attn_mfma_prefill.h"

namespace pkv {
namespace {

template <int BS>
__global__ void __launch_bounds__(pf::kThreads, 2) attn_mfma_prefill_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[pf::kLdsBytes];
  pf::prefill_block<BS>(a, blockIdx.x, blockIdx.y, blockIdx.z + a.z_base, s_lds);
}

template <int BS>
__global__ void __launch_bounds__(pf::kThreads, 2) attn_mfma_prefix_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[pf::kLdsBytes];
  pf::prefill_block<BS, true>(a, blockIdx.x, blockIdx.y, blockIdx.z, s_lds);
}

}  // namespace

hipError_t launch_attn_mfma_prefix(const AttnArgs& a, int block_size, dim3 grid,
                                   hipStream_t stream) {
  switch (block_size) {
    case 8: hipLaunchKernelGGL((attn_mfma_prefix_kernel<8>), grid, dim3(pf::kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((attn_mfma_prefix_kernel<16>), grid, dim3(pf::kThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((attn_mfma_prefix_kernel<32>), grid, dim3(pf::kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_mfma_prefill(const AttnArgs& a, int block_size, dim3 grid,
                                    hipStream_t stream) {
  switch (block_size) {
    case 8: hipLaunchKernelGGL((attn_mfma_prefill_kernel<8>), grid, dim3(pf::kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((attn_mfma_prefill_kernel<16>), grid, dim3(pf::kThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((attn_mfma_prefill_kernel<32>), grid, dim3(pf::kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
