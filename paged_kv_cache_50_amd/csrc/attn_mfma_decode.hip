// Grouped-query (and fp8) decode kernel on the matrix cores: one workgroup per
// (kv-head chunk, row item, key range); the work itself is dec::decode_block.
#include "attn_mfma_decode.h"

namespace pkv {
namespace {

// Three workgroups per CU for fp8 caches (more loads in flight per CU for a
// kernel that moves half the bytes per token; four measured slower), two for
// bfloat16 (three would spill: measured slower).
template <int BS, bool FP8>
__global__ void __launch_bounds__(dec::kThreads, FP8 ? 3 : 2) attn_mfma_decode_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[dec::kLdsBytes];
  __shared__ float s_m[dec::kWaves][16];
  __shared__ float s_l[dec::kWaves][16];
  dec::decode_block<BS, FP8>(a, blockIdx.x, blockIdx.y + a.z_base, blockIdx.z, gridDim.z, s_lds,
                             s_m, s_l);
}

template <bool FP8>
hipError_t launch_typed(const AttnArgs& a, int block_size, dim3 grid, hipStream_t stream) {
  switch (block_size) {
    case 8: hipLaunchKernelGGL((attn_mfma_decode_kernel<8, FP8>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((attn_mfma_decode_kernel<16, FP8>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((attn_mfma_decode_kernel<32, FP8>), grid, dim3(dec::kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma_decode(const AttnArgs& a, int block_size, bool fp8, dim3 grid,
                                   hipStream_t stream) {
  return fp8 ? launch_typed<true>(a, block_size, grid, stream)
             : launch_typed<false>(a, block_size, grid, stream);
}

}  // namespace pkv
