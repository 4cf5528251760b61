// Grouped-query (and fp8) decode kernel on the matrix cores: one workgroup per
// (kv-head chunk, row item, key range); the work itself is dec::decode_block.
#include "attn_mfma_decode.h"

namespace pkv {
namespace {

// Three workgroups per CU for fp8 caches with one kv head per wave (more
// loads in flight per CU for a kernel that moves half the bytes per token;
// four measured slower), two with two heads per wave (twice the LDS) and for
// bfloat16 (three would spill: measured slower).
template <int BS, bool FP8, int HP>
__global__ void __launch_bounds__(dec::kThreads, FP8 && HP == 1 ? 3 : 2)
    attn_mfma_decode_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[dec::kLdsBytesHp<HP>];
  __shared__ float s_m[dec::kWaves][32];
  __shared__ float s_l[dec::kWaves][32];
  dec::decode_block<BS, FP8, HP>(a, blockIdx.x, blockIdx.y + a.z_base, blockIdx.z, gridDim.z,
                                 s_lds, s_m, s_l);
}

template <bool FP8, int HP>
hipError_t launch_typed(const AttnArgs& a, int block_size, dim3 grid, hipStream_t stream) {
  switch (block_size) {
    case 8: hipLaunchKernelGGL((attn_mfma_decode_kernel<8, FP8, HP>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((attn_mfma_decode_kernel<16, FP8, HP>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((attn_mfma_decode_kernel<32, FP8, HP>), grid, dim3(dec::kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma_decode(const AttnArgs& a, int block_size, bool fp8, dim3 grid,
                                   hipStream_t stream) {
  if (!fp8) return a.heads_per_wave == 2 ? hipErrorInvalidValue
                                         : launch_typed<false, 1>(a, block_size, grid, stream);
  return a.heads_per_wave == 2 ? launch_typed<true, 2>(a, block_size, grid, stream)
                               : launch_typed<true, 1>(a, block_size, grid, stream);
}

}  // namespace pkv
