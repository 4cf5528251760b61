// Grouped-query (and fp8) decode kernel on the matrix cores: one workgroup per
// (kv-head chunk, row item, key range); the work itself is dec::decode_block.
#include "attn_mfma_decode.h"

namespace pkv {
namespace {

// Three workgroups per CU for fp8 caches with one kv head per wave (more
// loads in flight per CU for a kernel that moves half the bytes per token;
// four measured slower), two with two heads per wave (twice the LDS) and for
// 16-bit caches (three would spill: measured slower).
template <int BS, int DT, int HP, int D>
__global__ void __launch_bounds__(dec::kThreads, DT == PKV_FP8_E4M3 && HP == 1 ? 3 : 2)
    attn_mfma_decode_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[dec::kLdsBytesHp<HP, D>];
  __shared__ float s_m[dec::kWaves][32];
  __shared__ float s_l[dec::kWaves][32];
  dec::decode_block<BS, DT, HP, D>(a, blockIdx.x, blockIdx.y + a.z_base, blockIdx.z, gridDim.z,
                                   s_lds, s_m, s_l);
}

template <int DT, int HP, int D>
hipError_t launch_typed(const AttnArgs& a, int block_size, dim3 grid, hipStream_t stream) {
  switch (block_size) {
    case 8: hipLaunchKernelGGL((attn_mfma_decode_kernel<8, DT, HP, D>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((attn_mfma_decode_kernel<16, DT, HP, D>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((attn_mfma_decode_kernel<32, DT, HP, D>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((attn_mfma_decode_kernel<64, DT, HP, D>), grid, dim3(dec::kThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((attn_mfma_decode_kernel<128, DT, HP, D>), grid, dim3(dec::kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma_decode(const AttnArgs& a, int block_size, int head_size, int dtype,
                                   dim3 grid, hipStream_t stream) {
  if (head_size == 256) {
    // 16-bit caches, one kv head per wave (16-token tiles)
    if (a.heads_per_wave != 1) return hipErrorInvalidValue;
    if (dtype == PKV_BF16) return launch_typed<PKV_BF16, 1, 256>(a, block_size, grid, stream);
    if (dtype == PKV_F16) return launch_typed<PKV_F16, 1, 256>(a, block_size, grid, stream);
    return hipErrorInvalidValue;
  }
  if (head_size != 128) return hipErrorInvalidValue;
  if (dtype == PKV_FP8_E4M3)
    return a.heads_per_wave == 2 ? launch_typed<PKV_FP8_E4M3, 2, 128>(a, block_size, grid, stream)
                                 : launch_typed<PKV_FP8_E4M3, 1, 128>(a, block_size, grid, stream);
  if (a.heads_per_wave == 2) return hipErrorInvalidValue;
  if (dtype == PKV_BF16) return launch_typed<PKV_BF16, 1, 128>(a, block_size, grid, stream);
  if (dtype == PKV_F16) return launch_typed<PKV_F16, 1, 128>(a, block_size, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
