// Chunked-prefill kernel on the matrix cores: one workgroup per (query tile,
// head group, sequence); the work itself is pf::prefill_block.  The cascade
// prefix pass uses the same body over (query tile of the whole batch, head
// group, prefix key partition).  Both number the workgroups of a z slice so
// that each XCD takes whole (head group, z) streams (pf::xcd_stream_order).
// DT is the cache's pkv_dtype (bfloat16, binary16 or e4m3).
#include "attn_mfma_prefill.h"

namespace pkv {
namespace {

template <int BS, int DT>
__global__ void __launch_bounds__(pf::kThreads, 2) attn_mfma_prefill_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[pf::kLdsBytes];
  pf::prefill_block<BS, false, DT, true>(a, blockIdx.x, blockIdx.y, blockIdx.z + a.z_base, s_lds);
}

template <int BS, int DT>
__global__ void __launch_bounds__(pf::kThreads, 2) attn_mfma_prefix_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s_lds[pf::kLdsBytes];
  pf::prefill_block<BS, true, DT, true>(a, blockIdx.x, blockIdx.y, blockIdx.z, s_lds);
}

template <bool PREFIX, int BS, int DT>
hipError_t launch_one(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (PREFIX)
    hipLaunchKernelGGL((attn_mfma_prefix_kernel<BS, DT>), grid, dim3(pf::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_mfma_prefill_kernel<BS, DT>), grid, dim3(pf::kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool PREFIX, int DT>
hipError_t launch_bs(const AttnArgs& a, int block_size, dim3 grid, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_one<PREFIX, 8, DT>(a, grid, stream);
    case 16: return launch_one<PREFIX, 16, DT>(a, grid, stream);
    case 32: return launch_one<PREFIX, 32, DT>(a, grid, stream);
    case 64: return launch_one<PREFIX, 64, DT>(a, grid, stream);
    case 128: return launch_one<PREFIX, 128, DT>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool PREFIX>
hipError_t launch_dt(const AttnArgs& a, int block_size, int dtype, dim3 grid, hipStream_t stream) {
  switch (dtype) {
    case PKV_BF16: return launch_bs<PREFIX, PKV_BF16>(a, block_size, grid, stream);
    case PKV_F16: return launch_bs<PREFIX, PKV_F16>(a, block_size, grid, stream);
    case PKV_FP8_E4M3: return launch_bs<PREFIX, PKV_FP8_E4M3>(a, block_size, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_mfma_prefix(const AttnArgs& a, int block_size, int dtype, dim3 grid,
                                   hipStream_t stream) {
  return launch_dt<true>(a, block_size, dtype, grid, stream);
}

hipError_t launch_attn_mfma_prefill(const AttnArgs& a, int block_size, int dtype, dim3 grid,
                                    hipStream_t stream) {
  return launch_dt<false>(a, block_size, dtype, grid, stream);
}

}  // namespace pkv
