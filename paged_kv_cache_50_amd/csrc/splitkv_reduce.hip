// Merge of split-KV partial results by log-sum-exp (the merge of partial
// attention states named in the vLLM book, ch. 6 "forward()", applied to the
// split buffer of "build() étape par étape").
//
// Each partition p of a row's key range left a normalised partial output o_p
// and lse_p = log2 sum_j 2^(s_j) over its keys (logits in log2 units).  With
// M = max_p lse_p:  LSE = M + log2 sum_p 2^(lse_p - M),
//                   out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
// Rows whose key range was not split were written by the partition kernel and
// are skipped here.  Only partitions that start before the row's last key are
// read, so stale workspace entries from earlier calls are never used.
#include "attn_common.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <typename T, int D>
__global__ void __launch_bounds__(256) splitkv_reduce_kernel(const AttnArgs a) {
  constexpr int HPB = 256 / D;  // heads per workgroup
  const int head = blockIdx.y * HPB + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (head >= a.num_heads) return;
  Item it;
  if (!resolve_item(a, blockIdx.x, it)) return;
  if (it.nparts <= 1) return;
  const int64_t stride = (int64_t)a.num_heads * a.num_seqs;  // between partitions
  const int64_t base = (int64_t)head * a.num_seqs + it.seq;
  float M = -INFINITY;
  for (int p = 0; p < it.nparts; ++p) M = fmaxf(M, a.ws_lse[base + p * stride]);
  const float Mref = (M == -INFINITY) ? 0.f : M;
  float O = 0.f, Ls = 0.f;
  for (int p = 0; p < it.nparts; ++p) {
    const float w = fast_exp2(a.ws_lse[base + p * stride] - Mref);
    O = fmaf(w, a.ws_o[(base + p * stride) * D + d], O);
    Ls += w;
  }
  const float v = Ls > 0.f ? O / Ls : 0.f;
  const int64_t oidx = ((int64_t)it.row * a.num_heads + head) * D + d;
  if constexpr (sizeof(T) == 4)
    static_cast<float*>(a.out)[oidx] = v;
  else
    static_cast<uint16_t*>(a.out)[oidx] = static_cast<uint16_t>(f32_to_bf16_rne(v));
  if (d == 0 && a.lse_out)
    a.lse_out[(int64_t)it.row * a.num_heads + head] =
        Ls > 0.f ? (M + acc_log2(Ls)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_splitkv_reduce(const AttnArgs& a, int dtype, int head_size, hipStream_t st) {
  const int hpb = 256 / head_size;
  dim3 grid(a.num_seqs, (a.num_heads + hpb - 1) / hpb);
  if (dtype == 0 && head_size == 64)
    hipLaunchKernelGGL((splitkv_reduce_kernel<float, 64>), grid, dim3(256), 0, st, a);
  else if (dtype == 0 && head_size == 128)
    hipLaunchKernelGGL((splitkv_reduce_kernel<float, 128>), grid, dim3(256), 0, st, a);
  else if (dtype == 1 && head_size == 64)
    hipLaunchKernelGGL((splitkv_reduce_kernel<uint16_t, 64>), grid, dim3(256), 0, st, a);
  else if (dtype == 1 && head_size == 128)
    hipLaunchKernelGGL((splitkv_reduce_kernel<uint16_t, 128>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
