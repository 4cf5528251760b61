// Merge of split-KV partial results by log-sum-exp (the merge of partial
// attention states named in the vLLM book, ch. 6 "forward()", applied to the
// split buffer of "build() étape par étape").
//
// Each partition p of a row's key range left a normalised partial output o_p
// and lse_p = log2 sum_j 2^(s_j) over its keys (logits in log2 units).  With
// M = max_p lse_p:  LSE = M + log2 sum_p 2^(lse_p - M),
//                   out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
// Partials are kept per workgroup range (parts_per_wg consecutive partitions,
// already merged by the same rule inside the workgroup).  Rows with a single
// range were written by the partition kernel and are skipped here.  Only partitions that start before the row's last key are
// read, so stale workspace entries from earlier calls are never used.
#include "attn_common.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// One workgroup per (sequence, query head).  The partials of one row are
// read in parallel: lanes of a group of D/4 lanes hold 4 dims of one
// partition's row, and the 256 / (D/4) groups take partitions round-robin,
// so many rows are in flight at once; the groups are then combined in LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256) splitkv_reduce_kernel(const AttnArgs a) {
  constexpr int LR = D / 4;            // lanes per partial row (4 floats each)
  constexpr int NG = 256 / LR;         // row groups
  __shared__ float s_red[256 / 64];
  __shared__ f32x4 s_acc[NG][LR];
  __shared__ float s_w[NG];
  const int head = blockIdx.y;
  Item it;
  if (!resolve_item(a, blockIdx.x, it)) return;
  if (it.nranges <= 1) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t stride = (int64_t)a.num_heads * a.num_seqs;   // between partitions
  const int64_t base = (int64_t)head * a.num_seqs + it.seq;

  // max of the partitions' log-sum-exps
  float M = -INFINITY;
  for (int p = tid; p < it.nranges; p += 256) M = fmaxf(M, a.ws_lse[base + p * stride]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) s_red[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float Mref = (M == -INFINITY) ? 0.f : M;

  // weighted sum of the partial rows
  const int g = tid / LR, c = tid % LR;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll 4
  for (int p = g; p < it.nranges; p += NG) {
    const float w = fast_exp2(a.ws_lse[base + p * stride] - Mref);
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.ws_o + (base + p * stride) * D + 4 * c);
    acc += w * v;
    wsum += w;
  }
  s_acc[g][c] = acc;
  if (c == 0) s_w[g] = wsum;
  __syncthreads();
  if (tid < D) {
    const int cc = tid / 4, e = tid % 4;
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      O += s_acc[gg][cc][e];
      Ls += s_w[gg];
    }
    const float v = Ls > 0.f ? O / Ls : 0.f;
    const int64_t oidx = ((int64_t)it.row * a.num_heads + head) * D + tid;
    if constexpr (sizeof(T) == 4)
      static_cast<float*>(a.out)[oidx] = v;
    else
      static_cast<uint16_t*>(a.out)[oidx] = static_cast<uint16_t>(f32_to_bf16_rne(v));
    if (tid == 0 && a.lse_out)
      a.lse_out[(int64_t)it.row * a.num_heads + head] =
          Ls > 0.f ? (M + acc_log2(Ls)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_splitkv_reduce(const AttnArgs& a, int dtype, int head_size, hipStream_t st) {
  dim3 grid(a.num_seqs, a.num_heads);
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
