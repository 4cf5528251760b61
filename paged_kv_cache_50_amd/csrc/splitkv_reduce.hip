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
#include <type_traits>

#include "attn_common.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// T: the output element, float, uint16_t (bfloat16 bits) or _Float16.
template <typename T>
constexpr bool kIsF16 = std::is_same<T, _Float16>::value;

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
      static_cast<uint16_t*>(a.out)[oidx] = static_cast<uint16_t>(Fmt16<kIsF16<T>>::rne(v));
    if (tid == 0 && a.lse_out)
      a.lse_out[(int64_t)it.row * a.num_heads + head] =
          Ls > 0.f ? (M + acc_log2(Ls)) * kLn2 : -INFINITY;
  }
}

// Few ranges per row (at most kMaxFewRanges): grid = (rows, head groups).
// A group of D/4 lanes owns one query head and issues every load of it at
// once (all ranges' lse and partial rows, indices clamped in bounds, unused
// ranges weighted 0), so a row costs one memory round trip, and rows that
// were not split cost one early-exiting workgroup per head group.
constexpr int kMaxFewRanges = 8;

template <typename T, int D>
__global__ void __launch_bounds__(256) splitkv_reduce_few_kernel(const AttnArgs a) {
  constexpr int LR = D / 4;
  constexpr int NG = 256 / LR;
  Item it;
  if (!resolve_item(a, blockIdx.x, it)) return;
  if (it.nranges <= 1) return;
  const int nr = min(it.nranges, kMaxFewRanges);
  const int g = threadIdx.x / LR, c = threadIdx.x % LR;
  const int head = blockIdx.y * NG + g;
  if (head >= a.num_heads) return;
  const int64_t stride = (int64_t)a.num_heads * a.num_seqs;   // between partitions
  const int64_t base = (int64_t)head * a.num_seqs + it.seq;
  float l[kMaxFewRanges];
  f32x4 v[kMaxFewRanges];
#pragma unroll
  for (int p = 0; p < kMaxFewRanges; ++p) {
    const int64_t e = base + (int64_t)min(p, nr - 1) * stride;
    l[p] = a.ws_lse[e];
    v[p] = *reinterpret_cast<const f32x4*>(a.ws_o + e * D + 4 * c);
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kMaxFewRanges; ++p) M = fmaxf(M, p < nr ? l[p] : -INFINITY);
  const float Mref = (M == -INFINITY) ? 0.f : M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int p = 0; p < kMaxFewRanges; ++p) {
    const float w = p < nr ? fast_exp2(l[p] - Mref) : 0.f;
    acc += w * v[p];
    wsum += w;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t oidx = ((int64_t)it.row * a.num_heads + head) * D + 4 * c;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + oidx) = acc * inv;
  } else {
    const uint32_t w0 = pack16x2<kIsF16<T>>(acc[0] * inv, acc[1] * inv);
    const uint32_t w1 = pack16x2<kIsF16<T>>(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + oidx) = make_uint2(w0, w1);
  }
  if (c == 0 && a.lse_out)
    a.lse_out[(int64_t)it.row * a.num_heads + head] =
        wsum > 0.f ? (M + acc_log2(wsum)) * kLn2 : -INFINITY;
}

template <typename T, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  const int max_ranges = a.partition_size > 0
      ? (a.num_splits + a.parts_per_wg - 1) / a.parts_per_wg : 1;
  constexpr int NG = 256 / (D / 4);
  if (max_ranges <= kMaxFewRanges)
    hipLaunchKernelGGL((splitkv_reduce_few_kernel<T, D>),
                       dim3(a.num_seqs, (a.num_heads + NG - 1) / NG), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((splitkv_reduce_kernel<T, D>), dim3(a.num_seqs, a.num_heads), dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitkv_reduce(const AttnArgs& a, int dtype, int head_size, hipStream_t st) {
  auto by_head = [&](auto elem) -> hipError_t {
    using T = decltype(elem);
    switch (head_size) {
      case 64: return launch_typed<T, 64>(a, st);
      case 128: return launch_typed<T, 128>(a, st);
      case 256: return launch_typed<T, 256>(a, st);
      default: return hipErrorInvalidValue;
    }
  };
  if (dtype == PKV_F32) return by_head(float{});
  if (dtype == PKV_BF16) return by_head(uint16_t{});
  if (dtype == PKV_F16) return by_head(_Float16{});
  return hipErrorInvalidValue;
}

}  // namespace pkv
