// Cascade merge: the result of the suffix pass (each row against its own
// keys) combined with the partials of the prefix pass (every row against
// the shared prefix), the merge of attention states that follows the two
// cascade calls in the vLLM book, ch. 6 "forward()".
//
// For one (row, query head) the suffix pass left its normalised output in
// `out` (float32, bfloat16 or binary16: T) and its log-sum-exp (natural log) in lse_suffix; the
// prefix pass left num_parts normalised fp32 partials o_p with log-sum-exps
// lse_p in log2 units.  With every lse in log2 units and M their maximum:
//   out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M),
//   LSE = M + log2 sum_i 2^(lse_i - M)   (written in natural log).
// Rows of sequences with seq_len 0 (batch padding) take no prefix: they keep
// the suffix pass's zeros and -inf.  Rows that belong to no sequence are left
// untouched, as by the plain call.
#include <type_traits>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kMaxPrefixParts = 16;

// T: the output element, float, uint16_t (bfloat16 bits) or _Float16.
template <typename T>
constexpr bool kIsF16 = std::is_same<T, _Float16>::value;

// grid = (rows, head groups of 256 / (D/4) heads); a group of D/4 lanes owns
// one query head and issues all of its loads at once.  NP (a power of two,
// at least num_parts) fixes how many partial slots are loaded; slots past
// num_parts are clamped in bounds and weighted 0.
template <int D, int NP, typename T>
__global__ void __launch_bounds__(256) cascade_merge_kernel(const AttnArgs a,
                                                            const float* __restrict__ lse_suffix,
                                                            int num_parts) {
  constexpr int LR = D / 4;
  constexpr int NG = 256 / LR;
  const int row = blockIdx.x;
  const int g = threadIdx.x / LR, c = threadIdx.x % LR;
  const int head = blockIdx.y * NG + g;
  if (head >= a.num_heads) return;
  // the row's sequence: the last one whose query range starts at or before it
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clamp_i(a.cu_seqlens_q[mid], 0, a.num_tokens) <= row) lo = mid; else hi = mid - 1;
  }
  // rows outside every query range, or past the host bound on query rows,
  // are written by neither pass
  const int qs = clamp_i(a.cu_seqlens_q[lo], 0, a.num_tokens);
  const int qe = clamp_i(a.cu_seqlens_q[lo + 1], 0, a.num_tokens);
  if (row < qs || row >= qe || row - qs >= a.max_query_len) return;
  const bool with_prefix = a.seq_lens[lo] > 0;
  const int np = max(1, min(num_parts, NP));
  const int64_t stride = (int64_t)a.num_heads * a.num_tokens;     // between partitions
  const int64_t base = (int64_t)head * a.num_tokens + row;
  float l[NP];
  f32x4 v[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t e = base + (int64_t)min(p, np - 1) * stride;
    l[p] = a.ws_lse[e];
    v[p] = *reinterpret_cast<const f32x4*>(a.ws_o + e * D + 4 * c);
  }
  const int64_t oi = (int64_t)row * a.num_heads + head;
  f32x4 vs;
  if constexpr (sizeof(T) == 4) {
    vs = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.out) + oi * D + 4 * c);
  } else {
    using H = Fmt16<kIsF16<T>>;
    const uint2 sb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.out) + oi * D + 4 * c);
    vs = f32x4{H::lo(sb.x), H::hi(sb.x), H::lo(sb.y), H::hi(sb.y)};
  }
  const float ls = lse_suffix[oi] * kLog2e;
  float M = ls;
#pragma unroll
  for (int p = 0; p < NP; ++p)
    M = fmaxf(M, with_prefix && p < np ? l[p] : -INFINITY);
  const float Mref = (M == -INFINITY) ? 0.f : M;
  const float ws = ls == -INFINITY ? 0.f : fast_exp2(ls - Mref);
  f32x4 acc = ws * vs;
  float wsum = ws;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float w = with_prefix && p < np ? fast_exp2(l[p] - Mref) : 0.f;
    acc += w * v[p];
    wsum += w;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + oi * D + 4 * c) = acc * inv;
  } else {
    const uint32_t w0 = pack16x2<kIsF16<T>>(acc[0] * inv, acc[1] * inv);
    const uint32_t w1 = pack16x2<kIsF16<T>>(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + oi * D + 4 * c) = make_uint2(w0, w1);
  }
  if (c == 0 && a.lse_out) a.lse_out[oi] = wsum > 0.f ? (M + acc_log2(wsum)) * kLn2 : -INFINITY;
}

template <int D, typename T>
hipError_t launch_np(const AttnArgs& a, const float* lse_suffix, int num_parts,
                     hipStream_t stream) {
  constexpr int NG = 256 / (D / 4);
  const dim3 grid(a.num_tokens, (a.num_heads + NG - 1) / NG), block(256);
  if (num_parts <= 2)
    hipLaunchKernelGGL((cascade_merge_kernel<D, 2, T>), grid, block, 0, stream, a, lse_suffix,
                       num_parts);
  else if (num_parts <= 4)
    hipLaunchKernelGGL((cascade_merge_kernel<D, 4, T>), grid, block, 0, stream, a, lse_suffix,
                       num_parts);
  else if (num_parts <= 8)
    hipLaunchKernelGGL((cascade_merge_kernel<D, 8, T>), grid, block, 0, stream, a, lse_suffix,
                       num_parts);
  else
    hipLaunchKernelGGL((cascade_merge_kernel<D, kMaxPrefixParts, T>), grid, block, 0, stream, a,
                       lse_suffix, num_parts);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_head(const AttnArgs& a, const float* lse_suffix, int num_parts, int head_size,
                       hipStream_t stream) {
  switch (head_size) {
    case 64: return launch_np<64, T>(a, lse_suffix, num_parts, stream);
    case 128: return launch_np<128, T>(a, lse_suffix, num_parts, stream);
    case 256: return launch_np<256, T>(a, lse_suffix, num_parts, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cascade_merge(const AttnArgs& a, const float* lse_suffix, int num_parts,
                                int out_dtype, int head_size, hipStream_t stream) {
  if (num_parts < 1 || num_parts > kMaxPrefixParts) return hipErrorInvalidValue;
  if (out_dtype == PKV_F32) return launch_head<float>(a, lse_suffix, num_parts, head_size, stream);
  if (out_dtype == PKV_BF16)
    return launch_head<uint16_t>(a, lse_suffix, num_parts, head_size, stream);
  if (out_dtype == PKV_F16)
    return launch_head<_Float16>(a, lse_suffix, num_parts, head_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
