// Dispatch order of the sequences of a decode launch: longest first.
//
// The attention workgroups of one (kv head, sequence, key range) stream very
// different amounts of cache when sequence lengths vary widely; dispatching
// them in the caller's order leaves long workgroups starting last, so the
// launch ends with a tail in which few workgroups run.  This kernel writes a
// permutation of the sequence indices sorted by length, longest first, which
// the decode kernel follows (longest-processing-time-first scheduling).
// Results do not depend on the order: each workgroup computes the same values
// whichever grid index runs it.
//
// One workgroup, counting sort on 32-token length buckets (coarser for very
// long sequences so that at most kBuckets buckets exist): histogram in LDS,
// exclusive scan from the longest bucket down, then a scatter.  Ties (one
// bucket) come out in an arbitrary order, which is harmless.
//
// For the one-launch mixed step it also lists the sequences with several
// query rows (the prefill work, in any order) with their count, and zeroes
// the two work-queue counters that launch uses; the attention kernel that
// reads them is the next launch on the same stream.
#include <algorithm>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kBuckets = 4096;
constexpr int kPerThread = kBuckets / kThreads;

__global__ void __launch_bounds__(kThreads) seq_order_kernel(const int32_t* __restrict__ seq_lens,
                                                             int32_t num_seqs, int32_t max_len,
                                                             int32_t bucket_tokens,
                                                             int32_t* __restrict__ order,
                                                             const int32_t* __restrict__ cu,
                                                             int32_t num_tokens,
                                                             int32_t* __restrict__ multi_list,
                                                             int32_t* __restrict__ multi_count,
                                                             int32_t* __restrict__ queues) {
  __shared__ int32_t s_cnt[kBuckets];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int32_t s_multi;
  const int tid = threadIdx.x;
  for (int b = tid; b < kBuckets; b += kThreads) s_cnt[b] = 0;
  if (tid == 0) s_multi = 0;
  __syncthreads();
  // sequences with several query rows (query ranges clamped as the
  // attention kernels clamp them)
  if (cu) {
    for (int s = tid; s < num_seqs; s += kThreads) {
      const int qs = clamp_i(cu[s], 0, num_tokens), qe = clamp_i(cu[s + 1], 0, num_tokens);
      if (qe - qs > 1) multi_list[atomicAdd(&s_multi, 1)] = s;
    }
  }
  auto bucket = [&](int s) {
    const int L = clamp_i(seq_lens[s], 0, max_len);
    // longest first: bucket 0 holds the longest sequences
    return kBuckets - 1 - min(kBuckets - 1, (L + bucket_tokens - 1) / bucket_tokens);
  };
  for (int s = tid; s < num_seqs; s += kThreads) atomicAdd(&s_cnt[bucket(s)], 1);
  __syncthreads();

  // exclusive scan over the buckets: thread t owns buckets t*kPerThread ..
  int v[kPerThread];
  int run = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    v[i] = run;
    run += s_cnt[tid * kPerThread + i];
  }
  const int lane = tid & 63, wave = tid >> 6;
  int incl = run;                                   // inclusive scan of thread totals
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += s_wave[w];
  const int tbase = wbase + incl - run;             // exclusive prefix of this thread
  __syncthreads();                                  // every count read before rewriting
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) s_cnt[tid * kPerThread + i] = tbase + v[i];
  __syncthreads();

  for (int s = tid; s < num_seqs; s += kThreads) {
    const int pos = atomicAdd(&s_cnt[bucket(s)], 1);
    order[pos] = s;
  }
  if (cu && tid == 0) multi_count[0] = s_multi;     // s_multi is final after the barriers
  if (queues && tid < 2) queues[tid] = 0;            // work queues of the mixed launch
}

}  // namespace

hipError_t launch_seq_order(const int32_t* seq_lens, int32_t num_seqs, int32_t max_len,
                            int32_t* order, const int32_t* cu_seqlens_q, int32_t num_tokens,
                            int32_t* multi_list, int32_t* multi_count, int32_t* queues,
                            hipStream_t stream) {
  if (num_seqs <= 0) return hipSuccess;
  const int64_t want = ((int64_t)max_len + kBuckets - 2) / (kBuckets - 1);   // tokens per bucket
  const int32_t bucket_tokens = (int32_t)std::max<int64_t>(32, ((want + 31) / 32) * 32);
  hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(kThreads), 0, stream, seq_lens, num_seqs,
                     max_len, bucket_tokens, order, cu_seqlens_q, num_tokens, multi_list,
                     multi_count, queues);
  return hipGetLastError();
}

}  // namespace pkv
