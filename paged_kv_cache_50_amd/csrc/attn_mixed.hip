// Mixed step in one launch: the chunked-prefill tiles and the decode rows of
// a varlen batch run in one persistent grid (vLLM book, ch. 6 "Structure des
// métadonnées": one forward over a batch that mixes prefill chunks and
// decode rows).  The same grid runs a cascade whose rows are all decode
// rows: the prefix pass on the matrix cores beside the suffix pass's decode
// rows streaming each request's own keys (ch. 6 "forward()", the cascade
// branch).
//
// The prefill tiles keep the matrix cores and vector ALUs busy while the
// decode rows stream the cache from HBM, so the two kinds of work should
// overlap instead of running one after the other.  The hardware refills a
// freed slot with the next workgroup in grid order, so a plain interleaved
// grid ends up with every slot holding prefill work; here the grid has two
// workgroups per CU, each starting on one kind and taking items from that
// kind's queue (an atomic counter the planner zeroes before the launch),
// moving to the other queue when its own is empty.  Every workgroup leaves
// once both queues are exhausted.
#include "attn_mfma_decode.h"
#include "attn_mfma_prefill.h"

namespace pkv {
namespace {

constexpr int kLdsBytes = pf::kLdsBytes > dec::kLdsBytes ? pf::kLdsBytes : dec::kLdsBytes;
static_assert(pf::kThreads == dec::kThreads, "one block shape");

// CASCADE: the first kind of work is the cascade prefix pass (items = query
// tile x head group x prefix partition, a fixed count) instead of the
// listed prefill chunks.  DT: the cache's pkv_dtype (bfloat16, binary16 or
// e4m3, for both kinds of work; the decode rows with one kv head per wave).
template <int BS, bool CASCADE, int DT>
__global__ void __launch_bounds__(dec::kThreads, 2) attn_mixed_kernel(const AttnArgs pre,
                                                                       const AttnArgs dcd,
                                                                       const MixedGrid g) {
  __shared__ __attribute__((aligned(16))) char s_lds[kLdsBytes];
  __shared__ float s_m[dec::kWaves][32];
  __shared__ float s_l[dec::kWaves][32];
  __shared__ int s_item;

  // prefill items of the listed multi-row sequences; decode items as in the
  // decode kernel's grid (kv-head chunk fastest, then row item, then range)
  const int64_t n_pre = CASCADE ? (int64_t)g.pre_x * g.pre_y * g.pre_z
                               : (int64_t)load_uniform_i32(g.pre_count, 0) * g.pre_x * g.pre_y;
  const int64_t n_dec = g.n_dec;
  // Start roles.  Workgroup i runs on XCD i % 8, and workgroups i and
  // i + 8k of one XCD fill its CUs in turn, so (i / 8) % 4 classes the CUs
  // of every XCD in four (the two workgroups of a CU, i and i + 256 on a
  // 256-CU chip, fall in one class).  For a mixed step, the CUs of the
  // classes below pre_share start on prefill tiles in every XCD, and the
  // others on decode rows: both kinds then draw on every XCD's share of HBM
  // bandwidth, and each CU keeps one kind.  For a cascade the XCDs with
  // i % 4 < pre_share start on prefix items (whole XCDs per role).  A
  // workgroup whose queue is empty moves to the other one, and stops when
  // both are.
  int role = CASCADE ? ((int)(blockIdx.x & 3) < g.pre_share ? 0 : 1)
                     : ((int)((blockIdx.x >> 3) & 3) < g.pre_share ? 0 : 1);
  bool switched = false;
  // Mixed step: a workgroup that starts on prefill takes its first item by
  // its rank among those workgroups (the first pre_share CU classes of every
  // whole group of 32: n_first of them, n_first / 8 on each XCD) instead of
  // by its order of arrival at the queue; later items come from the queue,
  // offset by n_first.  When a whole number of streams (the query tiles of
  // one head group of one chunk) fits each XCD's share, the streams are
  // dealt over the XCDs, whole: the tiles of a stream then share one L2,
  // and every XCD gets streams of every chunk.  Otherwise the first items
  // follow the ranks.
  const uint32_t whole = gridDim.x / 32 * 32;
  int n_first = CASCADE ? 0 : (int)(whole / 32) * 8 * g.pre_share;
  int first = -1;
  if (CASCADE && gridDim.x % 8 == 0) {
    // Cascade: the workgroups of the XCDs that start on prefix items
    // (x % 4 < pre_share, 2 * pre_share XCDs, gridDim.x / 8 workgroups on
    // each) take their first item by rank in the same way, whole streams
    // (the query tiles of one head group and prefix partition) dealt over
    // those XCDs when they fit, else in rank order.
    const int nx = 2 * g.pre_share;
    const int per_xcd = (int)(gridDim.x / 8);
    n_first = nx * per_xcd;
    const int x = (int)(blockIdx.x % 8);
    if ((x & 3) < g.pre_share) {
      const int xr = (x >> 2) * g.pre_share + (x & 3);
      const int j = (int)(blockIdx.x / 8);
      first = per_xcd % g.pre_x == 0 ? (xr + nx * (j / g.pre_x)) * g.pre_x + j % g.pre_x
                                     : j * nx + xr;
    }
  }
  if (!CASCADE && role == 0 && blockIdx.x < whole) {
    const int per_xcd = n_first / 8;
    const int j = (int)(blockIdx.x / 32) * g.pre_share + (int)((blockIdx.x % 32) / 8);
    if (per_xcd % g.pre_x == 0)
      first = ((int)(blockIdx.x % 8) + 8 * (j / g.pre_x)) * g.pre_x + j % g.pre_x;
    else
      first = (int)(blockIdx.x / 32) * 8 * g.pre_share + (int)(blockIdx.x % 32);
  }
  while (true) {
    __syncthreads();                       // the previous item's LDS use is over
    if (threadIdx.x == 0) {
      if (first >= 0) s_item = first;
      else s_item = atomicAdd(&g.queues[role], 1) + (role == 0 ? n_first : 0);
    }
    first = -1;
    __syncthreads();
    const int64_t item = s_item;
    if (item >= (role == 0 ? n_pre : n_dec)) {
      if (switched) break;
      switched = true;
      role ^= 1;
      continue;
    }
    if (role == 0 && CASCADE) {
      const int bx = (int)(item % g.pre_x);
      const int64_t t = item / g.pre_x;
      const int by = (int)(t % g.pre_y);
      const int part = (int)(t / g.pre_y);
      pf::prefill_block<BS, true, DT>(pre, bx, by, part, s_lds);
    } else if (role == 0) {
      // the last query tiles of a chunk see the most keys: they go first
      const int bx = g.pre_x - 1 - (int)(item % g.pre_x);
      const int64_t t = item / g.pre_x;
      const int by = (int)(t % g.pre_y);
      const int li = (int)(t / g.pre_y);
      pf::prefill_block<BS, false, DT>(pre, bx, by, load_uniform_i32(g.pre_list, li), s_lds);
    } else {
      const int bx = (int)(item % g.dec_x);
      const int64_t t = item / g.dec_x;
      const int zi = (int)(t % g.dec_y);
      const int bz = (int)(t / g.dec_y);
      dec::decode_block<BS, DT, 1>(dcd, bx, zi, bz, g.dec_z, s_lds, s_m, s_l);
    }
  }
}

template <bool CASCADE, int DT>
hipError_t launch(const AttnArgs& pre, const AttnArgs& dcd, const MixedGrid& g, int block_size,
                  hipStream_t stream) {
  if (g.workgroups <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)g.workgroups), block(dec::kThreads);
  switch (block_size) {
    case 8: hipLaunchKernelGGL((attn_mixed_kernel<8, CASCADE, DT>), grid, block, 0, stream, pre, dcd, g); break;
    case 16: hipLaunchKernelGGL((attn_mixed_kernel<16, CASCADE, DT>), grid, block, 0, stream, pre, dcd, g); break;
    case 32: hipLaunchKernelGGL((attn_mixed_kernel<32, CASCADE, DT>), grid, block, 0, stream, pre, dcd, g); break;
    case 64: hipLaunchKernelGGL((attn_mixed_kernel<64, CASCADE, DT>), grid, block, 0, stream, pre, dcd, g); break;
    case 128: hipLaunchKernelGGL((attn_mixed_kernel<128, CASCADE, DT>), grid, block, 0, stream, pre, dcd, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool CASCADE>
hipError_t launch_dt(const AttnArgs& pre, const AttnArgs& dcd, const MixedGrid& g, int block_size,
                     int dtype, hipStream_t stream) {
  switch (dtype) {
    case PKV_BF16: return launch<CASCADE, PKV_BF16>(pre, dcd, g, block_size, stream);
    case PKV_F16: return launch<CASCADE, PKV_F16>(pre, dcd, g, block_size, stream);
    case PKV_FP8_E4M3: return launch<CASCADE, PKV_FP8_E4M3>(pre, dcd, g, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_mixed(const AttnArgs& pre, const AttnArgs& dcd, const MixedGrid& g,
                             int block_size, int dtype, hipStream_t stream) {
  return launch_dt<false>(pre, dcd, g, block_size, dtype, stream);
}

hipError_t launch_attn_cascade(const AttnArgs& pre, const AttnArgs& dcd, const MixedGrid& g,
                               int block_size, int dtype, hipStream_t stream) {
  return launch_dt<true>(pre, dcd, g, block_size, dtype, stream);
}

}  // namespace pkv
