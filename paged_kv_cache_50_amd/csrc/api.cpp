// Host side of libpagedkv.so: argument validation, kernel selection, launch
// geometry, split workspace layout and the host-side metadata validation.
// The C ABI is declared in include/pagedkv.h.  Nothing here outlives a call:
// launch choices arrive with each call (pkv_call_options) and the kernels that
// ran are reported back through it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <unordered_set>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

namespace {

using pkv::AttnArgs;
using pkv::timing_begin;
using pkv::timing_end;

constexpr int32_t kDefaultPartition = 512;
constexpr int32_t kPartitionQuantum = 32;
constexpr int64_t kMaxGridZ = 65535;
constexpr int64_t kMaxGridY = 65535;
// Longest sequence a call takes: key positions plus a window (clamped below
// max_seq_len) and a tile then stay inside int32 in every kernel.
constexpr int32_t kMaxSeqLen = 1 << 30;

// Rows sit at positions below max_seq_len, so a window of max_seq_len - 1
// keys or more excludes no key: such windows are clamped to that width, which
// keeps the kernels' position + window sums inside int32.
int32_t clamp_window(int32_t window_left, int32_t max_seq_len) {
  return window_left >= max_seq_len ? std::max(0, max_seq_len - 1) : window_left;
}

int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_FP8_E4M3 ? 1 : 2; }
bool is_fp8(const pkv_kv_cache* c) { return c->dtype == PKV_FP8_E4M3; }
// bfloat16 or binary16: the two 16-bit formats the matrix-core kernels take
bool is16(int32_t dtype) { return dtype == PKV_BF16 || dtype == PKV_F16; }
// dtype of q / out (and of the split merge's output)
int32_t io_dtype(int32_t dtype) { return dtype == PKV_FP8_E4M3 ? PKV_BF16 : dtype; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch choices of one call (pkv_call_options, 0 = the library's choice)
// and the PKV_RAN_* bits of what it enqueued.
struct Choice {
  int32_t decode_kernel = 0;   // 1 VALU, 2 matrix cores
  int32_t prefill_kernel = 0;  // 1 VALU rows
  int32_t fp8_pairs = 0;       // 1 one kv head per wave
  int32_t mixed = 0;           // 1 separate launches
  int32_t cascade = 0;         // 1 separate launches
  uint32_t ran = 0;
};

pkv_status read_options(const pkv_call_options* o, Choice* c) {
  *c = Choice{};
  if (!o) return PKV_OK;
  if (o->decode_kernel < 0 || o->decode_kernel > 2 || o->prefill_kernel < 0 ||
      o->prefill_kernel > 1 || o->fp8_head_pairs < 0 || o->fp8_head_pairs > 1 ||
      o->mixed_launch < 0 || o->mixed_launch > 1 || o->cascade_launch < 0 ||
      o->cascade_launch > 1)
    return PKV_ERR_SHAPE;
  c->decode_kernel = o->decode_kernel;
  c->prefill_kernel = o->prefill_kernel;
  c->fp8_pairs = o->fp8_head_pairs;
  c->mixed = o->mixed_launch;
  c->cascade = o->cascade_launch;
  return PKV_OK;
}

// Writes the report into the caller's options when the call returns, on
// every path.
struct Report {
  pkv_call_options* o;
  const Choice& c;
  ~Report() {
    if (o) o->launched = c.ran;
  }
};

const char* reason(int32_t dtype, int32_t head_size, int32_t block_size, int32_t num_heads,
                   int32_t num_kv_heads) {
  if (dtype != PKV_F32 && dtype != PKV_BF16 && dtype != PKV_F16 && dtype != PKV_FP8_E4M3)
    return "dtype must be PKV_F32, PKV_BF16, PKV_F16 or PKV_FP8_E4M3";
  if (dtype == PKV_FP8_E4M3 && head_size != 128) return "fp8 caches need head_size 128";
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return "head_size must be 64, 128 or 256";
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64 &&
      block_size != 128)
    return "block_size must be 8, 16, 32, 64 or 128";
  if (num_kv_heads <= 0) return "num_kv_heads must be positive";
  if (num_heads <= 0) return "num_heads must be positive";
  if (num_heads % num_kv_heads != 0) return "num_heads must be a multiple of num_kv_heads";
  return nullptr;
}

pkv_status check_cache(const pkv_kv_cache* c, int32_t num_heads) {
  if (!c || !c->k_cache || !c->v_cache) return PKV_ERR_NULL;
  // block ids are int32 in block tables and slot arithmetic stays in int64
  if (c->num_blocks <= 0 || c->num_blocks > INT32_MAX || c->block_size <= 0 ||
      c->num_kv_heads <= 0 || c->head_size <= 0)
    return PKV_ERR_SHAPE;
  if (reason(c->dtype, c->head_size, c->block_size, num_heads > 0 ? num_heads : c->num_kv_heads,
             c->num_kv_heads))
    return PKV_ERR_UNSUPPORTED;
  const int64_t dense = (int64_t)c->block_size * c->num_kv_heads * c->head_size;
  if (c->block_stride != 0 && c->block_stride < dense) return PKV_ERR_SHAPE;
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache)) return PKV_ERR_ALIGN;
  if (c->dtype == PKV_FP8_E4M3 && (!c->k_scale || !c->v_scale)) return PKV_ERR_NULL;
  const int64_t stride = c->block_stride ? c->block_stride : dense;
  // the kernels form block offsets as 32-bit block id x 32-bit block bytes
  if (stride > (int64_t)INT32_MAX / elem_bytes(c->dtype)) return PKV_ERR_SHAPE;
  if ((stride * elem_bytes(c->dtype)) % 16 != 0) return PKV_ERR_ALIGN;
  return PKV_OK;
}

// Product of two non-negative sizes, saturating at INT64_MAX: the launch
// planners' estimates stay ordered for arguments too large to launch.
int64_t sat_mul(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

int64_t block_stride_elems(const pkv_kv_cache* c) {
  return c->block_stride ? c->block_stride
                         : (int64_t)c->block_size * c->num_kv_heads * c->head_size;
}

// Decode kernel choice.  The matrix-core kernel pays off once a kv head
// serves several query heads (a dense g x tokens contraction).  At head size
// 128 it is also the faster gather with one query head per kv head, where
// the contraction is a matrix-vector product: 64 sequences x 32 heads of up
// to 4096 tokens, bfloat16, ran in 334.7-335.2 us against 341.1-341.3 us on
// the VALU kernel (one host, three runs each).  At head size 256 the VALU
// kernel keeps groups below kMfmaMinGroup.  A call's options may force either
// variant (A/B measurements).
constexpr int kMfmaMinGroup = 4;
constexpr int32_t kPlanMinSeqs = 64;
constexpr int kMfmaTokensPerWg = 2048;
constexpr int64_t kMfmaTargetWgs = 2048;   // about four rounds of 512 workgroup slots
constexpr int64_t kWgFixedTokens = 128;    // a workgroup's fixed cost in streamed tokens

bool use_mfma_decode(const pkv_kv_cache* c, int group, const Choice& ch) {
  if (c->dtype == PKV_FP8_E4M3) return true;          // the only fp8 decode kernel
  if (!is16(c->dtype) || (c->head_size != 128 && c->head_size != 256)) return false;
  if (ch.decode_kernel == 1) return false;
  if (ch.decode_kernel == 2) return true;
  return group >= kMfmaMinGroup || c->head_size == 128;
}

// Prefill kernel choice: the matrix-core kernel for bfloat16, binary16 or
// e4m3 caches with head 128 (the only prefill kernel for e4m3); a call's
// options may force the generic row kernel for 16-bit caches (A/B
// measurements).
bool use_mfma_prefill(const pkv_kv_cache* c, const Choice& ch) {
  if (c->head_size != 128) return false;
  if (c->dtype == PKV_FP8_E4M3) return true;
  if (!is16(c->dtype)) return false;
  return ch.prefill_kernel != 1;
}

// Query heads handled together by one workgroup of the VALU kernel.
int heads_per_chunk(int group) {
  for (int gt : {8, 4, 2, 1})
    if (group % gt == 0) return gt;
  return 1;
}

// ----------------------------------------------------------------- launch helpers
pkv_status launch_valu_z_chunks(AttnArgs a, int dtype, int head_size, int block_size, int gt,
                                unsigned gx, unsigned gy, int64_t z_total, hipStream_t st) {
  for (int64_t z0 = 0; z0 < z_total; z0 += kMaxGridZ) {
    a.z_base = (int32_t)z0;
    const unsigned gz = (unsigned)std::min<int64_t>(kMaxGridZ, z_total - z0);
    if (pkv::launch_attn_valu(a, dtype, head_size, block_size, gt, dim3(gx, gz, gy), st) !=
        hipSuccess)
      return PKV_ERR_HIP;
  }
  return PKV_OK;
}

// Matrix-core decode launch geometry for gy partitions: sets head chunks,
// partitions per workgroup and the range order in `a`; returns (gx, ranges).
int32_t device_cus();
std::pair<unsigned, unsigned> mfma_decode_geometry(AttnArgs& a, const pkv_kv_cache* cache,
                                                   unsigned gy, bool two_heads_ok = false) {
  const int group = a.num_heads / cache->num_kv_heads;
  {
    a.head_chunks = (group + 15) / 16;
    // e4m3 caches: a kv head's token row is 128 bytes, and whole 256-byte
    // rows gather faster (a microbenchmark of the two patterns: +7-9 %), so
    // each wave reads the rows of two adjacent kv heads when there is an
    // even number of them and a single head chunk.  Measured: MHA decode of
    // 64 sequences x 32 heads 200 -> 190 us; GQA decode of 256 sequences
    // (32 / 8 heads) unchanged (twice the LDS per workgroup: two workgroups
    // per CU instead of three).  Only for
    // the decode kernel's own launch (the one-launch forms keep one head),
    // and a call's options may keep one head per wave (A/B runs).
    a.heads_per_wave = (two_heads_ok && is_fp8(cache) && a.head_chunks == 1 &&
                        cache->num_kv_heads % 2 == 0) ? 2 : 1;
    // Tokens one workgroup streams.  The floor: the largest of 2048 .. 256
    // that still gives the launch about kMfmaTargetWgs workgroups (several
    // rounds of the workgroup slots; large batches keep 2048).  Above the
    // floor, the candidate with the least estimated makespan wins: rounds of
    // workgroup slots times (tokens per workgroup + a fixed cost of about
    // four tiles), with every row at its longest visible range (the host
    // does not read seq_lens).  It matters for small launches whose floor
    // leaves a short last round: sliding-window decode of 8 sequences gets
    // 320 workgroups of 1024 tokens instead of 576 of 512 (1.1 rounds of
    // 512 slots): 42 -> 29 us.  (Searching below the floor as well measured
    // slower on the large batches.)
    int64_t eff_len = a.window_left >= 0 ? std::min<int64_t>(a.max_seq_len, (int64_t)a.window_left + 1)
                                         : a.max_seq_len;
    eff_len = std::max<int64_t>(1, std::min<int64_t>(eff_len, a.max_seq_len - a.kv_start));
    const int64_t streams =
        sat_mul((int64_t)a.num_seqs * cache->num_kv_heads, a.head_chunks) / a.heads_per_wave;
    const int tpw_max = kMfmaTokensPerWg;
    int tpw = tpw_max;
    while (tpw > 256 && sat_mul(streams, eff_len) / tpw < kMfmaTargetWgs) tpw >>= 1;
    if (a.partition_size > 0) {
      const int P = a.partition_size;
      const int64_t span = eff_len + 31;             // the range starts at a multiple of 32
      const int64_t nparts = (span + P - 1) / P;
      const int dev_cus = device_cus();
      const int cus = dev_cus > 0 ? dev_cus : 256;
      const int64_t slots = (int64_t)cus * (is_fp8(cache) && a.heads_per_wave == 1 ? 3 : 2);
      int64_t best = -1;
      const int floor_tpw = tpw;
      for (int cand = tpw_max; cand >= floor_tpw; cand >>= 1) {
        const int ppw = (P <= cand / 4) ? 4 : std::max(1, cand / P);
        const int64_t wgs = sat_mul(streams, (nparts + ppw - 1) / ppw);
        const int64_t tok = std::min<int64_t>((int64_t)ppw * P, span);
        const int64_t est = sat_mul(wgs / slots + (wgs % slots != 0), tok + kWgFixedTokens);
        if (best < 0 || est < best) {
          best = est;
          tpw = cand;
        }
      }
    }
    // a workgroup streams about kMfmaTokensPerWg tokens: consecutive
    // partitions share its queries and block-table row, and its fixed cost
    // (queries, first loads, merge) is paid once per stream
    // Small partitions: a workgroup covers 4 of them, one per wave (merged in
    // LDS, then across workgroups by the split merge); larger ones: the waves
    // share the workgroup's partitions tile by tile.
    a.wave_per_part = (a.partition_size > 0 && a.partition_size <= tpw / 4) ? 1 : 0;
    a.parts_per_wg = a.partition_size <= 0 ? 1
                     : a.wave_per_part ? 4
                     : std::max(1, tpw / a.partition_size);
    // With the sequences ordered longest first, the last key ranges (which
    // only long sequences have) are dispatched first and the first ranges of
    // the shortest sequences last: close to longest-processing-time first.
    // (Without the order, ranges last first measured slower.)
    a.range_desc = a.seq_order ? 1 : 0;
    const unsigned gx = (unsigned)(cache->num_kv_heads * a.head_chunks / a.heads_per_wave);
    const unsigned gparts = (gy + a.parts_per_wg - 1) / a.parts_per_wg;
    return {gx, gparts};
  }
}

// One-row attention (decode, or the one-row sequences of a varlen batch):
// picks the kernel, the head chunking and the partitions per workgroup (left
// in `a` for the split merge that follows), launches over all z.
pkv_status launch_one_row(AttnArgs& a, const pkv_kv_cache* cache, unsigned gy, int64_t z_total,
                          hipStream_t st, Choice& ch) {
  const int group = a.num_heads / cache->num_kv_heads;
  if (use_mfma_decode(cache, group, ch)) {
    const auto [gx, gparts] = mfma_decode_geometry(a, cache, gy, ch.fp8_pairs == 0);
    ch.ran |= PKV_RAN_DECODE_MFMA | (a.heads_per_wave == 2 ? PKV_RAN_DECODE_PAIRS : 0u);
    for (int64_t z0 = 0; z0 < z_total; z0 += kMaxGridZ) {
      a.z_base = (int32_t)z0;
      const unsigned gz = (unsigned)std::min<int64_t>(kMaxGridZ, z_total - z0);
      if (pkv::launch_attn_mfma_decode(a, cache->block_size, cache->head_size, cache->dtype,
                                       dim3(gx, gz, gparts), st) != hipSuccess)
        return PKV_ERR_HIP;
    }
    a.z_base = 0;
    return PKV_OK;
  }
  const int gt = heads_per_chunk(group);
  a.head_chunks = group / gt;
  ch.ran |= PKV_RAN_DECODE_VALU;
  return launch_valu_z_chunks(a, cache->dtype, cache->head_size, cache->block_size, gt,
                              (unsigned)(cache->num_kv_heads * a.head_chunks), gy, z_total, st);
}

pkv_status launch_reduce(const AttnArgs& a, int dtype, int head_size, hipStream_t st,
                         Choice& ch) {
  // with a single workgroup range per row (every partition of a row in one
  // workgroup) the attention kernel wrote every row itself
  const int max_ranges = a.partition_size > 0 ? (a.num_splits + a.parts_per_wg - 1) / a.parts_per_wg : 1;
  if (max_ranges <= 1) return PKV_OK;
  ch.ran |= PKV_RAN_SPLIT_MERGE;
  if (pkv::launch_splitkv_reduce(a, dtype, head_size, st) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

// Workspace sizes are products of int32 arguments that can pass 2^64 for
// sizes no launch could take; they are formed in 128 bits and such sizes
// reported as (size_t)-1 rather than wrapped to a small number.
using u128 = unsigned __int128;
constexpr u128 kMaxWorkspace = (u128)1 << 62;

// Split workspace: partial outputs [rows, head_size] fp32, their lse [rows]
// fp32, then the sequence dispatch order int32 [num_seqs] (16-byte aligned).
size_t order_offset(size_t rows, int32_t head_size) {
  return align16(rows * head_size * sizeof(float) + rows * sizeof(float));
}

// Workspace tail: the sequence order [num_seqs], then the list of multi-row
// sequences [num_seqs] and its length [1].
int32_t* order_area(const AttnArgs& a, const pkv_kv_cache* cache, void* workspace) {
  const size_t rows = (size_t)a.num_splits * a.num_heads * a.num_seqs;
  return reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                    order_offset(rows, cache->head_size));
}

// One-row decode launches with a split workspace and at least
// kPlanMinSeqs sequences order their sequences longest first (the planner
// writes the order into the workspace).  With
// `multi`, the planner also lists the multi-row sequences (mixed launch).
pkv_status plan_seq_order(AttnArgs& a, const pkv_kv_cache* cache, void* workspace,
                          hipStream_t st, Choice& ch, bool multi = false) {
  if (a.num_splits <= 1 || !use_mfma_decode(cache, a.num_heads / cache->num_kv_heads, ch))
    return PKV_OK;
  // with few sequences the planner's launch costs more than the order saves
  // (8 sequences of 32k-131k tokens: the same step time; with a 4096-key
  // window: 47 -> 42 us)
  if (!multi && a.num_seqs < kPlanMinSeqs) return PKV_OK;
  int32_t* order = order_area(a, cache, workspace);
  ch.ran |= PKV_RAN_PLANNER;
  if (pkv::launch_seq_order(a.seq_lens, a.num_seqs, a.max_seq_len, order,
                            multi ? a.cu_seqlens_q : nullptr, a.num_tokens,
                            multi ? order + a.num_seqs : nullptr,
                            multi ? order + 2 * a.num_seqs : nullptr,
                            multi ? order + 2 * a.num_seqs + 1 : nullptr, st) != hipSuccess)
    return PKV_ERR_HIP;
  a.seq_order = order;
  return PKV_OK;
}

// Compute units of the current device, 0 if they cannot be read.  Asked of
// the runtime on each use (it answers from its own device properties).
int32_t device_cus() {
  int dev = 0, attr = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&attr, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return attr;
}

// CU classes in four (of every XCD) that start the mixed launch on prefill
// tiles: 2 over a 16-bit cache, 3 over an fp8 one (of 1-4 tried).  Over an
// fp8 cache the prefill tiles also convert their codes and the decode rows
// move half the bytes, so more of the chip starts on prefill (4 chunks of
// 512 rows beside 128 decode rows: 2 in four was 10-20 % slower there).
constexpr int32_t kMixedShare = 2;
constexpr int32_t kMixedShareFp8 = 3;

// Mixed batches (prefill chunks and decode rows) run as one interleaved
// launch when both kinds use the matrix-core kernels and a split workspace
// holds the planner's lists; a call's options may keep two launches (A/B).
bool use_mixed_launch(const AttnArgs& a, const pkv_kv_cache* cache, const Choice& ch) {
  if (ch.mixed == 1) return false;
  return a.num_splits > 1 && use_mfma_prefill(cache, ch) &&
         use_mfma_decode(cache, a.num_heads / cache->num_kv_heads, ch);
}

int32_t num_splits_for(int32_t max_seq_len, int32_t P) {
  if (P <= 0) return 1;
  return std::max<int32_t>(1, (int32_t)(((int64_t)max_seq_len + P - 1) / P));
}

AttnArgs base_args(void* out, const void* q, const pkv_kv_cache* cache,
                   const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                   int32_t num_seqs, int32_t num_tokens, int32_t num_heads, int32_t max_seq_len,
                   int32_t max_query_len, float scale, int32_t P, int32_t nsplits, float* lse_out,
                   void* workspace) {
  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = nullptr;
  a.lse_out = lse_out;
  a.ws_o = nullptr;
  a.ws_lse = nullptr;
  a.seq_order = nullptr;
  if (nsplits > 1) {
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = a.ws_o + (int64_t)nsplits * num_heads * num_seqs * cache->head_size;
  }
  a.block_stride = block_stride_elems(cache);
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks;
  a.block_size = cache->block_size;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.max_seq_len = max_seq_len;
  a.max_query_len = max_query_len;
  a.partition_size = nsplits > 1 ? P : 0;
  a.num_splits = nsplits;
  a.head_chunks = 1;
  a.parts_per_wg = 1;
  a.wave_per_part = 0;
  a.head_chunks_gc = 1;
  a.z_base = 0;
  a.mode = pkv::kModeDecode;
  a.causal = 0;
  a.skip_multi_row = 0;
  a.window_left = -1;
  a.kv_start = 0;
  a.prefix_len = 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  return a;
}

// ----------------------------------------------------------------- cascade
// Prefix pass geometry: the query tiles and head groups of the prefill
// kernel over all rows of the batch, and enough key partitions (of at least
// kPrefixMinPart tokens, at most kMaxPrefixParts) to give about target_wgs
// workgroups.  Depends only on the call's sizes, so the workspace size is
// known without a device; the workspace holds the partitions of the default
// target, which the one-launch form's smaller target never exceeds.
constexpr int32_t kMaxPrefixParts = 16;
constexpr int32_t kPrefixMinPart = 256;
// Target workgroups of the prefix pass: a launch of its own fills the chip;
// beside the decode rows of the one-launch form fewer, longer items do
// better (they share the chip with the decode rows, and fewer partitions
// mean fewer fp32 partials to write and merge).  Measured on the 256-request
// shared-prefix decode batch: 512 alone, 128 in the one-launch form.
constexpr int64_t kPrefixTargetWgs = 512;
constexpr int64_t kPrefixTargetWgsFused = 128;

// A cascade whose rows are all decode rows runs the prefix pass and the
// suffix pass as one persistent launch when the decode rows use the
// matrix-core kernel; a call's options may keep separate launches (A/B).
bool use_cascade_launch(const pkv_kv_cache* cache, int group, const Choice& ch) {
  if (ch.cascade == 1) return false;
  return use_mfma_prefill(cache, ch) && use_mfma_decode(cache, group, ch) && device_cus() > 0;
}

// XCDs in four (by workgroup index) that start the one-launch cascade on
// prefix items (of 1 and 2 tried, 1 was faster).
constexpr int32_t kCascadeShare = 1;

struct PrefixGeometry {
  int32_t gc = 1;        // query heads per column group
  unsigned qtiles = 0;   // query tiles over all rows
  unsigned gy = 0;       // head groups
  int32_t parts = 0;     // key partitions of the prefix
  int32_t P = 0;         // tokens per partition (multiple of 32)
};

PrefixGeometry prefix_geometry(int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                               int32_t cpl, int64_t target_wgs = kPrefixTargetWgs) {
  PrefixGeometry g;
  if (cpl <= 0 || num_tokens <= 0) return g;
  const int group = num_heads / num_kv_heads;
  int gc = 8;
  while (group % gc) gc >>= 1;
  g.gc = gc;
  const int rows_per_wg = 16 * (8 / gc);
  g.qtiles = (unsigned)(((int64_t)num_tokens + rows_per_wg - 1) / rows_per_wg);
  g.gy = (unsigned)(num_kv_heads * (group / gc));
  const int64_t base = (int64_t)g.qtiles * g.gy;
  const int64_t most =
      std::min<int64_t>(kMaxPrefixParts, ((int64_t)cpl + kPrefixMinPart - 1) / kPrefixMinPart);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(most, (target_wgs + base - 1) / base));
  g.P = (int32_t)((((cpl + want - 1) / want) + 31) / 32 * 32);
  g.parts = (int32_t)(((int64_t)cpl + g.P - 1) / g.P);
  return g;
}

// Cascade workspace: prefix partial outputs [parts, heads, rows, D] fp32 and
// their lse [parts, heads, rows], the suffix pass's lse [rows, heads], then
// the suffix pass's own split workspace.
struct CascadeLayout {
  size_t pre_o = 0, pre_lse = 0, suf_lse = 0, plan = 0, varlen = 0, total = 0;
};

// ... then the plan of the one-launch form (sequence order [num_seqs] and two
// work-queue counters), then the suffix pass's split workspace.
CascadeLayout cascade_layout(const PrefixGeometry& g, int32_t num_seqs, int32_t num_tokens,
                             int32_t num_heads, int32_t head_size, size_t varlen_bytes) {
  CascadeLayout l;
  const size_t rows = (size_t)g.parts * num_heads * num_tokens;
  l.pre_o = 0;
  l.pre_lse = rows * head_size * sizeof(float);
  l.suf_lse = align16(l.pre_lse + rows * sizeof(float));
  l.plan = align16(l.suf_lse + (size_t)num_tokens * num_heads * sizeof(float));
  l.varlen = align16(l.plan + ((size_t)num_seqs + 2) * sizeof(int32_t));
  l.total = l.varlen + varlen_bytes;
  return l;
}

// The varlen call; keys before kv_start are left out for every row (the
// suffix pass of a cascade, arguments already checked; 0 otherwise).  The
// split partitions and the workspace cover the span max_seq_len - (kv_start
// rounded down to 32) that a row's partitions can reach.
pkv_status varlen_impl(void* out, const void* q, const pkv_kv_cache* cache,
                       const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                       int32_t num_tokens, int32_t num_heads, int32_t max_query_len,
                       int32_t max_seq_len, float scale, int32_t causal, int32_t window_left,
                       int32_t partition_size, float* lse_out, void* workspace,
                       size_t workspace_bytes, void* stream, int32_t kv_start, Choice& ch) {
  pkv_status st = check_cache(cache, num_heads);
  if (st != PKV_OK) return st;
  if (window_left < -1) return PKV_ERR_SHAPE;
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || max_seq_len < 0 ||
      max_seq_len > kMaxSeqLen || max_query_len < 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_SHAPE;
  if (reason(cache->dtype, cache->head_size, cache->block_size, num_heads, cache->num_kv_heads))
    return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  // the prefill kernels take row maxima of the unscaled logits
  if (max_query_len > 1 && !(scale > 0.f)) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !block_tables || !seq_lens || !cu_seqlens_q) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q)) return PKV_ERR_ALIGN;
  const int32_t span = max_seq_len - (kv_start & ~31);
  const int32_t P = pkv_choose_partition_size(num_seqs, num_heads, cache->num_kv_heads, span,
                                              partition_size);
  if (P < 0) return PKV_ERR_SHAPE;
  const int32_t ns = num_splits_for(span, P);
  if (ns > kMaxGridY) return PKV_ERR_UNSUPPORTED;
  if (ns > 1) {
    const size_t need = pkv_attention_workspace_bytes(num_seqs, num_heads, cache->num_kv_heads,
                                                      cache->head_size, span, P);
    if (need == (size_t)-1) return PKV_ERR_SHAPE;
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnArgs a = base_args(out, q, cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                         num_tokens, num_heads, max_seq_len, std::max(max_query_len, 1), scale, P,
                         ns, lse_out, workspace);
  a.cu_seqlens_q = cu_seqlens_q;
  a.window_left = clamp_window(window_left, max_seq_len);
  a.causal = causal ? 1 : 0;
  a.kv_start = kv_start;
  const int group = num_heads / cache->num_kv_heads;
  const int gt = heads_per_chunk(group);
  a.head_chunks = group / gt;
  const unsigned gx = (unsigned)(cache->num_kv_heads * a.head_chunks);

  // Prefill chunks and decode rows of one batch: a single interleaved launch.
  if (max_query_len > 1 && use_mixed_launch(a, cache, ch)) {
    AttnArgs r = a;
    r.mode = pkv::kModeVarlenRows;
    r.partition_size = 0;
    r.ws_o = nullptr;
    r.ws_lse = nullptr;
    int gc = 8;
    while (group % gc) gc >>= 1;
    r.head_chunks_gc = gc;
    const int rows_per_wg = 16 * (8 / gc);
    AttnArgs d = a;
    d.mode = pkv::kModeVarlenOne;
    d.seq_order = order_area(d, cache, workspace);   // written by the planner below
    const auto [gx_d, gparts] = mfma_decode_geometry(d, cache, (unsigned)ns, false);
    pkv::MixedGrid g{};
    g.pre_x = (max_query_len + rows_per_wg - 1) / rows_per_wg;
    g.pre_y = cache->num_kv_heads * (group / gc);
    g.pre_z = 1;
    g.pre_share = is_fp8(cache) ? kMixedShareFp8 : kMixedShare;
    g.dec_x = (int32_t)gx_d;
    g.dec_y = num_seqs;
    g.dec_z = (int32_t)gparts;
    g.n_dec = (int64_t)g.dec_x * g.dec_y * g.dec_z;
    g.pre_list = d.seq_order + num_seqs;
    g.pre_count = d.seq_order + 2 * num_seqs;
    g.queues = order_area(d, cache, workspace) + 2 * num_seqs + 1;
    g.workgroups = 2 * device_cus();                // two per CU (LDS and registers allow two)
    const int64_t n_pre_max = (int64_t)g.pre_x * g.pre_y * num_seqs;
    if (g.workgroups > 0 && n_pre_max < (int64_t)INT32_MAX && g.n_dec < (int64_t)INT32_MAX) {
      st = plan_seq_order(d, cache, workspace, s, ch, /*multi=*/true);
      if (st != PKV_OK) return st;
      int tslot = 0;
      const bool timed = timing_begin(s, &tslot);
      ch.ran |= PKV_RAN_MIXED;
      if (pkv::launch_attn_mixed(r, d, g, cache->block_size, cache->dtype, s) != hipSuccess)
        st = PKV_ERR_HIP;
      if (timed) timing_end(s, tslot);
      if (st != PKV_OK) return st;
      return launch_reduce(d, io_dtype(cache->dtype), cache->head_size, s, ch);
    }
  }
  // Rows of sequences with several query rows (chunked prefill).
  if (max_query_len > 1) {
    AttnArgs r = a;
    r.mode = pkv::kModeVarlenRows;
    r.partition_size = 0;
    r.ws_o = nullptr;
    r.ws_lse = nullptr;
    int tslot = 0;
    const bool timed = timing_begin(s, &tslot);
    if (use_mfma_prefill(cache, ch)) {
      ch.ran |= PKV_RAN_PREFILL_MFMA;
      int gc = 8;
      while (group % gc) gc >>= 1;
      r.head_chunks_gc = gc;
      const int rows_per_wg = 16 * (8 / gc);
      const unsigned qtiles = (unsigned)(((int64_t)max_query_len + rows_per_wg - 1) / rows_per_wg);
      const unsigned gy = (unsigned)(cache->num_kv_heads * (group / gc));
      for (int64_t z0 = 0; z0 < num_seqs && st == PKV_OK; z0 += kMaxGridZ) {
        r.z_base = (int32_t)z0;
        const unsigned gz = (unsigned)std::min<int64_t>(kMaxGridZ, num_seqs - z0);
        if (pkv::launch_attn_mfma_prefill(r, cache->block_size, cache->dtype, dim3(qtiles, gy, gz),
                                          s) != hipSuccess)
          st = PKV_ERR_HIP;
      }
    } else {
      ch.ran |= PKV_RAN_PREFILL_VALU;
      st = launch_valu_z_chunks(r, cache->dtype, cache->head_size, cache->block_size, gt, gx, 1,
                                num_tokens, s);
    }
    if (timed) timing_end(s, tslot);
    if (st != PKV_OK) return st;
  }
  // Sequences with one query row (decode rows), split over the key range;
  // the main launch when the batch has no longer query ranges.
  a.mode = pkv::kModeVarlenOne;
  st = plan_seq_order(a, cache, workspace, s, ch);
  if (st != PKV_OK) return st;
  int tslot = 0;
  const bool timed = max_query_len <= 1 && timing_begin(s, &tslot);
  st = launch_one_row(a, cache, (unsigned)ns, num_seqs, s, ch);
  if (timed) timing_end(s, tslot);
  if (st != PKV_OK) return st;
  if (ns > 1) st = launch_reduce(a, io_dtype(cache->dtype), cache->head_size, s, ch);
  return st;
}

}  // namespace

namespace pkv {

pkv_status decode_host_checks(const void* out, const void* q, const pkv_kv_cache* cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t max_seq_len, float scale, int32_t window_left,
                              int32_t partition_size, const pkv_call_options* options) {
  Choice ch;
  pkv_status st = read_options(options, &ch);
  if (st != PKV_OK) return st;
  st = check_cache(cache, num_heads);
  if (st != PKV_OK) return st;
  if (window_left < -1) return PKV_ERR_SHAPE;
  if (num_seqs < 0 || num_heads <= 0 || max_seq_len < 0 || max_seq_len > kMaxSeqLen ||
      max_blocks_per_seq <= 0)
    return PKV_ERR_SHAPE;
  if (reason(cache->dtype, cache->head_size, cache->block_size, num_heads, cache->num_kv_heads))
    return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !block_tables || !seq_lens) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q)) return PKV_ERR_ALIGN;
  const int32_t P = pkv_choose_partition_size(num_seqs, num_heads, cache->num_kv_heads,
                                              max_seq_len, partition_size);
  if (P < 0) return PKV_ERR_SHAPE;
  if (num_splits_for(max_seq_len, P) > kMaxGridY) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

const char* pkv_unsupported_reason(int32_t dtype, int32_t head_size, int32_t block_size,
                                   int32_t num_heads, int32_t num_kv_heads) {
  return reason(dtype, head_size, block_size, num_heads, num_kv_heads);
}

const char* pkv_status_string(int32_t s) {
  // an int, not the enum: C callers may pass any code, and C++ gives a value
  // outside the enum's range no defined meaning
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid size or shape argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported dtype/head_size/block_size/head combination";
    case PKV_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_METADATA: return "invalid metadata";
    case PKV_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t pkv_choose_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t max_seq_len, int32_t partition_size) {
  (void)num_seqs;
  (void)num_heads;
  (void)num_kv_heads;
  if (max_seq_len < 0) return -1;
  if (partition_size == -1) return 0;
  if (partition_size < -1) return -1;
  if (partition_size > 0) {
    if (partition_size % kPartitionQuantum != 0) return -1;
    return partition_size;
  }
  return max_seq_len > kDefaultPartition ? kDefaultPartition : 0;
}

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t max_seq_len,
                                     int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || max_seq_len < 0)
    return (size_t)-1;
  const int32_t P =
      pkv_choose_partition_size(num_seqs, num_heads, num_kv_heads, max_seq_len, partition_size);
  if (P < 0) return (size_t)-1;
  const int32_t ns = num_splits_for(max_seq_len, P);
  if (ns <= 1) return 0;
  const u128 rows = (u128)ns * (u128)num_heads * (u128)num_seqs;
  if (rows * ((u128)head_size + 1) * sizeof(float) + 4 * (u128)num_seqs > kMaxWorkspace)
    return (size_t)-1;
  return order_offset((size_t)rows, head_size) +
         align16((2 * (size_t)num_seqs + 3) * sizeof(int32_t));
}

pkv_status pkv_kv_cache_write(const pkv_kv_cache* cache, const void* key, const void* value,
                              const int64_t* slot_mapping, int64_t num_tokens, void* stream) {
  pkv_status st = check_cache(cache, cache ? cache->num_kv_heads : 0);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(key) || !aligned16(value)) return PKV_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0) return PKV_ERR_ALIGN;
  pkv::KvWriteArgs a{};
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.key = key;
  a.value = value;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_slots = cache->num_blocks * cache->block_size;
  a.block_stride_bytes = block_stride_elems(cache) * elem_bytes(cache->dtype);
  a.head_size = cache->head_size;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_size = cache->block_size;
  a.row_bytes = cache->num_kv_heads * cache->head_size * elem_bytes(cache->dtype);
  if (num_tokens > (int64_t)INT32_MAX * 4) return PKV_ERR_SHAPE;
  return pkv::launch_kv_write(a, is_fp8(cache), static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
                                                                                 : PKV_ERR_HIP;
}

pkv_status pkv_paged_attention_decode(void* out, const void* q, const pkv_kv_cache* cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                      int32_t max_seq_len, float scale, int32_t window_left,
                                      int32_t partition_size, float* lse_out, void* workspace,
                                      size_t workspace_bytes, pkv_call_options* options,
                                      void* stream) {
  Choice ch;
  const Report report{options, ch};
  pkv_status st = pkv::decode_host_checks(out, q, cache, block_tables, max_blocks_per_seq,
                                          seq_lens, num_seqs, num_heads, max_seq_len, scale,
                                          window_left, partition_size, options);
  if (st != PKV_OK) return st;
  st = read_options(options, &ch);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  const int32_t P = pkv_choose_partition_size(num_seqs, num_heads, cache->num_kv_heads,
                                              max_seq_len, partition_size);
  const int32_t ns = num_splits_for(max_seq_len, P);
  if (ns > 1) {
    const size_t need = pkv_attention_workspace_bytes(num_seqs, num_heads, cache->num_kv_heads,
                                                      cache->head_size, max_seq_len, P);
    if (need == (size_t)-1) return PKV_ERR_SHAPE;
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnArgs a = base_args(out, q, cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                         num_seqs, num_heads, max_seq_len, 1, scale, P, ns, lse_out, workspace);
  a.mode = pkv::kModeDecode;
  a.window_left = clamp_window(window_left, max_seq_len);
  st = plan_seq_order(a, cache, workspace, s, ch);
  if (st != PKV_OK) return st;
  int tslot = 0;
  const bool timed = timing_begin(s, &tslot);
  st = launch_one_row(a, cache, (unsigned)ns, num_seqs, s, ch);
  if (timed) timing_end(s, tslot);
  if (st != PKV_OK) return st;
  if (ns > 1) st = launch_reduce(a, io_dtype(cache->dtype), cache->head_size, s, ch);
  return st;
}

pkv_status pkv_paged_attention_varlen(void* out, const void* q, const pkv_kv_cache* cache,
                                      const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                      int32_t max_query_len, int32_t max_seq_len, float scale,
                                      int32_t causal, int32_t window_left, int32_t partition_size,
                                      float* lse_out, void* workspace, size_t workspace_bytes,
                                      pkv_call_options* options, void* stream) {
  Choice ch;
  const Report report{options, ch};
  const pkv_status st = read_options(options, &ch);
  if (st != PKV_OK) return st;
  return varlen_impl(out, q, cache, cu_seqlens_q, seq_lens, block_tables, max_blocks_per_seq,
                     num_seqs, num_tokens, num_heads, max_query_len, max_seq_len, scale, causal,
                     window_left, partition_size, lse_out, workspace, workspace_bytes, stream, 0,
                     ch);
}

size_t pkv_cascade_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_size, int32_t max_seq_len,
                                   int32_t common_prefix_len, int32_t partition_size) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      max_seq_len < 0 || common_prefix_len < 0 || common_prefix_len > max_seq_len ||
      num_heads % num_kv_heads != 0)
    return (size_t)-1;
  const int32_t span = max_seq_len - (common_prefix_len & ~31);
  const size_t vw = pkv_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size,
                                                  span, partition_size);
  if (vw == (size_t)-1) return vw;
  if (common_prefix_len == 0) return vw;
  const PrefixGeometry g = prefix_geometry(num_tokens, num_heads, num_kv_heads, common_prefix_len);
  // prefix partials, their lse, the suffix lse and the plan, bounded first
  const u128 rows = (u128)g.parts * (u128)num_heads * (u128)num_tokens;
  if (rows * ((u128)head_size + 2) * sizeof(float) + 4 * (u128)num_seqs + vw > kMaxWorkspace)
    return (size_t)-1;
  return cascade_layout(g, num_seqs, num_tokens, num_heads, head_size, vw).total;
}

const char* pkv_cascade_reason(int32_t common_prefix_len, int32_t num_seqs, int32_t num_tokens,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                               int32_t dtype, int32_t window_left) {
  if ((!is16(dtype) && dtype != PKV_FP8_E4M3) || head_size != 128)
    return "the prefix pass would run on the VALU kernel (float32 caches or head_size other "
           "than 128), one query row per workgroup: the plain call is as fast or faster";
  if (num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads != 0)
    return "num_heads must be a positive multiple of num_kv_heads";
  if (window_left >= 0) return "sliding-window attention does not use the cascade";
  if (common_prefix_len < 256) return "common prefix shorter than 256 tokens";
  if (num_seqs < 8) return "fewer than 8 requests";
  if (num_tokens <= 0) return "no query rows";
  // Rough cost model of the prefix's share of the work.  The plain form
  // streams the prefix once per request and does the rows' prefix flops in
  // the shadow of that stream (or on the matrix cores for prefill rows):
  // max(requests x prefix bytes / HBM, flops / MFMA).  The cascade streams it
  // once, does the same flops on the matrix cores, and writes and reads the
  // fp32 partials: max(prefix bytes / HBM, flops / MFMA) + partials / HBM.
  const double kv_bytes = 2.0 * common_prefix_len * num_kv_heads * head_size * elem_bytes(dtype);
  const PrefixGeometry g = prefix_geometry(num_tokens, num_heads, num_kv_heads, common_prefix_len);
  const double partial_bytes = 2.0 * g.parts * num_heads * (double)num_tokens * (head_size + 1) * 4;
  const double flops = 4.0 * num_tokens * num_heads * (double)head_size * common_prefix_len;
  const double hbm = 8.0e12 * 0.7, mfma = 2.5e15 * 0.3;   // sustained rates assumed
  const double t_plain = std::max(num_seqs * kv_bytes / hbm, flops / mfma);
  const double t_cascade = std::max(kv_bytes / hbm, flops / mfma) + partial_bytes / hbm;
  if (t_cascade >= t_plain)
    return "the prefix pass would cost more than re-reading the prefix per request";
  return nullptr;
}

pkv_status pkv_cascade_attention(void* out, const void* q, const pkv_kv_cache* cache,
                                 const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* prefix_blocks, int32_t num_seqs,
                                 int32_t num_tokens, int32_t num_heads, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t common_prefix_len, float scale,
                                 int32_t causal, int32_t partition_size, float* lse_out,
                                 void* workspace, size_t workspace_bytes,
                                 pkv_call_options* options, void* stream) {
  Choice ch;
  const Report report{options, ch};
  pkv_status st = read_options(options, &ch);
  if (st != PKV_OK) return st;
  st = check_cache(cache, num_heads);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || max_seq_len < 0 ||
      max_seq_len > kMaxSeqLen || max_query_len < 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_SHAPE;
  if (reason(cache->dtype, cache->head_size, cache->block_size, num_heads, cache->num_kv_heads))
    return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  const int32_t cpl = common_prefix_len;
  if (cpl < 0 || cpl % cache->block_size != 0 || cpl > max_seq_len ||
      (int64_t)cpl > (int64_t)max_blocks_per_seq * cache->block_size)
    return PKV_ERR_SHAPE;
  if (cpl == 0)
    return varlen_impl(out, q, cache, cu_seqlens_q, seq_lens, block_tables, max_blocks_per_seq,
                       num_seqs, num_tokens, num_heads, max_query_len, max_seq_len, scale, causal,
                       -1, partition_size, lse_out, workspace, workspace_bytes, stream, 0, ch);
  // the prefix pass is the prefill kernel: row maxima of the unscaled logits
  if (!(scale > 0.f)) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !block_tables || !seq_lens || !cu_seqlens_q || !prefix_blocks)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q)) return PKV_ERR_ALIGN;
  const int32_t span = max_seq_len - (cpl & ~31);
  const size_t vw = pkv_attention_workspace_bytes(num_seqs, num_heads, cache->num_kv_heads,
                                                  cache->head_size, span, partition_size);
  if (vw == (size_t)-1) return PKV_ERR_SHAPE;
  const PrefixGeometry g = prefix_geometry(num_tokens, num_heads, cache->num_kv_heads, cpl);
  if (g.parts < 1 || g.parts > kMaxPrefixParts || g.qtiles > (unsigned)INT32_MAX) return PKV_ERR_SHAPE;
  if (pkv_cascade_workspace_bytes(num_seqs, num_tokens, num_heads, cache->num_kv_heads,
                                  cache->head_size, max_seq_len, cpl, partition_size) ==
      (size_t)-1)
    return PKV_ERR_SHAPE;
  const CascadeLayout lay = cascade_layout(g, num_seqs, num_tokens, num_heads, cache->head_size, vw);
  if (!workspace || workspace_bytes < lay.total) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // 1. prefix pass: every row against the shared prefix, fp32 partials
  AttnArgs p = base_args(out, q, cache, prefix_blocks, cpl / cache->block_size, seq_lens, num_seqs,
                         num_tokens, num_heads, max_seq_len, std::max(max_query_len, 1), scale, 0,
                         1, nullptr, nullptr);
  p.mode = pkv::kModePrefix;
  p.prefix_len = cpl;
  p.partition_size = g.P;
  p.num_splits = g.parts;
  p.head_chunks_gc = g.gc;
  p.ws_o = reinterpret_cast<float*>(ws + lay.pre_o);
  p.ws_lse = reinterpret_cast<float*>(ws + lay.pre_lse);
  float* lse_suffix = reinterpret_cast<float*>(ws + lay.suf_lse);
  const int group = num_heads / cache->num_kv_heads;
  if (max_query_len <= 1 && use_cascade_launch(cache, group, ch)) {
    // 1 + 2 in one persistent launch: prefix items on the matrix cores beside
    // the decode rows of the suffix pass
    const PrefixGeometry gf = prefix_geometry(num_tokens, num_heads, cache->num_kv_heads, cpl,
                                              kPrefixTargetWgsFused);
    p.partition_size = gf.P;
    p.num_splits = gf.parts;
    const int32_t P = pkv_choose_partition_size(num_seqs, num_heads, cache->num_kv_heads, span,
                                                partition_size);
    const int32_t ns = num_splits_for(span, P);
    if (P < 0) return PKV_ERR_SHAPE;
    if (ns > kMaxGridY) return PKV_ERR_UNSUPPORTED;
    AttnArgs d = base_args(out, q, cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                           num_tokens, num_heads, max_seq_len, 1, scale, P, ns, lse_suffix,
                           vw ? ws + lay.varlen : nullptr);
    d.cu_seqlens_q = cu_seqlens_q;
    d.mode = pkv::kModeVarlenOne;
    d.causal = causal ? 1 : 0;
    d.kv_start = cpl;
    int32_t* plan = reinterpret_cast<int32_t*>(ws + lay.plan);
    d.seq_order = plan;
    const auto [gx_d, gparts] = mfma_decode_geometry(d, cache, (unsigned)ns, false);
    pkv::MixedGrid mg{};
    mg.pre_x = (int32_t)gf.qtiles;
    mg.pre_y = (int32_t)gf.gy;
    mg.pre_z = gf.parts;
    mg.pre_share = kCascadeShare;
    mg.dec_x = (int32_t)gx_d;
    mg.dec_y = num_seqs;
    mg.dec_z = (int32_t)gparts;
    mg.n_dec = (int64_t)mg.dec_x * mg.dec_y * mg.dec_z;
    mg.queues = plan + num_seqs;
    mg.workgroups = 2 * device_cus();
    if (mg.workgroups <= 0 || mg.n_dec >= (int64_t)INT32_MAX) return PKV_ERR_HIP;
    ch.ran |= PKV_RAN_PLANNER;
    if (pkv::launch_seq_order(seq_lens, num_seqs, max_seq_len, plan, nullptr, num_tokens, nullptr,
                              nullptr, mg.queues, s) != hipSuccess)
      return PKV_ERR_HIP;
    int tslot = 0;
    const bool timed = timing_begin(s, &tslot);
    ch.ran |= PKV_RAN_CASCADE_ONE;
    if (pkv::launch_attn_cascade(p, d, mg, cache->block_size, cache->dtype, s) != hipSuccess)
      st = PKV_ERR_HIP;
    if (timed) timing_end(s, tslot);
    if (st != PKV_OK) return st;
    if (ns > 1) st = launch_reduce(d, io_dtype(cache->dtype), cache->head_size, s, ch);
    if (st != PKV_OK) return st;
  } else {
    ch.ran |= PKV_RAN_PREFIX;
    if (use_mfma_prefill(cache, ch)) {
      if (pkv::launch_attn_mfma_prefix(p, cache->block_size, cache->dtype,
                                       dim3(g.qtiles, g.gy, (unsigned)g.parts), s) != hipSuccess)
        return PKV_ERR_HIP;
    } else {
      // other dtypes and head sizes: the VALU kernel, one workgroup per
      // (kv-head chunk, query row, prefix partition); its partials are
      // indexed by row, so the launch takes num_seqs = rows
      AttnArgs pv = p;
      pv.num_seqs = num_tokens;
      const int gt = heads_per_chunk(group);
      pv.head_chunks = group / gt;
      st = launch_valu_z_chunks(pv, cache->dtype, cache->head_size, cache->block_size, gt,
                                (unsigned)(cache->num_kv_heads * pv.head_chunks),
                                (unsigned)g.parts, num_tokens, s);
      if (st != PKV_OK) return st;
    }
    // 2. suffix pass: each row against its own keys (from the prefix end on)
    st = varlen_impl(out, q, cache, cu_seqlens_q, seq_lens, block_tables, max_blocks_per_seq,
                     num_seqs, num_tokens, num_heads, max_query_len, max_seq_len, scale, causal,
                     -1, partition_size, lse_suffix, vw ? ws + lay.varlen : nullptr, vw, stream,
                     cpl, ch);
    if (st != PKV_OK) return st;
  }
  // 3. merge of the two results, in place in out
  AttnArgs m = p;
  m.cu_seqlens_q = cu_seqlens_q;
  m.lse_out = lse_out;
  ch.ran |= PKV_RAN_CASCADE_MERGE;
  if (pkv::launch_cascade_merge(m, lse_suffix, p.num_splits, io_dtype(cache->dtype),
                                cache->head_size, s) != hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

pkv_status pkv_validate_cascade(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t num_seqs,
                                const int32_t* cu_seqlens_q, const int32_t* prefix_blocks,
                                int32_t common_prefix_len, int32_t block_size, char* msg,
                                size_t msg_len) {
  auto fail = [&](const char* fmt, ...) {
    if (msg && msg_len) {
      va_list ap;
      va_start(ap, fmt);
      vsnprintf(msg, msg_len, fmt, ap);
      va_end(ap);
    }
    return PKV_ERR_METADATA;
  };
  if (msg && msg_len) msg[0] = '\0';
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0) return fail("bad sizes");
  const int32_t cpl = common_prefix_len;
  if (cpl < 0 || cpl % block_size) return fail("common_prefix_len %d is not a whole number of blocks", cpl);
  const int32_t nb = cpl / block_size;
  if (nb > max_blocks_per_seq) return fail("prefix of %d blocks exceeds max_blocks_per_seq", nb);
  if (num_seqs > 0 && (!block_tables || !seq_lens || !cu_seqlens_q))
    return fail("NULL block_tables, seq_lens or cu_seqlens_q");
  if (nb > 0 && !prefix_blocks) return fail("NULL prefix_blocks");
  std::unordered_set<int32_t> pre(prefix_blocks, prefix_blocks + nb);
  if ((int32_t)pre.size() != nb) return fail("a prefix block is listed twice");
  std::unordered_set<int32_t> own;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s];
    if (L == 0) continue;
    const int32_t ql = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    if (cpl > L - ql) return fail("sequence %d: prefix of %d tokens reaches its query rows", s, cpl);
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int32_t i = 0; i < nb; ++i)
      if (row[i] != prefix_blocks[i])
        return fail("sequence %d: block_tables[%d] = %d, prefix block %d", s, i, row[i], prefix_blocks[i]);
    const int32_t n = (int32_t)std::min<int64_t>(((int64_t)L + block_size - 1) / block_size, max_blocks_per_seq);
    for (int32_t i = nb; i < n; ++i) {
      if (pre.count(row[i])) return fail("sequence %d: own block %d is a prefix block", s, row[i]);
      if (!own.insert(row[i]).second) return fail("block %d owned twice (seq %d)", row[i], s);
    }
  }
  return PKV_OK;
}

pkv_status pkv_validate_metadata(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t num_seqs,
                                 const int32_t* cu_seqlens_q, int32_t num_tokens,
                                 int32_t max_query_len, int32_t max_seq_len,
                                 const int64_t* slot_mapping, int64_t num_slots,
                                 int64_t num_blocks, int32_t block_size, char* msg,
                                 size_t msg_len) {
  auto fail = [&](const char* fmt, ...) {
    if (msg && msg_len) {
      va_list ap;
      va_start(ap, fmt);
      vsnprintf(msg, msg_len, fmt, ap);
      va_end(ap);
    }
    return PKV_ERR_METADATA;
  };
  if (msg && msg_len) msg[0] = '\0';
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail("bad sizes");
  if (num_seqs > 0 && (!block_tables || !seq_lens)) return fail("NULL block_tables or seq_lens");
  std::unordered_set<int32_t> used;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s];
    if (L < 0) return fail("seq_lens[%d] = %d is negative", s, L);
    if (L > max_seq_len) return fail("seq_lens[%d] = %d exceeds max_seq_len %d", s, L, max_seq_len);
    if ((int64_t)L > (int64_t)max_blocks_per_seq * block_size)
      return fail("seq_lens[%d] = %d needs more than %d blocks", s, L, max_blocks_per_seq);
    const int32_t nb = (L + block_size - 1) / block_size;
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + i];
      if (b <= 0 || b >= num_blocks)
        return fail("block_tables[%d][%d] = %d outside [1, %lld)", s, i, b, (long long)num_blocks);
      if (!used.insert(b).second) return fail("block %d used twice (seq %d)", b, s);
    }
  }
  if (cu_seqlens_q) {
    if (cu_seqlens_q[0] != 0) return fail("cu_seqlens_q[0] = %d, expected 0", cu_seqlens_q[0]);
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t ql = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
      if (ql < 0) return fail("cu_seqlens_q decreases at %d", s);
      if (ql > max_query_len) return fail("query length %d of seq %d > max_query_len", ql, s);
      if (ql > seq_lens[s]) return fail("query length %d of seq %d > seq_len %d", ql, s, seq_lens[s]);
    }
    if (cu_seqlens_q[num_seqs] != num_tokens)
      return fail("cu_seqlens_q[-1] = %d, expected num_tokens %d", cu_seqlens_q[num_seqs],
                  num_tokens);
  }
  if (slot_mapping) {
    std::unordered_set<int64_t> slots;
    const int64_t cap = num_blocks * block_size;
    for (int64_t t = 0; t < num_slots; ++t) {
      const int64_t sl = slot_mapping[t];
      if (sl == -1) continue;
      if (sl < 0 || sl >= cap) return fail("slot_mapping[%lld] = %lld outside the pool", (long long)t, (long long)sl);
      if (!slots.insert(sl).second) return fail("slot %lld written twice", (long long)sl);
    }
  }
  return PKV_OK;
}


}  // extern "C"
