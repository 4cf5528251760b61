// Internal declarations shared by the host API and the kernel translation
// units of libpagedkv.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

// How the attention kernels map grid.z to work.
enum AttnMode : int32_t {
  kModeDecode = 0,     // z = sequence; one query row per sequence (row = sequence)
  kModeVarlenOne = 1,  // z = sequence; only sequences with exactly one query row
  kModeVarlenRows = 2, // z = query row; only rows of sequences with > 1 query rows, no split
  kModePrefix = 3      // cascade prefix pass: every query row of the batch against the shared
                       // prefix (keys 0 .. prefix_len-1 through block_tables row 0), no mask;
                       // z = key partition of partition_size tokens, fp32 partials out (the
                       // VALU kernel: grid.y = query row, grid.z = partition, num_seqs = rows)
};

// Arguments of the attention kernels (passed by value).
struct AttnArgs {
  void* out;                       // [rows, num_heads, D], cache dtype
  const void* q;                   // [rows, num_heads, D]
  const void* k_cache;             // [num_blocks, BS, Hkv, D]
  const void* v_cache;
  const int32_t* block_tables;     // [num_seqs, max_blocks_per_seq]
  const int32_t* seq_lens;         // [num_seqs]
  const int32_t* cu_seqlens_q;     // [num_seqs + 1] or nullptr (decode)
  float* lse_out;                  // [rows, num_heads] or nullptr
  float* ws_o;                     // [num_splits, num_heads, num_seqs, D]
  float* ws_lse;                   // [num_splits, num_heads, num_seqs]
  const int32_t* seq_order;        // [num_seqs] dispatch order of sequences, or nullptr
  int64_t block_stride;            // elements between blocks
  int64_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t block_size;
  int32_t num_seqs;
  int32_t num_tokens;              // rows of q/out
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_seq_len;
  int32_t max_query_len;
  int32_t partition_size;          // tokens per split; 0 = one partition
  int32_t num_splits;              // splits the workspace holds
  int32_t head_chunks;             // query-head chunks per kv head
  int32_t parts_per_wg;            // consecutive partitions one workgroup covers (>= 1);
                                   // the workspace holds one partial per workgroup range
  int32_t wave_per_part;           // 1: wave w of a workgroup owns partition w of its range
  int32_t heads_per_wave;          // grouped decode over e4m3 caches: 2 = each wave reads two
                                   // adjacent kv heads (grid.x = kv-head pairs); else 1
  int32_t head_chunks_gc;          // prefill: query heads per column group (power of 2, <= 8)
  int32_t z_base;                  // offset added to blockIdx.z
  int32_t range_desc;              // 1: grid.z runs over key ranges from the last one down
  int32_t mode;                    // AttnMode
  int32_t causal;
  int32_t window_left;             // sliding window (keys >= pos - window_left; symmetric
                                   // when not causal), -1 = none
  int32_t skip_multi_row;          // kModeVarlenRows: 1 if another kernel owns multi-row seqs
  int32_t kv_start;                // keys before this position are left out for every row
                                   // (cascade suffix pass; 0 otherwise)
  int32_t prefix_len;              // kModePrefix: keys of the shared prefix
  float scale_log2;                // scale * log2(e)
  const float* k_scale;            // fp8 caches: per-kv-head scales (value = code * scale)
  const float* v_scale;
};

struct KvWriteArgs {
  void* k_cache;
  void* v_cache;
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;               // num_blocks * block_size
  int64_t block_stride_bytes;
  int32_t block_size;
  int32_t row_bytes;               // num_kv_heads * head_size * elem_bytes (of the cache)
  int32_t head_size;
  const float* k_scale;            // fp8 caches: per-kv-head scales, else nullptr
  const float* v_scale;
};

// Host checks of pkv_paged_attention_decode's arguments, all but the
// workspace: PKV_OK when the call would go on to launch (or, for
// num_seqs == 0, return PKV_OK without launching).
pkv_status decode_host_checks(const void* out, const void* q, const pkv_kv_cache* cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t max_seq_len, float scale, int32_t window_left,
                              int32_t partition_size, const pkv_call_options* options);

// Benchmark timing (timing.cpp): timing_begin returns true, with a slot, when
// this launch is one of the sampled ones and its start event was recorded;
// timing_end then records the stop event after the launch.
bool timing_begin(hipStream_t st, int* slot);
void timing_end(hipStream_t st, int slot);

// Launchers (return the launch error, hipSuccess on success).
// fp8 = true: bfloat16 key/value quantised into e4m3 caches.
hipError_t launch_kv_write(const KvWriteArgs& a, bool fp8, hipStream_t stream);

// General VALU attention kernel: float32, bfloat16 or binary16 caches (dtype
// is the pkv_dtype), head size 64/128, block size 8/16/32/64/128, any GQA
// ratio.
hipError_t launch_attn_valu(const AttnArgs& a, int dtype, int head_size, int block_size,
                            int heads_per_chunk, dim3 grid, hipStream_t stream);

// The matrix-core kernels below take the cache's pkv_dtype: PKV_BF16,
// PKV_F16 or PKV_FP8_E4M3 (any other value: hipErrorInvalidValue).
// Grouped-query decode on the matrix cores: head size 128 (256 over 16-bit
// caches), up to 16 query heads per kv-head chunk (head_chunks =
// ceil(group / 16)).
// grid = (num_kv_heads * head_chunks, sequences, ceil(partitions / parts_per_wg)).
hipError_t launch_attn_mfma_decode(const AttnArgs& a, int block_size, int head_size, int dtype,
                                   dim3 grid, hipStream_t stream);

// Chunked prefill on the matrix cores (rows of sequences with > 1 query
// rows): head size 128.
// grid = (query tiles of 128 / head_chunks_gc rows, num_kv_heads * group /
// head_chunks_gc, sequences).
hipError_t launch_attn_mfma_prefill(const AttnArgs& a, int block_size, int dtype, dim3 grid,
                                    hipStream_t stream);

// Permutation of 0..num_seqs-1 ordering sequences longest first (one
// workgroup; seq_lens clamped to max_len).  With cu_seqlens_q, also the list
// of sequences with more than one query row (any order) and its length.
hipError_t launch_seq_order(const int32_t* seq_lens, int32_t num_seqs, int32_t max_len,
                            int32_t* order, const int32_t* cu_seqlens_q, int32_t num_tokens,
                            int32_t* multi_list, int32_t* multi_count, int32_t* queues,
                            hipStream_t stream);

// One launch for a mixed varlen batch: prefill tiles (args `pre`, mode
// kModeVarlenRows) over the listed multi-row sequences, and decode rows
// (args `dcd`, mode kModeVarlenOne, grouped matrix-core decode), interleaved.
struct MixedGrid {
  int64_t n_dec;                   // decode items: dec_x * dec_y * dec_z
  int32_t pre_x, pre_y;            // prefill items per listed sequence: query tiles x head groups
  int32_t pre_z;                   // cascade: prefix partitions (items = pre_x * pre_y * pre_z)
  int32_t pre_share;               // in four, the CU classes ((index / 8) % 4; mixed step) or XCDs
                                   // (index % 4; cascade) that start on the first queue
  int32_t dec_x, dec_y, dec_z;     // kv-head chunks, row items, key ranges
  int32_t workgroups;              // persistent grid size
  const int32_t* pre_list;         // [num_seqs] multi-row sequences (planner)
  const int32_t* pre_count;        // [1] how many
  int32_t* queues;                 // [2] item counters (prefill, decode), zeroed by the planner
};
hipError_t launch_attn_mixed(const AttnArgs& pre, const AttnArgs& dcd, const MixedGrid& g,
                             int block_size, int dtype, hipStream_t stream);
// The same persistent grid for a cascade of decode rows: prefix-pass items
// (args `pre`, mode kModePrefix) and the suffix pass's decode rows (`dcd`).
hipError_t launch_attn_cascade(const AttnArgs& pre, const AttnArgs& dcd, const MixedGrid& g,
                               int block_size, int dtype, hipStream_t stream);

// Cascade prefix pass on the matrix cores (mode kModePrefix, head size
// 128): grid = (query tiles of 128 / head_chunks_gc rows over all
// num_tokens rows, num_kv_heads * group / head_chunks_gc, key partitions).
// Writes normalised fp32 partials to ws_o [part][head][row][D] and their
// log2-domain log-sum-exps to ws_lse [part][head][row].
hipError_t launch_attn_mfma_prefix(const AttnArgs& a, int block_size, int dtype, dim3 grid,
                                   hipStream_t stream);

// Cascade merge: out (the suffix result, in place) and its natural-log lse
// `lse_suffix` [rows, heads] are combined with `num_parts` prefix partials
// (layout of launch_attn_mfma_prefix); rows of sequences with seq_len 0 keep
// the suffix result (zeros).  out_dtype PKV_F32, PKV_BF16 or PKV_F16; head
// size 64, 128 or 256.
hipError_t launch_cascade_merge(const AttnArgs& a, const float* lse_suffix, int num_parts,
                                int out_dtype, int head_size, hipStream_t stream);

// Log-sum-exp merge of split partial results (modes kModeDecode/kModeVarlenOne).
hipError_t launch_splitkv_reduce(const AttnArgs& a, int dtype, int head_size,
                                 hipStream_t stream);

}  // namespace pkv
