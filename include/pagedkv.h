/*
 * pagedkv.h — C ABI of libpagedkv.so: paged KV-cache attention on AMD MI355X
 * (gfx950).
 *
 * Operations (as described by the vLLM pages):
 *   - the KV-cache slot write ("reshape_and_cache"): vLLM book
 *     «Implémentation du cœur du moteur d'inférence haute performance vLLM»,
 *     ch. 6 "Écriture du KV cache : do_kv_cache_update", and ch. 5.2
 *     "slot_mapping et la block table";
 *   - attention over a paged cache, decode and variable-length (chunked
 *     prefill) batches, with an optional split of the key range whose partial
 *     results are merged by log-sum-exp: ch. 6 "Structure des métadonnées",
 *     "build() étape par étape" (split buffer), "Flux des paramètres du chemin
 *     non-cascadé" and "forward()" (merge of partial attention states);
 *   - element formats: fp16 and bf16 models, caches also in fp8 (the
 *     backend's capability fields, ch. 6 "Sélection du backend", "Matrice de
 *     capacités : les champs comme contrat");
 *   - block bytes = 2 * block_size * num_kv_heads * head_size * dtype_bytes:
 *     «Khám phá vLLM: Giải phẫu hệ thống suy luận LLM thông lượng cao», §1 note.
 *
 * Conventions shared by every entry point
 *   Cache layout: K and V are separate tensors, each
 *     [num_blocks, block_size, num_kv_heads, head_size], row-major inside a
 *     block (ch. 6 "Transformation de la disposition mémoire du KV cache").
 *     Consecutive blocks are block_stride elements apart (0 = dense, i.e.
 *     block_size * num_kv_heads * head_size), so a block-outermost buffer
 *     shared by several layers can be passed as is.
 *   Slots: slot = physical_block * block_size + offset_in_block.
 *   Block tables: int32 [num_seqs, max_blocks_per_seq]; row s lists sequence
 *     s's physical blocks in logical order; only the first
 *     ceil(seq_len / block_size) entries are read.  Padding entries should be
 *     the null block 0 (ch. 5.2); the kernels never read a padding entry.
 *   seq_lens: int32 [num_seqs] = cached context + new query tokens (ch. 6
 *     "Structure des métadonnées"); the new tokens' K/V must already be in the
 *     cache when attention runs.  seq_len 0 is legal and yields zero output
 *     and lse = -inf.
 *   GQA: query head h reads kv head h / (num_heads / num_kv_heads).
 *   Causal (varlen only): query row i of a sequence with q_len rows sits at
 *     absolute position i + seq_len - q_len and sees keys j <= that position
 *     (ch. 6 "Branche de masque").
 *   Output: written in place, same dtype and layout as q; the float32
 *     results are rounded to bfloat16 or binary16 by round-to-nearest-even.
 *   lse_out (optional, may be NULL): float32 [rows, num_heads], natural-log
 *     log-sum-exp of the scaled logits each row saw; -inf for an empty row.
 *
 * Memory and execution
 *   Every pointer argument of type void* / int32_t* / int64_t* / float* that
 *   names a tensor is a DEVICE pointer, except in pkv_validate_metadata, which
 *   takes host pointers.  The caller allocates and owns every buffer,
 *   including the split workspace; the library never allocates, frees, copies
 *   to the host or synchronizes.  Calls are asynchronous on `stream` (a
 *   hipStream_t; NULL = the null stream), so they can be captured in a HIP
 *   graph.  `out` must not alias q, the caches or the workspace.
 *   Device tensors must be 16-byte aligned and dense in the last dimension;
 *   q/out/key/value are dense [rows, heads, head_size].
 *
 * Errors
 *   Host-side checks return a status and never abort: NULL pointers, bad sizes,
 *   unsupported dtype/head_size/block_size combinations (a reason string is
 *   available from pkv_unsupported_reason), misalignment, a too small
 *   workspace.  A failed kernel launch returns PKV_ERR_HIP.
 *   Device-resident metadata (block ids, slots, seq_lens, cu_seqlens_q) is not
 *   validated on the fast path.  Out-of-range values give unspecified results
 *   but never an out-of-bounds access: block ids are clamped into the pool,
 *   slots outside the pool are skipped, seq_lens are clamped to
 *   [0, min(max_seq_len, max_blocks_per_seq * block_size)] and query ranges
 *   to [0, num_tokens] and at most max_query_len rows.  pkv_validate_metadata
 *   checks all of this on host copies for tests and debugging.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 2

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                         */
  PKV_ERR_SHAPE = 2,       /* a size is negative / zero where it must be positive */
  PKV_ERR_UNSUPPORTED = 3, /* dtype/head_size/block_size/head ratio not supported */
  PKV_ERR_ALIGN = 4,       /* a pointer or stride is not 16-byte aligned          */
  PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required          */
  PKV_ERR_METADATA = 6,    /* pkv_validate_metadata found invalid metadata        */
  PKV_ERR_HIP = 7          /* a HIP launch failed                                 */
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3 = 2,  /* cache only: e4m3 codes (OCP "fn" variant: bias 7, max 448,
                        no infinities, 0x7F/0xFF NaN) with per-kv-head float32
                        scales; q, out, key and value are then bfloat16 */
  PKV_F16 = 3        /* IEEE 754 binary16 (fp16) caches, q, out, key and value;
                        outputs are rounded to nearest even (magnitudes past
                        65504 would become infinities: attention outputs are
                        weighted means of V rows, so they stay in range) */
} pkv_dtype;

/* Descriptor of one layer's paged KV cache (no ownership is transferred). */
typedef struct pkv_kv_cache {
  void*   k_cache;       /* device [num_blocks, block_size, num_kv_heads, head_size] */
  void*   v_cache;       /* device, same shape, dtype and block_stride as k_cache    */
  int64_t num_blocks;    /* pool size, 1 .. INT32_MAX (block ids are int32)         */
  int32_t block_size;    /* tokens per block: 8, 16, 32, 64 or 128                  */
  int32_t num_kv_heads;  /* > 0                                                     */
  int32_t head_size;     /* 64, 128 or 256 (256: float32, bfloat16 and binary16
                            caches; the capability matrix of ch. 6 "Matrice de
                            capacités : les champs comme contrat" lists a
                            backend of head size 256)                          */
  int32_t dtype;         /* pkv_dtype of both caches (and of q/out/key/value, which
                            are bfloat16 for PKV_FP8_E4M3)                          */
  int64_t block_stride;  /* elements between consecutive blocks; 0 = dense; the
                            stride in bytes must be below 2 GiB (PKV_ERR_SHAPE)    */
  const float* k_scale;  /* PKV_FP8_E4M3: device float32 [num_kv_heads]; cached code
                            c of kv head h stands for e4m3(c) * k_scale[h].  The
                            pages' (num_sequences, num_kv_heads) descale (vLLM book,
                            ch. 6 "Flux des paramètres du chemin non-cascadé") is a
                            broadcast of these per-layer scales.  NULL otherwise.  */
  const float* v_scale;  /* the same for V                                          */
} pkv_kv_cache;

/*
 * Per-call launch choices (in) and a report of what the call enqueued (out),
 * for measurements and tests.  Optional: the attention calls take a pointer
 * that may be NULL, which means the library's own choices and no report.
 * Every choice selects one of the library's kernel variants; all of them
 * compute the same attention within the stated tolerances.  A choice that
 * does not apply to a call (a forced VALU decode over an fp8 cache, which has
 * only the matrix-core kernel) is ignored.  Values other than those listed
 * return PKV_ERR_SHAPE.  The library keeps nothing of it after the call.
 */
typedef struct pkv_call_options {
  int32_t decode_kernel;   /* 0 library choice; 1 the VALU kernel; 2 the matrix-core
                              kernel (16-bit caches with head_size 128 or 256)     */
  int32_t prefill_kernel;  /* 0 library choice; 1 the VALU row kernel (16-bit)       */
  int32_t fp8_head_pairs;  /* 0 library choice; 1 one kv head per wave in fp8 decode  */
  int32_t mixed_launch;    /* 0 library choice; 1 prefill rows and decode rows of a
                              varlen batch in separate launches                     */
  int32_t cascade_launch;  /* 0 library choice; 1 the cascade's prefix and suffix
                              passes in separate launches                           */
  uint32_t launched;       /* out: PKV_RAN_* bits of the kernels the call enqueued
                              (0 when it returned before launching)                 */
} pkv_call_options;

#define PKV_RAN_PLANNER        0x001u  /* longest-first sequence order / work queues   */
#define PKV_RAN_DECODE_VALU    0x002u  /* one-row attention on the VALU                */
#define PKV_RAN_DECODE_MFMA    0x004u  /* one-row attention on the matrix cores        */
#define PKV_RAN_DECODE_PAIRS   0x008u  /* ... fp8, each wave reading two kv heads      */
#define PKV_RAN_PREFILL_MFMA   0x010u  /* multi-row (chunked prefill) launch, matrix cores */
#define PKV_RAN_PREFILL_VALU   0x020u  /* multi-row rows on the VALU row kernel        */
#define PKV_RAN_MIXED          0x040u  /* prefill tiles and decode rows in one launch  */
#define PKV_RAN_PREFIX         0x080u  /* cascade prefix pass, a launch of its own     */
#define PKV_RAN_CASCADE_ONE    0x100u  /* cascade prefix pass and decode rows in one launch */
#define PKV_RAN_SPLIT_MERGE    0x200u  /* log-sum-exp merge of key-range partials      */
#define PKV_RAN_CASCADE_MERGE  0x400u  /* merge of the cascade's prefix and suffix results */

/*
 * Scatter new K/V rows into the cache ("reshape_and_cache", ch. 6 "Écriture du
 * KV cache"): for t in [0, num_tokens) with slot = slot_mapping[t] >= 0,
 *   k_cache[slot / block_size, slot % block_size, :, :] = key[t, :, :]
 * and the same for value.  slot -1 (padding, ch. 5.2) writes nothing.  The
 * token count is num_tokens (the length of slot_mapping); key/value may hold
 * more, padded rows, which are never read.  Elements are copied bit for bit,
 * except into an fp8 cache: element x (bfloat16) of kv head h is stored as the
 * e4m3 code nearest to x / k_scale[h] (v_scale for V), the quotient taken in
 * float32 and saturated to +-448, ties to even, NaN as 0x7F.
 *   key, value   device [>= num_tokens, num_kv_heads, head_size], cache dtype
 *                (bfloat16 for an fp8 cache)
 *   slot_mapping device int64 [num_tokens]
 * Duplicate non-negative slots are undefined (one of the rows wins).
 * num_tokens == 0 is a no-op returning PKV_OK.
 */
pkv_status pkv_kv_cache_write(const pkv_kv_cache* cache, const void* key, const void* value,
                              const int64_t* slot_mapping, int64_t num_tokens, void* stream);

/*
 * Partition size (tokens per key-range split) the attention calls use for
 * these arguments: partition_size > 0 is used as given (a multiple of 32);
 * -1 means never split; 0 selects the library default.  Returns 0 when the
 * key range is not split, or a negative value if partition_size is invalid.
 */
int32_t pkv_choose_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t max_seq_len, int32_t partition_size);

/*
 * Workspace bytes an attention call needs (0 when it does not split): one
 * float32 partial output [num_splits, num_heads, num_seqs, head_size] and one
 * float32 log-sum-exp [num_splits, num_heads, num_seqs], the split buffer
 * shape of ch. 6 "build() étape par étape", with
 * num_splits = ceil(max_seq_len / partition) and rows indexed by sequence,
 * followed by an int32 [num_seqs] dispatch order of the sequences (each part
 * 16-byte aligned).  The contents are scratch of one call: nothing needs to
 * be initialised, and calls sharing a workspace must be ordered on a stream.
 * Returns (size_t)-1 for invalid arguments.
 */
size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t max_seq_len,
                                     int32_t partition_size);

/*
 * Decode attention: one query row per sequence.
 *   out, q        device [num_seqs, num_heads, head_size], cache dtype
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs]
 *   max_seq_len   host upper bound of seq_lens (sizes the launch and the split),
 *                 at most 2^30 (PKV_ERR_SHAPE above; the same bound holds for
 *                 the varlen and cascade calls)
 *   scale         logit scale (usually 1/sqrt(head_size)), finite; any sign
 *   window_left   sliding window (vLLM book, ch. 6 "forward()": the window
 *                 symmetrisation): the row at position p = seq_len - 1 sees
 *                 keys p - window_left .. p; -1 = no window.  A window of
 *                 max_seq_len - 1 or more excludes no key (any int32 width is
 *                 taken, as that one).  Key tiles start
 *                 at a multiple of 32 positions, so at most 31 keys before the
 *                 window start are read (and masked out); blocks that hold
 *                 none of those and none of the window are never read.
 *   partition_size see pkv_choose_partition_size
 *   lse_out       optional device float32 [num_seqs, num_heads]
 *   workspace     device, >= pkv_attention_workspace_bytes(...) bytes, 16-byte
 *                 aligned; may be NULL when that size is 0
 *   options       optional launch choices and report (pkv_call_options)
 * num_seqs == 0 is a no-op.
 */
pkv_status pkv_paged_attention_decode(void* out, const void* q, const pkv_kv_cache* cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                      int32_t max_seq_len, float scale, int32_t window_left,
                                      int32_t partition_size, float* lse_out, void* workspace,
                                      size_t workspace_bytes, pkv_call_options* options,
                                      void* stream);

/*
 * pkv_paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc.  It runs the same kernels with the
 * same results; the split partials and the sequence order that the workspace
 * would hold live instead in a scratch array of PKV_NOALLOC_SCRATCH_BYTES in
 * the library's device memory, one per GPU, held from the first call on that
 * GPU to the end of the process.  The call allocates nothing.
 *   Limit: a call for which pkv_attention_workspace_bytes(num_seqs,
 *   num_heads, num_kv_heads, head_size, max_seq_len, partition_size) exceeds
 *   PKV_NOALLOC_SCRATCH_BYTES returns PKV_ERR_WORKSPACE (128 MiB holds, for
 *   example, 256 sequences of 32 query heads up to 8192 tokens with
 *   512-token partitions).
 *   Every call on one GPU shares that GPU's array: calls that may overlap in
 *   time on one GPU (on different streams, or from threads that do not
 *   order them) race and give undefined results.  Order them on one stream.
 *   Nothing in the array needs to be cleared between calls.
 * Arguments and errors otherwise as for pkv_paged_attention_decode; PKV_ERR_HIP
 * also when the device's scratch address cannot be obtained.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const pkv_kv_cache* cache,
                                              const int32_t* block_tables,
                                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                              int32_t num_seqs, int32_t num_heads,
                                              int32_t max_seq_len, float scale,
                                              int32_t window_left, int32_t partition_size,
                                              float* lse_out, pkv_call_options* options,
                                              void* stream);

/*
 * Variable-length attention over a flattened batch (ch. 6 "Structure des
 * métadonnées": query_start_loc / seq_lens; «Khám phá vLLM» "Chạy forward
 * pass": all sequences flattened into one super-sequence).  Sequence s owns
 * query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of q/out and attends to
 * its seq_lens[s] cached tokens, causally if `causal` is non-zero.  Rows of
 * sequences with one query row are computed by the decode kernels (split by
 * partition_size, using the workspace); longer query ranges by the
 * matrix-core prefill kernel.
 *   out, q        device [num_tokens, num_heads, head_size]
 *   cu_seqlens_q  device int32 [num_seqs + 1], non-decreasing, from 0
 *   seq_lens      device int32 [num_seqs]
 *   max_query_len host upper bound of the query lengths
 *   scale         finite; must be positive when max_query_len > 1
 *                 (PKV_ERR_SHAPE otherwise): the prefill kernels take the
 *                 row maxima of the unscaled logits
 *   window_left   sliding window, -1 = none: a row at absolute position p sees
 *                 keys p - window_left .. p when causal, and
 *                 p - window_left .. p + window_left when not (the causal
 *                 window (w, 0) made symmetric, ch. 6 "forward()"); widths of
 *                 max_seq_len - 1 or more exclude no key, as for decode
 *   lse_out       optional device float32 [num_tokens, num_heads]
 *   options       optional launch choices and report (pkv_call_options)
 * Over an fp8 cache the prefill kernels fold k_scale into the logit scale,
 * so with max_query_len > 1 every k_scale entry must be positive as well
 * (device values, not checked; results are undefined otherwise).
 */
pkv_status pkv_paged_attention_varlen(void* out, const void* q, const pkv_kv_cache* cache,
                                      const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                      int32_t max_query_len, int32_t max_seq_len, float scale,
                                      int32_t causal, int32_t window_left, int32_t partition_size,
                                      float* lse_out, void* workspace, size_t workspace_bytes,
                                      pkv_call_options* options, void* stream);

/*
 * Cascade (shared-prefix) attention (vLLM book, ch. 6: "Structure des
 * métadonnées" for the cascade fields common_prefix_len and the prefix query
 * lengths; "forward()" for the cascade branch, a prefix call and a suffix
 * call merged by merge_attn_states; "Réflexion de conception" for when to
 * use it).  The result is that of pkv_paged_attention_varlen on the same
 * arguments (no window); only the work is regrouped:
 *   1. every query row of the batch attends to the shared prefix (keys
 *      0 .. common_prefix_len-1 read through prefix_blocks, no mask), on the
 *      matrix cores, the prefix split into key partitions with fp32 partials
 *      in the workspace: the prefix is read once for the whole batch instead
 *      of once per request;
 *   2. each row attends to its own keys common_prefix_len .. seq_len-1 under
 *      the usual mask (the varlen kernels; out and a suffix lse written);
 *   3. a log-sum-exp merge combines the two results in place in out.
 * Preconditions (not checked on this path; see pkv_validate_cascade):
 * common_prefix_len is a multiple of block_size, every sequence with
 * seq_len > 0 has its block table start with the prefix_blocks entries and
 * holds the prefix in its context (common_prefix_len <= seq_len - query
 * length).  Sequences with seq_len 0 are batch padding: zeros, lse -inf.
 *   prefix_blocks  device int32 [common_prefix_len / block_size] (row 0 of
 *                  block_tables will do)
 *   other arguments as for pkv_paged_attention_varlen
 *   workspace      >= pkv_cascade_workspace_bytes(...) bytes, 16-byte aligned
 * Takes every cache the varlen call takes.  Over bfloat16, binary16 and fp8
 * (e4m3) caches with head_size 128 the prefix pass runs on the matrix cores;
 * over float32 caches and other head sizes (or with the VALU row kernel
 * requested) it runs on the VALU kernel, one query row per workgroup, and
 * is then no faster than the plain call (pkv_cascade_reason says so).  When
 * common_prefix_len > 0 the scale must be positive (PKV_ERR_SHAPE
 * otherwise), and so must the fp8 k_scale entries, as for the prefill rows
 * of pkv_paged_attention_varlen.  common_prefix_len 0 is the plain varlen
 * call.
 * Asynchronous on `stream`.
 * The suffix result is rounded to the output dtype (bfloat16 or binary16)
 * before the merge, as the output of the pages' suffix call is; the prefix
 * partials stay fp32.
 */
pkv_status pkv_cascade_attention(void* out, const void* q, const pkv_kv_cache* cache,
                                 const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* prefix_blocks, int32_t num_seqs,
                                 int32_t num_tokens, int32_t num_heads, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t common_prefix_len, float scale,
                                 int32_t causal, int32_t partition_size, float* lse_out,
                                 void* workspace, size_t workspace_bytes,
                                 pkv_call_options* options, void* stream);

/*
 * Workspace bytes of pkv_cascade_attention: the prefix partials
 * [parts, num_heads, num_tokens, head_size] fp32 and their lse, the suffix
 * lse [num_tokens, num_heads] fp32, then the suffix pass's split workspace
 * (pkv_attention_workspace_bytes over the keys past the prefix).  The number
 * of prefix partitions depends only on these arguments.  (size_t)-1 for
 * invalid arguments.
 */
size_t pkv_cascade_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_size, int32_t max_seq_len,
                                   int32_t common_prefix_len, int32_t partition_size);

/*
 * Should a batch use cascade attention?  NULL when it is advised, else a
 * static string saying why not.  Caches whose prefix pass would run on the
 * VALU kernel (float32, or head_size other than 128) are not advised: there
 * the cascade measured no faster than the plain call.  Then the pages'
 * thresholds (ch. 6
 * "Réflexion de conception": a shared prefix of at least 256 tokens, at least
 * 8 requests, no sliding window), then a rough cost model of this library
 * for the prefix's share of the work: the plain form takes the longer of
 * num_seqs reads of the prefix from HBM and the rows' prefix flops on the
 * matrix cores; the cascade the longer of one read and the same flops, plus
 * writing and reading its fp32 partials.  dtype is a pkv_dtype;
 * window_left -1 = none.
 */
const char* pkv_cascade_reason(int32_t common_prefix_len, int32_t num_seqs, int32_t num_tokens,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                               int32_t dtype, int32_t window_left);

/*
 * Debug check of HOST copies of a cascade batch's metadata: common_prefix_len
 * a whole number of blocks, distinct prefix blocks, every sequence with
 * seq_len > 0 starting its table with them and holding the prefix in its
 * context, and its other blocks neither prefix blocks nor another sequence's.
 * Arrays the caller must supply in full (their lengths are not passed):
 * block_tables [num_seqs, max_blocks_per_seq], seq_lens [num_seqs],
 * cu_seqlens_q [num_seqs + 1], prefix_blocks [common_prefix_len / block_size]
 * (may be NULL when that is 0).  Returns PKV_OK or PKV_ERR_METADATA (message
 * as pkv_validate_metadata).
 */
pkv_status pkv_validate_cascade(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t num_seqs,
                                const int32_t* cu_seqlens_q, const int32_t* prefix_blocks,
                                int32_t common_prefix_len, int32_t block_size, char* msg,
                                size_t msg_len);

/*
 * Capability check in the spirit of supports_combination (ch. 6 "Matrice de
 * capacités"): NULL when the combination is supported, else a static string
 * saying why not.
 */
const char* pkv_unsupported_reason(int32_t dtype, int32_t head_size, int32_t block_size,
                                   int32_t num_heads, int32_t num_kv_heads);

/* Static, human-readable name of a status code (a pkv_status value; any
 * other integer gives "unknown status"). */
const char* pkv_status_string(int32_t status);

/*
 * Debug check of HOST copies of the metadata (synchronous, no GPU use):
 * block ids of used entries in [1, num_blocks) (block 0 is the reserved null
 * block), no block shared between used entries, seq_lens in
 * [0, min(max_seq_len, max_blocks_per_seq * block_size)], cu_seqlens_q (may
 * be NULL for decode) starting at 0, non-decreasing, ending at num_tokens,
 * query lengths <= min(seq_len, max_query_len), and slot_mapping (may be NULL)
 * entries either -1 or inside the pool, with no slot repeated.
 * Arrays the caller must supply in full (their lengths are not passed, and
 * the check reads up to these extents): block_tables
 * [num_seqs, max_blocks_per_seq], seq_lens [num_seqs], cu_seqlens_q
 * [num_seqs + 1], slot_mapping [num_slots].
 * Returns PKV_OK or PKV_ERR_METADATA; when `msg` is not NULL a description of
 * the first problem (or "") is written there, truncated to msg_len bytes.
 */
pkv_status pkv_validate_metadata(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t num_seqs,
                                 const int32_t* cu_seqlens_q, int32_t num_tokens,
                                 int32_t max_query_len, int32_t max_seq_len,
                                 const int64_t* slot_mapping, int64_t num_slots,
                                 int64_t num_blocks, int32_t block_size,
                                 char* msg, size_t msg_len);

/*
 * Per-launch timing of the main attention kernel, for benchmarks.  With
 * every_n > 0, one attention call in every_n (the first, then every n-th)
 * records a pair of HIP events on its stream around its main kernel (the
 * decode partition kernel; for a varlen call the mixed or prefill launch,
 * or the decode-row launch when every query range is one row; for a cascade
 * call that of its suffix pass); each
 * record costs a few microseconds of stream time, so sampling keeps the
 * timed steps close to untimed ones.  every_n = 0 disables timing.
 * pkv_timing_read waits for the recorded events, writes up to `cap`
 * durations in milliseconds (oldest first) and returns how many were
 * written; it then clears the record.  Up to 4096 launches are kept.  Not
 * for use under graph capture.  Returns PKV_OK, PKV_ERR_SHAPE for
 * every_n < 0, or PKV_ERR_HIP.
 */
pkv_status pkv_timing_enable(int32_t every_n);
int32_t pkv_timing_read(float* ms, int32_t cap);

/*
 * Dispatch probe (benchmark support): launches n one-wave workgroups on
 * `stream`; workgroup i writes to xcd_out[i] the index (0-7) of the XCD it
 * ran on.  The hardware places consecutive workgroups of a launch on
 * consecutive XCDs from a start that is dispatcher state (the same for
 * consecutive launches on a queue; it can change when other queues run),
 * and the decode kernels' speed depends on it by a few per cent, so a
 * benchmark records it beside its timings.
 *   xcd_out  device int32 [n], 1 <= n <= 1024
 * Returns PKV_ERR_NULL, PKV_ERR_SHAPE (n out of range) or PKV_ERR_HIP.
 * Asynchronous on `stream`.
 */
pkv_status pkv_xcd_probe(int32_t* xcd_out, int32_t n, void* stream);

/*
 * Host KV block pool: the step before the attention calls, which hands out
 * the cache's physical blocks to requests and produces their block tables
 * and slot mappings (vLLM book, ch. 4.1 and 4.4; «Khám phá vLLM»,
 * "Scheduler", allocate_slots).  Host memory only; thread safe per pool.
 *   - Block 0 is the null block: never handed out, used to pad block tables.
 *   - A request of n tokens owns ceil(n / block_size) blocks.  Free blocks
 *     are reused last-freed first when they hold no prefix-cache entry, and
 *     least recently used first when they do.
 *   - With prefix caching, full blocks entered with pkv_pool_cache_full_blocks
 *     are found again by later requests with the same leading tokens
 *     (hash chained over the block's token ids; at most num_tokens - 1 tokens
 *     of a new request come from the cache).
 */
typedef struct pkv_block_pool pkv_block_pool;

/* num_blocks >= 2 (the pool size of the cache), block_size > 0.  NULL on bad
 * arguments or out of memory. */
pkv_block_pool* pkv_pool_create(int64_t num_blocks, int32_t block_size, int32_t prefix_caching);
void pkv_pool_destroy(pkv_block_pool* pool);
/* Free blocks (the null block excluded). */
int64_t pkv_pool_num_free(pkv_block_pool* pool);
/* Make request `req` own blocks for num_tokens tokens (growing it if it
 * exists).  token_ids (host int32 [num_tokens], may be NULL) lets a new
 * request reuse cached full blocks.  Returns the number of leading tokens
 * found in the cache (0 for an existing request), -1 when the pool cannot
 * provide every block needed (nothing changes), -2 on bad arguments. */
int64_t pkv_pool_allocate(pkv_block_pool* pool, int64_t req, int64_t num_tokens,
                          const int32_t* token_ids);
/* Enter the request's full blocks among its first num_tokens tokens (host
 * int32 token_ids) into the prefix cache. */
pkv_status pkv_pool_cache_full_blocks(pkv_block_pool* pool, int64_t req, const int32_t* token_ids,
                                      int64_t num_tokens);
/* Release a request's blocks. */
pkv_status pkv_pool_free(pkv_block_pool* pool, int64_t req);
/* Blocks the request owns, or -1 if unknown. */
int64_t pkv_pool_num_blocks_of(pkv_block_pool* pool, int64_t req);
/* Host int32 [n, max_blocks] block table of the listed requests, padded with
 * the null block; PKV_ERR_SHAPE if a request is unknown or owns more blocks. */
pkv_status pkv_pool_block_table(pkv_block_pool* pool, const int64_t* reqs, int32_t n,
                                int32_t max_blocks, int32_t* out);
/* Host int64 [count] slots (block * block_size + offset) of token positions
 * first_pos .. first_pos + count - 1 of a request (inside its blocks). */
pkv_status pkv_pool_slot_mapping(pkv_block_pool* pool, int64_t req, int64_t first_pos,
                                 int64_t count, int64_t* out);
/* The free queue, head first, written up to cap entries; returns its length
 * (inspection and tests). */
int64_t pkv_pool_free_queue(pkv_block_pool* pool, int32_t* out, int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
