// Chunked-prefill paged attention on the matrix cores (gfx950 MFMA).
//
// Rows of sequences with several query rows: a prefill chunk of q_len new
// tokens attends to the sequence's seq_len cached tokens (its own new tokens
// already written by the slot write), query row i sitting at absolute
// position i + seq_len - q_len and, when causal, seeing keys j <= that
// position (vLLM book, ch. 6 "Branche de masque" for the bottom-right
// alignment; "Structure des métadonnées" for query_start_loc / seq_lens;
// «Khám phá vLLM», "Chạy forward pass", for the flattened batch).
//
// Work decomposition: a workgroup of 4 waves owns 8 column tiles of one kv
// head's query-head group, a column tile being 16 consecutive query rows of
// one query head; wave w owns column tiles 2w and 2w+1.  With g query heads
// per kv head (chunks of GC <= 8 heads), the workgroup covers 8 / GC row
// blocks of 16 rows.  Several workgroups share a CU, so their MFMA and
// softmax phases interleave.  The key range [0, kv_end) is walked in 32-token
// tiles that the 256 threads load cooperatively (two 16-byte chunks of K and
// two of V per thread: whole 256-byte token rows) straight into a 4-stage LDS
// ring with global_load_lds (no registers held), one barrier per tile, three
// tiles in flight ahead of the one being computed.  The direct loads write
// lane l's 16 bytes at offset 16*l, so the swizzled LDS layouts (16-byte slot
// c ^ f(row)) are produced by choosing which chunk each lane fetches.  Tokens
// past the key range load the last valid token (finite data; their
// probabilities are exactly 0).  Per wave and tile, every LDS read issued
// first:
//   S^T[32 tok x 16 rows] = K . Q^T        (8 A reads from LDS, 8 MFMAs per column tile)
//   online softmax per column (= query row), causal mask by select
//   O^T[128 x 16] += V^T . P^T             (V^T via ds_read_b64_tr_b16, shared by both tiles)
// with the second column tile's exponentials interleaved between the first
// tile's PV products (fenced, so that the VALU and matrix work overlap).
// Tiles lying wholly above a wave's rows on the causal diagonal are skipped,
// and masks are applied only to tiles that cross a diagonal or the range end.
// The running max used as the exponent reference is raised only when a
// column's max grows by more than 2^8 (then the accumulators are rescaled);
// otherwise probabilities up to 2^8 are accumulated against the old
// reference.  The result is unchanged: output and log-sum-exp are formed
// from the same reference.  Unmasked tiles form their probabilities against
// the current reference first and compute the maxima only when some lane's
// sum exceeds 2^8 (the only case in which the reference can need raising).
// Tiles inside the key range whose successor tiles are all in flight run a
// steady step without end-of-range tests, four at a time, each with its LDS
// stage fixed at compile time.
#pragma once

#include <type_traits>

#include "attn_common.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace pf {


constexpr int kWaves = 4;
constexpr int kColTiles = 2 * kWaves;          // column tiles per workgroup
constexpr float kRescaleSlack = 8.f;            // log2 of the largest unscaled probability
constexpr float kSlackSum = 256.f;              // 2^kRescaleSlack
// Initial exponent reference: a finite stand-in for -inf, far below any
// logit, so that no step needs an infinity test (the first visible key
// raises it; a column that sees no key keeps it and has sum 0)
constexpr float kMinRef = -3.0e38f;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;
constexpr int kTile = 32;
constexpr int kKBytes = kTile * kD * 2;          // 8 KiB
constexpr int kVBytes = kTile * kD * 2;
constexpr int kStageBytes = kKBytes + kVBytes;   // 16 KiB
constexpr int kStages = 4;                       // LDS ring depth
constexpr int kLdsBytes = kStages * kStageBytes;
// fp8 caches: a ring of kStages stages of codes (K rows of 128 B, then V
// rows), then two bfloat16 tiles laid out as the stages above
constexpr int kKBytes8 = kTile * kD;             // 4 KiB
constexpr int kStageBytes8 = 2 * kKBytes8;       // 8 KiB
constexpr int kRingBytes8 = kStages * kStageBytes8;
static_assert(kRingBytes8 + 2 * kStageBytes <= kLdsBytes, "fp8 layout fits the LDS of a workgroup");
// A scheduling fence: the compiler moves no instruction across it, so code
// written interleaved stays interleaved.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte slot of chunk c of token row t: K rows are swizzled so 16 lanes
// reading one chunk of 16 rows (MFMA A operand) hit distinct bank groups; V
// rows so the transposed reads (16 rows x 32 bytes) spread over all banks.
__device__ __forceinline__ int kslot(int t, int c) { return c ^ (t & 15); }
__device__ __forceinline__ int vslot(int t, int c) { return c ^ ((t & 7) << 1); }
__device__ __forceinline__ int ktile_off(int t, int c) { return t * (kD * 2) + (kslot(t, c) << 4); }

// Transposed LDS read (ds_read_b64_tr_b16) written as inline asm.  Before
// the intrinsic form the compiler waits for every outstanding direct-to-LDS
// load, since it cannot tell which LDS bytes they write; here that would
// drain the tile ring on every tile.  The reads of a tile are ordered after
// its loads by each thread's own wait for them plus the barrier; their
// results are waited for with lds_results_ready.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t lds_addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF) : "memory");
  return r;
}
// 16-byte LDS read written as inline asm, for the same reason: the compiler
// cannot always tell a plain read of the current stage apart from the ring's
// direct-to-LDS loads in flight, and then waits for all of them before it
// (inside the persistent launches it did so on every tile).
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128_at(uint32_t lds_addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF) : "memory");
  return r;
}
// Waits until at most N LDS operations are outstanding (they complete in
// order), then marks the K registers written so that no use of them is
// scheduled before the wait.
template <int N>
__device__ __forceinline__ void lds_k_ready(u32x4 (&r)[2][4]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is four bits");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(r[tt][j]));
}
// Waits for every outstanding LDS read, then marks the registers written so
// that no use of them is scheduled before the wait.
template <int N>
__device__ __forceinline__ void lds_results_ready(u32x2 (&r)[N][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) {
    asm volatile("" : "+v"(r[i][0]));
    asm volatile("" : "+v"(r[i][1]));
  }
}

// NaN-propagating max (v_maximum3_f32): unlike fmaxf it needs no
// canonicalisation of its operands.
__device__ __forceinline__ float vmax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

__device__ __forceinline__ float xmax16_32(float x) {
  auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = vmax(__int_as_float(p16[0]), __int_as_float(p16[1]));
  auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return vmax(__int_as_float(p32[0]), __int_as_float(p32[1]));
}
__device__ __forceinline__ float xsum16_32(float x) {
  auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(p16[0]) + __int_as_float(p16[1]);
  auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p32[0]) + __int_as_float(p32[1]);
}

// One workgroup's work: query tile bx, head group by of sequence seq.  The
// caller provides the LDS ring (kLdsBytes, 16-byte aligned).
// PREFIX (cascade prefix pass): the rows are all num_tokens query rows of
// the batch, the keys are partition `seq` (partition_size tokens) of the
// shared prefix read through block_tables row 0, no mask applies, and the
// result is a normalised fp32 partial with its log2-domain log-sum-exp.
// FP8: e4m3 caches.  The tile loads bring the codes into a ring of 8 KiB
// stages (K rows of 128 B, then V rows); each step the workgroup converts
// the next tile exactly to bfloat16 into one of two 16 KiB tiles laid out
// as the bfloat16 stages are (each thread converts the 16 + 16 codes it
// loaded itself), and the products read those.  The per-kv-head k_scale is
// folded into the logit scale and v_scale into the output.
// DT is the cache's pkv_dtype: PKV_BF16, PKV_F16 (binary16 operands and
// output; the unscaled probabilities stay below 2^8, well inside its range)
// or PKV_FP8_E4M3.
// Workgroup i of a launch runs on XCD i % 8.  The query tiles (x) of one
// stream -- a head group (y) of one sequence or prefix partition (z) --
// read the same keys and values.  Numbering the workgroups of a z slice so
// that each XCD takes whole streams lets one L2 serve all of a stream's
// tiles.  Only slices of a multiple of 8 workgroups are renumbered (then
// workgroup l of the slice runs on XCD l % 8 whatever z is); z keeps its
// order, since the slices of one-row sequences in a varlen launch are empty.
__device__ __forceinline__ void xcd_stream_order(int& bx, int& by) {
  const uint32_t X = gridDim.x, n = X * gridDim.y;
  if (n % 8 != 0) return;
  const uint32_t l = blockIdx.x + X * blockIdx.y;
  const uint32_t i = (l % 8) * (n / 8) + l / 8;   // stream-major item of the slice
  by = (int)(i / X);
  bx = (int)(i - (uint32_t)by * X);
}

// XCD_ORDER: (bx, by) are the launch's block indices, renumbered by
// xcd_stream_order once the workgroup is known to hold prefill rows.
template <int BS, bool PREFIX, int DT, bool XCD_ORDER = false>
__device__ __forceinline__ void prefill_block(const AttnArgs& a, int bx, int by, int seq,
                                              char* __restrict__ s_lds) {
  static_assert(DT == PKV_BF16 || DT == PKV_F16 || DT == PKV_FP8_E4M3, "cache dtype");
  constexpr bool FP8 = DT == PKV_FP8_E4M3;
  using H = Fmt16<DT == PKV_F16>;                    // operand format of the products
  using x8 = typename H::x8;
  int qs, q_len, L, off;
  const int part = PREFIX ? seq : 0;
  if constexpr (PREFIX) {
    seq = 0;
    qs = 0;
    q_len = a.num_tokens;
    L = a.prefix_len;
    off = 0;
  } else {
    qs = clamp_i(load_uniform_i32(a.cu_seqlens_q, seq), 0, a.num_tokens);
    const int qe = clamp_i(load_uniform_i32(a.cu_seqlens_q, seq + 1), 0, a.num_tokens);
    q_len = min(qe - qs, a.max_query_len);
    if (qe - qs <= 1) return;                        // one-row sequences: decode kernels
    L = clamp_seq_len(load_uniform_i32(a.seq_lens, seq), a.max_seq_len, a.max_blocks_per_seq, BS);
    off = L - (qe - qs);                             // absolute position of row i = i + off
  }
  if constexpr (XCD_ORDER) xcd_stream_order(bx, by);
  const int GC = a.head_chunks_gc;                   // query heads per column group (<= 8)
  const int R = kColTiles / GC;                      // row blocks per workgroup
  const int q0 = bx * 16 * R;
  if (q0 >= q_len) return;
  const int group = a.num_heads / a.num_kv_heads;
  const int chunks = group / GC;
  const int kvh = by / chunks;
  const int hbase = kvh * group + (by % chunks) * GC;
  // logit scale (log2 domain) and output scale: the fp8 cache's per-head
  // scales fold into them
  const float sl2 = FP8 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float oscale = FP8 ? a.v_scale[kvh] : 1.f;

  // The thread index passes through an empty asm: in a persistent grid that
  // runs this body and another per item, the lane-derived offsets are then
  // formed inside each body, not hoisted above the item loop and held in
  // registers across both bodies.
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int kg = lane >> 4;

  // key range of the workgroup
  const int q_last = min(q0 + 16 * R, q_len) - 1;
  // sliding window w: row at position p sees keys p - w .. p (causal) or
  // p - w .. p + w (not causal)
  const int win = PREFIX ? -1 : a.window_left;
  const bool causal = PREFIX ? false : a.causal != 0;
  // first key of the range for every row: the prefix partition's start, or
  // kv_start (keys before it belong to a cascade's prefix pass)
  const int key_lo = PREFIX ? min(part * a.partition_size, L) : a.kv_start;
  int kv_end = causal ? max(0, min(L, q_last + off + 1)) : L;
  if (PREFIX) kv_end = min(L, key_lo + a.partition_size);
  if (win >= 0 && !causal) kv_end = max(0, min(kv_end, q_last + off + win + 1));
  const int kv_begin = min(max(win >= 0 ? max(0, q0 + off - win) : 0, key_lo), kv_end);
  const int ntiles = (kv_end + kTile - 1) / kTile;   // tiles t_begin .. ntiles - 1
  const int t_begin = kv_begin / kTile;

  // this wave's two column tiles: (row block, head)
  int rowb[2], head[2];
  bool live[2];
  int wave_last_pos = -1;                            // largest key position this wave may see
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ct = 2 * wave + c;
    rowb[c] = q0 + (ct / GC) * 16;
    head[c] = hbase + ct % GC;
    live[c] = rowb[c] < q_len;
    if (live[c]) wave_last_pos = max(wave_last_pos, min(rowb[c] + 15, q_len - 1) + off);
  }
  if (!causal) wave_last_pos = win >= 0 ? min(L - 1, wave_last_pos + win) : L - 1;
  // smallest key position this wave may see (sliding window, range start)
  const int wave_first_key = max(win >= 0 ? min(rowb[0], rowb[1]) + off - win : 0, key_lo);

  // Q^T B operands, lane (kg, n): row rowb + n, dims (4j + kg)*8 .. +8
  x8 qb[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = rowb[c] + n;
    const bool ok = live[c] && row < q_len;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)(qs + row) * a.num_heads + head[c]) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(qp + (4 * j + kg) * 8);
      qb[c][j] = H::as_x8(v);
    }
  }
  // the queries must be resident before any tile load is issued: otherwise
  // the first use of them inside the tile loop would wait for every load in
  // flight on each iteration
  __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));

  f32x4 o[2][8];
  float m[2], lsum[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) o[c][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = kMinRef;
    lsum[c] = 0.f;
  }

  // cooperative tile loads: load u (0, 1) of thread tid fills LDS row
  // r = 16u + tid/16, slot tid%16, with the chunk of token r that belongs
  // there; each wave covers 4 consecutive tokens per load, inside one block
  // (block ids wave uniform).
  const int lrow = tid >> 4;
  const int lslot = tid & 15;
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
  const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = static_cast<const char*>(a.v_cache);
  // token row and head offsets in elements (bfloat16) or bytes (fp8)
  const uint32_t tok_stride = (uint32_t)a.num_kv_heads * kD;
  const uint32_t head_off = (uint32_t)kvh * kD;
  // block ids are clamped into the pool: num_blocks < 2^31, and a block is
  // far below 4 GiB, so the byte offset is one 32 x 32 -> 64-bit product
  const uint32_t max_blk = (uint32_t)min<int64_t>(a.num_blocks - 1, INT32_MAX);
  const uint32_t blk_bytes = (uint32_t)(a.block_stride * (FP8 ? 1 : 2));
  const int last_tok = max(0, kv_end - 1);

  // block ids of tile t's token groups for this wave (two 16-token halves;
  // fp8: one group of 8 tokens), as scalar loads fetched one iteration
  // before they are used; the arithmetic on them waits until then, so the
  // load's latency hides behind a tile of work
  auto fetch_ids = [&](int t, int32_t* raw) {
#pragma unroll
    for (int u = 0; u < (FP8 ? 1 : 2); ++u) {
      const uint32_t tw = min((uint32_t)t * kTile + (FP8 ? 8 * wave : 16 * u + 4 * wave),
                              (uint32_t)last_tok);
      const uint32_t bi = __builtin_amdgcn_readfirstlane(tw / BS);
      raw[u] = load_uniform_i32(bt, bi);
    }
  };
  // bfloat16: load u (0, 1) of thread tid fills LDS row r = 16u + tid/16,
  // slot tid%16, with the chunk of token r that belongs there (each wave
  // covers 4 consecutive tokens per load, inside one block).  fp8: thread
  // tid loads codes 16 (tid%8) .. +15 of token r = tid/8 (each wave covers 8
  // consecutive tokens, inside one block), into the stage row r.
  // Lane part (bytes) of the loads of a tile inside the key range: token
  // t * 32 + r sits at offset r % BS of its block when 32 is a multiple of
  // BS; with larger blocks at offset (t * 32) % BS + r, the first term added
  // per tile.
  constexpr int kEB = FP8 ? 1 : 2;                   // cache element bytes
  uint32_t klane[2], vlane[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (FP8) {
      const int r = tid >> 3;
      klane[u] = vlane[u] = ((uint32_t)(r % BS) * tok_stride + head_off) + (tid & 7) * 16;
    } else {
      const int r = 16 * u + lrow;
      const uint32_t lo = (uint32_t)(r % BS) * tok_stride + head_off;
      klane[u] = (lo + kslot(r, lslot) * 8) * 2;   // slot s holds chunk s ^ f(r): involution
      vlane[u] = (lo + vslot(r, lslot) * 8) * 2;
    }
  }
  // issue the direct-to-LDS loads of tile t into stage buf (4 per thread;
  // fp8: 2); in the last, partial tile tokens past the range are clamped to
  // the last valid one, which stays in the block of the wave's first token
  auto issue = [&](int t, const int32_t* raw, char* buf, auto full_tag) {
    const bool full = decltype(full_tag)::value || (t + 1) * kTile <= kv_end;
    // blocks larger than a tile: the tile's first row within its block
    uint32_t toff = 0;
    if constexpr (BS > kTile) toff = ((uint32_t)(t * kTile) % BS) * tok_stride * kEB;
#pragma unroll
    for (int u = 0; u < (FP8 ? 1 : 2); ++u) {
      const uint64_t boff = (uint64_t)min((uint32_t)max(raw[u], 0), max_blk) * blk_bytes;
      const char* kb = reinterpret_cast<const char*>(kc) + boff;
      const char* vb = reinterpret_cast<const char*>(vc) + boff;
      char* kdst = buf + (FP8 ? 0 : u * 4096) + wave * 1024;
      char* vdst = buf + (FP8 ? kKBytes8 : kKBytes + u * 4096) + wave * 1024;
      if (full) {
        __builtin_amdgcn_global_load_lds(kb + toff + klane[u], (lds_void*)kdst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + toff + vlane[u], (lds_void*)vdst, 16, 0, 0);
      } else if constexpr (FP8) {
        const int r = tid >> 3;
        const int tok = min(t * kTile + r, last_tok);
        const uint32_t lo = (uint32_t)(tok % BS) * tok_stride + head_off + (tid & 7) * 16;
        __builtin_amdgcn_global_load_lds(kb + lo, (lds_void*)kdst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + lo, (lds_void*)vdst, 16, 0, 0);
      } else {
        const int r = 16 * u + lrow;
        const int tok = min(t * kTile + r, last_tok);
        const uint32_t lo = (uint32_t)(tok % BS) * tok_stride + head_off;
        __builtin_amdgcn_global_load_lds(kb + (lo + kslot(r, lslot) * 8) * 2, (lds_void*)kdst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + (lo + vslot(r, lslot) * 8) * 2, (lds_void*)vdst, 16, 0, 0);
      }
    }
  };
  // fp8: convert this thread's codes of the stage (K chunk pair and V chunk
  // pair of token r = tid/8, dims 16 (tid%8) .. +15) into the bfloat16 tile
  // dst, at the slots the bfloat16 layouts give them
  auto convert = [&](const char* stage, char* dst) {
    if constexpr (FP8) {
      const int r = tid >> 3, c8 = tid & 7;
      const u32x4 kw = *reinterpret_cast<const u32x4*>(stage + tid * 16);
      const u32x4 vw = *reinterpret_cast<const u32x4*>(stage + kKBytes8 + tid * 16);
      u32x4 k0, k1, v0, v1;
      e4m3x16_to_bf16x16(kw, k0, k1);
      e4m3x16_to_bf16x16(vw, v0, v1);
      *reinterpret_cast<u32x4*>(dst + ktile_off(r, 2 * c8)) = k0;
      *reinterpret_cast<u32x4*>(dst + ktile_off(r, 2 * c8 + 1)) = k1;
      *reinterpret_cast<u32x4*>(dst + kKBytes + r * (kD * 2) + (vslot(r, 2 * c8) << 4)) = v0;
      *reinterpret_cast<u32x4*>(dst + kKBytes + r * (kD * 2) + (vslot(r, 2 * c8 + 1) << 4)) = v1;
    }
  };

  // LDS read offsets of this lane inside a stage: K chunk 4j + kg of row n
  // (row n + 16 adds 4096 B); V rows t0 = 4kg + n/4 (and t0 + 16, + 4096 B)
  // for dims 16jd + 4(n%4) .. +3, i.e. half (n%4)&1 of chunk 2jd + (n%4)/2
  uint32_t koff[4], voff[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = ktile_off(n, 4 * j + kg);
  {
    const int jj = n >> 2, q4 = n & 3;
    const int t0 = 4 * kg + jj;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const int ch = 2 * jd + (q4 >> 1);
      voff[jd] = kKBytes + t0 * (kD * 2) + (vslot(t0, ch) << 4) + (q4 & 1) * 8;
    }
  }

  // MASKED: the tile may hold keys past a row's causal limit or the range
  // end, or lie wholly above this wave's rows (skipped).
  // SO: the tile's byte offset from s_lds when known at compile time (>= 0),
  // else -1; the transposed reads then take it as their immediate offset, so
  // their address registers do not depend on the stage
  auto compute = [&](int t, const char* buf, auto masked_tag, auto so_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int SO = decltype(so_tag)::value;
    const int j0 = t * kTile;
    // wholly above this wave's diagonal, or below its window
    if (MASKED && (j0 > wave_last_pos || j0 + kTile - 1 < wave_first_key)) return;
    // every LDS read of the tile issued up front: the 8 K chunks for the A
    // operands, then the 16 transposed V rows (waited for before the first PV
    // product).  The K chunks are waited for after the first 8 V reads
    // (lgkmcnt counts to 15).  With the stage known at compile time the
    // reads take its offset as an immediate.
    constexpr int KO = SO >= 0 ? SO : 0;
    const uint32_t lbase = SO >= 0 ? (uint32_t)(uintptr_t)(lds_void*)s_lds
                                   : (uint32_t)(uintptr_t)(lds_void*)buf;
    u32x4 kr[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kr[0][j] = ds_read_b128_at<KO>(lbase + koff[j]);
      kr[1][j] = ds_read_b128_at<KO + 4096>(lbase + koff[j]);
    }
    u32x2 vr[8][2];
#pragma unroll
    for (int jd = 0; jd < 4; ++jd) {
      vr[jd][0] = ds_read_tr16_b64<KO>(lbase + voff[jd]);
      vr[jd][1] = ds_read_tr16_b64<KO + 16 * kD * 2>(lbase + voff[jd]);
    }
    lds_k_ready<8>(kr);
#pragma unroll
    for (int jd = 4; jd < 8; ++jd) {
      vr[jd][0] = ds_read_tr16_b64<KO>(lbase + voff[jd]);
      vr[jd][1] = ds_read_tr16_b64<KO + 16 * kD * 2>(lbase + voff[jd]);
    }
    x8 ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) ka[tt][j] = H::as_x8(kr[tt][j]);
    // S^T = K Q^T for both column tiles
    f32x4 sacc[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sacc[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[c][tt] = H::mfma(ka[tt][j], qb[c][j], sacc[c][tt]);
      }
    // masked raw logits (the scale is applied inside the exponent), row
    // maxima and the reference decisions of both column tiles
    float s[2][8], mn[2];
    bool raise[2];
    if constexpr (!MASKED) {
      // Unmasked tiles: the probabilities are formed against the current
      // reference without the tile's maxima first.  If a column's max
      // outgrew the reference by more than the slack, some probability
      // exceeds 2^slack and so does its lane's sum; then (and only then) that
      // column tile takes the full step: maxima, raised reference, rescale,
      // probabilities again.  The result is the same as always taking it.
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[c][tt * 4 + i] = sacc[c][tt][i];
      auto full_step = [&](int c, x8& pb, float& psum) {
        float mx = vmax(vmax(vmax(s[c][0], s[c][1]), vmax(s[c][2], s[c][3])),
                        vmax(vmax(s[c][4], s[c][5]), vmax(s[c][6], s[c][7])));
        mx = xmax16_32(mx) * sl2;
        if (mx > m[c] + kRescaleSlack) {
          const float alpha = fast_exp2(m[c] - mx);
          lsum[c] *= alpha;
#pragma unroll
          for (int jd = 0; jd < 8; ++jd) o[c][jd] *= alpha;
          m[c] = mx;
        }
        psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(s[c][e], sl2, -m[c]));
          psum += p;
          pb[e] = (typename H::elem)p;
        }
      };
      x8 pb0, pb1;
      float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(fmaf(s[0][e], sl2, -m[0]));
        psum0 += p;
        pb0[e] = (typename H::elem)p;
      }
      if (__builtin_amdgcn_ballot_w64(!(psum0 <= kSlackSum))) full_step(0, pb0, psum0);
      lsum[0] += psum0;
      lds_results_ready(vr);
      x8 va[8];
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        const u32x4 w = {vr[jd][0][0], vr[jd][0][1], vr[jd][1][0], vr[jd][1][1]};
        va[jd] = H::as_x8(w);
      }
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        sched_fence();
        o[0][jd] = H::mfma(va[jd], pb0, o[0][jd]);
        const float p = fast_exp2(fmaf(s[1][jd], sl2, -m[1]));
        psum1 += p;
        pb1[jd] = (typename H::elem)p;
      }
      sched_fence();
      if (__builtin_amdgcn_ballot_w64(!(psum1 <= kSlackSum))) full_step(1, pb1, psum1);
      lsum[1] += psum1;
#pragma unroll
      for (int jd = 0; jd < 8; ++jd)
        o[1][jd] = H::mfma(va[jd], pb1, o[1][jd]);
      return;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qpos = rowb[c] + n + off;            // this lane's column = query row
      const int lim = causal ? min(qpos, kv_end - 1)
                              : (win >= 0 ? min(qpos + win, kv_end - 1) : kv_end - 1);
      const int lo = max(win >= 0 ? qpos - win : 0, key_lo);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + tt * 16 + 4 * kg + i;
          s[c][tt * 4 + i] = (!MASKED || (j <= lim && j >= lo)) ? sacc[c][tt][i] : -INFINITY;
        }
      float mx = vmax(vmax(vmax(s[c][0], s[c][1]), vmax(s[c][2], s[c][3])),
                      vmax(vmax(s[c][4], s[c][5]), vmax(s[c][6], s[c][7])));
      mx = xmax16_32(mx) * sl2;             // scale > 0 preserves the max
      // raise the reference only when the max outgrows it by the slack
      raise[c] = mx > m[c] + kRescaleSlack;
      mn[c] = raise[c] ? mx : m[c];
    }
    // rescale the accumulators of the columns whose reference rose (alpha
    // = 2^0 = 1 for the others; the reference starts at kMinRef, so a first
    // raise gives alpha = 0)
    if (__builtin_amdgcn_ballot_w64(raise[0] || raise[1])) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float alpha = fast_exp2(m[c] - mn[c]);
        lsum[c] *= alpha;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) o[c][jd] *= alpha;
      }
    }
    m[0] = mn[0];
    m[1] = mn[1];
    // probabilities and O^T += V^T P^T: the first column tile's
    // exponentials, then its eight products, each followed (in program
    // order, fenced so that the compiler keeps it) by one exponential of the
    // second column tile, whose products come last
    x8 pb0, pb1;
    float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(fmaf(s[0][e], sl2, -m[0]));
      psum0 += p;
      pb0[e] = (typename H::elem)p;
    }
    lsum[0] += psum0;
    lds_results_ready(vr);
    x8 va[8];
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const u32x4 w = {vr[jd][0][0], vr[jd][0][1], vr[jd][1][0], vr[jd][1][1]};
      va[jd] = H::as_x8(w);
    }
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      sched_fence();
      o[0][jd] = H::mfma(va[jd], pb0, o[0][jd]);
      const float p = fast_exp2(fmaf(s[1][jd], sl2, -m[1]));
      psum1 += p;
      pb1[jd] = (typename H::elem)p;
    }
    sched_fence();
    lsum[1] += psum1;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd)
      o[1][jd] = H::mfma(va[jd], pb1, o[1][jd]);
  };

  // LDS ring: tile t lives in stage t % kStages.  bfloat16: before
  // computing tile t a thread waits for its own loads of t (the loads of up
  // to kStages - 2 later tiles may stay in flight), then the barrier makes t
  // visible to all and guarantees every wave has finished tile t - 1, whose
  // stage is refilled.  fp8: at step t a thread waits for its own loads of
  // tile t + 1 and for its conversion writes of tile t, the barrier makes
  // the bfloat16 tile t visible and frees the bfloat16 tile of t - 1, into
  // which the thread then converts its codes of t + 1.
  constexpr int kLoadsPerTile = FP8 ? 2 : 4;
  auto stage = [&](int t) {
    return s_lds + ((uint32_t)t % kStages) * (FP8 ? kStageBytes8 : kStageBytes);
  };
  auto tile = [&](int t) { return FP8 ? s_lds + kRingBytes8 + (t & 1) * kStageBytes : stage(t); };
  // the same with the stage known at compile time: PH = t % kStages (>= 0),
  // so that the LDS addresses become immediate offsets
  auto stage_ph = [&](int t, auto ph, int k) {
    constexpr int PH = decltype(ph)::value;
    if constexpr (PH >= 0)
      return s_lds + ((PH + k) % kStages) * (FP8 ? kStageBytes8 : kStageBytes);
    else
      return stage(t + k);
  };
  auto tile_ph = [&](int t, auto ph, int k) {
    constexpr int PH = decltype(ph)::value;
    if constexpr (PH >= 0)
      return FP8 ? s_lds + kRingBytes8 + ((PH + k) & 1) * kStageBytes : stage_ph(t, ph, k);
    else
      return tile(t + k);
  };
  int32_t ids[2];
#pragma unroll
  for (int t = t_begin; t < t_begin + kStages - 1; ++t)
    if (t < ntiles) {
      fetch_ids(t, ids);
      issue(t, ids, stage(t), std::false_type{});
    }
  if (t_begin + kStages - 1 < ntiles) fetch_ids(t_begin + kStages - 1, ids);
  if constexpr (FP8) {
    if (t_begin < ntiles) {
      const int ahead = min(kStages - 2, ntiles - 1 - t_begin);   // tiles issued after t_begin
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * kLoadsPerTile));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(kLoadsPerTile));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
      convert(stage(t_begin), tile(t_begin));
    }
  }
  // STEADY: t + kStages < ntiles, so the tiles issued after t are in flight
  // (kStages - 2 of them), and the tile issued now (t + kStages - 1) is whole
  // and has a successor whose block ids are fetched.
  // PH: t % kStages when known at compile time, else -1
  constexpr std::integral_constant<int, -1> kNoPhase{};
  auto step = [&](int t, auto masked_tag, auto steady_tag, auto ph) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    if constexpr (FP8) {
      const int ahead = STEADY ? 1 : min(1, ntiles - 2 - t);   // tiles issued after t + 1
      if (ahead >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(kLoadsPerTile));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this thread's conversion writes
    } else {
      const int ahead = STEADY ? kStages - 2 : min(kStages - 2, ntiles - 1 - t);   // tiles issued after t
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * kLoadsPerTile));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(kLoadsPerTile));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    }
    // a bare barrier: __syncthreads() would add a fence that drains the
    // loads of the tiles still in flight.  Each thread has waited for its own
    // loads of tile t above; LDS reads of tile t - 1 were consumed before.
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if constexpr (FP8)
      if (STEADY || t + 1 < ntiles) convert(stage_ph(t, ph, 1), tile_ph(t, ph, 1));
    const int tn = t + kStages - 1;
    if (STEADY || tn < ntiles) issue(tn, ids, stage_ph(t, ph, kStages - 1), steady_tag);
    {
      constexpr int PH = decltype(ph)::value;
      constexpr int SO = PH < 0 ? -1
                         : FP8 ? kRingBytes8 + (PH & 1) * kStageBytes
                               : (PH % kStages) * kStageBytes;
      compute(t, tile_ph(t, ph, 0), masked_tag, std::integral_constant<int, SO>{});
    }
    // the next tile's block ids: loaded after this tile's LDS reads, so that
    // their waits do not include the scalar loads
    if (STEADY || tn + 1 < ntiles) fetch_ids(tn + 1, ids);
  };
  // Tiles wholly at or below the workgroup's first row position and inside
  // the key range need no mask for any wave; the rest (the diagonal band and
  // the range end) take the masked path.  Every wave runs both loops over
  // the same tiles, so the barriers stay matched.
  // With a window, tiles below the last row's window start are masked too.
  int unmasked_end = causal ? min(q0 + off, kv_end - 1) : kv_end - 1;
  if (win >= 0 && !causal) unmasked_end = min(unmasked_end, q0 + off + win);
  const int unmasked_begin = max(win >= 0 ? max(0, q_last + off - win) : 0, key_lo);
  const int tu = min(ntiles, max(t_begin, (unmasked_begin + kTile - 1) / kTile));
  const int tm = min(ntiles, max(tu, (unmasked_end + 1) / kTile));
  const int ts = max(tu, min(tm, ntiles - kStages));   // steady unmasked tiles: [tu, ts)
  for (int t = t_begin; t < tu; ++t) step(t, std::true_type{}, std::false_type{}, kNoPhase);
  // steady tiles: up to a multiple of kStages one by one, then kStages at a
  // time with every stage known at compile time
  int t = tu;
  for (; t < ts && ((uint32_t)t % kStages) != 0; ++t) step(t, std::false_type{}, std::true_type{}, kNoPhase);
  static_assert(kStages == 4, "the unrolled steady loop covers four stages");
  for (; t + kStages <= ts; t += kStages) {
    step(t, std::false_type{}, std::true_type{}, std::integral_constant<int, 0>{});
    step(t + 1, std::false_type{}, std::true_type{}, std::integral_constant<int, 1>{});
    step(t + 2, std::false_type{}, std::true_type{}, std::integral_constant<int, 2>{});
    step(t + 3, std::false_type{}, std::true_type{}, std::integral_constant<int, 3>{});
  }
  for (; t < ts; ++t) step(t, std::false_type{}, std::true_type{}, kNoPhase);
  for (int t = ts; t < tm; ++t) step(t, std::false_type{}, std::false_type{}, kNoPhase);
  for (int t = tm; t < ntiles; ++t) step(t, std::true_type{}, std::false_type{}, kNoPhase);

  // normalise and write the rows this lane holds: O^T[16jd + 4kg + r][n]
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float ls = xsum16_32(lsum[c]);
    const int row = rowb[c] + n;
    if (!live[c] || row >= q_len) continue;
    const float inv = ls > 0.f ? oscale / ls : 0.f;
    if constexpr (PREFIX) {
      const int64_t e = ((int64_t)part * a.num_heads + head[c]) * a.num_tokens + row;
      float* op = a.ws_o + e * kD;
#pragma unroll
      for (int jd = 0; jd < 8; ++jd)
        *reinterpret_cast<f32x4*>(op + 16 * jd + 4 * kg) = o[c][jd] * inv;
      if (kg == 0) a.ws_lse[e] = ls > 0.f ? m[c] + acc_log2(ls) : -INFINITY;
      continue;
    }
    uint16_t* op = static_cast<uint16_t*>(a.out) + ((int64_t)(qs + row) * a.num_heads + head[c]) * kD;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const uint32_t w0 = pack16x2<DT == PKV_F16>(o[c][jd][0] * inv, o[c][jd][1] * inv);
      const uint32_t w1 = pack16x2<DT == PKV_F16>(o[c][jd][2] * inv, o[c][jd][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * jd + 4 * kg) = make_uint2(w0, w1);
    }
    if (kg == 0 && a.lse_out)
      a.lse_out[(int64_t)(qs + row) * a.num_heads + head[c]] =
          ls > 0.f ? (m[c] + acc_log2(ls)) * kLn2 : -INFINITY;
  }
}

}  // namespace pf
}  // namespace pkv
