// Work-item resolution shared by the attention and reduce kernels: maps a
// workgroup's grid.z index to (sequence, query row, visible key range,
// partitioning).  Both kernels must agree exactly, so it lives in one place.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// Kv head (or kv-head pair) that grid column `col` of a decode launch works
// on, for launches with one column per kv head, whose rows of row_bytes bytes
// sit side by side in every token row.  The dispatcher places workgroup i on
// XCD (i + s) % 8, where the start s is its own state (0 for a new queue, and
// usually after launches whose workgroup counts are multiples of 8), so
// column c runs on an XCD of the parity of c + s.  A workgroup streams
// measurably faster (2-3 % over a whole decode launch) when its XCD's parity
// differs from that of the 256-byte slot its rows occupy.  With 256-byte rows
// the slot's parity is the head's, so adjacent heads swap columns; with
// 128-byte rows (two heads to a slot) the columns of each group of four take
// heads 2, 0, 3, 1: at s = 0 every head then runs on an XCD of the other
// parity.  A fixed permutation of the columns, correct whatever the
// dispatcher does; heads of an incomplete pair or group keep their columns,
// and other row sizes keep the identity.
__device__ __forceinline__ int column_head(int col, int num, int row_bytes) {
  if (row_bytes == 256) {
    const int h = col ^ 1;
    return h < num ? h : col;
  }
  if (row_bytes == 128) {
    const int base = col & ~3;
    if (base + 3 >= num) return col;
    const int r = col & 3;
    return base + (r == 0 ? 2 : r == 1 ? 0 : r == 2 ? 3 : 1);
  }
  return col;
}

// Resolved work item of one workgroup.
struct Item {
  int seq;
  int row;       // query row in q / out
  int L_begin;   // keys L_begin .. L_end-1 are visible to this row
  int L_end;
  int base;      // L_begin rounded down to 32: partition p covers base + [pP, (p+1)P)
  int nparts;    // partitions the row's key range is split into
  int nranges;   // workgroup ranges of parts_per_wg partitions (one partial each)
  int P;         // partition size in tokens
};

// Maps the workgroup to (sequence, row, key range).  Returns false when the
// workgroup has nothing to do.  Identical logic runs in the reduce kernel.
__device__ __forceinline__ bool resolve_item(const AttnArgs& a, int z, Item& it) {
  if (a.mode == kModePrefix) {
    // cascade prefix pass on the VALU kernel: query row z of the batch
    // against the shared prefix (keys 0 .. prefix_len-1, read through
    // block-table row 0), unmasked, one partial per partition; the partials
    // are indexed by row (the launch passes num_seqs = rows)
    if (z >= a.num_tokens || a.partition_size <= 0) return false;
    it.seq = z;
    it.row = z;
    it.L_begin = 0;
    it.L_end = min(max(a.prefix_len, 0), a.max_blocks_per_seq * a.block_size);
    it.base = 0;
    it.P = a.partition_size;
    it.nparts = max(1, (it.L_end + it.P - 1) / it.P);
    it.nranges = it.nparts;
    return true;
  }
  int seq, row, qlen = 1, qidx = 0;
  if (a.mode == kModeDecode) {
    seq = z;
    row = z;
  } else if (a.mode == kModeVarlenOne) {
    seq = z;
    int qs = clamp_i(a.cu_seqlens_q[seq], 0, a.num_tokens);
    int qe = clamp_i(a.cu_seqlens_q[seq + 1], 0, a.num_tokens);
    if (qe - qs != 1) return false;
    row = qs;
  } else {
    row = z;
    // last sequence whose query range starts at or before this row
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (clamp_i(a.cu_seqlens_q[mid], 0, a.num_tokens) <= row) lo = mid; else hi = mid - 1;
    }
    seq = lo;
    int qs = clamp_i(a.cu_seqlens_q[seq], 0, a.num_tokens);
    int qe = clamp_i(a.cu_seqlens_q[seq + 1], 0, a.num_tokens);
    qlen = qe - qs;
    qidx = row - qs;
    if (qidx < 0 || qidx >= qlen) return false;       // row outside every range
    if (qlen == 1) return false;                       // owned by the one-row launch
    if (a.skip_multi_row) return false;
    if (qidx >= a.max_query_len) return false;         // beyond the host bound: not computed
  }
  int L = clamp_seq_len(a.seq_lens[seq], a.max_seq_len, a.max_blocks_per_seq, a.block_size);
  // absolute position of the row: L - 1 for one-row sequences
  const int pos = qidx + L - qlen;
  int L_end = L;
  if (a.causal && a.mode == kModeVarlenRows) L_end = min(L, max(0, pos + 1));
  int L_begin = 0;
  if (a.window_left >= 0) {
    // sliding window: keys pos - w .. pos (causal); pos - w .. pos + w otherwise
    L_begin = min(max(0, pos - a.window_left), L_end);
    if (!(a.causal || a.mode != kModeVarlenRows)) L_end = min(L_end, max(0, pos + a.window_left + 1));
  }
  // keys before kv_start are left out (cascade suffix pass)
  L_begin = max(L_begin, min(a.kv_start, L_end));
  it.seq = seq;
  it.row = row;
  it.L_begin = L_begin;
  it.L_end = L_end;
  it.base = L_begin & ~31;
  if (a.partition_size > 0 && a.mode != kModeVarlenRows) {
    it.P = a.partition_size;
    it.nparts = max(1, (L_end - it.base + it.P - 1) / it.P);
    // partials are kept per workgroup range of parts_per_wg partitions
    it.nranges = (it.nparts + a.parts_per_wg - 1) / a.parts_per_wg;
  } else {
    it.P = max(L_end - it.base, 1);
    it.nparts = 1;
    it.nranges = 1;
  }
  return true;
}

}  // namespace pkv
