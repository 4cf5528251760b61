// pkv_paged_attention_decode_noalloc: decode attention whose split partials
// and sequence order live in a scratch array of the library's own device
// memory instead of a caller-allocated workspace, for callers that cannot
// allocate (graph capture, serving loops).  The kernels are those of
// pkv_paged_attention_decode; only where the workspace comes from differs.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

// One copy per GPU, at its own address on each.  In host code the name only
// stands for the symbol: the device address comes from hipGetSymbolAddress
// (scratch_address below), and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device (threads that race on the first lookup store the same address).
pkv_status scratch_address(void** addr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode_noalloc(
    void* out, const void* q, const pkv_kv_cache* cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
    int32_t max_seq_len, float scale, int32_t window_left, int32_t partition_size,
    float* lse_out, pkv_call_options* options, void* stream) {
  if (options) options->launched = 0;
  // the decode call's own checks first, so that errors match it
  const pkv_status chk =
      pkv::decode_host_checks(out, q, cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                              num_heads, max_seq_len, scale, window_left, partition_size, options);
  if (chk != PKV_OK) return chk;
  const size_t need = pkv_attention_workspace_bytes(num_seqs, num_heads, cache->num_kv_heads,
                                                    cache->head_size, max_seq_len,
                                                    partition_size);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (num_seqs > 0 && need > 0) {
    if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
    const pkv_status st = scratch_address(&ws);
    if (st != PKV_OK) return st;
    ws_bytes = PKV_NOALLOC_SCRATCH_BYTES;
  }
  return pkv_paged_attention_decode(out, q, cache, block_tables, max_blocks_per_seq, seq_lens,
                                    num_seqs, num_heads, max_seq_len, scale, window_left,
                                    partition_size, lse_out, ws, ws_bytes, options, stream);
}
