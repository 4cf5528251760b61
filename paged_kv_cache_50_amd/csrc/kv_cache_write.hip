// KV-cache slot write ("reshape_and_cache"; vLLM book, ch. 6 "Écriture du KV
// cache : do_kv_cache_update", ch. 5.2 "slot_mapping et la block table").
//
// For token t with slot = slot_mapping[t] >= 0:
//   K[slot / bs, slot % bs, :, :] = key[t],  V[...] = value[t].
// slot -1 marks padding and writes nothing; slots outside the pool are
// skipped as well, so bad metadata cannot write out of bounds.
// One wave copies one token's row of num_kv_heads * head_size elements for K
// and for V with 16-byte loads and stores (the row is contiguous both in
// key/value and inside the destination block).
#include "pkv_internal.h"
#include "device_common.h"

namespace pkv {
namespace {

constexpr int kTokensPerWg = 4;

__global__ void __launch_bounds__(64 * kTokensPerWg) kv_write_kernel(const KvWriteArgs a) {
  const int64_t t = (int64_t)blockIdx.x * kTokensPerWg + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.num_tokens) return;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot % a.block_size;
  const int64_t dst = blk * a.block_stride_bytes + off * a.row_bytes;
  const int64_t src = t * a.row_bytes;
  const char* __restrict__ ks = static_cast<const char*>(a.key) + src;
  const char* __restrict__ vs = static_cast<const char*>(a.value) + src;
  char* __restrict__ kd = static_cast<char*>(a.k_cache) + dst;
  char* __restrict__ vd = static_cast<char*>(a.v_cache) + dst;
  for (int i = lane * 16; i < a.row_bytes; i += 64 * 16) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(ks + i);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(vs + i);
    *reinterpret_cast<u32x4*>(kd + i) = kv;
    *reinterpret_cast<u32x4*>(vd + i) = vv;
  }
}

// e4m3 caches: key/value rows are bfloat16; element x of kv head h is stored
// as the e4m3 code nearest to x / scale[h] (float32 division, saturated to
// +-448, ties to even; NaN -> 0x7F).  A lane quantises 8 elements (16 bytes
// in, 8 out), all of one head since head_size is a multiple of 8.
__global__ void __launch_bounds__(64 * kTokensPerWg) kv_write_fp8_kernel(const KvWriteArgs a) {
  const int64_t t = (int64_t)blockIdx.x * kTokensPerWg + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.num_tokens) return;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot % a.block_size;
  const int elems = a.row_bytes;                     // one byte per cached element
  const int64_t dst = blk * a.block_stride_bytes + off * elems;
  const int64_t src = t * (int64_t)elems * 2;
  const char* __restrict__ ks = static_cast<const char*>(a.key) + src;
  const char* __restrict__ vs = static_cast<const char*>(a.value) + src;
  char* __restrict__ kd = static_cast<char*>(a.k_cache) + dst;
  char* __restrict__ vd = static_cast<char*>(a.v_cache) + dst;
  auto quant8 = [](const u32x4 x, float s) {
    uint2 r;
    r.x = f32x4_to_e4m3x4(e4m3_sat(bf16_lo(x[0]) / s), e4m3_sat(bf16_hi(x[0]) / s),
                          e4m3_sat(bf16_lo(x[1]) / s), e4m3_sat(bf16_hi(x[1]) / s));
    r.y = f32x4_to_e4m3x4(e4m3_sat(bf16_lo(x[2]) / s), e4m3_sat(bf16_hi(x[2]) / s),
                          e4m3_sat(bf16_lo(x[3]) / s), e4m3_sat(bf16_hi(x[3]) / s));
    return r;
  };
  for (int e = lane * 8; e < elems; e += 64 * 8) {
    const int h = e / a.head_size;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(ks + 2 * e);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(vs + 2 * e);
    *reinterpret_cast<uint2*>(kd + e) = quant8(kv, a.k_scale[h]);
    *reinterpret_cast<uint2*>(vd + e) = quant8(vv, a.v_scale[h]);
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs& a, bool fp8, hipStream_t stream) {
  const int64_t wgs = (a.num_tokens + kTokensPerWg - 1) / kTokensPerWg;
  if (fp8)
    hipLaunchKernelGGL(kv_write_fp8_kernel, dim3((unsigned)wgs), dim3(64 * kTokensPerWg), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)wgs), dim3(64 * kTokensPerWg), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace pkv
