// Per-launch timing of the main attention kernel (benchmark support): HIP
// events recorded around sampled launches on the caller's stream.  Kept
// apart from the launch logic: it never changes what the kernels do.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

struct Timing {
  std::mutex mu;
  bool enabled = false;
  int64_t every = 1;   // time one launch in `every`
  int64_t calls = 0;   // launches seen since timing was enabled
  static constexpr int kCap = 4096;
  hipEvent_t start[kCap] = {};
  hipEvent_t stop[kCap] = {};
  int64_t head = 0;  // oldest unread record
  int64_t tail = 0;  // next record
};
Timing g_timing;
constexpr int kEagerSlots = 64;

}  // namespace

// Creates the events of record slot i if needed.  Timing-only events:
// without the system-scope fence a record costs no L2 writeback/invalidate
// (which would otherwise add a few microseconds around every timed launch
// and cool the caches of the next kernel).
bool ensure_events(int i) {
  if (g_timing.start[i]) return true;
  if (hipEventCreateWithFlags(&g_timing.start[i], hipEventDisableSystemFence) != hipSuccess)
    return false;
  if (hipEventCreateWithFlags(&g_timing.stop[i], hipEventDisableSystemFence) != hipSuccess) {
    (void)hipEventDestroy(g_timing.start[i]);
    g_timing.start[i] = nullptr;
    return false;
  }
  return true;
}

bool timing_begin(hipStream_t st, int* slot) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!g_timing.enabled) return false;
  if (g_timing.calls++ % g_timing.every != 0) return false;
  const int i = (int)(g_timing.tail % Timing::kCap);
  if (!ensure_events(i)) return false;
  if (g_timing.tail - g_timing.head >= Timing::kCap) g_timing.head++;  // overwrite oldest
  if (hipEventRecord(g_timing.start[i], st) != hipSuccess) return false;
  *slot = i;
  return true;
}

void timing_end(hipStream_t st, int slot) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (hipEventRecord(g_timing.stop[slot], st) == hipSuccess) g_timing.tail++;
}

}  // namespace pkv

using pkv::ensure_events;
using pkv::g_timing;
using pkv::kEagerSlots;
using pkv::Timing;

extern "C" {

pkv_status pkv_timing_enable(int32_t every_n) {
  if (every_n < 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.enabled = every_n != 0;
  g_timing.every = every_n > 0 ? every_n : 1;
  g_timing.calls = 0;
  g_timing.head = g_timing.tail = 0;
  // the first records' events are created here, not between the launches
  // being timed (a creation costs host time that a short step can notice)
  if (g_timing.enabled)
    for (int i = 0; i < kEagerSlots; ++i)
      if (!ensure_events(i)) return PKV_ERR_HIP;
  return PKV_OK;
}

int32_t pkv_timing_read(float* ms, int32_t cap) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  int32_t n = 0;
  for (int64_t k = g_timing.head; k < g_timing.tail && n < cap; ++k) {
    const int i = (int)(k % Timing::kCap);
    if (hipEventSynchronize(g_timing.stop[i]) != hipSuccess) return -1;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_timing.start[i], g_timing.stop[i]) != hipSuccess) return -1;
    if (ms) ms[n] = t;
    ++n;
  }
  g_timing.head = g_timing.tail;
  return n;
}

}  // extern "C"

// ---- dispatch probe

namespace {

// Workgroup i writes the XCD it runs on (hardware register XCC_ID, bits 3:0).
__global__ void __launch_bounds__(64) xcd_probe_kernel(int32_t* out, int32_t n) {
  if (threadIdx.x == 0 && (int32_t)blockIdx.x < n)
    out[blockIdx.x] = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xF;
}

}  // namespace

extern "C" pkv_status pkv_xcd_probe(int32_t* xcd_out, int32_t n, void* stream) {
  if (!xcd_out) return PKV_ERR_NULL;
  if (n < 1 || n > 1024) return PKV_ERR_SHAPE;
  hipLaunchKernelGGL(xcd_probe_kernel, dim3(n), dim3(64), 0, static_cast<hipStream_t>(stream),
                     xcd_out, n);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
