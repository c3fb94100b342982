// Per-kernel timing: while enabled on a thread, every kernel the library
// launches from that thread is bracketed by a pair of hipEvents recorded on
// its stream.  Used by the benchmark to attribute time to kernels and to
// cross-check the rocprofv3 kernel trace.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <vector>

#include "host.h"

namespace fp8mlp {

namespace {
struct Rec {
  const char* name;
  hipEvent_t begin, end;
};
struct TraceState {
  bool on = false;
  std::vector<Rec> pool;  // created events, reused
  int used = 0;
  int dropped = 0;
};
thread_local TraceState g_trace;
// the launch in progress on this thread (set between a TraceScope's
// construction and destruction) and the last kernel the sync check saw fail
thread_local const char* g_cur_name = nullptr;
thread_local hipStream_t g_cur_stream = nullptr;
thread_local bool g_cur_set = false;
thread_local const char* g_failed_kernel = nullptr;
}  // namespace

bool sync_check_on() {
  const char* e = std::getenv("FP8MLP_SYNC_CHECK");
  return e != nullptr && e[0] == '1';
}

int sync_check() {
  hipError_t e = hipSuccess;
  if (g_cur_set) {
    // never under graph capture: a capturing stream cannot be waited on
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(g_cur_stream, &cs);
    if (e == hipSuccess && cs != hipStreamCaptureStatusNone) return FP8MLP_OK;
    if (e == hipSuccess) e = hipStreamSynchronize(g_cur_stream);
  } else {
    e = hipDeviceSynchronize();
  }
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) g_failed_kernel = g_cur_set ? g_cur_name : "(launch outside a named scope)";
  return hip_status(e);
}

TraceScope::TraceScope(const char* name, hipStream_t s) : stream_(s), slot_(-1) {
  g_cur_name = name;
  g_cur_stream = s;
  g_cur_set = true;
  TraceState& t = g_trace;
  if (!t.on) return;
  if (t.used >= (int)t.pool.size()) {
    t.dropped++;
    return;
  }
  slot_ = t.used++;
  t.pool[slot_].name = name;
  (void)hipEventRecord(t.pool[slot_].begin, s);
}

TraceScope::~TraceScope() {
  g_cur_set = false;
  if (slot_ >= 0) (void)hipEventRecord(g_trace.pool[slot_].end, stream_);
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

int fp8mlp_timing_start(int capacity) {
  FP8MLP_REQUIRE(capacity > 0 && capacity <= (1 << 20), FP8MLP_E_ARG);
  TraceState& t = g_trace;
  while ((int)t.pool.size() < capacity) {
    Rec r{nullptr, nullptr, nullptr};
    FP8MLP_TRY(hip_status(hipEventCreate(&r.begin)));
    if (hipEventCreate(&r.end) != hipSuccess) {
      (void)hipEventDestroy(r.begin);
      return FP8MLP_E_HIP;
    }
    t.pool.push_back(r);
  }
  t.used = 0;
  t.dropped = 0;
  t.on = true;
  return FP8MLP_OK;
}

int fp8mlp_timing_stop(void) {
  g_trace.on = false;
  return g_trace.used;
}

int fp8mlp_timing_get(int i, const char** name, float* ms) {
  TraceState& t = g_trace;
  FP8MLP_REQUIRE(i >= 0 && i < t.used, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(name && ms, FP8MLP_E_NULL);
  *name = t.pool[i].name;
  return hip_status(hipEventElapsedTime(ms, t.pool[i].begin, t.pool[i].end));
}

int fp8mlp_timing_dropped(void) { return g_trace.dropped; }

const char* fp8mlp_last_failed_kernel(void) { return g_failed_kernel; }

}  // extern "C"
