// Host-side helpers of libfp8mlp: status handling, argument validation,
// device architecture check and launch error capture.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fp8mlp.h"

namespace fp8mlp {

// hipError_t of the last failed HIP call on this thread.
extern thread_local int g_last_hip_error;

// FP8MLP_OK when the current device is gfx950, FP8MLP_E_ARCH otherwise,
// FP8MLP_E_HIP if the device cannot be queried.  Cached per device.
int check_device();
// Compute units of the current device (256 on MI355X; cached per device).
int num_cus();

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return FP8MLP_OK;
  g_last_hip_error = (int)e;
  return FP8MLP_E_HIP;
}
// FP8MLP_SYNC_CHECK=1 debug mode (trace.hip): after a launch, wait for the
// launching stream and report a failure of that kernel as FP8MLP_E_HIP,
// naming it for fp8mlp_last_failed_kernel().
int sync_check();
bool sync_check_on();
// Status of the most recent kernel launch on this thread.
inline int launch_status() {
  const int st = hip_status(hipGetLastError());
  return st == FP8MLP_OK && sync_check_on() ? sync_check() : st;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The GEMMs address memory through buffer resources with 32-bit byte
// offsets: from a tile's origin across its rows (up to 256 rows of a matrix
// whose rows hold a feature size of elements), and across a whole weight
// matrix where the weight is the row-contiguous operand.  Feature sizes up to
// 2^22 and weights below 2^31 elements keep both inside 2^32 bytes.
constexpr int64_t kMaxFeature = (int64_t)1 << 22;
inline bool weight_dims_ok(int64_t rows, int64_t cols) {
  return rows <= kMaxFeature && cols <= kMaxFeature && rows * cols < ((int64_t)1 << 31);
}
// Rows of a row-contiguous operand that one GEMM launch may address in a
// single k range: rows of row_bytes bytes within 2^31 bytes, a multiple of
// 64 (the split-k granule).
inline int64_t max_k_range(int64_t row_bytes) {
  const int64_t r = (((int64_t)1 << 31) / row_bytes) / 64 * 64;
  return r > 64 ? r : 64;
}

#define FP8MLP_TRY(...)                  \
  do {                                   \
    int _st = (__VA_ARGS__);             \
    if (_st != FP8MLP_OK) return _st;    \
  } while (0)
#define FP8MLP_REQUIRE(cond, status)     \
  do {                                   \
    if (!(cond)) return (status);        \
  } while (0)

// Brackets one kernel launch with timing events while fp8mlp_timing_start is
// in effect on this thread (trace.hip); a no-op otherwise.
class TraceScope {
 public:
  TraceScope(const char* name, hipStream_t s);
  ~TraceScope();

 private:
  hipStream_t stream_;
  int slot_;
};

// Shared launchers (defined in abi.hip) used by several entry points.
// Reduce n fp32 values that are >= +0 or NaN to their maximum, written to
// out (and, if scale_out is given, the delayed scale from amax_prev/margin).
int launch_max_small(const float* x, int64_t n, float* out, const float* amax_prev, float margin,
                     float* scale_out, hipStream_t stream);
int launch_amax(int dtype, const void* x, int64_t n, float* out, void* workspace, size_t ws_bytes,
                hipStream_t stream);
size_t amax_ws_bytes(int64_t n);
// Xq = e4m3(fp32(X * *scale)) over n elements (a multiple of 128) in at
// most kQuantBlocks blocks (linear.hip).  When partial is given, block b
// writes max |X| over its elements to partial[b]; *count receives the number
// of blocks (0 for n = 0, which launches nothing).
// out[i] = (accumulate ? out[i] : 0) + sum of the split partials part[s * n + i]
// in split order; out[0 .. n) = 0 (n a multiple of 4; mlp_bwd.hip).
int launch_reduce(const float* part, int splits, int64_t n, float* out, int accumulate, hipStream_t st);
int launch_zero(float* out, int64_t n, hipStream_t st);
constexpr int kQuantBlocks = 4096;
constexpr size_t quantize_partial_bytes() { return (size_t)kQuantBlocks * 4; }
int launch_quantize(const uint16_t* X, int64_t n, const float* scale, uint8_t* Xq, uint32_t* partial,
                    int64_t* count, hipStream_t stream);

}  // namespace fp8mlp
