// Matrix-core rate probe (a measurement aid, not part of the method).
//
// The published MI355X peaks assume the 2.4 GHz boost clock.  Under a dense
// MFMA load the clock falls with the switching activity of the operands, so
// the rate a GEMM can reach depends on the data it multiplies.  This kernel
// issues nothing but independent MFMAs on operand registers filled from the
// caller's data (e.g. the benchmark's own X and W1), so the benchmark can
// report the matrix-core rate the chip sustains on that data alongside the
// published figure.  Each wave keeps 16 accumulators of 32 x 32 and runs
// `iters` rounds of 16 MFMAs.
#include <type_traits>

#include "common.h"
#include "host.h"

namespace fp8mlp {

template <int ELT>
__global__ void __launch_bounds__(256, 1) k_mfma_probe(const i32x4* __restrict__ a, int64_t na,
                                                       const i32x4* __restrict__ b, int64_t nb, int iters,
                                                       float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  using Frag = typename std::conditional<ELT == 2, bf16x8_t, i32x8>::type;
  Frag fa[4], fb[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    // 16 (bf16) or 32 (e4m3) bytes per lane and fragment, taken modulo the buffers
    if constexpr (ELT == 2) {
      fa[i] = __builtin_bit_cast(bf16x8_t, a[((w * 4 + i) * 64 + lane) % na]);
      fb[i] = __builtin_bit_cast(bf16x8_t, b[((w * 4 + i) * 64 + lane) % nb]);
    } else {
      const i32x4 a0 = a[((w * 8 + 2 * i) * 64 + lane) % na], a1 = a[((w * 8 + 2 * i + 1) * 64 + lane) % na];
      const i32x4 b0 = b[((w * 8 + 2 * i) * 64 + lane) % nb], b1 = b[((w * 8 + 2 * i + 1) * 64 + lane) % nb];
      fa[i] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      fb[i] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (ELT == 2) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
        }
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) s += acc[i][j][0];
  sink[w * 64 + lane] = s;
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

int fp8mlp_mfma_probe(int dtype, const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, int64_t iters,
                      float* sink, void* stream) {
  FP8MLP_REQUIRE(dtype == FP8MLP_MFMA_BF16 || dtype == FP8MLP_MFMA_E4M3, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(a_bytes >= 16 && b_bytes >= 16 && iters > 0 && iters <= (1 << 24), FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(a && b && sink, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(aligned16(a) && aligned16(b) && ((uintptr_t)sink & 3) == 0, FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  TraceScope trace("mfma_probe", st);
  if (dtype == FP8MLP_MFMA_BF16) {
    hipLaunchKernelGGL(k_mfma_probe<2>, dim3(FP8MLP_PROBE_BLOCKS), dim3(256), 0, st, (const i32x4*)a, a_bytes / 16,
                       (const i32x4*)b, b_bytes / 16, (int)iters, sink);
  } else {
    hipLaunchKernelGGL(k_mfma_probe<1>, dim3(FP8MLP_PROBE_BLOCKS), dim3(256), 0, st, (const i32x4*)a, a_bytes / 16,
                       (const i32x4*)b, b_bytes / 16, (int)iters, sink);
  }
  return launch_status();
}

}  // extern "C"
