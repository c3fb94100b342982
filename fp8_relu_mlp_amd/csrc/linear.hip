// fp8_linear: FP8 forward projection with the activation quantised inside the
// GEMM ("NanoGPT Speedrun (Track 1)", "Changes vs Record #83" item 1: QKV and
// output projections in float8_e4m3 on the forward pass, weights stored
// transposed).  The bf16 activation tile is loaded into LDS, scaled and
// encoded to e4m3 there, and fed to the e4m3 MFMA; it never goes back to HBM.
#include "launch.h"

namespace fp8mlp {

// X [M,K] bf16 (quantised on load) . Wt_q [K,N] e4m3 (transposing LDS reads)
using CfgLin = GemmCfg<1, 128, 256, 2, KC, MNC, true>;

__global__ void k_zero_scalar(float* p) { *p = 0.0f; }

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

int fp8_linear(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv_scale,
               uint16_t* Y, float* x_amax_out, int64_t M, int64_t K, int64_t N, void* stream) {
  FP8MLP_REQUIRE(M >= 0 && K > 0 && N > 0 && K % 128 == 0 && N % 64 == 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(x_scale && w_inv_scale && Wt_q, FP8MLP_E_NULL);
  if (M > 0) FP8MLP_REQUIRE(X && Y, FP8MLP_E_NULL);
  for (const void* p : {(const void*)X, (const void*)Wt_q, (const void*)Y})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  for (const void* p : {(const void*)x_scale, (const void*)w_inv_scale, (const void*)x_amax_out})
    FP8MLP_REQUIRE(((uintptr_t)p & 3) == 0, FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (x_amax_out) {
    hipLaunchKernelGGL(k_zero_scalar, dim3(1), dim3(1), 0, st, x_amax_out);
    FP8MLP_TRY(launch_status());
  }
  GemmArgs a{X, K, Wt_q, N, M, N, K, (int)cdiv(M, CfgLin::BM), (int)cdiv(N, CfgLin::BN), 1, K, x_scale};
  EpiBf16Out epi{Y, N, 2, nullptr, 0.0f, x_scale, w_inv_scale, x_amax_out};
  return launch_gemm<CfgLin>(a, epi, st);
}

}  // extern "C"
