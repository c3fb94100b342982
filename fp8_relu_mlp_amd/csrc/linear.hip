// fp8_linear: FP8 forward projection ("NanoGPT Speedrun (Track 1)", "Changes
// vs Record #83" item 1: QKV and output projections in float8_e4m3 on the
// forward pass, weights stored transposed).
//
// Two launches: a bandwidth-bound pass quantises the bf16 activation once
// (e4m3, RNE, saturating; optionally also max |X|), then the e4m3 MFMA GEMM
// reads the quantised copy.  Quantising inside the GEMM instead would repeat
// the conversion in every one of the N / BN column blocks that share an
// activation tile, and on CDNA4 that conversion is vector-ALU work the
// matrix cores cannot hide.
#include "launch.h"

namespace fp8mlp {

// Xq [M,K] e4m3 . Wt_q [K,N] e4m3 (transposing LDS reads)
using CfgLin = GemmCfg<1, 192, 128, 128, 2, 2, KC, MNC>;

// Xq = e4m3(fp32(X * s)); 16 elements per thread and step.  With `partial`,
// block b also writes the maximum of |X| over the elements it converted to
// partial[b] (fp32 bit pattern), for the consumer to finish the reduction.
__global__ void __launch_bounds__(256) k_quantize(const uint16_t* __restrict__ X, int64_t n16,
                                                  const float* __restrict__ scale, uint8_t* __restrict__ Xq,
                                                  uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  const float s = *scale;
  uint32_t mx = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const i32x4 a = __builtin_nontemporal_load((const i32x4*)X + 2 * i);
    const i32x4 b = __builtin_nontemporal_load((const i32x4*)X + 2 * i + 1);
    uint32_t w[8] = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3],
                     (uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
    i32x4 q;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      mx = max_abs_bf16x2(mx, w[2 * j]);
      mx = max_abs_bf16x2(mx, w[2 * j + 1]);
      q[j] = (int)pack_e4m3x4(bf16_lo(w[2 * j]) * s, bf16_hi(w[2 * j]) * s, bf16_lo(w[2 * j + 1]) * s,
                              bf16_hi(w[2 * j + 1]) * s);
    }
    *((i32x4*)Xq + i) = q;
  }
  if (partial) {
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m01 = red[0] > red[1] ? red[0] : red[1], m23 = red[2] > red[3] ? red[2] : red[3];
      partial[blockIdx.x] = m01 > m23 ? m01 : m23;
    }
  }
}

// The same conversion into rows of Kp >= K codes: X [rows, K] -> Xq [rows, Kp],
// codes K .. Kp - 1 of each row zero (K, Kp multiples of 16).
__global__ void __launch_bounds__(256) k_quantize_rows(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                       int64_t Kp, const float* __restrict__ scale,
                                                       uint8_t* __restrict__ Xq, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  const float s = *scale;
  const int64_t cr = K / 16, cp = Kp / 16, n16 = rows * cp;
  uint32_t mx = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cp, c = i - r * cp;
    i32x4 q = {0, 0, 0, 0};
    if (c < cr) {
      const i32x4* src = (const i32x4*)(X + r * K) + 2 * c;
      const i32x4 a = __builtin_nontemporal_load(src);
      const i32x4 b = __builtin_nontemporal_load(src + 1);
      uint32_t w[8] = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3],
                       (uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        mx = max_abs_bf16x2(mx, w[2 * j]);
        mx = max_abs_bf16x2(mx, w[2 * j + 1]);
        q[j] = (int)pack_e4m3x4(bf16_lo(w[2 * j]) * s, bf16_hi(w[2 * j]) * s, bf16_lo(w[2 * j + 1]) * s,
                                bf16_hi(w[2 * j + 1]) * s);
      }
    }
    *((i32x4*)Xq + i) = q;
  }
  if (partial) {
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m01 = red[0] > red[1] ? red[0] : red[1], m23 = red[2] > red[3] ? red[2] : red[3];
      partial[blockIdx.x] = m01 > m23 ? m01 : m23;
    }
  }
}

int launch_quantize(const uint16_t* X, int64_t n, const float* scale, uint8_t* Xq, uint32_t* partial,
                    int64_t* count, hipStream_t st) {
  *count = 0;
  if (n == 0) return FP8MLP_OK;
  const int64_t n16 = n / 16;
  int64_t blocks = cdiv(n16, 256 * 4);
  if (blocks > kQuantBlocks) blocks = kQuantBlocks;
  TraceScope trace("quantize_e4m3", st);
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, st, X, n16, scale, Xq, partial);
  *count = blocks;
  return launch_status();
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

// K rounded up to whole e4m3 k-tiles (128 codes): the row length of Xq.
static int64_t lin_kp(int64_t K) { return cdiv(K, 128) * 128; }

size_t fp8_linear_workspace(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return align_up((size_t)(M * lin_kp(K)), 256) + quantize_partial_bytes();
}

int fp8_linear(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv_scale,
               uint16_t* Y, float* x_amax_out, int64_t M, int64_t K, int64_t N, void* workspace,
               size_t workspace_bytes, void* stream) {
  FP8MLP_REQUIRE(M >= 0 && K > 0 && N > 0 && K % 64 == 0 && N % 64 == 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(x_scale && w_inv_scale && Wt_q, FP8MLP_E_NULL);
  // block 0 of the GEMM writes x_amax_out while its other blocks read the scales
  FP8MLP_REQUIRE(x_amax_out != x_scale && x_amax_out != w_inv_scale, FP8MLP_E_ARG);
  if (M > 0) FP8MLP_REQUIRE(X && Y, FP8MLP_E_NULL);
  for (const void* p : {(const void*)X, (const void*)Wt_q, (const void*)Y})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  for (const void* p : {(const void*)x_scale, (const void*)w_inv_scale, (const void*)x_amax_out})
    FP8MLP_REQUIRE(((uintptr_t)p & 3) == 0, FP8MLP_E_ALIGN);
  const size_t need = fp8_linear_workspace(M, K);
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (M == 0) {
    // nothing to convert: max |X| over no elements is 0
    return x_amax_out ? launch_max_small(nullptr, 0, x_amax_out, nullptr, 0.0f, nullptr, st) : FP8MLP_OK;
  }
  // K not a multiple of the 128-code k-tile: Xq rows padded with zero codes
  // to Kp, and the loads of Wt_q rows past K return zeros
  const int64_t Kp = lin_kp(K);
  uint8_t* Xq = (uint8_t*)workspace;
  uint32_t* xpart = (uint32_t*)((uint8_t*)workspace + align_up((size_t)(M * Kp), 256));
  int64_t nx = 0;
  if (Kp == K) {
    FP8MLP_TRY(launch_quantize(X, M * K, x_scale, Xq, x_amax_out ? xpart : nullptr, &nx, st));
  } else {
    int64_t blocks = cdiv(M * Kp / 16, 256 * 4);
    if (blocks > kQuantBlocks) blocks = kQuantBlocks;
    TraceScope trace("quantize_e4m3", st);
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, st, X, M, K, Kp, x_scale, Xq,
                       x_amax_out ? xpart : nullptr);
    FP8MLP_TRY(launch_status());
    nx = blocks;
  }
  GemmArgs a{Xq, Kp, Wt_q, N, M, N, Kp, (int)cdiv(M, CfgLin::BM), (int)cdiv(N, CfgLin::BN), 1, Kp, 0};
  a.p_rows = K;
  if (x_amax_out) {
    // block 0 of the GEMM finishes max |X| from the conversion's partial maxima
    a.red_in = xpart;
    a.red_n = nx;
    a.red_out = x_amax_out;
  }
  EpiBf16Out epi{Y, N, 2, nullptr, 0.0f, x_scale, w_inv_scale};
  return launch_gemm<CfgLin, KID_LINEAR>(a, epi, st);
}

}  // extern "C"
