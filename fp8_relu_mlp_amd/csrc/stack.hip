// Layer-stack helpers around the MLP block: weightless RMSNorm (forward and
// backward fused with the residual-stream gradient), the bf16 residual add
// and the SGD weight update.
//
// The speedrun pages run the MLP block inside a pre-norm transformer whose
// FP8 state is carried per layer from step to step ("A Retrospective on Our
// World Records", Main Track: delayed scaling from amax(t-1), the transposed
// FP8 W2 cache refreshed after each optimizer update).  These kernels let the
// block be trained as a stack of layers; they are bandwidth-bound elementwise
// and row-reduction passes, one 64-lane wave per row.
//   rmsnorm:  r = 1 / sqrt(mean(x^2) + eps);  xn = bf16(x * r)
//   backward: g_out = bf16(g_in + r * (dxn - xh * mean(dxn * xh))),  xh = x * r
//   add:      out = bf16(a + b)
//   SGD:      W = bf16(W - fp32(lr * dW))
// Sums of a row are taken in fp32; the square root and the quotients are IEEE
// (the library is built with correctly rounded fp32 division and sqrt).
#include "common.h"
#include "host.h"

namespace fp8mlp {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void unpack8(const uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x), f[1] = bf16_hi(w.x), f[2] = bf16_lo(w.y), f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z), f[5] = bf16_hi(w.z), f[6] = bf16_lo(w.w), f[7] = bf16_hi(w.w);
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return uint4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// One wave per row; each lane handles 16-byte chunks (8 values) at stride 64.
__global__ void __launch_bounds__(256) k_rmsnorm_fwd(const uint4* __restrict__ x, uint4* __restrict__ xn,
                                                     float* __restrict__ inv_rms, int64_t M, int chunks,
                                                     float fd, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const uint4* xr = x + row * chunks;
  float ss = 0.0f;
  for (int c = lane; c < chunks; c += 64) {
    float f[8];
    unpack8(xr[c], f);
#pragma unroll
    for (int i = 0; i < 8; i++) ss += f[i] * f[i];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / fd + eps);
  if (lane == 0) inv_rms[row] = r;
  uint4* outr = xn + row * chunks;
  for (int c = lane; c < chunks; c += 64) {
    float f[8];
    unpack8(xr[c], f);
#pragma unroll
    for (int i = 0; i < 8; i++) f[i] *= r;
    outr[c] = pack8(f);
  }
}

__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const uint4* __restrict__ x, const float* __restrict__ inv_rms,
                                                     const uint4* __restrict__ dxn, const uint4* __restrict__ g_in,
                                                     uint4* __restrict__ g_out, int64_t M, int chunks, float fd) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const float r = inv_rms[row];
  const uint4 *xr = x + row * chunks, *dr = dxn + row * chunks;
  float dot = 0.0f;
  for (int c = lane; c < chunks; c += 64) {
    float a[8], b[8];
    unpack8(xr[c], a);
    unpack8(dr[c], b);
#pragma unroll
    for (int i = 0; i < 8; i++) dot += b[i] * (a[i] * r);
  }
  const float mean = wave_sum(dot) / fd;
  const uint4* gr = g_in + row * chunks;
  uint4* outr = g_out + row * chunks;
  for (int c = lane; c < chunks; c += 64) {
    float a[8], b[8], g[8];
    unpack8(xr[c], a);
    unpack8(dr[c], b);
    unpack8(gr[c], g);
#pragma unroll
    for (int i = 0; i < 8; i++) g[i] += r * (b[i] - (a[i] * r) * mean);
    outr[c] = pack8(g);
  }
}

__global__ void __launch_bounds__(256) k_add_bf16(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                  uint4* __restrict__ out, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float fa[8], fb[8];
    unpack8(a[i], fa);
    unpack8(b[i], fb);
#pragma unroll
    for (int k = 0; k < 8; k++) fa[k] += fb[k];
    out[i] = pack8(fa);
  }
}

__global__ void __launch_bounds__(256) k_sgd_bf16(uint4* __restrict__ W, const float4* __restrict__ dW, int64_t n8,
                                                  float lr) {
  // two roundings, as specified: fp32(lr * dW), then fp32(W - step)
#pragma clang fp contract(off)
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float w[8];
    unpack8(W[i], w);
    const float4 g0 = dW[2 * i], g1 = dW[2 * i + 1];
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float step = lr * g[k];
      w[k] = w[k] - step;
    }
    W[i] = pack8(w);
  }
}

static unsigned grid_for(int64_t n, int64_t per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  if (b > 8192) b = 8192;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

int rmsnorm_fwd(const uint16_t* x, uint16_t* xn, float* inv_rms, int64_t M, int64_t d, float eps, void* stream) {
  FP8MLP_REQUIRE(M >= 0 && d > 0 && d % 8 == 0 && d <= (int64_t)1 << 24, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(eps >= 0.0f && eps <= 3.4e38f, FP8MLP_E_ARG);
  if (M == 0) return FP8MLP_OK;
  FP8MLP_REQUIRE(x && xn && inv_rms, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(aligned16(x) && aligned16(xn) && ((uintptr_t)inv_rms & 3) == 0, FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  TraceScope trace("rmsnorm_fwd", st);
  hipLaunchKernelGGL(k_rmsnorm_fwd, dim3((unsigned)cdiv(M, 4)), dim3(256), 0, st, (const uint4*)x, (uint4*)xn,
                     inv_rms, M, (int)(d / 8), (float)d, eps);
  return launch_status();
}

int rmsnorm_bwd(const uint16_t* x, const float* inv_rms, const uint16_t* dxn, const uint16_t* g_in, uint16_t* g_out,
                int64_t M, int64_t d, void* stream) {
  FP8MLP_REQUIRE(M >= 0 && d > 0 && d % 8 == 0 && d <= (int64_t)1 << 24, FP8MLP_E_SHAPE);
  if (M == 0) return FP8MLP_OK;
  FP8MLP_REQUIRE(x && inv_rms && dxn && g_in && g_out, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(aligned16(x) && aligned16(dxn) && aligned16(g_in) && aligned16(g_out) &&
                     ((uintptr_t)inv_rms & 3) == 0,
                 FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  TraceScope trace("rmsnorm_bwd", st);
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3((unsigned)cdiv(M, 4)), dim3(256), 0, st, (const uint4*)x, inv_rms,
                     (const uint4*)dxn, (const uint4*)g_in, (uint4*)g_out, M, (int)(d / 8), (float)d);
  return launch_status();
}

int add_bf16(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n, void* stream) {
  FP8MLP_REQUIRE(n >= 0 && n % 8 == 0, FP8MLP_E_SHAPE);
  if (n == 0) return FP8MLP_OK;
  FP8MLP_REQUIRE(a && b && out, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(aligned16(a) && aligned16(b) && aligned16(out), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  TraceScope trace("add_bf16", st);
  hipLaunchKernelGGL(k_add_bf16, dim3(grid_for(n / 8, 256)), dim3(256), 0, st, (const uint4*)a, (const uint4*)b,
                     (uint4*)out, n / 8);
  return launch_status();
}

int sgd_update_bf16(uint16_t* W, const float* dW, int64_t n, float lr, void* stream) {
  FP8MLP_REQUIRE(n >= 0 && n % 8 == 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(lr == lr && lr >= -3.4e38f && lr <= 3.4e38f, FP8MLP_E_ARG);
  if (n == 0) return FP8MLP_OK;
  FP8MLP_REQUIRE(W && dW, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(aligned16(W) && aligned16(dW), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  TraceScope trace("sgd_update_bf16", st);
  hipLaunchKernelGGL(k_sgd_bf16, dim3(grid_for(n / 8, 256)), dim3(256), 0, st, (uint4*)W, (const float4*)dW, n / 8,
                     lr);
  return launch_status();
}

}  // extern "C"
