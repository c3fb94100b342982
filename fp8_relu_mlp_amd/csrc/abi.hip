// libfp8mlp: status / version / device check, the amax reduction, the scale
// computation and the FP8 weight cast-transpose.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "common.h"
#include "host.h"

namespace fp8mlp {

thread_local int g_last_hip_error = 0;

// ------------------------------------------------------------------ device check
namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
}  // namespace

int check_device() {
  int dev = 0;
  FP8MLP_TRY(hip_status(hipGetDevice(&dev)));
  if (dev < 0 || dev >= kMaxDevices) return FP8MLP_E_ARCH;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    FP8MLP_TRY(hip_status(hipGetDeviceProperties(&prop, dev)));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? FP8MLP_OK : FP8MLP_E_ARCH;
}

namespace {
std::atomic<int> g_dev_cus[kMaxDevices];
}  // namespace

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_dev_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_dev_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ------------------------------------------------------------------ amax
// Maximum of |x| taken on bit patterns: for fp32, |x| bits order like the
// values (+0 < ... < +inf < NaN), so the unsigned maximum is exact, NaN
// propagating and independent of the reduction order.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t m = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); i++) m = red[i] > m ? red[i] : m;
  return m;
}

template <int DT>
__global__ void __launch_bounds__(256) k_amax_partial(const void* __restrict__ x, int64_t n,
                                                      uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  constexpr int PER = DT == FP8MLP_F32 ? 4 : 8;  // elements per 16-byte vector
  const int64_t nv = n / PER;
  const i32x4* v = (const i32x4*)x;
  for (int64_t i = tid; i < nv; i += stride) {
    const i32x4 q = __builtin_nontemporal_load(v + i);
    const uint32_t w[4] = {(uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if constexpr (DT == FP8MLP_F32) {
        uint32_t a = w[j] & 0x7fffffffu;
        m = a > m ? a : m;
      } else {
        uint32_t a0 = (w[j] & 0x7fffu) << 16, a1 = (w[j] >> 16 & 0x7fffu) << 16;
        m = a0 > m ? a0 : m;
        m = a1 > m ? a1 : m;
      }
    }
  }
  for (int64_t i = nv * PER + tid; i < n; i += stride) {
    uint32_t a;
    if constexpr (DT == FP8MLP_F32) a = ((const uint32_t*)x)[i] & 0x7fffffffu;
    else a = (uint32_t)(((const uint16_t*)x)[i] & 0x7fffu) << 16;
    m = a > m ? a : m;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// One block: max over n unsigned |x| bit patterns -> out (as fp32).
// Optionally writes the delayed scale computed from *amax_prev and margin.
__global__ void __launch_bounds__(256) k_max_final(const uint32_t* __restrict__ bits, int64_t n, float* out,
                                                   const float* amax_prev, float margin, float* scale_out) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    uint32_t a = bits[i] & 0x7fffffffu;
    m = a > m ? a : m;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) {
    *out = __uint_as_float(m);
    if (scale_out) *scale_out = scale_from_amax(*amax_prev, margin);
  }
}

// Direct single-block amax of a small tensor.
template <int DT>
__global__ void __launch_bounds__(256) k_amax_small(const void* __restrict__ x, int64_t n, float* out) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    uint32_t a;
    if constexpr (DT == FP8MLP_F32) a = ((const uint32_t*)x)[i] & 0x7fffffffu;
    else a = (uint32_t)(((const uint16_t*)x)[i] & 0x7fffu) << 16;
    m = a > m ? a : m;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) *out = __uint_as_float(m);
}

constexpr int64_t kAmaxSmall = 1 << 16;
constexpr int kAmaxBlocks = 2048;

size_t amax_ws_bytes(int64_t n) { return n <= kAmaxSmall ? 0 : (size_t)kAmaxBlocks * 4; }

int launch_max_small(const float* x, int64_t n, float* out, const float* amax_prev, float margin,
                     float* scale_out, hipStream_t stream) {
  TraceScope trace("amax_final", stream);
  hipLaunchKernelGGL(k_max_final, dim3(1), dim3(256), 0, stream, (const uint32_t*)x, n, out, amax_prev, margin,
                     scale_out);
  return launch_status();
}

int launch_amax(int dtype, const void* x, int64_t n, float* out, void* workspace, size_t ws_bytes,
                hipStream_t stream) {
  if (n <= kAmaxSmall) {
    TraceScope trace("amax_small", stream);
    if (dtype == FP8MLP_F32)
      hipLaunchKernelGGL(k_amax_small<FP8MLP_F32>, dim3(1), dim3(256), 0, stream, x, n, out);
    else
      hipLaunchKernelGGL(k_amax_small<FP8MLP_BF16>, dim3(1), dim3(256), 0, stream, x, n, out);
    return launch_status();
  }
  const int per = dtype == FP8MLP_F32 ? 4 : 8;
  int64_t blocks = cdiv(cdiv(n, per), 256 * 4);
  if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;
  uint32_t* partial = (uint32_t*)workspace;
  {
    TraceScope trace("amax_partial", stream);
    if (dtype == FP8MLP_F32)
      hipLaunchKernelGGL(k_amax_partial<FP8MLP_F32>, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, partial);
    else
      hipLaunchKernelGGL(k_amax_partial<FP8MLP_BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, partial);
  }
  FP8MLP_TRY(launch_status());
  TraceScope trace("amax_final", stream);
  hipLaunchKernelGGL(k_max_final, dim3(1), dim3(256), 0, stream, (const uint32_t*)partial, blocks, out,
                     (const float*)nullptr, 0.0f, (float*)nullptr);
  return launch_status();
}

// First phase of an amax whose consumer finishes the reduction itself:
// writes |x| maxima as fp32 bit patterns to partial[0 .. *count) (one value
// for small tensors, one per block otherwise).  partial needs
// max(4, amax_ws_bytes(n)) bytes.
int launch_amax_partials(int dtype, const void* x, int64_t n, uint32_t* partial, int* count, hipStream_t stream) {
  if (n <= kAmaxSmall) {
    *count = 1;
    TraceScope trace("amax_small", stream);
    if (dtype == FP8MLP_F32)
      hipLaunchKernelGGL(k_amax_small<FP8MLP_F32>, dim3(1), dim3(256), 0, stream, x, n, (float*)partial);
    else
      hipLaunchKernelGGL(k_amax_small<FP8MLP_BF16>, dim3(1), dim3(256), 0, stream, x, n, (float*)partial);
    return launch_status();
  }
  const int per = dtype == FP8MLP_F32 ? 4 : 8;
  int64_t blocks = cdiv(cdiv(n, per), 256 * 4);
  if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;
  *count = (int)blocks;
  TraceScope trace("amax_partial", stream);
  if (dtype == FP8MLP_F32)
    hipLaunchKernelGGL(k_amax_partial<FP8MLP_F32>, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, partial);
  else
    hipLaunchKernelGGL(k_amax_partial<FP8MLP_BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, partial);
  return launch_status();
}

// ------------------------------------------------------------------ scale
__global__ void k_scale_from_amax(const float* amax, float margin, float* scale_out, float* inv_out) {
  const float s = scale_from_amax(*amax, margin);
  if (scale_out) *scale_out = s;
  if (inv_out) *inv_out = 1.0f / s;
}

// ------------------------------------------------------------------ cast-transpose
// bf16 W [N, K] -> e4m3 Wt [K, N] in 128 (n) x kCtBK (k) tiles.  Thread t
// loads a 4 x (kCtBK / 8) block (rows 4 (t / 8) .. +3, columns
// (kCtBK / 8) (t % 8) ..: 2 kCtBK bytes of a row per 8 lanes), casts it,
// transposes it in registers to words of 4 n each and writes those to LDS
// with 4-byte stores; the tile leaves in rows of 128 codes (16 bytes per
// lane).  LDS image: row k of 32 words, word c at c ^ (8 ((k / 8) & 3)), so a
// wave's writes reach 32 banks each twice and its 16-byte reads are
// conflict-free.  Consecutive blocks take consecutive n-tiles: their rows of
// Wt continue each other.  The scale is read from scale_in, or computed as
// 448 / amax (exact policy) from the maxima in amax_part.
constexpr int kCtBN = 128, kCtBK = 64, kCtKT = kCtBK / 8;

__device__ __forceinline__ uint32_t ct_word(int k, int c) { return (uint32_t)(k * 32 + (c ^ (((k >> 3) & 3) << 3))); }

__global__ void __launch_bounds__(256) k_cast_transpose(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                        uint8_t* __restrict__ Wt, const float* scale_in,
                                                        const uint32_t* amax_part, int npart, float* scale_out,
                                                        float* inv_out, float* amax_out) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[kCtBK * 32];
  __shared__ uint32_t red[4];
  const int tid = (int)threadIdx.x;
  float amax = 0.0f;
  if (amax_part) {
    uint32_t m = 0;
    for (int i = tid; i < npart; i += 256) m = amax_part[i] > m ? amax_part[i] : m;
    amax = __uint_as_float(block_max_u32(m, red));
  }
  const float s = scale_in ? *scale_in : scale_from_amax(amax, 1.0f);
  const int64_t n0 = (int64_t)blockIdx.x * kCtBN, k0 = (int64_t)blockIdx.y * kCtBK;
  const int rg = tid >> 3, kg = tid & 7;
  // 1. the block, cast: w[r][h] holds columns kCtKT kg + 4 h .. +3 of row 4 rg + r
  uint32_t w[4][kCtKT / 4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int64_t n = n0 + 4 * rg + r;
#pragma unroll
    for (int q = 0; q < kCtKT / 8; q++) {
      const int64_t k = k0 + kCtKT * kg + 8 * q;
      uint4 v = uint4{0, 0, 0, 0};
      if (n < N && k < K) v = *(const uint4*)(W + n * K + k);
      w[r][2 * q] = pack_e4m3x4(bf16_lo(v.x) * s, bf16_hi(v.x) * s, bf16_lo(v.y) * s, bf16_hi(v.y) * s);
      w[r][2 * q + 1] = pack_e4m3x4(bf16_lo(v.z) * s, bf16_hi(v.z) * s, bf16_lo(v.w) * s, bf16_hi(v.w) * s);
    }
  }
  // 2. transposed: column kCtKT kg + j, rows 4 rg .. +3 -> one word
#pragma unroll
  for (int j = 0; j < kCtKT; j++) {
    const int h = j >> 2, b = 8 * (j & 3);
    const uint32_t o = ((w[0][h] >> b) & 0xffu) | (((w[1][h] >> b) & 0xffu) << 8) | (((w[2][h] >> b) & 0xffu) << 16) |
                       (((w[3][h] >> b) & 0xffu) << 24);
    tile[ct_word(kCtKT * kg + j, rg)] = o;
  }
  __syncthreads();
  // 3. rows of Wt: kCtBK k x 8 chunks of 16 n
#pragma unroll
  for (int it = 0; it < kCtBK / 32; it++) {
    const int i = tid + it * 256, k = i >> 3, ch = i & 7;
    const int64_t kk = k0 + k, n = n0 + ch * 16;
    const uint4 v = *(const uint4*)&tile[ct_word(k, 4 * ch)];
    if (kk < K && n < N) *(uint4*)(Wt + kk * N + n) = v;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    if (scale_out) *scale_out = s;
    if (inv_out) *inv_out = 1.0f / s;
    if (amax_out) *amax_out = amax;
  }
}

// ------------------------------------------------------------------ saturation count
// Number of e4m3 codes of magnitude 448 (0x7E, 0xFE): the top code, which every
// value from 432 up (after scaling) receives, clipped or not.  Per-block
// counts go to partial[], a one-block pass adds them up.
__device__ __forceinline__ uint32_t top_codes_in_word(uint32_t w) {
  const uint32_t y = (w & 0x7f7f7f7fu) ^ 0x7e7e7e7eu;          // byte 0 <=> top code
  const uint32_t nz = ((y & 0x7f7f7f7fu) + 0x7f7f7f7fu) | y;    // bit 7 of a byte: byte != 0
  return (uint32_t)__builtin_popcount(~nz & 0x80808080u);
}

__global__ void __launch_bounds__(256) k_count_top(const i32x4* __restrict__ q, int64_t n16,
                                                   uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  uint32_t c = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const i32x4 v = __builtin_nontemporal_load(q + i);
    c += top_codes_in_word((uint32_t)v[0]) + top_codes_in_word((uint32_t)v[1]) + top_codes_in_word((uint32_t)v[2]) +
         top_codes_in_word((uint32_t)v[3]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ void __launch_bounds__(256) k_sum_counts(const uint32_t* __restrict__ partial, int n,
                                                    unsigned long long* out) {
  __shared__ unsigned long long red[4];
  unsigned long long c = 0;
  for (int i = threadIdx.x; i < n; i += 256) c += partial[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) *out = red[0] + red[1] + red[2] + red[3];
}

constexpr int kCountBlocks = 2048;

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

int fp8mlp_abi_version(void) { return FP8MLP_ABI_VERSION; }

const char* fp8mlp_status_str(int status) {
  switch (status) {
    case FP8MLP_OK: return "ok";
    case FP8MLP_E_NULL: return "a required pointer is NULL";
    case FP8MLP_E_SHAPE: return "invalid size (negative, zero where not allowed, not a multiple of 64, or beyond the 32-bit addressing limits)";
    case FP8MLP_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FP8MLP_E_WORKSPACE: return "workspace missing or too small";
    case FP8MLP_E_ARCH: return "the current device is not gfx950 (MI355X)";
    case FP8MLP_E_HIP: return "a HIP call failed";
    case FP8MLP_E_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

int fp8mlp_last_hip_error(void) { return g_last_hip_error; }

size_t amax_reduce_workspace(int64_t n) { return n < 0 ? 0 : amax_ws_bytes(n); }

int amax_reduce(int dtype, const void* x, int64_t n, float* amax_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  FP8MLP_REQUIRE(dtype == FP8MLP_F32 || dtype == FP8MLP_BF16, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(n >= 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(amax_out && (x || n == 0), FP8MLP_E_NULL);
  FP8MLP_REQUIRE((x == nullptr || aligned16(x)) && ((uintptr_t)amax_out & 3) == 0, FP8MLP_E_ALIGN);
  const size_t need = amax_ws_bytes(n);
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  return launch_amax(dtype, x, n, amax_out, workspace, workspace_bytes, (hipStream_t)stream);
}

int fp8_scale_from_amax(const float* amax, float margin, float* scale_out, float* inv_scale_out, void* stream) {
  FP8MLP_REQUIRE(amax != nullptr, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(margin > 0.0f && margin <= 3.4e38f, FP8MLP_E_ARG);
  FP8MLP_TRY(check_device());
  TraceScope trace("scale_from_amax", (hipStream_t)stream);
  hipLaunchKernelGGL(k_scale_from_amax, dim3(1), dim3(1), 0, (hipStream_t)stream, amax, margin, scale_out,
                     inv_scale_out);
  return launch_status();
}

size_t fp8_cast_transpose_workspace(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return 256 + amax_ws_bytes(N * K);
}

int fp8_cast_transpose(const uint16_t* W, int64_t N, int64_t K, uint8_t* Wt_q, const float* scale_in,
                       float* scale_out, float* inv_scale_out, float* amax_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  FP8MLP_REQUIRE(N > 0 && K > 0 && N % 16 == 0 && K % 16 == 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(W && Wt_q, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(aligned16(W) && aligned16(Wt_q), FP8MLP_E_ALIGN);
  const bool need_amax = scale_in == nullptr || amax_out != nullptr;
  const size_t need = need_amax ? fp8_cast_transpose_workspace(N, K) : 0;
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  uint32_t* part = nullptr;
  int npart = 0;
  if (need_amax) {
    part = N * K <= kAmaxSmall ? (uint32_t*)workspace : (uint32_t*)((char*)workspace + 256);
    FP8MLP_TRY(launch_amax_partials(FP8MLP_BF16, W, N * K, part, &npart, st));
  }
  dim3 grid((unsigned)cdiv(N, kCtBN), (unsigned)cdiv(K, kCtBK));
  if (npart > 1 && (int64_t)grid.x * grid.y * npart > (int64_t)1 << 20) {
    // a large weight: one block finishes the maximum once (into the
    // workspace's first word) instead of every block re-reading the partials
    FP8MLP_TRY(launch_max_small((const float*)part, npart, (float*)workspace, nullptr, 0.0f, nullptr, st));
    part = (uint32_t*)workspace;
    npart = 1;
  }
  TraceScope trace("cast_transpose", st);
  hipLaunchKernelGGL(k_cast_transpose, grid, dim3(256), 0, st, W, N, K, Wt_q, scale_in, (const uint32_t*)part, npart,
                     scale_out, inv_scale_out, amax_out);
  return launch_status();
}

int fp8_cast_transpose_w2(const uint16_t* W2, int64_t d, int64_t h, uint8_t* W2t_q, float* scale_out,
                          float* inv_scale_out, float* amax_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return fp8_cast_transpose(W2, d, h, W2t_q, nullptr, scale_out, inv_scale_out, amax_out, workspace,
                            workspace_bytes, stream);
}

size_t fp8_saturation_count_workspace(int64_t n) { return n <= 0 ? 0 : (size_t)kCountBlocks * 4; }

int fp8_saturation_count(const uint8_t* q, int64_t n, uint64_t* count_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  FP8MLP_REQUIRE(n >= 0 && n % 16 == 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(count_out && (q || n == 0), FP8MLP_E_NULL);
  FP8MLP_REQUIRE((q == nullptr || aligned16(q)) && ((uintptr_t)count_out & 7) == 0, FP8MLP_E_ALIGN);
  const size_t need = fp8_saturation_count_workspace(n);
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  const hipStream_t st = (hipStream_t)stream;
  int64_t blocks = 0;
  if (n > 0) {
    blocks = cdiv(n / 16, 256 * 4);
    if (blocks > kCountBlocks) blocks = kCountBlocks;
    TraceScope trace("count_top_codes", st);
    hipLaunchKernelGGL(k_count_top, dim3((unsigned)blocks), dim3(256), 0, st, (const i32x4*)q, n / 16,
                       (uint32_t*)workspace);
    FP8MLP_TRY(launch_status());
  }
  TraceScope trace("sum_counts", st);
  hipLaunchKernelGGL(k_sum_counts, dim3(1), dim3(256), 0, st, (const uint32_t*)workspace, (int)blocks,
                     (unsigned long long*)count_out);
  return launch_status();
}

}  // extern "C"
