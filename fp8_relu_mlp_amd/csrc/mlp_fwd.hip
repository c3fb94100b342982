// mlp_relu2_fwd: fused up-projection + ReLU^2 + e4m3 quantisation + partial
// amax, the partial-amax reduction, and the FP8 (or, at eval, bf16)
// down-projection.  All launches go to the caller's stream, back to back.
#include <atomic>
#include <mutex>

#include "launch.h"

namespace fp8mlp {

// X [M,d] . W1[h,d]^T : both operands k-contiguous; 256 x 256 tiles, two
// groups of four waves taking turns at the matrix cores, X loaded two k-tiles
// ahead (three X buffers: 160 KB of LDS).
using CfgUp = GemmCfg<2, 256, 256, 128, 2, 1, KC, KC, 0, 8, 0, 3>;
// post_q [M,h] . W2t_q [h,d] : e4m3, the cache is read with transposing LDS
// loads; 192 x 384 two-group tiles (d = 768 is two of them, M = 49152 two
// rounds of 256 blocks; nine MFMAs per phase and wave), two post_q buffers
// (a third does not fit beside the 48 KB W2t_q tiles).
using CfgDown8 = GemmCfg<1, 192, 384, 128, 2, 1, KC, MNC, 0, 8, 0, 2>;
// Xq [M,d] . W1t_q [d,h] : the up-projection in e4m3 (the W1 cache is read
// with transposing LDS loads), 256 x 256 tiles, two groups of four waves,
// three Xq buffers.
using CfgUp8 = GemmCfg<1, 256, 256, 128, 2, 1, KC, MNC, 0, 8, 0, 3>;
// post [M,h] . W2[d,h]^T : bf16 eval path; the same shape as the backward's
// dX GEMM, on the same 192 x 256 two-group tiles with three post buffers.
using CfgDownBf16 = GemmCfg<2, 192, 256, 128, 2, 1, KC, KC, 0, 8, 0, 3>;

struct FwdPlan {
  int64_t tm, tn;          // up-projection tiles
  size_t partial_bytes;
};
static FwdPlan fwd_plan(int64_t M, int64_t h) {
  static_assert(CfgUp::BM == CfgUp8::BM && CfgUp::BN == CfgUp8::BN, "one partial-amax layout");
  FwdPlan p;
  p.tm = cdiv(M, CfgUp::BM);
  p.tn = cdiv(h, CfgUp::BN);
  p.partial_bytes = align_up((size_t)(p.tm * p.tn) * 4, 256);
  return p;
}

// Argument checks of mlp_relu2_fwd that do not involve the workspace.
static int fwd_check_args(int mode, const uint16_t* X, const uint16_t* W1, const uint8_t* W2t_q,
                          const float* w2_inv_scale, const uint16_t* W2, const float* amax_prev, float margin,
                          const uint16_t* post, const uint8_t* post_q, const float* amax_out, const float* scale_out,
                          const uint16_t* Y, int64_t M, int64_t d, int64_t h) {
  const bool train = mode == FP8MLP_TRAIN_FP8;
  FP8MLP_REQUIRE(mode == FP8MLP_TRAIN_FP8 || mode == FP8MLP_EVAL_BF16, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(M >= 0 && d > 0 && h > 0 && d % 64 == 0 && h % 64 == 0 && weight_dims_ok(h, d), FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(!train || h % 128 == 0, FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(amax_out != nullptr, FP8MLP_E_NULL);
  if (M > 0) FP8MLP_REQUIRE(X && W1 && Y && (post || train), FP8MLP_E_NULL);
  if (train) {
    FP8MLP_REQUIRE(amax_prev != nullptr, FP8MLP_E_NULL);
    // block 0 of the down-projection writes amax_out / scale_out while later
    // blocks still read amax_prev: the three must be distinct words
    FP8MLP_REQUIRE(amax_out != amax_prev && scale_out != amax_prev && scale_out != amax_out, FP8MLP_E_ARG);
    if (M > 0) FP8MLP_REQUIRE(W2t_q && w2_inv_scale && post_q, FP8MLP_E_NULL);
    FP8MLP_REQUIRE(margin > 0.0f && margin <= 3.4e38f, FP8MLP_E_ARG);
  } else if (M > 0) {
    FP8MLP_REQUIRE(W2 != nullptr, FP8MLP_E_NULL);
  }
  for (const void* p : {(const void*)X, (const void*)W1, (const void*)W2t_q, (const void*)W2, (const void*)post,
                        (const void*)post_q, (const void*)Y})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  for (const void* p : {(const void*)w2_inv_scale, (const void*)amax_prev, (const void*)amax_out,
                        (const void*)scale_out})
    FP8MLP_REQUIRE(((uintptr_t)p & 3) == 0, FP8MLP_E_ALIGN);
  return FP8MLP_OK;
}

// The launches of mlp_relu2_fwd; `partial` holds fwd_plan(M, h).partial_bytes.
static int fwd_launch(int mode, const uint16_t* X, const uint16_t* W1, const uint8_t* W2t_q,
                      const float* w2_inv_scale, const uint16_t* W2, const float* amax_prev, float margin,
                      uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y, int64_t M,
                      int64_t d, int64_t h, float* partial, hipStream_t st) {
  const bool train = mode == FP8MLP_TRAIN_FP8;
  const FwdPlan plan = fwd_plan(M, h);

  // 1. up-projection with the fused ReLU^2 / quantise / partial-amax epilogue
  {
    GemmArgs a{X, d, W1, d, M, h, d, (int)plan.tm, (int)plan.tn, 1, d};
    EpiRelu2Quant epi{post, train ? post_q : nullptr, partial, amax_prev, margin, h, (int)plan.tn};
    FP8MLP_TRY(launch_gemm<CfgUp, KID_UP>(a, epi, st));
  }
  if (M == 0) {
    // nothing to multiply: amax = 0 (and the scale that would have been used)
    return launch_max_small(partial, 0, amax_out, amax_prev, margin, train ? scale_out : nullptr, st);
  }
  // 2. down-projection; its block 0 also reduces the partial amax tensor and
  //    records the scale that was used
  auto side = [&](GemmArgs& a) {
    a.red_in = (const uint32_t*)partial;
    a.red_n = plan.tm * plan.tn;
    a.red_out = amax_out;
    a.red_amax_prev = amax_prev;
    a.red_margin = margin;
    a.red_scale_out = train ? scale_out : nullptr;
  };
  if (train) {
    GemmArgs a{post_q, h, W2t_q, d, M, d, h, (int)cdiv(M, CfgDown8::BM), (int)cdiv(d, CfgDown8::BN), 1, h};
    side(a);
    EpiBf16Out epi{Y, d, 1, amax_prev, margin, nullptr, w2_inv_scale};
    FP8MLP_TRY(launch_gemm<CfgDown8, KID_DOWN8>(a, epi, st));
  } else {
    GemmArgs a{post, h, W2, h, M, d, h, (int)cdiv(M, CfgDownBf16::BM), (int)cdiv(d, CfgDownBf16::BN), 1, h};
    side(a);
    EpiBf16Out epi{Y, d, 0, nullptr, 0.0f, nullptr, nullptr};
    FP8MLP_TRY(launch_gemm<CfgDownBf16, KID_DOWN_BF16>(a, epi, st));
  }
  return FP8MLP_OK;
}

// ------------------------------------------------------------------ allocation-free forward
// The partial-amax tensor of mlp_relu2_fwd_noalloc lives in this file-scope
// device array instead of a caller workspace: one copy per GPU, held until the
// process ends, shared by every call on that GPU.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol);
// it passes the device address that hipGetSymbolAddress returns, looked up
// once per device on the first call with that device current.
constexpr size_t kFwdScratchBytes = 256 * 1024;
static __device__ __align__(256) uint8_t scratch[kFwdScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

// Device address of this GPU's scratch array.
static int scratch_ptr(void** out) {
  int dev = 0;
  FP8MLP_TRY(hip_status(hipGetDevice(&dev)));
  if (dev < 0 || dev >= kScratchDevices) return FP8MLP_E_ARCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      FP8MLP_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))));
      if (p == nullptr) return FP8MLP_E_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8MLP_OK;
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

size_t mlp_relu2_fwd_workspace(int64_t M, int64_t d, int64_t h) {
  if (M < 0 || d <= 0 || h <= 0) return 0;
  return fwd_plan(M, h).partial_bytes;
}

int mlp_relu2_fwd(int mode, const uint16_t* X, const uint16_t* W1, const uint8_t* W2t_q,
                  const float* w2_inv_scale, const uint16_t* W2, const float* amax_prev, float margin,
                  uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y, int64_t M,
                  int64_t d, int64_t h, void* workspace, size_t workspace_bytes, void* stream) {
  FP8MLP_TRY(fwd_check_args(mode, X, W1, W2t_q, w2_inv_scale, W2, amax_prev, margin, post, post_q, amax_out,
                            scale_out, Y, M, d, h));
  const FwdPlan plan = fwd_plan(M, h);
  FP8MLP_REQUIRE(workspace_bytes >= plan.partial_bytes && (plan.partial_bytes == 0 || workspace),
                 FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(plan.partial_bytes == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  return fwd_launch(mode, X, W1, W2t_q, w2_inv_scale, W2, amax_prev, margin, post, post_q, amax_out, scale_out, Y,
                    M, d, h, (float*)workspace, (hipStream_t)stream);
}

size_t mlp_relu2_fwd_noalloc_max_bytes(void) { return kFwdScratchBytes; }

int mlp_relu2_fwd_noalloc(int mode, const uint16_t* X, const uint16_t* W1, const uint8_t* W2t_q,
                          const float* w2_inv_scale, const uint16_t* W2, const float* amax_prev, float margin,
                          uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y, int64_t M,
                          int64_t d, int64_t h, void* stream) {
  FP8MLP_TRY(fwd_check_args(mode, X, W1, W2t_q, w2_inv_scale, W2, amax_prev, margin, post, post_q, amax_out,
                            scale_out, Y, M, d, h));
  FP8MLP_REQUIRE(fwd_plan(M, h).partial_bytes <= kFwdScratchBytes, FP8MLP_E_WORKSPACE);
  FP8MLP_TRY(check_device());
  void* ptr = nullptr;
  FP8MLP_TRY(scratch_ptr(&ptr));
  return fwd_launch(mode, X, W1, W2t_q, w2_inv_scale, W2, amax_prev, margin, post, post_q, amax_out, scale_out, Y,
                    M, d, h, (float*)ptr, (hipStream_t)stream);
}

size_t mlp_relu2_fwd_fp8up_workspace(int64_t M, int64_t d, int64_t h) {
  if (M < 0 || d <= 0 || h <= 0) return 0;
  if (M == 0) return 0;
  return fwd_plan(M, h).partial_bytes + quantize_partial_bytes() + align_up((size_t)(M * d), 256);
}

int mlp_relu2_fwd_fp8up(const uint16_t* X, const float* x_scale, const uint8_t* W1t_q, const float* w1_inv_scale,
                        const uint8_t* W2t_q, const float* w2_inv_scale, const float* amax_prev, float margin,
                        uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y,
                        float* x_amax_out, int64_t M, int64_t d, int64_t h, void* workspace, size_t workspace_bytes,
                        void* stream) {
  FP8MLP_REQUIRE(M >= 0 && d > 0 && h > 0 && d % 128 == 0 && h % 128 == 0 && weight_dims_ok(h, d), FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(x_scale && W1t_q && w1_inv_scale && W2t_q && w2_inv_scale && amax_prev && amax_out, FP8MLP_E_NULL);
  if (M > 0) FP8MLP_REQUIRE(X && post_q && Y, FP8MLP_E_NULL);
  FP8MLP_REQUIRE(margin > 0.0f && margin <= 3.4e38f, FP8MLP_E_ARG);
  // amax_out / scale_out are written by block 0 of the down-projection while
  // later blocks still read amax_prev; x_amax_out by block 0 of the
  // up-projection while its other blocks read x_scale
  FP8MLP_REQUIRE(amax_out != amax_prev && scale_out != amax_prev && scale_out != amax_out, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(x_amax_out == nullptr || (x_amax_out != x_scale && x_amax_out != amax_prev &&
                                           x_amax_out != amax_out && x_amax_out != scale_out),
                 FP8MLP_E_ARG);
  for (const void* p : {(const void*)X, (const void*)W1t_q, (const void*)W2t_q, (const void*)post,
                        (const void*)post_q, (const void*)Y})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  for (const void* p : {(const void*)x_scale, (const void*)w1_inv_scale, (const void*)w2_inv_scale,
                        (const void*)amax_prev, (const void*)amax_out, (const void*)scale_out,
                        (const void*)x_amax_out})
    FP8MLP_REQUIRE(((uintptr_t)p & 3) == 0, FP8MLP_E_ALIGN);
  const FwdPlan plan = fwd_plan(M, h);
  const size_t need = mlp_relu2_fwd_fp8up_workspace(M, d, h);
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());

  hipStream_t st = (hipStream_t)stream;
  if (M == 0) {
    // no tokens: both maxima are 0 (and the scale that would have been used)
    if (x_amax_out) FP8MLP_TRY(launch_max_small(nullptr, 0, x_amax_out, nullptr, 0.0f, nullptr, st));
    return launch_max_small(nullptr, 0, amax_out, amax_prev, margin, scale_out, st);
  }
  float* partial = (float*)workspace;
  uint32_t* xpart = (uint32_t*)((uint8_t*)workspace + plan.partial_bytes);
  uint8_t* Xq = (uint8_t*)workspace + plan.partial_bytes + quantize_partial_bytes();

  // 1. Xq = e4m3(fp32(X * x_scale)), with per-block maxima of |X| if asked
  int64_t nx = 0;
  FP8MLP_TRY(launch_quantize(X, M * d, x_scale, Xq, x_amax_out ? xpart : nullptr, &nx, st));
  // 2. e4m3 up-projection with the dequantising ReLU^2 / quantise / partial-amax
  //    epilogue; its block 0 also finishes max |X|
  {
    GemmArgs a{Xq, d, W1t_q, h, M, h, d, (int)plan.tm, (int)plan.tn, 1, d};
    if (x_amax_out) {
      a.red_in = xpart;
      a.red_n = nx;
      a.red_out = x_amax_out;
    }
    EpiRelu2QuantT<true> epi{post, post_q, partial, amax_prev, margin, h, (int)plan.tn, x_scale, w1_inv_scale};
    FP8MLP_TRY(launch_gemm<CfgUp8, KID_UP8>(a, epi, st));
  }
  // 3. e4m3 down-projection; its block 0 also finishes the partial amax
  GemmArgs a{post_q, h, W2t_q, d, M, d, h, (int)cdiv(M, CfgDown8::BM), (int)cdiv(d, CfgDown8::BN), 1, h};
  a.red_in = (const uint32_t*)partial;
  a.red_n = plan.tm * plan.tn;
  a.red_out = amax_out;
  a.red_amax_prev = amax_prev;
  a.red_margin = margin;
  a.red_scale_out = scale_out;
  EpiBf16Out epi{Y, d, 1, amax_prev, margin, nullptr, w2_inv_scale};
  return launch_gemm<CfgDown8, KID_DOWN8>(a, epi, st);
}

}  // extern "C"
