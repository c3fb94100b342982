// mlp_relu2_bwd: the bf16 backward of the ReLU^2 MLP block.
//   dpost = dY W2            fused epilogue: dpre = bf16(2 sqrt(post) dpost)
//   dX    = dpre W1          bf16 out
//   dW1   = dpre^T X         fp32, split-k over M, reduced in split order
//   dW2   = dY^T post        fp32, split-k over M, reduced in split order
// mlp_relu2_bwd_fp8post: the same backward when only the e4m3 copy of post
// was kept; post_hat = dec(post_q) / scale takes post's place, the dgrad
// epilogue decodes the codes and dW2 runs on them directly (e4m3 widened to
// bf16 as its fragments are read, the 1/scale applied to the fp32 result).
// W1 and W2 are first transposed into the workspace (4.7 MB each at the
// GPT-2-small shape) so that both dgrad GEMMs read k-contiguous operands
// with plain 16-byte LDS reads.
#include "persist.h"

namespace fp8mlp {

// dY [M,d] . W2t [h,d]^T: 256 x 256 tiles, two groups of four waves, dY
// loaded two k-tiles ahead (three dY buffers).
using CfgDpost = GemmCfg<2, 256, 256, 128, 2, 1, KC, KC, 0, 8, 0, 3>;
// dpre [M,h] . W1t [d,h]^T: 192 x 256 tiles (d = 768 is three of them, and
// M = 49152 gives exactly three rounds of 256 blocks); three dpre buffers.
using CfgDx = GemmCfg<2, 192, 256, 128, 2, 1, KC, KC, 0, 8, 0, 3>;
// dpre^T . X and dY^T . post: both operands are row-contiguous with k = token;
// 256 x 256 tiles, two groups of four waves, three buffers for the A operand.
using CfgDw = GemmCfg<2, 256, 256, 128, 2, 1, MNC, MNC, 0, 8, 0, 3>;
// dY^T . dec(post_q): the same tiles with the e4m3 codes as the P operand.
using CfgDw2q = GemmCfg<2, 256, 256, 128, 2, 1, MNC, MNC, 0, 8, 1, 3>;

struct BwdPlan {
  size_t dpre_bytes, wt_bytes, part_bytes;   // dpre; W1t + W2t; split-k partials of dW1 and dW2
  int splits;
  int64_t k_per_split;
  int64_t split_stride;                      // floats per split partial (whole tiles of one gradient)
};

static BwdPlan bwd_plan(int64_t M, int64_t d, int64_t h) {
  BwdPlan p;
  p.dpre_bytes = align_up((size_t)(M * h) * 2, 256);
  p.wt_bytes = 2 * align_up((size_t)(h * d) * 2, 256);
  const int64_t tiles = cdiv(h, CfgDw::BM) * cdiv(d, CfgDw::BN);
  // about two rounds of blocks over 256 CUs x OCC resident blocks
  int64_t s = (256 * CfgDw::OCC * 2 + tiles - 1) / (tiles > 0 ? tiles : 1) / 2;
  const int64_t max_s = cdiv(M, 512);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  p.k_per_split = cdiv(cdiv(M, s), 64) * 64;
  if (p.k_per_split == 0) p.k_per_split = 64;
  // the dW GEMMs read one token range of dpre, X, dY and post per block
  const int64_t kmax = max_k_range(2 * (d > h ? d : h));
  if (p.k_per_split > kmax) p.k_per_split = kmax;
  p.splits = (int)(M > 0 ? cdiv(M, p.k_per_split) : 1);
  // the partials of dW1, then those of dW2, each split a whole number of
  // tiles (dW1 [h, d] and dW2 [d, h] have the same tile count)
  static_assert(CfgDw::BM == CfgDw::BN, "dW1 and dW2 tile the same way");
  p.split_stride = tiles * CfgDw::BM * CfgDw::BN;
  p.part_bytes = p.splits > 1 ? 2 * align_up((size_t)p.splits * (size_t)p.split_stride * 4, 256) : 0;
  return p;
}

// W1t [d, h] = W1 [h, d]^T and W2t [h, d] = 2 W2 [d, h]^T in one launch,
// 64 x 64 bf16 tiles through LDS (d and h are multiples of 64), one block per
// tile.  Doubling a bf16 value is exact (short of overflow
// past 3.4e38), so the dgrad GEMM on W2t accumulates exactly 2 dpost and its
// epilogue needs no separate doubling for dpre = 2 sqrt(post) dpost.
__global__ void __launch_bounds__(256) k_transpose_weights(const uint16_t* __restrict__ W1,
                                                           const uint16_t* __restrict__ W2, int64_t d, int64_t h,
                                                           uint16_t* __restrict__ W1t, uint16_t* __restrict__ W2t) {
  __shared__ uint16_t tile[64][64 + 2];   // [c][r]
  // blocks [0, n) transpose W1's (h/64) x (d/64) tiles, blocks [n, 2n) W2's
  const int64_t n = (h / 64) * (d / 64);
  const bool second = blockIdx.x >= n;
  const int64_t b = second ? blockIdx.x - n : blockIdx.x;
  const uint16_t* src = second ? W2 : W1;
  uint16_t* dst = second ? W2t : W1t;
  const int64_t R = second ? d : h, C = second ? h : d;   // src is [R, C]
  const int64_t r0 = (b / (C / 64)) * 64, c0 = (b % (C / 64)) * 64;
#pragma unroll
  for (int it = 0; it < 2; it++) {
    const int i = threadIdx.x + it * 256;
    const int r = i >> 3, ch = i & 7;
    const uint4 v = *(const uint4*)(src + (r0 + r) * C + c0 + ch * 8);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if (second) {
#pragma unroll
      for (int e = 0; e < 4; e++) w[e] = pack_bf16x2(2.0f * bf16_lo(w[e]), 2.0f * bf16_hi(w[e]));
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      tile[ch * 8 + 2 * e][r] = (uint16_t)(w[e] & 0xffffu);
      tile[ch * 8 + 2 * e + 1][r] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; it++) {
    const int i = threadIdx.x + it * 256;
    const int c = i >> 3, ch = i & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; e++) w[e] = (uint32_t)tile[c][ch * 8 + 2 * e] | ((uint32_t)tile[c][ch * 8 + 2 * e + 1] << 16);
    *(uint4*)(dst + (c0 + c) * R + r0 + ch * 8) = uint4{w[0], w[1], w[2], w[3]};
  }
}

static int launch_transpose_weights(const uint16_t* W1, const uint16_t* W2, int64_t d, int64_t h, uint16_t* W1t,
                                    uint16_t* W2t, hipStream_t st) {
  const unsigned blocks = (unsigned)(2 * (h / 64) * (d / 64));
  TraceScope trace("transpose_weights", st);
  hipLaunchKernelGGL(k_transpose_weights, dim3(blocks), dim3(256), 0, st, W1, W2, d, h, W1t, W2t);
  return launch_status();
}

// out[i] = (accumulate ? out[i] : 0) + part[0][i] + part[1][i] + ... in split order.
__global__ void __launch_bounds__(256) k_splitk_reduce(const float4* __restrict__ part, int splits, int64_t n4,
                                                       float4* __restrict__ out, int accumulate) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 a = accumulate ? out[i] : float4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; s++) {
      const float4 v = part[s * n4 + i];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    out[i] = a;
  }
}

__global__ void __launch_bounds__(256) k_fill_zero(float4* __restrict__ out, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    out[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// One weight gradient whose split-k partials EpiF32Part wrote.
struct RedProb {
  const float* part;     // split s at part + s * split_stride
  float* out;            // [rows, cols] fp32, leading dimension cols
  int64_t rows, cols;
  int tiles_n, tiles;
  int perm;              // 1: a lane holds 16 consecutive columns of a fragment (GemmCfg::PERM)
};

// out = (accumulate ? out : 0) + part[0] + part[1] + ... in split order, for
// the partials EpiF32Part wrote with the tile configuration C.  Block
// (g, t, z): problem z, tile t, the 32 rows of fragment row g (the wave row
// wm = g / FM, fragment fm = g % FM); it sums the partials of those rows
// (contiguous 16-byte reads), stages the 32 x BN result in LDS and writes it
// row by row.
template <class C>
__global__ void __launch_bounds__(256) k_splitk_reduce_tiles(RedProb p0, RedProb p1, int splits,
                                                             int64_t split_stride, int accumulate) {
  static_assert(C::NW == 8 && C::BN % 64 == 0 && (32 * C::BN / 4) % 256 == 0, "two-group tiles");
  constexpr int C4 = C::BN / 4;                     // float4 per tile row
  constexpr int PER = 32 * C4 / 256;                // float4 per thread
  __shared__ float4 img[32][C4 + 1];
  const RedProb& P = blockIdx.z ? p1 : p0;
  const int tile = blockIdx.y;
  if (tile >= P.tiles) return;
  const int tm = tile / P.tiles_n, tn = tile % P.tiles_n;
  const int wm = blockIdx.x / C::FM, fm = blockIdx.x % C::FM;
  const int64_t m0 = (int64_t)tm * C::BM + wm * C::WTM + fm * 32, n0 = (int64_t)tn * C::BN;
  const float* base = P.part + (int64_t)tile * (C::BM * C::BN);
  int pos[PER], rr[PER], cc[PER];
  float4 a[PER];
#pragma unroll
  for (int k = 0; k < PER; k++) {
    const int i = threadIdx.x + 256 * k;
    const int b = i >> 6, lane = i & 63;
    // the four waves of wave row wm, then fragment column fn, then float4 j
    const int wi = b / (4 * C::FN), fn = (b >> 2) % C::FN, j = b & 3;
    const int w = (wi & 1) + 2 * wm + 4 * (wi >> 1);
    const int wn = 2 * (w & 1) + (w >> 2);
    pos[k] = (((fm * C::FN + fn) * 4 + j) * C::NW + w) * 64 + lane;
    const int h = lane >> 5;
    rr[k] = lane & 31;
    cc[k] = wn * C::WTN + fn * 32 + (P.perm ? 16 * h + 4 * j : 8 * j + 4 * h);
    a[k] = float4{0.f, 0.f, 0.f, 0.f};
    if (accumulate && m0 + rr[k] < P.rows && n0 + cc[k] < P.cols)
      a[k] = *(const float4*)(P.out + (m0 + rr[k]) * P.cols + n0 + cc[k]);
  }
  // every split's loads in flight together, then added in split order
  for (int s = 0; s < splits; s++) {
    f32x4 v[PER];
#pragma unroll
    for (int k = 0; k < PER; k++) v[k] = __builtin_nontemporal_load((const f32x4*)(base + s * split_stride) + pos[k]);
#pragma unroll
    for (int k = 0; k < PER; k++) {
      a[k].x += v[k][0];
      a[k].y += v[k][1];
      a[k].z += v[k][2];
      a[k].w += v[k][3];
    }
  }
#pragma unroll
  for (int k = 0; k < PER; k++) img[rr[k]][cc[k] >> 2] = a[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; k++) {
    const int i = threadIdx.x + 256 * k;
    const int r = i / C4, c4 = i % C4;
    const int64_t m = m0 + r, n = n0 + 4 * c4;
    if (m < P.rows && n < P.cols) *(float4*)(P.out + m * P.cols + n) = img[r][c4];
  }
}

template <class C>
static int launch_reduce_tiles(const RedProb& p0, const RedProb& p1, int splits, int64_t split_stride,
                               int accumulate, hipStream_t st) {
  const int tiles = p0.tiles > p1.tiles ? p0.tiles : p1.tiles;
  TraceScope trace("splitk_reduce", st);
  hipLaunchKernelGGL(k_splitk_reduce_tiles<C>, dim3(2 * C::FM, (unsigned)tiles, 2), dim3(256), 0, st, p0, p1,
                     splits, split_stride, accumulate);
  return launch_status();
}

int launch_reduce(const float* part, int splits, int64_t n, float* out, int accumulate, hipStream_t st) {
  const int64_t n4 = n / 4;
  int64_t blocks = cdiv(n4, 256);
  if (blocks > 4096) blocks = 4096;
  TraceScope trace("splitk_reduce", st);
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, st, (const float4*)part, splits, n4,
                     (float4*)out, accumulate);
  return launch_status();
}

int launch_zero(float* out, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  int64_t blocks = cdiv(n4, 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return FP8MLP_OK;
  TraceScope trace("fill_zero", st);
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (float4*)out, n4);
  return launch_status();
}

// The two entry points differ in the dgrad epilogue and the dW2 operand.
template <bool Q>
static int mlp_bwd_impl(const uint16_t* dY, const uint16_t* X, const uint16_t* W1, const uint16_t* W2,
                        const void* post, const float* post_scale, uint16_t* dX, float* dW1, float* dW2,
                        int accumulate, int64_t M, int64_t d, int64_t h, void* workspace, size_t workspace_bytes,
                        hipStream_t st) {
  FP8MLP_REQUIRE(M >= 0 && d > 0 && h > 0 && d % 64 == 0 && h % 64 == 0 && weight_dims_ok(h, d), FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(accumulate == 0 || accumulate == 1, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(dW1 && dW2, FP8MLP_E_NULL);
  if (M > 0) FP8MLP_REQUIRE(dY && X && W1 && W2 && post && dX && (!Q || post_scale), FP8MLP_E_NULL);
  for (const void* p : {(const void*)dY, (const void*)X, (const void*)W1, (const void*)W2, (const void*)post,
                        (const void*)dX, (const void*)dW1, (const void*)dW2})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  FP8MLP_REQUIRE(((uintptr_t)post_scale & 3) == 0, FP8MLP_E_ALIGN);
  const BwdPlan plan = bwd_plan(M, d, h);
  const size_t need = plan.dpre_bytes + plan.wt_bytes + plan.part_bytes;
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());

  if (M == 0) {
    if (!accumulate) {
      FP8MLP_TRY(launch_zero(dW1, h * d, st));
      FP8MLP_TRY(launch_zero(dW2, d * h, st));
    }
    return FP8MLP_OK;
  }
  uint16_t* dpre = (uint16_t*)workspace;
  uint16_t* W1t = (uint16_t*)((char*)workspace + plan.dpre_bytes);                    // [d, h]
  uint16_t* W2t = (uint16_t*)((char*)W1t + plan.wt_bytes / 2);                         // [h, d]
  float* part = (float*)((char*)workspace + plan.dpre_bytes + plan.wt_bytes);

  FP8MLP_TRY(launch_transpose_weights(W1, W2, d, h, W1t, W2t, st));
  // 1. dpost = dY W2 with the sqrt(post) epilogue -> dpre
  {
    GemmArgs a{dY, d, W2t, d, M, h, d, (int)cdiv(M, CfgDpost::BM), (int)cdiv(h, CfgDpost::BN), 1, d};
    if constexpr (Q) {
      EpiDpreQ epi{(const uint8_t*)post, post_scale, dpre, h};
      FP8MLP_TRY(launch_gemm<CfgDpost, KID_DPOST>(a, epi, st));
    } else {
      EpiDpre epi{(const uint16_t*)post, dpre, h};
      EpiDpreWP wp{(const uint16_t*)post, dpre, h};
      FP8MLP_TRY((launch_gemm_persist<CfgDpost, KID_DPOST>(a, wp, epi, st)));
    }
  }
  // 2. dX = dpre W1
  {
    GemmArgs a{dpre, h, W1t, h, M, d, h, (int)cdiv(M, CfgDx::BM), (int)cdiv(d, CfgDx::BN), 1, h};
    EpiBf16Out epi{dX, d, 0, nullptr, 0.0f, nullptr, nullptr};
    FP8MLP_TRY(launch_gemm<CfgDx, KID_DX>(a, epi, st));
  }
  // 3. dW1 = dpre^T X and 4. dW2 = dY^T post (or (dY^T dec(post_q)) / scale):
  // C [Mo, No] = A^T B with A [M, Mo], B [M, No], split-k over the M tokens
  // into fp32 partials (split order), reduced by one launch for both.
  {
    static_assert(CfgDw2q::BM == CfgDw::BM && CfgDw2q::BN == CfgDw::BN, "the plan's split count assumes these tiles");
    GemmArgs a1{dpre, h, X, d, h, d, M, (int)cdiv(h, CfgDw::BM), (int)cdiv(d, CfgDw::BN), plan.splits,
                plan.k_per_split};
    GemmArgs a2{dY, d, post, h, d, h, M, (int)cdiv(d, CfgDw::BM), (int)cdiv(h, CfgDw::BN), plan.splits,
                plan.k_per_split};
    const bool split = plan.splits > 1;
    float* part2 = part + (size_t)plan.splits * (size_t)plan.split_stride;
    const float* div2 = Q ? post_scale : nullptr;
    if (split) {
      static_assert(CfgDw2q::FM == CfgDw::FM && CfgDw2q::FN == CfgDw::FN && CfgDw2q::NW == CfgDw::NW &&
                        CfgDw2q::WTM == CfgDw::WTM && CfgDw2q::WTN == CfgDw::WTN,
                    "one partial layout for both gradients");
      const EpiF32Part e1{part, plan.split_stride, a1.tiles_n, nullptr};
      const EpiF32Part e2{part2, plan.split_stride, a2.tiles_n, div2};
      if constexpr (Q) {
        FP8MLP_TRY((launch_gemm<CfgDw, KID_DW1>(a1, e1, st)));
        FP8MLP_TRY((launch_gemm<CfgDw2q, KID_DW2>(a2, e2, st)));
      } else {
        // both in one launch (same tiles, same kernel)
        FP8MLP_TRY((launch_gemm2<CfgDw, KID_DW>(a1, e1, a2, e2, st)));
      }
      const RedProb r1{part, dW1, h, d, a1.tiles_n, a1.tiles_m * a1.tiles_n, CfgDw::PERM ? 1 : 0};
      const RedProb r2{part2, dW2, d, h, a2.tiles_n, a2.tiles_m * a2.tiles_n, (Q ? CfgDw2q::PERM : CfgDw::PERM) ? 1 : 0};
      FP8MLP_TRY(launch_reduce_tiles<CfgDw>(r1, r2, plan.splits, plan.split_stride, accumulate, st));
    } else {
      const EpiF32 e1{dW1, d, 0, accumulate, nullptr};
      const EpiF32 e2{dW2, h, 0, accumulate, div2};
      if constexpr (Q) {
        FP8MLP_TRY((launch_gemm<CfgDw, KID_DW1>(a1, e1, st)));
        FP8MLP_TRY((launch_gemm<CfgDw2q, KID_DW2>(a2, e2, st)));
      } else {
        FP8MLP_TRY((launch_gemm2<CfgDw, KID_DW>(a1, e1, a2, e2, st)));
      }
    }
  }
  return FP8MLP_OK;
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

size_t mlp_relu2_bwd_workspace(int64_t M, int64_t d, int64_t h) {
  if (M < 0 || d <= 0 || h <= 0) return 0;
  const BwdPlan p = bwd_plan(M, d, h);
  return p.dpre_bytes + p.wt_bytes + p.part_bytes;
}

int mlp_relu2_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* W1, const uint16_t* W2,
                  const uint16_t* post, uint16_t* dX, float* dW1, float* dW2, int accumulate, int64_t M,
                  int64_t d, int64_t h, void* workspace, size_t workspace_bytes, void* stream) {
  return mlp_bwd_impl<false>(dY, X, W1, W2, post, nullptr, dX, dW1, dW2, accumulate, M, d, h, workspace,
                             workspace_bytes, (hipStream_t)stream);
}

int mlp_relu2_bwd_fp8post(const uint16_t* dY, const uint16_t* X, const uint16_t* W1, const uint16_t* W2,
                          const uint8_t* post_q, const float* post_scale, uint16_t* dX, float* dW1, float* dW2,
                          int accumulate, int64_t M, int64_t d, int64_t h, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return mlp_bwd_impl<true>(dY, X, W1, W2, post_q, post_scale, dX, dW1, dW2, accumulate, M, d, h, workspace,
                            workspace_bytes, (hipStream_t)stream);
}

}  // extern "C"
