// softcap_ce_fwd_bwd: fused softcapped cross-entropy over a language-model
// head ("NanoGPT Speedrun (Track 1)", "From Unoptimized", "Approach" item 5:
// the fused softcapped cross-entropy never materialises the [M, V] logits in
// fp32; "A Retrospective on Our World Records", SlowRun part: one head
// trained against several successive targets per position).
//
//   z = X W^T, z' = c tanh(z / c)           (per tile, in registers)
//   pass 1: per tile and row, max and sum exp(z' - max) -> partials; the
//           target logits z'[m, t[m, j]] are picked up where they fall
//   rows:   lse = max + log(sum), loss_m = sum_j w_j (lse - z'_t)
//   pass 2: the head GEMM again; G = bf16(dL/dz) in the epilogue
//   dX = bf16(G W), dW = G^T X              (the GEMM core)
// The logits exist only as fp32 accumulators and as the bf16 gradient G.
#include <type_traits>

#include "launch.h"

namespace fp8mlp {

// Every two-group GEMM here keeps three LDS buffers for its A operand
// (loaded two k-tiles ahead).
// X [M,d] . W [V,d]^T: both k-contiguous, two groups of four waves.
using CfgCeHead = GemmCfg<2, 256, 256, 128, 2, 1, KC, KC, 0, 8, 0, 3>;
// The FP8 form: Xq [M,d] . Wt_q [d,V] (the transposed e4m3 cache, read with
// transposing LDS loads).
using CfgCeHead8 = GemmCfg<1, 256, 256, 128, 2, 1, KC, MNC, 0, 8, 0, 3>;
// G [M,V] . W [V,d]: G k-contiguous, W row-contiguous (k = vocabulary row).
using CfgCeDx = GemmCfg<2, 192, 256, 128, 2, 1, KC, MNC, 0, 8, 0, 3>;
// G^T . X: both row-contiguous with k = token.
using CfgCeDw = GemmCfg<2, 256, 256, 128, 2, 1, MNC, MNC, 0, 8, 0, 3>;

constexpr int kCeMaxTargets = 4;

// z' = c tanh(z / c) for c > 0, z for c = 0.  tanh(x) = sign(x) (1 - 2 / (e^(2|x|) + 1))
// with the hardware exp and reciprocal (each within a few ulps): absolute
// error a few fp32 ulps of 1, which is what the softmax sees.
__device__ __forceinline__ float softcap_f(float z, float c, float inv_c) {
  if (c == 0.0f) return z;
  const float a = fabsf(z * inv_c);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(2.0f * a) + 1.0f);
  return copysignf(c * t, z);
}

struct CeParams {
  const int32_t* targets;   // [M, T]
  int T;
  const float* weights;     // [T], device
  float c, inv_c;
  int64_t M, V;
  const float* x_scale;     // FP8 form: z = (acc * fp32(1 / *x_scale)) * *w_inv
  const float* w_inv;
};

// The logit of accumulator value a: the FP8 form dequantises first.
template <bool DEQ>
__device__ __forceinline__ float head_logit(float a, float dq_x, float dq_w) {
  return DEQ ? (a * dq_x) * dq_w : a;
}

// Pass 1: per-row maximum and sum of exp over the tile's columns, and the
// target logits that fall in the tile.  Columns follow the accumulator
// layout of the configuration (16 consecutive per lane, or four runs of four
// under transposed e4m3 reads).
template <bool DEQ>
struct EpiCeStatsT {
  CeParams p;
  float* pmax;    // [tiles_n, M]
  float* psum;    // [tiles_n, M]
  float* zt;      // [M, T]

  template <class C>
  static constexpr int lds_bytes() { return (C::NW / 2) * C::BM * 8; }

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char* smem) {
    constexpr int NWN = C::NW / 2;                 // wave columns of the tile
    float* red = (float*)smem;                     // [NWN][BM][2]
    const int h = c.lane >> 5;
    float dq_x = 1.0f, dq_w = 1.0f;
    if constexpr (DEQ) {
      dq_x = 1.0f / *p.x_scale;
      dq_w = *p.w_inv;
    }
    __syncthreads();   // every wave is done with the last pipeline stage
    // columns past V only in the last column tile
    const bool cols_in = c.n0 + C::BN <= p.V;
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      const int r = c.wm * C::WTM + fm * 32 + (c.lane & 31);
      const int64_t m = c.m0 + r;
      float mx = -INFINITY, s = 0.0f;
      auto row_stats = [&]<bool EDGE>() {
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) {
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const float v = softcap_f(head_logit<DEQ>(acc[fm][fn][e], dq_x, dq_w), p.c, p.inv_c);
            acc[fm][fn][e] = v;
            if (!EDGE || c.n0 + epi_col<C>(c, fn, e) < p.V) mx = fmaxf(mx, v);
          }
        }
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) {
#pragma unroll
          for (int e = 0; e < 16; e++)
            if (!EDGE || c.n0 + epi_col<C>(c, fn, e) < p.V) s += __expf(acc[fm][fn][e] - mx);
        }
      };
      if (cols_in) {
        row_stats.template operator()<false>();
      } else {
        row_stats.template operator()<true>();
      }
      // the other lane half holds the same row's other 16 columns
      const float mo = __shfl_xor(mx, 32, 64), so = __shfl_xor(s, 32, 64);
      const float mm = fmaxf(mx, mo);
      s = (mx == -INFINITY ? 0.0f : s * __expf(mx - mm)) + (mo == -INFINITY ? 0.0f : so * __expf(mo - mm));
      if (h == 0) {
        red[(c.wn * C::BM + r) * 2] = mm;
        red[(c.wn * C::BM + r) * 2 + 1] = s;
      }
      // target logits of this row that fall in this lane's columns
      if (m < p.M) {
        for (int j = 0; j < p.T; j++) {
          const int32_t t = p.targets[m * p.T + j];
          if (t < 0 || t >= p.V) continue;
#pragma unroll
          for (int fn = 0; fn < C::FN; fn++) {
            // the fragment's 32 columns start here; this lane holds 16 of them
            const int64_t f0 = c.n0 + c.wn * C::WTN + fn * 32;
            if (t >= f0 && t < f0 + 32) {
#pragma unroll
              for (int e = 0; e < 16; e++)
                if (c.n0 + epi_col<C>(c, fn, e) == t) zt[m * p.T + j] = acc[fm][fn][e];
            }
          }
        }
      }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < C::BM; r += C::NT) {
      const int64_t m = c.m0 + r;
      if (m >= p.M) continue;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWN; w++) mm = fmaxf(mm, red[(w * C::BM + r) * 2]);
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NWN; w++) {
        const float mw = red[(w * C::BM + r) * 2];
        if (mw != -INFINITY) s += red[(w * C::BM + r) * 2 + 1] * __expf(mw - mm);
      }
      pmax[(int64_t)c.tn * p.M + m] = mm;
      psum[(int64_t)c.tn * p.M + m] = s;
    }
  }
};

// Pass 2: the logit gradient, bf16, staged through LDS and stored row by row.
//   G = bf16(g (wsum p - sum_j w_j [n == t_j]) (1 - (z'/c)^2)),  p = exp(z' - lse)
template <bool DEQ>
struct EpiCeGradT {
  CeParams p;
  const float* lse;     // [M]
  const float* zt;      // [M, T] target logits from pass 1
  const float* dloss;   // device scalar or nullptr (1)
  uint16_t* G;          // [M, V]

  template <class C>
  static constexpr int lds_bytes() { return Tile16<C>::BYTES; }

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char* smem) {
    using T = Tile16<C>;
    const float g = (dloss ? *dloss : 1.0f) / (float)p.M;
    float dq_x = 1.0f, dq_w = 1.0f;
    if constexpr (DEQ) {
      dq_x = 1.0f / *p.x_scale;
      dq_w = *p.w_inv;
    }
    float w[kCeMaxTargets];
#pragma unroll
    for (int j = 0; j < kCeMaxTargets; j++) w[j] = j < p.T ? p.weights[j] : 0.0f;
    __syncthreads();   // every wave is done with the last pipeline stage
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      const int64_t m = c.m0 + c.wm * C::WTM + fm * 32 + (c.lane & 31);
      const bool row_in = m < p.M;
      const float l = row_in ? lse[m] : 0.0f;
      int32_t t[kCeMaxTargets];
      float wsum = 0.0f;
#pragma unroll
      for (int j = 0; j < kCeMaxTargets; j++) {
        t[j] = (row_in && j < p.T) ? p.targets[m * p.T + j] : -1;
        if (t[j] >= p.V) t[j] = -1;
        if (t[j] >= 0) wsum += w[j];
      }
      // every column as if no target fell in it (rows past M are not stored)
#pragma unroll
      for (int fn = 0; fn < C::FN; fn++) {
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          float gv[2];
#pragma unroll
          for (int u = 0; u < 2; u++) {
            const float zc = softcap_f(head_logit<DEQ>(acc[fm][fn][e + u], dq_x, dq_w), p.c, p.inv_c);
            float d = wsum * __expf(zc - l);
            if (p.c != 0.0f) {
              const float q = zc * p.inv_c;
              d *= 1.0f - q * q;
            }
            gv[u] = g * d;
          }
          pk[e / 2] = pack_bf16x2(gv[0], gv[1]);
        }
        T::put(smem, c, fm, fn, pk);
      }
    }
    __syncthreads();
    // The target columns of the tile's rows (at most kCeMaxTargets a row):
    // the same value with the targets' weights subtracted, from the target
    // logit pass 1 stored (the same fp32 value the accumulator gives here),
    // written over the staged entry.
    for (int r = threadIdx.x; r < C::BM; r += C::NT) {
      const int64_t m = c.m0 + r;
      if (m >= p.M) continue;
      const float l = lse[m];
      int32_t t[kCeMaxTargets];
      float wsum = 0.0f;
#pragma unroll
      for (int j = 0; j < kCeMaxTargets; j++) {
        t[j] = j < p.T ? p.targets[m * p.T + j] : -1;
        if (t[j] >= p.V) t[j] = -1;
        if (t[j] >= 0) wsum += w[j];
      }
#pragma unroll
      for (int j = 0; j < kCeMaxTargets; j++) {
        if (t[j] < c.n0 || t[j] >= c.n0 + C::BN) continue;
        const float zc = zt[m * p.T + j];
        float d = wsum * __expf(zc - l);
#pragma unroll
        for (int i = 0; i < kCeMaxTargets; i++) d -= (t[i] == t[j]) ? w[i] : 0.0f;
        if (p.c != 0.0f) {
          const float q = zc * p.inv_c;
          d *= 1.0f - q * q;
        }
        const int col = (int)(t[j] - c.n0);
        *(FP8MLP_LDS uint16_t*)(smem + T::off(r, col >> 3) + 2 * (col & 7)) = (uint16_t)(pack_bf16x2(g * d, 0.0f) & 0xffffu);
      }
    }
    __syncthreads();
    T::store(smem, c, G, p.V);
  }
};

// Per row: lse from the tile partials, the row's loss; per block: the sum
// of its rows' losses (in row order) for the final, ordered reduction.
__global__ void __launch_bounds__(256) k_ce_rows(const float* __restrict__ pmax, const float* __restrict__ psum,
                                                 int tiles_n, const float* __restrict__ zt, CeParams p,
                                                 float* __restrict__ lse, float* __restrict__ loss_part) {
  __shared__ float red[256];
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float loss = 0.0f;
  if (m < p.M) {
    float mm = -INFINITY;
    for (int t = 0; t < tiles_n; t++) mm = fmaxf(mm, pmax[(int64_t)t * p.M + m]);
    float s = 0.0f;
    for (int t = 0; t < tiles_n; t++) {
      const float mt = pmax[(int64_t)t * p.M + m];
      if (mt != -INFINITY) s += psum[(int64_t)t * p.M + m] * __expf(mt - mm);
    }
    const float l = mm + logf(s);
    lse[m] = l;
    for (int j = 0; j < p.T; j++) {
      const int32_t t = p.targets[m * p.T + j];
      if (t >= 0 && t < p.V) loss += p.weights[j] * (l - zt[m * p.T + j]);
    }
  }
  red[threadIdx.x] = loss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss_part[blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(256) k_ce_loss(const float* __restrict__ loss_part, int n, float inv_m,
                                                 float* loss_out) {
  __shared__ float red[256];
  float s = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) s += loss_part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss_out = red[0] * inv_m;
}

struct CePlan {
  int64_t tiles_m, tiles_n, row_blocks;
  int dw_splits;              // dW over token ranges: the GEMM addresses one range with 32-bit offsets
  int64_t dw_k_per_split;
  size_t g_bytes, stat_bytes, zt_bytes, lse_bytes, part_bytes, dw_part_bytes;
  size_t total() const { return g_bytes + 2 * stat_bytes + zt_bytes + lse_bytes + part_bytes + dw_part_bytes; }
};
static CePlan ce_plan(int64_t M, int64_t V, int64_t d, int T) {
  CePlan q;
  q.tiles_m = cdiv(M, CfgCeHead::BM);
  q.tiles_n = cdiv(V, CfgCeHead::BN);
  q.row_blocks = cdiv(M, 256);
  // a token range of G rows must stay below 2^31 bytes
  const int64_t row_bytes = 2 * (V > d ? V : d);
  int64_t kps = (((int64_t)1 << 31) / row_bytes) / CfgCeDw::BK * CfgCeDw::BK;
  if (kps < CfgCeDw::BK) kps = CfgCeDw::BK;
  q.dw_splits = (int)(M > 0 ? cdiv(M, kps) : 1);
  q.dw_k_per_split = q.dw_splits > 1 ? kps : (M > 0 ? M : 1);
  q.g_bytes = align_up((size_t)(M * V) * 2, 256);
  q.stat_bytes = align_up((size_t)(q.tiles_n * M) * 4, 256);
  q.zt_bytes = align_up((size_t)(M * T) * 4, 256);
  q.lse_bytes = align_up((size_t)M * 4, 256);
  q.part_bytes = align_up((size_t)q.row_blocks * 4, 256);
  q.dw_part_bytes = q.dw_splits > 1 ? align_up((size_t)q.dw_splits * (size_t)(V * d) * 4, 256) : 0;
  return q;
}

// Both entry points: FP8 selects the e4m3 head (Xq from X in the workspace,
// Wt_q [d, V]); the gradient GEMMs run on the bf16 X and W either way.
template <bool FP8>
static int ce_impl(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv,
                   const uint16_t* W, const int32_t* targets, int T, const float* weights, float softcap,
                   const float* dloss, float* loss_out, float* lse_out, uint16_t* dX, float* dW, int accumulate,
                   int64_t M, int64_t V, int64_t d, void* workspace, size_t workspace_bytes, hipStream_t st) {
  FP8MLP_REQUIRE(M >= 0 && V > 0 && d > 0 && V % 64 == 0 && d % (FP8 ? 128 : 64) == 0 &&
                     M * V < ((int64_t)1 << 40) && weight_dims_ok(V, d),
                 FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(T >= 1 && T <= kCeMaxTargets, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(softcap >= 0.0f && softcap <= 3.4e38f, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(accumulate == 0 || accumulate == 1, FP8MLP_E_ARG);
  FP8MLP_REQUIRE(loss_out && dW && W && weights, FP8MLP_E_NULL);
  if (FP8) FP8MLP_REQUIRE(x_scale && Wt_q && w_inv, FP8MLP_E_NULL);
  if (M > 0) FP8MLP_REQUIRE(X && targets && dX, FP8MLP_E_NULL);
  for (const void* p : {(const void*)X, (const void*)W, (const void*)Wt_q, (const void*)dX, (const void*)dW})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  for (const void* p : {(const void*)targets, (const void*)weights, (const void*)dloss, (const void*)loss_out,
                        (const void*)lse_out, (const void*)x_scale, (const void*)w_inv})
    FP8MLP_REQUIRE(((uintptr_t)p & 3) == 0, FP8MLP_E_ALIGN);
  const CePlan plan = ce_plan(M, V, d, T);
  const size_t xq_bytes = FP8 ? align_up((size_t)(M * d), 256) : 0;
  const size_t need = M > 0 ? plan.total() + xq_bytes : 0;
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  if (M == 0) {
    // no positions: the loss is 0 and dW receives nothing
    {
      TraceScope trace("ce_loss", st);
      hipLaunchKernelGGL(k_ce_loss, dim3(1), dim3(256), 0, st, (const float*)nullptr, 0, 0.0f, loss_out);
      FP8MLP_TRY(launch_status());
    }
    return accumulate ? FP8MLP_OK : launch_zero(dW, V * d, st);
  }
  char* w = (char*)workspace;
  uint16_t* G = (uint16_t*)w;
  float* pmax = (float*)(w + plan.g_bytes);
  float* psum = (float*)(w + plan.g_bytes + plan.stat_bytes);
  float* zt = (float*)(w + plan.g_bytes + 2 * plan.stat_bytes);
  float* lse = lse_out ? lse_out : (float*)(w + plan.g_bytes + 2 * plan.stat_bytes + plan.zt_bytes);
  float* part = (float*)(w + plan.g_bytes + 2 * plan.stat_bytes + plan.zt_bytes + plan.lse_bytes);
  float* dw_part = (float*)((char*)part + plan.part_bytes);
  CeParams p{targets, T, weights, softcap, softcap > 0.0f ? 1.0f / softcap : 0.0f, M, V, x_scale, w_inv};

  // the head: X W^T in bf16, or e4m3(X * x_scale) . Wt_q
  using CH = typename std::conditional<FP8, CfgCeHead8, CfgCeHead>::type;
  static_assert(CH::BM == CfgCeHead::BM && CH::BN == CfgCeHead::BN, "one tiling of the statistics");
  GemmArgs head{X, d, W, d, M, V, d, (int)plan.tiles_m, (int)plan.tiles_n, 1, d};
  if constexpr (FP8) {
    uint8_t* Xq = (uint8_t*)w + plan.total();
    int64_t nx = 0;
    FP8MLP_TRY(launch_quantize(X, M * d, x_scale, Xq, nullptr, &nx, st));
    head.q = Xq;
    head.p = Wt_q;
    head.ldp = V;
  }
  // pass 1: row statistics and target logits
  {
    EpiCeStatsT<FP8> epi{p, pmax, psum, zt};
    FP8MLP_TRY((launch_gemm<CH, FP8 ? KID_CE8_STATS : KID_CE_STATS>(head, epi, st)));
  }
  {
    TraceScope trace("ce_rows", st);
    hipLaunchKernelGGL(k_ce_rows, dim3((unsigned)plan.row_blocks), dim3(256), 0, st, pmax, psum, (int)plan.tiles_n,
                       zt, p, lse, part);
    FP8MLP_TRY(launch_status());
  }
  {
    TraceScope trace("ce_loss", st);
    hipLaunchKernelGGL(k_ce_loss, dim3(1), dim3(256), 0, st, part, (int)plan.row_blocks, 1.0f / (float)M, loss_out);
    FP8MLP_TRY(launch_status());
  }
  // pass 2: the logit gradient
  {
    EpiCeGradT<FP8> epi{p, lse, zt, dloss, G};
    FP8MLP_TRY((launch_gemm<CH, FP8 ? KID_CE8_GRAD : KID_CE_GRAD>(head, epi, st)));
  }
  // dX = G W
  {
    GemmArgs a{G, V, W, d, M, d, V, (int)cdiv(M, CfgCeDx::BM), (int)cdiv(d, CfgCeDx::BN), 1, V};
    EpiBf16Out epi{dX, d, 0, nullptr, 0.0f, nullptr, nullptr};
    FP8MLP_TRY(launch_gemm<CfgCeDx, KID_CE_DX>(a, epi, st));
  }
  // dW = G^T X over token ranges, the partials reduced in range order
  GemmArgs a{G, V, X, d, V, d, M, (int)cdiv(V, CfgCeDw::BM), (int)cdiv(d, CfgCeDw::BN), plan.dw_splits,
             plan.dw_k_per_split};
  if (plan.dw_splits == 1) {
    EpiF32 epi{dW, d, 0, accumulate};
    return launch_gemm<CfgCeDw, KID_CE_DW>(a, epi, st);
  }
  EpiF32 epi{dw_part, d, V * d, 0};
  FP8MLP_TRY(launch_gemm<CfgCeDw, KID_CE_DW>(a, epi, st));
  return launch_reduce(dw_part, plan.dw_splits, V * d, dW, accumulate, st);
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

size_t softcap_ce_workspace(int64_t M, int64_t V, int64_t d, int T) {
  if (M <= 0 || V <= 0 || d <= 0 || T < 1 || T > kCeMaxTargets) return 0;
  return ce_plan(M, V, d, T).total();
}

size_t softcap_ce_fp8_workspace(int64_t M, int64_t V, int64_t d, int T) {
  if (M <= 0 || V <= 0 || d <= 0 || T < 1 || T > kCeMaxTargets) return 0;
  return ce_plan(M, V, d, T).total() + align_up((size_t)(M * d), 256);
}

int softcap_ce_fwd_bwd(const uint16_t* X, const uint16_t* W, const int32_t* targets, int T, const float* weights,
                       float softcap, const float* dloss, float* loss_out, float* lse_out, uint16_t* dX, float* dW,
                       int accumulate, int64_t M, int64_t V, int64_t d, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return ce_impl<false>(X, nullptr, nullptr, nullptr, W, targets, T, weights, softcap, dloss, loss_out, lse_out, dX,
                        dW, accumulate, M, V, d, workspace, workspace_bytes, (hipStream_t)stream);
}

int softcap_ce_fwd_bwd_fp8(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv_scale,
                           const uint16_t* W, const int32_t* targets, int T, const float* weights, float softcap,
                           const float* dloss, float* loss_out, float* lse_out, uint16_t* dX, float* dW,
                           int accumulate, int64_t M, int64_t V, int64_t d, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return ce_impl<true>(X, x_scale, Wt_q, w_inv_scale, W, targets, T, weights, softcap, dloss, loss_out, lse_out, dX,
                       dW, accumulate, M, V, d, workspace, workspace_bytes, (hipStream_t)stream);
}

}  // extern "C"
