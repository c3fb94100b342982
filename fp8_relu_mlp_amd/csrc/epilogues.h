// Epilogues of the MLP GEMMs: what each contraction does with its fp32
// accumulators while they are still in registers.
#pragma once

#include "gemm.h"

namespace fp8mlp {

// Up-projection epilogue ("A Retrospective on Our World Records", Main
// Track: while the fused up-projection kernel holds the post-activation in
// registers it writes the BF16 tensor for backward, emits the FP8 version and
// accumulates a tiny partial-amax tensor; "NanoGPT Speedrun (Track 1)",
// "Changes vs Record #83" item 4: only post = relu(pre)^2 is stored):
//   post   = bf16(relu(pre)^2)
//   post_q = e4m3(fp32(post * scale)),  scale from amax(t-1) and the margin
//   partial[tile] = max(post over the tile)
// relu keeps NaN and the maximum is taken on bit patterns, so a NaN anywhere
// reaches amax; post >= +0, so the e4m3 encode uses the non-negative fast
// path.
struct EpiRelu2Quant {
  uint16_t* post;
  uint8_t* post_q;        // nullptr: no quantised copy (eval)
  float* partial;         // [tiles_m * tiles_n]
  const float* amax_prev;
  float margin;
  int64_t ld;             // h
  int tiles_n;

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char* smem) {
    static_assert(C::PERM, "needs 16 consecutive columns per lane");
    const float s = post_q ? scale_from_amax(*amax_prev, margin) : 1.0f;
    uint32_t mx = 0;
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      const int64_t m = c.m0 + epi_row<C>(c, fm);
#pragma unroll
      for (int fn = 0; fn < C::FN; fn++) {
        const int64_t n = c.n0 + epi_col<C>(c, fn, 0);
        uint32_t pk[8];
        float pv[16];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          pk[e / 2] = opaque(pack_bf16x2(relu_sq(acc[fm][fn][e]), relu_sq(acc[fm][fn][e + 1])));
          pv[e] = bf16_lo(pk[e / 2]);
          pv[e + 1] = bf16_hi(pk[e / 2]);
        }
        if (m < c.M && n < c.N) {
          uint16_t* dst = post + m * ld + n;
          *(uint4*)dst = uint4{pk[0], pk[1], pk[2], pk[3]};
          *(uint4*)(dst + 8) = uint4{pk[4], pk[5], pk[6], pk[7]};
          if (post_q) {
            uint4 q;
            q.x = pack_e4m3x4_nonneg(pv[0] * s, pv[1] * s, pv[2] * s, pv[3] * s);
            q.y = pack_e4m3x4_nonneg(pv[4] * s, pv[5] * s, pv[6] * s, pv[7] * s);
            q.z = pack_e4m3x4_nonneg(pv[8] * s, pv[9] * s, pv[10] * s, pv[11] * s);
            q.w = pack_e4m3x4_nonneg(pv[12] * s, pv[13] * s, pv[14] * s, pv[15] * s);
            *(uint4*)(post_q + m * ld + n) = q;
          }
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const uint32_t b = __float_as_uint(pv[e]);
            mx = b > mx ? b : mx;
          }
        }
      }
    }
    mx = wave_max_u32(mx);
    uint32_t* red = (uint32_t*)smem;
    __syncthreads();  // other waves may still read the last pipeline stage
    if (c.lane == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m4 = red[0];
      for (int i = 1; i < 4; i++) m4 = red[i] > m4 ? red[i] : m4;
      partial[c.tm * tiles_n + c.tn] = __uint_as_float(m4);
    }
  }
};

// bf16 output, optionally dequantised:
//   mode 0: Y = bf16(acc)
//   mode 1: Y = bf16(acc * fp32(1/scale) * w_inv), scale from *amax_prev, margin
//   mode 2: Y = bf16(acc * fp32(1 / *x_scale) * w_inv)
struct EpiBf16Out {
  uint16_t* y;
  int64_t ld;
  int mode;
  const float* amax_prev;
  float margin;
  const float* x_scale;
  const float* w_inv;

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char*) {
    float inv_s = 1.0f, inv_w = 1.0f;
    if (mode == 1) {
      inv_s = 1.0f / scale_from_amax(*amax_prev, margin);
      inv_w = *w_inv;
    } else if (mode == 2) {
      inv_s = 1.0f / *x_scale;
      inv_w = *w_inv;
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      const int64_t m = c.m0 + epi_row<C>(c, fm);
      if (m >= c.M) continue;
#pragma unroll
      for (int fn = 0; fn < C::FN; fn++) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; e++) v[e] = mode ? (acc[fm][fn][e] * inv_s) * inv_w : acc[fm][fn][e];
        if constexpr (C::PERM) {
          const int64_t n = c.n0 + epi_col<C>(c, fn, 0);
          if (n < c.N) {
            uint16_t* dst = y + m * ld + n;
            *(uint4*)dst = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                 pack_bf16x2(v[6], v[7])};
            *(uint4*)(dst + 8) = uint4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                                       pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15])};
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; g++) {
            const int64_t n = c.n0 + epi_col<C>(c, fn, 4 * g);
            if (n < c.N)
              *(uint2*)(y + m * ld + n) =
                  uint2{pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3])};
          }
        }
      }
    }
  }
};

// Backward dgrad epilogue ("NanoGPT Speedrun (Track 1)", "Changes vs Record
// #83" item 4: relu(pre) is rebuilt from the stored post as sqrt(post)):
//   dpre = bf16(2 * sqrt(post) * dpost),  dpost = the accumulator
struct EpiDpre {
  const uint16_t* post;
  uint16_t* dpre;
  int64_t ld;  // h

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char*) {
    static_assert(C::PERM, "needs 16 consecutive columns per lane");
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      const int64_t m = c.m0 + epi_row<C>(c, fm);
      if (m >= c.M) continue;
#pragma unroll
      for (int fn = 0; fn < C::FN; fn++) {
        const int64_t n = c.n0 + epi_col<C>(c, fn, 0);
        if (n >= c.N) continue;
        const uint16_t* src = post + m * ld + n;
        const uint4 p0 = *(const uint4*)src, p1 = *(const uint4*)(src + 8);
        const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          // v_sqrt_f32 (within 1 ulp of fp32) is far below the bf16 rounding of dpre
          const float r0 = __builtin_amdgcn_sqrtf(bf16_lo(pw[i])), r1 = __builtin_amdgcn_sqrtf(bf16_hi(pw[i]));
          o[i] = pack_bf16x2((2.0f * r0) * acc[fm][fn][2 * i], (2.0f * r1) * acc[fm][fn][2 * i + 1]);
        }
        uint16_t* dst = dpre + m * ld + n;
        *(uint4*)dst = uint4{o[0], o[1], o[2], o[3]};
        *(uint4*)(dst + 8) = uint4{o[4], o[5], o[6], o[7]};
      }
    }
  }
};

// fp32 output: either the final weight gradient (optionally added to what is
// there) or one split-k partial, written to out + split * split_stride.
struct EpiF32 {
  float* out;
  int64_t ld;
  int64_t split_stride;   // elements between split partials (0: single split)
  int accumulate;         // add into out (single split only)

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char*) {
    static_assert(C::PERM, "needs 16 consecutive columns per lane");
    float* base = out + (int64_t)c.split * split_stride;
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      const int64_t m = c.m0 + epi_row<C>(c, fm);
      if (m >= c.M) continue;
#pragma unroll
      for (int fn = 0; fn < C::FN; fn++) {
        const int64_t n = c.n0 + epi_col<C>(c, fn, 0);
        if (n >= c.N) continue;
        float4* dst = (float4*)(base + m * ld + n);
#pragma unroll
        for (int g = 0; g < 4; g++) {
          float4 v = {acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2], acc[fm][fn][4 * g + 3]};
          if (accumulate) {
            const float4 o = dst[g];
            v.x += o.x;
            v.y += o.y;
            v.z += o.z;
            v.w += o.w;
          }
          dst[g] = v;
        }
      }
    }
  }
};

}  // namespace fp8mlp
