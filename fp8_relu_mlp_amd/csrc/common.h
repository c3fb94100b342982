// Device helpers shared by the gfx950 kernels of libfp8mlp.
//
// Number formats follow the method as described on the speedrun pages:
//  * bf16 activations / weights ("A Retrospective on Our World Records",
//    Modded-NanoGPT Main Track: the BF16 post-activation kept for backward),
//  * OCP e4m3 ("E4M3FN", largest finite 448) for the FP8 copies (NanoGPT
//    Speedrun (Track 1), "Changes vs Record #83" item 1: float8_e4m3).
// Both conversions use the CDNA4 hardware converters, which round to nearest
// even; the e4m3 converter maps |x| > 464 to NaN, so values are clamped to
// +-448 first (saturating encode, NaN kept as NaN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mlp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;

#define FP8MLP_LDS __attribute__((address_space(3)))

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- formats
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Saturate to the largest finite e4m3 magnitude; NaN stays NaN.
__device__ __forceinline__ float sat_e4m3(float x) {
  return fabsf(x) > kE4M3Max ? __builtin_copysignf(kE4M3Max, x) : x;
}
// Four fp32 values -> four e4m3 codes (byte 0 = a), RNE, saturating.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
  return (uint32_t)w;
}

// e4m3 codes of four values that are >= +0 or NaN (byte 0 = a).  The
// converter rounds to nearest even and already gives 0x7E on (448, 464];
// above 464 and at +inf it gives 0x7F, which is rewritten to 0x7E
// (saturation), while a NaN input gives 0xFF and stays a NaN code.  Cheaper
// than clamping each value before the conversion.
__device__ __forceinline__ uint32_t pack_e4m3x4_nonneg(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  const uint32_t u = (uint32_t)w;
  const uint32_t m = u ^ 0x7f7f7f7fu;                        // bytes that were 0x7F are now 0
  const uint32_t nz = ((m & 0x7f7f7f7fu) + 0x7f7f7f7fu) | m;  // bit 7 of a byte: byte != 0
  const uint32_t z = ~nz & 0x80808080u;                      // bit 7 of a byte: code was 0x7F
  return u - (z >> 7);                                        // 0x7F -> 0x7E, no borrow
}

// e4m3 codes of four values known to lie in [+0, 464] (no NaN): the
// converter's round-to-nearest-even result needs no saturation fix-up there
// ((448, 464] already rounds to 0x7E).  The first conversion's other half is
// overwritten by the second, so any register serves as its "old" operand.
__device__ __forceinline__ uint32_t pack_e4m3x4_inrange(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Keeps the compiler from re-deriving a value from its operands (the packed
// bf16 word below would otherwise be re-converted value by value).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// relu(a)^2 with NaN kept and -inf sent to 0: IEEE maximum(a, +0) (NaN
// propagating, one v_maximum3_f32 on gfx950) then a square.
__device__ __forceinline__ float relu_sq(float a) {
  const float r = __builtin_elementwise_maximum(a, 0.0f);
  return r * r;
}

// Running max of |x| over two packed bf16 values, on fp32 bit patterns.
__device__ __forceinline__ uint32_t max_abs_bf16x2(uint32_t m, uint32_t w) {
  const uint32_t a0 = (w & 0x7fffu) << 16, a1 = (w >> 16 & 0x7fffu) << 16;
  m = a0 > m ? a0 : m;
  return a1 > m ? a1 : m;
}

// ---------------------------------------------------------------- scales
// Quantisation multiplier from an amax and a safety margin:
// scale = 448 / (margin * amax), each operation rounded to fp32; a
// non-positive / non-finite denominator or an overflowing quotient gives 1.
// ("A Retrospective on Our World Records", Main Track: the FP8 scale at step
// t comes from amax(t-1) times a safety margin.)  The division is IEEE
// correctly rounded: the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt.
__device__ __forceinline__ float scale_from_amax(float amax, float margin) {
  float denom = margin * amax;
  if (!(denom > 0.0f) || !(denom <= 3.402823466e38f)) return 1.0f;
  float s = kE4M3Max / denom;
  if (!(s <= 3.402823466e38f)) return 1.0f;
  return s;
}

// ---------------------------------------------------------------- memory
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
  // word3 0x00020000: raw (untyped) 32-bit data format, no swizzle.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
// 16 bytes per lane from a buffer straight into LDS: lane i writes
// lds_wave_base + 16*i.  Offsets past the buffer's size read as zero.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, FP8MLP_LDS void* lds_wave_base,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voffset, 0, 0, 0);
}
// The same with the non-temporal (streaming) cache policy, for data read once.
__device__ __forceinline__ void buffer_load_lds16_stream(__amdgpu_buffer_rsrc_t r, FP8MLP_LDS void* lds_wave_base,
                                                         uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voffset, 0, 0, 2 /* nt */);
}
// Non-temporal stores of 16 and 8 bytes (written once, not re-read soon).
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  __builtin_nontemporal_store(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, (i32x4*)p);
}
__device__ __forceinline__ void store_stream(void* p, uint2 v) {
  __builtin_nontemporal_store(i32x2{(int)v.x, (int)v.y}, (i32x2*)p);
}

// Non-temporal buffer stores at a 32-bit byte offset from a resource's base;
// offsets at or past the resource's size are dropped by the hardware.
__device__ __forceinline__ void buffer_store_stream16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, r, off, 0, 2 /* nt */);
}
__device__ __forceinline__ void buffer_store_stream8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)v.x, (int)v.y}, r, off, 0, 2 /* nt */);
}

// s_waitcnt vmcnt(n) with the other counters left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Block barrier for the GEMM main loops: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads, including loads that write LDS directly, whose
// completion the loops wait for explicitly (and only where needed).  The
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ i32x4 lds_read_b128(const FP8MLP_LDS char* base, uint32_t off) {
  return *(const FP8MLP_LDS i32x4*)(base + off);
}
// The transposing reads.  Their base is declared __restrict__ so that the
// read carries alias information: an LDS read without it makes the compiler
// wait for every buffer_load ... lds still in flight (vmcnt(0)) before it, in
// case that load writes the bytes read, which in the GEMM main loops would
// cut the prefetch distance of every k-tile to one phase.  Those loops order
// their LDS reads after the loads they need with explicit vmcnt waits and
// block barriers.
__device__ __forceinline__ i16x4 lds_read_tr16(const FP8MLP_LDS char* __restrict__ base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FP8MLP_LDS i16x4*)(base + off));
}
__device__ __forceinline__ i32x2 lds_read_tr8(const FP8MLP_LDS char* __restrict__ base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FP8MLP_LDS i32x2*)(base + off));
}

// ---------------------------------------------------------------- reductions
// Max over the wave of a non-negative-or-NaN float carried as its bit pattern
// (unsigned order: +0 < ... < +inf < NaN), so NaN propagates exactly.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Block index -> logical tile index such that the blocks the hardware places
// on one XCD (consecutive block ids go round-robin over the 8 XCDs) process a
// contiguous range of tiles, which then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int x = b & 7, i = b >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

}  // namespace fp8mlp
