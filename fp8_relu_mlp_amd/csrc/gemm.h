// Templated MFMA GEMM core for gfx950 (CDNA4), shared by every contraction of
// the MLP path.
//
// C[m][n] = sum_k A[m][k] * B[k][n], fp32 accumulation, one 256-thread block
// (4 waves of 64, 2 x 2) per BM x BN output tile.
//
// Operand naming follows the MFMA: the MFMA "A" operand holds rows p and is fed
// with the GEMM's B matrix (P[n][k]); the MFMA "B" operand holds columns q and
// is fed with the GEMM's A matrix (Q[k][m]).  The MFMA result D[p][q] leaves
// each lane with consecutive n for one m, which is what a row-major C wants.
//
// Global layouts (per operand, template parameters):
//   KC  "k-contiguous": element (row, k) at row * ld + k      (e.g. X, W1 in
//        the forward, post_q)
//   MNC "row-contiguous": element (row, k) at k * ld + row    (e.g. W2 and W1
//        read in the backward, the fp8 weight caches, dpre^T / dY^T)
// Both go global -> LDS with buffer_load ... lds (16 bytes per lane, no VGPR
// staging; reads past the buffer's end return zero, which masks ragged M / K
// tails).  KC tiles are read by ds_read_b128, MNC tiles by the CDNA4
// transposing reads ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (fp8), so no
// operand is ever transposed in registers.
//
// bf16 uses v_mfma_f32_32x32x16_bf16; fp8 (OCP e4m3) uses
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit (E8M0 127) block scales.
#pragma once

#include "common.h"

namespace fp8mlp {

enum { KC = 0, MNC = 1 };

template <int ELT_, int BM_, int BN_, int STAGES_, int QL_, int PL_, bool QCVT_ = false>
struct GemmCfg {
  static constexpr int ELT = ELT_;                 // bytes per element: 2 bf16, 1 e4m3
  // QCVT: the A matrix is bf16 in memory and is quantised to e4m3 in LDS
  // (e4m3 MFMA, k-contiguous A only)
  static constexpr bool QCVT = QCVT_;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int BK = 128 / ELT;             // 128 bytes of k per tile row
  static constexpr int STAGES = STAGES_;
  static constexpr int QL = QL_, PL = PL_;
  static constexpr int WTM = BM / 2, WTN = BN / 2; // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int Q_BYTES = BM * 128 * (QCVT ? 2 : 1), P_BYTES = BN * 128;
  static constexpr int STAGE_BYTES = Q_BYTES + P_BYTES;
  static constexpr int QF_BYTES = QCVT ? BM * 128 : 0;   // quantised A tile
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + QF_BYTES;
  static constexpr int Q_LOADS = Q_BYTES / 4096;   // 16 B x 64 lanes x 4 waves per round
  static constexpr int P_LOADS = P_BYTES / 4096;
  static constexpr int LOADS = Q_LOADS + P_LOADS;
  // the P operand's row order gives each lane 16 consecutive n, except for
  // transposed fp8 reads, which give 4 runs of 4
  static constexpr bool PERM = !(ELT == 1 && PL == MNC);
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(Q_BYTES % 4096 == 0 && P_BYTES % 4096 == 0, "loads");
  static_assert(QL == KC || (BM * ELT) % 256 == 0, "row-contiguous Q tile rows must be 256-byte multiples");
  static_assert(PL == KC || (BN * ELT) % 256 == 0, "row-contiguous P tile rows must be 256-byte multiples");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(!QCVT || (ELT == 1 && QL == KC), "quantise-on-load needs an e4m3 GEMM with k-contiguous A");
};

struct GemmArgs {
  const void* q;      // GEMM A matrix (rows m)
  int64_t ldq;        // elements
  const void* p;      // GEMM B matrix (columns n)
  int64_t ldp;
  int64_t M, N, K;    // full problem
  int tiles_m, tiles_n, splits;
  int64_t k_per_split;  // multiple of BK
  const float* q_scale; // QCVT: multiplier applied to A before the e4m3 encode
};

// Per-block tile coordinates handed to the epilogue.
struct TileCtx {
  int64_t m0, n0;     // tile origin
  int tm, tn, split;
  int wm, wn, lane;
  int64_t M, N;
  uint32_t qamax;     // QCVT: max |A| bits over the elements this thread converted
};

// ------------------------------------------------------------------ swizzles
// k-contiguous tiles: 128-byte rows of 8 16-byte chunks; the chunk index is
// XOR-ed with a function of the row so that the fragment reads of 8 or 16
// consecutive lanes hit distinct banks.
__device__ __forceinline__ int swz_rows_q(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_rows_p(int n) { return ((n ^ (n >> 2)) & 1) | (n & 2) | ((n >> 2) & 4); }
// row-contiguous tiles: rows are k; the byte offset within a row is XOR-ed
// with (k & 3) << 6 (bf16) or (k & 7) << 4 (e4m3).
template <int ELT>
__device__ __forceinline__ int swz_mn(int k) {
  return ELT == 2 ? ((k & 3) << 6) : ((k & 7) << 4);
}

// P row permutation inside a 32-row fragment: MFMA row p' = 8g + 4h + r holds
// tile row 16h + 4g + r, so lane half h ends up with rows 16h .. 16h+15.
__device__ __forceinline__ int perm_p(int p) { return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3); }

template <class C>
struct GemmCore {
  // ---------------------------------------------------------------- loads
  // LDS-linear 16-byte chunk c of an operand tile -> byte offset in global
  // memory relative to the tile origin (at k = 0 of this block's range).
  template <int L, int ROWS, bool IS_P>
  __device__ static __forceinline__ uint32_t load_off(int c, int64_t ld_bytes) {
    if constexpr (!IS_P && C::QCVT) {
      return (uint32_t)((c >> 4) * ld_bytes + (c & 15) * 16);
    } else if constexpr (L == KC) {
      const int row = c >> 3, pc = c & 7;
      const int lc = pc ^ (IS_P ? swz_rows_p(row) : swz_rows_q(row));
      return (uint32_t)(row * ld_bytes + lc * 16);
    } else {
      constexpr int CPR = ROWS * C::ELT / 16;   // chunks per LDS row (one k)
      const int k = c / CPR, pc = c % CPR;
      const int lc = ((pc * 16) ^ swz_mn<C::ELT>(k)) / 16;
      return (uint32_t)(k * ld_bytes + lc * 16);
    }
  }
  template <int L, bool IS_Q = false>
  __device__ static __forceinline__ uint32_t k_step_bytes(int64_t ld_bytes) {
    if (IS_Q && C::QCVT) return 256u;
    return L == KC ? 128u : (uint32_t)(C::BK * ld_bytes);
  }
};

// ------------------------------------------------------------------ kernel
template <class C, class Epi>
__global__ void __launch_bounds__(256, 1) gemm_kernel(GemmArgs a, Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
  FP8MLP_LDS char* smem = (FP8MLP_LDS char*)smem_raw;
  using Core = GemmCore<C>;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile assignment (XCD-aware; split fastest, then n, then m)
  int t = xcd_remap(blockIdx.x, gridDim.x);
  const int split = t % a.splits;
  t /= a.splits;
  const int tn = t % a.tiles_n, tm = t / a.tiles_n;
  const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
  const int64_t kb = (int64_t)split * a.k_per_split;
  const int64_t ke = min(a.K, kb + a.k_per_split);
  const int KT = (int)((ke - kb + C::BK - 1) / C::BK);

  // ---- buffer resources anchored at the tile origin
  const int64_t ldq_b = a.ldq * C::ELT, ldp_b = a.ldp * C::ELT;
  __amdgpu_buffer_rsrc_t rq, rp;
  {
    const char* q = (const char*)a.q;
    const char* p = (const char*)a.p;
    if constexpr (C::QCVT) {
      rq = make_rsrc(q + m0 * ldq_b * 2 + kb * 2, (uint64_t)((a.M - m0) * ldq_b * 2 - kb * 2));
    } else if constexpr (C::QL == KC) {
      rq = make_rsrc(q + m0 * ldq_b + kb * C::ELT, (uint64_t)((a.M - m0) * ldq_b - kb * C::ELT));
    } else {
      rq = make_rsrc(q + kb * ldq_b + m0 * C::ELT, (uint64_t)((ke - kb) * ldq_b - m0 * C::ELT));
    }
    if constexpr (C::PL == KC) {
      rp = make_rsrc(p + n0 * ldp_b + kb * C::ELT, (uint64_t)((a.N - n0) * ldp_b - kb * C::ELT));
    } else {
      rp = make_rsrc(p + kb * ldp_b + n0 * C::ELT, (uint64_t)((ke - kb) * ldp_b - n0 * C::ELT));
    }
  }
  // Rows k >= ke of a row-contiguous operand fall past the resource's end and
  // load as zero; for k-contiguous operands K is a multiple of BK.

  uint32_t qoff[C::Q_LOADS], poff[C::P_LOADS];
#pragma unroll
  for (int j = 0; j < C::Q_LOADS; j++)
    qoff[j] = Core::template load_off<C::QL, C::BM, false>((j * 4 + wave) * 64 + lane,
                                                           C::QCVT ? ldq_b * 2 : ldq_b);
#pragma unroll
  for (int j = 0; j < C::P_LOADS; j++)
    poff[j] = Core::template load_off<C::PL, C::BN, true>((j * 4 + wave) * 64 + lane, ldp_b);
  const uint32_t qstep = Core::template k_step_bytes<C::QL, true>(ldq_b);
  const uint32_t pstep = Core::template k_step_bytes<C::PL>(ldp_b);

  auto issue = [&](int kt, int stage) {
    FP8MLP_LDS char* sq = smem + stage * C::STAGE_BYTES;
    FP8MLP_LDS char* sp = sq + C::Q_BYTES;
    const uint32_t dq = (uint32_t)kt * qstep, dp = (uint32_t)kt * pstep;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++) buffer_load_lds16(rq, sq + (j * 4 + wave) * 1024, qoff[j] + dq);
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++) buffer_load_lds16(rp, sp + (j * 4 + wave) * 1024, poff[j] + dp);
  };

  // ---- fragment read offsets (bytes within a stage's Q / P tile)
  const int h = lane >> 5;
  // Q: MFMA column q = lane & 31 -> tile row wm*WTM + fm*32 + (lane & 31)
  // P: MFMA row p' = lane & 31  -> tile row wn*WTN + fn*32 + perm_p(p') (or p')
  int qrow_off;   // per-lane part, fragments add fm*32 rows
  int prow_off;
  int qx, px;     // swizzle terms
  if constexpr (C::QL == KC) {
    const int r = wm * C::WTM + (lane & 31);
    qrow_off = r * 128;
    qx = swz_rows_q(r);
  } else {
    // transposed read: source lane supplies (k = .. + ((lane & 15) >> 2) [bf16]
    // or ((lane & 15) >> 1) [fp8], rows base ..)
    if constexpr (C::ELT == 2) {
      const int kq = (lane & 15) >> 2;
      const int mb = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      qrow_off = (8 * h + kq) * (C::BM * 2);
      qx = 2 * (wm * C::WTM + mb);        // byte within row before swizzle (fm adds 64)
      (void)mb;
    } else {
      const int kq = (lane & 15) >> 1;
      const int nb = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
      qrow_off = (32 * h + kq) * C::BM;
      qx = wm * C::WTM + nb;
    }
  }
  if constexpr (C::PL == KC) {
    const int pr = C::PERM ? perm_p(lane & 31) : (lane & 31);
    const int r = wn * C::WTN + pr;
    prow_off = r * 128;
    px = swz_rows_p(r);
  } else {
    if constexpr (C::ELT == 2) {
      const int kq = (lane & 15) >> 2;
      const int q4 = lane & 3;
      const int mb = 16 * (q4 & 1) + 8 * ((lane >> 4) & 1) + 4 * (q4 >> 1);
      prow_off = (8 * h + kq) * (C::BN * 2);
      px = 2 * (wn * C::WTN + mb);
    } else {
      const int kq = (lane & 15) >> 1;
      const int nb = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
      prow_off = (32 * h + kq) * C::BN;
      px = wn * C::WTN + nb;
    }
  }

  uint32_t qamax_acc = 0;
  const float qs = C::QCVT ? *a.q_scale : 1.0f;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; i++)
#pragma unroll
    for (int j = 0; j < C::FN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // ---- main loop
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; s++)
    if (s < KT) issue(s, s);

  for (int kt = 0; kt < KT; kt++) {
    if (kt + C::STAGES - 2 < KT) {
      wait_vmcnt<C::LOADS * (C::STAGES - 2)>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (kt + C::STAGES - 1 < KT) issue(kt + C::STAGES - 1, (kt + C::STAGES - 1) % C::STAGES);

    const FP8MLP_LDS char* sq = smem + (kt % C::STAGES) * C::STAGE_BYTES;
    const FP8MLP_LDS char* sp = sq + C::Q_BYTES;
    if constexpr (C::QCVT) {
      // bf16 A tile [BM][128 k] (256-byte rows, linear) -> e4m3 tile in the
      // k-contiguous swizzled layout the fragment reads expect.
      FP8MLP_LDS char* qf = smem + C::STAGES * C::STAGE_BYTES;
#pragma unroll
      for (int j = 0; j < C::BM * 16 / 256; j++) {
        const int cidx = j * 256 + threadIdx.x;
        const int row = cidx >> 4, ch = cidx & 15;
        const i32x4 v = lds_read_b128(sq, cidx * 16);
        const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
        qamax_acc = max_abs_bf16x2(qamax_acc, w0);
        qamax_acc = max_abs_bf16x2(qamax_acc, w1);
        qamax_acc = max_abs_bf16x2(qamax_acc, w2);
        qamax_acc = max_abs_bf16x2(qamax_acc, w3);
        const uint32_t lo = pack_e4m3x4(bf16_lo(w0) * qs, bf16_hi(w0) * qs, bf16_lo(w1) * qs, bf16_hi(w1) * qs);
        const uint32_t hi = pack_e4m3x4(bf16_lo(w2) * qs, bf16_hi(w2) * qs, bf16_lo(w3) * qs, bf16_hi(w3) * qs);
        const uint32_t off = row * 128 + ((((ch >> 1) ^ swz_rows_q(row)) * 16) + 8 * (ch & 1));
        *(FP8MLP_LDS i32x2*)(qf + off) = i32x2{(int)lo, (int)hi};
      }
      __syncthreads();
      sq = qf;
    }

    if constexpr (C::ELT == 2) {
#pragma unroll
      for (int s = 0; s < 4; s++) {          // 4 x k16 slices of the 64-wide tile
        bf16x8_t qf[C::FM], pf[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; fm++) {
          if constexpr (C::QL == KC) {
            const uint32_t off = qrow_off + fm * 32 * 128 + (((2 * s + h) ^ qx) * 16);
            qf[fm] = __builtin_bit_cast(bf16x8_t, lds_read_b128(sq, off));
          } else {
            const int kq = (lane & 15) >> 2;
            const uint32_t col = (uint32_t)((qx + fm * 64) ^ ((kq & 3) << 6));
            const uint32_t o0 = qrow_off + (16 * s) * (C::BM * 2) + col;
            i16x4 lo = lds_read_tr16(sq, o0);
            i16x4 hi = lds_read_tr16(sq, o0 + 4 * (C::BM * 2));
            i32x4 v = {(int)((uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16)),
                       (int)((uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16)),
                       (int)((uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16)),
                       (int)((uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16))};
            qf[fm] = __builtin_bit_cast(bf16x8_t, v);
          }
        }
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) {
          if constexpr (C::PL == KC) {
            const uint32_t off = prow_off + fn * 32 * 128 + (((2 * s + h) ^ px) * 16);
            pf[fn] = __builtin_bit_cast(bf16x8_t, lds_read_b128(sp, off));
          } else {
            const int kq = (lane & 15) >> 2;
            const uint32_t col = (uint32_t)((px + fn * 64) ^ ((kq & 3) << 6));
            const uint32_t o0 = prow_off + (16 * s) * (C::BN * 2) + col;
            i16x4 lo = lds_read_tr16(sp, o0);
            i16x4 hi = lds_read_tr16(sp, o0 + 4 * (C::BN * 2));
            i32x4 v = {(int)((uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16)),
                       (int)((uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16)),
                       (int)((uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16)),
                       (int)((uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16))};
            pf[fn] = __builtin_bit_cast(bf16x8_t, v);
          }
        }
#pragma unroll
        for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
          for (int fn = 0; fn < C::FN; fn++)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[fn], qf[fm], acc[fm][fn], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; s++) {          // 2 x k64 steps of the 128-wide tile
        i32x8 qf[C::FM], pf[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; fm++) {
          static_assert(C::QL == KC, "e4m3 A operand is k-contiguous");
          const uint32_t base = qrow_off + fm * 32 * 128;
          i32x4 v0 = lds_read_b128(sq, base + (((4 * s + 2 * h) ^ qx) * 16));
          i32x4 v1 = lds_read_b128(sq, base + (((4 * s + 2 * h + 1) ^ qx) * 16));
          qf[fm] = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) {
          if constexpr (C::PL == KC) {
            const uint32_t base = prow_off + fn * 32 * 128;
            i32x4 v0 = lds_read_b128(sp, base + (((4 * s + 2 * h) ^ px) * 16));
            i32x4 v1 = lds_read_b128(sp, base + (((4 * s + 2 * h + 1) ^ px) * 16));
            pf[fn] = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          } else {
            const int kq = (lane & 15) >> 1;
            const uint32_t col = (uint32_t)((px + fn * 32) ^ ((kq & 7) << 4));
            const uint32_t o0 = prow_off + (64 * s) * C::BN + col;
            i32x2 r0 = lds_read_tr8(sp, o0);
            i32x2 r1 = lds_read_tr8(sp, o0 + 8 * C::BN);
            i32x2 r2 = lds_read_tr8(sp, o0 + 16 * C::BN);
            i32x2 r3 = lds_read_tr8(sp, o0 + 24 * C::BN);
            pf[fn] = i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
          }
        }
#pragma unroll
        for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
          for (int fn = 0; fn < C::FN; fn++)
            acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pf[fn], qf[fm], acc[fm][fn], 0, 0, 0,
                                                                          127, 0, 127);
      }
    }
  }

  TileCtx ctx{m0, n0, tm, tn, split, wm, wn, lane, a.M, a.N, qamax_acc};
  epi.template run<C>(ctx, acc, smem);
}

// ------------------------------------------------------------------ epilogue helpers
// Row (m) held by this lane for fragment fm, relative to the tile origin.
template <class C>
__device__ __forceinline__ int epi_row(const TileCtx& c, int fm) {
  return c.wm * C::WTM + fm * 32 + (c.lane & 31);
}
// Column (n) of accumulator element e of fragment fn, relative to the tile origin.
template <class C>
__device__ __forceinline__ int epi_col(const TileCtx& c, int fn, int e) {
  const int h = c.lane >> 5;
  if constexpr (C::PERM) {
    return c.wn * C::WTN + fn * 32 + 16 * h + e;
  } else {
    return c.wn * C::WTN + fn * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
  }
}

}  // namespace fp8mlp
