// Templated MFMA GEMM core for gfx950 (CDNA4), shared by every contraction of
// the MLP path.
//
// C[m][n] = sum_k A[m][k] * B[k][n], fp32 accumulation, one 256-thread block
// (4 waves of 64, 2 x 2) per BM x BN output tile.  Blocks are sized so that
// OCC of them fit on one CU (registers and LDS), which lets one block's
// epilogue and barrier waits overlap another block's MFMAs.
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
// operand is ever transposed in registers.  A tile holds RB bytes of k per
// row; STAGES tiles are in flight.
//
// bf16 uses v_mfma_f32_32x32x16_bf16; fp8 (OCP e4m3) uses
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit (E8M0 127) block scales.
#pragma once

#include <utility>

#include "common.h"

namespace fp8mlp {

enum { KC = 0, MNC = 1 };

template <int ELT_, int BM_, int BN_, int RB_, int STAGES_, int OCC_, int QL_, int PL_, int REG_ = 0>
struct GemmCfg {
  static constexpr int ELT = ELT_;                 // bytes per element: 2 bf16, 1 e4m3
  // REG == 1: tiles go global -> VGPRs -> LDS (buffer_load_dwordx4 +
  // ds_write_b128), the next tile waiting in registers while the current one
  // is computed; REG == 0: global -> LDS directly (buffer_load ... lds) with
  // STAGES LDS buffers.
  static constexpr int REG = REG_;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int RB = RB_;                   // bytes of k per tile row
  static constexpr int CPR = RB / 16;              // 16-byte chunks per k-contiguous row
  static constexpr int BK = RB / ELT;              // k per tile
  static constexpr int STAGES = STAGES_, OCC = OCC_;
  static constexpr int QL = QL_, PL = PL_;
  static constexpr int WTM = BM / 2, WTN = BN / 2; // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int KSTEP = ELT == 2 ? 32 : 64; // bytes of k per MFMA
  static constexpr int SL = RB / KSTEP;            // MFMA k-steps per tile
  static constexpr int Q_BYTES = BM * RB, P_BYTES = BN * RB;
  static constexpr int STAGE_BYTES = Q_BYTES + P_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int Q_LOADS = Q_BYTES / 4096;   // 16 B x 64 lanes x 4 waves per round
  static constexpr int P_LOADS = P_BYTES / 4096;
  static constexpr int LOADS = Q_LOADS + P_LOADS;
  // the P operand's row order gives each lane 16 consecutive n, except for
  // transposed fp8 reads, which give 4 runs of 4
  static constexpr bool PERM = !(ELT == 1 && PL == MNC);
  static_assert(RB == 64 || RB == 128, "row bytes");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(Q_BYTES % 4096 == 0 && P_BYTES % 4096 == 0, "loads");
  // the row-contiguous swizzle XORs bits 6-7 (bf16) or 4-6 (e4m3) of the byte offset
  static_assert(QL == KC || (BM * ELT) % (ELT == 2 ? 256 : 128) == 0, "row-contiguous Q tile rows");
  static_assert(PL == KC || (BN * ELT) % (ELT == 2 ? 256 : 128) == 0, "row-contiguous P tile rows");
  static_assert(LDS_BYTES * OCC <= 160 * 1024, "LDS");
  static_assert(LOADS * (STAGES - 2) < 64, "vmcnt");
  static_assert(REG == 0 || (REG == 1 && STAGES == 2), "register staging: two LDS buffers, one register set");
};

struct GemmArgs {
  const void* q;      // GEMM A matrix (rows m)
  int64_t ldq;        // elements
  const void* p;      // GEMM B matrix (columns n)
  int64_t ldp;
  int64_t M, N, K;    // full problem
  int tiles_m, tiles_n, splits;
  int64_t k_per_split;  // multiple of BK
  int stagger;          // > 0: blocks of the second residency slot start ~stagger x 4 us late
  int group_m;          // tile rows per group of the tile order (set by launch_gemm)
};

// Per-block tile coordinates handed to the epilogue.
struct TileCtx {
  int64_t m0, n0;     // tile origin
  int tm, tn, split;
  int wm, wn, lane;
  int64_t M, N;
};

// ------------------------------------------------------------------ swizzles
// k-contiguous tiles: rows of CPR 16-byte chunks; the chunk index is XOR-ed
// with a function of the row so that the fragment reads of 8 or 16
// consecutive lanes hit distinct banks (Q rows are read in order, P rows in
// the perm_p order below).
template <int CPR>
__device__ __forceinline__ int swz_rows_q(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 2)) & 3;
}
template <int CPR>
__device__ __forceinline__ int swz_rows_p(int n) {
  if constexpr (CPR == 8) return ((n ^ (n >> 2)) & 1) | (n & 2) | ((n >> 2) & 4);
  else return (((n >> 1) ^ (n >> 2)) & 1) | (((n >> 4) & 1) << 1);
}
// row-contiguous tiles: rows are k; the byte offset within a row is XOR-ed
// with (k & 3) << 6 (bf16) or (k & 7) << 4 (e4m3).
template <int ELT>
__device__ __forceinline__ int swz_mn(int k) {
  return ELT == 2 ? ((k & 3) << 6) : ((k & 7) << 4);
}

// P row permutation inside a 32-row fragment: MFMA row p' = 8g + 4h + r holds
// tile row 16h + 4g + r, so lane half h ends up with rows 16h .. 16h+15.
__device__ __forceinline__ int perm_p(int p) { return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3); }

template <int ELT>
struct FragT;
template <>
struct FragT<2> {
  using type = bf16x8_t;   // 8 bf16 of k per lane (32x32x16 MFMA operand)
};
template <>
struct FragT<1> {
  using type = i32x8;      // 32 e4m3 of k per lane (32x32x64 MFMA operand)
};

// Two transposed 4 x bf16 reads (k .. k+3, k+4 .. k+7) -> one 8 x bf16 operand.
__device__ __forceinline__ bf16x8_t tr16_pair(i16x4 lo, i16x4 hi) {
  const i32x4 v = {(int)((uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16)),
                   (int)((uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16)),
                   (int)((uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16)),
                   (int)((uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16))};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Scheduling groups for one k-tile: the reads of slice 0 first, then for each
// of the SL slices NM MFMAs with the NR reads of the next slice spread evenly
// between them (none after the last slice).
template <int NM, int NR, int I>
__device__ __forceinline__ void sched_slice() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int r = (NR * (I + 1)) / NM - (NR * I) / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    sched_slice<NM, NR, I + 1>();
  }
}
template <int NM, int NR, int SL>
__device__ __forceinline__ void sched_tile() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  [&]<int... S>(std::integer_sequence<int, S...>) {
    ((S + 1 < SL ? sched_slice<NM, NR, 0>() : sched_slice<NM, 0, 0>()), ...);
  }(std::make_integer_sequence<int, SL>{});
}

// LDS-linear 16-byte chunk c of an operand tile -> byte offset in global
// memory relative to the tile origin (at k = 0 of this block's range).
template <class C, int L, int ROWS, bool IS_P>
__device__ __forceinline__ uint32_t load_off(int c, int64_t ld_bytes) {
  if constexpr (L == KC) {
    const int row = c / C::CPR, pc = c % C::CPR;
    const int lc = pc ^ (IS_P ? swz_rows_p<C::CPR>(row) : swz_rows_q<C::CPR>(row));
    return (uint32_t)(row * ld_bytes + lc * 16);
  } else {
    constexpr int MCPR = ROWS * C::ELT / 16;   // chunks per LDS row (one k)
    const int k = c / MCPR, pc = c % MCPR;
    const int lc = ((pc * 16) ^ swz_mn<C::ELT>(k)) / 16;
    return (uint32_t)(k * ld_bytes + lc * 16);
  }
}

// ------------------------------------------------------------------ kernel
template <class C, class Epi>
__global__ void __launch_bounds__(256, C::OCC) gemm_kernel(GemmArgs a, Epi epi) {
  // the pipeline buffers, reused by the epilogue once the last tile is read
  constexpr int EPI_BYTES = Epi::template lds_bytes<C>();
  constexpr int SMEM = C::LDS_BYTES > EPI_BYTES ? C::LDS_BYTES : EPI_BYTES;
  static_assert(SMEM * C::OCC <= 160 * 1024, "LDS with the epilogue's staging");
  __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
  FP8MLP_LDS char* smem = (FP8MLP_LDS char*)smem_raw;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;

  // With two blocks per CU, blocks that start together reach their
  // epilogues together and leave the matrix cores idle meanwhile.  Delaying
  // the blocks that the dispatcher places in the second residency slot of
  // each CU (the second 256 of the first 512) shifts the two slots by part of
  // a tile; later blocks inherit the offset when they take over a slot.
  if (C::OCC > 1 && a.stagger > 0 && blockIdx.x >= 256 && blockIdx.x < 512) {
    for (int i = 0; i < a.stagger; i++) __builtin_amdgcn_s_sleep(127);
  }

  // ---- tile assignment.  Consecutive blocks go round-robin over the 8 XCDs;
  // xcd_remap gives each XCD a contiguous run of logical tiles.  Logical
  // order: split-k index slowest (blocks of one split share their k-range of
  // both operands), then groups of GROUP_M tile rows, inside a group the row
  // fastest, so the tiles an XCD runs at once form a near-square window that
  // shares few A- and B-slabs in that XCD's L2.
  const int GROUP_M = a.group_m;
  int t = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = a.tiles_m * a.tiles_n;
  const int split = t / per_split;
  t -= split * per_split;
  const int per_group = GROUP_M * a.tiles_n;
  const int grp = t / per_group, rem = t - grp * per_group;
  const int gm = min(GROUP_M, a.tiles_m - grp * GROUP_M);
  const int tm = grp * GROUP_M + rem % gm, tn = rem / gm;
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
    if constexpr (C::QL == KC) {
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
  for (int j = 0; j < C::Q_LOADS; j++) qoff[j] = load_off<C, C::QL, C::BM, false>((j * 4 + wave) * 64 + lane, ldq_b);
#pragma unroll
  for (int j = 0; j < C::P_LOADS; j++) poff[j] = load_off<C, C::PL, C::BN, true>((j * 4 + wave) * 64 + lane, ldp_b);
  const uint32_t qstep = C::QL == KC ? (uint32_t)C::RB : (uint32_t)(C::BK * ldq_b);
  const uint32_t pstep = C::PL == KC ? (uint32_t)C::RB : (uint32_t)(C::BK * ldp_b);

  // register staging: the next tile in flight in VGPRs
  i32x4 rq_regs[1][C::REG ? C::Q_LOADS : 1], rp_regs[1][C::REG ? C::P_LOADS : 1];
  auto gload = [&](int kt, int slot) {
    const uint32_t dq = (uint32_t)kt * qstep, dp = (uint32_t)kt * pstep;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++)
      rq_regs[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[j] + dq, 0, 0);
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++)
      rp_regs[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(rp, poff[j] + dp, 0, 0);
  };
  auto dswrite = [&](int stage, int slot) {
    FP8MLP_LDS char* sq = smem + stage * C::STAGE_BYTES;
    FP8MLP_LDS char* sp = sq + C::Q_BYTES;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++)
      *(FP8MLP_LDS i32x4*)(sq + ((j * 4 + wave) * 64 + lane) * 16) = rq_regs[slot][j];
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++)
      *(FP8MLP_LDS i32x4*)(sp + ((j * 4 + wave) * 64 + lane) * 16) = rp_regs[slot][j];
  };

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
  // Q: MFMA column q = lane & 31  -> tile row wm*WTM + fm*32 + (lane & 31)
  // P: MFMA row p' = lane & 31   -> tile row wn*WTN + fn*32 + perm_p(p') (or p')
  int qrow_off, prow_off;   // per-lane part; fragments add fm*32 / fn*32 rows
  int qx, px;               // swizzle terms
  if constexpr (C::QL == KC) {
    const int r = wm * C::WTM + (lane & 31);
    qrow_off = r * C::RB;
    qx = swz_rows_q<C::CPR>(r);
  } else {
    // transposed read: source lanes supply k = .. + ((lane & 15) >> 2) and
    // 4 consecutive rows starting at mb
    const int kq = (lane & 15) >> 2;
    const int mb = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    qrow_off = (8 * h + kq) * (C::BM * 2);
    qx = 2 * (wm * C::WTM + mb);
  }
  if constexpr (C::PL == KC) {
    const int r = wn * C::WTN + (C::PERM ? perm_p(lane & 31) : (lane & 31));
    prow_off = r * C::RB;
    px = swz_rows_p<C::CPR>(r);
  } else if constexpr (C::ELT == 2) {
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

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; i++)
#pragma unroll
    for (int j = 0; j < C::FN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // ---- fragment loaders and the MFMA
  using Frag = typename FragT<C::ELT>::type;
  constexpr int QR = C::QL == KC ? (C::ELT == 2 ? 1 : 2) : (C::ELT == 2 ? 2 : 4);  // LDS reads per fragment
  constexpr int PR = C::PL == KC ? (C::ELT == 2 ? 1 : 2) : (C::ELT == 2 ? 2 : 4);
  constexpr int NREADS = C::FM * QR + C::FN * PR;

  auto load_q = [&](const FP8MLP_LDS char* sq, int s, int fm) -> Frag {
    if constexpr (C::ELT == 2) {
      if constexpr (C::QL == KC) {
        const uint32_t off = qrow_off + fm * 32 * C::RB + (((2 * s + h) ^ qx) * 16);
        return __builtin_bit_cast(bf16x8_t, lds_read_b128(sq, off));
      } else {
        const int kq = (lane & 15) >> 2;
        const uint32_t col = (uint32_t)((qx + fm * 64) ^ ((kq & 3) << 6));
        const uint32_t o0 = qrow_off + (16 * s) * (C::BM * 2) + col;
        return tr16_pair(lds_read_tr16(sq, o0), lds_read_tr16(sq, o0 + 4 * (C::BM * 2)));
      }
    } else {
      const uint32_t base = qrow_off + fm * 32 * C::RB;
      const i32x4 v0 = lds_read_b128(sq, base + (((4 * s + 2 * h) ^ qx) * 16));
      const i32x4 v1 = lds_read_b128(sq, base + (((4 * s + 2 * h + 1) ^ qx) * 16));
      return i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
  };
  auto load_p = [&](const FP8MLP_LDS char* sp, int s, int fn) -> Frag {
    if constexpr (C::ELT == 2) {
      if constexpr (C::PL == KC) {
        const uint32_t off = prow_off + fn * 32 * C::RB + (((2 * s + h) ^ px) * 16);
        return __builtin_bit_cast(bf16x8_t, lds_read_b128(sp, off));
      } else {
        const int kq = (lane & 15) >> 2;
        const uint32_t col = (uint32_t)((px + fn * 64) ^ ((kq & 3) << 6));
        const uint32_t o0 = prow_off + (16 * s) * (C::BN * 2) + col;
        return tr16_pair(lds_read_tr16(sp, o0), lds_read_tr16(sp, o0 + 4 * (C::BN * 2)));
      }
    } else {
      if constexpr (C::PL == KC) {
        const uint32_t base = prow_off + fn * 32 * C::RB;
        const i32x4 v0 = lds_read_b128(sp, base + (((4 * s + 2 * h) ^ px) * 16));
        const i32x4 v1 = lds_read_b128(sp, base + (((4 * s + 2 * h + 1) ^ px) * 16));
        return i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      } else {
        const int kq = (lane & 15) >> 1;
        const uint32_t col = (uint32_t)((px + fn * 32) ^ ((kq & 7) << 4));
        const uint32_t o0 = prow_off + (64 * s) * C::BN + col;
        const i32x2 r0 = lds_read_tr8(sp, o0);
        const i32x2 r1 = lds_read_tr8(sp, o0 + 8 * C::BN);
        const i32x2 r2 = lds_read_tr8(sp, o0 + 16 * C::BN);
        const i32x2 r3 = lds_read_tr8(sp, o0 + 24 * C::BN);
        return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
      }
    }
  };
  auto mma = [](const Frag& p, const Frag& q, const f32x16& c) -> f32x16 {
    if constexpr (C::ELT == 2) {
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(p, q, c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(p, q, c, 0, 0, 0, 127, 0, 127);
    }
  };

  // ---- main loop: one barrier per tile
  if constexpr (C::REG > 0) {
    // tile kt+1 waits in registers while tile kt is computed from LDS; at the
    // end of the iteration it goes to the other LDS buffer and the registers
    // are refilled with tile kt+2
    if (KT > 0) {
      gload(0, 0);
      wait_vmcnt<0>();
      dswrite(0, 0);
      if (KT > 1) gload(1, 0);
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; s++)
      if (s < KT) issue(s, s);
  }

  auto ktile = [&](int kt) {
    if constexpr (C::REG == 0) {
      if (kt + C::STAGES - 2 < KT) {
        wait_vmcnt<C::LOADS * (C::STAGES - 2)>();
      } else {
        wait_vmcnt<0>();
      }
    }
    __syncthreads();
    if constexpr (C::REG == 0) {
      if (kt + C::STAGES - 1 < KT) issue(kt + C::STAGES - 1, (kt + C::STAGES - 1) % C::STAGES);
    }

    const FP8MLP_LDS char* sq = smem + (kt % C::STAGES) * C::STAGE_BYTES;
    const FP8MLP_LDS char* sp = sq + C::Q_BYTES;
    // Fragments are double-buffered across the k-slices of the tile: the LDS
    // reads of slice s+1 are issued while the MFMAs of slice s run, and the
    // scheduling groups interleave them one by one.
    Frag qf[2][C::FM], pf[2][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) qf[0][fm] = load_q(sq, 0, fm);
#pragma unroll
    for (int fn = 0; fn < C::FN; fn++) pf[0][fn] = load_p(sp, 0, fn);
#pragma unroll
    for (int s = 0; s < C::SL; s++) {
      if (s + 1 < C::SL) {
#pragma unroll
        for (int fm = 0; fm < C::FM; fm++) qf[(s + 1) & 1][fm] = load_q(sq, s + 1, fm);
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) pf[(s + 1) & 1][fn] = load_p(sp, s + 1, fn);
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) acc[fm][fn] = mma(pf[s & 1][fn], qf[s & 1][fm], acc[fm][fn]);
    }
    sched_tile<C::FM * C::FN, NREADS, C::SL>();
    if constexpr (C::REG > 0) {
      if (kt + 1 < KT) {
        wait_vmcnt<0>();
        dswrite((kt + 1) & 1, 0);
        if (kt + 2 < KT) gload(kt + 2, 0);
      }
    }
  };
  for (int kt = 0; kt < KT; kt++) ktile(kt);

  TileCtx ctx{m0, n0, tm, tn, split, wm, wn, lane, a.M, a.N};
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
