// Templated MFMA GEMM core for gfx950 (CDNA4), shared by every contraction of
// the MLP path.
//
// C[m][n] = sum_k A[m][k] * B[k][n], fp32 accumulation, one block per BM x BN
// output tile, in one of two kernels:
//   gemm_kernel     256 threads (4 waves of 64, 2 x 2); OCC blocks fit on one
//                   CU (registers and LDS), so one block's epilogue and
//                   barrier waits overlap another block's MFMAs.
//   gemm_pp_kernel  512 threads in two groups of four waves, one block per
//                   CU; the groups take turns between fragment reads / global
//                   loads and MFMAs.  With QB == 3 the Q operand has three
//                   LDS buffers and is loaded two k-tiles ahead.
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
// row; STAGES tiles (two for the two-group kernel, with QB Q buffers) are in
// flight.
//
// bf16 uses v_mfma_f32_32x32x16_bf16; fp8 (OCP e4m3) uses
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit (E8M0 127) block scales.
#pragma once

#include <utility>

#include "common.h"

namespace fp8mlp {

enum { KC = 0, MNC = 1 };

// Which contraction of the path a kernel instance serves.  It is a template
// argument of the kernels only so that every launch site has its own kernel
// symbol, which profilers report per symbol.
enum : int {
  KID_UP = 1, KID_DOWN8, KID_DOWN_BF16, KID_DPOST, KID_DX, KID_DW1, KID_DW2, KID_LINEAR, KID_UP8,
  KID_CE_STATS, KID_CE_GRAD, KID_CE_DX, KID_CE_DW, KID_CE8_STATS, KID_CE8_GRAD, KID_DW
};

template <int ELT_, int BM_, int BN_, int RB_, int STAGES_, int OCC_, int QL_, int PL_, int REG_ = 0, int NW_ = 4,
          int PELT_ = 0, int QB_ = 2>
struct GemmCfg {
  static constexpr int ELT = ELT_;                 // bytes per element: 2 bf16, 1 e4m3
  // bytes per element of the P operand in memory and LDS (default ELT).
  // PELT == 1 with ELT == 2: an e4m3 P operand under the bf16 MFMA, widened
  // to bf16 exactly (every e4m3 value is a bf16 value) as its fragments are
  // read; row-contiguous only.
  static constexpr int PELT = PELT_ ? PELT_ : ELT_;
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
  // NW == 4: one 256-thread block, 2 x 2 waves, every wave loads and
  // computes.  NW == 8: 512 threads, 2 x 4 waves in two groups of four (one
  // wave of each group per SIMD) that take turns: while one group issues its
  // MFMAs the other reads its next fragments and issues the global loads
  // (gemm_pp_kernel).
  static constexpr int NW = NW_, NT = 64 * NW_;
  static constexpr int WTM = BM / 2, WTN = BN / (NW_ / 2); // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int KSTEP = ELT == 2 ? 32 : 64; // bytes of k per MFMA
  static constexpr int SL = RB / KSTEP;            // MFMA k-steps per tile
  static constexpr int Q_BYTES = BM * RB, P_BYTES = BN * BK * PELT;
  static constexpr int STAGE_BYTES = Q_BYTES + P_BYTES;
  // QB == 3 (two-group kernel only): three Q buffers beside the two P
  // buffers, so each Q k-tile is loaded two k-tiles ahead of its use and only
  // the P share has to arrive within one.
  static constexpr int QB = QB_;
  static constexpr int LDS_BYTES = QB == 3 ? 3 * Q_BYTES + 2 * P_BYTES : STAGES * STAGE_BYTES;
  static constexpr int Q_LOADS = Q_BYTES / (1024 * NW);   // 16 B x 64 lanes x NW waves per round
  static constexpr int P_LOADS = P_BYTES / (1024 * NW);
  static constexpr int LOADS = Q_LOADS + P_LOADS;
  // the P operand's row order gives each lane 16 consecutive n, except for
  // transposed fp8 reads, which give 4 runs of 4
  static constexpr bool PERM = !((ELT == 1 || PELT == 1) && PL == MNC);
  static_assert(PELT == ELT || (ELT == 2 && PELT == 1 && PL == MNC && REG == 0),
                "e4m3 P under the bf16 MFMA: row-contiguous, loaded straight into LDS");
  static_assert(RB == 64 || RB == 128, "row bytes");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(NW == 4 || NW == 8, "waves");
  static_assert(WTN % 32 == 0 && WTM % 32 == 0, "wave tile");
  static_assert(Q_BYTES % (1024 * NW) == 0 && P_BYTES % (1024 * NW) == 0, "loads");
  static_assert(NW == 4 || (REG == 0 && STAGES == 2 && OCC == 1), "the two-group kernel: direct loads, two buffers");
  static_assert(QB == 2 || (QB == 3 && NW == 8), "three Q buffers: the two-group kernel");
  // the row-contiguous swizzle XORs bits 6-7 (bf16) or 4-6 (e4m3) of the byte offset
  static_assert(QL == KC || (BM * ELT) % (ELT == 2 ? 256 : 128) == 0, "row-contiguous Q tile rows");
  static_assert(PL == KC || (BN * PELT) % (PELT == 2 ? 256 : 128) == 0, "row-contiguous P tile rows");
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
  // > 0: a row-contiguous P operand has only rows k < p_rows (K is padded up
  // to a whole k-tile and the A operand carries zeros there); the loads of
  // rows past it return zeros
  int64_t p_rows;
  // Optional side job for wave 0 of block 0 (red_in != nullptr): the
  // maximum of red_n fp32 values >= +0 or NaN, given as bit patterns, ->
  // *red_out, and, if red_scale_out is set, the scale of *red_amax_prev and
  // red_margin -> *red_scale_out.  Finishes a partial-amax reduction without
  // a launch of its own.
  const uint32_t* red_in;
  int64_t red_n;
  float* red_out;
  const float* red_amax_prev;
  float red_margin;
  float* red_scale_out;
};

__device__ __forceinline__ void side_amax(const GemmArgs& a, int wave, int lane) {
  if (a.red_in == nullptr || blockIdx.x != 0 || wave != 0) return;
  uint32_t m = 0;
  for (int64_t i = lane; i < a.red_n; i += 64) {
    const uint32_t v = a.red_in[i] & 0x7fffffffu;
    m = v > m ? v : m;
  }
  m = wave_max_u32(m);
  if (lane == 0) {
    *a.red_out = __uint_as_float(m);
    if (a.red_scale_out) *a.red_scale_out = scale_from_amax(*a.red_amax_prev, a.red_margin);
  }
}

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

// 8 e4m3 codes (byte i = k + i) -> the same 8 values as bf16, exactly: the
// converter gives fp32, whose upper half is the bf16 pattern (an e4m3 value
// has at most 4 significant bits).
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(i32x2 c) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(c[0], false), b = __builtin_amdgcn_cvt_pk_f32_fp8(c[0], true);
  const f32x2 e = __builtin_amdgcn_cvt_pk_f32_fp8(c[1], false), f = __builtin_amdgcn_cvt_pk_f32_fp8(c[1], true);
  const auto hi2 = [](float x, float y) {
    return (int)__builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
  };
  const i32x4 v = {hi2(a.x, a.y), hi2(b.x, b.y), hi2(e.x, e.y), hi2(f.x, f.y)};
  return __builtin_bit_cast(bf16x8_t, v);
}

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

// Scheduling groups for one k-slice of NM MFMAs.  After MFMA i comes its
// share of the other instructions of the slice:
//  * NR LDS reads (fragments of the next slice), over the first half of the
//    MFMAs when there are LDS writes, else over all of them, front-loaded;
//  * NW LDS writes (register staging) over the third quarter and then the NV
//    global loads that refill those registers over the last quarter (in the
//    program order the reads, the writes and the loads come in that order,
//    and the writes may alias the reads);
//  * without LDS writes, the NV global loads (direct to LDS, which may alias
//    the reads as far as the compiler knows) over the second half.
template <int N, int LEN, int I>
constexpr int share_front() { return (N * (I + 1) + LEN - 1) / LEN - (N * I + LEN - 1) / LEN; }
template <int NM, int NR, int NW, int NV, int I = 0>
__device__ __forceinline__ void sched_mix() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (NW > 0) {
      constexpr int H = NM / 2, Q3 = (3 * NM) / 4;
      if constexpr (I < H) {
        constexpr int r = share_front<NR, H, I>();
        if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      } else if constexpr (I < Q3) {
        constexpr int w = share_front<NW, Q3 - H, I - H>();
        if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);
      } else {
        constexpr int v = share_front<NV, NM - Q3, I - Q3>();
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
      }
    } else if constexpr (NV > 0) {
      constexpr int H = NM / 2;
      if constexpr (I < H) {
        constexpr int r = share_front<NR, H, I>();
        if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      } else {
        constexpr int v = share_front<NV, NM - H, I - H>();
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
      }
    } else {
      constexpr int r = share_front<NR, NM, I>();
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    }
    sched_mix<NM, NR, NW, NV, I + 1>();
  }
}

// LDS-linear 16-byte chunk c of an operand tile -> byte offset in global
// memory relative to the tile origin (at k = 0 of this block's range).
template <class C, int L, int ROWS, bool IS_P>
__device__ __forceinline__ uint32_t load_off(int c, int64_t ld_bytes) {
  constexpr int E = IS_P ? C::PELT : C::ELT;
  if constexpr (L == KC) {
    const int row = c / C::CPR, pc = c % C::CPR;
    const int lc = pc ^ (IS_P ? swz_rows_p<C::CPR>(row) : swz_rows_q<C::CPR>(row));
    return (uint32_t)(row * ld_bytes + lc * 16);
  } else {
    constexpr int MCPR = ROWS * E / 16;   // chunks per LDS row (one k)
    const int k = c / MCPR, pc = c % MCPR;
    const int lc = ((pc * 16) ^ swz_mn<E>(k)) / 16;
    return (uint32_t)(k * ld_bytes + lc * 16);
  }
}

// ------------------------------------------------------------------ shared kernel pieces
// Tile assignment.  Consecutive blocks go round-robin over the 8 XCDs;
// xcd_remap gives each XCD a contiguous run of logical tiles.  Logical order:
// split-k index slowest (blocks of one split share their k-range of both
// operands), then groups of group_m tile rows, inside a group the row fastest,
// so the tiles an XCD runs at once form a near-square window that shares few
// A- and B-slabs in that XCD's L2.
struct TilePos {
  int tm, tn, split, KT;
  int64_t m0, n0, kb, ke;
};
template <class C>
__device__ __forceinline__ TilePos tile_pos(const GemmArgs& a, int b, int nblocks) {
  TilePos t;
  const int GROUP_M = a.group_m;
  int i = xcd_remap(b, nblocks);
  const int per_split = a.tiles_m * a.tiles_n;
  t.split = i / per_split;
  i -= t.split * per_split;
  const int per_group = GROUP_M * a.tiles_n;
  const int grp = i / per_group, rem = i - grp * per_group;
  const int gm = min(GROUP_M, a.tiles_m - grp * GROUP_M);
  t.tm = grp * GROUP_M + rem % gm;
  t.tn = rem / gm;
  t.m0 = (int64_t)t.tm * C::BM;
  t.n0 = (int64_t)t.tn * C::BN;
  t.kb = (int64_t)t.split * a.k_per_split;
  t.ke = min(a.K, t.kb + a.k_per_split);
  t.KT = (int)((t.ke - t.kb + C::BK - 1) / C::BK);
  return t;
}
template <class C>
__device__ __forceinline__ TilePos tile_pos(const GemmArgs& a) {
  return tile_pos<C>(a, blockIdx.x, gridDim.x);
}

// Global -> LDS loads of the two operand tiles: buffer resources anchored at
// the tile origin (rows k >= ke of a row-contiguous operand fall past the
// resource's end and load as zero; for k-contiguous operands K is a multiple
// of BK) and this lane's byte offsets for each of its 16-byte chunks.
template <class C>
struct TileLoads {
  __amdgpu_buffer_rsrc_t rq, rp;
  uint32_t qoff[C::Q_LOADS], poff[C::P_LOADS];
  uint32_t qstep, pstep;   // bytes between consecutive k-tiles

  __device__ __forceinline__ void init(const GemmArgs& a, const TilePos& t, int wave, int lane) {
    const int64_t ldq_b = a.ldq * C::ELT, ldp_b = a.ldp * C::PELT;
    const char* q = (const char*)a.q;
    const char* p = (const char*)a.p;
    if constexpr (C::QL == KC) {
      rq = make_rsrc(q + t.m0 * ldq_b + t.kb * C::ELT, (uint64_t)((a.M - t.m0) * ldq_b - t.kb * C::ELT));
    } else {
      rq = make_rsrc(q + t.kb * ldq_b + t.m0 * C::ELT, (uint64_t)((t.ke - t.kb) * ldq_b - t.m0 * C::ELT));
    }
    if constexpr (C::PL == KC) {
      rp = make_rsrc(p + t.n0 * ldp_b + t.kb * C::PELT, (uint64_t)((a.N - t.n0) * ldp_b - t.kb * C::PELT));
    } else {
      const int64_t pke = a.p_rows > 0 && a.p_rows < t.ke ? a.p_rows : t.ke;
      const int64_t pbytes = (pke - t.kb) * ldp_b - t.n0 * C::PELT;
      rp = make_rsrc(p + t.kb * ldp_b + t.n0 * C::PELT, (uint64_t)(pbytes > 0 ? pbytes : 0));
    }
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++)
      qoff[j] = load_off<C, C::QL, C::BM, false>((j * C::NW + wave) * 64 + lane, ldq_b);
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++)
      poff[j] = load_off<C, C::PL, C::BN, true>((j * C::NW + wave) * 64 + lane, ldp_b);
    qstep = C::QL == KC ? (uint32_t)C::RB : (uint32_t)(C::BK * ldq_b);
    pstep = C::PL == KC ? (uint32_t)C::RB : (uint32_t)(C::BK * ldp_b);
  }
  // this wave's share of k-tile kt, straight into LDS stage `stage`
  __device__ __forceinline__ void issue(FP8MLP_LDS char* smem, int kt, int stage, int wave) const {
    FP8MLP_LDS char* sq = smem + stage * C::STAGE_BYTES;
    FP8MLP_LDS char* sp = sq + C::Q_BYTES;
    const uint32_t dq = (uint32_t)kt * qstep, dp = (uint32_t)kt * pstep;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++) buffer_load_lds16(rq, sq + (j * C::NW + wave) * 1024, qoff[j] + dq);
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++) buffer_load_lds16(rp, sp + (j * C::NW + wave) * 1024, poff[j] + dp);
  }
  // only the Q (or only the P) share of k-tile kt, to LDS address sq (sp)
  __device__ __forceinline__ void issue_q(FP8MLP_LDS char* sq, int kt, int wave) const {
    const uint32_t dq = (uint32_t)kt * qstep;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++) buffer_load_lds16(rq, sq + (j * C::NW + wave) * 1024, qoff[j] + dq);
  }
  __device__ __forceinline__ void issue_p(FP8MLP_LDS char* sp, int kt, int wave) const {
    const uint32_t dp = (uint32_t)kt * pstep;
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++) buffer_load_lds16(rp, sp + (j * C::NW + wave) * 1024, poff[j] + dp);
  }
};

// MFMA operand fragments read from one LDS stage.
//   Q: MFMA column q = lane & 31  -> tile row wm*WTM + fm*32 + (lane & 31)
//   P: MFMA row p' = lane & 31   -> tile row wn*WTN + fn*32 + perm_p(p') (or p')
template <class C>
struct FragReader {
  using Frag = typename FragT<C::ELT>::type;
  int lane, h;
  int qrow_off, prow_off;   // per-lane part; fragments add fm*32 / fn*32 rows
  int qx, px;               // swizzle terms

  __device__ __forceinline__ void init(int wm, int wn, int lane_) {
    lane = lane_;
    h = lane >> 5;
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
    } else if constexpr (C::ELT == 2 && C::PELT == 1) {
      // one transposed e4m3 read gives this lane k = 8h .. 8h+7 of one column,
      // the bf16 operand's k range; the columns follow the e4m3 order below
      const int kq = (lane & 15) >> 1;
      const int nb = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
      prow_off = (8 * h + kq) * C::BN;
      px = wn * C::WTN + nb;
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
  }
  // LDS reads per fragment
  static constexpr int QR = C::QL == KC ? (C::ELT == 2 ? 1 : 2) : (C::ELT == 2 ? 2 : 4);
  static constexpr int PR = C::PL == KC ? (C::ELT == 2 ? 1 : 2) : (C::ELT == 2 ? (C::PELT == 2 ? 2 : 1) : 4);

  __device__ __forceinline__ Frag q(const FP8MLP_LDS char* sq, int s, int fm) const {
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
  }
  __device__ __forceinline__ Frag p(const FP8MLP_LDS char* sp, int s, int fn) const {
    if constexpr (C::ELT == 2 && C::PELT == 1) {
      const int kq = (lane & 15) >> 1;
      const uint32_t col = (uint32_t)((px + fn * 32) ^ ((kq & 7) << 4));
      return e4m3x8_to_bf16x8(lds_read_tr8(sp, prow_off + (16 * s) * C::BN + col));
    } else if constexpr (C::ELT == 2) {
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
  }
};

template <class C>
__device__ __forceinline__ f32x16 mma(const typename FragT<C::ELT>::type& p, const typename FragT<C::ELT>::type& q,
                                      const f32x16& c) {
  if constexpr (C::ELT == 2) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(p, q, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(p, q, c, 0, 0, 0, 127, 0, 127);
  }
}

// ------------------------------------------------------------------ kernel: 4 waves
template <class C, class Epi, int KID>
__global__ void __launch_bounds__(256, C::OCC) gemm_kernel(GemmArgs a, Epi epi) {
  static_assert(C::NW == 4, "four-wave kernel");
  // the pipeline buffers, reused by the epilogue once the last tile is read
  constexpr int EPI_BYTES = Epi::template lds_bytes<C>();
  constexpr int SMEM = C::LDS_BYTES > EPI_BYTES ? C::LDS_BYTES : EPI_BYTES;
  static_assert(SMEM * C::OCC <= 160 * 1024, "LDS with the epilogue's staging");
  __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
  FP8MLP_LDS char* smem = (FP8MLP_LDS char*)smem_raw;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  side_amax(a, wave, lane);

  // With two blocks per CU, blocks that start together reach their
  // epilogues together and leave the matrix cores idle meanwhile.  Delaying
  // the blocks that the dispatcher places in the second residency slot of
  // each CU (the second 256 of the first 512) shifts the two slots by part of
  // a tile; later blocks inherit the offset when they take over a slot.
  if (C::OCC > 1 && a.stagger > 0 && blockIdx.x >= 256 && blockIdx.x < 512) {
    for (int i = 0; i < a.stagger; i++) __builtin_amdgcn_s_sleep(127);
  }

  const TilePos t = tile_pos<C>(a);
  const int KT = t.KT;
  TileLoads<C> ld;
  ld.init(a, t, wave, lane);

  // register staging: the next tile in flight in VGPRs
  i32x4 rq_regs[C::REG ? C::Q_LOADS : 1], rp_regs[C::REG ? C::P_LOADS : 1];
  auto gload = [&](int kt) {
    const uint32_t dq = (uint32_t)kt * ld.qstep, dp = (uint32_t)kt * ld.pstep;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++) rq_regs[j] = __builtin_amdgcn_raw_buffer_load_b128(ld.rq, ld.qoff[j] + dq, 0, 0);
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++) rp_regs[j] = __builtin_amdgcn_raw_buffer_load_b128(ld.rp, ld.poff[j] + dp, 0, 0);
  };
  auto dswrite = [&](int stage) {
    FP8MLP_LDS char* sq = smem + stage * C::STAGE_BYTES;
    FP8MLP_LDS char* sp = sq + C::Q_BYTES;
#pragma unroll
    for (int j = 0; j < C::Q_LOADS; j++) *(FP8MLP_LDS i32x4*)(sq + ((j * 4 + wave) * 64 + lane) * 16) = rq_regs[j];
#pragma unroll
    for (int j = 0; j < C::P_LOADS; j++) *(FP8MLP_LDS i32x4*)(sp + ((j * 4 + wave) * 64 + lane) * 16) = rp_regs[j];
  };

  FragReader<C> fr;
  fr.init(wm, wn, lane);
  using Frag = typename FragT<C::ELT>::type;
  constexpr int NREADS = C::FM * FragReader<C>::QR + C::FN * FragReader<C>::PR;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; i++)
#pragma unroll
    for (int j = 0; j < C::FN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // ---- main loop.  One barrier per tile, placed just before the tile's last
  // k-slice: by then every wave has read the slices it needs from this tile
  // and the next tile is in LDS, so the reads of the next tile's first slice
  // overlap the MFMAs of the last slice (fragments are double-buffered across
  // slices and across tiles).  Global loads -- and, with register staging,
  // the LDS writes -- are spread between the MFMAs of the earlier slices.
  //   direct:   tile kt+STAGES-1 is issued in slice 0 of iteration kt, into
  //             the buffer that held tile kt-1;
  //   registers: in slice SL-2 of iteration kt, tile kt+1 goes from VGPRs to
  //             LDS and tile kt+2 is loaded into the VGPRs.
  static_assert(C::SL % 2 == 0, "fragment double-buffering across tiles needs an even slice count");
  Frag qf[2][C::FM], pf[2][C::FN];
  auto read_slice = [&](int stage, int s, Frag(&q)[C::FM], Frag(&p)[C::FN]) {
    const FP8MLP_LDS char* sq = smem + stage * C::STAGE_BYTES;
    const FP8MLP_LDS char* sp = sq + C::Q_BYTES;
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) q[fm] = fr.q(sq, s, fm);
#pragma unroll
    for (int fn = 0; fn < C::FN; fn++) p[fn] = fr.p(sp, s, fn);
  };

  if constexpr (C::REG > 0) {
    if (KT > 0) {
      gload(0);
      dswrite(0);
      if (KT > 1) gload(1);
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; s++)
      if (s < KT) ld.issue(smem, s, s, wave);
    if (KT >= C::STAGES - 1) {
      wait_vmcnt<C::LOADS * (C::STAGES - 2)>();
    } else {
      wait_vmcnt<0>();
    }
  }
  __syncthreads();
  if (KT > 0) read_slice(0, 0, qf[0], pf[0]);

  constexpr int NM = C::FM * C::FN;
  constexpr int MEM_SLICE = C::REG ? C::SL - 2 : 0;
  // LOAD: direct -- issue tile kt+STAGES-1; registers -- refill the VGPRs
  // with tile kt+2.  NEXT: there is a tile kt+1 (registers: write it to LDS).
  auto body = [&]<bool LOAD, bool NEXT>(int kt) {
    const int stage = kt % C::STAGES, next_stage = (kt + 1) % C::STAGES;
#pragma unroll
    for (int s = 0; s < C::SL; s++) {
      if (s == C::SL - 1 && NEXT) {
        if constexpr (C::REG == 0) {
          if constexpr (LOAD) {
            wait_vmcnt<C::LOADS * (C::STAGES - 2)>();
          } else {
            wait_vmcnt<0>();
          }
        }
        // nothing crosses the barrier: the MFMAs of the last slice stay
        // after it, where they cover the next tile's first reads
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s + 1 < C::SL) {
        read_slice(stage, s + 1, qf[(s + 1) & 1], pf[(s + 1) & 1]);
      } else if (NEXT) {
        read_slice(next_stage, 0, qf[0], pf[0]);
      }
      if (s == MEM_SLICE) {
        if constexpr (C::REG == 0) {
          if constexpr (LOAD) ld.issue(smem, kt + C::STAGES - 1, (kt + C::STAGES - 1) % C::STAGES, wave);
        } else {
          // (the compiler waits for each staging register before its write)
          if constexpr (NEXT) dswrite((kt + 1) & 1);
          if constexpr (LOAD) gload(kt + 2);
        }
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) acc[fm][fn] = mma<C>(pf[s & 1][fn], qf[s & 1][fm], acc[fm][fn]);
      const bool reads = s + 1 < C::SL || NEXT;
      const bool mem = s == MEM_SLICE;
      if (reads && mem && (C::REG == 0 ? LOAD : NEXT)) {
        if constexpr (C::REG == 0) {
          sched_mix<NM, NREADS, 0, C::LOADS>();
        } else {
          sched_mix<NM, NREADS, C::LOADS, LOAD ? C::LOADS : 0>();
        }
      } else if (reads) {
        sched_mix<NM, NREADS, 0, 0>();
      } else {
        sched_mix<NM, 0, 0, 0>();
      }
      __builtin_amdgcn_sched_barrier(0);   // slices do not mix
    }
  };
  {
    int kt = 0;
    if constexpr (C::REG == 0) {
      for (; kt + C::STAGES - 1 < KT; kt++) body.template operator()<true, true>(kt);
      for (; kt + 1 < KT; kt++) body.template operator()<false, true>(kt);
    } else {
      for (; kt + 2 < KT; kt++) body.template operator()<true, true>(kt);
      if (kt + 1 < KT) body.template operator()<false, true>(kt++);
    }
    if (kt < KT) body.template operator()<false, false>(kt);
  }

  TileCtx ctx{t.m0, t.n0, t.tm, t.tn, t.split, wm, wn, lane, a.M, a.N};
  epi.template run<C>(ctx, acc, smem);
}

// ------------------------------------------------------------------ kernel: two groups of 4 waves
// 512 threads, one block per CU, 2 x 4 wave tiles.  Wave w belongs to group
// g = w / 4 and shares its SIMD with wave w ^ 4 of the other group.  Each
// wave's k-loop alternates two phases of equal length, separated by block
// barriers, and the groups run one phase apart:
//   M(j): read the fragments for the next HALF k-slices from LDS into
//         registers; for even j also issue this wave's share of the global
//         loads of the tile after the current one; for odd j wait for them;
//   C(j): the MFMAs of those HALF k-slices, nothing else.
// So in every phase one wave per SIMD only issues MFMAs while the other does
// the memory work, and a stalled load or LDS instruction never holds up the
// matrix core (a wave issues in order).  Tile s is read in the phases
// 4s-1 .. 4s+2 (group 0 runs C(j) in phase 2j, group 1 in phase 2j+1); tile
// s+1 goes into the other LDS buffer from phase 4s-1 on and is complete,
// for every wave, at the barrier that ends phase 4s+2.
// With three Q buffers (QB == 3) the loads of a k-tile leave in two bursts:
// M(2s) issues the P share of tile s+1 (into the P buffer of tile s-1), and
// M(2s+1), after waiting for everything issued so far (tile s+1 complete),
// issues the Q share of tile s+2 (into the Q buffer of tile s-1).  Before the
// loop only tile 0 is loaded; tile 1's Q share goes out in M(0).  Tile s-1
// was last read in phase 4s-2 and the earliest of these issues is in phase
// 4s-1 (group 0's M(2s)), so both buffers are free by then.
template <class C, class Epi>
constexpr int pp_smem_bytes() {
  constexpr int EPI_BYTES = Epi::template lds_bytes<C>();
  return C::LDS_BYTES > EPI_BYTES ? C::LDS_BYTES : EPI_BYTES;
}

// One tile (block b of nblocks in the tile order of a) of the two-group kernel.
template <class C, class Epi>
__device__ __forceinline__ void pp_tile(const GemmArgs& a, Epi& epi, FP8MLP_LDS char* smem, int b, int nblocks) {
  static_assert(C::NW == 8 && C::STAGES == 2 && C::REG == 0 && C::OCC == 1, "two-group kernel");
  static_assert(C::SL % 2 == 0, "k-slices split into two phases");
  static_assert(pp_smem_bytes<C, Epi>() <= 160 * 1024, "LDS with the epilogue's staging");
  constexpr bool Q3 = C::QB == 3;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = wave >> 2, wm = (wave >> 1) & 1, wn = 2 * (wave & 1) + g;
  side_amax(a, wave, lane);
  const TilePos t = tile_pos<C>(a, b, nblocks);
  const int KT = t.KT;
  TileLoads<C> ld;
  ld.init(a, t, wave, lane);
  FragReader<C> fr;
  fr.init(wm, wn, lane);
  using Frag = typename FragT<C::ELT>::type;
  constexpr int HALF = C::SL / 2;
  // LDS addresses of k-tile s's Q and P shares
  auto qbuf = [&](int s) -> FP8MLP_LDS char* {
    return Q3 ? smem + (s % 3) * C::Q_BYTES : smem + (s & 1) * C::STAGE_BYTES;
  };
  auto pbuf = [&](int s) -> FP8MLP_LDS char* {
    return Q3 ? smem + 3 * C::Q_BYTES + (s & 1) * C::P_BYTES : smem + (s & 1) * C::STAGE_BYTES + C::Q_BYTES;
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; i++)
#pragma unroll
    for (int j = 0; j < C::FN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
  Frag qf[HALF][C::FM], pf[HALF][C::FN];

  // tile 0 in LDS for everyone, then group 1 sits out one phase
  if constexpr (Q3) {
    // only tile 0 before the start (every block of a round issues these at
    // once); tile 1's Q share goes out with its P share in M(0)
    if (KT > 0) {
      ld.issue_q(qbuf(0), 0, wave);
      ld.issue_p(pbuf(0), 0, wave);
    }
    wait_vmcnt<0>();
  } else {
    if (KT > 0) ld.issue(smem, 0, 0, wave);
    wait_vmcnt<0>();
  }
  __syncthreads();
  if (g == 1) __syncthreads();

  for (int j = 0; j < 2 * KT; j++) {
    const int s = j >> 1, half = j & 1;
    // ---- M(j)
    {
      const FP8MLP_LDS char* sq = qbuf(s);
      const FP8MLP_LDS char* sp = pbuf(s);
#pragma unroll
      for (int k = 0; k < HALF; k++) {
#pragma unroll
        for (int fm = 0; fm < C::FM; fm++) qf[k][fm] = fr.q(sq, half * HALF + k, fm);
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) pf[k][fn] = fr.p(sp, half * HALF + k, fn);
      }
      if constexpr (Q3) {
        // B share of k-tile s + 1 in the first memory phase; the A share of
        // k-tile s + 2 in the second, once k-tile s + 1 is in (two bursts of
        // loads per k-tile instead of one keep the load queues from filling)
        if (half == 0) {
          if (s == 0 && KT > 1) ld.issue_q(qbuf(1), 1, wave);
          if (s + 1 < KT) ld.issue_p(pbuf(s + 1), s + 1, wave);
        } else {
          wait_vmcnt<0>();
          if (s + 2 < KT) ld.issue_q(qbuf(s + 2), s + 2, wave);
        }
      } else {
        if (half == 0) {
          if (s + 1 < KT) ld.issue(smem, s + 1, (s + 1) & 1, wave);
        } else {
          wait_vmcnt<0>();
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- C(j)
#pragma unroll
    for (int k = 0; k < HALF; k++)
#pragma unroll
      for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) acc[fm][fn] = mma<C>(pf[k][fn], qf[k][fm], acc[fm][fn]);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  // group 0 matches group 1's extra barrier
  if (g == 0) __syncthreads();

  TileCtx ctx{t.m0, t.n0, t.tm, t.tn, t.split, wm, wn, lane, a.M, a.N};
  epi.template run<C>(ctx, acc, smem);
}

template <class C, class Epi, int KID>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel(GemmArgs a, Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[pp_smem_bytes<C, Epi>()];
  pp_tile<C>(a, epi, (FP8MLP_LDS char*)smem_raw, blockIdx.x, gridDim.x);
}

// Two problems of one configuration and epilogue type in one launch: blocks
// [0, n0) run a0's tiles, blocks [off1, gridDim.x) run a1's; off1 is n0
// rounded up to a multiple of 8, so that block b of either problem runs on
// XCD b % 8 as the XCD-aware tile order assumes (blocks n0 .. off1 - 1 exit).
template <class C, class Epi, int KID>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel2(GemmArgs a0, Epi e0, GemmArgs a1, Epi e1, int n0,
                                                          int off1) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[pp_smem_bytes<C, Epi>()];
  const int b = blockIdx.x;
  if (b < off1) {
    if (b < n0) pp_tile<C>(a0, e0, (FP8MLP_LDS char*)smem_raw, b, n0);
  } else {
    pp_tile<C>(a1, e1, (FP8MLP_LDS char*)smem_raw, b - off1, (int)gridDim.x - off1);
  }
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
