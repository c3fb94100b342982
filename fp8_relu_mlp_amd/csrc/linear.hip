// fp8_linear: FP8 forward projection ("NanoGPT Speedrun (Track 1)", "Changes
// vs Record #83" item 1: QKV and output projections in float8_e4m3 on the
// forward pass, weights stored transposed).
//
// K <= 768 (the model's width): one launch of the row-panel kernel below,
// which converts every row of X to e4m3 once, inside the GEMM, and keeps the
// codes in LDS for all the column tiles of the row.  Larger K: two launches,
// a bandwidth-bound pass that quantises X once into the workspace, then the
// e4m3 MFMA GEMM on the quantised copy.  Quantising inside a GEMM whose
// blocks each own one output tile would repeat the conversion in every one
// of the N / BN column blocks that share an activation tile.
#include "persist.h"

namespace fp8mlp {

// Xq [M,K] e4m3 . Wt_q [K,N] e4m3 (transposing LDS reads)
using CfgLin = GemmCfg<1, 192, 128, 128, 2, 2, KC, MNC>;

// Xq = e4m3(fp32(X * s)); 16 elements per thread and step.  With `partial`,
// block b also writes the maximum of |X| over the elements it converted to
// partial[b] (fp32 bit pattern), for the consumer to finish the reduction.
__global__ void __launch_bounds__(256) k_quantize(const uint16_t* __restrict__ X, int64_t n16,
                                                  const float* __restrict__ scale, uint8_t* __restrict__ Xq,
                                                  uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  const float s = *scale;
  uint32_t mx = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const i32x4 a = __builtin_nontemporal_load((const i32x4*)X + 2 * i);
    const i32x4 b = __builtin_nontemporal_load((const i32x4*)X + 2 * i + 1);
    uint32_t w[8] = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3],
                     (uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
    i32x4 q;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      mx = max_abs_bf16x2(mx, w[2 * j]);
      mx = max_abs_bf16x2(mx, w[2 * j + 1]);
      q[j] = (int)pack_e4m3x4(bf16_lo(w[2 * j]) * s, bf16_hi(w[2 * j]) * s, bf16_lo(w[2 * j + 1]) * s,
                              bf16_hi(w[2 * j + 1]) * s);
    }
    *((i32x4*)Xq + i) = q;
  }
  if (partial) {
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m01 = red[0] > red[1] ? red[0] : red[1], m23 = red[2] > red[3] ? red[2] : red[3];
      partial[blockIdx.x] = m01 > m23 ? m01 : m23;
    }
  }
}

// The same conversion into rows of Kp >= K codes: X [rows, K] -> Xq [rows, Kp],
// codes K .. Kp - 1 of each row zero (K, Kp multiples of 16).
__global__ void __launch_bounds__(256) k_quantize_rows(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                       int64_t Kp, const float* __restrict__ scale,
                                                       uint8_t* __restrict__ Xq, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  const float s = *scale;
  const int64_t cr = K / 16, cp = Kp / 16, n16 = rows * cp;
  uint32_t mx = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cp, c = i - r * cp;
    i32x4 q = {0, 0, 0, 0};
    if (c < cr) {
      const i32x4* src = (const i32x4*)(X + r * K) + 2 * c;
      const i32x4 a = __builtin_nontemporal_load(src);
      const i32x4 b = __builtin_nontemporal_load(src + 1);
      uint32_t w[8] = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3],
                       (uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        mx = max_abs_bf16x2(mx, w[2 * j]);
        mx = max_abs_bf16x2(mx, w[2 * j + 1]);
        q[j] = (int)pack_e4m3x4(bf16_lo(w[2 * j]) * s, bf16_hi(w[2 * j]) * s, bf16_lo(w[2 * j + 1]) * s,
                                bf16_hi(w[2 * j + 1]) * s);
      }
    }
    *((i32x4*)Xq + i) = q;
  }
  if (partial) {
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m01 = red[0] > red[1] ? red[0] : red[1], m23 = red[2] > red[3] ? red[2] : red[3];
      partial[blockIdx.x] = m01 > m23 ? m01 : m23;
    }
  }
}

// ------------------------------------------------------------------ row-panel kernel
// One block of four waves per CU walks a contiguous range of output tiles
// (128 rows x 256 columns), row panel by row panel.  On entering a panel the
// block converts the panel's 128 rows of X to e4m3 (RNE, saturating, the
// arithmetic of k_quantize) straight into LDS, in slabs of 128 codes laid out
// as the k-contiguous operand tiles of the GEMM core, and keeps them for
// every column tile of the panel.  Wave w computes all 128 rows of columns
// 64 w .. 64 w + 63 with v_mfma_scale_f32_32x32x64_f8f6f4 and streams its
// own 64 columns of Wt_q (64-k tiles of 4 KB, four buffers, three tiles
// ahead; Wt_q is a few MB and stays in L2): no wave reads another wave's
// share, so the k loop has no block barrier, only waits for the wave's own
// loads.  The block synchronises only to change panels.  A wave's epilogue
// goes through its own share of the buffer its last k-tile used.  A panel
// split between two blocks is converted by both.  The order of the k
// accumulation is that of the two-launch path: both give the same Y bit for
// bit.
namespace lp {
constexpr int BM = 128, BN = 256, NT = 256;
constexpr int KMAX = 768;                            // codes per row the panel holds
constexpr int SLAB = BM * 128;                       // 128 codes of k for the panel's rows
constexpr int PANEL = (KMAX / 128) * SLAB;           // 96 KB
constexpr int WS = 64 * 64;                          // one wave's share of a 64-k tile: 4 KB
constexpr int WT = 4 * WS;                           // a 64-k tile of Wt_q columns: 16 KB
constexpr int NWB = 4;                               // Wt_q tile buffers
constexpr int LDS = PANEL + NWB * WT;                // 160 KB
}  // namespace lp

struct PanelArgs {
  const uint16_t* X;
  const uint8_t* W;
  uint16_t* Y;
  const float* x_scale;
  const float* w_inv;
  uint32_t* partial;      // nullptr, or per-block max |X| (fp32 bit patterns)
  int64_t M, K, N;
  uint32_t KN;            // K * N (< 2^32)
  int Kp, T;              // K rounded up to 128; 64-k tiles per output tile (even)
  int tiles_n;
  int items;              // output tiles
};

// LDS reads through a restrict base: with the alias information the compiler
// does not wait for the Wt_q loads in flight (buffer_load ... lds) before
// them; the loop orders its reads after the loads they need.
__device__ __forceinline__ i32x4 lds_read_b128_r(const FP8MLP_LDS char* __restrict__ base, uint32_t off) {
  return *(const FP8MLP_LDS i32x4*)(base + off);
}

// A wave's share of a Wt_q k-tile: 64 rows k of its 64 columns, 64 bytes
// each, the 16-byte chunks of rows with k & 4 swapped in pairs (chunk c at
// c ^ 2), so that the eight rows a transposing read touches fall on distinct
// banks.
__device__ __forceinline__ uint32_t wshare_off(int k, int chunk) {
  return (uint32_t)(k * 64 + ((chunk ^ (((k >> 2) & 1) << 1)) << 4));
}

__global__ void __launch_bounds__(lp::NT, 1) k_lin_panel(PanelArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[lp::LDS];
  FP8MLP_LDS char* const smem = (FP8MLP_LDS char*)smem_raw;
  FP8MLP_LDS char* const panel = smem;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // this wave's share of Wt_q buffer b
  FP8MLP_LDS char* const wshare = smem + lp::PANEL + wave * lp::WS;
  auto wsh = [&](int b) __attribute__((always_inline)) { return wshare + b * lp::WT; };

  // Scalars: the compiler keeps a value it cannot prove wave-uniform in
  // vector registers, and a buffer resource built from one turns every
  // access into a loop over lanes.
  const int i0 = __builtin_amdgcn_readfirstlane((int)((int64_t)blockIdx.x * a.items / gridDim.x));
  const int i1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(blockIdx.x + 1) * a.items / gridDim.x));
  const int T = a.T, NI = i1 - i0, tiles_n = a.tiles_n;
  const float s = *a.x_scale;
  const float inv_s = 1.0f / s, inv_w = *a.w_inv;
  float xmaxf = 0.0f;   // max |X| over the rows this block converted

  // ---- this wave's Wt_q stream over the block's output tiles: the next
  // k-tile to load is k-tile wt of the output tile in column wtn of the
  // block's wi-th tile; it goes into buffer wb.  Load j of a k-tile fills
  // rows 16 j .. 16 j + 15 of the share (1 KB); lane l brings row 16 j + l/4,
  // stored chunk l % 4.
  uint32_t woff[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int k = 16 * j + lane / 4, p = lane & 3;
    woff[j] = (uint32_t)k * (uint32_t)a.N + (uint32_t)((p ^ (((k >> 2) & 1) << 1)) << 4);
  }
  int wi = 0, wt = 0, wb = 0;
  int wtn = __builtin_amdgcn_readfirstlane(i0 % tiles_n);
  // Past the end of the stream the resource is empty: the loads still go out
  // (every step issues the same number) and fill a share nobody reads with
  // zeros.
  struct WLoad {
    __amdgpu_buffer_rsrc_t r;
    FP8MLP_LDS char* dst;
    uint32_t dk;
  };
  auto next_w = [&]() __attribute__((always_inline)) {
    WLoad l;
    const uint32_t n0 = (uint32_t)wtn * lp::BN + (uint32_t)wave * 64;
    // rows k >= K lie past the resource's end and load as zero (K * N <
    // 2^32; 32-bit scalar arithmetic keeps the k loop free of branches)
    l.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.W) + n0, (short)0,
                                            wi < NI ? (int)(a.KN - n0) : 0, 0x00020000);
    l.dst = wsh(wb);
    l.dk = (uint32_t)wt * 64u * (uint32_t)a.N;
    wb = (wb + 1) & (lp::NWB - 1);
    if (++wt == T) {
      wt = 0;
      wi++;
      wtn = wtn + 1 == tiles_n ? 0 : wtn + 1;
    }
    return l;
  };
  auto issue_w = [&](const WLoad& l) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; j++) buffer_load_lds16(l.r, l.dst + j * 1024, woff[j] + l.dk);
  };

  // ---- the row panel: X rows m0 .. m0 + 127 -> e4m3 codes in LDS, slab by
  // slab (128 codes of k).  In a slab thread t converts the 8-value chunk
  // t % 16 of rows t / 16 + 16 u (u = 0 .. 7): its LDS addresses differ by
  // constants (the row swizzle repeats every 16 rows) and its global ones by
  // a scalar.
  const int pc = (int)threadIdx.x & 15, pr = (int)threadIdx.x >> 4;
  const uint32_t pl_off = (uint32_t)pr * 128u + (uint32_t)((((pc >> 1) ^ swz_rows_q<8>(pr)) << 4) + ((pc & 1) << 3));
  auto load_panel = [&](int tm) __attribute__((always_inline)) {
    const int64_t m0 = (int64_t)tm * lp::BM;
    const int64_t rows = a.M - m0 < lp::BM ? a.M - m0 : lp::BM;
    // rows past M read as zero
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X + m0 * a.K, (uint64_t)(rows * a.K * 2));
    const uint32_t row_b = (uint32_t)a.K * 2u, t_off = (uint32_t)pr * row_b + (uint32_t)pc * 16u;
    const int nslab = a.Kp / 128;
    auto issue = [&](int j, i32x4(&v)[8]) __attribute__((always_inline)) {
      // codes K .. Kp - 1 of a row are zero
      const bool in_k = j * 128 + pc * 8 < a.K;
#pragma unroll
      for (int u = 0; u < 8; u++)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, in_k ? t_off + (uint32_t)u * 16u * row_b + (uint32_t)j * 256u : 0xffffffffu,
                                                     0, 2 /* nt */);
    };
    auto convert = [&](int j, const i32x4(&v)[8]) __attribute__((always_inline)) {
      FP8MLP_LDS char* dst = panel + j * lp::SLAB + pl_off;
#pragma unroll
      for (int u = 0; u < 8; u++) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          x[2 * e] = bf16_lo((uint32_t)v[u][e]);
          x[2 * e + 1] = bf16_hi((uint32_t)v[u][e]);
        }
        // max |X| (NaN-propagating, so a NaN reaches it) and the codes: the
        // product clamped to [-448, 448] (NaN kept) and converted RNE, as
        // pack_e4m3x4 does
#pragma unroll
        for (int e = 0; e < 8; e++) xmaxf = __builtin_elementwise_maximum(xmaxf, __builtin_fabsf(x[e]));
        auto cl = [&](float y) {
          return __builtin_elementwise_minimum(__builtin_elementwise_maximum(y * s, -kE4M3Max), kE4M3Max);
        };
        int c0 = __builtin_amdgcn_cvt_pk_fp8_f32(cl(x[0]), cl(x[1]), 0, false);
        c0 = __builtin_amdgcn_cvt_pk_fp8_f32(cl(x[2]), cl(x[3]), c0, true);
        int c1 = __builtin_amdgcn_cvt_pk_fp8_f32(cl(x[4]), cl(x[5]), 0, false);
        c1 = __builtin_amdgcn_cvt_pk_fp8_f32(cl(x[6]), cl(x[7]), c1, true);
        *(FP8MLP_LDS i32x2*)(dst + u * 16 * 128) = i32x2{c0, c1};
      }
    };
    // the next slab's loads in flight while one is converted
    i32x4 va[8], vb[8];
    issue(0, va);
    for (int j = 0; j < nslab; j += 2) {
      if (j + 1 < nslab) issue(j + 1, vb);
      convert(j, va);
      if (j + 1 < nslab) {
        if (j + 2 < nslab) issue(j + 2, va);
        convert(j + 1, vb);
      }
    }
    wait_vmcnt<0>();
  };

  // ---- fragments of one k-tile: the panel's slab and half, a Wt_q share
  // (the operand layouts of FragReader for k-contiguous Q and transposing
  // e4m3 P reads)
  const int h = lane >> 5, q31 = lane & 31;
  const int qx = swz_rows_q<8>(q31);
  const int kq = (lane & 15) >> 1, nb = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  uint32_t poff[2];
#pragma unroll
  for (int fn = 0; fn < 2; fn++)
    poff[fn] = wshare_off(32 * h + kq, 2 * fn + (nb >> 4)) + (uint32_t)(nb & 8);
  auto read_frags = [&](int t, int buf, i32x8(&q)[4], i32x8(&p)[2]) __attribute__((always_inline)) {
    const FP8MLP_LDS char* sq = panel + (t >> 1) * lp::SLAB;
    const FP8MLP_LDS char* sp = wsh(buf);
    const uint32_t c = 4 * (t & 1) + 2 * h;
#pragma unroll
    for (int fm = 0; fm < 4; fm++) {
      const uint32_t base = (uint32_t)(fm * 32 + q31) * 128u;
      const i32x4 v0 = lds_read_b128_r(sq, base + ((c ^ qx) << 4));
      const i32x4 v1 = lds_read_b128_r(sq, base + (((c + 1) ^ qx) << 4));
      q[fm] = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
#pragma unroll
    for (int fn = 0; fn < 2; fn++) {
      // rows k, k + 8, k + 16, k + 24 (k & 4 is the same for the four)
      const i32x2 r0 = lds_read_tr8(sp, poff[fn]);
      const i32x2 r1 = lds_read_tr8(sp, poff[fn] + 8 * 64);
      const i32x2 r2 = lds_read_tr8(sp, poff[fn] + 16 * 64);
      const i32x2 r3 = lds_read_tr8(sp, poff[fn] + 24 * 64);
      p[fn] = i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    }
  };

  f32x16 acc[4][2];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
  };
  zero_acc();

  // ---- epilogue of the output tile (tm, tn): Y = bf16((acc * fp32(1 / x_scale)) * w_inv),
  // staged 32 rows at a time through the wave's 4 KB share of buffer buf
  using S = WaveStage<64>;
  auto epilogue = [&](int tm, int tn, int buf) __attribute__((always_inline)) {
    FP8MLP_LDS char* st = wsh(buf);
    const int64_t m0 = (int64_t)tm * lp::BM, nw = (int64_t)tn * lp::BN + wave * 64;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.Y + m0 * a.N + nw, (uint64_t)lp::BM * a.N * 2);
#pragma unroll
    for (int fm = 0; fm < 4; fm++) {
#pragma unroll
      for (int fn = 0; fn < 2; fn++) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
          w[i] = pack_bf16x2((acc[fm][fn][2 * i] * inv_s) * inv_w, (acc[fm][fn][2 * i + 1] * inv_s) * inv_w);
        S::put<false>(st, lane, fn, w);
      }
#pragma unroll
      for (int k = 0; k < S::PASSES; k++) {
        const int r = fm * 32 + S::prow(k, lane), col = S::pchunk(lane) * 8;
        // every store is issued (the vmcnt accounting counts them); those
        // outside the matrix go to an offset past the resource
        const uint32_t off = m0 + r < a.M && nw + col < a.N ? (uint32_t)(r * a.N + col) * 2u : 0xffffffffu;
        buffer_store_stream16(ry, off, S::pread(st, k, lane));
      }
    }
  };
  static_assert(4 * S::PASSES == 16 && S::BYTES == lp::WS, "sixteen stores per wave and output tile, one share");

  int tm = __builtin_amdgcn_readfirstlane(i0 / tiles_n), tn = __builtin_amdgcn_readfirstlane(i0 % tiles_n);
  load_panel(tm);
#pragma unroll
  for (int i = 0; i < 4; i++) issue_w(next_w());
  wait_vmcnt<12>();
  __syncthreads();   // the panel
  i32x8 qf[2][4], pf[2][2];
  read_frags(0, 0, qf[0], pf[0]);
  int cb = 0;   // buffer of the current k-tile

  // This wave's memory operations, in issue order: the 4 loads of every
  // k-tile and, after the last k-tile of each output tile, its epilogue's 16
  // stores followed by the loads that step left out.  k-tile g's loads go
  // out in step g - 4 (into the buffer whose fragments step g - 4 used);
  // waiting in step g for k-tile g + 1 leaves the loads of k-tiles g + 2 and
  // g + 3 outstanding, and 16 stores as well in the first two steps of an
  // output tile (FIRST).  LAST: the last step of an output tile, whose loads
  // wait until its epilogue is through the buffer.
  auto step = [&]<int B, bool FIRST, bool LAST>(int t) __attribute__((always_inline)) {
    wait_vmcnt<FIRST ? 24 : 8>();
    const WLoad wl = next_w();
    const int nb1 = (cb + 1) & (lp::NWB - 1);
    // (past the end, or from a panel about to be replaced: read and discarded)
    read_frags(LAST ? 0 : t + 1, nb1, qf[B ^ 1], pf[B ^ 1]);
#pragma unroll
    for (int fm = 0; fm < 4; fm++)
#pragma unroll
      for (int fn = 0; fn < 2; fn++) acc[fm][fn] = mma<CfgLin>(pf[B][fn], qf[B][fm], acc[fm][fn]);
    if constexpr (!LAST) {
      // after the MFMAs, which have consumed this buffer's fragments
      issue_w(wl);
      sched_mix<8, 16, 0, 4>();
    } else {
      sched_mix<8, 16, 0, 0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LAST) {
      epilogue(tm, tn, cb);
      zero_acc();
      issue_w(wl);
    }
    cb = nb1;
  };
  // Sixteen stores the hardware drops stand in for an epilogue before the
  // first output tile, so that every tile's first steps count alike.
  {
    const __amdgpu_buffer_rsrc_t none = make_rsrc(nullptr, 0);
#pragma unroll
    for (int k = 0; k < 16; k++) buffer_store_stream16(none, 0xffffffffu, uint4{0, 0, 0, 0});
  }
  for (int il = 0; il < NI; il++) {
    if (T == 2) {
      step.template operator()<0, true, false>(0);
      step.template operator()<1, true, true>(1);
    } else {
      step.template operator()<0, true, false>(0);
      step.template operator()<1, true, false>(1);
      for (int t = 2; t + 2 < T; t += 2) {
        step.template operator()<0, false, false>(t);
        step.template operator()<1, false, false>(t + 1);
      }
      step.template operator()<0, false, false>(T - 2);
      step.template operator()<1, false, true>(T - 1);
    }
    if (++tn == tiles_n) {
      tn = 0;
      tm++;
      if (il + 1 < NI) {
        // a new panel, once every wave's reads of the old one are complete
        // (including the discarded ones of its last step)
        lds_barrier();
        load_panel(tm);
        lds_barrier();
        read_frags(0, cb, qf[0], pf[0]);
      }
    }
  }
  wait_vmcnt<0>();

  if (a.partial) {
    // (the buffers are idle now)
    const uint32_t m = wave_max_u32(__float_as_uint(xmaxf));
    __syncthreads();
    if (lane == 0) ((FP8MLP_LDS uint32_t*)(smem + lp::PANEL))[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      const FP8MLP_LDS uint32_t* v = (const FP8MLP_LDS uint32_t*)(smem + lp::PANEL);
      const uint32_t m01 = v[0] > v[1] ? v[0] : v[1], m23 = v[2] > v[3] ? v[2] : v[3];
      a.partial[blockIdx.x] = m01 > m23 ? m01 : m23;
    }
  }
}

int launch_quantize(const uint16_t* X, int64_t n, const float* scale, uint8_t* Xq, uint32_t* partial,
                    int64_t* count, hipStream_t st) {
  *count = 0;
  if (n == 0) return FP8MLP_OK;
  const int64_t n16 = n / 16;
  int64_t blocks = cdiv(n16, 256 * 4);
  if (blocks > kQuantBlocks) blocks = kQuantBlocks;
  TraceScope trace("quantize_e4m3", st);
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, st, X, n16, scale, Xq, partial);
  *count = blocks;
  return launch_status();
}

}  // namespace fp8mlp

using namespace fp8mlp;

extern "C" {

// K rounded up to whole e4m3 k-tiles (128 codes): the row length of Xq.
static int64_t lin_kp(int64_t K) { return cdiv(K, 128) * 128; }

size_t fp8_linear_workspace(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return align_up((size_t)(M * lin_kp(K)), 256) + quantize_partial_bytes();
}

int fp8_linear(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv_scale,
               uint16_t* Y, float* x_amax_out, int64_t M, int64_t K, int64_t N, void* workspace,
               size_t workspace_bytes, void* stream) {
  FP8MLP_REQUIRE(M >= 0 && K > 0 && N > 0 && K % 64 == 0 && N % 64 == 0 && weight_dims_ok(K, N), FP8MLP_E_SHAPE);
  FP8MLP_REQUIRE(x_scale && w_inv_scale && Wt_q, FP8MLP_E_NULL);
  // block 0 of the GEMM writes x_amax_out while its other blocks read the scales
  FP8MLP_REQUIRE(x_amax_out != x_scale && x_amax_out != w_inv_scale, FP8MLP_E_ARG);
  if (M > 0) FP8MLP_REQUIRE(X && Y, FP8MLP_E_NULL);
  for (const void* p : {(const void*)X, (const void*)Wt_q, (const void*)Y})
    FP8MLP_REQUIRE(p == nullptr || aligned16(p), FP8MLP_E_ALIGN);
  for (const void* p : {(const void*)x_scale, (const void*)w_inv_scale, (const void*)x_amax_out})
    FP8MLP_REQUIRE(((uintptr_t)p & 3) == 0, FP8MLP_E_ALIGN);
  const size_t need = fp8_linear_workspace(M, K);
  FP8MLP_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), FP8MLP_E_WORKSPACE);
  FP8MLP_REQUIRE(need == 0 || aligned16(workspace), FP8MLP_E_ALIGN);
  FP8MLP_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (M == 0) {
    // nothing to convert: max |X| over no elements is 0
    return x_amax_out ? launch_max_small(nullptr, 0, x_amax_out, nullptr, 0.0f, nullptr, st) : FP8MLP_OK;
  }
  // K not a multiple of the 128-code k-tile: Xq rows padded with zero codes
  // to Kp, and the loads of Wt_q rows past K return zeros
  const int64_t Kp = lin_kp(K);
  uint8_t* Xq = (uint8_t*)workspace;
  uint32_t* xpart = (uint32_t*)((uint8_t*)workspace + align_up((size_t)(M * Kp), 256));
  if (Kp <= lp::KMAX && cdiv(M, lp::BM) * cdiv(N, lp::BN) < (int64_t)1 << 31) {
    const int64_t tiles_m = cdiv(M, lp::BM), tiles_n = cdiv(N, lp::BN), items = tiles_m * tiles_n;
    const int64_t grid = items < num_cus() ? items : num_cus();
    PanelArgs pa{X, Wt_q, Y, x_scale, w_inv_scale, x_amax_out ? xpart : nullptr, M, K, N, (uint32_t)(K * N),
                 (int)Kp, (int)(Kp / 64), (int)tiles_n, (int)items};
    {
      TraceScope trace("fp8_linear_panel", st);
      hipLaunchKernelGGL(k_lin_panel, dim3((unsigned)grid), dim3(lp::NT), 0, st, pa);
      FP8MLP_TRY(launch_status());
    }
    // max |X| from the blocks' maxima
    return x_amax_out ? launch_max_small((const float*)xpart, grid, x_amax_out, nullptr, 0.0f, nullptr, st)
                      : FP8MLP_OK;
  }
  int64_t nx = 0;
  if (Kp == K) {
    FP8MLP_TRY(launch_quantize(X, M * K, x_scale, Xq, x_amax_out ? xpart : nullptr, &nx, st));
  } else {
    int64_t blocks = cdiv(M * Kp / 16, 256 * 4);
    if (blocks > kQuantBlocks) blocks = kQuantBlocks;
    TraceScope trace("quantize_e4m3", st);
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, st, X, M, K, Kp, x_scale, Xq,
                       x_amax_out ? xpart : nullptr);
    FP8MLP_TRY(launch_status());
    nx = blocks;
  }
  GemmArgs a{Xq, Kp, Wt_q, N, M, N, Kp, (int)cdiv(M, CfgLin::BM), (int)cdiv(N, CfgLin::BN), 1, Kp, 0};
  a.p_rows = K;
  if (x_amax_out) {
    // block 0 of the GEMM finishes max |X| from the conversion's partial maxima
    a.red_in = xpart;
    a.red_n = nx;
    a.red_out = x_amax_out;
  }
  EpiBf16Out epi{Y, N, 2, nullptr, 0.0f, x_scale, w_inv_scale};
  return launch_gemm<CfgLin, KID_LINEAR>(a, epi, st);
}

}  // extern "C"
