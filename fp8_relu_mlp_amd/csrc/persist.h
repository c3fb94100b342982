// Persistent form of the two-group GEMM kernel: one block per CU walks its
// tiles (b, b + grid, b + 2 grid, ...) with one unbroken stream of k-tile
// loads, and each tile's epilogue is private to each wave.  The dgrad GEMM
// uses it (short k loop, an epilogue that loads as many bytes as it stores);
// for the up-projection, dX and the e4m3 down-projection one block per tile
// measured faster, their epilogue stores then draining while the next block
// waits for its first k-tile instead of during the next tile's main loop.
//
// The k-tiles of consecutive tiles form one stream with a running index G
// (G0 = the index of the current tile's first k-tile).  Q k-tile G lives in
// Q buffer G % 3, P k-tile G in P buffer G % 2, and the protocol of
// pp_tile continues across tile ends: M(2s) issues the P share of k-tile
// s + 1 and M(2s + 1), after its wait, the Q share of k-tile s + 2, where
// k-tiles past the end of the tile are the next tile's first ones.  After the
// last k-tile of a tile the P share of the next tile's k-tile 1 is issued
// into the P buffer just freed, so the next tile starts with its first two
// k-tiles in flight and only the Q buffer of the tile's last k-tile is free:
// the epilogue runs in it, 4 KB per wave (one 32-row fragment row of the
// wave's 64-column region), with no block barrier, so waves finish their
// epilogues at their own pace and their stores drain while the next tile's
// first k-tile is read.
//
// Counting of vmcnt (which retires loads and stores in issue order): before
// reading k-tile 0 of a tile a wave waits until at most the loads of k-tile 1
// and the epilogue's memory operations (Epi::vm_ops) are outstanding; in M(1)
// only the epilogue's.
#pragma once

#include "launch.h"

namespace fp8mlp {

// A wave's LDS slot in the epilogue: 32 rows of WC bf16 columns (WC = 64:
// 4 KB, both fragment columns of the wave region at once; WC = 32: 2 KB, one
// fragment column at a time, for tiles whose Q buffer holds less than eight
// 4 KB slots).  Chunk c (16 bytes) of row r sits at r * 2 WC + (c ^ (r &
// (CH - 1))) * 16, so the fragment-order writes (32 rows, one chunk) and the
// row-order reads spread over the banks.
template <int WC>
struct WaveStage {
  static constexpr int RB = 2 * WC, CH = WC / 8, BYTES = 32 * RB;
  static constexpr int RPP = 64 / CH, PASSES = 32 / RPP;   // rows per row-order pass, passes
  __device__ static __forceinline__ uint32_t off(int r, int c) {
    return (uint32_t)(r * RB + ((c ^ (r & (CH - 1))) << 4));
  }
  // fragment column fnl (of this slot) held by this lane: with PERM 16
  // consecutive columns (two chunks), else four runs of four columns at
  // 8g + 4h (half a chunk each; the transposed e4m3 operand reads)
  template <bool PERM = true>
  __device__ static __forceinline__ void put(FP8MLP_LDS char* st, int lane, int fnl, const uint32_t (&w)[8]) {
    const int r = lane & 31, h = lane >> 5;
    if constexpr (PERM) {
      const int c = fnl * 4 + 2 * h;
      *(FP8MLP_LDS i32x4*)(st + off(r, c)) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *(FP8MLP_LDS i32x4*)(st + off(r, c + 1)) = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    } else {
#pragma unroll
      for (int g = 0; g < 4; g++)
        *(FP8MLP_LDS i32x2*)(st + off(r, fnl * 4 + g) + 8 * h) = i32x2{(int)w[2 * g], (int)w[2 * g + 1]};
    }
  }
  __device__ static __forceinline__ void get(const FP8MLP_LDS char* st, int lane, int fnl, uint32_t (&w)[8]) {
    const int r = lane & 31, c = fnl * 4 + 2 * (lane >> 5);
    const i32x4 a = lds_read_b128(st, off(r, c)), b = lds_read_b128(st, off(r, c + 1));
    w[0] = a[0], w[1] = a[1], w[2] = a[2], w[3] = a[3], w[4] = b[0], w[5] = b[1], w[6] = b[2], w[7] = b[3];
  }
  // row-order pass k: this lane's row and 16-byte chunk
  __device__ static __forceinline__ int prow(int k, int lane) { return RPP * k + lane / CH; }
  __device__ static __forceinline__ int pchunk(int lane) { return lane % CH; }
  __device__ static __forceinline__ uint4 pread(const FP8MLP_LDS char* st, int k, int lane) {
    const i32x4 v = lds_read_b128(st, off(prow(k, lane), pchunk(lane)));
    return uint4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
  }
  __device__ static __forceinline__ void pwrite(FP8MLP_LDS char* st, int k, int lane, uint4 v) {
    *(FP8MLP_LDS i32x4*)(st + off(prow(k, lane), pchunk(lane))) = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  }
};
// The slot width a configuration's epilogue uses (eight slots fit in its Q buffer).
template <class C>
constexpr int wave_slot_cols() { return C::Q_BYTES >= 8 * 4096 ? 64 : 32; }
template <class C>
constexpr int wave_slot_bytes() { return WaveStage<wave_slot_cols<C>()>::BYTES; }

// Byte offset, from the wave region's origin (row wm * WTM, column wn * WTN
// of the tile), of the 16 bytes (8 elements) this lane stores or loads in
// row-order pass k of fragment row fm, for the slot columns starting at
// column cb of the region; 0xffffffff (past any buffer's end: the hardware
// drops the store, a load returns 0) when the element lies outside the
// matrix.  ld_b: bytes per matrix row; eb: bytes per element.
template <class C, int WC>
__device__ __forceinline__ uint32_t wp_off(const TileCtx& c, int fm, int k, int cb, int64_t ld_b, int eb) {
  using S = WaveStage<WC>;
  const int r = fm * 32 + S::prow(k, c.lane), col = cb + S::pchunk(c.lane) * 8;
  const int64_t m = c.m0 + c.wm * C::WTM + r, n = c.n0 + c.wn * C::WTN + col;
  if (m >= c.M || n >= c.N) return 0xffffffffu;
  return (uint32_t)((int64_t)r * ld_b + (int64_t)col * eb);
}
// Resource for a wave region of a 2-byte or 1-byte matrix (origin at the
// region's first element); size 0 (everything dropped) for a missing output.
template <class C>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wp_rsrc(const TileCtx& c, const void* g, int64_t ld, int eb) {
  if (g == nullptr) return make_rsrc(nullptr, 0);
  const int64_t m = c.m0 + c.wm * C::WTM, n = c.n0 + c.wn * C::WTN;
  return make_rsrc((const char*)g + (m * ld + n) * eb, (uint64_t)C::WTM * ld * eb);
}

// Backward dgrad epilogue, wave-private (the computation of EpiDpre):
// dpre = bf16(sqrt(post) * acc), acc = 2 dpost.  The wave's post rows come
// straight into registers (row order, 16 bytes per lane, two fragment rows
// ahead), go through its LDS slot to the accumulator layout, and dpre goes
// back the same way.
struct EpiDpreWP {
  const uint16_t* post;
  uint16_t* dpre;
  int64_t ld;  // h

  template <class C>
  static constexpr int vm_ops() { return 8 * C::FM; }

  template <class C>
  __device__ __forceinline__ void run(const TileCtx& c, f32x16 (&acc)[C::FM][C::FN], FP8MLP_LDS char* st) {
    static_assert(C::PERM && C::WTN == 64 && C::FM == 4 && wave_slot_cols<C>() == 64,
                  "16 consecutive columns per lane, four fragment rows, 4 KB slots");
    using S = WaveStage<64>;
    const __amdgpu_buffer_rsrc_t rp = wp_rsrc<C>(c, post, ld, 2), rd = wp_rsrc<C>(c, dpre, ld, 2);
    uint4 pv[2][4];
    auto load = [&](int fm, uint4 (&dst)[4]) {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rp, wp_off<C, 64>(c, fm, k, 0, ld * 2, 2), 0, 2 /* nt */);
        dst[k] = uint4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
      }
    };
    load(0, pv[0]);
    load(1, pv[1]);
#pragma unroll
    for (int fm = 0; fm < C::FM; fm++) {
      // loads of fragment row fm done: later ones (row fm + 1) and the
      // stores of row fm - 1 may still be outstanding
      if (fm == 0) {
        wait_vmcnt<4>();
      } else if (fm < C::FM - 1) {
        wait_vmcnt<8>();
      } else {
        wait_vmcnt<4>();
      }
#pragma unroll
      for (int k = 0; k < 4; k++) S::pwrite(st, k, c.lane, pv[fm & 1][k]);
#pragma unroll
      for (int fn = 0; fn < C::FN; fn++) {
        uint32_t pw[8], o[8];
        S::get(st, c.lane, fn, pw);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          // v_sqrt_f32 (within 1 ulp of fp32) is far below the bf16 rounding of dpre
          const float r0 = __builtin_amdgcn_sqrtf(bf16_lo(pw[i])), r1 = __builtin_amdgcn_sqrtf(bf16_hi(pw[i]));
          o[i] = pack_bf16x2(r0 * acc[fm][fn][2 * i], r1 * acc[fm][fn][2 * i + 1]);
        }
        S::put(st, c.lane, fn, o);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) buffer_store_stream16(rd, wp_off<C, 64>(c, fm, k, 0, ld * 2, 2), S::pread(st, k, c.lane));
      if (fm + 2 < C::FM) load(fm + 2, pv[fm & 1]);
    }
  }
};

// The persistent loop (see the top of this file).  Requires at least two
// k-tiles per tile (K >= 2 BK; the launcher checks).
template <class C, class Epi>
__device__ __forceinline__ void pp_persistent(const GemmArgs& a, Epi& epi, FP8MLP_LDS char* smem, int ntiles) {
  static_assert(C::NW == 8 && C::STAGES == 2 && C::REG == 0 && C::OCC == 1 && C::QB == 3, "two-group kernel, Q3");
  static_assert(C::SL % 2 == 0, "k-slices split into two phases");
  static_assert(C::Q_BYTES >= 8 * wave_slot_bytes<C>(), "a Q buffer holds the eight wave slots");
  constexpr int VM = Epi::template vm_ops<C>();
  static_assert(C::LOADS + VM < 64, "vmcnt");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = wave >> 2, wm = (wave >> 1) & 1, wn = 2 * (wave & 1) + g;
  side_amax(a, wave, lane);
  int tile = blockIdx.x;
  if (tile >= ntiles) return;
  const int stride = gridDim.x;
  FragReader<C> fr;
  fr.init(wm, wn, lane);
  using Frag = typename FragT<C::ELT>::type;
  constexpr int HALF = C::SL / 2;
  auto qbuf = [&](int G) -> FP8MLP_LDS char* { return smem + (G % 3) * C::Q_BYTES; };
  auto pbuf = [&](int G) -> FP8MLP_LDS char* { return smem + 3 * C::Q_BYTES + (G & 1) * C::P_BYTES; };

  TilePos t = tile_pos<C>(a, tile, ntiles);
  TileLoads<C> cur;
  cur.init(a, t, wave, lane);
  // the first tile's k-tiles 0 and 1
  cur.issue_q(qbuf(0), 0, wave);
  cur.issue_p(pbuf(0), 0, wave);
  cur.issue_q(qbuf(1), 1, wave);
  cur.issue_p(pbuf(1), 1, wave);
  wait_vmcnt<C::LOADS>();
  lds_barrier();
  if (g == 1) lds_barrier();   // group 1 runs one interval behind
  int G0 = 0;
  bool first = true;           // no epilogue issued yet (nothing to count in M(1)'s wait)

  for (;;) {
    const int next = tile + stride;
    const bool has_next = next < ntiles;
    TilePos tn_pos = t;
    TileLoads<C> nxt = cur;
    if (has_next) {
      tn_pos = tile_pos<C>(a, next, ntiles);
      nxt.init(a, tn_pos, wave, lane);
    }
    const int KT = t.KT;

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
      for (int j = 0; j < C::FN; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
    Frag qf[HALF][C::FM], pf[HALF][C::FN];

    for (int j = 0; j < 2 * KT; j++) {
      const int s = j >> 1, half = j & 1;
      // ---- M(j)
      {
        const FP8MLP_LDS char* sq = qbuf(G0 + s);
        const FP8MLP_LDS char* sp = pbuf(G0 + s);
#pragma unroll
        for (int k = 0; k < HALF; k++) {
#pragma unroll
          for (int fm = 0; fm < C::FM; fm++) qf[k][fm] = fr.q(sq, half * HALF + k, fm);
#pragma unroll
          for (int fn = 0; fn < C::FN; fn++) pf[k][fn] = fr.p(sp, half * HALF + k, fn);
        }
        if (half == 0) {
          // the P share of k-tile s + 1 (k-tile 1 of a tile is already in flight)
          if (s >= 1) {
            if (s + 1 < KT) {
              cur.issue_p(pbuf(G0 + s + 1), s + 1, wave);
            } else if (has_next) {
              nxt.issue_p(pbuf(G0 + s + 1), s + 1 - KT, wave);
            }
          }
        } else {
          // k-tile s + 1 complete for this wave's loads
          if (s == 0 && !first) {
            wait_vmcnt<VM>();
          } else {
            wait_vmcnt<0>();
          }
          if (s + 2 < KT) {
            cur.issue_q(qbuf(G0 + s + 2), s + 2, wave);
          } else if (has_next && s + 2 - KT < 2) {
            nxt.issue_q(qbuf(G0 + s + 2), s + 2 - KT, wave);
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
    // group 0 matches group 1's extra barrier: both groups are done with the
    // tile's last k-tile
    if (g == 0) lds_barrier();
    // the P share of the next tile's k-tile 1, into the P buffer just freed
    if (has_next) nxt.issue_p(pbuf(G0 + KT + 1), 1, wave);

    // ---- epilogue in this wave's slot of the last k-tile's Q buffer
    {
      // the lane index through an opaque copy: the epilogue's per-lane
      // offsets depend on nothing else that changes from tile to tile, and
      // hoisted out of the tile loop they would stay live through it
      int elane = lane;
      asm volatile("" : "+v"(elane));
      TileCtx ctx{t.m0, t.n0, t.tm, t.tn, t.split, wm, wn, elane, a.M, a.N};
      epi.template run<C>(ctx, acc, qbuf(G0 + KT - 1) + wave * wave_slot_bytes<C>());
    }
    if (!has_next) break;
    // the next tile's k-tile 0 complete for this wave (k-tile 1 and the
    // epilogue's memory operations may be outstanding), then for everyone
    wait_vmcnt<C::LOADS + VM>();
    lds_barrier();
    if (g == 1) lds_barrier();
    G0 += KT;
    tile = next;
    t = tn_pos;
    cur = nxt;
    first = false;
  }
}

template <class C, class Epi, int KID>
__global__ void __launch_bounds__(512, 1) gemm_pp_persist_kernel(GemmArgs a, Epi epi, int ntiles) {
  static_assert(3 * C::Q_BYTES + 2 * C::P_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem_raw[3 * C::Q_BYTES + 2 * C::P_BYTES];
  pp_persistent<C>(a, epi, (FP8MLP_LDS char*)smem_raw, ntiles);
}

// Launch of the persistent kernel: one block per CU (fewer for small
// problems).  Block b runs on XCD b % 8 and its tiles are b + k * grid with
// grid a multiple of 8 whenever there are more tiles than CUs, so the
// XCD-aware tile order of tile_pos holds.  Falls back to one block per tile
// (gemm_pp_kernel with the tile-wide epilogue Fallback) when a tile has fewer
// than two k-tiles.
template <class C, int KID, class Epi, class Fallback>
inline int launch_gemm_persist(const GemmArgs& args, const Epi& epi, const Fallback& fb, hipStream_t st) {
  const int64_t tiles = (int64_t)args.tiles_m * args.tiles_n * args.splits;
  if (tiles == 0) return FP8MLP_OK;
  if (args.k_per_split < 2 * C::BK || args.K < 2 * C::BK) return launch_gemm<C, KID>(args, fb, st);
  GemmArgs a = args;
  a.group_m = tile_group_m(a.tiles_m, a.tiles_n, C::OCC);
  const int cus = num_cus();
    const int64_t grid = tiles < cus ? tiles : cus;
  TraceScope trace(kid_name(KID), st);
  hipLaunchKernelGGL((gemm_pp_persist_kernel<C, Epi, KID>), dim3((unsigned)grid), dim3(C::NT), 0, st, a, epi,
                     (int)tiles);
  return launch_status();
}

}  // namespace fp8mlp
