// Host launcher for the templated GEMM kernel.
#pragma once

#include "epilogues.h"
#include "host.h"

namespace fp8mlp {

// Tile rows per group of the tile order: the ~32 x OCC tiles an XCD runs at
// once should form a near-square window of the tile grid (whole rows when the
// grid is narrow), so they share as few operand slabs as possible.
inline int tile_group_m(int tiles_m, int tiles_n, int occ) {
  const int window = 32 * occ;
  int side = 1;
  while ((side + 1) * (side + 1) <= window) side++;
  int g = tiles_n <= side ? window / (tiles_n > 0 ? tiles_n : 1) : side;
  if (g < 1) g = 1;
  if (g > tiles_m) g = tiles_m > 0 ? tiles_m : 1;
  return g;
}

inline const char* kid_name(int kid) {
  switch (kid) {
    case KID_UP: return "up_gemm_relu2_quant";
    case KID_DOWN8: return "down_gemm_e4m3";
    case KID_DOWN_BF16: return "down_gemm_bf16_eval";
    case KID_DPOST: return "dpost_gemm_dpre";
    case KID_DX: return "dx_gemm";
    case KID_DW1: return "dw1_gemm";
    case KID_DW2: return "dw2_gemm";
    case KID_LINEAR: return "fp8_linear_gemm";
    case KID_UP8: return "up_gemm_e4m3_relu2_quant";
    case KID_CE_STATS: return "ce_head_gemm_stats";
    case KID_CE_GRAD: return "ce_head_gemm_grad";
    case KID_CE_DX: return "ce_dx_gemm";
    case KID_CE_DW: return "ce_dw_gemm";
    case KID_CE8_STATS: return "ce_head_gemm_e4m3_stats";
    case KID_CE8_GRAD: return "ce_head_gemm_e4m3_grad";
    case KID_DW: return "dw_gemm";
  }
  return "gemm";
}

template <class C, int KID, class Epi>
inline int launch_gemm(const GemmArgs& args, const Epi& epi, hipStream_t st) {
  const int64_t blocks = (int64_t)args.tiles_m * args.tiles_n * args.splits;
  if (blocks == 0) return FP8MLP_OK;
  GemmArgs a = args;
  a.group_m = tile_group_m(a.tiles_m, a.tiles_n, C::OCC);
  TraceScope trace(kid_name(KID), st);
  if constexpr (C::NW == 8) {
    hipLaunchKernelGGL((gemm_pp_kernel<C, Epi, KID>), dim3((unsigned)blocks), dim3(C::NT), 0, st, a, epi);
  } else {
    hipLaunchKernelGGL((gemm_kernel<C, Epi, KID>), dim3((unsigned)blocks), dim3(C::NT), 0, st, a, epi);
  }
  return launch_status();
}

// Two problems of one two-group configuration in one launch (gemm_pp_kernel2).
// Neither may carry a side job: it would run in block 0 only.
template <class C, int KID, class Epi>
inline int launch_gemm2(const GemmArgs& args0, const Epi& epi0, const GemmArgs& args1, const Epi& epi1,
                        hipStream_t st) {
  static_assert(C::NW == 8, "the two-group kernel");
  FP8MLP_REQUIRE(args0.red_in == nullptr && args1.red_in == nullptr, FP8MLP_E_ARG);
  const int64_t n0 = (int64_t)args0.tiles_m * args0.tiles_n * args0.splits;
  const int64_t n1 = (int64_t)args1.tiles_m * args1.tiles_n * args1.splits;
  if (n0 == 0 && n1 == 0) return FP8MLP_OK;
  const int64_t off1 = (n0 + 7) / 8 * 8;
  GemmArgs a0 = args0, a1 = args1;
  a0.group_m = tile_group_m(a0.tiles_m, a0.tiles_n, C::OCC);
  a1.group_m = tile_group_m(a1.tiles_m, a1.tiles_n, C::OCC);
  TraceScope trace(kid_name(KID), st);
  hipLaunchKernelGGL((gemm_pp_kernel2<C, Epi, KID>), dim3((unsigned)(off1 + n1)), dim3(C::NT), 0, st, a0, epi0, a1,
                     epi1, (int)n0, (int)off1);
  return launch_status();
}

}  // namespace fp8mlp
