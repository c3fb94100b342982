// Host launcher for the templated GEMM kernel.
#pragma once

#include "epilogues.h"
#include "host.h"

namespace fp8mlp {

template <class C, class Epi>
inline int launch_gemm(const char* name, const GemmArgs& a, const Epi& epi, hipStream_t st) {
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n * a.splits;
  if (blocks == 0) return FP8MLP_OK;
  TraceScope trace(name, st);
  hipLaunchKernelGGL((gemm_kernel<C, Epi>), dim3((unsigned)blocks), dim3(256), 0, st, a, epi);
  return launch_status();
}

}  // namespace fp8mlp
