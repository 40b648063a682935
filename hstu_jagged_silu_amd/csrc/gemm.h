// Launch interface of the layer's dense product (gemm.hip).
#pragma once

#include "common.h"

namespace hstu {

enum GemmEpilogue : int32_t { GEMM_EPI_NONE = 0, GEMM_EPI_SILU_SPLIT = 1 };

// C = A B, A [M, K] and B [K, N] row-major bf16. N % 256 == 0, K % 64 == 0.
// GEMM_EPI_NONE: C [M, N]. GEMM_EPI_SILU_SPLIT: SiLU, then column n goes to
// block n / split (each [M, split], split_stride elements apart), column
// n % split; split % 32 == 0.
struct GemmArgs {
  const bf16* a;
  const bf16* b;
  bf16* c;
  int64_t M;
  int32_t N, K;
  int64_t mt_count;  // ceil(M / 256)
  int32_t epilogue;
  int32_t split;
  int64_t split_stride;
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

}  // namespace hstu
