// LayerNorm over the H*d values of each token, affine, then elementwise
// gating with U: y = (LN(o) * w + b) * u ("How Generative Recommenders Are
// Redefining RecSys at Scale", Takeaways: elementwise gating before the output
// projection). On the KV-cache path the attention output arrives as fp32
// partial sums over key splits; they are added here, in split order, first.
//
// One wave64 per token row; every load and store is a contiguous row segment
// (16 bytes per lane for fp32 O, 8 or 16 bytes for U and Y). HBM-bound: per
// element it reads 4 bytes of O per split plus U and writes Y.
#include "kernels.h"

namespace hstu {

constexpr int LN_ROWS = 4;   // rows (waves) per workgroup
constexpr int LN_MAXC = 8;   // max 4-element chunks per lane (H*d <= 2048)

__device__ inline float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <typename T>
__global__ __launch_bounds__(64 * LN_ROWS) void ln_gate_kernel(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * LN_ROWS + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const int nch = a.HD / 4;  // 4-element chunks in a row

  // number of key splits that wrote this row (cached path)
  int nsplit = 1;
  if (a.chunk_keys > 0) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int m = (int)(row - a.offsets[b]);
    const int Lb = a.offsets[b + 1] - a.offsets[b];
    const int qt = m / QT;
    const int kend = a.cache_lens[b] + min((qt + 1) * QT, Lb);
    nsplit = min((int)ceil_div(kend, a.chunk_keys), a.n_chunks);
  }

  f32x4 z[LN_MAXC];
  float s = 0.0f;
  #pragma unroll
  for (int i = 0; i < LN_MAXC; ++i) {
    const int c = lane + 64 * i;
    z[i] = f32x4{0, 0, 0, 0};
    if (c < nch) {
      for (int k = 0; k < nsplit; ++k) {
        const f32x4 x = *(const f32x4*)(a.o + k * a.o_chunk_stride + row * a.HD + 4 * c);
        z[i] += x;
      }
      s += z[i][0] + z[i][1] + z[i][2] + z[i][3];
    }
  }
  const float mean = wave_sum(s) / (float)a.HD;
  float ss = 0.0f;
  #pragma unroll
  for (int i = 0; i < LN_MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dlt = z[i][e] - mean;
        ss = fmaf(dlt, dlt, ss);
      }
    }
  }
  const float rstd = rsqrtf(wave_sum(ss) / (float)a.HD + a.eps);
  #pragma unroll
  for (int i = 0; i < LN_MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      f32x4 w = {1, 1, 1, 1}, bb = {0, 0, 0, 0};
      if (a.ln_w) w = *(const f32x4*)(a.ln_w + 4 * c);
      if (a.ln_b) bb = *(const f32x4*)(a.ln_b + 4 * c);
      float uu[4];
      if constexpr (sizeof(T) == 2) {
        const bf16x4 u4 = *(const bf16x4*)((const bf16*)a.u + row * a.HD + 4 * c);
        for (int e = 0; e < 4; ++e) uu[e] = (float)u4[e];
      } else {
        const f32x4 u4 = *(const f32x4*)((const float*)a.u + row * a.HD + 4 * c);
        for (int e = 0; e < 4; ++e) uu[e] = u4[e];
      }
      float yv[4];
      #pragma unroll
      for (int e = 0; e < 4; ++e) yv[e] = fmaf((z[i][e] - mean) * rstd, w[e], bb[e]) * uu[e];
      if constexpr (sizeof(T) == 2) {
        bf16x4 y4;
        for (int e = 0; e < 4; ++e) y4[e] = (bf16)yv[e];
        *(bf16x4*)((bf16*)a.y + row * a.HD + 4 * c) = y4;
      } else {
        *(f32x4*)((float*)a.y + row * a.HD + 4 * c) = f32x4{yv[0], yv[1], yv[2], yv[3]};
      }
    }
  }
}

hipError_t launch_ln_gate(const LnArgs& a, int dtype, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t grid = ceil_div(a.T, LN_ROWS);
  if (dtype == 1) hipLaunchKernelGGL(ln_gate_kernel<bf16>, dim3((unsigned)grid), dim3(64 * LN_ROWS), 0, s, a);
  else hipLaunchKernelGGL(ln_gate_kernel<float>, dim3((unsigned)grid), dim3(64 * LN_ROWS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
