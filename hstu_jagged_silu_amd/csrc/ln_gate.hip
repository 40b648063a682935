// LayerNorm over the H*d values of each token, affine, then elementwise
// gating with U: y = (LN(o) * w + b) * u ("How Generative Recommenders Are
// Redefining RecSys at Scale", Takeaways: elementwise gating before the output
// projection). On the KV-cache path the attention output arrives as fp32
// partial sums over key splits; they are added here, in split order, first.
//
// One wave64 per token row. Every global access is a contiguous row segment
// (16 bytes of O per lane, 8 or 16 bytes of U and Y; the norm-ready form
// reads 16 bytes of deviations and of U per lane where the row width allows),
// and all loads of a row are issued before the first reduction so that they
// overlap. HBM-bound: per
// element it reads 4 bytes of O per split plus U and writes Y. A second form
// finishes the attention kernel's norm-ready store (bf16 deviations and
// per-head statistics) with 2 bytes of O per element.
#include "kernels.h"

namespace hstu {

constexpr int LN_ROWS = 4;   // rows (waves) per workgroup

__device__ inline float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <typename T>
__device__ inline f32x4 load4(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *(const bf16x4*)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *(const f32x4*)p;
  }
}

template <typename T>
__device__ inline void store4(T* p, f32x4 x) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v;
    for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
    *(bf16x4*)p = v;
  } else {
    *(f32x4*)p = x;
  }
}

// NCH: 4-element chunks per lane (H*d = 256 * NCH when FULL_LANES, else the
// row has fewer than 256 * NCH elements and trailing lanes idle).
template <typename T, int NCH, bool FULL_LANES>
__global__ __launch_bounds__(64 * LN_ROWS) void ln_gate_kernel(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * LN_ROWS + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const int nch = a.HD / 4;

  bool on[NCH];
  int col[NCH];
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    on[i] = FULL_LANES || c < nch;
    col[i] = 4 * (FULL_LANES ? c : min(c, nch - 1));
  }
  // the row's own loads first: they do not depend on the split count
  const float* orow = a.o + row * a.HD;
  const T* urow = (const T*)a.u + row * a.HD;
  f32x4 z[NCH], u[NCH];
  #pragma unroll
  for (int i = 0; i < NCH; ++i) z[i] = *(const f32x4*)(orow + col[i]);
  #pragma unroll
  for (int i = 0; i < NCH; ++i) u[i] = load4(urow + col[i]);

  // number of key splits that wrote this row (cached path)
  int nsplit = 1;
  if (a.chunk_keys > 0) {
    // the row's user b: how many of offsets[1..B] are <= row (offsets ascend
    // and offsets[B] = T > row)
    int b = 0, off_b, off_b1, clen;
    if (a.B <= 64) {
      // one wave-wide load of offsets[1..B] and cache_lens[0..B-1]
      const int o = lane < a.B ? a.offsets[lane + 1] : INT_MAX;
      const int c = lane < a.B ? a.cache_lens[lane] : 0;
      b = min(__popcll(__ballot(o <= row)), a.B - 1);
      off_b1 = __shfl(o, b);
      const int prev = __shfl(o, max(b - 1, 0));
      off_b = b > 0 ? prev : 0;  // offsets[0] = 0
      clen = __shfl(c, b);
    } else {
      for (int base = 0; base < a.B; base += 64) {
        const int i = base + 1 + lane;
        b += __popcll(__ballot(i <= a.B && a.offsets[i] <= row));
      }
      b = min(b, a.B - 1);
      off_b = a.offsets[b];
      off_b1 = a.offsets[b + 1];
      clen = a.cache_lens[b];
    }
    const int m = (int)(row - off_b);
    const int Lb = off_b1 - off_b;
    // keys seen by the work item that holds this row: causal new tokens end at
    // their tile's last row; paged candidates see the whole history
    const int kend = a.mode == MODE_MFALCON_PAGED ? clen : clen + min((m / QT + 1) * QT, Lb);
    nsplit = max(1, min((int)ceil_div(kend, a.chunk_keys), a.n_chunks));
  }

  // splits in groups whose loads are all in flight before the first add;
  // the adds keep split order
  constexpr int GS = NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1);
  int k = 1;
  for (; k + GS <= nsplit; k += GS) {
    f32x4 t[GS][NCH];
    #pragma unroll
    for (int j = 0; j < GS; ++j) {
      #pragma unroll
      for (int i = 0; i < NCH; ++i) t[j][i] = *(const f32x4*)(orow + (k + j) * a.o_chunk_stride + col[i]);
    }
    #pragma unroll
    for (int j = 0; j < GS; ++j) {
      #pragma unroll
      for (int i = 0; i < NCH; ++i) z[i] += t[j][i];
    }
  }
  for (; k < nsplit; ++k) {
    #pragma unroll
    for (int i = 0; i < NCH; ++i) z[i] += *(const f32x4*)(orow + k * a.o_chunk_stride + col[i]);
  }

  float s = 0.0f;
  #pragma unroll
  for (int i = 0; i < NCH; ++i)
    if (on[i]) s += (z[i][0] + z[i][1]) + (z[i][2] + z[i][3]);
  const float mean = wave_sum(s) / (float)a.HD;
  float ss = 0.0f;
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (on[i]) {
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dlt = z[i][e] - mean;
        ss = fmaf(dlt, dlt, ss);
      }
    }
  }
  const float rstd = rsqrtf(wave_sum(ss) / (float)a.HD + a.eps);
  T* yrow = (T*)a.y + row * a.HD;
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (!on[i]) continue;
    f32x4 w = {1, 1, 1, 1}, bb = {0, 0, 0, 0};
    if (a.ln_w) w = *(const f32x4*)(a.ln_w + col[i]);
    if (a.ln_b) bb = *(const f32x4*)(a.ln_b + col[i]);
    f32x4 yv;
    #pragma unroll
    for (int e = 0; e < 4; ++e) yv[e] = fmaf((z[i][e] - mean) * rstd, w[e], bb[e]) * u[i][e];
    store4(yrow + col[i], yv);
  }
}

// The same norm and gating from the attention kernel's norm-ready store: per
// row, H (mean_h, M2_h) pairs over head_dim values each and the bf16
// deviations o - mean_h. The pairs merge exactly (Chan et al.'s pairwise
// update with equal counts): mean = average of mean_h, and
// M2 = sum M2_h + head_dim * sum (mean_h - mean)^2. Then
// y = ((dev + mean_h - mean) / sqrt(M2 / HD + eps) * w + b) * u.
// Reads 2 bytes of deviation per element (and 8 bytes per head) instead of
// 4 bytes of O.
template <int CW>
__device__ inline void load_bf16(const bf16* p, float (&x)[CW]) {
  if constexpr (CW == 8) {
    const bf16x8 v = *(const bf16x8*)p;
    #pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else {
    const bf16x4 v = *(const bf16x4*)p;
    #pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
  }
}

// NCH chunks of CW values per lane (CW = 8: 16-byte accesses, for rows of a
// multiple of 512 values; CW = 4: 8-byte accesses, H*d = 256 * NCH when
// FULL_LANES, else the row has fewer than 256 * NCH values and trailing
// lanes idle). A chunk lies inside one head (head_dim is a multiple of CW).
template <int NCH, bool FULL_LANES, int CW>
__global__ __launch_bounds__(64 * LN_ROWS) void ln_gate_dev_kernel(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * LN_ROWS + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const int nch = a.HD / CW;
  const int H = a.HD / a.head_dim;

  bool on[NCH];
  int col[NCH];
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    on[i] = FULL_LANES || c < nch;
    col[i] = CW * (FULL_LANES ? c : min(c, nch - 1));
  }
  const bf16* drow = a.o_dev + row * a.HD;
  const bf16* urow = (const bf16*)a.u + row * a.HD;
  const float* srow = a.o_stats + 2 * row * H;
  float z[NCH][CW], u[NCH][CW];
  #pragma unroll
  for (int i = 0; i < NCH; ++i) load_bf16<CW>(drow + col[i], z[i]);
  #pragma unroll
  for (int i = 0; i < NCH; ++i) load_bf16<CW>(urow + col[i], u[i]);
  float mh[NCH];
  #pragma unroll
  for (int i = 0; i < NCH; ++i) mh[i] = srow[2 * (col[i] / a.head_dim)];

  // merge the heads' statistics (H <= 64: one head per lane)
  const f32x2 st = lane < H ? *(const f32x2*)(srow + 2 * lane) : f32x2{0.0f, 0.0f};
  const float mean = wave_sum(st[0]) / (float)H;
  const float dm = lane < H ? st[0] - mean : 0.0f;
  const float m2 = wave_sum(fmaf((float)a.head_dim * dm, dm, st[1]));
  const float rstd = rsqrtf(m2 / (float)a.HD + a.eps);
  bf16* yrow = (bf16*)a.y + row * a.HD;
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (!on[i]) continue;
    const float shift = mh[i] - mean;
    float yv[CW];
    #pragma unroll
    for (int e0 = 0; e0 < CW; e0 += 4) {
      f32x4 w = {1, 1, 1, 1}, bb = {0, 0, 0, 0};
      if (a.ln_w) w = *(const f32x4*)(a.ln_w + col[i] + e0);
      if (a.ln_b) bb = *(const f32x4*)(a.ln_b + col[i] + e0);
      #pragma unroll
      for (int e = 0; e < 4; ++e) yv[e0 + e] = fmaf((z[i][e0 + e] + shift) * rstd, w[e], bb[e]) * u[i][e0 + e];
    }
    if constexpr (CW == 8) {
      bf16x8 v;
      #pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)yv[e];
      *(bf16x8*)(yrow + col[i]) = v;
    } else {
      bf16x4 v;
      #pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)yv[e];
      *(bf16x4*)(yrow + col[i]) = v;
    }
  }
}

static void launch_dev(const LnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(a.T, LN_ROWS)), blk(64 * LN_ROWS);
  if (a.head_dim % 8 == 0) {  // 16-byte accesses
    switch (a.HD) {
      case 512: hipLaunchKernelGGL((ln_gate_dev_kernel<1, true, 8>), grid, blk, 0, s, a); return;
      case 1024: hipLaunchKernelGGL((ln_gate_dev_kernel<2, true, 8>), grid, blk, 0, s, a); return;
      case 2048: hipLaunchKernelGGL((ln_gate_dev_kernel<4, true, 8>), grid, blk, 0, s, a); return;
    }
  }
  if (a.HD == 256) { hipLaunchKernelGGL((ln_gate_dev_kernel<1, true, 4>), grid, blk, 0, s, a); return; }
  const int nch = (int)ceil_div(a.HD / 4, 64);
  if (nch <= 1) hipLaunchKernelGGL((ln_gate_dev_kernel<1, false, 4>), grid, blk, 0, s, a);
  else if (nch <= 2) hipLaunchKernelGGL((ln_gate_dev_kernel<2, false, 4>), grid, blk, 0, s, a);
  else if (nch <= 4) hipLaunchKernelGGL((ln_gate_dev_kernel<4, false, 4>), grid, blk, 0, s, a);
  else hipLaunchKernelGGL((ln_gate_dev_kernel<8, false, 4>), grid, blk, 0, s, a);
}

template <typename T>
static void launch_t(const LnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(a.T, LN_ROWS)), blk(64 * LN_ROWS);
  switch (a.HD) {
    case 256: hipLaunchKernelGGL((ln_gate_kernel<T, 1, true>), grid, blk, 0, s, a); return;
    case 512: hipLaunchKernelGGL((ln_gate_kernel<T, 2, true>), grid, blk, 0, s, a); return;
    case 1024: hipLaunchKernelGGL((ln_gate_kernel<T, 4, true>), grid, blk, 0, s, a); return;
    case 2048: hipLaunchKernelGGL((ln_gate_kernel<T, 8, true>), grid, blk, 0, s, a); return;
  }
  const int nch = (int)ceil_div(a.HD / 4, 64);
  if (nch <= 1) hipLaunchKernelGGL((ln_gate_kernel<T, 1, false>), grid, blk, 0, s, a);
  else if (nch <= 2) hipLaunchKernelGGL((ln_gate_kernel<T, 2, false>), grid, blk, 0, s, a);
  else if (nch <= 4) hipLaunchKernelGGL((ln_gate_kernel<T, 4, false>), grid, blk, 0, s, a);
  else hipLaunchKernelGGL((ln_gate_kernel<T, 8, false>), grid, blk, 0, s, a);
}

hipError_t launch_ln_gate(const LnArgs& a, int dtype, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.o_dev != nullptr) {
    if (dtype != 1 || a.head_dim < 4 || a.HD % a.head_dim != 0 || a.HD / a.head_dim > 64) return hipErrorInvalidValue;
    launch_dev(a, s);
  } else if (dtype == 1) launch_t<bf16>(a, s);
  else launch_t<float>(a, s);
  return hipGetLastError();
}

}  // namespace hstu
