// Backward of the LayerNorm + U gating epilogue, y = (n * w + b) * u with
// n = (o - mean) * rstd over the H*d values of a token (population variance).
// The chain rule of that definition gives, per row,
//   du = dy * (n * w + b),   g = dy * u * w,
//   do = rstd * (g - mean(g) - n * mean(g * n)),
// and over all rows dw = sum dy * u * n, db = sum dy * u. The norm and gating
// follow "How Generative Recommenders Are Redefining RecSys at Scale",
// Takeaways (elementwise gating before the output projection).
//
// A workgroup of four waves owns a.rows_per_block consecutive rows (one wave
// per row at a time); each wave keeps its share of dw and db in registers, the four
// are added in wave order through LDS and written once as the workgroup's
// partial. A second kernel adds the partials in a fixed order, so the result
// does not depend on timing.
// HBM-bound: per element it reads O (4 B; 2 B of deviations from the saved
// forward), U and dY (2 B each) and writes dU and dO (2 B each).
#include "kernels.h"

namespace hstu {

constexpr int LNB_WAVES = 4;   // waves per workgroup

__device__ inline float lnb_wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ inline f32x4 ld_bf4(const bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ inline void st_bf4(bf16* p, f32x4 x) {
  bf16x4 v;
  for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
  *(bf16x4*)p = v;
}

// NCH: 4-element chunks per lane (see ln_gate_kernel). DEV: the input is the
// forward's norm-ready store instead of fp32 O: the row's mean and variance
// come from the heads' (mean, M2) pairs (merged as in the forward's norm,
// mean = average of mean_h, M2 = sum M2_h + d sum (mean_h - mean)^2), and
// o - mean = deviation + (mean_h - mean).
template <int NCH, bool FULL_LANES, bool DEV>
__global__ __launch_bounds__(64 * LNB_WAVES) void ln_bwd_kernel(LnBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = a.HD / 4;
  bool on[NCH];
  int col[NCH];
  f32x4 w[NCH], bb[NCH], dw[NCH], db[NCH];
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    on[i] = FULL_LANES || c < nch;
    col[i] = 4 * (FULL_LANES ? c : min(c, nch - 1));
    w[i] = a.ln_w ? *(const f32x4*)(a.ln_w + col[i]) : f32x4{1, 1, 1, 1};
    bb[i] = a.ln_b ? *(const f32x4*)(a.ln_b + col[i]) : f32x4{0, 0, 0, 0};
    dw[i] = f32x4{0, 0, 0, 0};
    db[i] = f32x4{0, 0, 0, 0};
  }
  const float inv_hd = 1.0f / (float)a.HD;
  const int64_t row_end = min<int64_t>(a.T, (int64_t)(blockIdx.x + 1) * a.rows_per_block);
  for (int64_t row = (int64_t)blockIdx.x * a.rows_per_block + wave; row < row_end; row += LNB_WAVES) {
    const bf16* urow = (const bf16*)a.u + row * a.HD;
    const bf16* yrow = (const bf16*)a.dy + row * a.HD;
    f32x4 z[NCH], u[NCH], g[NCH];
    float rstd;
    if constexpr (DEV) {
      const int H = a.HD / a.head_dim;
      const bf16* drow = a.o_dev + row * a.HD;
      const float* srow = a.o_stats + 2 * row * H;
      float mh[NCH];
      #pragma unroll
      for (int i = 0; i < NCH; ++i) {
        z[i] = ld_bf4(drow + col[i]);
        u[i] = ld_bf4(urow + col[i]);
        g[i] = ld_bf4(yrow + col[i]);  // dy for now
        mh[i] = srow[2 * (col[i] / a.head_dim)];
      }
      const f32x2 st = lane < H ? *(const f32x2*)(srow + 2 * lane) : f32x2{0.0f, 0.0f};
      const float mean = lnb_wave_sum(st[0]) / (float)H;
      const float dm = lane < H ? st[0] - mean : 0.0f;
      const float m2 = lnb_wave_sum(fmaf((float)a.head_dim * dm, dm, st[1]));
      rstd = rsqrtf(m2 * inv_hd + a.eps);
      #pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const float shift = mh[i] - mean;
        #pragma unroll
        for (int e = 0; e < 4; ++e) z[i][e] += shift;
      }
    } else {
      const float* orow = a.o + row * a.HD;
      #pragma unroll
      for (int i = 0; i < NCH; ++i) {
        z[i] = *(const f32x4*)(orow + col[i]);
        u[i] = ld_bf4(urow + col[i]);
        g[i] = ld_bf4(yrow + col[i]);  // dy for now
      }
      float s = 0.0f;
      #pragma unroll
      for (int i = 0; i < NCH; ++i)
        if (on[i]) s += (z[i][0] + z[i][1]) + (z[i][2] + z[i][3]);
      const float mean = lnb_wave_sum(s) * inv_hd;
      float ss = 0.0f;
      #pragma unroll
      for (int i = 0; i < NCH; ++i) {
        if (!on[i]) continue;
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[i][e] -= mean;
          ss = fmaf(z[i][e], z[i][e], ss);
        }
      }
      rstd = rsqrtf(lnb_wave_sum(ss) * inv_hd + a.eps);
    }
    bf16* durow = (bf16*)a.du + row * a.HD;
    float s1 = 0.0f, s2 = 0.0f;
    #pragma unroll
    for (int i = 0; i < NCH; ++i) {
      f32x4 du;
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float n = z[i][e] * rstd;
        z[i][e] = n;
        du[e] = g[i][e] * fmaf(n, w[i][e], bb[i][e]);
        const float gu = g[i][e] * u[i][e];  // gradient reaching n * w + b
        dw[i][e] = fmaf(gu, n, dw[i][e]);
        db[i][e] += gu;
        g[i][e] = gu * w[i][e];              // gradient reaching n
      }
      if (on[i]) {
        st_bf4(durow + col[i], du);
        s1 += (g[i][0] + g[i][1]) + (g[i][2] + g[i][3]);
        #pragma unroll
        for (int e = 0; e < 4; ++e) s2 = fmaf(g[i][e], z[i][e], s2);
      }
    }
    const float m1 = lnb_wave_sum(s1) * inv_hd, m2 = lnb_wave_sum(s2) * inv_hd;
    bf16* dorow = (bf16*)a.dout + row * a.HD;
    #pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (!on[i]) continue;
      f32x4 d;
      #pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = rstd * (g[i][e] - m1 - z[i][e] * m2);
      st_bf4(dorow + col[i], d);
    }
  }
  if (!a.part) return;
  // add the four waves' shares in wave order: waves 1..3 stage, wave 0 adds
  __shared__ f32x4 stage[LNB_WAVES - 1][2][NCH][64];
  if (wave > 0) {
    #pragma unroll
    for (int i = 0; i < NCH; ++i) {
      stage[wave - 1][0][i][lane] = dw[i];
      stage[wave - 1][1][i][lane] = db[i];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float* pw = a.part + (int64_t)blockIdx.x * a.HD;
  float* pb = a.part + ((int64_t)a.nwaves + blockIdx.x) * a.HD;
  #pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (!on[i]) continue;
    f32x4 w_ = dw[i], b_ = db[i];
    #pragma unroll
    for (int k = 0; k < LNB_WAVES - 1; ++k) {
      w_ += stage[k][0][i][lane];
      b_ += stage[k][1][i][lane];
    }
    *(f32x4*)(pw + col[i]) = w_;
    *(f32x4*)(pb + col[i]) = b_;
  }
}

// dw[c] = sum over workgroups of the partials. 16 groups of 64 threads split
// them (group g takes partials g, g + 16, ...), then one thread adds the 16
// group sums in group order.
constexpr int RED_GROUPS = 16;
__global__ __launch_bounds__(64 * RED_GROUPS) void ln_affine_reduce_kernel(LnBwdArgs a) {
  __shared__ float sw_s[RED_GROUPS][64], sb_s[RED_GROUPS][64];
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  float sw = 0.0f, sb = 0.0f;
  if (c < a.HD && a.part) {
    // 16 partials' loads in flight before their adds; the adds keep order
    constexpr int U = 16;
    int w = grp;
    for (; w + (U - 1) * RED_GROUPS < a.nwaves; w += U * RED_GROUPS) {
      float xw[U], xb[U];
      #pragma unroll
      for (int j = 0; j < U; ++j) {
        xw[j] = a.part[(int64_t)(w + j * RED_GROUPS) * a.HD + c];
        xb[j] = a.part[((int64_t)a.nwaves + w + j * RED_GROUPS) * a.HD + c];
      }
      #pragma unroll
      for (int j = 0; j < U; ++j) {
        sw += xw[j];
        sb += xb[j];
      }
    }
    for (; w < a.nwaves; w += RED_GROUPS) {
      sw += a.part[(int64_t)w * a.HD + c];
      sb += a.part[((int64_t)a.nwaves + w) * a.HD + c];
    }
  }
  sw_s[grp][cl] = sw;
  sb_s[grp][cl] = sb;
  __syncthreads();
  if (grp == 0 && c < a.HD) {
    float tw = 0.0f, tb = 0.0f;
    for (int g = 0; g < RED_GROUPS; ++g) {
      tw += sw_s[g][cl];
      tb += sb_s[g][cl];
    }
    if (a.d_ln_w) a.d_ln_w[c] = tw;
    if (a.d_ln_b) a.d_ln_b[c] = tb;
  }
}

template <bool DEV>
static void launch_ln_bwd_rows(const LnBwdArgs& a, dim3 grid, dim3 blk, hipStream_t s) {
  switch (a.HD) {
    case 256: hipLaunchKernelGGL((ln_bwd_kernel<1, true, DEV>), grid, blk, 0, s, a); return;
    case 512: hipLaunchKernelGGL((ln_bwd_kernel<2, true, DEV>), grid, blk, 0, s, a); return;
    case 1024: hipLaunchKernelGGL((ln_bwd_kernel<4, true, DEV>), grid, blk, 0, s, a); return;
    case 2048: hipLaunchKernelGGL((ln_bwd_kernel<8, true, DEV>), grid, blk, 0, s, a); return;
  }
  const int nch = (int)ceil_div(a.HD / 4, 64);
  if (nch <= 1) hipLaunchKernelGGL((ln_bwd_kernel<1, false, DEV>), grid, blk, 0, s, a);
  else if (nch <= 2) hipLaunchKernelGGL((ln_bwd_kernel<2, false, DEV>), grid, blk, 0, s, a);
  else if (nch <= 4) hipLaunchKernelGGL((ln_bwd_kernel<4, false, DEV>), grid, blk, 0, s, a);
  else hipLaunchKernelGGL((ln_bwd_kernel<8, false, DEV>), grid, blk, 0, s, a);
}

hipError_t launch_ln_bwd(const LnBwdArgs& a, hipStream_t s) {
  if (a.HD <= 0) return hipSuccess;
  if (a.T <= 0 || a.nwaves <= 0) {  // no rows: the affine gradients are zero
    if (!a.d_ln_w && !a.d_ln_b) return hipSuccess;
    hipLaunchKernelGGL(ln_affine_reduce_kernel, dim3((unsigned)ceil_div(a.HD, 64)), dim3(64 * RED_GROUPS), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.nwaves), blk(64 * LNB_WAVES);
  if (a.o_dev != nullptr) {
    if (a.head_dim < 4 || a.head_dim % 4 != 0 || a.HD % a.head_dim != 0 || a.HD / a.head_dim > 64)
      return hipErrorInvalidValue;
    launch_ln_bwd_rows<true>(a, grid, blk, s);
  } else {
    launch_ln_bwd_rows<false>(a, grid, blk, s);
  }
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (a.d_ln_w || a.d_ln_b)
    hipLaunchKernelGGL(ln_affine_reduce_kernel, dim3((unsigned)ceil_div(a.HD, 64)), dim3(64 * RED_GROUPS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
