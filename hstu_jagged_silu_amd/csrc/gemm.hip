// Dense bf16 product C = A B on v_mfma_f32_32x32x16_bf16 with the layer's
// epilogues fused: plain (f2, the output projection) or SiLU followed by the
// split of the columns into U, V, Q, K (f1). The layer structure (pointwise
// projection with SiLU producing the gate U and the attention inputs, gating
// before the output projection) follows "How Generative Recommenders Are
// Redefining RecSys at Scale", Takeaways.
//
// A is [M, K] row-major (tokens x features), B is [K, N] row-major (weights).
// A workgroup of four waves computes a 256 x 256 tile of C, each wave a
// 128 x 128 quarter as 4 x 4 blocks of 32 x 32 (256 fp32 accumulators per
// lane, one wave per SIMD). It is computed transposed, C^T = B^T A^T: the
// MFMA's first operand is a column block of B (read from the row-major B
// tile with transposing LDS reads), the second a row block of A (plain
// 16-byte LDS reads), and the accumulator then gives each lane four
// consecutive output columns per register group, stored 8 bytes at a time.
// K advances in steps of 64 with two LDS stages filled by LDS DMA
// (global_load_lds, 16 bytes per lane). Per step every operand is first read
// from LDS into registers, then the next step's DMA is issued into the other
// stage, then the 64 MFMAs run from registers while it lands (one call site
// for the step keeps the 256 accumulators in one register assignment, in the
// accumulation registers).
// Swizzles (XOR on 16-byte chunks): A rows are 128 bytes, two per 256-byte
// bank window, so row r uses (r >> 1) mod 8 and 16 consecutive rows read at
// one chunk hit 16 distinct chunk slots; B rows are 512 bytes and a
// transposing read covers 4 rows x 64 bytes, so row r uses 4 (r mod 4).
#include "gemm.h"

namespace hstu {

constexpr int GM = 256, GN = 256, GK = 64;
constexpr int G_THREADS = 256;

typedef short g_v4i16 __attribute__((ext_vector_type(4)));
#define G_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

struct GemmStage {
  unsigned char a[GM * GK * 2] __attribute__((aligned(16)));  // [256 rows (m)][64 k]
  unsigned char b[GK * GN * 2] __attribute__((aligned(16)));  // [64 rows (k)][256 n]
};

__device__ inline int swz_a(int r) { return (r >> 1) & 7; }
__device__ inline int swz_b(int r) { return 4 * (r & 3); }

template <int EPI>
__global__ __launch_bounds__(G_THREADS) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ GemmStage stages[2];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // tiles of one XCD (workgroups i, i + 8, ...) take a contiguous range, so
  // that the A rows they share stay in that XCD's L2
  const int nt_count = g.N / GN;
  const int64_t total = (int64_t)g.mt_count * nt_count;
  int64_t t = blockIdx.x;
  if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
  const int64_t mt = t / nt_count;
  const int nt = (int)(t % nt_count);
  const int64_t m0 = mt * GM;
  const int n0 = nt * GN;

  // ---- staging: every thread moves 8 chunks of A and 8 of B per K step ----
  auto issue = [&](GemmStage& st, int k0) {
    #pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int base = i * 256 + wave * 64;  // first chunk of this instruction
      const int P = base + lane;
      {
        const int r = P >> 3, cs = P & 7;
        const int c = cs ^ swz_a(r);
        const int64_t row = min(m0 + r, g.M - 1);
        __builtin_amdgcn_global_load_lds((const void*)(g.a + row * g.K + k0 + c * 8), G_LDS(void, st.a + base * 16), 16,
                                         0, 0);
      }
      {
        const int r = P >> 5, cs = P & 31;
        const int c = cs ^ swz_b(r);
        __builtin_amdgcn_global_load_lds((const void*)(g.b + (int64_t)(k0 + r) * g.N + n0 + c * 8),
                                         G_LDS(void, st.b + base * 16), 16, 0, 0);
      }
    }
  };
  auto finish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // per-lane LDS offsets: A rows of the four m blocks (chunk of k substep 0),
  // and the transposing reads of B for the four n blocks (two halves)
  uint32_t aoff[4], boff[4][2];
  #pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int r = wm * 128 + mb * 32 + l32;
    aoff[mb] = (uint32_t)(r * 128);
  }
  const int tr_g = lane >> 4, tr_j = lane & 15;
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    #pragma unroll
    for (int s4 = 0; s4 < 2; ++s4) {
      const int r = 8 * (tr_g >> 1) + 4 * s4 + (tr_j >> 2);  // k row within a 16-row substep
      const int col = (wn * 4 + nb) * 32 + 16 * (tr_g & 1) + 4 * (tr_j & 3);
      boff[nb][s4] = (uint32_t)(r * 512 + (((col >> 3) ^ swz_b(r)) << 4) + (col & 7) * 2);
    }
  }
  const int a_sw = swz_a(wm * 128 + l32);  // (r >> 1) & 7 is the same for r + 32 mb

  f32x16 acc[16];
  #pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x16{};

  // One K step: every operand of the step is read from LDS into registers
  // first, then the DMA of the next step is issued into the other stage, then
  // the 64 MFMAs run from registers while that DMA lands.
  auto step = [&](int kk, int nk) {
    auto* al = G_LDS(unsigned char, stages[kk & 1].a);
    auto* bl = G_LDS(unsigned char, stages[kk & 1].b);
    bf16x8 bo[GK / 16][4], ao[GK / 16][4];
    #pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int o = ks * 16 * 512;  // the B swizzle depends on r mod 4 only
        const g_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) g_v4i16*)(bl + boff[nb][0] + o));
        const g_v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) g_v4i16*)(bl + boff[nb][1] + o));
        bo[ks][nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      #pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int c = (2 * ks + hl) ^ a_sw;
        ao[ks][mb] = *(__attribute__((address_space(3))) const bf16x8*)(al + aoff[mb] + (c << 4));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kk + 1 < nk) issue(stages[(kk + 1) & 1], (kk + 1) * GK);
    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks)
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        #pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb * 4 + mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[ks][nb], ao[ks][mb], acc[nb * 4 + mb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // the MFMAs stay ahead of the wait for the DMA
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  const int nk = g.K / GK;
  issue(stages[0], 0);
  finish();
  for (int kk = 0; kk < nk; ++kk) step(kk, nk);

  // ---- epilogue: lane holds row m = .. + l32 and columns 8 g + 4 hl + (0..3) of each n block
  #pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int64_t m = m0 + wm * 128 + mb * 32 + l32;
    if (m >= g.M) continue;
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nblk = n0 + (wn * 4 + nb) * 32;
      bf16* dst;
      if (EPI == GEMM_EPI_SILU_SPLIT) {
        const int part = nblk / g.split;  // split is a multiple of 32
        dst = g.c + part * g.split_stride + m * g.split + (nblk - part * g.split);
      } else {
        dst = g.c + m * g.N + nblk;
      }
      #pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 out;
        #pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = acc[nb * 4 + mb][4 * gq + r];
          if (EPI == GEMM_EPI_SILU_SPLIT) x = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * x));
          out[r] = (bf16)x;
        }
        *(bf16x4*)(dst + 8 * gq + 4 * hl) = out;
      }
    }
  }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const int64_t grid = a.mt_count * (int64_t)(a.N / GN);
  if (a.epilogue == GEMM_EPI_SILU_SPLIT) hipLaunchKernelGGL(gemm_bf16_kernel<GEMM_EPI_SILU_SPLIT>, dim3((unsigned)grid), dim3(G_THREADS), 0, s, a);
  else hipLaunchKernelGGL(gemm_bf16_kernel<GEMM_EPI_NONE>, dim3((unsigned)grid), dim3(G_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
