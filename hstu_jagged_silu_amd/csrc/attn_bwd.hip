// Backward of the fused HSTU SiLU attention on the full causal path (bf16),
// for training ("HSTU Generative Recommenders: Deploy on GPU Cloud", section
// "Scaling Training and Serving Across Multiple GPUs"; "Generative
// recommenders at scale", section "Inside NVIDIA's GPU-native stack for HSTU
// and Semantic IDs"). The pages print no backward; these are the chain rule
// of the forward. With s = alpha q k^T + bias, x = s, a = SiLU(x) / N on
// allowed pairs, o = a v and dO the gradient reaching o:
//   dV = a^T dO,  dP = dO V^T,  dS = dP * SiLU'(x) / N (0 on masked pairs),
//   dQ = alpha dS K,  dK = alpha dS^T Q,
//   d(position table)[c] = sum of dS over pairs in position bucket c, and the
//   same for the time table.
// In the exp2 form of the forward, y = -x log2(e), sigma = 1 / (1 + 2^y),
// SiLU(x) = -ln2 * y * sigma and SiLU'(x) = sigma * (1 + x (1 - sigma)). The
// constant factors (-ln2 / N, alpha / N, 1 / N) are applied once, at the end.
//
// Two kernels, neither with atomics on global memory:
//   * attn_bwd_dkdv_kernel owns 128 keys and walks the query tiles that can
//     see them: S = Q K^T and dP = dO V^T (Q and dO rows from LDS, K and V in
//     registers), then dV^T += dO^T P and dK^T += Q^T dS. The item of query
//     tile t of a user maps to key block (tiles - 1 - t), whose cost matches.
//     For d = 128, attn_bwd_dkdv8_kernel does the same work with eight waves
//     (two per SIMD) and K and V held in LDS instead of registers, and also
//     writes dS (bf16) of every causal 64 x 64 block to HBM.
//   * attn_bwd_dq_kernel owns 128 query rows (one work item of the forward
//     scheduler) and walks their key tiles like the forward: S^T = K Q^T and
//     dP^T = V dO^T on MFMA (K and V rows from LDS, Q and dO in registers),
//     dS^T elementwise, dQ^T += K^T dS^T (K^T by transposing LDS reads). It
//     also sums dS into per-wave position/time histograms in LDS. For d =
//     128, attn_bwd_dq_ds_kernel reads the stored dS instead of recomputing
//     it (dQ^T += K^T dS^T only), after the dK/dV kernel.
// A third kernel adds the per-item histograms in canonical item order.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "tile.h"

namespace hstu {

// time-bucket index z = clz64(|dt| + 1): from the low 32-bit words when the
// tile's |dt| is known to stay below 2^31 - 2 (the 32-bit difference of the
// low words is then exact), from the full 64-bit difference otherwise
template <bool SMALL>
__device__ inline int time_z(int64_t ta, int64_t tb, int32_t ta_lo, int32_t tb_lo) {
  if constexpr (SMALL) {
    const int32_t dt = ta_lo - tb_lo;
    return __builtin_clz((uint32_t)(dt < 0 ? -dt : dt) + 1u) + 32;
  } else {
    const int64_t dt = ta - tb;
    return __builtin_clzll((uint64_t)(dt < 0 ? -dt : dt) + 1u);
  }
}

// Time class of a wave tile: the other side's timestamp range [o_min, o_max]
// (keys for dQ, queries for dK / dV; an empty range is replaced by the
// wave's own minimum) against the wave's own [w_min, w_max]. Bits 0..6:
// z = clz64(|dt| + 1) when every pair of the tile falls in one (clamped)
// time bucket, else 127; bit 7: every |dt| stays below 2^31 - 2, so the
// 32-bit bucket form is exact; bit 8: the other side's times all follow the
// wave's and the pairs span exactly two unclamped buckets, the upper one
// b in bits 9..14 (a pair is in b iff its dt >= 2^b - 1). A wave computes
// it for 64 tiles at a time, lane i for tile t0 + i, and each tile reads
// its class with one readlane.
__device__ inline int time_class(int64_t o_min, int64_t o_max, int64_t w_min, int64_t w_max, int n_time_eff) {
  if (o_min > o_max) o_min = o_max = w_min;
  const int64_t d1 = w_max - o_min, d2 = o_max - w_min;
  const bool small = max(d1 < 0 ? -d1 : d1, d2 < 0 ? -d2 : d2) < ((int64_t)1 << 31) - 2;
  int z = 127, two = 0;
  int64_t lo = -1, hi = -1;
  if (w_min >= o_max) { lo = w_min - o_max; hi = w_max - o_min; }
  else if (o_min >= w_max) { lo = o_min - w_max; hi = o_max - w_min; }
  if (lo >= 0) {
    const int zlo = __builtin_clzll((uint64_t)lo + 1), zhi = __builtin_clzll((uint64_t)hi + 1);
    if (min(63 - zlo, n_time_eff - 1) == min(63 - zhi, n_time_eff - 1)) z = zlo;
    else if (small && o_min >= w_max && zhi == zlo - 1 && 63 - zhi <= n_time_eff - 1) two = 256 | ((63 - zhi) << 9);
  }
  return (small ? 128 : 0) | z | two;
}

// Timestamp range (conservative superset) of the packed rows r0 .. r0 + 63,
// from the per-64-row-block ranges the scheduler wrote; per lane.
__device__ inline void row_time_range(const BwdArgs& a, int64_t r0, int64_t& mn, int64_t& mx) {
  const int64_t i0 = min(r0 / KT, a.n_stat_blocks - 1), i1 = min((r0 + KT - 1) / KT, a.n_stat_blocks - 1);
  mn = min(a.tstats[2 * i0], a.tstats[2 * i1]);
  mx = max(a.tstats[2 * i0 + 1], a.tstats[2 * i1 + 1]);
}

__device__ inline int64_t readlane64(int64_t x, int l) {
  return (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l) |
         ((int64_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), l) << 32);
}

// Unpacks a tile's time class (see time_class) for the wave-uniform tile t.
__device__ inline void tile_class(int tcls, int t, bool& time_uniform, int& z_tile, bool& small_span) {
  const int c = __builtin_amdgcn_readlane(tcls, t & 63);
  small_span = (c & 128) != 0;
  time_uniform = (c & 127) != 127;
  if (time_uniform) z_tile = c & 127;
}

struct BwdTables {
  float pos_t[BWD_MAX_NPOS];  // -log2(e) * position table
  float time_t[64];           // -log2(e) * time table, indexed by clz64(|dt| + 1)
};

// Adds v to a float in LDS (ds_add_f32, no return value). The compiler's own
// form of this atomic first waits for every LDS DMA in flight, since it does
// not separate the histogram from the DMA targets, and that would drain the
// next tile's prefetch at every run flush. The barrier that ends each tile
// waits for the add (lgkmcnt(0)); a later read by the same wave is ordered
// behind it because LDS serves a wave's requests in order.
__device__ inline void lds_add_f32(float* p, float v) {
  const uint32_t addr = (uint32_t)(uintptr_t)LDS_PTR(float, p);
  asm volatile("ds_add_f32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// The same add without the memory clobber, for a histogram that receives
// only these adds between two barriers: later LDS reads of other data may
// then be issued ahead of it instead of waiting for it. The compiler does
// not count the add in flight, which only makes its own LDS waits stricter
// (a wave's LDS operations complete in order); the barriers order the adds
// against the plain accesses before and after.
__device__ inline void lds_add_f32_unordered(float* p, float v) {
  const uint32_t addr = (uint32_t)(uintptr_t)LDS_PTR(float, p);
  asm volatile("ds_add_f32 %0, %1" : : "v"(addr), "v"(v));
}

// Eight LDS reads (byte addresses in LDS, 16-bit zero-extended or 32-bit),
// waited for inside the same asm block. For reads of a stage that is
// complete while a DMA fills the other stage: an ordinary LDS load that the
// compiler cannot attribute to one stage makes it wait for every DMA in
// flight first. The early-clobber outputs keep a result from overwriting an
// address still to be read.
__device__ inline void lds_read8_u16(const uint32_t (&a)[8], uint32_t (&v)[8]) {
  asm volatile(
      "ds_read_u16 %0, %8\n\tds_read_u16 %1, %9\n\tds_read_u16 %2, %10\n\tds_read_u16 %3, %11\n\t"
      "ds_read_u16 %4, %12\n\tds_read_u16 %5, %13\n\tds_read_u16 %6, %14\n\tds_read_u16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}
__device__ inline void lds_read8_b32(const uint32_t (&a)[8], uint32_t (&v)[8]) {
  asm volatile(
      "ds_read_b32 %0, %8\n\tds_read_b32 %1, %9\n\tds_read_b32 %2, %10\n\tds_read_b32 %3, %11\n\t"
      "ds_read_b32 %4, %12\n\tds_read_b32 %5, %13\n\tds_read_b32 %6, %14\n\tds_read_b32 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}
__device__ inline float bf16_bits_to_f32(uint32_t x) { return __uint_as_float(x << 16); }

// One histogram per wave (no two waves add to the same word, so every sum
// runs in program order and the result does not depend on wave timing).
struct RabHist {
  float pos[NWAVES][BWD_MAX_NPOS];  // sum of dS' per position bucket
  float time[NWAVES][64];           // per time bucket
};

template <int NT = NTHREADS>
__device__ inline void load_bwd_tables(const BwdArgs& a, int h, BwdTables& tab, int n_pos) {
  const int tid = threadIdx.x;
  const float* pt = a.pos_tab ? a.pos_tab + (int64_t)h * a.pos_stride : nullptr;
  for (int i = tid; i < n_pos; i += NT) tab.pos_t[i] = pt ? pt[i] * -LOG2E : 0.0f;
  if (tid < 64) {
    float t = 0.0f;
    if (a.time_tab) t = a.time_tab[(int64_t)h * a.time_stride + min(63 - tid, a.n_time - 1)] * -LOG2E;
    tab.time_t[tid] = t;
  }
}

__device__ inline float wave_sum_f(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// XOR swizzle (on 16-byte chunks) of the tiles the backward reads both by
// rows (16 lanes, 16 rows, one chunk) and transposed (32 lanes: 4 rows x 4
// chunks per 256-byte window). For d = 128, s(r) = (r mod 16) xor 4 (r mod 4)
// gives 16 rows 16 distinct chunk offsets, and 4 consecutive rows x 4 chunks
// 16 distinct chunks, so both reads are free of bank conflicts. It depends on
// r mod 16 only, so row offsets that are multiples of 16 can be added later.
// Other head dims use the row swizzle of the forward.
template <int D>
__device__ inline int swz_b(int r) {
  if constexpr (D == 128) return (r & 15) ^ (4 * (r & 3));
  else return Geo<bf16, D>::swz_k(r);
}
template <int D>
__device__ inline int b_off(int r, int c) { return r * Geo<bf16, D>::ROWB + ((c ^ swz_b<D>(r)) << 4); }

// Offset of this lane's transposing read (ds_read_b64_tr_b16): rows
// 16c .. 16c + 15 of the tile (c = 16-row chunk), columns 32db .. 32db + 31,
// half s4 of the 8 rows a lane supplies.
template <int D>
__device__ inline uint32_t tr_off_b(int lane, int db, int c, int s4) {
  using G = Geo<bf16, D>;
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int row = 16 * c + 8 * (tr_g >> 1) + 4 * s4 + (tr_j >> 2);
  const int d = 32 * db + 16 * (tr_g & 1) + 4 * (tr_j & 3);
  return (uint32_t)(b_off<D>(row, d / G::EPC) + (d % G::EPC) * 2);
}

// y -> (P', dS') for one score: P' = y * sigma, dS' = dp * sigma * (1 + x (1 - sigma)), x = -ln2 y.
// Since x sigma = -ln2 P', the last factor is 1 - ln2 y + ln2 P': two fma
// instead of a multiply, a subtract and an fma (both forms carry an absolute
// error of order |x| 2^-24 in that factor)
__device__ inline void silu_fwd_bwd(float y, float dp, float& p, float& ds) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
  p = y * sg;
  const float w = fmaf(LN2, p, fmaf(-LN2, y, 1.0f));
  ds = (dp * sg) * w;
}

// Stage HBM -> LDS of KT rows of two [T, H, D] tensors (rows r0 .. r0 + KT - 1
// of head h, clamped to the last valid row) plus their timestamps, by the NW
// waves of the workgroup.
template <int D, int NW = NWAVES>
__device__ inline void stage_rows(const BwdArgs& a, const void* x0, const void* x1, Stage<bf16, D>& st, int64_t r0,
                                  int nvalid, int h, int64_t& tsreg) {
  using G = Geo<bf16, D>;
  constexpr int ND = G::TILE / (NW * 1024);  // 1 KB LDS DMA instructions per wave and tensor
  static_assert(ND >= 1 && ND * NW * 1024 == G::TILE, "tile staging map");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int last = max(nvalid - 1, 0);
  // a lane's source is the tile's base (wave-uniform) plus a 32-bit offset:
  // at most 63 rows of H * D <= 2048 elements (a 24-bit product)
  const uint32_t rstride = (uint32_t)(a.H * G::ROWB);
  const unsigned char* b0 = (const unsigned char*)x0 + ((r0 * a.H + h) * D) * 2;
  const unsigned char* b1 = (const unsigned char*)x1 + ((r0 * a.H + h) * D) * 2;
  #pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int base = (wave * ND + i) * 64;
    const int P = base + lane;
    const int r = P / G::CPR, pc = P % G::CPR;
    const uint32_t off = __umul24((uint32_t)min(r, last), rstride) + (uint32_t)((pc ^ swz_b<D>(r)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)(b0 + off), LDS_PTR(void, st.k + base * 16), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(b1 + off), LDS_PTR(void, st.v + base * 16), 16, 0, 0);
  }
  if (wave == 0) tsreg = a.ts[r0 + min(lane, last)];
}

template <int D>
__device__ inline void finish_stage(Stage<bf16, D>& st, int64_t tsreg) {
  __builtin_amdgcn_s_waitcnt(0);
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) {
    st.ts_lo[threadIdx.x & 63] = (int32_t)tsreg;
    st.ts64[threadIdx.x & 63] = tsreg;
  }
  __syncthreads();
}

// Store 128 rows x D of fp32 accumulators (O^T layout: lane = row, registers =
// d) scaled by `scale` as bf16 rows of a [T, H, D] tensor, through LDS.
template <int D>
__device__ inline void store_rows_t(const f32x16* acc, float scale, Stage<bf16, D>& st0, Stage<bf16, D>& st1,
                                    void* dst, int64_t row0, int nrows, int h, int H) {
  constexpr int OCPR = D / 4;
  constexpr int NDB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = tid >> 6;
  const int row_w = wave * 32 + l32;
  auto ostage = [&](int r) { return (float*)(r < 64 ? (unsigned char*)&st0 : (unsigned char*)&st1) + (r & 63) * D; };
  __syncthreads();
  #pragma unroll
  for (int db = 0; db < NDB; ++db) {
    #pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = (32 * db + 8 * g + 4 * hl) / 4;
      f32x4 x = {acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale, acc[db][4 * g + 2] * scale,
                 acc[db][4 * g + 3] * scale};
      *(f32x4*)(ostage(row_w) + (c ^ (row_w % OCPR)) * 4) = x;
    }
  }
  __syncthreads();
  for (int i = tid; i < QT * OCPR; i += NTHREADS) {
    const int r = i / OCPR, c = i % OCPR;
    if (r < nrows) {
      const f32x4 x = *(const f32x4*)(ostage(r) + (c ^ (r % OCPR)) * 4);
      bf16x4 v = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
      *(bf16x4*)((bf16*)dst + ((row0 + r) * H + h) * D + c * 4) = v;
    }
  }
}

// ============================================================================
// dQ and the bias-table gradients: one forward work item (128 query rows)
// ============================================================================
template <int D>
__global__ __launch_bounds__(NTHREADS, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  using T = bf16;
  using G = Geo<T, D>;
  using M = Mfma<T>;
  __shared__ Stage<T, D> st0;  // k: K rows, v: V rows (both with swz_b)
  __shared__ Stage<T, D> st1;
  __shared__ BwdTables tab;
  __shared__ RabHist hist;

  const int tid = threadIdx.x;
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t count = ldc(a.count);
  const WorkItem it = ldc(a.items + blockIdx.x);  // in bounds for every workgroup of the grid
  if ((int64_t)blockIdx.x >= (int64_t)count) return;
  const int b = it.b, h = it.h, q_start = it.q_start, q_len = it.q_len;
  const int k_begin = it.k_begin, k_end = it.k_end;
  const int H = a.H;
  const int64_t q_off = it.off;
  const int L = it.L;
  const int n_norm = a.norm_n > 0 ? a.norm_n : L;
  const int n_pos = a.pos_tab ? a.n_pos : 1;
  load_bwd_tables(a, h, tab, n_pos);
  for (int i = tid; i < NWAVES * BWD_MAX_NPOS; i += NTHREADS) (&hist.pos[0][0])[i] = 0.0f;
  for (int i = tid; i < NWAVES * 64; i += NTHREADS) (&hist.time[0][0])[i] = 0.0f;

  const int row_w = wave * 32 + l32;
  const bool row_ok = row_w < q_len;
  const int row_c = min(row_w, q_len - 1);
  const int64_t qrow = q_off + q_start + row_c;
  const int p_lane = q_start + row_c;
  const int64_t tsq = a.ts[qrow];
  const int w_first = wave * 32;
  const bool w_rows = w_first < q_len;
  const int w_last = min(w_first + 31, q_len - 1);
  const int w_lim_min = q_start + w_first, w_lim_max = q_start + w_last;
  int64_t w_ts_min = row_ok ? tsq : INT64_MAX, w_ts_max = row_ok ? tsq : INT64_MIN;
  for (int m = 32; m >= 1; m >>= 1) {
    w_ts_min = min(w_ts_min, shfl_xor64(w_ts_min, m));
    w_ts_max = max(w_ts_max, shfl_xor64(w_ts_max, m));
  }
  w_ts_min = uniform64(w_ts_min);
  w_ts_max = uniform64(w_ts_max);

  // Q and dO rows of this lane as MFMA B operands
  bf16x8 qop[G::NQOP], dop[G::NQOP];
  {
    const T* qp = (const T*)a.q + (qrow * H + h) * D;
    const T* gp = (const T*)a.dout + (qrow * H + h) * D;
    #pragma unroll
    for (int s = 0; s < G::NQOP; ++s) {
      bf16x8 x = *(const bf16x8*)(qp + 16 * s + 8 * hl);
      bf16x8 y = *(const bf16x8*)(gp + 16 * s + 8 * hl);
      if (!row_ok) { x = bf16x8{}; y = bf16x8{}; }
      qop[s] = x;
      dop[s] = y;
    }
  }
  // Operand offsets. K / V rows (A operand, in the order of M::krow): the
  // chunk of step i of row r sits at r * ROWB + ((2i + hl) xor swz(r)) * 16
  // = (r * ROWB + (hl xor swz(r)) * 16) xor 32i, since the row and chunk
  // fields do not overlap. Transposing reads of d block db: the offset of
  // block 0 xor 64db.
  const int kr = M::krow(0, l32);
  const uint32_t k_base = (uint32_t)(kr * G::ROWB + ((hl ^ swz_b<D>(kr)) << 4));
  const uint32_t t_base0 = tr_off_b<D>(lane, 0, 0, 0), t_base1 = tr_off_b<D>(lane, 0, 0, 1);
  f32x16 dqacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) dqacc[i] = f32x16{};
  const float sc = a.alpha * -LOG2E;
  const bool has_time = a.time_tab != nullptr;
  const int n_time_eff = has_time ? min(a.n_time, 64) : 1;
  using LB = __attribute__((address_space(3))) unsigned char;

  int tcls = 0;  // this lane's tile time class (time_class), filled 64 tiles at a time
  auto compute_tile = [&](Stage<T, D>& st, int j0, int t) {
    if (!w_rows || j0 > w_lim_max) return;
    const bool need_mask = j0 + KT - 1 > w_lim_min;
    // one bias constant for the whole wave tile?
    const bool pos_uniform = (a.pos_tab == nullptr) || (w_lim_min - (j0 + KT - 1) >= n_pos - 1);
    bool time_uniform = !has_time;
    int z_tile = 63;
    bool small_span = true;
    if (has_time) tile_class(tcls, t, time_uniform, z_tile, small_span);
    const bool fast = pos_uniform && time_uniform && !need_mask;
    const float c_uni = (a.pos_tab ? tab.pos_t[n_pos - 1] : 0.0f) + (has_time ? tab.time_t[z_tile] : 0.0f);
    const int lim_rel = p_lane - j0 - M::HLK * hl;  // key_of(kb, v, 0) <= lim_rel: allowed
    const int64_t* ts_l = st.ts64 + M::HLK * hl;
    const int32_t* tsl_lo = st.ts_lo + M::HLK * hl;
    const int32_t tsq_lo = (int32_t)tsq;
    LB* kl = LDS_PTR(unsigned char, st.k);
    LB* vl = LDS_PTR(unsigned char, st.v);
    // the bases pass through an empty asm so that the offsets derived from
    // them are formed here, in every tile, instead of being kept in registers
    uint32_t kb_t = k_base, tb0 = t_base0, tb1 = t_base1;
    asm volatile("" : "+v"(kb_t), "+v"(tb0), "+v"(tb1));
    float tile_sum = 0.0f;
    // General path: a lane's keys come in increasing order along v, so with
    // ordered timestamps its time bucket (and a clamped position bucket)
    // stays the same over runs of keys. dS' is summed per run and added to
    // the wave's histogram when the bucket changes, not once per pair.
    int cur_p = -1, cur_t = -1;
    float run_p = 0.0f, run_t = 0.0f;
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T and dP^T as two interleaved chains, the K and V operands of step
      // i + 1 read while the MFMAs of step i run
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 op[2][2];
      auto read_step = [&](int i, bf16x8* o) {
        const uint32_t off = (kb_t ^ (uint32_t)(i << 5)) + kb * 32 * G::ROWB;
        o[0] = *(__attribute__((address_space(3))) const bf16x8*)(kl + off);
        o[1] = *(__attribute__((address_space(3))) const bf16x8*)(vl + off);
      };
      read_step(0, op[0]);
      #pragma unroll
      for (int i = 0; i < G::NQOP; ++i) {
        if (i + 1 < G::NQOP) read_step(i + 1, op[(i + 1) & 1]);
        s = M::run(op[i & 1][0], qop[i], s);
        dp = M::run(op[i & 1][1], dop[i], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 dsb[2];
      if (fast) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p, ds;
          silu_fwd_bwd(fmaf(s[v], sc, c_uni), dp[v], p, ds);
          tile_sum += ds;
          dsb[v >> 3][v & 7] = (bf16)ds;
        }
      } else {
        auto general = [&](auto small_tag) {
          constexpr bool SMALL = decltype(small_tag)::value;
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kk = M::key_of(kb, v, 0);
            const bool ok = kk <= lim_rel;
            const int rel = lim_rel - kk;  // query position - key position
            const int pb = min((unsigned)rel, (unsigned)(n_pos - 1));
            float cb = a.pos_tab ? tab.pos_t[pb] : 0.0f;
            int tb = 0;
            if (has_time) {
              const int zc = time_z<SMALL>(tsq, SMALL ? 0 : ts_l[kk], tsq_lo, SMALL ? tsl_lo[kk] : 0);
              cb += tab.time_t[zc];
              tb = min(63 - zc, n_time_eff - 1);
            }
            float p, ds;
            silu_fwd_bwd(ok ? fmaf(s[v], sc, cb) : MASKED_Y, dp[v], p, ds);
            dsb[v >> 3][v & 7] = (bf16)ds;
            if (ok && row_ok) {
              if (a.pos_tab) {
                if (pb != cur_p) {
                  if (cur_p >= 0) lds_add_f32(&hist.pos[wave][cur_p], run_p);
                  cur_p = pb;
                  run_p = 0.0f;
                }
                run_p += ds;
              }
              if (has_time) {
                if (tb != cur_t) {
                  if (cur_t >= 0) lds_add_f32(&hist.time[wave][cur_t], run_t);
                  cur_t = tb;
                  run_t = 0.0f;
                }
                run_t += ds;
              }
            }
          }
        };
        if (small_span) general(std::true_type{});
        else general(std::false_type{});
      }
      // dQ^T += K^T dS^T for the 32 keys of block kb, the transposed
      // operands of d block db + 1 read during the MFMAs of block db
      bf16x8 kt[2][2];
      auto read_tr = [&](int db, bf16x8* o) {
        #pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int off = (2 * kb + cc) * 16 * G::ROWB;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(kl + (tb0 ^ (uint32_t)(db << 6)) + off));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(kl + (tb1 ^ (uint32_t)(db << 6)) + off));
          o[cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      read_tr(0, kt[0]);
      __builtin_amdgcn_sched_barrier(0);
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        if (db + 1 < G::NDB) read_tr(db + 1, kt[(db + 1) & 1]);
        #pragma unroll
        for (int cc = 0; cc < 2; ++cc) dqacc[db] = M::run(kt[db & 1][cc], dsb[cc], dqacc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (cur_p >= 0) lds_add_f32(&hist.pos[wave][cur_p], run_p);
    if (cur_t >= 0) lds_add_f32(&hist.time[wave][cur_t], run_t);
    if (fast) {
      // rows past q_len have zero dO, so their dS' is 0 and they add nothing
      const float tot = wave_sum_f(tile_sum);
      if (lane == 0) {
        if (a.pos_tab) hist.pos[wave][n_pos - 1] += tot;
        if (has_time) hist.time[wave][min(63 - z_tile, n_time_eff - 1)] += tot;
      }
    }
  };

  const int ntiles = k_end > k_begin ? (int)ceil_div(k_end - k_begin, KT) : 0;
  int64_t tsreg = 0;
  auto issue = [&](Stage<T, D>& st, int j0) {
    stage_rows<D>(a, a.k, a.v, st, q_off + j0, min(KT, L - j0), h, tsreg);
  };
  if (ntiles > 0) {
    issue(st0, k_begin);
    finish_stage<D>(st0, tsreg);
  } else {
    __syncthreads();
  }
  // time classes of the next 64 tiles, lane i for tile t0 + i; the loads are
  // issued before the step's DMA, so waiting for them does not wait for it
  auto time_batch = [&](int t0) {
    const int tl = t0 + lane;
    int c = 255;
    if (tl < ntiles) {
      int64_t mn, mx;
      row_time_range(a, q_off + k_begin + tl * KT, mn, mx);
      c = time_class(mn, mx, w_ts_min, w_ts_max, n_time_eff);
    }
    tcls = c;
  };
  for (int t = 0; t < ntiles; t += 2) {
    if (has_time && (t & 63) == 0) time_batch(t);
    const int j0 = k_begin + t * KT;
    if (t + 1 < ntiles) issue(st1, j0 + KT);
    compute_tile(st0, j0, t);
    if (t + 1 >= ntiles) break;
    finish_stage<D>(st1, tsreg);
    if (t + 2 < ntiles) issue(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT, t + 1);
    if (t + 2 < ntiles) finish_stage<D>(st0, tsreg);
  }

  store_rows_t<D>(dqacc, a.alpha / (float)n_norm, st0, st1, a.dq, q_off + q_start, q_len, h, H);

  // per-item bias gradients (scaled by 1 / N), head-major: the items of head h
  // are [h * tiles, (h + 1) * tiles), tiles = query tiles over all users
  // (the scheduler's prefix counts H items per tile)
  const int64_t tiles = ldc(a.prefix + a.B) / H;
  const int64_t canon = (int64_t)h * tiles + ldc(a.prefix + b) / H + q_start / QT;
  float* part = a.rab_part + canon * RAB_SLOTS;
  const float inv_n = 1.0f / (float)n_norm;
  if (a.pos_tab) {
    for (int i = tid; i < n_pos; i += NTHREADS) {
      float x = 0.0f;
      #pragma unroll
      for (int w = 0; w < NWAVES; ++w) x += hist.pos[w][i];
      part[i] = x * inv_n;
    }
  }
  if (has_time && tid < 64) {
    float x = 0.0f;
    #pragma unroll
    for (int w = 0; w < NWAVES; ++w) x += hist.time[w][tid];
    part[BWD_MAX_NPOS + tid] = x * inv_n;
  }
}

// ============================================================================
// dK and dV: 128 keys, all query tiles at or after them
// ============================================================================
template <int D>
__global__ __launch_bounds__(NTHREADS, D == 128 ? 1 : 2) void attn_bwd_dkdv_kernel(BwdArgs a) {
  using T = bf16;
  using G = Geo<T, D>;
  using M = Mfma<T>;
  __shared__ Stage<T, D> st0;  // k: Q rows, v: dO rows (both with swz_b), ts64: query timestamps
  __shared__ Stage<T, D> st1;
  __shared__ BwdTables tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t count = ldc(a.count);
  const WorkItem it = ldc(a.items + blockIdx.x);  // in bounds for every workgroup of the grid
  if ((int64_t)blockIdx.x >= (int64_t)count) return;
  const int b = it.b, h = it.h;
  const int H = a.H;
  const int64_t q_off = it.off;
  const int L = it.L;
  const int n_norm = a.norm_n > 0 ? a.norm_n : L;
  const int nq = (int)ceil_div(L, QT);
  const int k0 = (nq - 1 - it.q_start / QT) * QT;  // mirrored key block
  const int klen = min(QT, L - k0);
  const int n_pos = a.pos_tab ? a.n_pos : 1;
  load_bwd_tables(a, h, tab, n_pos);

  const int key_w = wave * 32 + l32;
  const bool key_ok = key_w < klen;
  const int kc = min(key_w, klen - 1);
  const int64_t krow = q_off + k0 + kc;
  const int kpos = k0 + kc;
  const int64_t tsk = a.ts[krow];
  const int w_first = wave * 32;
  const bool w_keys = w_first < klen;
  const bool w_full = w_first + 31 < klen;          // every key of the wave valid
  const int w_kmin = k0 + w_first, w_kmax = k0 + min(w_first + 31, klen - 1);
  int64_t w_ts_min = key_ok ? tsk : INT64_MAX, w_ts_max = key_ok ? tsk : INT64_MIN;
  for (int m = 32; m >= 1; m >>= 1) {
    w_ts_min = min(w_ts_min, shfl_xor64(w_ts_min, m));
    w_ts_max = max(w_ts_max, shfl_xor64(w_ts_max, m));
  }
  w_ts_min = uniform64(w_ts_min);
  w_ts_max = uniform64(w_ts_max);
  const int n_time_eff = a.time_tab ? min(a.n_time, 64) : 1;

  bf16x8 kop[G::NQOP], vop[G::NQOP];
  {
    const T* kp = (const T*)a.k + (krow * H + h) * D;
    const T* vp = (const T*)a.v + (krow * H + h) * D;
    #pragma unroll
    for (int s = 0; s < G::NQOP; ++s) {
      bf16x8 x = *(const bf16x8*)(kp + 16 * s + 8 * hl);
      bf16x8 y = *(const bf16x8*)(vp + 16 * s + 8 * hl);
      if (!key_ok) { x = bf16x8{}; y = bf16x8{}; }
      kop[s] = x;
      vop[s] = y;
    }
  }
  uint32_t qoff[G::NQOP], qtr[G::NDB][2];
  {
    const int qr = M::krow(0, l32);
    #pragma unroll
    for (int s = 0; s < G::NQOP; ++s) qoff[s] = (uint32_t)b_off<D>(qr, 2 * s + hl);
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      qtr[db][0] = tr_off_b<D>(lane, db, 0, 0);
      qtr[db][1] = tr_off_b<D>(lane, db, 0, 1);
    }
  }
  f32x16 dkacc[G::NDB], dvacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) { dkacc[i] = f32x16{}; dvacc[i] = f32x16{}; }
  const float sc = a.alpha * -LOG2E;
  const bool has_time = a.time_tab != nullptr;
  using LB = __attribute__((address_space(3))) unsigned char;

  int tcls = 0;  // this lane's tile time class (time_class), filled 64 tiles at a time
  auto compute_tile = [&](Stage<T, D>& st, int j0, int t) {
    // every query of the tile precedes every key of this wave: all masked
    if (!w_keys || j0 + KT - 1 < w_kmin) return;
    // one bias constant and no mask for the whole wave tile? (as in the forward)
    const bool need_mask = !w_full || j0 < w_kmax || j0 + KT > L;
    const bool pos_uniform = (a.pos_tab == nullptr) || (j0 - w_kmax >= n_pos - 1);
    bool time_uniform = !has_time;
    int z_tile = 63;
    bool small_span = true;
    if (has_time) tile_class(tcls, t, time_uniform, z_tile, small_span);
    const bool fast = pos_uniform && time_uniform && !need_mask;
    const float c_uni = (a.pos_tab ? tab.pos_t[n_pos - 1] : 0.0f) + (has_time ? tab.time_t[z_tile] : 0.0f);
    const int64_t* ts_l = st.ts64 + M::HLK * hl;
    const int32_t* tsl_lo = st.ts_lo + M::HLK * hl;
    const int32_t tsk_lo = (int32_t)tsk;
    LB* ql = LDS_PTR(unsigned char, st.k);
    LB* gl = LDS_PTR(unsigned char, st.v);
    #pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (j0 + 32 * qb + 31 < w_kmin) continue;
      // One wave per SIMD leaves nothing to hide LDS latency behind, and
      // registers to spare: every operand read of the step is issued before
      // the MFMA that needs the first one, the two chains interleave, and the
      // transposed operands of dV and dK are read while the SiLU runs.
      bf16x8 qa[G::NQOP], ga[G::NQOP];
      #pragma unroll
      for (int i = 0; i < G::NQOP; ++i) {
        qa[i] = *(__attribute__((address_space(3))) const bf16x8*)(ql + qoff[i] + qb * 32 * G::ROWB);
        ga[i] = *(__attribute__((address_space(3))) const bf16x8*)(gl + qoff[i] + qb * 32 * G::ROWB);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = f32x16{}, dp = f32x16{};
      #pragma unroll
      for (int i = 0; i < G::NQOP; ++i) {
        s = M::run(qa[i], kop[i], s);
        dp = M::run(ga[i], vop[i], dp);
      }
      bf16x8 gt[G::NDB][2], qt[G::NDB][2];
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        #pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int o = (2 * qb + cc) * 16 * G::ROWB;
          const v4i16 glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(gl + qtr[db][0] + o));
          const v4i16 ghi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(gl + qtr[db][1] + o));
          gt[db][cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7));
          const v4i16 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ql + qtr[db][0] + o));
          const v4i16 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ql + qtr[db][1] + o));
          qt[db][cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pb[2], dsb[2];
      if (fast) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p, ds;
          silu_fwd_bwd(fmaf(s[v], sc, c_uni), dp[v], p, ds);
          pb[v >> 3][v & 7] = (bf16)p;
          dsb[v >> 3][v & 7] = (bf16)ds;
        }
      } else {
        // bias of the 16 pairs first (table reads in one batch per table),
        // then the SiLU terms
        auto general = [&](auto small_tag) {
          constexpr bool SMALL = decltype(small_tag)::value;
          float cb[16];
          if (a.pos_tab) {
            #pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rel = j0 + M::key_of(qb, v, hl) - kpos;
              cb[v] = tab.pos_t[min((unsigned)rel, (unsigned)(n_pos - 1))];
            }
          } else {
            #pragma unroll
            for (int v = 0; v < 16; ++v) cb[v] = 0.0f;
          }
          if (has_time) {
            #pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int qv = M::key_of(qb, v, 0);
              cb[v] += tab.time_t[time_z<SMALL>(SMALL ? 0 : ts_l[qv], tsk, SMALL ? tsl_lo[qv] : 0, tsk_lo)];
            }
          }
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qpos = j0 + M::key_of(qb, v, hl);  // query row
            const bool ok = key_ok && qpos >= kpos && qpos < L;
            float p, ds;
            silu_fwd_bwd(ok ? fmaf(s[v], sc, cb[v]) : MASKED_Y, dp[v], p, ds);
            pb[v >> 3][v & 7] = (bf16)p;
            dsb[v >> 3][v & 7] = (bf16)ds;
          }
        };
        if (small_span) general(std::true_type{});
        else general(std::false_type{});
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries of block qb
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        #pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          dvacc[db] = M::run(gt[db][cc], pb[cc], dvacc[db]);
          dkacc[db] = M::run(qt[db][cc], dsb[cc], dkacc[db]);
        }
      }
    }
  };

  const int ntiles = (int)ceil_div(L - k0, KT);
  int64_t tsreg = 0;
  auto issue = [&](Stage<T, D>& st, int j0) {
    stage_rows<D>(a, a.q, a.dout, st, q_off + j0, min(KT, L - j0), h, tsreg);
  };
  issue(st0, k0);
  finish_stage<D>(st0, tsreg);
  // time classes of the next 64 tiles, lane i for tile t0 + i; the loads are
  // issued before the step's DMA, so waiting for them does not wait for it
  auto time_batch = [&](int t0) {
    const int tl = t0 + lane;
    int c = 255;
    if (tl < ntiles) {
      int64_t mn, mx;
      row_time_range(a, q_off + k0 + tl * KT, mn, mx);
      c = time_class(mn, mx, w_ts_min, w_ts_max, n_time_eff);
    }
    tcls = c;
  };
  for (int t = 0; t < ntiles; t += 2) {
    if (has_time && (t & 63) == 0) time_batch(t);
    const int j0 = k0 + t * KT;
    if (t + 1 < ntiles) issue(st1, j0 + KT);
    compute_tile(st0, j0, t);
    if (t + 1 >= ntiles) break;
    finish_stage<D>(st1, tsreg);
    if (t + 2 < ntiles) issue(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT, t + 1);
    if (t + 2 < ntiles) finish_stage<D>(st0, tsreg);
  }
  store_rows_t<D>(dvacc, -LN2 / (float)n_norm, st0, st1, a.dv, q_off + k0, klen, h, H);
  store_rows_t<D>(dkacc, a.alpha / (float)n_norm, st0, st1, a.dk, q_off + k0, klen, h, H);
}

// ============================================================================
// dK and dV for d = 128: eight waves, two per SIMD
// ============================================================================
// The four-wave kernel above keeps K, V and both accumulators of its 32 keys
// in registers (344 and more), so it runs one wave per SIMD, and a lone wave
// in order of issue leaves the matrix unit idle while it waits on LDS reads
// and computes the SiLU. Here K and V of the workgroup's 128 keys stay in LDS
// for the whole item, which brings a wave under 256 registers: wave w owns the
// 32 keys of group w mod 4 and the query half w / 4 of every 64-query tile,
// and the two waves of a SIMD cover each other's waits. The two query halves
// keep partial dK and dV sums that are added through LDS at the end, half 0
// first, so the result does not depend on wave timing.
constexpr int DKDV8_WAVES = 8;
constexpr int DKDV8_THREADS = 64 * DKDV8_WAVES;

// K and V rows of the key block (swz_b<128> layout). The two Q/dO stages are
// LDS objects of their own, as in the forward, so the compiler sees that the
// DMA into one stage cannot touch the reads of the other and does not wait
// for it.
struct Dkdv8Keys {
  unsigned char k[QT * 256] __attribute__((aligned(16)));
  unsigned char v[QT * 256] __attribute__((aligned(16)));
};
// The end of the kernel reuses all three: the fp32 partial sums of half 1,
// then the fp32 rows of dV and dK on their way out; dV's 64 KB go to the key
// rows, dK's to the two stages (32 KB each).
static_assert(sizeof(Dkdv8Keys) == QT * 128 * 4 && sizeof(Stage<bf16, 128>) >= QT / 2 * 128 * 4,
              "reduction buffers");

__global__ __launch_bounds__(DKDV8_THREADS, 2) void attn_bwd_dkdv8_kernel(BwdArgs a) {
  constexpr int D = 128;
  using T = bf16;
  using G = Geo<T, D>;
  using M = Mfma<T>;
  static_assert(G::ROWB == 256 && G::CPR == 16, "resident key rows of 256 bytes");
  __shared__ Stage<T, D> st0;
  __shared__ Stage<T, D> st1;
  __shared__ Dkdv8Keys kv;
  __shared__ BwdTables tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, qb = wave >> 2;  // key group, query half
  const int32_t count = ldc(a.count);
  const WorkItem it = ldc(a.items + blockIdx.x);  // in bounds for every workgroup of the grid
  if ((int64_t)blockIdx.x >= (int64_t)count) return;
  const int h = it.h;
  const int H = a.H;
  const int64_t q_off = it.off;
  const int L = it.L;
  const int n_norm = a.norm_n > 0 ? a.norm_n : L;
  const int nq = (int)ceil_div(L, QT);
  const int k0 = (nq - 1 - it.q_start / QT) * QT;  // mirrored key block
  const int klen = min(QT, L - k0);
  const int n_pos = a.pos_tab ? a.n_pos : 1;
  load_bwd_tables<DKDV8_THREADS>(a, h, tab, n_pos);
  // dS of every causal 64 x 64 (key, query) block of the user goes to HBM
  // for the dQ kernel: this wave writes key rows 32 (kg mod 2) .. + 31 of
  // block row kt, query columns 32 qb .. + 31 (8 per half-wave and register
  // group), zeros where the pair is masked
  const int nbb = (int)ceil_div(L, KT);
  const int64_t ds_blk0 = (int64_t)H * ldc(a.ds_prefix + it.b) + (int64_t)h * nbb * (nbb + 1) / 2;
  const int ds_kt = k0 / KT + (kg >> 1);
  const uint32_t ds_lane = (uint32_t)((32 * (kg & 1) + l32) * KT + 32 * qb + 8 * hl);
  auto store_ds = [&](int j0, bf16x8 x0, bf16x8 x1) {
    const int qt = j0 / KT;
    const int64_t gb = ds_blk0 + (int64_t)qt * (qt + 1) / 2 + ds_kt;
    if (gb < a.ds_cap) {
      bf16* p = a.ds + gb * (KT * KT) + ds_lane;
      __builtin_nontemporal_store(x0, (bf16x8*)p);
      __builtin_nontemporal_store(x1, (bf16x8*)(p + 16));
    }
  };

  // K and V of the 128 keys into LDS (rows past the user's end are copies of
  // its last row; their pairs are masked): 2,048 16-byte chunks per tensor
  {
    const int64_t rstride = (int64_t)H * G::ROWB;
    const unsigned char* kb = (const unsigned char*)a.k + (((q_off + k0) * H + h) * D) * 2;
    const unsigned char* vb = (const unsigned char*)a.v + (((q_off + k0) * H + h) * D) * 2;
    constexpr int NR = QT * G::CPR / DKDV8_THREADS;  // chunks per lane and tensor
    #pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int base = (wave * NR + i) * 64;
      const int P = base + lane;
      const int r = P / G::CPR, pc = P % G::CPR;
      const int64_t off = min(r, klen - 1) * rstride + ((pc ^ swz_b<D>(r)) << 4);
      __builtin_amdgcn_global_load_lds((const void*)(kb + off), LDS_PTR(void, kv.k + base * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb + off), LDS_PTR(void, kv.v + base * 16), 16, 0, 0);
    }
  }

  const int key_w = kg * 32 + l32;
  const bool key_ok = key_w < klen;
  const int kc = min(key_w, klen - 1);
  const int64_t krow = q_off + k0 + kc;
  const int kpos = k0 + kc;
  const int64_t tsk = a.ts[krow];
  const int w_first = kg * 32;
  const bool w_keys = w_first < klen;
  const bool w_full = w_first + 31 < klen;          // every key of the wave valid
  const int w_kmin = k0 + w_first, w_kmax = k0 + min(w_first + 31, klen - 1);
  int64_t w_ts_min = key_ok ? tsk : INT64_MAX, w_ts_max = key_ok ? tsk : INT64_MIN;
  for (int m = 32; m >= 1; m >>= 1) {
    w_ts_min = min(w_ts_min, shfl_xor64(w_ts_min, m));
    w_ts_max = max(w_ts_max, shfl_xor64(w_ts_max, m));
  }
  w_ts_min = uniform64(w_ts_min);
  w_ts_max = uniform64(w_ts_max);
  const int n_time_eff = a.time_tab ? min(a.n_time, 64) : 1;

  // Operand offsets. Q / dO rows of this half (A operand, rows in the order
  // of M::krow so the accumulators are the B operands of dV and dK) and K / V
  // rows of this key group (B operand): the chunk of step i of row r sits at
  // r * 256 + ((2i + hl) xor swz(r)) * 16 = (r * 256 + (hl xor swz(r)) * 16)
  // xor 32i. Transposing reads of d block db: the offset of block 0 xor 64db.
  const int qr = M::krow(0, l32) + 32 * qb;
  const uint32_t q_base = (uint32_t)(qr * G::ROWB + ((hl ^ swz_b<D>(qr)) << 4));
  const uint32_t k_base = (uint32_t)(key_w * G::ROWB + ((hl ^ swz_b<D>(key_w)) << 4));
  const uint32_t t_base0 = tr_off_b<D>(lane, 0, 0, 0) + qb * 32 * G::ROWB;
  const uint32_t t_base1 = tr_off_b<D>(lane, 0, 0, 1) + qb * 32 * G::ROWB;
  f32x16 dkacc[G::NDB], dvacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) { dkacc[i] = f32x16{}; dvacc[i] = f32x16{}; }
  const float sc = a.alpha * -LOG2E;
  const bool has_time = a.time_tab != nullptr;
  using LB = __attribute__((address_space(3))) unsigned char;
  using LV = __attribute__((address_space(3))) const bf16x8;
  using LT = __attribute__((address_space(3))) v4i16;
  LB* kl = LDS_PTR(unsigned char, kv.k);
  LB* vl = LDS_PTR(unsigned char, kv.v);

  int tcls = 0;  // this lane's tile time class (time_class), filled 64 tiles at a time
  auto compute_tile = [&](Stage<T, D>& st, int j0, int t) {
    // every query of this half precedes every key of this wave (or the
    // wave has no keys): all masked (the zeros of its dS are written after
    // the loop)
    if (!w_keys || j0 + 32 * qb + 31 < w_kmin) return;
    // one bias constant and no mask for the whole wave tile? (as in the forward)
    const bool need_mask = !w_full || j0 < w_kmax || j0 + KT > L;
    const bool pos_uniform = (a.pos_tab == nullptr) || (j0 - w_kmax >= n_pos - 1);
    bool time_uniform = !has_time;
    int z_tile = 63;
    bool small_span = true;
    if (has_time) tile_class(tcls, t, time_uniform, z_tile, small_span);
    const bool fast = pos_uniform && time_uniform && !need_mask;
    // two time buckets (queries after this wave's keys), constant position
    // bias, no mask: bucket by one 32-bit subtract per pair
    int two_b = -1;
    if (has_time && !fast && pos_uniform && !need_mask) {
      const int c = __builtin_amdgcn_readlane(tcls, t & 63);
      if (c & 256) two_b = (c >> 9) & 63;
    }
    const float c_uni = (a.pos_tab ? tab.pos_t[n_pos - 1] : 0.0f) + (has_time ? tab.time_t[z_tile] : 0.0f);
    const int64_t* ts_l = st.ts64 + M::HLK * hl;
    const int32_t* tsl_lo = st.ts_lo + M::HLK * hl;
    const int32_t tsk_lo = (int32_t)tsk;
    LB* ql = LDS_PTR(unsigned char, st.k);
    LB* gl = LDS_PTR(unsigned char, st.v);
    // S = Q K^T and dP = dO V^T over the 32 queries of this half; the
    // operands of step i + 1 are read while the MFMAs of step i run (one step
    // ahead only: reading further ahead costs registers the two waves of a
    // SIMD do not have)
    // the bases pass through an empty asm so that the offsets derived from
    // them are formed here, in every tile, instead of being kept in registers
    uint32_t qb_t = q_base, kb_t = k_base, tb0 = t_base0, tb1 = t_base1;
    asm volatile("" : "+v"(qb_t), "+v"(kb_t), "+v"(tb0), "+v"(tb1));
    f32x16 s = f32x16{}, dp = f32x16{};
    bf16x8 op[2][4];
    auto read_step = [&](int i, bf16x8* o) {
      const uint32_t qo = qb_t ^ (uint32_t)(i << 5), ko = kb_t ^ (uint32_t)(i << 5);
      o[0] = *(LV*)(ql + qo);
      o[1] = *(LV*)(kl + ko);
      o[2] = *(LV*)(gl + qo);
      o[3] = *(LV*)(vl + ko);
    };
    read_step(0, op[0]);
    #pragma unroll
    for (int i = 0; i < G::NQOP; ++i) {
      if (i + 1 < G::NQOP) read_step(i + 1, op[(i + 1) & 1]);
      s = M::run(op[i & 1][0], op[i & 1][1], s);
      dp = M::run(op[i & 1][2], op[i & 1][3], dp);
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb[2], dsb[2];
    if (fast) {
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p, ds;
        silu_fwd_bwd(fmaf(s[v], sc, c_uni), dp[v], p, ds);
        pb[v >> 3][v & 7] = (bf16)p;
        dsb[v >> 3][v & 7] = (bf16)ds;
      }
    } else if (two_b >= 0) {
      // x = (t_q - t_k) - (2^b - 1) in 32 bits (exact: 0 <= dt < 2^31 - 2);
      // the pair is in bucket b iff x >= 0, else in b - 1
      const float c_pos = a.pos_tab ? tab.pos_t[n_pos - 1] : 0.0f;
      const float c_hi = c_pos + tab.time_t[63 - two_b], c_lo = c_pos + tab.time_t[64 - two_b];
      const uint32_t b_lane = (uint32_t)tsk_lo + (uint32_t)((1 << two_b) - 1);
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int32_t x = (int32_t)((uint32_t)tsl_lo[M::key_of(qb, v, 0)] - b_lane);
        float p, ds;
        silu_fwd_bwd(fmaf(s[v], sc, x >= 0 ? c_hi : c_lo), dp[v], p, ds);
        pb[v >> 3][v & 7] = (bf16)p;
        dsb[v >> 3][v & 7] = (bf16)ds;
      }
    } else {
      auto general = [&](auto small_tag) {
        constexpr bool SMALL = decltype(small_tag)::value;
        float cb[16];
        if (a.pos_tab) {
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rel = j0 + M::key_of(qb, v, hl) - kpos;
            cb[v] = tab.pos_t[min((unsigned)rel, (unsigned)(n_pos - 1))];
          }
        } else {
          #pragma unroll
          for (int v = 0; v < 16; ++v) cb[v] = 0.0f;
        }
        if (has_time) {
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qv = M::key_of(qb, v, 0);
            cb[v] += tab.time_t[time_z<SMALL>(SMALL ? 0 : ts_l[qv], tsk, SMALL ? tsl_lo[qv] : 0, tsk_lo)];
          }
        }
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int qpos = j0 + M::key_of(qb, v, hl);  // query row
          const bool ok = key_ok && qpos >= kpos && qpos < L;
          float p, ds;
          silu_fwd_bwd(ok ? fmaf(s[v], sc, cb[v]) : MASKED_Y, dp[v], p, ds);
          pb[v >> 3][v & 7] = (bf16)p;
          dsb[v >> 3][v & 7] = (bf16)ds;
        }
      };
      if (small_span) general(std::true_type{});
      else general(std::false_type{});
    }
    store_ds(j0, dsb[0], dsb[1]);
    // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries of this half,
    // the transposed operands of step db + 1 read during the MFMAs of step db
    bf16x8 tp[2][4];
    auto read_tr = [&](int db, bf16x8* o) {
      #pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const uint32_t o0 = (tb0 ^ (uint32_t)(db << 6)) + cc * 16 * G::ROWB;
        const uint32_t o1 = (tb1 ^ (uint32_t)(db << 6)) + cc * 16 * G::ROWB;
        const v4i16 glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LT*)(gl + o0));
        const v4i16 ghi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LT*)(gl + o1));
        const v4i16 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LT*)(ql + o0));
        const v4i16 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LT*)(ql + o1));
        o[cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[2 + cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    read_tr(0, tp[0]);
    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      if (db + 1 < G::NDB) read_tr(db + 1, tp[(db + 1) & 1]);
      #pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        dvacc[db] = M::run(tp[db & 1][cc], pb[cc], dvacc[db]);
        dkacc[db] = M::run(tp[db & 1][2 + cc], dsb[cc], dkacc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int ntiles = (int)ceil_div(L - k0, KT);
  int64_t tsreg = 0;
  auto issue = [&](Stage<T, D>& st, int j0) {
    stage_rows<D, DKDV8_WAVES>(a, a.q, a.dout, st, q_off + j0, min(KT, L - j0), h, tsreg);
  };
  issue(st0, k0);
  finish_stage<D>(st0, tsreg);  // also waits for the K and V rows
  // time classes of the next 64 tiles, lane i for tile t0 + i; the loads are
  // issued before the step's DMA, so waiting for them does not wait for it
  auto time_batch = [&](int t0) {
    const int tl = t0 + lane;
    int c = 255;
    if (tl < ntiles) {
      int64_t mn, mx;
      row_time_range(a, q_off + k0 + tl * KT, mn, mx);
      c = time_class(mn, mx, w_ts_min, w_ts_max, n_time_eff);
    }
    tcls = c;
  };
  for (int t = 0; t < ntiles; t += 2) {
    if (has_time && (t & 63) == 0) time_batch(t);
    const int j0 = k0 + t * KT;
    if (t + 1 < ntiles) issue(st1, j0 + KT);
    compute_tile(st0, j0, t);
    if (t + 1 >= ntiles) break;
    finish_stage<D>(st1, tsreg);
    if (t + 2 < ntiles) issue(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT, t + 1);
    if (t + 2 < ntiles) finish_stage<D>(st0, tsreg);
  }
  // the all-masked wave tiles of existing dS blocks: zeros (a separate loop,
  // so that the tile loop keeps its register allocation)
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = k0 + t * KT;
    if ((!w_keys || j0 + 32 * qb + 31 < w_kmin) && ds_kt <= j0 / KT && ds_kt * KT < L)
      store_ds(j0, bf16x8{}, bf16x8{});
  }

  // half 1 hands its partial sums to half 0, per tensor [key group][db][4][lane]
  // x f32x4: dV's in the key rows, dK's in stage 0 (key groups 0, 1) and
  // stage 1 (key groups 2, 3)
  __syncthreads();
  using LF4 = __attribute__((address_space(3))) f32x4;
  LF4* red_v = LDS_PTR(f32x4, &kv) + kg * (G::NDB * 4 * 64) + lane;
  LF4* red_k = LDS_PTR(f32x4, kg < 2 ? (void*)&st0 : (void*)&st1) + (kg & 1) * (G::NDB * 4 * 64) + lane;
  if (qb == 1) {
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      #pragma unroll
      for (int g = 0; g < 4; ++g) {
        red_v[(db * 4 + g) * 64] = f32x4{dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
        red_k[(db * 4 + g) * 64] = f32x4{dkacc[db][4 * g], dkacc[db][4 * g + 1], dkacc[db][4 * g + 2], dkacc[db][4 * g + 3]};
      }
    }
  }
  __syncthreads();
  if (qb == 0) {
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      #pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = red_v[(db * 4 + g) * 64], y = red_k[(db * 4 + g) * 64];
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
          dvacc[db][4 * g + j] += x[j];
          dkacc[db][4 * g + j] += y[j];
        }
      }
    }
  }
  __syncthreads();
  // fp32 rows of dV (in the key rows) and dK (rows 0..63 in stage 0, 64..127
  // in stage 1) in LDS, 16-byte chunk c of row r at c xor (r mod 32), then
  // bf16 rows out by all eight waves
  constexpr int OCPR = D / 4;
  using LFP = __attribute__((address_space(3))) float;
  auto orow = [&](int t, int r) -> LFP* {
    if (t == 0) return LDS_PTR(float, &kv) + r * D;
    return LDS_PTR(float, r < 64 ? (void*)&st0 : (void*)&st1) + (r & 63) * D;
  };
  if (qb == 0) {
    const float sv = -LN2 / (float)n_norm, sk = a.alpha / (float)n_norm;
    const int row_w = key_w;
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      #pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = (32 * db + 8 * g + 4 * hl) / 4;
        const int off = (c ^ (row_w % OCPR)) * 4;
        *(LF4*)(orow(0, row_w) + off) =
            f32x4{dvacc[db][4 * g] * sv, dvacc[db][4 * g + 1] * sv, dvacc[db][4 * g + 2] * sv, dvacc[db][4 * g + 3] * sv};
        *(LF4*)(orow(1, row_w) + off) =
            f32x4{dkacc[db][4 * g] * sk, dkacc[db][4 * g + 1] * sk, dkacc[db][4 * g + 2] * sk, dkacc[db][4 * g + 3] * sk};
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < 2 * QT * OCPR; i += DKDV8_THREADS) {
    const int t = i / (QT * OCPR), r = (i / OCPR) % QT, c = i % OCPR;
    if (r < klen) {
      const f32x4 x = *(const LF4*)(orow(t, r) + (c ^ (r % OCPR)) * 4);
      const bf16x4 v = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
      *(bf16x4*)((bf16*)(t == 0 ? a.dv : a.dk) + ((q_off + k0 + r) * H + h) * D + c * 4) = v;
    }
  }
}

// ============================================================================
// dQ and the bias-table gradients for d = 128 from the stored dS
// ============================================================================
// The eight-wave dK/dV kernel has already written dS of every causal 64 x 64
// (key, query) block to HBM, so no score is recomputed here: for each key
// tile of a work item (128 query rows) the workgroup stages the K rows and
// the item's two dS blocks of that tile in LDS, and wave w (rows 32w .. 32w
// + 31, columns 32 (w mod 2) .. of block w / 2) adds K^T dS^T to its dQ^T
// (16 MFMAs per tile, both operands from transposing reads). The histograms
// of the bias-table gradients sum the same bf16 dS values the MFMAs use. The
// kernel is bound by the dS stream from HBM.

// LDS layout of a dS block: 64 key rows of 64 bf16 queries (128 bytes), the
// 16-byte chunk c of row r at c xor (2r mod 8). The transposing reads of a
// B operand cover 4 consecutive rows x 64 bytes per 256-byte window, which
// this swizzle spreads over 64 distinct banks.
constexpr int DS_BLOCK = KT * KT;  // elements of one block
__device__ inline uint32_t ds_chunk_off(int r, int c) { return (uint32_t)(r * (KT * 2) + ((c ^ ((2 * r) & 7)) << 4)); }
// This lane's transposing read of a dS block: key rows 8 (lane / 32) + 4 s4
// + 0..3 (plus 16 per key step), query column 32 db + lane mod 32.
__device__ inline uint32_t ds_tr_off(int lane, int db, int s4) {
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int row = 8 * (tr_g >> 1) + 4 * s4 + (tr_j >> 2);
  const int col = 32 * db + 16 * (tr_g & 1) + 4 * (tr_j & 3);
  return ds_chunk_off(row, col >> 3) + (uint32_t)((col & 7) * 2);
}

__global__ __launch_bounds__(NTHREADS, 2) void attn_bwd_dq_ds_kernel(BwdArgs a) {
  constexpr int D = 128;
  using T = bf16;
  using G = Geo<T, D>;
  __shared__ Stage<T, D> st0;  // k: K rows (swz_b), v: the item's two dS blocks of the tile
  __shared__ Stage<T, D> st1;
  __shared__ RabHist hist;
  static_assert(sizeof(Stage<T, D>::v) == 2 * DS_BLOCK * 2, "two dS blocks per stage");

  const int tid = threadIdx.x;
  const int lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t count = ldc(a.count);
  const WorkItem it = ldc(a.items + blockIdx.x);  // in bounds for every workgroup of the grid
  if ((int64_t)blockIdx.x >= (int64_t)count) return;
  const int b = it.b, h = it.h, q_start = it.q_start, q_len = it.q_len;
  const int k_begin = it.k_begin, k_end = it.k_end;
  const int H = a.H;
  const int64_t q_off = it.off;
  const int L = it.L;
  const int n_norm = a.norm_n > 0 ? a.norm_n : L;
  const bool has_pos = a.pos_tab != nullptr, has_time = a.time_tab != nullptr;
  const int n_pos = has_pos ? a.n_pos : 1;
  const int n_time_eff = has_time ? min(a.n_time, 64) : 1;
  if (has_pos)
    for (int i = tid; i < NWAVES * BWD_MAX_NPOS; i += NTHREADS) (&hist.pos[0][0])[i] = 0.0f;
  if (has_time)
    for (int i = tid; i < NWAVES * 64; i += NTHREADS) (&hist.time[0][0])[i] = 0.0f;

  const int row_w = wave * 32 + (lane & 31);
  const bool row_ok = row_w < q_len;
  const int p_lane = q_start + min(row_w, q_len - 1);
  const int64_t tsq = a.ts[q_off + p_lane];
  const int w_first = wave * 32;
  const bool w_rows = w_first < q_len;
  const int w_last = min(w_first + 31, q_len - 1);
  const int w_lim_min = q_start + w_first, w_lim_max = q_start + w_last;
  int64_t w_ts_min = row_ok ? tsq : INT64_MAX, w_ts_max = row_ok ? tsq : INT64_MIN;
  for (int m = 32; m >= 1; m >>= 1) {
    w_ts_min = min(w_ts_min, shfl_xor64(w_ts_min, m));
    w_ts_max = max(w_ts_max, shfl_xor64(w_ts_max, m));
  }
  w_ts_min = uniform64(w_ts_min);
  w_ts_max = uniform64(w_ts_max);

  // dS blocks of this user and head; block (kt, qt) at blk0 + qt (qt + 1) / 2 + kt
  const int nbb = (int)ceil_div(L, KT);
  const int64_t blk0 = (int64_t)H * ldc(a.ds_prefix + b) + (int64_t)h * nbb * (nbb + 1) / 2;
  const int qt0 = q_start / KT;
  const int qt_w = qt0 + (wave >> 1);  // block column of this wave's rows (and of its DMA)

  // K^T operands (A) of d block db and key step ks: the offset of (0, 0) xor
  // 64 db, plus 16 rows per step; dS^T operands (B) of key step ks
  const uint32_t t_base0 = tr_off_b<D>(lane, 0, 0, 0), t_base1 = tr_off_b<D>(lane, 0, 0, 1);
  const uint32_t s_base0 = ds_tr_off(lane, wave & 1, 0) + (uint32_t)((wave >> 1) * DS_BLOCK * 2);
  const uint32_t s_base1 = ds_tr_off(lane, wave & 1, 1) + (uint32_t)((wave >> 1) * DS_BLOCK * 2);
  f32x16 dqacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) dqacc[i] = f32x16{};
  using LB = __attribute__((address_space(3))) unsigned char;
  using LT = __attribute__((address_space(3))) v4i16;
  // LDS reads through address-space-3 pointers derived from the stage: the
  // compiler then sees which stage they read and does not wait for the DMA
  // that is filling the other one
  using LH = __attribute__((address_space(3))) const bf16;
  using LI = __attribute__((address_space(3))) const int32_t;
  using LL = __attribute__((address_space(3))) const int64_t;
  using LFP = __attribute__((address_space(3))) float;
  auto tr8 = [](LB* p0, LB* p1) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LT*)p0);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LT*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  int tcls = 0;  // this lane's tile time class (time_class), filled 64 tiles at a time
  int64_t tb_mn = 0, tb_mx = 0;  // and the timestamp range (a superset) of that tile's keys
  bf16x8 ones;
  #pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (bf16)1.0f;
  // Histogram state. LDS float atomics are slow, so the sums are kept in
  // registers and reduced across the wave only rarely: pos_acc (MFMA sums of
  // the tiles entirely in bucket n_pos - 1) and pos_far (that bucket's pairs
  // in the other tiles) once per item; time_acc (MFMA sums
  // of the tiles in time bucket time_cur) folds into a per-lane window of 8
  // time buckets [wb, wb + 8), reduced when the window moves (time buckets
  // fall along an item's key tiles when timestamps grow with position).
  f32x16 pos_acc = f32x16{}, time_acc = f32x16{};
  float pos_far = 0.0f;  // per lane: its pairs at distance n_pos - 1 or more in the other tiles
  int time_cur = -1;
  float win[8];
  #pragma unroll
  for (int s = 0; s < 8; ++s) win[s] = 0.0f;
  int wb = 0;
  // The eight slot sums over the wave by recursive halving: across lane bit
  // 5, then 4, then 3, a lane keeps half of its slots and adds its partner's
  // copies of them (4 + 2 + 1 shuffles), then a plain sum over lane bits 2..0
  // (3 more), instead of eight separate six-shuffle wave sums. Lane l ends
  // with slot 4 b5 + 2 b4 + b3 of its bits; lanes 8s add slot s.
  auto flush_win = [&]() {
    const bool b5 = (lane & 32) != 0, b4 = (lane & 16) != 0, b3 = (lane & 8) != 0;
    // in place: after each level win[0 ..) holds the lane's remaining slots
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float send = b5 ? win[j] : win[j + 4], keep = b5 ? win[j + 4] : win[j];
      win[j] = keep + __shfl_xor(send, 32);
    }
    #pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float send = b4 ? win[j] : win[j + 2], keep = b4 ? win[j + 2] : win[j];
      win[j] = keep + __shfl_xor(send, 16);
    }
    float x = (b3 ? win[1] : win[0]) + __shfl_xor(b3 ? win[0] : win[1], 8);
    #pragma unroll
    for (int m = 4; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    const int slot = (b5 ? 4 : 0) + (b4 ? 2 : 0) + (b3 ? 1 : 0);
    if ((lane & 7) == 0 && wb + slot < 64) lds_add_f32_unordered(&hist.time[wave][wb + slot], x);
    #pragma unroll
    for (int j = 0; j < 8; ++j) win[j] = 0.0f;
  };
  // make buckets [lo, hi] (hi - lo < 8, wave-uniform) fit the window
  auto win_fit = [&](int lo, int hi) {
    if (lo < wb || hi >= wb + 8) {
      flush_win();
      wb = max(0, hi - 7);
    }
  };
  auto win_add = [&](int bkt, float v) {
    #pragma unroll
    for (int s = 0; s < 8; ++s) win[s] += bkt - wb == s ? v : 0.0f;
  };
  auto fold_time = [&]() {
    if (time_cur >= 0) {
      win_fit(time_cur, time_cur);
      win_add(time_cur, hl == 0 ? time_acc[0] : 0.0f);  // lanes 32..63 repeat lanes 0..31
      time_acc = f32x16{};
    }
  };
  auto compute_tile = [&](Stage<T, D>& st, int j0, int t) {
    // keys all after this wave's rows: the block is absent or all zeros
    if (!w_rows || j0 > w_lim_max) return;
    LB* kl = LDS_PTR(unsigned char, st.k);
    LB* dl = LDS_PTR(unsigned char, st.v);
    uint32_t tb0 = t_base0, tb1 = t_base1, sb0 = s_base0, sb1 = s_base1;
    asm volatile("" : "+v"(tb0), "+v"(tb1), "+v"(sb0), "+v"(sb1));
    bf16x8 dsb[4];
    #pragma unroll
    for (int ks = 0; ks < 4; ++ks) dsb[ks] = tr8(dl + sb0 + ks * 16 * KT * 2, dl + sb1 + ks * 16 * KT * 2);
    // dQ^T += K^T dS^T, the K^T operands of step ks + 1 read during the
    // MFMAs of step ks
    bf16x8 kt[2][G::NDB];
    auto read_k = [&](int ks, bf16x8* o) {
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        o[db] = tr8(kl + (tb0 ^ (uint32_t)(db << 6)) + ks * 16 * G::ROWB,
                    kl + (tb1 ^ (uint32_t)(db << 6)) + ks * 16 * G::ROWB);
    };
    read_k(0, kt[0]);
    #pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) read_k(ks + 1, kt[(ks + 1) & 1]);
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) dqacc[db] = Mfma<T>::run(kt[ks & 1][db], dsb[ks], dqacc[db]);
    }
    if (!has_pos && !has_time) return;
    // dsb[ks] for a key step held in a scalar register (selects, no dynamic
    // register indexing): element j is dS of key 16 ks + 8 hl + j and this
    // lane's query, the same bf16 value the block in LDS holds
    auto dsb_step = [&](int ks) { return ks == 0 ? dsb[0] : ks == 1 ? dsb[1] : ks == 2 ? dsb[2] : dsb[3]; };
    // Bias-table histograms. A sum over a set of pairs is an MFMA of their
    // dS^T operands against a ones operand (every row of the result holds the
    // per-query sums; lane l < 32 has query l). Tiles whose pairs all share
    // the position bucket (n_pos - 1) add into pos_acc, tiles that share one
    // time bucket into time_acc (flushed when the bucket changes); the other
    // tiles are handled below
    const bool pos_uniform = !has_pos || (w_lim_min - (j0 + KT - 1) >= n_pos - 1);
    bool time_uniform = !has_time;
    int z_tile = 63;
    bool small_span = true;
    if (has_time) tile_class(tcls, t, time_uniform, z_tile, small_span);
    if (has_pos && pos_uniform) {
      #pragma unroll
      for (int ks = 0; ks < 4; ++ks) pos_acc = Mfma<T>::run(ones, dsb[ks], pos_acc);
    }
    if (has_time && time_uniform) {
      const int tb = min(63 - z_tile, n_time_eff - 1);
      if (tb != time_cur) {
        fold_time();
        time_cur = tb;
      }
      #pragma unroll
      for (int ks = 0; ks < 4; ++ks) time_acc = Mfma<T>::run(ones, dsb[ks], time_acc);
    }
    if (pos_uniform && time_uniform) return;
    // the remaining tiles, pair by pair without branches: a masked pair or a
    // row past the user has dS = 0, so it may be added anywhere in range
    const int lim_rel = p_lane - j0 - 8 * hl;  // query position - position of tile key 8 hl
    if (has_pos && !pos_uniform) {
      // near-diagonal distances r < n_pos - 1: lane r gathers the pairs at
      // distance r along the wave's valid queries from the dS block in LDS
      // and adds them to its own bucket (no two lanes share a bucket)
      LB* blk = dl + (wave >> 1) * DS_BLOCK * 2;
      const int c0 = (wave & 1) * 32, nq = w_last - w_first + 1;
      const int r_lo = max(w_lim_min - (j0 + KT - 1), 0), r_hi = min(w_lim_max - j0, n_pos - 2);
      for (int r0 = r_lo; r0 <= r_hi; r0 += 64) {
        const int r = r0 + lane;
        if (r <= r_hi) {
          float acc = 0.0f;
          #pragma unroll 1
          for (int i0 = 0; i0 < 32; i0 += 8) {
            uint32_t ad[8], v[8];
            bool ok[8];
            #pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int i = i0 + e, k = w_lim_min + i - r - j0;  // tile key of query i at distance r
              ok[e] = i < nq && (unsigned)k < (unsigned)KT;
              const int col = c0 + i;
              ad[e] = (uint32_t)(uintptr_t)blk + (ok[e] ? ds_chunk_off(k, col >> 3) + (col & 7) * 2 : 0u);
            }
            lds_read8_u16(ad, v);
            #pragma unroll
            for (int e = 0; e < 8; ++e) acc += ok[e] ? bf16_bits_to_f32(v[e]) : 0.0f;
          }
          *(LFP*)&hist.pos[wave][r] += acc;
        }
      }
      // distances n_pos - 1 and beyond: the lane's own pairs, one key step at
      // a time (a rolled loop keeps the selects from holding many masks)
      #pragma unroll 1
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 d = dsb_step(ks);
        #pragma unroll
        for (int j = 0; j < 8; ++j) pos_far += lim_rel - 16 * ks - j >= n_pos - 1 ? (float)d[j] : 0.0f;
      }
    }
    if (!has_time || time_uniform) return;
    // Time buckets [b_lo, b_hi] of the wave tile, from the tile's key range
    // and the wave's query range. When every key precedes every query and
    // the tile spans at most 4 buckets, a pair is in bucket b_lo + i or above
    // exactly when t_key <= t_query - (2^(b_lo + i) - 1): one compare per
    // boundary, summed as nested totals and differenced at the end. Other
    // tiles (near the diagonal) add pair by pair.
    const int64_t kmin = readlane64(tb_mn, t & 63), kmax = readlane64(tb_mx, t & 63);
    int b_lo = 0, nb = 0;
    if (small_span && kmax <= w_ts_min) {
      b_lo = min(63 - __builtin_clzll((uint64_t)(w_ts_min - kmax) + 1), n_time_eff - 1);
      const int b_hi = min(63 - __builtin_clzll((uint64_t)(w_ts_max - kmin) + 1), n_time_eff - 1);
      nb = b_hi - b_lo + 1;
    }
    LI* tsl_lo = LDS_PTR(const int32_t, st.ts_lo) + 8 * hl;
    const int32_t tsq_lo = (int32_t)tsq;
    // NB boundaries (NB + 1 buckets from b_lo): per pair, the key's offset
    // from the query's timestamp against -(2^(b_lo + i + 1) - 1), exact in
    // 32 bits on a small-span tile
    auto by_threshold = [&](auto nb_tag) {
      constexpr int NB = decltype(nb_tag)::value;
      int32_t bound[NB > 0 ? NB : 1];
      #pragma unroll
      for (int i = 0; i < NB; ++i) bound[i] = -(int32_t)(((uint32_t)2 << (b_lo + i)) - 1u);
      float tot = 0.0f, ge[NB > 0 ? NB : 1] = {};
      // the pairs' dS are this lane's MFMA operands (dsb), 8 pairs at a time
      #pragma unroll 1
      for (int ks = 0; ks < 4; ++ks) {
        uint32_t at[8], vt[8];
        #pragma unroll
        for (int j = 0; j < 8; ++j) at[j] = (uint32_t)(uintptr_t)(tsl_lo + 16 * ks + j);
        lds_read8_b32(at, vt);
        const bf16x8 d = dsb_step(ks);
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float ds = (float)d[j];
          const int32_t dk = (int32_t)vt[j] - tsq_lo;
          tot += ds;
          #pragma unroll
          for (int i = 0; i < NB; ++i) ge[i] += dk <= bound[i] ? ds : 0.0f;
        }
      }
      // bucket b_lo + k holds the pairs at or above boundary k - 1 and below boundary k
      win_fit(b_lo, b_lo + NB);
      #pragma unroll
      for (int k = 0; k <= NB; ++k)
        win_add(b_lo + k, (k == 0 ? tot : ge[k > 0 ? k - 1 : 0]) - (k < NB ? ge[k < NB ? k : 0] : 0.0f));
    };
    if (nb == 1) { by_threshold(std::integral_constant<int, 0>{}); return; }
    if (nb == 2) { by_threshold(std::integral_constant<int, 1>{}); return; }
    if (nb == 3) { by_threshold(std::integral_constant<int, 2>{}); return; }
    if (nb == 4) { by_threshold(std::integral_constant<int, 3>{}); return; }
    // Pair by pair: the window is placed on the tile's highest possible
    // bucket, so no pair lies above it; pairs below it (only where keys come
    // very close in time to a query) are summed by further passes, eight
    // buckets at a time
    {
      const int64_t span = max(w_ts_max - kmin, kmax - w_ts_min);
      const int b_top = min(63 - __builtin_clzll((uint64_t)max(span, (int64_t)0) + 1), n_time_eff - 1);
      win_fit(max(0, b_top - 7), b_top);
    }
    // (a rolled loop over the lane's 32 pairs, 8 at a time, their dS taken
    // from this lane's MFMA operands: this path is rare, and unrolled
    // selects would hold too many lane masks)
    auto per_pair = [&](auto small_tag) {
      constexpr bool SMALL = decltype(small_tag)::value;
      const uint32_t t_lo = (uint32_t)(uintptr_t)LDS_PTR(const int32_t, st.ts_lo);
      const uint32_t t64 = (uint32_t)(uintptr_t)LDS_PTR(const int64_t, st.ts64);
      // pairs e0 .. e0 + 7 of the lane (keys 16 (e / 8) + 8 hl + e mod 8): dS and bucket
      auto pairs8 = [&](int e0, float (&ds)[8], int (&bkt)[8]) {
        uint32_t at[8], vt[8], vh[8];
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = 16 * (e0 >> 3) + 8 * hl + e;
          at[e] = SMALL ? t_lo + 4 * kk : t64 + 8 * kk;
        }
        lds_read8_b32(at, vt);
        const bf16x8 d = dsb_step(e0 >> 3);
        if constexpr (!SMALL) {
          #pragma unroll
          for (int e = 0; e < 8; ++e) at[e] += 4;
          lds_read8_b32(at, vh);
        }
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          ds[e] = (float)d[e];
          const int64_t tk = SMALL ? 0 : (int64_t)(((uint64_t)vh[e] << 32) | vt[e]);
          bkt[e] = min(63 - time_z<SMALL>(tsq, tk, tsq_lo, (int32_t)vt[e]), n_time_eff - 1);
        }
      };
      int b_below = 64;  // lowest bucket of this lane under the window
      #pragma unroll 1
      for (int e0 = 0; e0 < 32; e0 += 8) {
        float ds[8];
        int bkt[8];
        pairs8(e0, ds, bkt);
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          win_add(bkt[e], ds[e]);
          // masked pairs (dS exactly 0, often with a small |dt|) add nothing
          b_below = (bkt[e] < wb && ds[e] != 0.0f) ? min(b_below, bkt[e]) : b_below;
        }
      }
      for (int m = 32; m >= 1; m >>= 1) b_below = min(b_below, __shfl_xor(b_below, m));
      // buckets [b_below, wb): the window moves down to the eight buckets
      // under the last ones counted (after a flush), and a pass adds the
      // pairs below those only; wave-uniform, usually one pass at most
      int top = wb;
      while (b_below < top) {
        const int base = max(b_below, top - 8);
        flush_win();
        wb = base;
        #pragma unroll 1
        for (int e0 = 0; e0 < 32; e0 += 8) {
          float ds[8];
          int bkt[8];
          pairs8(e0, ds, bkt);
          #pragma unroll
          for (int e = 0; e < 8; ++e) win_add(bkt[e], bkt[e] < top ? ds[e] : 0.0f);
        }
        top = base;
      }
    };
    if (small_span) per_pair(std::true_type{});
    else per_pair(std::false_type{});
  };

  const int ntiles = k_end > k_begin ? (int)ceil_div(k_end - k_begin, KT) : 0;
  int64_t tsreg = 0;
  // Stage of key tile j0: K rows (as stage_rows, clamped to the user's last
  // row) and the dS blocks (kt, qt0) (waves 0, 1) and (kt, qt0 + 1) (waves
  // 2, 3), each where it exists; an absent block is never read
  auto issue = [&](Stage<T, D>& st, int j0) {
    constexpr int ND = G::TILE / (NWAVES * 1024);
    const int last = min(KT, L - j0) - 1;
    const uint32_t rstride = (uint32_t)(H * G::ROWB);
    const unsigned char* kb = (const unsigned char*)a.k + (((q_off + j0) * H + h) * D) * 2;
    #pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int base = (wave * ND + i) * 64;
      const int P = base + lane;
      const int r = P / G::CPR, pc = P % G::CPR;
      const uint32_t off = __umul24((uint32_t)min(r, last), rstride) + (uint32_t)((pc ^ swz_b<D>(r)) << 4);
      __builtin_amdgcn_global_load_lds((const void*)(kb + off), LDS_PTR(void, st.k + base * 16), 16, 0, 0);
    }
    const int kt = j0 / KT;
    const int64_t gb = blk0 + (int64_t)qt_w * (qt_w + 1) / 2 + kt;
    if (kt <= qt_w && qt_w < nbb && gb < a.ds_cap) {
      const unsigned char* src = (const unsigned char*)(a.ds + gb * DS_BLOCK);
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int base = ((wave & 1) * 4 + i) * 64;  // chunk index within the block
        const int P = base + lane;
        const int r = P >> 3, pc = P & 7;
        __builtin_amdgcn_global_load_lds((const void*)(src + ds_chunk_off(r, pc)),
                                         LDS_PTR(void, st.v + (wave >> 1) * DS_BLOCK * 2 + base * 16), 16, 0, 2);
      }
    }
    if (wave == 0) tsreg = a.ts[q_off + j0 + min(lane, last)];
  };
  if (ntiles > 0) {
    issue(st0, k_begin);
    finish_stage<D>(st0, tsreg);
  } else {
    __syncthreads();
  }
  // time classes of the next 64 tiles, lane i for tile t0 + i
  auto time_batch = [&](int t0) {
    const int tl = t0 + lane;
    int c = 255;
    if (tl < ntiles) {
      row_time_range(a, q_off + k_begin + tl * KT, tb_mn, tb_mx);
      c = time_class(tb_mn, tb_mx, w_ts_min, w_ts_max, n_time_eff);
    }
    tcls = c;
  };
  for (int t = 0; t < ntiles; t += 2) {
    if (has_time && (t & 63) == 0) time_batch(t);
    const int j0 = k_begin + t * KT;
    if (t + 1 < ntiles) issue(st1, j0 + KT);
    compute_tile(st0, j0, t);
    if (t + 1 >= ntiles) break;
    finish_stage<D>(st1, tsreg);
    if (t + 2 < ntiles) issue(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT, t + 1);
    if (t + 2 < ntiles) finish_stage<D>(st0, tsreg);
  }

  if (w_rows) {
    if (has_time) {
      fold_time();
      flush_win();
    }
    if (has_pos) {
      const float x = wave_sum_f((hl == 0 ? pos_acc[0] : 0.0f) + pos_far);
      if (lane == 0) lds_add_f32_unordered(&hist.pos[wave][n_pos - 1], x);
    }
  }
  store_rows_t<D>(dqacc, a.alpha / (float)n_norm, st0, st1, a.dq, q_off + q_start, q_len, h, H);

  // per-item bias gradients (scaled by 1 / N) in the slot of the item's
  // canonical index, as the four-wave kernel writes them
  const int64_t tiles = ldc(a.prefix + a.B) / H;
  const int64_t canon = (int64_t)h * tiles + ldc(a.prefix + b) / H + q_start / QT;
  float* part = a.rab_part + canon * RAB_SLOTS;
  const float inv_n = 1.0f / (float)n_norm;
  if (has_pos) {
    for (int i = tid; i < n_pos; i += NTHREADS) {
      float x = 0.0f;
      #pragma unroll
      for (int w = 0; w < NWAVES; ++w) x += hist.pos[w][i];
      part[i] = x * inv_n;
    }
  }
  if (has_time && tid < 64) {
    float x = 0.0f;
    #pragma unroll
    for (int w = 0; w < NWAVES; ++w) x += hist.time[w][tid];
    part[BWD_MAX_NPOS + tid] = x * inv_n;
  }
}

// ============================================================================
// Bias-table gradients: add the per-item histograms in canonical order
// ============================================================================
// Block (x, y): 64 buckets of table row y (a head, or the one shared row;
// position rows first, then time rows). 16 groups of 64 threads split the
// row's items (group g takes items g, g + 16, ...); one thread then adds the
// 16 group sums in order, so the result does not depend on timing.
constexpr int RAB_GROUPS = 16;
__global__ __launch_bounds__(64 * RAB_GROUPS) void rab_reduce_kernel(RabReduceArgs a) {
  __shared__ float acc[RAB_GROUPS][64];
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int pos_rows = a.d_pos ? (a.pos_stride > 0 ? a.H : 1) : 0;
  const int y = blockIdx.y;
  const bool is_pos = y < pos_rows;
  const int row = is_pos ? y : y - pos_rows;
  const int n = is_pos ? a.n_pos : a.n_time;
  const int c = blockIdx.x * 64 + cl;
  const bool shared = is_pos ? a.pos_stride == 0 : a.time_stride == 0;
  const int64_t tiles = a.B > 0 ? a.prefix[a.B] / a.H : 0;
  const int64_t lo = shared ? 0 : (int64_t)row * tiles, hi = shared ? (int64_t)a.H * tiles : lo + tiles;
  float sum = 0.0f;
  if (c < n && (is_pos || c < 64)) {
    const int slot = is_pos ? c : BWD_MAX_NPOS + c;
    // 16 items' loads in flight before their adds; the adds keep item order
    constexpr int U = 16;
    int64_t i = lo + grp;
    for (; i + (U - 1) * RAB_GROUPS < hi; i += U * RAB_GROUPS) {
      float x[U];
      #pragma unroll
      for (int j = 0; j < U; ++j) x[j] = a.part[(i + j * RAB_GROUPS) * RAB_SLOTS + slot];
      #pragma unroll
      for (int j = 0; j < U; ++j) sum += x[j];
    }
    for (; i < hi; i += RAB_GROUPS) sum += a.part[i * RAB_SLOTS + slot];
  }
  acc[grp][cl] = sum;
  __syncthreads();
  if (grp == 0 && c < n) {
    float t = 0.0f;
    for (int g = 0; g < RAB_GROUPS; ++g) t += acc[g][cl];
    if (is_pos) a.d_pos[(int64_t)row * a.pos_stride + c] = t;
    else a.d_time[(int64_t)row * a.time_stride + c] = t;
  }
}

hipError_t launch_attn_bwd(const BwdArgs& a, int D, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), blk(NTHREADS);
  if (D == 128) {
    // dK and dV first: that kernel writes the dS blocks the dQ kernel reads
    if (!a.ds || !a.ds_prefix) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_bwd_dkdv8_kernel, g, dim3(DKDV8_THREADS), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dq_ds_kernel, g, blk, 0, s, a);
  } else if (D == 64) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, g, blk, 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, g, blk, 0, s, a);
  } else if (D == 32) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<32>, g, blk, 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<32>, g, blk, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rab_reduce(const RabReduceArgs& a, hipStream_t s) {
  const int pos_rows = a.d_pos ? (a.pos_stride > 0 ? a.H : 1) : 0;
  const int time_rows = a.d_time ? (a.time_stride > 0 ? a.H : 1) : 0;
  if (pos_rows + time_rows == 0) return hipSuccess;
  const int n = max(pos_rows ? a.n_pos : 0, time_rows ? a.n_time : 0);
  hipLaunchKernelGGL(rab_reduce_kernel, dim3((unsigned)ceil_div(n, 64), (unsigned)(pos_rows + time_rows)),
                     dim3(64 * RAB_GROUPS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
