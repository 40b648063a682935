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
//   * attn_bwd_dq_kernel owns 128 query rows (one work item of the forward
//     scheduler) and walks their key tiles like the forward: S^T = K Q^T and
//     dP^T = V dO^T on MFMA (K and V rows from LDS, Q and dO in registers),
//     dS^T elementwise, dQ^T += K^T dS^T (K^T by transposing LDS reads). It
//     also sums dS into per-wave position/time histograms in LDS.
//   * attn_bwd_dkdv_kernel owns 128 keys and walks the query tiles that can
//     see them: S = Q K^T and dP = dO V^T (Q and dO rows from LDS, K and V in
//     registers), then dV^T += dO^T P and dK^T += Q^T dS. The item of query
//     tile t of a user maps to key block (tiles - 1 - t), whose cost matches.
// A third kernel adds the per-item histograms in canonical item order.
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

// One histogram per wave (no two waves add to the same word, so every sum
// runs in program order and the result does not depend on wave timing).
struct RabHist {
  float pos[NWAVES][BWD_MAX_NPOS];  // sum of dS' per position bucket
  float time[NWAVES][64];           // per time bucket
};

__device__ inline void load_bwd_tables(const BwdArgs& a, int h, BwdTables& tab, int n_pos) {
  const int tid = threadIdx.x;
  const float* pt = a.pos_tab ? a.pos_tab + (int64_t)h * a.pos_stride : nullptr;
  for (int i = tid; i < n_pos; i += NTHREADS) tab.pos_t[i] = pt ? pt[i] * -LOG2E : 0.0f;
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

// y -> (P', dS') for one score: P' = y * sigma, dS' = dp * sigma * (1 + x (1 - sigma)), x = -ln2 y
__device__ inline void silu_fwd_bwd(float y, float dp, float& p, float& ds) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
  p = y * sg;
  const float x = -LN2 * y;
  ds = dp * sg * fmaf(x, 1.0f - sg, 1.0f);
}

// Stage HBM -> LDS of KT rows of two [T, H, D] tensors (rows r0 .. r0 + KT - 1
// of head h, clamped to the last valid row) plus their timestamps.
template <int D>
__device__ inline void stage_rows(const BwdArgs& a, const void* x0, const void* x1, Stage<bf16, D>& st, int64_t r0,
                                  int nvalid, int h, int64_t& tsreg) {
  using G = Geo<bf16, D>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int last = max(nvalid - 1, 0);
  const int64_t rstride = (int64_t)a.H * G::ROWB;
  const unsigned char* b0 = (const unsigned char*)x0 + ((r0 * a.H + h) * D) * 2;
  const unsigned char* b1 = (const unsigned char*)x1 + ((r0 * a.H + h) * D) * 2;
  #pragma unroll
  for (int i = 0; i < G::NDMA; ++i) {
    const int base = (wave * G::NDMA + i) * 64;
    const int P = base + lane;
    const int r = P / G::CPR, pc = P % G::CPR;
    const int64_t off = min(r, last) * rstride + ((pc ^ swz_b<D>(r)) << 4);
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
  if ((int64_t)blockIdx.x >= (int64_t)ldc(a.count)) return;
  const WorkItem it = ldc(a.items + blockIdx.x);
  const int b = it.b, h = it.h, q_start = it.q_start, q_len = it.q_len;
  const int k_begin = it.k_begin, k_end = it.k_end;
  const int H = a.H;
  const int64_t q_off = ldc(a.offsets + b);
  const int L = ldc(a.offsets + b + 1) - (int)q_off;
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
  uint32_t koff[G::NQOP], ktr[G::NDB][2];
  {
    const int kr = M::krow(0, l32);
    #pragma unroll
    for (int s = 0; s < G::NQOP; ++s) koff[s] = (uint32_t)b_off<D>(kr, 2 * s + hl);
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      ktr[db][0] = tr_off_b<D>(lane, db, 0, 0);
      ktr[db][1] = tr_off_b<D>(lane, db, 0, 1);
    }
  }
  f32x16 dqacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) dqacc[i] = f32x16{};
  const float sc = a.alpha * -LOG2E;
  const bool has_time = a.time_tab != nullptr;
  const int n_time_eff = has_time ? min(a.n_time, 64) : 1;
  using LB = __attribute__((address_space(3))) unsigned char;

  auto key_time_range = [&](int j0, int64_t& kmin, int64_t& kmax) {
    const int64_t r0 = q_off + j0;
    const int64_t i0 = min(r0 / KT, a.n_stat_blocks - 1), i1 = min((r0 + KT - 1) / KT, a.n_stat_blocks - 1);
    kmin = min(ldc(a.tstats + 2 * i0), ldc(a.tstats + 2 * i1));
    kmax = max(ldc(a.tstats + 2 * i0 + 1), ldc(a.tstats + 2 * i1 + 1));
    if (kmin > kmax) kmin = kmax = w_ts_min;
  };

  auto compute_tile = [&](Stage<T, D>& st, int j0) {
    if (!w_rows || j0 > w_lim_max) return;
    const bool need_mask = j0 + KT - 1 > w_lim_min;
    // one bias constant for the whole wave tile?
    const bool pos_uniform = (a.pos_tab == nullptr) || (w_lim_min - (j0 + KT - 1) >= n_pos - 1);
    bool time_uniform = !has_time;
    int z_tile = 63;
    bool small_span = true;
    if (has_time) {
      int64_t k_min, k_max;
      key_time_range(j0, k_min, k_max);
      const int64_t d1 = w_ts_max - k_min, d2 = k_max - w_ts_min;
      small_span = max(d1 < 0 ? -d1 : d1, d2 < 0 ? -d2 : d2) < ((int64_t)1 << 31) - 2;
      int64_t lo = -1, hi = -1;
      if (w_ts_min >= k_max) { lo = w_ts_min - k_max; hi = w_ts_max - k_min; }
      else if (k_min >= w_ts_max) { lo = k_min - w_ts_max; hi = k_max - w_ts_min; }
      if (lo >= 0) {
        const int zlo = __builtin_clzll((uint64_t)lo + 1), zhi = __builtin_clzll((uint64_t)hi + 1);
        if (min(63 - zlo, n_time_eff - 1) == min(63 - zhi, n_time_eff - 1)) { time_uniform = true; z_tile = zlo; }
      }
    }
    const bool fast = pos_uniform && time_uniform && !need_mask;
    const float c_uni = (a.pos_tab ? tab.pos_t[n_pos - 1] : 0.0f) + (has_time ? tab.time_t[z_tile] : 0.0f);
    const int lim_rel = p_lane - j0 - M::HLK * hl;  // key_of(kb, v, 0) <= lim_rel: allowed
    const int64_t* ts_l = st.ts64 + M::HLK * hl;
    const int32_t* tsl_lo = st.ts_lo + M::HLK * hl;
    const int32_t tsq_lo = (int32_t)tsq;
    LB* kl = LDS_PTR(unsigned char, st.k);
    LB* vl = LDS_PTR(unsigned char, st.v);
    float tile_sum = 0.0f;
    // General path: a lane's keys come in increasing order along v, so with
    // ordered timestamps its time bucket (and a clamped position bucket)
    // stays the same over runs of keys. dS' is summed per run and added to
    // the wave's histogram when the bucket changes, not once per pair.
    int cur_p = -1, cur_t = -1;
    float run_p = 0.0f, run_t = 0.0f;
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      #pragma unroll
      for (int i = 0; i < G::NQOP; ++i) {
        const bf16x8 kop = *(__attribute__((address_space(3))) const bf16x8*)(kl + koff[i] + kb * 32 * G::ROWB);
        s = M::run(kop, qop[i], s);
      }
      #pragma unroll
      for (int i = 0; i < G::NQOP; ++i) {
        const bf16x8 vop = *(__attribute__((address_space(3))) const bf16x8*)(vl + koff[i] + kb * 32 * G::ROWB);
        dp = M::run(vop, dop[i], dp);
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
      // dQ^T += K^T dS^T for the 32 keys of block kb
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        #pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int o = (2 * kb + cc) * 16 * G::ROWB;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(kl + ktr[db][0] + o));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(kl + ktr[db][1] + o));
          const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          dqacc[db] = M::run(kt, dsb[cc], dqacc[db]);
        }
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
  for (int t = 0; t < ntiles; t += 2) {
    const int j0 = k_begin + t * KT;
    if (t + 1 < ntiles) issue(st1, j0 + KT);
    compute_tile(st0, j0);
    if (t + 1 >= ntiles) break;
    finish_stage<D>(st1, tsreg);
    if (t + 2 < ntiles) issue(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT);
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
  if ((int64_t)blockIdx.x >= (int64_t)ldc(a.count)) return;
  const WorkItem it = ldc(a.items + blockIdx.x);
  const int b = it.b, h = it.h;
  const int H = a.H;
  const int64_t q_off = ldc(a.offsets + b);
  const int L = ldc(a.offsets + b + 1) - (int)q_off;
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

  auto compute_tile = [&](Stage<T, D>& st, int j0) {
    // every query of the tile precedes every key of this wave: all masked
    if (!w_keys || j0 + KT - 1 < w_kmin) return;
    // one bias constant and no mask for the whole wave tile? (as in the forward)
    const bool need_mask = !w_full || j0 < w_kmax || j0 + KT > L;
    const bool pos_uniform = (a.pos_tab == nullptr) || (j0 - w_kmax >= n_pos - 1);
    bool time_uniform = !has_time;
    int z_tile = 63;
    bool small_span = true;
    if (has_time) {
      const int64_t r0 = q_off + j0;
      const int64_t i0 = min(r0 / KT, a.n_stat_blocks - 1), i1 = min((r0 + KT - 1) / KT, a.n_stat_blocks - 1);
      int64_t q_min = min(ldc(a.tstats + 2 * i0), ldc(a.tstats + 2 * i1));
      int64_t q_max = max(ldc(a.tstats + 2 * i0 + 1), ldc(a.tstats + 2 * i1 + 1));
      if (q_min > q_max) q_min = q_max = w_ts_min;
      // rows past the user's end (last tile) are clamped copies of its last row
      const int64_t d1 = q_max - w_ts_min, d2 = w_ts_max - q_min;
      small_span = max(d1 < 0 ? -d1 : d1, d2 < 0 ? -d2 : d2) < ((int64_t)1 << 31) - 2;
      int64_t lo = -1, hi = -1;
      if (q_min >= w_ts_max) { lo = q_min - w_ts_max; hi = q_max - w_ts_min; }
      else if (w_ts_min >= q_max) { lo = w_ts_min - q_max; hi = w_ts_max - q_min; }
      if (lo >= 0 && !need_mask && pos_uniform) {
        const int zlo = __builtin_clzll((uint64_t)lo + 1), zhi = __builtin_clzll((uint64_t)hi + 1);
        if (min(63 - zlo, n_time_eff - 1) == min(63 - zhi, n_time_eff - 1)) { time_uniform = true; z_tile = zlo; }
      }
    }
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
  for (int t = 0; t < ntiles; t += 2) {
    const int j0 = k0 + t * KT;
    if (t + 1 < ntiles) issue(st1, j0 + KT);
    compute_tile(st0, j0);
    if (t + 1 >= ntiles) break;
    finish_stage<D>(st1, tsreg);
    if (t + 2 < ntiles) issue(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT);
    if (t + 2 < ntiles) finish_stage<D>(st0, tsreg);
  }
  store_rows_t<D>(dvacc, -LN2 / (float)n_norm, st0, st1, a.dv, q_off + k0, klen, h, H);
  store_rows_t<D>(dkacc, a.alpha / (float)n_norm, st0, st1, a.dk, q_off + k0, klen, h, H);
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
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, g, blk, 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, g, blk, 0, s, a);
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
