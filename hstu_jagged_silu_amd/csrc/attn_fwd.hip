// Fused HSTU SiLU attention for gfx950: S^T = K Q^T on MFMA, relative bias,
// SiLU, mask, O^T += V^T P^T on MFMA, for one (user, head, 128-row query tile,
// key range) work item per workgroup.
//
// The operation (pointwise SiLU weighting in place of softmax, plus a relative
// position/time bias, over causal jagged sequences) follows "Generative
// recommenders at scale", section "Inside NVIDIA's GPU-native stack for HSTU
// and Semantic IDs", and "How Generative Recommenders Are Redefining RecSys at
// Scale", Takeaways. The cached-prefix and M-FALCON masks follow "Deploying an
// HSTU Generative Recommender with NVIDIA Dynamo-Triton", section "Technical
// Stack and Performance Gains", and "HSTU Generative Recommenders: Deploy on
// GPU Cloud", section "M-FALCON: Microbatched Attention ...".
//
// Data flow inside one wave (32 query rows, one 64-key tile):
//   * The score tile is computed transposed, S^T[key][q] = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (fp32: v_mfma_f32_32x32x2_f32). The 32x32
//     accumulator puts query q = lane % 32 in every register of a lane, and
//     keys along the registers.
//   * K rows are fed to the MFMA in a permuted order so that, after SiLU, the
//     8 consecutive accumulator registers of a lane hold 8 consecutive keys:
//     they are exactly the B operand (P^T) of the second product
//     O^T[d][q] += V^T[d][key] P^T[key][q]. No shuffle or LDS round trip sits
//     between the two products.
//   * V is stored transposed in LDS (V^T[d][key]) while it is staged, so the
//     A operand of the second product is one 16-byte LDS read.
//   * The bias is folded into one FMA per score: y = s * (-alpha log2 e) + b'
//     with b' = -log2(e) (P[.] + T[.]); then SiLU(x) = -ln2 * y / (1 + 2^y),
//     and the -ln2 / N factor moves to the epilogue. Far from the diagonal a
//     wave tile's bias is usually one constant (position clamped, one time
//     bucket); the per-element bucket path only runs where it varies.
#include "kernels.h"

namespace hstu {

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KS = 16;  // reduction depth of one instruction
  using op = bf16x8;
  __device__ static inline f32x16 run(op a, op b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // key (0..63 within the tile) held by accumulator register v of key block kb
  __device__ static constexpr int key_of(int kb, int v, int hl) { return kb * 32 + 16 * (v >> 3) + 8 * hl + (v & 7); }
  // physical key fed to MFMA row r of key block kb (see key_of)
  __device__ static inline int krow(int kb, int r) {
    int r16 = r & 15;
    int pr = (r16 < 4 || r16 >= 12) ? r16 : (r16 < 8 ? r16 + 4 : r16 - 4);
    return kb * 32 + (r & 16) + pr;
  }
};

template <> struct Mfma<float> {
  static constexpr int KS = 2;
  using op = float;
  __device__ static inline f32x16 run(op a, op b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static constexpr int key_of(int kb, int v, int hl) { return kb * 32 + 8 * (v >> 2) + 4 * hl + (v & 3); }
  __device__ static inline int krow(int kb, int r) { return kb * 32 + r; }
};

// LDS geometry of one key tile for element type T and head dim D.
template <typename T, int D> struct Geo {
  static constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int KCPR = D / EPC;                  // chunks per K row (one key)
  static constexpr int VCPR = KT / EPC;                 // chunks per V^T row (one d)
  static constexpr int KPT = KCPR * KT / NTHREADS;      // keys staged per thread
  static constexpr int TILE = KT * D * (int)sizeof(T);  // bytes of one K (or V) tile
  static constexpr int NDB = D / 32;                    // 32-wide d blocks of O
  static constexpr int NQOP = D / Mfma<T>::KS;          // Q operands per lane
  static_assert(KPT >= 1 && KCPR * (KT / KPT) == NTHREADS, "staging map");
  // XOR swizzles on 16-byte chunks keep the MFMA operand reads conflict-free
  __device__ static inline int k_off(int r, int c) { return (r * KCPR + (c ^ (r % KCPR))) * 16; }
  __device__ static inline int v_off(int d, int c) { return (d * VCPR + (c ^ ((d ^ (d / VCPR)) % VCPR))) * 16; }
};

template <typename T, int D> struct Smem {
  unsigned char kv[2][2][Geo<T, D>::TILE] __attribute__((aligned(16)));  // [buffer][K, V^T]
  int32_t ts_lo[2][KT];
  int64_t ts64[2][KT];
  int64_t ts_mm[2][2];
  float pos_t[MAX_NPOS];   // -log2(e) * position table
  float time_t[64];        // -log2(e) * time table, indexed by clz64(|dt| + 1)
};

__device__ inline int64_t shfl_xor64(int64_t x, int m) {
  return (int64_t)__shfl_xor((long long)x, m);
}

template <int NB> __device__ inline void store_bytes(unsigned char* p, const unsigned char* src) {
  if constexpr (NB == 16) *(i32x4*)p = *(const i32x4*)src;
  else if constexpr (NB == 8) *(uint64_t*)p = *(const uint64_t*)src;
  else if constexpr (NB == 4) *(uint32_t*)p = *(const uint32_t*)src;
  else *(uint16_t*)p = *(const uint16_t*)src;
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(NTHREADS, (sizeof(T) == 4 && D == 128) ? 1 : 2)  // fp32 d=128: LDS allows one
void attn_fwd_kernel(AttnArgs a) {
  using G = Geo<T, D>;
  using M = Mfma<T>;
  __shared__ Smem<T, D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  if ((int64_t)blockIdx.x >= (int64_t)*a.count) return;
  const WorkItem it = a.items[blockIdx.x];
  const int b = it.b, h = it.h, kind = it.kind;
  const int q_start = it.q_start, q_len = it.q_len;
  const int k_begin = it.k_begin, k_end = it.k_end;
  const int H = a.H;

  // ---- per-user geometry -------------------------------------------------
  const int64_t q_off = a.offsets[b];
  const int Lq = a.offsets[b + 1] - (int)q_off;
  int kcount, pos0, n_norm;
  bool cand = false;
  if (MODE == MODE_CACHED) {
    const int C = a.cache_lens[b];
    kcount = C + Lq;
    pos0 = C + q_start;
    n_norm = C + Lq;
  } else if (MODE == MODE_MFALCON) {
    const int n = Lq - a.num_cand[b];
    kcount = n;
    cand = (kind == KIND_CANDIDATE);
    pos0 = cand ? n : q_start;
    n_norm = n + 1;
  } else {
    kcount = Lq;
    pos0 = q_start;
    n_norm = Lq;
  }
  if (a.norm_n > 0) n_norm = a.norm_n;

  // ---- bias tables, pre-scaled by -log2(e) --------------------------------
  const int n_pos = a.pos_tab ? a.n_pos : 1;
  {
    const float* pt = a.pos_tab ? a.pos_tab + (int64_t)h * a.pos_stride : nullptr;
    for (int i = tid; i < n_pos; i += NTHREADS) sm.pos_t[i] = pt ? pt[i] * -LOG2E : 0.0f;
    if (tid < 64) {
      float t = 0.0f;
      if (a.time_tab) {
        int bk = min(63 - tid, a.n_time - 1);
        t = a.time_tab[(int64_t)h * a.time_stride + bk] * -LOG2E;
      }
      sm.time_t[tid] = t;
    }
  }

  // ---- this lane's query row ------------------------------------------------
  const int row_w = wave * 32 + l32;               // row within the tile
  const bool row_ok = row_w < q_len;
  const int row_c = min(row_w, q_len - 1);         // clamped for loads
  const int64_t qrow = min(q_off + q_start + row_c, a.Tq - 1);  // packed query row
  const int p_lane = cand ? pos0 : pos0 + row_c;   // position of the query
  const int lim_lane = cand ? pos0 - 1 : p_lane;   // largest key it may see
  const int64_t tsq = a.ts[qrow];

  // wave-level (uniform) row facts
  const int w_first = wave * 32;
  const bool w_rows = w_first < q_len;
  const int w_last = min(w_first + 31, q_len - 1);
  const int w_lim_min = cand ? pos0 - 1 : pos0 + w_first;
  const int w_lim_max = cand ? pos0 - 1 : pos0 + w_last;
  const int w_p_min = cand ? pos0 : pos0 + w_first;
  int64_t w_ts_min = row_ok ? tsq : INT64_MAX, w_ts_max = row_ok ? tsq : INT64_MIN;
  for (int m = 32; m >= 1; m >>= 1) {
    w_ts_min = min(w_ts_min, shfl_xor64(w_ts_min, m));
    w_ts_max = max(w_ts_max, shfl_xor64(w_ts_max, m));
  }

  // ---- Q operands in registers ---------------------------------------------
  typename M::op qop[G::NQOP];
  {
    const T* qp = (const T*)a.q + (qrow * H + h) * D;
    #pragma unroll
    for (int s = 0; s < G::NQOP; ++s) {
      if constexpr (sizeof(T) == 2) {
        bf16x8 x = *(const bf16x8*)(qp + 16 * s + 8 * hl);
        if (!row_ok) x = bf16x8{};
        qop[s] = x;
      } else {
        float x = qp[2 * s + hl];
        qop[s] = row_ok ? x : 0.0f;
      }
    }
  }

  // ---- key tile staging -----------------------------------------------------
  const int dchunk = tid % G::KCPR, kgroup = tid / G::KCPR;
  i32x4 kreg[G::KPT], vreg[G::KPT];
  int64_t tsreg = 0;

  auto load_tile = [&](int j0) {
    const T* kbase = nullptr;
    const T* vbase = nullptr;
    int64_t rstride = 0;
    const int64_t* tsbase = nullptr;
    int64_t kmax_rows = KT;   // rows readable from kbase
    if (MODE == MODE_CACHED) {
      const int page = j0 / PAGE < a.max_pages ? a.page_table[(int64_t)b * a.max_pages + j0 / PAGE] : -1;
      if (page >= 0 && page < a.num_pages) {
        const int64_t pb = ((int64_t)page * H + h) * PAGE * D;
        kbase = (const T*)a.k_pages + pb;
        vbase = (const T*)a.v_pages + pb;
        rstride = D;
        tsbase = a.ts_pages + (int64_t)page * PAGE;
      }
    } else {
      if (q_off + j0 < a.Tq) {
        kbase = (const T*)a.k + ((q_off + j0) * H + h) * D;
        vbase = (const T*)a.v + ((q_off + j0) * H + h) * D;
        rstride = (int64_t)H * D;
        tsbase = a.ts + q_off + j0;
        kmax_rows = a.Tq - (q_off + j0);
      }
    }
    #pragma unroll
    for (int i = 0; i < G::KPT; ++i) {
      const int kl = kgroup * G::KPT + i;
      if (kbase && j0 + kl < kcount && kl < kmax_rows) {
        kreg[i] = *(const i32x4*)(kbase + kl * rstride + dchunk * G::EPC);
        vreg[i] = *(const i32x4*)(vbase + kl * rstride + dchunk * G::EPC);
      } else {
        kreg[i] = i32x4{};
        vreg[i] = i32x4{};
      }
    }
    if (wave == 0) {
      const bool ok = tsbase && j0 + lane < kcount && lane < kmax_rows;
      tsreg = ok ? tsbase[lane] : 0;
    }
  };

  auto store_tile = [&](int buf, int j0) {
    unsigned char* kl = sm.kv[buf][0];
    unsigned char* vl = sm.kv[buf][1];
    #pragma unroll
    for (int i = 0; i < G::KPT; ++i) *(i32x4*)(kl + G::k_off(kgroup * G::KPT + i, dchunk)) = kreg[i];
    // transpose: V^T[d][keys kgroup*KPT ...] for every d of this thread's chunk
    constexpr int PIECE = G::KPT < G::EPC ? G::KPT : G::EPC;  // keys per LDS store
    #pragma unroll
    for (int e = 0; e < G::EPC; ++e) {
      const int d = dchunk * G::EPC + e;
      #pragma unroll
      for (int i0 = 0; i0 < G::KPT; i0 += PIECE) {
        T vals[PIECE];
        #pragma unroll
        for (int i = 0; i < PIECE; ++i) vals[i] = ((const T*)&vreg[i0 + i])[e];
        const int key = kgroup * G::KPT + i0;
        store_bytes<PIECE * (int)sizeof(T)>(vl + G::v_off(d, key / G::EPC) + (key % G::EPC) * sizeof(T),
                                            (const unsigned char*)vals);
      }
    }
    if (wave == 0) {
      const bool ok = j0 + lane < kcount;
      sm.ts_lo[buf][lane] = (int32_t)tsreg;
      sm.ts64[buf][lane] = tsreg;
      int64_t mn = ok ? tsreg : INT64_MAX, mx = ok ? tsreg : INT64_MIN;
      for (int m = 32; m >= 1; m >>= 1) {
        mn = min(mn, shfl_xor64(mn, m));
        mx = max(mx, shfl_xor64(mx, m));
      }
      if (lane == 0) {
        sm.ts_mm[buf][0] = mn;
        sm.ts_mm[buf][1] = mx;
      }
    }
  };

  // ---- accumulators -------------------------------------------------------
  f32x16 oacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) oacc[i] = f32x16{};

  const float sc = a.alpha * -LOG2E;
  const bool has_time = a.time_tab != nullptr;
  const int n_time_eff = a.time_tab ? min(a.n_time, 64) : 1;

  auto compute_tile = [&](int buf, int j0) {
    if (!w_rows || j0 > w_lim_max) return;  // every pair of this wave masked
    const unsigned char* kl = sm.kv[buf][0];
    const unsigned char* vl = sm.kv[buf][1];

    // classify the wave tile: mask, constant bias, or per-element bias
    const bool need_mask = j0 + KT - 1 > w_lim_min;
    const int64_t k_min = sm.ts_mm[buf][0], k_max = sm.ts_mm[buf][1];
    const bool pos_uniform = (a.pos_tab == nullptr) || (w_p_min - (j0 + KT - 1) >= n_pos - 1);
    bool time_uniform = !has_time;
    float c_time = 0.0f;
    int64_t span_hi = 0;
    if (has_time) {
      int64_t lo, hi;
      bool ordered = true;
      if (w_ts_min >= k_max) { lo = w_ts_min - k_max; hi = w_ts_max - k_min; }
      else if (k_min >= w_ts_max) { lo = k_min - w_ts_max; hi = k_max - w_ts_min; }
      else { ordered = false; lo = 0; hi = max(w_ts_max - k_min, k_max - w_ts_min); }
      span_hi = hi;
      if (ordered) {
        const int zlo = __builtin_clzll((uint64_t)lo + 1), zhi = __builtin_clzll((uint64_t)hi + 1);
        const int blo = min(63 - zlo, n_time_eff - 1), bhi = min(63 - zhi, n_time_eff - 1);
        if (blo == bhi) { time_uniform = true; c_time = sm.time_t[zlo]; }
      }
    }
    const bool uniform = pos_uniform && time_uniform;
    const float cb_uniform = sm.pos_t[n_pos - 1] * (a.pos_tab ? 1.0f : 0.0f) + c_time;
    const bool small_span = span_hi < ((int64_t)1 << 31) - 2;
    const int32_t tsq_lo = (int32_t)tsq;
    const int lim_rel = lim_lane - j0;

    // one 32-key block at a time: S^T = K Q^T, SiLU, O^T += V^T P^T
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc = f32x16{};
      #pragma unroll
      for (int s = 0; s < G::NQOP; ++s) {
        typename M::op kop;
        if constexpr (sizeof(T) == 2) {
          kop = *(const bf16x8*)(kl + G::k_off(M::krow(kb, l32), 2 * s + hl));
        } else {
          const int d = 2 * s + hl;
          kop = *(const float*)(kl + G::k_off(M::krow(kb, l32), d / 4) + (d % 4) * 4);
        }
        acc = M::run(kop, qop[s], acc);
      }

      float p[16];
      if (uniform) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float y = fmaf(acc[v], sc, cb_uniform);
          const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
          p[v] = y * r;
        }
      } else {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kl_idx = M::key_of(kb, v, hl);
          const unsigned rel = (unsigned)(p_lane - (j0 + kl_idx));
          float cb = sm.pos_t[min(rel, (unsigned)(n_pos - 1))];
          if (has_time) {
            int z;
            if (small_span) {
              const int32_t dt = tsq_lo - sm.ts_lo[buf][kl_idx];
              const uint32_t x = (uint32_t)(dt < 0 ? -dt : dt) + 1u;
              z = __builtin_clz(x) + 32;
            } else {
              const int64_t dt = tsq - sm.ts64[buf][kl_idx];
              const uint64_t x = (uint64_t)(dt < 0 ? -dt : dt) + 1u;
              z = __builtin_clzll(x);
            }
            cb += sm.time_t[z];
          }
          const float y = fmaf(acc[v], sc, cb);
          const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
          p[v] = y * r;
        }
      }
      if (need_mask) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = (M::key_of(kb, v, hl) <= lim_rel) ? p[v] : 0.0f;
      }

      if constexpr (sizeof(T) == 2) {
        bf16x8 pb[2];
        #pragma unroll
        for (int c = 0; c < 2; ++c) {
          #pragma unroll
          for (int e = 0; e < 8; ++e) pb[c][e] = (bf16)p[8 * c + e];
        }
        #pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          #pragma unroll
          for (int c = 0; c < 2; ++c) {
            const bf16x8 vop = *(const bf16x8*)(vl + G::v_off(32 * db + l32, 2 * (2 * kb + c) + hl));
            oacc[db] = M::run(vop, pb[c], oacc[db]);
          }
        }
      } else {
        #pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = M::key_of(kb, v, hl);
            const float vop = *(const float*)(vl + G::v_off(32 * db + l32, key / 4) + (key % 4) * 4);
            oacc[db] = M::run(vop, p[v], oacc[db]);
          }
        }
      }
    }
  };

  // ---- main loop over key tiles (double-buffered LDS, one barrier per tile)
  const int ntiles = k_end > k_begin ? (int)ceil_div(k_end - k_begin, KT) : 0;
  if (ntiles > 0) {
    load_tile(k_begin);
    store_tile(0, k_begin);
    if (ntiles > 1) load_tile(k_begin + KT);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = k_begin + t * KT;
    compute_tile(t & 1, j0);
    if (t + 1 < ntiles) {
      store_tile((t + 1) & 1, j0 + KT);
      if (t + 2 < ntiles) load_tile(j0 + 2 * KT);
    }
    __syncthreads();
  }

  // ---- M-FALCON: a candidate's own key (relative position 0, dt = 0) -------
  if (MODE == MODE_MFALCON && cand) {
    const T* kp = (const T*)a.k + (qrow * H + h) * D;
    const T* vp = (const T*)a.v + (qrow * H + h) * D;
    float dot = 0.0f;
    #pragma unroll
    for (int s = 0; s < G::NQOP; ++s) {
      if constexpr (sizeof(T) == 2) {
        const bf16x8 kx = *(const bf16x8*)(kp + 16 * s + 8 * hl);
        #pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf((float)qop[s][e], (float)kx[e], dot);
      } else {
        dot = fmaf(qop[s], kp[2 * s + hl], dot);
      }
    }
    dot += __shfl_xor(dot, 32);
    const float y = fmaf(dot, sc, sm.pos_t[0] + sm.time_t[63]);
    const float pself = y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int d = 32 * db + 8 * (v >> 2) + 4 * hl + (v & 3);
        oacc[db][v] = fmaf(pself, (float)vp[d], oacc[db][v]);
      }
    }
  }

  // ---- epilogue: scale by -ln2 / N, stage through LDS, coalesced store -----
  const float oscale = -LN2 / (float)n_norm;
  float* st = (float*)&sm.kv[0][0][0];
  constexpr int OCPR = D / 4;  // 16-byte chunks per output row
  #pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
    #pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = (32 * db + 8 * g + 4 * hl) / 4;
      f32x4 x = {oacc[db][4 * g] * oscale, oacc[db][4 * g + 1] * oscale, oacc[db][4 * g + 2] * oscale,
                 oacc[db][4 * g + 3] * oscale};
      *(f32x4*)(st + (row_w * OCPR + (c ^ (row_w % OCPR))) * 4) = x;
    }
  }
  __syncthreads();
  float* obase = a.o + (int64_t)it.chunk * a.o_chunk_stride;
  for (int i = tid; i < QT * OCPR; i += NTHREADS) {
    const int r = i / OCPR, c = i % OCPR;
    if (r < q_len && q_off + q_start + r < a.Tq && it.chunk < a.n_chunks) {
      const f32x4 x = *(const f32x4*)(st + (r * OCPR + (c ^ (r % OCPR))) * 4);
      *(f32x4*)(obase + ((q_off + q_start + r) * H + h) * D + c * 4) = x;
    }
  }
}

template <typename T, int D>
static hipError_t launch_mode(const AttnArgs& a, int mode, int64_t grid, hipStream_t s) {
  dim3 g((unsigned)grid), blk(NTHREADS);
  if (mode == MODE_FULL) hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_FULL>), g, blk, 0, s, a);
  else if (mode == MODE_CACHED) hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_CACHED>), g, blk, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_MFALCON>), g, blk, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int dtype, int D, int mode, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (dtype == 1) {
    if (D == 128) return launch_mode<bf16, 128>(a, mode, grid, s);
    if (D == 64) return launch_mode<bf16, 64>(a, mode, grid, s);
    if (D == 32) return launch_mode<bf16, 32>(a, mode, grid, s);
  } else {
    if (D == 128) return launch_mode<float, 128>(a, mode, grid, s);
    if (D == 64) return launch_mode<float, 64>(a, mode, grid, s);
    if (D == 32) return launch_mode<float, 32>(a, mode, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
