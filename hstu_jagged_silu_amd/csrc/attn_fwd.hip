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
//   * K and V tiles go from HBM straight into LDS (global_load_lds, 16 bytes
//     per lane), row-major with an XOR swizzle on 16-byte chunks chosen by
//     which global chunk each lane fetches. No registers hold the prefetch;
//     the next tile streams in while the current one is computed.
//   * The score tile is computed transposed, S^T[key][q] = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (fp32: v_mfma_f32_32x32x2_f32). The 32x32
//     accumulator puts query q = lane % 32 in every register of a lane, and
//     keys along the registers.
//   * K rows are fed to the MFMA in a permuted order so that, after SiLU, the
//     8 consecutive accumulator registers of a lane hold 8 consecutive keys:
//     they are exactly the B operand (P^T) of the second product
//     O^T[d][q] += V^T[d][key] P^T[key][q]. No shuffle sits between the two.
//   * The A operand V^T of the second product is read from the row-major V
//     tile with two transposing LDS reads (ds_read_b64_tr_b16).
//   * The bias is folded into one FMA per score: y = s * (-alpha log2 e) + b'
//     with b' = -log2(e) (P[.] + T[.]); then SiLU(x) = -ln2 * y / (1 + 2^y),
//     and the -ln2 / N factor moves to the epilogue. Far from the diagonal a
//     wave tile's bias is usually one constant (position clamped, one time
//     bucket); the per-element bucket path only runs where it varies, and
//     there a masked pair gets a huge bias that makes its SiLU exactly 0.
//   * Per tile, the score MFMAs of both 32-key blocks, the P V MFMAs and the
//     accumulators are shared by every tile kind; only the SiLU inputs
//     differ. The compiler then keeps one register assignment for O and
//     overlaps the second block's SiLU with the P V MFMAs.
#include "tile.h"

namespace hstu {

template <typename T, int D, int MODE>
__global__ __launch_bounds__(NTHREADS, (sizeof(T) == 4 && D == 128) ? 1 : 2)  // fp32 d=128: LDS allows one
void attn_fwd_kernel(AttnArgs a) {
  using G = Geo<T, D>;
  using M = Mfma<T>;
  // Two distinct LDS objects (not one array indexed by stage): the compiler
  // can then tell that reads of one stage never alias the DMA into the other
  // and does not wait for the prefetch before every operand read.
  __shared__ Stage<T, D> st0;
  __shared__ Stage<T, D> st1;
  __shared__ Tables tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave facts in SGPRs
  // the item and the count load together (the item array holds an entry for
  // every workgroup of the grid; one past the count is never used)
  const int32_t count = ldc(a.count);
  const WorkItem it = ldc(a.items + blockIdx.x);
  if ((int64_t)blockIdx.x >= (int64_t)count) return;
  const int b = it.b, h = it.h, kind = it.kind;
  const int q_start = it.q_start, q_len = it.q_len;
  const int k_begin = it.k_begin, k_end = it.k_end;
  const int H = a.H;

  // ---- per-user geometry -------------------------------------------------
  const int64_t q_off = it.off;
  const int Lq = it.L;
  int kcount, pos0, n_norm;
  bool cand = false;
  if (MODE == MODE_CACHED) {
    const int C = it.X;
    kcount = C + Lq;
    pos0 = C + q_start;
    n_norm = C + Lq;
  } else if (MODE == MODE_MFALCON_PAGED) {
    const int C = it.X;  // history length; every row is a candidate at position C
    kcount = C;
    cand = true;
    pos0 = C;
    n_norm = C + 1;
  } else if (MODE == MODE_MFALCON) {
    const int n = Lq - it.X;
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
    for (int i = tid; i < n_pos; i += NTHREADS) tab.pos_t[i] = pt ? pt[i] * -LOG2E : 0.0f;
    if (tid < 64) {
      float t = 0.0f;
      if (a.time_tab) {
        int bk = min(63 - tid, a.n_time - 1);
        t = a.time_tab[(int64_t)h * a.time_stride + bk] * -LOG2E;
      }
      tab.time_t[tid] = t;
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
  w_ts_min = uniform64(w_ts_min);
  w_ts_max = uniform64(w_ts_max);

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

  // ---- key tile staging (HBM -> LDS, no registers) --------------------------
  // Keys past the end of a user (partial last tile) read a copy of the last
  // valid row: finite values that the causal mask zeroes. A missing page of
  // the cached path reads as zeros.
  int64_t tsreg = 0;
  // full path: the item's K, V and timestamp rows start at the user's first
  // row; rows_left rows of the buffer exist from there on
  const int rows_left = (int)min<int64_t>(a.Tq - q_off, (int64_t)INT_MAX);
  const unsigned char* k_item = (const unsigned char*)a.k + ((q_off * H + h) * D) * (int64_t)sizeof(T);
  const unsigned char* v_item = (const unsigned char*)a.v + ((q_off * H + h) * D) * (int64_t)sizeof(T);

  auto issue_tile = [&](Stage<T, D>& st, int j0) {
    const unsigned char* kbase;
    const unsigned char* vbase;
    const int64_t* tsbase;
    int64_t rstride;  // bytes between consecutive keys
    int nvalid = min(KT, kcount - j0);
    bool missing = false;
    if (mode_paged(MODE)) {
      int page = j0 / PAGE < a.max_pages ? ldc(a.page_table + (int64_t)b * a.max_pages + j0 / PAGE) : -1;
      if (page < 0 || page >= a.num_pages) {
        page = 0;
        missing = true;
      }
      const int64_t pb = (((int64_t)page * H + h) * PAGE * D) * (int64_t)sizeof(T);
      kbase = (const unsigned char*)a.k_pages + pb;
      vbase = (const unsigned char*)a.v_pages + pb;
      rstride = G::ROWB;
      tsbase = a.ts_pages + (int64_t)page * PAGE;
    } else {
      // row q_off + jr = min(q_off + j0, Tq - 1), in 32-bit arithmetic
      const int jr = min(j0, rows_left - 1);
      nvalid = min(nvalid, rows_left - jr);
      rstride = (int64_t)H * G::ROWB;
      kbase = k_item + (int64_t)jr * rstride;
      vbase = v_item + (int64_t)jr * rstride;
      tsbase = a.ts + (q_off + jr);
    }
    const int last = max(nvalid - 1, 0);
    if (missing) {
      #pragma unroll
      for (int i = 0; i < G::NDMA; ++i) {
        const int P = (wave * G::NDMA + i) * 64 + lane;  // 16-byte LDS chunk this lane fills
        *(i32x4*)(st.k + P * 16) = i32x4{};
        *(i32x4*)(st.v + P * 16) = i32x4{};
      }
    } else {
      // a lane's source is the tile's base (wave-uniform) plus a 32-bit
      // offset: at most 63 rows of H * D <= 2048 elements (a 24-bit product)
      const uint32_t rs32 = (uint32_t)rstride;
      #pragma unroll
      for (int i = 0; i < G::NDMA; ++i) {
        const int base = (wave * G::NDMA + i) * 64;      // first LDS chunk of this instruction
        const int P = base + lane;
        const int r = P / G::CPR, pc = P % G::CPR;
        const uint32_t row = __umul24((uint32_t)min(r, last), rs32);
        __builtin_amdgcn_global_load_lds((const void*)(kbase + (row + (uint32_t)((pc ^ G::swz_k(r)) << 4))),
                                         LDS_PTR(void, st.k + base * 16), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vbase + (row + (uint32_t)((pc ^ G::swz_v(r)) << 4))),
                                         LDS_PTR(void, st.v + base * 16), 16, 0, 0);
      }
    }
    if (wave == 0) tsreg = tsbase[min(lane, last)];
  };

  // Wait for this wave's DMA, publish the timestamps, then the barrier makes
  // the whole tile visible to every wave.
  auto finish_tile = [&](Stage<T, D>& st) {
    __builtin_amdgcn_s_waitcnt(0);
    if (wave == 0) {
      st.ts_lo[lane] = (int32_t)tsreg;
      st.ts64[lane] = tsreg;
    }
    __syncthreads();
  };

  // timestamp range of the keys of the tile at j0 (conservative superset)
  auto key_time_range = [&](int j0, int64_t& kmin, int64_t& kmax) {
    if (mode_paged(MODE)) {
      const int64_t blk = (int64_t)b * a.stat_stride + j0 / KT;
      kmin = ldc(a.tstats + 2 * blk);
      kmax = ldc(a.tstats + 2 * blk + 1);
    } else {
      const int64_t r0 = q_off + j0;
      const int64_t i0 = min(r0 / KT, a.n_stat_blocks - 1), i1 = min((r0 + KT - 1) / KT, a.n_stat_blocks - 1);
      kmin = min(ldc(a.tstats + 2 * i0), ldc(a.tstats + 2 * i1));
      kmax = max(ldc(a.tstats + 2 * i0 + 1), ldc(a.tstats + 2 * i1 + 1));
    }
    if (kmin > kmax) kmin = kmax = w_ts_min;  // no valid key: the bias value is irrelevant
  };

  // ---- accumulators -------------------------------------------------------
  f32x16 oacc[G::NDB];
  #pragma unroll
  for (int i = 0; i < G::NDB; ++i) oacc[i] = f32x16{};

  const float sc = a.alpha * -LOG2E;
  const bool has_time = a.time_tab != nullptr;
  const int n_time_eff = a.time_tab ? min(a.n_time, 64) : 1;

  // source address of this lane for the transposing V read of operand (db, c), half s4
  const int tr_g = lane >> 4, tr_j = lane & 15;
  auto v_tr_off = [&](int db, int c, int s4) {
    const int key = 16 * c + 8 * (tr_g >> 1) + 4 * s4 + (tr_j >> 2);
    const int d = 32 * db + 16 * (tr_g & 1) + 4 * (tr_j & 3);
    return G::v_off(key, d / G::EPC) + (d % G::EPC) * (int)sizeof(T);
  };

  // Per-lane byte offsets of this lane's MFMA operand reads inside a stage's K
  // and V tiles, for key block 0 (the second 32-key block adds 32 rows, the
  // second 16-key half of a V operand 16 rows: compile-time offsets).
  // In bf16 the K chunk of step s of row r sits at r * ROWB + ((2s + hl) xor
  // swz(r)) * 16 = (r * ROWB + (hl xor swz(r)) * 16) xor 32s (row and chunk
  // fields do not overlap), so one base per lane serves every step.
  uint32_t voff[G::NDB][2];
  const uint32_t k_base = (uint32_t)G::k_off(M::krow(0, l32), sizeof(T) == 2 ? hl : 0);
  {
    #pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      voff[db][0] = (uint32_t)v_tr_off(db, 0, 0);
      voff[db][1] = (uint32_t)v_tr_off(db, 0, 1);
    }
  }

  using LB = __attribute__((address_space(3))) unsigned char;

  // Time-bias constant of each key tile for this wave, 64 tiles at a time
  // (lane i holds tile t0 + i): the table value when every pair of the wave
  // tile falls in one time bucket (ordered timestamps whose |dt| range stays
  // inside one power of two, or the clamped last bucket), NaN where the
  // bucket varies. One lane-parallel pass replaces a per-tile scalar
  // classification (range loads, 64-bit compares, clz, table read).
  // Two-bucket tiles (queries after keys, |dt| range crossing one power of
  // two, every |dt| below 2^31 - 2) also carry their threshold 2^b - 1 and
  // the two table values, so that such a tile needs no range loads either
  // and picks its bucket with one 32-bit subtract per element; tthr < 0
  // marks every other tile.
  float tc = 0.0f, tclo = 0.0f, tchi = 0.0f;
  int tthr = -1;
  auto time_batch = [&](int t0, int ntiles) {
    const int t = t0 + lane;
    float c = __builtin_nanf("");
    float clo = 0.0f, chi = 0.0f;
    int thr = -1;
    if (t < ntiles) {
      const int j0 = k_begin + t * KT;
      int64_t kmin, kmax;
      if (mode_paged(MODE)) {
        const int64_t blk = (int64_t)b * a.stat_stride + min(j0 / KT, a.stat_stride - 1);
        kmin = a.tstats[2 * blk];
        kmax = a.tstats[2 * blk + 1];
      } else {
        const int64_t r0 = q_off + j0;
        const int64_t i0 = min(r0 / KT, a.n_stat_blocks - 1), i1 = min((r0 + KT - 1) / KT, a.n_stat_blocks - 1);
        kmin = min(a.tstats[2 * i0], a.tstats[2 * i1]);
        kmax = max(a.tstats[2 * i0 + 1], a.tstats[2 * i1 + 1]);
      }
      if (kmin > kmax) kmin = kmax = w_ts_min;  // no valid key: the bias value is irrelevant
      int64_t lo = -1, hi = 0;
      if (w_ts_min >= kmax) { lo = w_ts_min - kmax; hi = w_ts_max - kmin; }
      else if (kmin >= w_ts_max) { lo = kmin - w_ts_max; hi = kmax - w_ts_min; }
      if (lo >= 0) {
        const int zlo = __builtin_clzll((uint64_t)lo + 1), zhi = __builtin_clzll((uint64_t)hi + 1);
        const int blo = min(63 - zlo, n_time_eff - 1), bhi = min(63 - zhi, n_time_eff - 1);
        if (blo == bhi) {
          c = tab.time_t[zlo];
        } else if (w_ts_min >= kmax && zhi == zlo - 1 && 63 - zhi <= n_time_eff - 1 &&
                   hi < ((int64_t)1 << 31) - 2) {
          thr = (1 << (63 - zhi)) - 1;  // |dt| >= thr selects the upper bucket
          clo = tab.time_t[zlo];
          chi = tab.time_t[zhi];
        }
      }
    }
    tc = c;
    tclo = clo;
    tchi = chi;
    tthr = thr;
  };

  auto compute_tile = [&](Stage<T, D>& st, int j0, int t) {
    if (!w_rows || j0 > w_lim_max) return;  // every pair of this wave masked

    // classify the wave tile: mask, constant bias, or per-element bias
    const bool need_mask = j0 + KT - 1 > w_lim_min;
    const bool pos_uniform = (a.pos_tab == nullptr) || (w_p_min - (j0 + KT - 1) >= n_pos - 1);
    bool time_uniform = !has_time;
    float c_time = 0.0f;
    int two_thr_t = -1;  // >= 0: a two-bucket tile classified by the batch pass
    if (has_time) {
      const float ct = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tc), t & 63));
      time_uniform = ct == ct;  // NaN: the bucket varies over the tile
      c_time = time_uniform ? ct : 0.0f;
      if (!time_uniform) two_thr_t = __builtin_amdgcn_readlane(tthr, t & 63);
    }
    const bool uniform = pos_uniform && time_uniform;
    const float c_pos = a.pos_tab ? tab.pos_t[n_pos - 1] : 0.0f;
    // the keys' time range and |dt| span, needed only where the time bucket
    // varies (per-element path)
    int64_t k_min = 0, k_max = 0;
    bool small_span = true;
    auto load_time_range = [&]() {
      if (time_uniform) return;
      key_time_range(j0, k_min, k_max);
      int64_t hi;
      if (w_ts_min >= k_max) hi = w_ts_max - k_min;
      else if (k_min >= w_ts_max) hi = k_max - w_ts_min;
      else hi = max(w_ts_max - k_min, k_max - w_ts_min);
      small_span = hi < ((int64_t)1 << 31) - 2;
    };
    const int32_t tsq_lo = (int32_t)tsq;
    // per-lane bases: the per-register offsets key_of(kb, v, 0) are constants
    const int lim_rel = lim_lane - j0 - M::HLK * hl;   // allowed iff key_of(kb, v, 0) <= lim_rel
    const int rel_base = p_lane - j0 - M::HLK * hl;    // relative position = rel_base - key_of(kb, v, 0)
    const int32_t* ts_lo_l = st.ts_lo + M::HLK * hl;
    const int64_t* ts64_l = st.ts64 + M::HLK * hl;

    // Per-element bias of key block kb, scaled by -log2(e); masked pairs get
    // MASKED_Y when fold_mask (SiLU of it is exactly zero).
    auto element_bias = [&](int kb, float* cb, bool fold_mask) {
      // Two-bucket tiles (ordered timestamps whose |dt| range crosses one
      // power of two) need only a threshold compare per element.
      int two_thr = -1;   // |dt| >= two_thr selects the upper bucket
      float c_lo = 0.0f, c_hi = 0.0f;
      bool q_after_k = false;
      if (has_time && !time_uniform && small_span) {
        int64_t lo = -1, hi = -1;
        if (w_ts_min >= k_max) { lo = w_ts_min - k_max; hi = w_ts_max - k_min; q_after_k = true; }
        else if (k_min >= w_ts_max) { lo = k_min - w_ts_max; hi = k_max - w_ts_min; }
        if (lo >= 0) {
          const int zlo = __builtin_clzll((uint64_t)lo + 1), zhi = __builtin_clzll((uint64_t)hi + 1);
          const int blo = 63 - zlo, bhi = 63 - zhi;
          if (bhi == blo + 1 && bhi <= n_time_eff - 1) {
            two_thr = (1 << bhi) - 1;
            c_lo = tab.time_t[zlo];
            c_hi = tab.time_t[zhi];
          }
        }
      }
      #pragma unroll
      for (int v = 0; v < 16; ++v) {
        if (pos_uniform) {
          cb[v] = c_pos;
        } else {
          const unsigned rel = (unsigned)(rel_base - M::key_of(kb, v, 0));
          cb[v] = tab.pos_t[min(rel, (unsigned)(n_pos - 1))];
        }
      }
      if (time_uniform) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) cb[v] += c_time;
      } else if (two_thr >= 0) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t dt = tsq_lo - ts_lo_l[M::key_of(kb, v, 0)];
          cb[v] += ((q_after_k ? dt : -dt) >= two_thr) ? c_hi : c_lo;
        }
      } else if (small_span) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t dt = tsq_lo - ts_lo_l[M::key_of(kb, v, 0)];
          const uint32_t x = (uint32_t)(dt < 0 ? -dt : dt) + 1u;
          cb[v] += tab.time_t[__builtin_clz(x) + 32];
        }
      } else {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t dt = tsq - ts64_l[M::key_of(kb, v, 0)];
          const uint64_t x = (uint64_t)(dt < 0 ? -dt : dt) + 1u;
          cb[v] += tab.time_t[__builtin_clzll(x)];
        }
      }
      if (fold_mask && need_mask) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) cb[v] = (M::key_of(kb, v, 0) <= lim_rel) ? cb[v] : MASKED_Y;
      }
    };

    if constexpr (sizeof(T) == 2) {
      LB* kl = LDS_PTR(unsigned char, st.k);
      LB* vl = LDS_PTR(unsigned char, st.v);
      // S^T = K Q^T for both 32-key blocks as two interleaved chains, the K
      // operands of step s + 1 read while the MFMAs of step s run; the base
      // passes through an empty asm so that the step offsets are formed here,
      // in every tile, instead of being kept in registers
      auto s_chains = [&](f32x16& s0, f32x16& s1) {
        uint32_t kb_t = k_base;
        asm volatile("" : "+v"(kb_t));
        s0 = f32x16{};
        s1 = f32x16{};
        bf16x8 op[2][2];
        auto read_step = [&](int i, bf16x8* o) {
          const uint32_t off = kb_t ^ (uint32_t)(i << 5);
          o[0] = *(__attribute__((address_space(3))) const bf16x8*)(kl + off);
          o[1] = *(__attribute__((address_space(3))) const bf16x8*)(kl + off + 32 * G::ROWB);
        };
        read_step(0, op[0]);
        #pragma unroll
        for (int i = 0; i < G::NQOP; ++i) {
          if (i + 1 < G::NQOP) read_step(i + 1, op[(i + 1) & 1]);
          s0 = M::run(op[i & 1][0], qop[i], s0);
          s1 = M::run(op[i & 1][1], qop[i], s1);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // O^T += V^T P^T for block kb; V^T operands from two transposing reads
      auto pv = [&](int kb, const bf16x8* pb) {
        #pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          #pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int o = (2 * kb + cc) * 16 * G::ROWB;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(vl + voff[db][0] + o));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(vl + voff[db][1] + o));
            const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = M::run(vop, pb[cc], oacc[db]);
          }
        }
      };
      // SiLU of y = s * (-alpha log2 e) + bias, packed to bf16
      auto silu_pack = [&](const float* y, bf16x8* pb) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = y[v] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y[v]));
          pb[v >> 3][v & 7] = (bf16)p;
        }
      };

      // Score MFMAs of both 32-key blocks, then the biased scores y (one bias
      // constant, or per-element bias with the mask folded in), then SiLU and
      // the P V MFMAs. The accumulators and the SiLU are only touched by code
      // shared by every tile; the empty asm keeps each kind's bias FMAs in its
      // own branch, so that the shared code does not take a 16-value bias
      // (which the constant kind would fill with 16 register copies per tile).
      f32x16 s0, s1;
      s_chains(s0, s1);
      float y0[16], y1[16];
      if (uniform && !need_mask) {
        const float cu = c_pos + c_time;
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          y0[v] = fmaf(s0[v], sc, cu);
          y1[v] = fmaf(s1[v], sc, cu);
          asm volatile("" : "+v"(y0[v]), "+v"(y1[v]));
        }
      } else if (two_thr_t >= 0 && pos_uniform && !need_mask) {
        // x = dt - thr in 32 bits (exact: 0 <= dt < 2^31 - 2), upper bucket iff x >= 0
        const float clo = c_pos + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tclo), t & 63));
        const float chi = c_pos + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tchi), t & 63));
        const uint32_t b_lane = (uint32_t)tsq_lo - (uint32_t)two_thr_t;
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t x0 = (int32_t)(b_lane - (uint32_t)ts_lo_l[M::key_of(0, v, 0)]);
          const int32_t x1 = (int32_t)(b_lane - (uint32_t)ts_lo_l[M::key_of(1, v, 0)]);
          y0[v] = fmaf(s0[v], sc, x0 >= 0 ? chi : clo);
          y1[v] = fmaf(s1[v], sc, x1 >= 0 ? chi : clo);
          asm volatile("" : "+v"(y0[v]), "+v"(y1[v]));
        }
      } else {
        load_time_range();
        float cb[16];
        element_bias(0, cb, true);
        #pragma unroll
        for (int v = 0; v < 16; ++v) y0[v] = fmaf(s0[v], sc, cb[v]);
        element_bias(1, cb, true);
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          y1[v] = fmaf(s1[v], sc, cb[v]);
          asm volatile("" : "+v"(y0[v]), "+v"(y1[v]));
        }
      }
      bf16x8 p0[2], p1[2];
      silu_pack(y0, p0);
      silu_pack(y1, p1);
      pv(0, p0);
      pv(1, p1);
    } else {
      const unsigned char* kl = st.k;
      const unsigned char* vl = st.v;
      if (!uniform) load_time_range();
      #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float acc_p[16];
        {
          f32x16 acc = f32x16{};
          const int kr = M::krow(kb, l32);
          #pragma unroll
          for (int s = 0; s < G::NQOP; ++s) {
            const int d = 2 * s + hl;
            acc = M::run(*(const float*)(kl + G::k_off(kr, d / 4) + (d % 4) * 4), qop[s], acc);
          }
          float cb[16];
          if (uniform) {
            #pragma unroll
            for (int v = 0; v < 16; ++v) cb[v] = c_pos + c_time;
          } else {
            element_bias(kb, cb, false);
          }
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float y = fmaf(acc[v], sc, cb[v]);
            acc_p[v] = y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
            if (need_mask) acc_p[v] = (M::key_of(kb, v, 0) <= lim_rel) ? acc_p[v] : 0.0f;
          }
        }
        #pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = M::key_of(kb, v, hl);
            const int d = 32 * db + l32;
            const float vv = *(const float*)(vl + G::v_off(key, d / 4) + (d % 4) * 4);
            oacc[db] = M::run(vv, acc_p[v], oacc[db]);
          }
        }
      }
    }
  };

  // ---- main loop over key tiles: compute one stage while the next streams in
  const int ntiles = k_end > k_begin ? (int)ceil_div(k_end - k_begin, KT) : 0;
  if (ntiles > 0) {
    issue_tile(st0, k_begin);
    finish_tile(st0);
  } else {
    __syncthreads();  // tables
  }
  for (int t = 0; t < ntiles; t += 2) {
    // the next 64 tiles' time classes: loads issued before this step's DMA,
    // so waiting for them does not wait for the DMA
    if (has_time && (t & 63) == 0) time_batch(t, ntiles);
    const int j0 = k_begin + t * KT;
    if (t + 1 < ntiles) issue_tile(st1, j0 + KT);
    compute_tile(st0, j0, t);
    if (t + 1 >= ntiles) break;
    finish_tile(st1);
    if (t + 2 < ntiles) issue_tile(st0, j0 + 2 * KT);
    compute_tile(st1, j0 + KT, t + 1);
    if (t + 2 < ntiles) finish_tile(st0);
  }

  // ---- M-FALCON: a candidate's own key (relative position 0, dt = 0) -------
  if ((MODE == MODE_MFALCON || MODE == MODE_MFALCON_PAGED) && cand && it.chunk == 0) {
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
    const float y = fmaf(dot, sc, tab.pos_t[0] + tab.time_t[63]);
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
  // Rows 0..63 are staged in stage 0's memory and rows 64..127 in stage 1's
  // (each holds 64 rows of D fp32 values); chunks are XOR-swizzled by row.
  __syncthreads();  // every wave is done reading the stages
  const float oscale = -LN2 / (float)n_norm;
  if constexpr (sizeof(T) == 2 && (MODE == MODE_FULL || MODE == MODE_MFALCON)) {
    if (a.o_dev != nullptr) {
      // Norm-ready store. This lane holds half of its row's D values (the
      // other half is in lane ^ 32). The head's mean and sum of squared
      // deviations come from the fp32 values (two passes over registers);
      // the deviations go out as bf16, so their rounding is relative to the
      // head's spread, not to a common offset of the row.
      float sum = 0.0f;
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          oacc[db][v] *= oscale;
          sum += oacc[db][v];
        }
      }
      sum += __shfl_xor(sum, 32);
      const float mean_h = sum * (1.0f / (float)D);
      float m2 = 0.0f;
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
          oacc[db][v] -= mean_h;
          m2 = fmaf(oacc[db][v], oacc[db][v], m2);
        }
      }
      m2 += __shfl_xor(m2, 32);
      const int64_t grow = q_off + q_start + row_w;
      if (hl == 0 && row_ok && grow < a.Tq)
        *(f32x2*)(a.o_stats + 2 * (grow * H + h)) = f32x2{mean_h, m2};
      // bf16 rows staged in stage 0's memory (128 rows x D x 2 bytes)
      constexpr int BCPR = D / 8;  // 16-byte chunks (8 values) per bf16 row
      static_assert(sizeof(Stage<T, D>) >= QT * D * 2, "bf16 output staging fits one stage");
      auto bstage = [&](int r) { return (bf16*)(unsigned char*)&st0 + r * D; };
      #pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        #pragma unroll
        for (int g = 0; g < 4; ++g) {
          // values d = 32 db + 8 g + 4 hl + (0..3): half of a 16-byte chunk
          const int d0 = 32 * db + 8 * g + 4 * hl;
          bf16x4 x;
          #pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)oacc[db][4 * g + e];
          const int c = d0 / 8;
          *(bf16x4*)(bstage(row_w) + (c ^ (row_w % BCPR)) * 8 + (d0 % 8)) = x;
        }
      }
      __syncthreads();
      for (int i = tid; i < QT * BCPR; i += NTHREADS) {
        const int r = i / BCPR, c = i % BCPR;
        if (r < q_len && q_off + q_start + r < a.Tq) {
          const bf16x8 x = *(const bf16x8*)(bstage(r) + (c ^ (r % BCPR)) * 8);
          *(bf16x8*)(a.o_dev + ((q_off + q_start + r) * H + h) * D + c * 8) = x;
        }
      }
      return;
    }
  }
  constexpr int OCPR = D / 4;  // 16-byte chunks per output row
  static_assert(sizeof(Stage<T, D>) >= 64 * D * 4, "output staging fits one stage per 64 rows");
  auto ostage = [&](int r) { return (float*)(r < 64 ? (unsigned char*)&st0 : (unsigned char*)&st1) + (r & 63) * D; };
  #pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
    #pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = (32 * db + 8 * g + 4 * hl) / 4;
      f32x4 x = {oacc[db][4 * g] * oscale, oacc[db][4 * g + 1] * oscale, oacc[db][4 * g + 2] * oscale,
                 oacc[db][4 * g + 3] * oscale};
      *(f32x4*)(ostage(row_w) + (c ^ (row_w % OCPR)) * 4) = x;
    }
  }
  __syncthreads();
  float* obase = a.o + (int64_t)it.chunk * a.o_chunk_stride;
  for (int i = tid; i < QT * OCPR; i += NTHREADS) {
    const int r = i / OCPR, c = i % OCPR;
    if (r < q_len && q_off + q_start + r < a.Tq && it.chunk < a.n_chunks) {
      const f32x4 x = *(const f32x4*)(ostage(r) + (c ^ (r % OCPR)) * 4);
      *(f32x4*)(obase + ((q_off + q_start + r) * H + h) * D + c * 4) = x;
    }
  }
}

template <typename T, int D>
static hipError_t launch_mode(const AttnArgs& a, int mode, int64_t grid, hipStream_t s) {
  dim3 g((unsigned)grid), blk(NTHREADS);
  if (mode == MODE_FULL) hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_FULL>), g, blk, 0, s, a);
  else if (mode == MODE_CACHED) hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_CACHED>), g, blk, 0, s, a);
  else if (mode == MODE_MFALCON) hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_MFALCON>), g, blk, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<T, D, MODE_MFALCON_PAGED>), g, blk, 0, s, a);
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
