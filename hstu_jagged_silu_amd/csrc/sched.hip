// Jagged tile scheduler: turns per-user lengths (device memory) into the
// attention work list, ordered longest first.
//
// User histories differ wildly in length ("HSTU Generative Recommenders:
// Deploy on GPU Cloud", section "Scaling Training and Serving Across
// Multiple GPUs", on sequence-length balancing). A causal query tile at row r
// costs about r / 64 key tiles, so the attention grid is launched over the
// items sorted by decreasing cost: the hardware dispatcher then hands the
// next-longest item to whichever compute unit frees up first (greedy longest
// processing time). Masked key tiles are never listed (causal tile skipping):
// an item's key range ends at its last row's limit.
//
// Workgroup 0 (1024 threads): count items per user, scan, histogram the
// costs, scan the histogram from the top, scatter. The other workgroups of
// the same launch compute key timestamp ranges. Runs on the caller's stream
// ahead of the attention kernel; no host synchronisation.
#include "kernels.h"

namespace hstu {

constexpr int SCHED_THREADS = 1024;
constexpr int SCHED_WAVES = SCHED_THREADS / 64;
constexpr int NBINS = 1024;
// Batches of at most this many users keep the per-user table and the item
// prefix in LDS; larger ones read them from global memory.
constexpr int LDS_USERS = 2048;

struct UserGeo {
  int nq_causal;   // causal query tiles
  int nq_cand;     // candidate query tiles (M-FALCON)
  int L, C, n;     // rows, cached prefix, history length
};

// What the work list needs to know of one user: its query rows, and its
// cached prefix (paged modes) or candidate count (M-FALCON).
struct UserRaw {
  int L, X, off;
};

__device__ inline UserRaw user_raw(const SchedArgs& a, int b) {
  UserRaw r;
  r.off = a.offsets[b];
  r.L = max(0, a.offsets[b + 1] - r.off);
  r.X = mode_paged(a.mode) ? a.cache_lens[b] : (a.mode == MODE_MFALCON ? a.num_cand[b] : 0);
  return r;
}

__device__ inline UserGeo user_geo(const SchedArgs& a, UserRaw r) {
  UserGeo g;
  g.L = r.L;
  g.C = mode_paged(a.mode) ? r.X : 0;
  g.n = g.L;
  g.nq_cand = 0;
  if (a.mode == MODE_MFALCON) {
    const int m = min(max(r.X, 0), g.L);
    g.n = g.L - m;
    g.nq_cand = (int)ceil_div(m, QT);
  }
  g.nq_causal = (int)ceil_div(g.n, QT);
  if (a.mode == MODE_MFALCON_PAGED) {  // every row is a candidate; the history is C
    g.n = 0;
    g.nq_causal = 0;
    g.nq_cand = (int)ceil_div(g.L, QT);
  }
  return g;
}

// key splits of causal tile qt on the cached path
__device__ inline int tile_chunks(const SchedArgs& a, const UserGeo& g, int qt) {
  if (a.mode != MODE_CACHED) return 1;
  const int kend = g.C + min((qt + 1) * QT, g.n);
  return (int)ceil_div(kend, a.chunk_keys);
}

// key splits of every candidate tile on the paged M-FALCON path (at least one,
// which carries the candidates' own keys when the history is empty)
__device__ inline int cand_chunks(const SchedArgs& a, const UserGeo& g) {
  return max(1, (int)ceil_div(g.C, a.chunk_keys));
}

__device__ inline int user_items_per_head(const SchedArgs& a, const UserGeo& g) {
  if (a.mode == MODE_MFALCON_PAGED) return g.nq_cand * cand_chunks(a, g);
  if (a.mode != MODE_CACHED) return g.nq_causal + g.nq_cand;
  int s = 0;
  for (int qt = 0; qt < g.nq_causal; ++qt) s += tile_chunks(a, g, qt);
  return s;
}

// the local-th item of user b
__device__ inline WorkItem make_item(const SchedArgs& a, int b, UserRaw r, int local) {
  const UserGeo g = user_geo(a, r);
  const int per_head = user_items_per_head(a, g);
  WorkItem w;
  w.b = b;
  w.off = r.off;
  w.L = r.L;
  w.X = r.X;
  w.pad = 0;
  w.h = local / per_head;
  int t = local % per_head;
  w.chunk = 0;
  w.kind = KIND_CAUSAL;
  if (a.mode == MODE_MFALCON_PAGED) {
    const int nc = cand_chunks(a, g);
    const int qt = t / nc;
    w.kind = KIND_CANDIDATE;
    w.chunk = t % nc;
    w.q_start = qt * QT;
    w.q_len = min(QT, g.L - w.q_start);
    w.k_begin = min(w.chunk * a.chunk_keys, g.C);
    w.k_end = min(g.C, (w.chunk + 1) * a.chunk_keys);
  } else if (a.mode == MODE_CACHED) {
    int qt = 0;
    while (t >= tile_chunks(a, g, qt)) { t -= tile_chunks(a, g, qt); ++qt; }
    w.q_start = qt * QT;
    w.q_len = min(QT, g.n - w.q_start);
    const int kend = g.C + w.q_start + w.q_len;
    w.chunk = t;
    w.k_begin = t * a.chunk_keys;
    w.k_end = min(kend, (t + 1) * a.chunk_keys);
  } else if (t < g.nq_causal) {
    w.q_start = t * QT;
    w.q_len = min(QT, g.n - w.q_start);
    w.k_begin = 0;
    w.k_end = w.q_start + w.q_len;
  } else {
    const int qc = t - g.nq_causal;
    w.kind = KIND_CANDIDATE;
    w.q_start = g.n + qc * QT;
    w.q_len = min(QT, g.L - w.q_start);
    w.k_begin = 0;
    w.k_end = g.n;
  }
  return w;
}

__device__ inline int item_bin(const SchedArgs& a, const WorkItem& w) {
  const int cost = (int)ceil_div(max(w.k_end - w.k_begin, 0), KT) + 1;
  return min(cost >> a.cost_shift, NBINS - 1);
}

// Block-wide exclusive scan of one value per thread; returns the block
// total. Shuffle scan inside each wave, then every thread adds the totals of
// the waves before its own: two barriers in all.
template <typename V>
__device__ inline V block_scan(V x, V* wsum, V& excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  V inc = x;
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const V y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  V before = 0, total = 0;
  #pragma unroll
  for (int w = 0; w < SCHED_WAVES; ++w) {
    const V t = wsum[w];
    before += w < wave ? t : 0;
    total += t;
  }
  excl = before + inc - x;
  __syncthreads();  // wsum is reused by the next scan
  return total;
}

// Timestamp range (min, max) of every 64-key block, one wave per block. The
// attention kernel uses it to decide per tile whether the time bucket is the
// same for every pair. Jagged keys: block i covers packed rows [64i, 64i+64)
// (it may straddle users; a wider range only makes the test conservative).
// Cached keys: block (b, kt) covers the valid keys of that user's page kt.
__device__ void key_time_ranges(const SchedArgs& a) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)(blockIdx.x - 1) * (SCHED_THREADS / 64) + (threadIdx.x >> 6);
  if (blk >= a.n_stat_blocks) return;
  bool ok;
  int64_t v = 0;
  if (mode_paged(a.mode)) {
    const int b = (int)(blk / a.stat_stride), kt = (int)(blk % a.stat_stride);
    const int kcount = a.cache_lens[b] + (a.mode == MODE_CACHED ? a.offsets[b + 1] - a.offsets[b] : 0);
    const int page = kt < a.max_pages ? a.page_table[(int64_t)b * a.max_pages + kt] : -1;
    ok = kt * KT + lane < kcount && page >= 0 && page < a.num_pages;
    if (ok) v = a.ts_pages[(int64_t)page * PAGE + lane];
  } else {
    const int64_t r = blk * KT + lane;
    ok = r < a.Tk;
    if (ok) v = a.ts[r];
  }
  int64_t mn = ok ? v : INT64_MAX, mx = ok ? v : INT64_MIN;
  for (int m = 32; m >= 1; m >>= 1) {
    mn = min(mn, (int64_t)__shfl_xor((long long)mn, m));
    mx = max(mx, (int64_t)__shfl_xor((long long)mx, m));
  }
  if (lane == 0) {
    a.tstats[2 * blk] = mn;
    a.tstats[2 * blk + 1] = mx;
  }
}

__global__ __launch_bounds__(SCHED_THREADS) void sched_kernel(SchedArgs a) {
  if (a.debug_flag && *a.debug_flag != 0) {
    // debug mode, bad index content: an empty work list (and empty per-user
    // counts for the reductions that read them)
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i <= a.B; i += SCHED_THREADS) a.prefix[i] = 0;
      if (threadIdx.x == 0) *a.count = 0;
    }
    return;
  }
  if (blockIdx.x > 0) {
    key_time_ranges(a);
    return;
  }
  __shared__ int wsum[SCHED_WAVES];
  __shared__ long long wsum64[SCHED_WAVES];
  __shared__ int hist[NBINS];
  __shared__ int start[NBINS];
  __shared__ int s_pref[LDS_USERS + 1];
  __shared__ UserRaw s_raw[LDS_USERS];
  const int tid = threadIdx.x;
  const bool in_lds = a.B <= LDS_USERS;
  for (int i = tid; i < NBINS; i += SCHED_THREADS) hist[i] = 0;

  // 1. items per user -> exclusive prefix over users (and, for the
  // backward at d = 128, the prefix of the users' dS blocks)
  int carry = 0;
  long long ds_carry = 0;
  for (int base = 0; base < a.B; base += SCHED_THREADS) {
    const int b = base + tid;
    int c = 0;
    long long c2 = 0;
    if (b < a.B) {
      const UserRaw r = user_raw(a, b);
      if (in_lds) s_raw[b] = r;
      c = a.H * user_items_per_head(a, user_geo(a, r));
      const long long nb = ceil_div(r.L, KT);
      c2 = nb * (nb + 1) / 2;
    }
    int excl;
    const int tot = block_scan(c, wsum, excl);
    if (b < a.B) {
      a.prefix[b] = carry + excl;
      if (in_lds) s_pref[b] = carry + excl;
    }
    carry += tot;
    if (a.ds_prefix) {  // a kernel argument: every thread takes the same branch
      long long excl2;
      const long long tot2 = block_scan(c2, wsum64, excl2);
      if (b < a.B) a.ds_prefix[b] = ds_carry + excl2;
      ds_carry += tot2;
    }
  }
  if (a.ds_prefix && tid == 0) a.ds_prefix[a.B] = ds_carry;
  int total = carry;
  if ((int64_t)total > a.max_items) total = (int)a.max_items;  // cannot happen with a valid bound
  if (tid == 0) {
    a.prefix[a.B] = carry;
    if (in_lds) s_pref[a.B] = carry;
  }
  __threadfence_block();
  __syncthreads();

  auto pref = [&](int i) { return in_lds ? s_pref[i] : a.prefix[i]; };
  auto raw = [&](int b) { return in_lds ? s_raw[b] : user_raw(a, b); };
  auto item = [&](int g) {
    int lo = 0, hi = a.B - 1;  // largest b with prefix[b] <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref(mid) <= g) lo = mid; else hi = mid - 1;
    }
    return make_item(a, lo, raw(lo), g - pref(lo));
  };

  // 2. cost histogram. A thread's first KEEP items stay in registers for the
  // scatter (lists of up to KEEP * 1024 items are built once); later ones
  // are rebuilt there.
  constexpr int KEEP = 4;
  WorkItem kept[KEEP];
  int kept_bin[KEEP];
  #pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    const int g = tid + k * SCHED_THREADS;
    kept_bin[k] = -1;
    if (g < total) {
      kept[k] = item(g);
      kept_bin[k] = item_bin(a, kept[k]);
      atomicAdd(&hist[kept_bin[k]], 1);
    }
  }
  for (int g = tid + KEEP * SCHED_THREADS; g < total; g += SCHED_THREADS) atomicAdd(&hist[item_bin(a, item(g))], 1);
  __syncthreads();

  // 3. start of each bin, most expensive bin first (one bin per thread)
  {
    static_assert(NBINS == SCHED_THREADS, "one cost bin per thread");
    const int bin = NBINS - 1 - tid;
    int excl;
    block_scan(hist[bin], wsum, excl);
    start[bin] = excl;
  }
  __syncthreads();

  // 4. scatter
  #pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    if (kept_bin[k] >= 0) a.items[atomicAdd(&start[kept_bin[k]], 1)] = kept[k];
  }
  for (int g = tid + KEEP * SCHED_THREADS; g < total; g += SCHED_THREADS) {
    const WorkItem w = item(g);
    const int pos = atomicAdd(&start[item_bin(a, w)], 1);
    a.items[pos] = w;
  }
  if (tid == 0) *a.count = total;
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t s) {
  const int64_t grid = 1 + ceil_div(a.n_stat_blocks, SCHED_THREADS / 64);
  hipLaunchKernelGGL(sched_kernel, dim3((unsigned)grid), dim3(SCHED_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
