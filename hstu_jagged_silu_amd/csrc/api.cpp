// C ABI of the HSTU attention library: host-side argument checks, workspace
// layout and the launch sequence of each entry point. No allocation, no host
// synchronisation; everything is queued on the caller's stream. The one
// device buffer the library owns is the scratch array of the no-allocation
// variant of the cached path.
#include <cstdlib>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <mutex>

#include "../../include/hstu.h"
#include "kernels.h"

using namespace hstu;

// Scratch of hstu_attn_fwd_cached_noalloc: one copy on every GPU the library
// runs on, alive until the process ends. In host code this name is only a
// handle for hipGetSymbolAddress; the device address comes from there.
static __device__ __align__(256) unsigned char scratch[HSTU_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
std::atomic<void*> scratch_addr[MAX_DEVICES];  // device address of `scratch`, per device

// Address of the current device's scratch, looked up once per device with
// that device current; nullptr when the lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

constexpr int32_t VERSION = 10000;  // 1.0.0
constexpr int MAX_SPLITS = 16;      // key splits of the cached path
constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hstu_status_t check_params(const hstu_params_t* p) {
  if (!p) return HSTU_ERR_INVALID_ARG;
  if (p->num_heads < 1) return HSTU_ERR_INVALID_ARG;
  if (p->dtype != HSTU_F32 && p->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128) return HSTU_ERR_UNSUPPORTED;
  if ((int64_t)p->num_heads * p->head_dim > 2048) return HSTU_ERR_UNSUPPORTED;
  if (p->norm_n < 0) return HSTU_ERR_INVALID_ARG;
  if (!(p->ln_eps > 0.0f)) return HSTU_ERR_INVALID_ARG;
  if (p->pos_tab) {
    if (p->n_pos < 1) return HSTU_ERR_INVALID_ARG;
    if (p->n_pos > MAX_NPOS) return HSTU_ERR_UNSUPPORTED;
    if (p->pos_head_stride != 0 && p->pos_head_stride < p->n_pos) return HSTU_ERR_INVALID_ARG;
  }
  if (p->time_tab) {
    if (p->n_time < 1) return HSTU_ERR_INVALID_ARG;
    if (p->time_head_stride != 0 && p->time_head_stride < p->n_time) return HSTU_ERR_INVALID_ARG;
  }
  if ((p->ln_w && !aligned16(p->ln_w)) || (p->ln_b && !aligned16(p->ln_b))) return HSTU_ERR_INVALID_ARG;
  if (p->flags & ~(HSTU_FLAG_FP32_NORM_INPUT | HSTU_FLAG_SAVED_FORWARD)) return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

int cost_shift_for(int64_t max_keys) {
  int64_t cost = ceil_div(max_keys, KT) + 1;
  int s = 0;
  while ((cost >> s) >= 1024) ++s;
  return s;
}

// Key split of the cached path: at most MAX_SPLITS chunks of whole key tiles.
int32_t chunk_keys_for(int64_t max_total) {
  int64_t per = ceil_div(ceil_div(max_total, MAX_SPLITS), KT) * KT;
  if (per < 8 * KT) per = 8 * KT;  // at least 512 keys per split
  return (int32_t)per;
}

// Workspace layout of one call; returns false when the arguments overflow.
bool layout(int fn, const hstu_params_t* p, int32_t B, int64_t Tq, int64_t max_len, WsLayout& w) {
  if (B < 0 || Tq < 0 || max_len < 0) return false;
  const int64_t H = p->num_heads, HD = (int64_t)p->num_heads * p->head_dim;
  const int64_t tiles = ceil_div(Tq, QT) + B;  // bound on sum_b ceil(L_b / QT)
  w.n_chunks = 1;
  w.chunk_keys = 0;
  w.stat_stride = 0;
  w.n_stat_blocks = ceil_div(Tq, KT);           // jagged keys: packed 64-row blocks
  if (fn == HSTU_FN_FULL || fn == HSTU_FN_FULL_BWD) {
    w.max_items = H * tiles;
  } else if (fn == HSTU_FN_MFALCON) {
    w.max_items = H * (tiles + B);
  } else if (fn == HSTU_FN_CACHED || fn == HSTU_FN_MFALCON_CACHED) {
    // splits actually used are ceil(max_len / chunk_keys) <= this bound, which
    // never decreases when max_len grows
    w.chunk_keys = chunk_keys_for(max_len);
    w.n_chunks = (int32_t)std::min<int64_t>(MAX_SPLITS, std::max<int64_t>(1, ceil_div(max_len, 8 * KT)));
    w.max_items = H * tiles * w.n_chunks;
    w.stat_stride = (int32_t)std::max<int64_t>(1, ceil_div(max_len, KT));
    w.n_stat_blocks = (int64_t)B * w.stat_stride;
  } else {
    return false;
  }
  if (w.max_items > INT_MAX / 2) return false;
  w.items_off = ALIGN;
  w.scratch_off = align_up(w.items_off + (size_t)w.max_items * sizeof(WorkItem));
  w.stats_off = align_up(w.scratch_off + (size_t)(B + 1) * sizeof(int32_t));
  w.o_off = align_up(w.stats_off + (size_t)w.n_stat_blocks * 2 * sizeof(int64_t));
  w.total = align_up(w.o_off + (size_t)w.n_chunks * (size_t)Tq * (size_t)HD * sizeof(float));
  w.dout_off = w.rab_off = w.lnp_off = w.ds_off = w.dsp_off = w.total;
  w.ds_blocks = 0;
  w.ln_waves = 0;
  if (fn == HSTU_FN_FULL_BWD) {
    const bool tables = p->pos_tab || p->time_tab;
    const bool affine = p->ln_w || p->ln_b;
    w.ln_waves = (int32_t)std::min<int64_t>(ceil_div(Tq, 16), 1024);  // row blocks of the norm backward
    w.rab_off = align_up(w.dout_off + (size_t)Tq * (size_t)HD * 2);
    w.lnp_off = align_up(w.rab_off + (tables ? (size_t)w.max_items * RAB_SLOTS * sizeof(float) : 0));
    w.total = align_up(w.lnp_off + (affine ? (size_t)2 * w.ln_waves * (size_t)HD * sizeof(float) : 0));
    w.ds_off = w.dsp_off = w.total;
    if (p->head_dim == 128) {
      // dS blocks of 64 x 64: sum_b nb (nb + 1) / 2 <= (n_max + 1) / 2 * sum_b nb,
      // with nb = ceil(L_b / 64) <= L_b / 64 + 1 and n_max = ceil(max_len / 64)
      const int64_t nb_sum = ceil_div(Tq, KT) + B, n_max = ceil_div(max_len, KT);
      if ((double)H * (double)nb_sum * (double)(n_max + 1) > 1e15) return false;
      w.ds_blocks = H * ceil_div(nb_sum * (n_max + 1), 2);
      w.ds_off = align_up(w.dsp_off + (size_t)(B + 1) * sizeof(int64_t));
      w.total = align_up(w.ds_off + (size_t)w.ds_blocks * KT * KT * 2);
    }
  }
  return true;
}

AttnArgs base_args(const hstu_params_t* p, const WsLayout& w, void* ws, int64_t Tq) {
  AttnArgs a = {};
  a.pos_tab = p->pos_tab;
  a.n_pos = p->n_pos;
  a.pos_stride = p->pos_head_stride;
  a.time_tab = p->time_tab;
  a.n_time = p->n_time;
  a.time_stride = p->time_head_stride;
  a.alpha = p->alpha;
  a.norm_n = p->norm_n;
  a.H = p->num_heads;
  a.Tq = Tq;
  a.items = (const WorkItem*)((char*)ws + w.items_off);
  a.count = (const int32_t*)ws;
  a.o = (float*)((char*)ws + w.o_off);
  a.o_chunk_stride = Tq * (int64_t)p->num_heads * p->head_dim;
  a.n_chunks = w.n_chunks;
  a.tstats = (const int64_t*)((char*)ws + w.stats_off);
  a.n_stat_blocks = w.n_stat_blocks;
  a.stat_stride = w.stat_stride;
  return a;
}

SchedArgs sched_args(int mode, const hstu_params_t* p, const WsLayout& w, void* ws, int32_t B,
                     const int32_t* offsets, int64_t max_keys) {
  SchedArgs s = {};
  s.mode = mode;
  s.B = B;
  s.H = p->num_heads;
  s.offsets = offsets;
  s.chunk_keys = w.chunk_keys > 0 ? w.chunk_keys : KT;
  s.cost_shift = cost_shift_for(max_keys);
  s.max_items = w.max_items;
  s.prefix = (int32_t*)((char*)ws + w.scratch_off);
  s.items = (WorkItem*)((char*)ws + w.items_off);
  s.count = (int32_t*)ws;
  s.tstats = (int64_t*)((char*)ws + w.stats_off);
  s.stat_stride = w.stat_stride;
  // ranges are only needed when a time table is present
  s.n_stat_blocks = p->time_tab ? w.n_stat_blocks : 0;
  return s;
}

// bf16 paths with one key split hand the norm a norm-ready store (bf16
// deviations from each head's mean, then the heads' (mean, M2) pairs) in the
// space of the fp32 O buffer, unless the caller asks for the fp32 round trip.
// T * H * d * 2 bytes of deviations keep the pairs 64-byte aligned, and
// 2 + 8 / d <= 4 bytes per element fit in the fp32 buffer.
void norm_ready(const hstu_params_t* p, const WsLayout& w, void* ws, int64_t T, AttnArgs& a, LnArgs& l) {
  if (p->dtype != HSTU_BF16 || w.n_chunks != 1 || (p->flags & HSTU_FLAG_FP32_NORM_INPUT)) return;
  const int64_t HD = (int64_t)p->num_heads * p->head_dim;
  bf16* dev = (bf16*)((char*)ws + w.o_off);
  float* stats = (float*)((char*)ws + w.o_off + (size_t)T * (size_t)HD * 2);
  a.o_dev = dev;
  l.o_dev = dev;
  a.o_stats = stats;
  l.o_stats = stats;
  l.head_dim = p->head_dim;
}

LnArgs ln_args(const hstu_params_t* p, const WsLayout& w, void* ws, const void* u, void* y, int64_t T) {
  LnArgs l = {};
  l.o = (const float*)((char*)ws + w.o_off);
  l.o_chunk_stride = T * (int64_t)p->num_heads * p->head_dim;
  l.u = u;
  l.y = y;
  l.ln_w = p->ln_w;
  l.ln_b = p->ln_b;
  l.eps = p->ln_eps;
  l.HD = p->num_heads * p->head_dim;
  l.T = T;
  l.n_chunks = w.n_chunks;
  return l;
}

static_assert(DBG_FLAG_OFFSET == HSTU_WS_DEBUG_FLAG_OFFSET && DBG_FLAG_OFFSET + 4 <= ALIGN,
              "debug word inside the workspace header, after the item count");
static_assert(DBG_BAD_OFFSETS == HSTU_DEBUG_BAD_OFFSETS && DBG_BAD_LENGTH == HSTU_DEBUG_BAD_LENGTH &&
                  DBG_BAD_CANDIDATES == HSTU_DEBUG_BAD_CANDIDATES && DBG_BAD_CACHE_LEN == HSTU_DEBUG_BAD_CACHE_LEN &&
                  DBG_BAD_PAGE == HSTU_DEBUG_BAD_PAGE,
              "debug bits as declared in hstu.h");

// Debug mode (HSTU_DEBUG=1 in the environment, read at every call).
bool debug_mode() {
  const char* e = std::getenv("HSTU_DEBUG");
  return e && e[0] == '1' && e[1] == 0;
}

// Debug mode: check the device-side index content first; the scheduler then
// reads the result and publishes no work when anything is wrong.
bool debug_check(ValidateArgs v, void* ws, SchedArgs& s, hipStream_t stream) {
  if (!debug_mode()) return true;
  v.flag = (int32_t*)((char*)ws + DBG_FLAG_OFFSET);
  s.debug_flag = v.flag;
  return launch_validate(v, stream) == hipSuccess;
}

ValidateArgs rows_check(int32_t B, const int32_t* offsets, int64_t total, int32_t max_len) {
  ValidateArgs v = {};
  v.B = B;
  v.offsets = offsets;
  v.total = total;
  v.max_len = max_len;
  return v;
}

hstu_status_t run_attention(const hstu_params_t* p, const SchedArgs& s, const AttnArgs& a, int mode,
                            const LnArgs& l, hipStream_t stream) {
  auto mark = [&](int i) {
    hipEvent_t ev = (hipEvent_t)p->timing_events[i];
    return !ev || hipEventRecord(ev, stream) == hipSuccess;
  };
  if (!mark(0) || launch_sched(s, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  if (!mark(1) || launch_attn(a, p->dtype, p->head_dim, mode, s.max_items, stream) != hipSuccess)
    return HSTU_ERR_LAUNCH;
  if (!mark(2) || launch_ln_gate(l, p->dtype, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  if (!mark(3)) return HSTU_ERR_LAUNCH;
  return HSTU_OK;
}

bool any_null(std::initializer_list<const void*> ps) {
  for (const void* x : ps)
    if (!x) return true;
  return false;
}

bool any_misaligned(std::initializer_list<const void*> ps) {
  for (const void* x : ps)
    if (!aligned16(x)) return true;
  return false;
}

}  // namespace

extern "C" {

const char* hstu_status_string(hstu_status_t s) {
  switch (s) {
    case HSTU_OK: return "HSTU_OK";
    case HSTU_ERR_INVALID_ARG: return "HSTU_ERR_INVALID_ARG: invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "HSTU_ERR_UNSUPPORTED: unsupported dtype, head_dim or table size";
    case HSTU_ERR_WORKSPACE: return "HSTU_ERR_WORKSPACE: workspace missing or too small";
    case HSTU_ERR_LAUNCH: return "HSTU_ERR_LAUNCH: kernel launch failed";
  }
  return "HSTU: unknown status";
}

int32_t hstu_version(void) { return VERSION; }

size_t hstu_workspace_size(int32_t fn, const hstu_params_t* params, int32_t batch, int64_t total_q_tokens,
                           int32_t max_len) {
  if (check_params(params) != HSTU_OK) return 0;
  WsLayout w;
  if (!layout(fn, params, batch, total_q_tokens, max_len, w)) return 0;
  return w.total;
}

hstu_status_t hstu_attn_fwd(const hstu_params_t* params, int32_t batch, const int32_t* seq_offsets,
                            int32_t max_len, int64_t total_tokens, const void* q, const void* k,
                            const void* v, const void* u, const int64_t* ts, void* y, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  hstu_status_t st = check_params(params);
  if (st != HSTU_OK) return st;
  if (batch < 0 || total_tokens < 0 || max_len < 0) return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || total_tokens == 0) return HSTU_OK;
  if (any_null({seq_offsets, q, k, v, u, ts, y})) return HSTU_ERR_INVALID_ARG;
  if (any_misaligned({q, k, v, u, ts, y})) return HSTU_ERR_INVALID_ARG;
  WsLayout w;
  if (!layout(HSTU_FN_FULL, params, batch, total_tokens, max_len, w)) return HSTU_ERR_INVALID_ARG;
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return HSTU_ERR_WORKSPACE;

  SchedArgs s = sched_args(MODE_FULL, params, w, ws, batch, seq_offsets, max_len);
  s.ts = ts;
  s.Tk = total_tokens;
  AttnArgs a = base_args(params, w, ws, total_tokens);
  a.q = q;
  a.k = k;
  a.v = v;
  a.ts = ts;
  a.offsets = seq_offsets;
  LnArgs l = ln_args(params, w, ws, u, y, total_tokens);
  norm_ready(params, w, ws, total_tokens, a, l);
  if (!debug_check(rows_check(batch, seq_offsets, total_tokens, max_len), ws, s, stream)) return HSTU_ERR_LAUNCH;
  return run_attention(params, s, a, MODE_FULL, l, stream);
}

hstu_status_t hstu_attn_bwd(const hstu_params_t* params, int32_t batch, const int32_t* seq_offsets,
                            int32_t max_len, int64_t total_tokens, const void* q, const void* k,
                            const void* v, const void* u, const int64_t* ts, const void* dy,
                            const hstu_grads_t* grads, void* ws, size_t ws_bytes, hipStream_t stream) {
  hstu_status_t st = check_params(params);
  if (st != HSTU_OK) return st;
  if (params->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (params->pos_tab && params->n_pos > BWD_MAX_NPOS) return HSTU_ERR_UNSUPPORTED;
  if (batch < 0 || total_tokens < 0 || max_len < 0 || !grads) return HSTU_ERR_INVALID_ARG;
  // saved forward: the workspace holds the norm-ready store of the matching forward call
  const bool saved = (params->flags & HSTU_FLAG_SAVED_FORWARD) != 0;
  if (saved && (params->flags & HSTU_FLAG_FP32_NORM_INPUT)) return HSTU_ERR_INVALID_ARG;
  if ((grads->d_pos_tab && !params->pos_tab) || (grads->d_time_tab && !params->time_tab) ||
      (grads->d_ln_w && !params->ln_w) || (grads->d_ln_b && !params->ln_b))
    return HSTU_ERR_INVALID_ARG;
  if (any_misaligned({grads->d_ln_w, grads->d_ln_b})) return HSTU_ERR_INVALID_ARG;
  if (batch > 0 && total_tokens > 0) {
    if (any_null({seq_offsets, q, k, v, u, ts, dy, grads->dq, grads->dk, grads->dv, grads->du}))
      return HSTU_ERR_INVALID_ARG;
    if (any_misaligned({q, k, v, u, ts, dy, grads->dq, grads->dk, grads->dv, grads->du}))
      return HSTU_ERR_INVALID_ARG;
  }
  WsLayout w;
  if (!layout(HSTU_FN_FULL_BWD, params, batch, total_tokens, max_len, w)) return HSTU_ERR_INVALID_ARG;
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return HSTU_ERR_WORKSPACE;
  const bool empty = batch == 0 || total_tokens == 0;
  auto mark = [&](int i) {
    hipEvent_t ev = (hipEvent_t)params->timing_events[i];
    return !ev || hipEventRecord(ev, stream) == hipSuccess;
  };
  const int HD = params->num_heads * params->head_dim;

  // 1. recompute the attention output O (fp32, in the workspace), unless the
  // forward's norm-ready store is there (the schedule is built either way:
  // the backward kernels read its work list and dS block prefix)
  SchedArgs s = sched_args(MODE_FULL, params, w, ws, batch, seq_offsets, max_len);
  s.ts = ts;
  s.Tk = total_tokens;
  if (w.ds_blocks > 0) s.ds_prefix = (int64_t*)((char*)ws + w.dsp_off);
  AttnArgs a = base_args(params, w, ws, total_tokens);
  a.q = q;
  a.k = k;
  a.v = v;
  a.ts = ts;
  a.offsets = seq_offsets;
  if (!empty && !debug_check(rows_check(batch, seq_offsets, total_tokens, max_len), ws, s, stream))
    return HSTU_ERR_LAUNCH;
  if (!mark(0)) return HSTU_ERR_LAUNCH;
  if (!empty) {
    if (launch_sched(s, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
    if (!saved && launch_attn(a, params->dtype, params->head_dim, MODE_FULL, s.max_items, stream) != hipSuccess)
      return HSTU_ERR_LAUNCH;
  }
  // 2. norm + gating backward: dU, dO, affine gradients
  LnBwdArgs l = {};
  l.o = (const float*)((char*)ws + w.o_off);
  if (saved) {  // the norm-ready store's layout (see norm_ready)
    l.o_dev = (const bf16*)((char*)ws + w.o_off);
    l.o_stats = (const float*)((char*)ws + w.o_off + (size_t)total_tokens * (size_t)HD * 2);
    l.head_dim = params->head_dim;
  }
  l.u = u;
  l.dy = dy;
  l.ln_w = params->ln_w;
  l.ln_b = params->ln_b;
  l.eps = params->ln_eps;
  l.HD = HD;
  l.T = empty ? 0 : total_tokens;
  l.du = grads->du;
  l.dout = (char*)ws + w.dout_off;
  l.part = (params->ln_w || params->ln_b) ? (float*)((char*)ws + w.lnp_off) : nullptr;
  // at least 16 rows per block, at most 1024 blocks (partials) in all
  l.rows_per_block = (int32_t)std::max<int64_t>(16, ceil_div(ceil_div(total_tokens, 1024), 4) * 4);
  l.nwaves = empty ? 0 : (int32_t)ceil_div(total_tokens, l.rows_per_block);
  l.d_ln_w = grads->d_ln_w;
  l.d_ln_b = grads->d_ln_b;
  if (!mark(1) || launch_ln_bwd(l, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  // 3. attention backward
  BwdArgs g = {};
  g.q = q;
  g.k = k;
  g.v = v;
  g.dout = l.dout;
  g.ts = ts;
  g.offsets = seq_offsets;
  g.pos_tab = params->pos_tab;
  g.n_pos = params->n_pos;
  g.pos_stride = params->pos_head_stride;
  g.time_tab = params->time_tab;
  g.n_time = params->n_time;
  g.time_stride = params->time_head_stride;
  g.alpha = params->alpha;
  g.norm_n = params->norm_n;
  g.H = params->num_heads;
  g.T = total_tokens;
  g.items = a.items;
  g.count = a.count;
  g.prefix = s.prefix;
  g.B = batch;
  g.tstats = a.tstats;
  g.n_stat_blocks = a.n_stat_blocks;
  g.dq = grads->dq;
  g.dk = grads->dk;
  g.dv = grads->dv;
  g.rab_part = (float*)((char*)ws + w.rab_off);
  if (w.ds_blocks > 0) {
    g.ds = (bf16*)((char*)ws + w.ds_off);
    g.ds_prefix = s.ds_prefix;
    g.ds_cap = w.ds_blocks;
  }
  if (!mark(2)) return HSTU_ERR_LAUNCH;
  if (!empty && launch_attn_bwd(g, params->head_dim, s.max_items, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  // 4. bias-table gradients
  RabReduceArgs r = {};
  r.part = g.rab_part;
  r.prefix = s.prefix;
  r.B = empty ? 0 : batch;
  r.H = params->num_heads;
  r.d_pos = grads->d_pos_tab;
  r.n_pos = params->n_pos;
  r.pos_stride = params->pos_head_stride;
  r.d_time = grads->d_time_tab;
  r.n_time = params->n_time;
  r.time_stride = params->time_head_stride;
  if (launch_rab_reduce(r, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  if (!mark(3)) return HSTU_ERR_LAUNCH;
  return HSTU_OK;
}

hstu_status_t hstu_mfalcon_fwd(const hstu_params_t* params, int32_t batch, const int32_t* seq_offsets,
                               const int32_t* num_candidates, int32_t max_len, int64_t total_tokens,
                               const void* q, const void* k, const void* v, const void* u,
                               const int64_t* ts, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  hstu_status_t st = check_params(params);
  if (st != HSTU_OK) return st;
  if (batch < 0 || total_tokens < 0 || max_len < 0) return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || total_tokens == 0) return HSTU_OK;
  if (any_null({seq_offsets, num_candidates, q, k, v, u, ts, y})) return HSTU_ERR_INVALID_ARG;
  if (any_misaligned({q, k, v, u, ts, y})) return HSTU_ERR_INVALID_ARG;
  WsLayout w;
  if (!layout(HSTU_FN_MFALCON, params, batch, total_tokens, max_len, w)) return HSTU_ERR_INVALID_ARG;
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return HSTU_ERR_WORKSPACE;

  SchedArgs s = sched_args(MODE_MFALCON, params, w, ws, batch, seq_offsets, max_len);
  s.num_cand = num_candidates;
  s.ts = ts;
  s.Tk = total_tokens;
  AttnArgs a = base_args(params, w, ws, total_tokens);
  a.q = q;
  a.k = k;
  a.v = v;
  a.ts = ts;
  a.offsets = seq_offsets;
  a.num_cand = num_candidates;
  LnArgs l = ln_args(params, w, ws, u, y, total_tokens);
  norm_ready(params, w, ws, total_tokens, a, l);
  ValidateArgs chk = rows_check(batch, seq_offsets, total_tokens, max_len);
  chk.num_cand = num_candidates;
  if (!debug_check(chk, ws, s, stream)) return HSTU_ERR_LAUNCH;
  return run_attention(params, s, a, MODE_MFALCON, l, stream);
}

hstu_status_t hstu_kv_append(const hstu_kv_cache_t* cache, const hstu_params_t* params, int32_t batch,
                             const int32_t* new_offsets, const int32_t* cache_lens, int64_t total_new,
                             const void* k_new, const void* v_new, const int64_t* ts_new,
                             hipStream_t stream) {
  hstu_status_t st = check_params(params);
  if (st != HSTU_OK) return st;
  if (!cache) return HSTU_ERR_INVALID_ARG;
  if (cache->page_size != PAGE) return HSTU_ERR_UNSUPPORTED;
  if (batch < 0 || total_new < 0 || cache->num_pages < 1 || cache->max_pages_per_seq < 1)
    return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || total_new == 0) return HSTU_OK;
  if (any_null({cache->k_pages, cache->v_pages, cache->ts_pages, cache->page_table, new_offsets, cache_lens,
                k_new, v_new, ts_new}))
    return HSTU_ERR_INVALID_ARG;
  if (any_misaligned({cache->k_pages, cache->v_pages, cache->ts_pages, k_new, v_new, ts_new}))
    return HSTU_ERR_INVALID_ARG;
  AppendArgs a = {};
  a.k_new = k_new;
  a.v_new = v_new;
  a.ts_new = ts_new;
  a.offsets = new_offsets;
  a.cache_lens = cache_lens;
  a.k_pages = cache->k_pages;
  a.v_pages = cache->v_pages;
  a.ts_pages = cache->ts_pages;
  a.page_table = cache->page_table;
  a.num_pages = cache->num_pages;
  a.max_pages = cache->max_pages_per_seq;
  a.B = batch;
  a.H = params->num_heads;
  a.D = params->head_dim;
  a.elem_bytes = params->dtype == HSTU_BF16 ? 2 : 4;
  a.T = total_new;
  return launch_kv_append(a, stream) == hipSuccess ? HSTU_OK : HSTU_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// The cached path with its workspace given (ws != nullptr), or with the
// library's per-device scratch (ws == nullptr; no HIP call before the size
// check passes).
hstu_status_t fwd_cached(const hstu_params_t* params, int32_t batch, const int32_t* new_offsets,
                         const int32_t* cache_lens, int32_t max_new, int32_t max_total, int64_t total_new,
                         const void* q_new, const void* u_new, const int64_t* ts_new, const hstu_kv_cache_t* cache,
                         void* y_new, void* ws, size_t ws_bytes, bool use_scratch, hipStream_t stream) {
  hstu_status_t st = check_params(params);
  if (st != HSTU_OK) return st;
  if (!cache) return HSTU_ERR_INVALID_ARG;
  if (cache->page_size != PAGE) return HSTU_ERR_UNSUPPORTED;
  if (batch < 0 || total_new < 0 || max_new < 0 || max_total < 0 || cache->num_pages < 1 ||
      cache->max_pages_per_seq < 1)
    return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || total_new == 0) return HSTU_OK;
  if (any_null({cache->k_pages, cache->v_pages, cache->ts_pages, cache->page_table, new_offsets, cache_lens,
                q_new, u_new, ts_new, y_new}))
    return HSTU_ERR_INVALID_ARG;
  if (any_misaligned({cache->k_pages, cache->v_pages, cache->ts_pages, q_new, u_new, ts_new, y_new}))
    return HSTU_ERR_INVALID_ARG;
  if ((int64_t)cache->max_pages_per_seq * PAGE < max_total) return HSTU_ERR_INVALID_ARG;
  WsLayout w;
  if (!layout(HSTU_FN_CACHED, params, batch, total_new, max_total, w)) return HSTU_ERR_INVALID_ARG;
  if (use_scratch) {
    if (w.total > HSTU_NOALLOC_SCRATCH_BYTES) return HSTU_ERR_WORKSPACE;
    ws = device_scratch();
    if (!ws) return HSTU_ERR_LAUNCH;
    ws_bytes = HSTU_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return HSTU_ERR_WORKSPACE;

  SchedArgs s = sched_args(MODE_CACHED, params, w, ws, batch, new_offsets, w.chunk_keys);
  s.cache_lens = cache_lens;
  s.ts_pages = cache->ts_pages;
  s.page_table = cache->page_table;
  s.num_pages = cache->num_pages;
  s.max_pages = cache->max_pages_per_seq;
  AttnArgs a = base_args(params, w, ws, total_new);
  a.q = q_new;
  a.ts = ts_new;
  a.offsets = new_offsets;
  a.cache_lens = cache_lens;
  a.k_pages = cache->k_pages;
  a.v_pages = cache->v_pages;
  a.ts_pages = cache->ts_pages;
  a.page_table = cache->page_table;
  a.num_pages = cache->num_pages;
  a.max_pages = cache->max_pages_per_seq;
  LnArgs l = ln_args(params, w, ws, u_new, y_new, total_new);
  l.chunk_keys = w.chunk_keys;
  l.mode = MODE_CACHED;
  l.B = batch;
  l.offsets = new_offsets;
  l.cache_lens = cache_lens;
  ValidateArgs chk = rows_check(batch, new_offsets, total_new, max_new);
  chk.cache_lens = cache_lens;
  chk.max_keys = max_total;
  chk.keys_add_rows = 1;
  chk.page_table = cache->page_table;
  chk.num_pages = cache->num_pages;
  chk.max_pages = cache->max_pages_per_seq;
  if (!debug_check(chk, ws, s, stream)) return HSTU_ERR_LAUNCH;
  return run_attention(params, s, a, MODE_CACHED, l, stream);
}

}  // namespace

extern "C" {

hstu_status_t hstu_attn_fwd_cached(const hstu_params_t* params, int32_t batch, const int32_t* new_offsets,
                                   const int32_t* cache_lens, int32_t max_new, int32_t max_total,
                                   int64_t total_new, const void* q_new, const void* u_new,
                                   const int64_t* ts_new, const hstu_kv_cache_t* cache, void* y_new,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_cached(params, batch, new_offsets, cache_lens, max_new, max_total, total_new, q_new, u_new, ts_new,
                    cache, y_new, ws, ws_bytes, false, stream);
}

hstu_status_t hstu_attn_fwd_cached_noalloc(const hstu_params_t* params, int32_t batch,
                                           const int32_t* new_offsets, const int32_t* cache_lens,
                                           int32_t max_new, int32_t max_total, int64_t total_new,
                                           const void* q_new, const void* u_new, const int64_t* ts_new,
                                           const hstu_kv_cache_t* cache, void* y_new, hipStream_t stream) {
  return fwd_cached(params, batch, new_offsets, cache_lens, max_new, max_total, total_new, q_new, u_new, ts_new,
                    cache, y_new, nullptr, 0, true, stream);
}

hstu_status_t hstu_mfalcon_fwd_cached(const hstu_params_t* params, int32_t batch, const int32_t* cand_offsets,
                                      const int32_t* hist_lens, int32_t max_cand, int32_t max_hist,
                                      int64_t total_cand, const void* q, const void* k, const void* v,
                                      const void* u, const int64_t* ts, const hstu_kv_cache_t* cache, void* y,
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  hstu_status_t st = check_params(params);
  if (st != HSTU_OK) return st;
  if (!cache) return HSTU_ERR_INVALID_ARG;
  if (cache->page_size != PAGE) return HSTU_ERR_UNSUPPORTED;
  if (batch < 0 || total_cand < 0 || max_cand < 0 || max_hist < 0 || cache->num_pages < 1 ||
      cache->max_pages_per_seq < 1)
    return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || total_cand == 0) return HSTU_OK;
  if (any_null({cache->k_pages, cache->v_pages, cache->ts_pages, cache->page_table, cand_offsets, hist_lens, q,
                k, v, u, ts, y}))
    return HSTU_ERR_INVALID_ARG;
  if (any_misaligned({cache->k_pages, cache->v_pages, cache->ts_pages, q, k, v, u, ts, y}))
    return HSTU_ERR_INVALID_ARG;
  if ((int64_t)cache->max_pages_per_seq * PAGE < max_hist) return HSTU_ERR_INVALID_ARG;
  WsLayout w;
  if (!layout(HSTU_FN_MFALCON_CACHED, params, batch, total_cand, max_hist, w)) return HSTU_ERR_INVALID_ARG;
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return HSTU_ERR_WORKSPACE;

  SchedArgs s = sched_args(MODE_MFALCON_PAGED, params, w, ws, batch, cand_offsets, w.chunk_keys);
  s.cache_lens = hist_lens;
  s.ts_pages = cache->ts_pages;
  s.page_table = cache->page_table;
  s.num_pages = cache->num_pages;
  s.max_pages = cache->max_pages_per_seq;
  AttnArgs a = base_args(params, w, ws, total_cand);
  a.q = q;
  a.k = k;  // candidates' own keys and values (the self term)
  a.v = v;
  a.ts = ts;
  a.offsets = cand_offsets;
  a.cache_lens = hist_lens;
  a.k_pages = cache->k_pages;
  a.v_pages = cache->v_pages;
  a.ts_pages = cache->ts_pages;
  a.page_table = cache->page_table;
  a.num_pages = cache->num_pages;
  a.max_pages = cache->max_pages_per_seq;
  LnArgs l = ln_args(params, w, ws, u, y, total_cand);
  l.chunk_keys = w.chunk_keys;
  l.mode = MODE_MFALCON_PAGED;
  l.B = batch;
  l.offsets = cand_offsets;
  l.cache_lens = hist_lens;
  ValidateArgs chk = rows_check(batch, cand_offsets, total_cand, max_cand);
  chk.cache_lens = hist_lens;
  chk.max_keys = max_hist;
  chk.page_table = cache->page_table;
  chk.num_pages = cache->num_pages;
  chk.max_pages = cache->max_pages_per_seq;
  if (!debug_check(chk, ws, s, stream)) return HSTU_ERR_LAUNCH;
  return run_attention(params, s, a, MODE_MFALCON_PAGED, l, stream);
}

}  // extern "C"
