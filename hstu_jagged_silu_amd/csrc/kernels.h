// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include "common.h"

namespace hstu {

// Arguments of the fused attention kernel (passed by value).
struct AttnArgs {
  const void* q;                 // [Tq, H, D] query rows
  const void* k;                 // [Tk, H, D] keys (jagged variants)
  const void* v;
  const int64_t* ts;             // [Tq] query timestamps (also key timestamps when jagged)
  const int32_t* offsets;        // [B+1] query row offsets
  const int32_t* cache_lens;     // [B] cached path
  const int32_t* num_cand;       // [B] M-FALCON
  const void* k_pages;           // [P, H, 64, D] cached path
  const void* v_pages;
  const int64_t* ts_pages;       // [P, 64]
  const int32_t* page_table;     // [B, max_pages]
  int32_t num_pages, max_pages;
  const float* pos_tab;
  int32_t n_pos, pos_stride;
  const float* time_tab;
  int32_t n_time, time_stride;
  float alpha;
  int32_t norm_n;
  int32_t H;
  int64_t Tq;                    // number of query rows
  const WorkItem* items;
  const int32_t* count;          // number of valid items
  float* o;                      // [n_chunks][Tq][H*D] fp32, scaled attention output
  int64_t o_chunk_stride;        // elements between key splits
  int32_t n_chunks;              // key splits the O buffer holds
  // Norm-ready store (bf16, one key split): when o_dev is set, the kernel
  // writes, instead of o, each (row, head)'s deviations from its head mean
  // as bf16 [Tq][H*D] and the head's (mean, sum of squared deviations) as
  // float2 [Tq][H], both from the fp32 accumulators
  bf16* o_dev;
  float* o_stats;
  // key timestamp range per 64-key block: jagged variants index packed rows
  // (block i = rows [64i, 64i + 64)), the cached path indexes [b][key tile]
  const int64_t* tstats;         // pairs (min, max)
  int64_t n_stat_blocks;         // jagged: number of packed blocks
  int32_t stat_stride;           // cached: key tiles per user
};

// Arguments of the single-workgroup jagged tile scheduler.
struct SchedArgs {
  int32_t mode;
  int32_t B, H;
  const int32_t* offsets;        // [B+1] query rows
  const int32_t* cache_lens;     // cached path
  const int32_t* num_cand;       // M-FALCON
  int32_t chunk_keys;            // key split (cached path), multiple of KT
  int32_t cost_shift;            // cost bin = min(cost >> shift, NBINS - 1)
  const int32_t* debug_flag;     // debug mode: nonzero content-check bits -> empty work list
  int64_t max_items;
  int32_t* prefix;               // [B+1] scratch
  WorkItem* items;
  int32_t* count;
  // key timestamp ranges, computed by the workgroups after the first
  int64_t* tstats;
  int64_t n_stat_blocks;         // blocks to fill
  const int64_t* ts;             // jagged: key timestamps [Tk]
  int64_t Tk;                    // jagged: key rows
  const int64_t* ts_pages;       // cached
  const int32_t* page_table;
  int32_t num_pages, max_pages, stat_stride;
  // backward, d = 128: per-user prefix of the dS blocks (64 x 64, causal:
  // nb (nb + 1) / 2 per head, nb = ceil(L / 64)), [B+1]; null elsewhere
  int64_t* ds_prefix;
};

// Arguments of the LayerNorm + U gating epilogue (sums key splits first).
struct LnArgs {
  const float* o;                // [n_chunks][T][HD]
  // norm-ready input (instead of o): bf16 deviations [T][HD] and per-head
  // (mean, sum of squared deviations) [T][H] with heads of head_dim values
  const bf16* o_dev;
  const float* o_stats;
  int32_t head_dim;
  int64_t o_chunk_stride;
  const void* u;                 // [T, HD]
  void* y;                       // [T, HD]
  const float* ln_w;
  const float* ln_b;
  float eps;
  int32_t HD;
  int64_t T;
  // split bookkeeping (paged paths); chunk_keys == 0 means one split
  int32_t chunk_keys;
  int32_t mode;                  // MODE_CACHED or MODE_MFALCON_PAGED when chunk_keys > 0
  int32_t n_chunks;
  int32_t B;
  const int32_t* offsets;
  const int32_t* cache_lens;
};

// Debug-mode content checks (HSTU_DEBUG=1): bits written to the workspace
// header word at DBG_FLAG_OFFSET (0 when the content is valid).
constexpr int DBG_FLAG_OFFSET = 128;
enum DebugBits : int32_t {
  DBG_BAD_OFFSETS = 1,     // offsets[0] != 0, a decreasing pair, or offsets[B] != total rows
  DBG_BAD_LENGTH = 2,      // a length above max_len
  DBG_BAD_CANDIDATES = 4,  // num_candidates[b] outside [0, L_b]
  DBG_BAD_CACHE_LEN = 8,   // a cache (history) length below 0 or keys above their bound
  DBG_BAD_PAGE = 16,       // a needed page missing from the table or outside the pool
};
struct ValidateArgs {
  int32_t B;
  const int32_t* offsets;        // [B+1] rows of this call
  int64_t total;                 // expected offsets[B]
  int32_t max_len;               // bound on every length
  const int32_t* num_cand;       // M-FALCON counts, or null
  const int32_t* cache_lens;     // cache (history) lengths, or null
  int64_t max_keys;              // bound on the keys per user
  int32_t keys_add_rows;         // keys = cache_len + L (cached, append) or cache_len (paged M-FALCON)
  int32_t first_pos_is_cache;    // pages checked from position cache_len (append) or 0 (forward)
  const int32_t* page_table;     // [B, max_pages], or null
  int32_t num_pages, max_pages;
  int32_t* flag;                 // result word
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* ts_new;
  const int32_t* offsets;        // [B+1] new rows
  const int32_t* cache_lens;     // [B]
  void* k_pages;
  void* v_pages;
  int64_t* ts_pages;
  const int32_t* page_table;
  int32_t num_pages, max_pages;
  int32_t B, H, D, elem_bytes;
  int64_t T;
};

// Backward of the full causal path (bf16). The bias-table gradients of each
// work item go to rab_part[canonical item][RAB_SLOTS] (position buckets at
// [0, n_pos), time buckets at [BWD_MAX_NPOS, BWD_MAX_NPOS + 64)) and are
// summed in a fixed order by the reduce kernel, so results are reproducible.
constexpr int BWD_MAX_NPOS = 512;
constexpr int RAB_SLOTS = BWD_MAX_NPOS + 64;

struct BwdArgs {
  const void* q;                 // [T, H, D]
  const void* k;
  const void* v;
  const void* dout;              // [T, H, D] bf16: gradient reaching the attention output
  const int64_t* ts;             // [T]
  const int32_t* offsets;        // [B+1]
  const float* pos_tab;
  int32_t n_pos, pos_stride;
  const float* time_tab;
  int32_t n_time, time_stride;
  float alpha;
  int32_t norm_n;
  int32_t H;
  int64_t T;
  const WorkItem* items;         // scheduler output of the full path
  const int32_t* count;
  const int32_t* prefix;         // [B+1] scheduler's item prefix over users (H items per query tile)
  int32_t B;
  const int64_t* tstats;         // key timestamp ranges per packed 64-row block
  int64_t n_stat_blocks;
  void* dq;                      // [T, H, D] bf16
  void* dk;
  void* dv;
  float* rab_part;               // [items][RAB_SLOTS]
  // d = 128: dS of every causal 64 x 64 (key, query) block, bf16 [key][query],
  // written by the dK/dV kernel and read by the dQ kernel; block (kt, qt) of
  // user b and head h at (H * ds_prefix[b] + h * nb (nb + 1) / 2 + qt (qt + 1)
  // / 2 + kt) * 4096 elements
  bf16* ds;
  const int64_t* ds_prefix;
  int64_t ds_cap;                // blocks the region holds; a block past it is neither written nor read
};

struct RabReduceArgs {
  const float* part;             // [H * tiles][RAB_SLOTS], head-major
  const int32_t* prefix;         // scheduler's item prefix; prefix[B] / H = tiles
  int32_t B, H;
  float* d_pos;                  // like pos_tab: [n_pos] shared or [H][pos_stride]
  int32_t n_pos, pos_stride;
  float* d_time;
  int32_t n_time, time_stride;
};

// LayerNorm + U gating backward: per row dU and the gradient reaching O
// (bf16), plus per-wave partial sums of the affine gradients.
struct LnBwdArgs {
  const float* o;                // [T, HD] attention output before the norm
  // or, when o_dev is set, the forward's norm-ready store: bf16 deviations
  // from each head's mean [T, HD] and per-head (mean, M2) [T, H]
  const bf16* o_dev;
  const float* o_stats;
  int32_t head_dim;
  const void* u;
  const void* dy;
  const float* ln_w;
  const float* ln_b;
  float eps;
  int32_t HD;
  int64_t T;
  void* du;                      // [T, HD], dtype of u
  void* dout;                    // [T, HD] bf16
  float* part;                   // [2][nwaves][HD] (dw, db), or null
  int32_t nwaves;                // row blocks, one partial each
  int32_t rows_per_block;
  float* d_ln_w;
  float* d_ln_b;
};

hipError_t launch_sched(const SchedArgs& a, hipStream_t s);  // scheduler + key timestamp ranges
hipError_t launch_validate(const ValidateArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int dtype, int D, int mode, int64_t grid, hipStream_t s);
hipError_t launch_ln_gate(const LnArgs& a, int dtype, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_ln_bwd(const LnBwdArgs& a, hipStream_t s);       // rows, then the affine reduce
hipError_t launch_attn_bwd(const BwdArgs& a, int D, int64_t grid, hipStream_t s);
hipError_t launch_rab_reduce(const RabReduceArgs& a, hipStream_t s);

}  // namespace hstu
