// Shared device-side definitions of the HSTU attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// Which attention variant a launch computes. MODE_MFALCON_PAGED scores
// candidates against a history held in the paged KV cache.
enum Mode : int32_t { MODE_FULL = 0, MODE_CACHED = 1, MODE_MFALCON = 2, MODE_MFALCON_PAGED = 3 };

// keys come from the page pool, and the cached path's key splits apply
__host__ __device__ constexpr bool mode_paged(int m) { return m == MODE_CACHED || m == MODE_MFALCON_PAGED; }

// Kinds of query tile: causal rows (full path, cached new tokens, M-FALCON
// history) or M-FALCON candidate rows.
enum Kind : int32_t { KIND_CAUSAL = 0, KIND_CANDIDATE = 1 };

// Tile geometry: a workgroup of 4 wave64s owns QT query rows (32 per wave)
// and walks the keys in tiles of KT.
constexpr int QT = 128;
constexpr int KT = 64;
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int MAX_NPOS = 2048;
constexpr int PAGE = 64;           // page size of the paged KV cache (one key tile)

// One unit of attention work: query rows [q_start, q_start + q_len) of user
// b (local indices), head h, against keys [k_begin, k_end). `chunk` numbers
// the key split of the KV-cache path (0 elsewhere).
// One work item of the attention kernels. The user's first row, row count
// and per-mode count (cached prefix or candidates) ride along, so that a
// workgroup needs no dependent load of the per-user arrays before it starts.
struct WorkItem {
  int32_t b, h, chunk, kind;
  int32_t q_start, q_len, k_begin, k_end;
  int32_t off;   // offsets[b]
  int32_t L;     // offsets[b + 1] - offsets[b]
  int32_t X;     // cache_lens[b] (paged modes), num_cand[b] (M-FALCON), else 0
  int32_t pad;
};

// Workspace layout (bytes), shared by the scheduler, the attention kernel
// and the epilogue: [header 256 B][items][per-user scratch][key timestamp
// ranges][O partials].
struct WsLayout {
  size_t items_off, scratch_off, stats_off, o_off, total;
  int64_t n_stat_blocks;  // key timestamp ranges (pairs of int64)
  int32_t stat_stride;    // cached path: key tiles per user
  int64_t max_items;
  int32_t n_chunks;       // key splits (1 except on the cached path)
  int32_t chunk_keys;     // keys per split (multiple of KT)
  // backward only: dO (bf16), bias-table gradient partials, affine partials,
  // and for d = 128 the dS blocks and their per-user prefix
  size_t dout_off, rab_off, lnp_off, ds_off, dsp_off;
  int64_t ds_blocks;      // capacity of the dS region in 64 x 64 blocks (0: none)
  int32_t ln_waves;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// log2(e) and ln(2) in float
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

}  // namespace hstu
