// Full HSTU layer: f1 product with SiLU, split into U, V, Q, K, the fused
// attention of this library, and the f2 output projection.
//
// Layer structure (pointwise projection with SiLU producing the gate U and
// the attention inputs, gating before the output projection): "How
// Generative Recommenders Are Redefining RecSys at Scale", Takeaways, and
// "Generative recommenders at scale", section "Inside NVIDIA's GPU-native
// stack for HSTU and Semantic IDs".
//
// The two products are plain dense GEMMs. They run on hipBLASLt (f1's SiLU
// is its SWISH epilogue, applied to the fp32 accumulator before the bf16
// store; f1 runs as one product per column block of W1, U, V, Q, K, so that
// each lands packed as [T, H*d], the layout the attention kernels read) or,
// when the caller asks for it, on this library's own MFMA kernel (gemm.hip),
// which does f1 as one product with the SiLU and the split in its epilogue.
//
// hipBLASLt works on column-major matrices. A row-major [R, C] matrix is the
// column-major [C, R] matrix with leading dimension C, so the row-major
// product Y = X W (X [T, k], W [k, m]) is computed as the column-major
// Y^T = W^T X^T with A = W^T ([m, k], ld = row length of W), B = X^T
// ([k, T], ld = k) and D = Y^T ([m, T], ld = m).
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/hstu.h"
#include "gemm.h"

namespace {

constexpr size_t ALIGN = 256;
constexpr size_t GEMM_WS = size_t(64) << 20;  // hipBLASLt workspace inside the caller's workspace
constexpr int MAX_DEVICES = 64;
constexpr size_t MAX_ALGOS = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct LayerLayout {
  size_t uvqk_off[4];  // U, V, Q, K buffers [T, HD] bf16
  size_t a_off;        // attention output [T, HD] bf16
  size_t attn_off;     // workspace of the attention call
  size_t attn_bytes;
  size_t gemm_off;     // hipBLASLt workspace
  size_t total;
};

bool layer_layout(const hstu_params_t* p, int32_t E, int32_t B, int64_t T, int32_t max_len, LayerLayout& w) {
  if (!p || E < 1 || (E % 8) != 0 || B < 0 || T < 0 || max_len < 0) return false;
  if (p->dtype != HSTU_BF16) return false;
  const size_t HD = (size_t)p->num_heads * (size_t)p->head_dim;
  const size_t buf = align_up((size_t)T * HD * 2);
  size_t off = 0;
  for (int i = 0; i < 4; ++i) {
    w.uvqk_off[i] = off;
    off += buf;
  }
  w.a_off = off;
  off += buf;
  w.attn_bytes = hstu_workspace_size(HSTU_FN_FULL, p, B, T, max_len);
  if (w.attn_bytes == 0) return false;
  w.attn_off = off;
  off += align_up(w.attn_bytes);
  w.gemm_off = off;
  off += GEMM_WS;
  w.total = off;
  return true;
}

// ---- hipBLASLt state: one handle per device, chosen algorithms by shape ----

struct AlgoKey {
  int dev;
  int64_t m, n, k, lda, ldb, ldd;
  uint32_t epilogue;
  bool operator==(const AlgoKey& o) const {
    return dev == o.dev && m == o.m && n == o.n && k == o.k && lda == o.lda && ldb == o.ldb && ldd == o.ldd &&
           epilogue == o.epilogue;
  }
};

struct AlgoEntry {
  AlgoKey key;
  hipblasLtMatmulAlgo_t algo;
};

std::mutex g_mu;
hipblasLtHandle_t g_handles[MAX_DEVICES] = {};
std::vector<AlgoEntry> g_algos;

hipblasLtHandle_t handle_for(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
  if (!g_handles[dev] && hipblasLtCreate(&g_handles[dev]) != HIPBLAS_STATUS_SUCCESS) g_handles[dev] = nullptr;
  return g_handles[dev];
}

// RAII holders for the per-call descriptors
struct Desc {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ~Desc() {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (d) hipblasLtMatrixLayoutDestroy(d);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

// Column-major D[m, n] = A[m, k] B[k, n] in bf16 with fp32 accumulation,
// optionally followed by SiLU on the accumulator.
hstu_status_t gemm_bf16(int dev, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, const void* Bm,
                        int64_t ldb, void* D, int64_t ldd, bool silu, void* ws, hipStream_t stream) {
  if (m == 0 || n == 0) return HSTU_OK;
  hipblasLtHandle_t h = handle_for(dev);
  if (!h) return HSTU_ERR_LAUNCH;
  Desc ds;
  const hipblasOperation_t opn = HIPBLAS_OP_N;
  const uint32_t epi = silu ? HIPBLASLT_EPILOGUE_SWISH_EXT : HIPBLASLT_EPILOGUE_DEFAULT;
  if (hipblasLtMatmulDescCreate(&ds.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(ds.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opn, sizeof(opn)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(ds.op, HIPBLASLT_MATMUL_DESC_TRANSB, &opn, sizeof(opn)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(ds.op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ds.a, HIP_R_16BF, m, k, lda) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ds.b, HIP_R_16BF, k, n, ldb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ds.d, HIP_R_16BF, m, n, ldd) != HIPBLAS_STATUS_SUCCESS)
    return HSTU_ERR_LAUNCH;

  const AlgoKey key{dev, m, n, k, lda, ldb, ldd, epi};
  hipblasLtMatmulAlgo_t algo;
  bool found = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    for (const AlgoEntry& e : g_algos)
      if (e.key == key) {
        algo = e.algo;
        found = true;
        break;
      }
  }
  if (!found) {
    const uint64_t max_ws = GEMM_WS;
    if (hipblasLtMatmulPreferenceCreate(&ds.pref) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulPreferenceSetAttribute(ds.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws,
                                              sizeof(max_ws)) != HIPBLAS_STATUS_SUCCESS)
      return HSTU_ERR_LAUNCH;
    hipblasLtMatmulHeuristicResult_t res[1];
    int got = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(h, ds.op, ds.a, ds.b, ds.d, ds.d, ds.pref, 1, res, &got) !=
            HIPBLAS_STATUS_SUCCESS ||
        got < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS || res[0].workspaceSize > GEMM_WS)
      return HSTU_ERR_UNSUPPORTED;
    algo = res[0].algo;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_algos.size() >= MAX_ALGOS) g_algos.erase(g_algos.begin());
    g_algos.push_back({key, algo});
  }
  const float one = 1.0f, zero = 0.0f;
  if (hipblasLtMatmul(h, ds.op, &one, A, ds.a, Bm, ds.b, &zero, D, ds.d, D, ds.d, &algo, ws, GEMM_WS, stream) !=
      HIPBLAS_STATUS_SUCCESS)
    return HSTU_ERR_LAUNCH;
  return HSTU_OK;
}

}  // namespace

extern "C" {

size_t hstu_layer_workspace_size(const hstu_params_t* params, int32_t embed_dim, int32_t batch,
                                 int64_t total_tokens, int32_t max_len) {
  LayerLayout w;
  if (!layer_layout(params, embed_dim, batch, total_tokens, max_len, w)) return 0;
  return w.total;
}

hstu_status_t hstu_layer_fwd(const hstu_params_t* params, const hstu_layer_weights_t* weights,
                             int32_t batch, const int32_t* seq_offsets, int32_t max_len,
                             int64_t total_tokens, const void* x, const int64_t* ts, void* out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!params || !weights) return HSTU_ERR_INVALID_ARG;
  if (params->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (batch < 0 || total_tokens < 0 || max_len < 0 || weights->embed_dim < 1 || (weights->embed_dim % 8) != 0)
    return HSTU_ERR_INVALID_ARG;
  const int32_t prod = weights->products;
  if (prod != HSTU_PRODUCTS_HIPBLASLT && prod != HSTU_PRODUCTS_OWN && prod != HSTU_PRODUCTS_AUTO)
    return HSTU_ERR_INVALID_ARG;
  bool own_fits;
  {
    const int64_t hd = (int64_t)params->num_heads * params->head_dim, e = weights->embed_dim;
    own_fits = (4 * hd) % 256 == 0 && e % 256 == 0 && e % 64 == 0 && hd % 64 == 0;
  }
  if (prod == HSTU_PRODUCTS_OWN && !own_fits) return HSTU_ERR_UNSUPPORTED;
  // which product runs where: f1 on the own kernel for OWN, and for AUTO
  // when it fits; f2 on the own kernel for OWN only
  const bool own_f1 = prod == HSTU_PRODUCTS_OWN || (prod == HSTU_PRODUCTS_AUTO && own_fits);
  const bool own_f2 = prod == HSTU_PRODUCTS_OWN;
  // the attention checks the remaining parameters; run them before anything is launched
  if (hstu_workspace_size(HSTU_FN_FULL, params, batch, total_tokens, max_len) == 0) return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || total_tokens == 0) return HSTU_OK;
  if (!seq_offsets || !x || !ts || !out || !weights->w1 || !weights->w2) return HSTU_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(ts) || !aligned16(out) || !aligned16(weights->w1) || !aligned16(weights->w2))
    return HSTU_ERR_INVALID_ARG;
  LayerLayout w;
  if (!layer_layout(params, weights->embed_dim, batch, total_tokens, max_len, w)) return HSTU_ERR_INVALID_ARG;
  if (!ws || ws_bytes < w.total || !aligned16(ws)) return HSTU_ERR_WORKSPACE;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HSTU_ERR_LAUNCH;
  auto mark = [&](int i) {
    hipEvent_t ev = (hipEvent_t)params->timing_events[i];
    return !ev || hipEventRecord(ev, stream) == hipSuccess;
  };
  char* base = (char*)ws;
  const int64_t E = weights->embed_dim;
  const int64_t HD = (int64_t)params->num_heads * params->head_dim;
  const int64_t T = total_tokens;
  void* bufs[4];
  for (int i = 0; i < 4; ++i) bufs[i] = base + w.uvqk_off[i];
  void* a = base + w.a_off;
  void* gws = base + w.gemm_off;

  // f1 with SiLU into U, V, Q, K
  if (!mark(0)) return HSTU_ERR_LAUNCH;
  const char* w1 = (const char*)weights->w1;
  if (own_f1) {
    // one product; the epilogue writes column block i to buffer i (the
    // buffers sit buf_elems apart in the workspace)
    hstu::GemmArgs g = {};
    g.a = (const hstu::bf16*)x;
    g.b = (const hstu::bf16*)weights->w1;
    g.c = (hstu::bf16*)bufs[0];
    g.M = T;
    g.N = (int32_t)(4 * HD);
    g.K = (int32_t)E;
    g.mt_count = (T + 255) / 256;
    g.epilogue = hstu::GEMM_EPI_SILU_SPLIT;
    g.split = (int32_t)HD;
    g.split_stride = (int64_t)(w.uvqk_off[1] - w.uvqk_off[0]) / 2;
    if (hstu::launch_gemm(g, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  } else {
    for (int i = 0; i < 4; ++i) {
      hstu_status_t st =
          gemm_bf16(dev, HD, T, E, w1 + (size_t)i * HD * 2, 4 * HD, x, E, bufs[i], HD, true, gws, stream);
      if (st != HSTU_OK) return st;
    }
  }
  if (!mark(1)) return HSTU_ERR_LAUNCH;

  hstu_params_t pa = *params;
  for (int i = 0; i < 4; ++i) pa.timing_events[i] = nullptr;
  hstu_status_t st = hstu_attn_fwd(&pa, batch, seq_offsets, max_len, total_tokens, bufs[2], bufs[3], bufs[1],
                                   bufs[0], ts, a, base + w.attn_off, w.attn_bytes, stream);
  if (st != HSTU_OK) return st;
  if (!mark(2)) return HSTU_ERR_LAUNCH;

  // f2: out = A W2
  if (own_f2) {
    hstu::GemmArgs g = {};
    g.a = (const hstu::bf16*)a;
    g.b = (const hstu::bf16*)weights->w2;
    g.c = (hstu::bf16*)out;
    g.M = T;
    g.N = (int32_t)E;
    g.K = (int32_t)HD;
    g.mt_count = (T + 255) / 256;
    g.epilogue = hstu::GEMM_EPI_NONE;
    g.split = (int32_t)E;
    g.split_stride = 0;
    if (hstu::launch_gemm(g, stream) != hipSuccess) return HSTU_ERR_LAUNCH;
  } else {
    st = gemm_bf16(dev, E, T, HD, weights->w2, E, a, HD, out, E, false, gws, stream);
    if (st != HSTU_OK) return st;
  }
  if (!mark(3)) return HSTU_ERR_LAUNCH;
  return HSTU_OK;
}

}  // extern "C"

extern "C" hstu_status_t hstu_matmul_bf16(int64_t M, int32_t N, int32_t K, const void* a, const void* b, void* c,
                                          int32_t epilogue, int32_t split_width, hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0) return HSTU_ERR_INVALID_ARG;
  if (epilogue != HSTU_EPI_NONE && epilogue != HSTU_EPI_SILU_SPLIT) return HSTU_ERR_INVALID_ARG;
  if (N % 256 != 0 || K % 64 != 0) return HSTU_ERR_UNSUPPORTED;
  if (epilogue == HSTU_EPI_SILU_SPLIT && (split_width <= 0 || split_width % 32 != 0 || N % split_width != 0))
    return HSTU_ERR_UNSUPPORTED;
  if ((M + 255) / 256 * (int64_t)(N / 256) > INT32_MAX) return HSTU_ERR_UNSUPPORTED;
  if (M == 0) return HSTU_OK;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || !aligned16(c)) return HSTU_ERR_INVALID_ARG;
  hstu::GemmArgs g = {};
  g.a = (const hstu::bf16*)a;
  g.b = (const hstu::bf16*)b;
  g.c = (hstu::bf16*)c;
  g.M = M;
  g.N = N;
  g.K = K;
  g.mt_count = (M + 255) / 256;
  g.epilogue = epilogue == HSTU_EPI_SILU_SPLIT ? hstu::GEMM_EPI_SILU_SPLIT : hstu::GEMM_EPI_NONE;
  g.split = epilogue == HSTU_EPI_SILU_SPLIT ? split_width : N;
  g.split_stride = M * (int64_t)g.split;
  return hstu::launch_gemm(g, stream) == hipSuccess ? HSTU_OK : HSTU_ERR_LAUNCH;
}
