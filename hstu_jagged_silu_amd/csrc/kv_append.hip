// Paged KV append for the KV-cache delta path.
#include "kernels.h"

namespace hstu {

// Paged KV append: new token m of user b goes to logical position
// cache_lens[b] + m, i.e. page page_table[b][pos / 64], slot pos % 64 (the
// append operation of the paged GPU table, page "recomendador-generativo-
// hstu-dynamo-triton", section "Como o recomendador generativo HSTU reutiliza
// o histórico"). One thread moves 16 bytes of one head's K and V row.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int cpr = a.D * a.elem_bytes / 16;               // 16-byte chunks per head row
  const int64_t per_tok = (int64_t)a.H * cpr;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = gid / per_tok;
  if (t >= a.T) return;
  const int rem = (int)(gid % per_tok);
  const int h = rem / cpr, c = rem % cpr;
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.offsets[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int pos = a.cache_lens[b] + (int)(t - a.offsets[b]);
  if (pos < 0 || pos / PAGE >= a.max_pages) return;
  const int page = a.page_table[(int64_t)b * a.max_pages + pos / PAGE];
  if (page < 0 || page >= a.num_pages) return;
  const int slot = pos % PAGE;
  const int64_t src = ((t * a.H + h) * a.D) * a.elem_bytes + c * 16;
  const int64_t dst = ((((int64_t)page * a.H + h) * PAGE + slot) * a.D) * a.elem_bytes + c * 16;
  *(i32x4*)((char*)a.k_pages + dst) = *(const i32x4*)((const char*)a.k_new + src);
  *(i32x4*)((char*)a.v_pages + dst) = *(const i32x4*)((const char*)a.v_new + src);
  if (h == 0 && c == 0) a.ts_pages[(int64_t)page * PAGE + slot] = a.ts_new[t];
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t n = a.T * a.H * (a.D * a.elem_bytes / 16);
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
