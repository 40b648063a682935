// Content checks of the debug mode: with HSTU_DEBUG=1 in the environment, an
// entry point first checks the device-side index data it is given (jagged
// offsets, lengths against their bounds, candidate counts, cache lengths and
// page-table entries) and writes the result into the workspace header; the
// scheduler then publishes an empty work list when anything is wrong, so the
// compute kernels never index with bad content. Without the debug mode such
// content is undefined behaviour.
#include "kernels.h"

namespace hstu {

__global__ __launch_bounds__(256) void validate_kernel(ValidateArgs a) {
  __shared__ int bits;
  const int tid = threadIdx.x;
  if (tid == 0) bits = 0;
  __syncthreads();
  int mine = 0;
  if (tid == 0 && (a.offsets[0] != 0 || (int64_t)a.offsets[a.B] != a.total)) mine |= DBG_BAD_OFFSETS;
  for (int b = tid; b < a.B; b += 256) {
    const int L = a.offsets[b + 1] - a.offsets[b];
    if (L < 0) {
      mine |= DBG_BAD_OFFSETS;
      continue;
    }
    if (L > a.max_len) mine |= DBG_BAD_LENGTH;
    if (a.num_cand) {
      const int m = a.num_cand[b];
      if (m < 0 || m > L) mine |= DBG_BAD_CANDIDATES;
    }
    if (a.cache_lens) {
      const int c = a.cache_lens[b];
      const int64_t keys = (int64_t)c + (a.keys_add_rows ? L : 0);
      if (c < 0 || keys > a.max_keys) {
        mine |= DBG_BAD_CACHE_LEN;
        continue;
      }
      if (a.page_table) {
        // pages holding key positions [first_pos, keys)
        const int64_t first = a.first_pos_is_cache ? c : 0;
        for (int64_t p = first / PAGE; p * PAGE < keys; ++p) {
          if (p >= a.max_pages) {
            mine |= DBG_BAD_PAGE;
            break;
          }
          const int page = a.page_table[(int64_t)b * a.max_pages + p];
          if (page < 0 || page >= a.num_pages) {
            mine |= DBG_BAD_PAGE;
            break;
          }
        }
      }
    }
  }
  if (mine) atomicOr(&bits, mine);
  __syncthreads();
  if (tid == 0) *a.flag = bits;
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
