// Opt-in check of the paged-pool metadata before any scorer runs: every valid length
// lies in [0, cap] and every block-table entry a row's valid keys resolve through names
// a page of the pool.  The scorers never check these (out-of-range data would make them
// read outside the pool), so a caller that cannot vouch for its tables asks for this
// check first.  The error convention follows [qsa.rs] "metrale_model_layers/layers/
// ops/qsa.rs": launchers return a Result instead of failing later.
#include <hip/hip_runtime.h>

#include <climits>

#include "internal.hpp"

namespace salb {

// One workgroup.  out[0] = first row whose valid length is outside [0, cap] (-1 if
// none); out[1] = first (row * max_lb + logical block) whose page id is outside
// [0, n_pages) among the blocks the row's valid keys use (-1 if none).  Blocks of a
// row with a bad valid length are checked up to max_lb.
__global__ __launch_bounds__(1024) void validate_pages_kernel(const int32_t* bt, int64_t bt_stride,
                                                              const int32_t* valid_lens, int T, int max_lb,
                                                              int epb, int cap, int n_pages, int64_t* out) {
  __shared__ unsigned long long s_row, s_blk;
  if (threadIdx.x == 0) {
    s_row = ULLONG_MAX;
    s_blk = ULLONG_MAX;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    const int v = valid_lens[t];
    if (v < 0 || v > cap) atomicMin(&s_row, (unsigned long long)t);
  }
  const int64_t total = (int64_t)T * max_lb;
  for (int64_t i = threadIdx.x; i < total; i += blockDim.x) {
    const int t = (int)(i / max_lb), lb = (int)(i % max_lb);
    const int v = valid_lens[t];
    const int used = v < 0 ? 0 : (v > cap ? max_lb : (int)(((int64_t)v + epb - 1) / epb));
    if (lb < used) {
      const int p = bt[(int64_t)t * bt_stride + lb];
      if (p < 0 || p >= n_pages) atomicMin(&s_blk, (unsigned long long)i);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    out[0] = s_row == ULLONG_MAX ? -1 : (int64_t)s_row;
    out[1] = s_blk == ULLONG_MAX ? -1 : (int64_t)s_blk;
  }
}

hipError_t validate_pages(const int32_t* bt, int64_t bt_stride, const int32_t* valid_lens, int T, int max_lb, int epb,
                          int cap, int n_pages, int64_t* dev_status, int64_t host_status[2], hipStream_t st) {
  hipLaunchKernelGGL(validate_pages_kernel, dim3(1), dim3(1024), 0, st, bt, bt_stride, valid_lens, T, max_lb, epb,
                     cap, n_pages, dev_status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(host_status, dev_status, 2 * sizeof(int64_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace salb
