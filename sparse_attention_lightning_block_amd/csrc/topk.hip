// Per-row top-k selection for gfx950.
//
// Order ([listing] "nvfp4-megamoe-kernel -- .../indexer_score_topk.cu": heap_insert's
// comparator and the final selection sort): score descending, equal scores by
// increasing index; K = min(k, valid) winners, then -1 (the heap's initial -1).
//
// The listing keeps a locked shared-memory heap and a one-thread O(k^2) sort.  Here
// every entry gets a unique 64-bit composite key (order key of the score << 32 |
// ~index) whose unsigned order is exactly the selection order, so selection is a
// radix select with no tie special cases:
//   * a workgroup (1024 threads) loads up to `seg` scores of one row into LDS,
//     finds the K-th largest composite with 11-bit-digit histogram passes over LDS
//     (stopping as soon as the bin of the K-th entry is taken whole), and keeps the
//     entries at or above it;
//   * long rows are cut into segments whose survivors (at most k each) are merged
//     by the same kernel reading candidate lists, level by level, until one
//     workgroup holds every survivor of the row;
//   * the last level sorts its K winners with an LDS bitonic network and writes
//     indices (and scores), padding with -1 (and -inf).
// Everything is deterministic: the result is a function of the composite keys.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 2048;

struct SelKernelArgs {
  // score-mode source
  const float* scores;
  int64_t score_stride;
  const int32_t* valid_lens;
  int64_t first_pos;
  int ratio;
  int n_cols;
  int seg;
  // candidate-mode source: lists [row][list][cap]
  const uint32_t* ckey;
  const int32_t* cidx;
  const int32_t* ccnt;
  int c_nlist;
  int c_cap;
  int c_group;
  int top_k;
  // outputs
  int final_out;
  int32_t* out_idx;
  float* out_scores;
  uint32_t* okey;
  int32_t* oidx;
  int32_t* ocnt;
  int o_nlist;
  int o_cap;
  int lds_entries;
  int sort_n;  // power of two >= top_k (final sort network size)
};

__device__ __forceinline__ int row_valid(const SelKernelArgs& a, int row) {
  int64_t v;
  if (a.valid_lens) {
    v = a.valid_lens[row];
  } else if (a.ratio > 0) {
    v = (a.first_pos + row + 1) / a.ratio;
  } else {
    v = a.n_cols;
  }
  if (v > a.n_cols) v = a.n_cols;
  if (v < 0) v = 0;
  return (int)v;
}

// Sum of v over all threads with a larger thread index (1024-thread block).
__device__ __forceinline__ uint32_t block_excl_suffix(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) wtot[wave] = x;
  __syncthreads();
  uint32_t above = 0;
  for (int w = wave + 1; w < kSelWaves; ++w) above += wtot[w];
  __syncthreads();
  return above + x - v;
}

template <int MODE>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelKernelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t s_wtot[kSelWaves];
  __shared__ uint32_t s_digit, s_gt, s_cnt;
  __shared__ int s_count;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  int32_t* idxs = reinterpret_cast<int32_t*>(keys + a.lds_entries);  // candidate mode only
  unsigned char* tail = smem + (size_t)a.lds_entries * (MODE ? 8 : 4);
  uint32_t* hist = reinterpret_cast<uint32_t*>(tail);
  uint64_t* sortbuf = reinterpret_cast<uint64_t*>(tail + kBins * 4);

  const int row = blockIdx.x;
  const int part = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // ---- load this workgroup's entries into LDS
  int n = 0;
  int base = 0;
  if (MODE == 0) {
    const int valid = row_valid(a, row);
    const int lo = part * a.seg;
    const int hi = min(valid, lo + a.seg);
    n = hi > lo ? hi - lo : 0;
    base = lo;
    const float* src = a.scores + (int64_t)row * a.score_stride + lo;
    for (int i = tid; i < n; i += kSelThreads) keys[i] = ord_key(src[i]);
  } else {
    const int l0 = part * a.c_group;
    const int l1 = min(a.c_nlist, l0 + a.c_group);
    int off = 0;
    for (int l = l0; l < l1; ++l) {
      const int64_t li = (int64_t)row * a.c_nlist + l;
      const int cnt = a.ccnt[li];
      const uint32_t* sk = a.ckey + li * a.c_cap;
      const int32_t* si = a.cidx + li * a.c_cap;
      for (int i = tid; i < cnt; i += kSelThreads) {
        keys[off + i] = sk[i];
        idxs[off + i] = si[i];
      }
      off += cnt;
    }
    n = off;
  }
  __syncthreads();

  auto comp = [&](int i) -> uint64_t {
    const uint32_t ix = MODE == 0 ? (uint32_t)(base + i) : (uint32_t)idxs[i];
    return composite(keys[i], ix);
  };

  const int ksel = min(a.top_k, n);
  uint64_t thr = 0;  // selected: composite >= thr
  if (ksel < n) {
    uint64_t prefix = 0, mask = 0;
    uint32_t rem = (uint32_t)ksel;
    for (int pass = 0; pass < 6; ++pass) {
      const int shift = pass < 5 ? 53 - 11 * pass : 0;
      const uint32_t dmask = pass < 5 ? 0x7ffu : 0x1ffu;
      for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const uint64_t c = comp(i);
        if ((c & mask) == prefix) atomicAdd(&hist[(uint32_t)(c >> shift) & dmask], 1u);
      }
      __syncthreads();
      const uint32_t h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
      const uint32_t above = block_excl_suffix(h0 + h1, s_wtot);
      const uint32_t ge1 = above + h1;
      const uint32_t ge0 = ge1 + h0;
      if (above < rem && ge1 >= rem) {
        s_digit = 2 * tid + 1;
        s_gt = above;
        s_cnt = h1;
      } else if (ge1 < rem && ge0 >= rem) {
        s_digit = 2 * tid;
        s_gt = ge1;
        s_cnt = h0;
      }
      __syncthreads();
      const uint32_t digit = s_digit, gt = s_gt, cnt = s_cnt;
      prefix |= (uint64_t)digit << shift;
      mask |= (uint64_t)dmask << shift;
      rem -= gt;
      if (cnt == rem) break;  // the K-th entry's bin is taken whole
    }
    thr = prefix;
  }

  // ---- keep the entries at or above the threshold
  if (tid == 0) s_count = 0;
  __syncthreads();
  const int64_t olist = (int64_t)row * a.o_nlist + part;
  for (int b0 = 0; b0 < n; b0 += kSelThreads) {
    const int i = b0 + tid;
    uint64_t c = 0;
    bool sel = false;
    if (i < n) {
      c = comp(i);
      sel = c >= thr;
    }
    const uint64_t m = __ballot(sel);
    int wbase = 0;
    if (lane == 0 && m) wbase = atomicAdd(&s_count, __popcll(m));
    wbase = __shfl(wbase, 0);
    if (sel) {
      const int pos = wbase + __popcll(m & ((1ull << lane) - 1ull));
      if (a.final_out) {
        sortbuf[pos] = c;
      } else {
        a.okey[olist * a.o_cap + pos] = (uint32_t)(c >> 32);
        a.oidx[olist * a.o_cap + pos] = (int32_t)(~(uint32_t)c);
      }
    }
  }
  if (!a.final_out) {
    if (tid == 0) a.ocnt[olist] = ksel;
    return;
  }

  // ---- final: sort the winners (descending composite) and write
  __syncthreads();
  const int P2 = a.sort_n;
  for (int i = ksel + tid; i < P2; i += kSelThreads) sortbuf[i] = 0ull;  // pads rank last
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (P2 >> 1); i += kSelThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t x = sortbuf[lo], y = sortbuf[hi];
        const bool desc = (lo & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          sortbuf[lo] = y;
          sortbuf[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  for (int i = tid; i < a.top_k; i += kSelThreads) {
    if (i < ksel) {
      const uint64_t c = sortbuf[i];
      oi[i] = (int32_t)(~(uint32_t)c);
      if (os) os[i] = ord_to_float((uint32_t)(c >> 32));
    } else {
      oi[i] = -1;
      if (os) os[i] = -INFINITY;
    }
  }
}

// ------------------------------------------------------------------ host planning

int max_lds_bytes() {
  static int cached = 0;
  if (cached) return cached;
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0) {
    cached = v;
  } else {
    cached = 65536;
  }
  return cached;
}

static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Sizes from the LDS budget.  max_lds is passed in so the plan can be computed
// (and the workspace sized) without touching the device.
static bool plan_with(int rows, int n_cols, int top_k, int max_lds, SelectPlan* p) {
  const int static_lds = 1024;  // __shared__ scalars and wave totals, rounded up
  const size_t sort_bytes = (size_t)8 * next_pow2(top_k);
  const size_t fixed = (size_t)kBins * 4 + sort_bytes + static_lds;
  if (fixed + 4096 > (size_t)max_lds) return false;
  int seg = 32768;
  while (seg > 1024 && (size_t)4 * seg + fixed > (size_t)max_lds) seg >>= 1;
  int cap = ((int)(((size_t)max_lds - fixed) / 8) / 1024) * 1024;
  if (cap > 32768) cap = 32768;
  p->rows = rows;
  p->n_cols = n_cols;
  p->top_k = top_k;
  if (n_cols <= seg) {
    p->seg = ((n_cols + 255) / 256) * 256;
    if (p->seg < 256) p->seg = 256;
    p->nseg = 1;
  } else {
    p->seg = seg;
    p->nseg = (n_cols + seg - 1) / seg;
  }
  p->kseg = top_k < p->seg ? top_k : p->seg;
  p->cap = cap;
  p->levels = 0;
  if (p->nseg > 1) {
    // merging levels keep top_k entries per list: every list must hold top_k
    if (p->seg < top_k || cap < 2 * top_k) return false;
    int lists = p->nseg;
    while ((int64_t)lists * p->kseg > cap) {
      const int group = cap / p->kseg;
      lists = (lists + group - 1) / group;
      ++p->levels;
    }
    ++p->levels;  // the final merge
  }
  p->lds_score = (size_t)4 * p->seg + fixed - static_lds;
  p->lds_cand = (size_t)8 * cap + fixed - static_lds;
  const size_t list_bytes = (size_t)rows * p->nseg * p->kseg * 8 + (size_t)rows * p->nseg * 4 + 256;
  p->bytes = p->nseg > 1 ? 2 * list_bytes : 0;
  return true;
}

bool plan_select(int rows, int n_cols, int top_k, SelectPlan* p) {
  return plan_with(rows, n_cols, top_k, max_lds_bytes(), p);
}

// Workspace bytes that suffice for any device LDS size the planner accepts
// (64 KiB .. 160 KiB); computed without touching the device.
size_t select_workspace_bytes(int rows, int n_cols, int top_k) {
  size_t best = 0;
  bool any = false;
  for (int lds : {65536, 98304, 131072, 163840}) {
    SelectPlan p;
    if (plan_with(rows, n_cols, top_k, lds, &p)) {
      any = true;
      if (p.bytes > best) best = p.bytes;
    }
  }
  return any ? (best > 0 ? best : 256) : 0;
}

static hipError_t set_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_select(const SelectPlan& p, const float* scores, int64_t score_stride,
                         const int32_t* valid_lens, int64_t first_pos, int ratio, int32_t* out_idx,
                         float* out_scores, void* ws, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  SelKernelArgs a{};
  a.scores = scores;
  a.score_stride = score_stride;
  a.valid_lens = valid_lens;
  a.first_pos = first_pos;
  a.ratio = ratio;
  a.n_cols = p.n_cols;
  a.seg = p.seg;
  a.top_k = p.top_k;
  a.out_idx = out_idx;
  a.out_scores = out_scores;
  a.sort_n = next_pow2(p.top_k);
  hipError_t e;
  if (p.nseg == 1) {
    a.final_out = 1;
    a.o_nlist = 1;
    a.lds_entries = p.seg;
    if ((e = set_lds((const void*)select_kernel<0>, p.lds_score)) != hipSuccess) return e;
    hipLaunchKernelGGL(select_kernel<0>, dim3(p.rows, 1), dim3(kSelThreads), p.lds_score, st, a);
    return hipGetLastError();
  }
  // ping-pong candidate buffers
  const size_t list_entries = (size_t)p.rows * p.nseg * p.kseg;
  unsigned char* w = static_cast<unsigned char*>(ws);
  uint32_t* keyA = reinterpret_cast<uint32_t*>(w);
  int32_t* idxA = reinterpret_cast<int32_t*>(keyA + list_entries);
  int32_t* cntA = reinterpret_cast<int32_t*>(idxA + list_entries);
  unsigned char* wb = w + p.bytes / 2;
  uint32_t* keyB = reinterpret_cast<uint32_t*>(wb);
  int32_t* idxB = reinterpret_cast<int32_t*>(keyB + list_entries);
  int32_t* cntB = reinterpret_cast<int32_t*>(idxB + list_entries);

  // level 0: segments of the score rows
  a.final_out = 0;
  a.okey = keyA;
  a.oidx = idxA;
  a.ocnt = cntA;
  a.o_nlist = p.nseg;
  a.o_cap = p.kseg;
  a.lds_entries = p.seg;
  if ((e = set_lds((const void*)select_kernel<0>, p.lds_score)) != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel<0>, dim3(p.rows, p.nseg), dim3(kSelThreads), p.lds_score, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if ((e = set_lds((const void*)select_kernel<1>, p.lds_cand)) != hipSuccess) return e;
  int lists = p.nseg;
  uint32_t *sk = keyA, *dk = keyB;
  int32_t *si = idxA, *di = idxB, *sc = cntA, *dc = cntB;
  a.lds_entries = p.cap;
  for (;;) {
    SelKernelArgs b = a;
    b.ckey = sk;
    b.cidx = si;
    b.ccnt = sc;
    b.c_nlist = lists;
    b.c_cap = p.kseg;
    if ((int64_t)lists * p.kseg <= p.cap) {
      b.c_group = lists;
      b.final_out = 1;
      b.o_nlist = 1;
      hipLaunchKernelGGL(select_kernel<1>, dim3(p.rows, 1), dim3(kSelThreads), p.lds_cand, st, b);
      return hipGetLastError();
    }
    const int group = p.cap / p.kseg;
    const int out_lists = (lists + group - 1) / group;
    b.c_group = group;
    b.final_out = 0;
    b.okey = dk;
    b.oidx = di;
    b.ocnt = dc;
    b.o_nlist = out_lists;
    b.o_cap = p.kseg;
    hipLaunchKernelGGL(select_kernel<1>, dim3(p.rows, out_lists), dim3(kSelThreads), p.lds_cand, st, b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    lists = out_lists;
    uint32_t* tk = sk; sk = dk; dk = tk;
    int32_t* ti = si; si = di; di = ti;
    int32_t* tc = sc; sc = dc; dc = tc;
  }
}

}  // namespace salb
