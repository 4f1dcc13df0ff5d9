// Per-row top-k selection for gfx950.
//
// Order ([listing] "nvfp4-megamoe-kernel -- .../indexer_score_topk.cu": heap_insert's
// comparator and the final selection sort): score descending, equal scores by
// increasing index; K = min(k, valid) winners, then -1 (the heap's initial -1).
//
// The listing keeps a locked shared-memory heap per query and sorts it with one
// thread.  Here every entry gets a unique 64-bit composite key (order key of the
// score << 32 | ~index) whose unsigned order is exactly the selection order, so
// the selection is a radix select with no tie special cases, and the result is a
// function of the composites alone (deterministic whatever the thread schedule).
//
//   * rows of at most kRowMax entries: one 256-thread workgroup per row holds the
//     row in registers, finds the K-th composite with 12-bit-digit LDS histogram
//     passes (stopping once the digit bin of the K-th entry is taken whole),
//     gathers the winners and sorts them;
//   * longer rows run as a pipeline of launches (kernel boundaries order them; no
//     grid-wide fences, which write back the whole L2 on this chip): every
//     workgroup of a (chunk, row) grid adds its chunk's LDS histogram of the top 12
//     order-key bits into one of eight global copies (one per XCD, so contended
//     atomics stay in one L2); one workgroup per row sums the copies and finds the
//     bin holding the K-th entry; the (chunk, row) grid then writes every entry at
//     or above that bin to the chunk's own candidate slots; one workgroup per row
//     gathers those candidates (about K plus one bin's worth) into LDS, selects
//     the K winners exactly and sorts them.
//   * the sort buckets the winners on the 12 highest bits where they differ and
//     ranks each against its bucket (a sorting network if a bucket is crowded).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kDigit = 12;
constexpr int kBins = 1 << kDigit;                   // 4096 histogram bins
constexpr int kBinsPerThread = kBins / kSelThreads;  // 16
constexpr int kTopShift = 64 - kDigit;               // first digit: the score's top 12 order bits
constexpr int kRowMax = 32 * kSelThreads;            // 8192: one-workgroup rows
constexpr int kBucketMax = 48;                       // crowded bucket: sorting network instead
constexpr int kHistCopies = 8;                       // one global histogram per XCD

struct RowInfo {
  uint32_t bin;    // bin of the K-th entry (0 when every entry wins)
  uint32_t above;  // entries in higher bins
  uint32_t cnt;    // entries in that bin
  uint32_t pad;
};

struct SelArgs {
  const float* scores;
  int64_t score_stride;
  const int32_t* valid_lens;
  int64_t first_pos;
  int ratio;
  int n_cols;
  int top_k;
  int32_t* out_idx;
  float* out_scores;
  // long-row pipeline
  int chunk;         // entries per chunk workgroup
  int chunks;        // chunks per row
  int cand_lds;      // candidates the final workgroup can hold in LDS
  uint32_t* ghist;   // [rows][kHistCopies][kBins]
  RowInfo* info;     // [rows]
  uint32_t* ccnt;    // [rows][chunks] candidates per chunk
  uint64_t* cand;    // [rows][chunks * chunk] candidate slots, chunk by chunk
};

__device__ __forceinline__ int row_valid(const SelArgs& a, int row) {
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

struct SelShared {
  uint32_t wsum[kSelWaves];
  uint64_t wred[2 * kSelWaves];
  uint32_t digit, gt, cnt;
  uint32_t fill;  // append counter of the candidate gather
};

// Sum of v over the threads with a larger index.  Two calls must be separated by a
// barrier after the first call's result is used.
__device__ __forceinline__ uint32_t block_suffix(uint32_t v, SelShared& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) sh.wsum[wave] = x;
  __syncthreads();
  uint32_t above = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) above += w > wave ? sh.wsum[w] : 0u;
  return above + x - v;
}

// Block-wide maximum and minimum (same barrier rule as block_suffix).
__device__ __forceinline__ void block_minmax(uint64_t& mx, uint64_t& mn, SelShared& sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t a = __shfl_xor(mx, off);
    const uint64_t b = __shfl_xor(mn, off);
    mx = a > mx ? a : mx;
    mn = b < mn ? b : mn;
  }
  if ((threadIdx.x & 63) == 0) {
    sh.wred[threadIdx.x >> 6] = mx;
    sh.wred[kSelWaves + (threadIdx.x >> 6)] = mn;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint64_t a = sh.wred[w], b = sh.wred[kSelWaves + w];
    mx = a > mx ? a : mx;
    mn = b < mn ? b : mn;
  }
}

__device__ __forceinline__ void load_bins(const uint32_t* hist, uint32_t (&h)[kBinsPerThread]) {
  const uint4* p = reinterpret_cast<const uint4*>(hist + threadIdx.x * kBinsPerThread);
#pragma unroll
  for (int j = 0; j < kBinsPerThread / 4; ++j) {
    const uint4 v = p[j];
    h[4 * j] = v.x;
    h[4 * j + 1] = v.y;
    h[4 * j + 2] = v.z;
    h[4 * j + 3] = v.w;
  }
}

__device__ __forceinline__ void clear_bins(uint32_t* hist) {
  uint4* p = reinterpret_cast<uint4*>(hist);
  for (int j = threadIdx.x; j < kBins / 4; j += kSelThreads) p[j] = make_uint4(0u, 0u, 0u, 0u);
}

// Digit search over a 4096-bin histogram (bins are owned 16 per thread, in
// order): the bin holding the rem-th largest counted entry, the count above it and
// its own count land in sh.digit / sh.gt / sh.cnt.  Requires 1 <= rem <= total.
__device__ __forceinline__ void find_digit(const uint32_t (&h)[kBinsPerThread], uint32_t rem, SelShared& sh) {
  uint32_t own = 0;
#pragma unroll
  for (int q = 0; q < kBinsPerThread; ++q) own += h[q];
  uint32_t ge = block_suffix(own, sh);
#pragma unroll
  for (int q = kBinsPerThread - 1; q >= 0; --q) {
    if (ge < rem && ge + h[q] >= rem) {
      sh.digit = threadIdx.x * kBinsPerThread + q;
      sh.gt = ge;
      sh.cnt = h[q];
    }
    ge += h[q];
  }
  __syncthreads();
}

// Radix select: the threshold thr such that exactly `rem` of the composites that
// agree with `prefix` on the bits of `mask` are >= thr (those above the prefix are
// already counted out by the caller).  `each(f)` calls f(c) on every composite
// this thread owns.  Digits are 12 bits wide, from bit `top` down.
template <typename Each>
__device__ uint64_t radix_select(Each each, uint64_t prefix, uint64_t mask, uint32_t rem, int top,
                                 uint32_t* hist, SelShared& sh) {
  for (;;) {
    const int width = top + 1 < kDigit ? top + 1 : kDigit;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    clear_bins(hist);
    __syncthreads();
    each([&](uint64_t c) {
      if ((c & mask) == prefix) atomicAdd(&hist[(uint32_t)(c >> shift) & dmask], 1u);
    });
    __syncthreads();
    uint32_t h[kBinsPerThread];
    load_bins(hist, h);
    find_digit(h, rem, sh);
    const uint32_t digit = sh.digit, gt = sh.gt, cnt = sh.cnt;
    prefix |= (uint64_t)digit << shift;
    mask |= (uint64_t)dmask << shift;
    rem -= gt;
    if (cnt == rem || shift == 0) return prefix;
    top = shift - 1;
  }
}

// Descending bitonic sort of buf[0, n2) (n2 a power of two) by the whole block.
__device__ void bitonic_desc(uint64_t* buf, int n2) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += kSelThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t x = buf[lo], y = buf[hi];
        const bool desc = (lo & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          buf[lo] = y;
          buf[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Sorts the K winners in sortbuf[0, K) (capacity pow2_at_least(K)) and writes the
// row's output: K indices (and scores) in selection order, then -1 (and -inf) up
// to top_k.  grp holds K entries; hist holds kBins + 4 counters.
__device__ void finish_row(uint64_t* sortbuf, uint64_t* grp, uint32_t* hist, int K, int top_k, int32_t* oi,
                           float* os, SelShared& sh) {
  const int tid = threadIdx.x;
  for (int i = K + tid; i < top_k; i += kSelThreads) {
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
  if (K <= 1) {
    if (K == 1 && tid == 0) {
      const uint64_t c = sortbuf[0];
      oi[0] = (int32_t)(~(uint32_t)c);
      if (os) os[0] = ord_to_float((uint32_t)(c >> 32));
    }
    return;
  }
  uint64_t mx = 0ull, mn = ~0ull;
  for (int i = tid; i < K; i += kSelThreads) {
    const uint64_t c = sortbuf[i];
    mx = c > mx ? c : mx;
    mn = c < mn ? c : mn;
  }
  block_minmax(mx, mn, sh);
  const int hb = 63 - __clzll(mx ^ mn);  // composites are distinct: mx != mn
  const int bsh = hb >= kDigit - 1 ? hb - (kDigit - 1) : 0;
  const uint64_t base = mn >> bsh;
  clear_bins(hist);
  if (tid == 0) {
    hist[kBins] = 0u;  // start of the bucket above the top one
    sh.digit = 0u;
  }
  __syncthreads();
  for (int i = tid; i < K; i += kSelThreads) atomicAdd(&hist[(uint32_t)((sortbuf[i] >> bsh) - base)], 1u);
  __syncthreads();
  uint32_t h[kBinsPerThread];
  load_bins(hist, h);
  uint32_t own = 0, bmax = 0;
#pragma unroll
  for (int q = 0; q < kBinsPerThread; ++q) {
    own += h[q];
    bmax = h[q] > bmax ? h[q] : bmax;
  }
  uint32_t start = block_suffix(own, sh);  // larger buckets come first
#pragma unroll
  for (int q = kBinsPerThread - 1; q >= 0; --q) {
    hist[tid * kBinsPerThread + q] = start;
    start += h[q];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) bmax = max(bmax, (uint32_t)__shfl_xor((int)bmax, off));
  if ((tid & 63) == 0) atomicMax(&sh.digit, bmax);
  __syncthreads();
  if (sh.digit > (uint32_t)kBucketMax) {
    const int n2 = pow2_at_least(K);
    for (int i = K + tid; i < n2; i += kSelThreads) sortbuf[i] = 0ull;  // composites are never 0
    __syncthreads();
    bitonic_desc(sortbuf, n2);
  } else {
    // scatter into buckets; afterwards hist[b] is the end of bucket b and
    // hist[b + 1] its start
    for (int i = tid; i < K; i += kSelThreads) {
      const uint64_t c = sortbuf[i];
      grp[atomicAdd(&hist[(uint32_t)((c >> bsh) - base)], 1u)] = c;
    }
    __syncthreads();
    for (int i = tid; i < K; i += kSelThreads) {
      const uint64_t c = grp[i];
      const uint32_t b = (uint32_t)((c >> bsh) - base);
      const uint32_t e = hist[b];
      const uint32_t s = hist[b + 1];
      uint32_t r = s;
      for (uint32_t j = s; j < e; ++j) r += grp[j] > c;
      sortbuf[r] = c;
    }
    __syncthreads();
  }
  for (int i = tid; i < K; i += kSelThreads) {
    const uint64_t c = sortbuf[i];
    oi[i] = (int32_t)(~(uint32_t)c);
    if (os) os[i] = ord_to_float((uint32_t)(c >> 32));
  }
}

// Dynamic LDS of a workgroup that finishes rows: sort buffer, bucket buffer, bins.
__host__ __device__ __forceinline__ size_t finish_lds_bytes(int top_k) {
  int p = 1;
  while (p < top_k) p <<= 1;
  return (size_t)8 * p + (size_t)8 * ((top_k + 1) & ~1) + (size_t)4 * (kBins + 4);
}

struct FinishLds {
  uint64_t* sortbuf;
  uint64_t* grp;
  uint32_t* hist;
};

__device__ __forceinline__ FinishLds carve(unsigned char* smem, int top_k) {
  const int p = pow2_at_least(top_k);
  FinishLds f;
  f.sortbuf = reinterpret_cast<uint64_t*>(smem);
  f.grp = f.sortbuf + p;
  f.hist = reinterpret_cast<uint32_t*>(f.grp + ((top_k + 1) & ~1));  // 16-byte aligned
  return f;
}

// ------------------------------------------------------------------ short rows

// One workgroup per row; entry e of the row sits in register i of thread t with
// e = i * 256 + t (coalesced loads).
template <int PER>
__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelShared sh;
  const int row = gridDim.x - 1 - blockIdx.x;  // causal rows grow with the index: longest first
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;
  const float* src = a.scores + (int64_t)row * a.score_stride;
  FinishLds f = carve(smem, a.top_k);

  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * kSelThreads + tid;
    key[i] = e < n ? ord_key(src[e]) : 0u;
  }
  auto each = [&](auto&& fn) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = i * kSelThreads + tid;
      if (e < n) fn(composite(key[i], (uint32_t)e));
    }
  };
  uint64_t thr = 0ull;
  if (K < n) thr = radix_select(each, 0ull, 0ull, (uint32_t)K, 63, f.hist, sh);
  // gather the winners
  uint32_t mine = 0;
  each([&](uint64_t c) { mine += c >= thr; });
  uint32_t off = block_suffix(mine, sh);
  each([&](uint64_t c) {
    if (c >= thr) f.sortbuf[off++] = c;
  });
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  finish_row(f.sortbuf, f.grp, f.hist, K, a.top_k, oi, os, sh);
}

// ------------------------------------------------------------------ long rows

// Stage 1: the chunk's histogram of the top 12 order-key bits, added into the
// global copy of the XCD the workgroup runs on (workgroups are dealt to the eight
// XCDs round robin by linear index).
template <int PER>
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelArgs a) {
  __shared__ __align__(16) uint32_t hist[kBins];
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int lo = blockIdx.x * (PER * kSelThreads);
  if (lo >= n) return;
  const float* src = a.scores + (int64_t)row * a.score_stride;
  clear_bins(hist);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lo + i * kSelThreads + tid;
    if (e < n) atomicAdd(&hist[ord_key(src[e]) >> (32 - kDigit)], 1u);
  }
  __syncthreads();
  const int copy = (blockIdx.y * gridDim.x + blockIdx.x) % kHistCopies;
  uint32_t* gh = a.ghist + ((int64_t)row * kHistCopies + copy) * kBins;
#pragma unroll
  for (int q = 0; q < kBinsPerThread; ++q) {
    const int b = q * kSelThreads + tid;
    const uint32_t v = hist[b];
    if (v) atomicAdd(&gh[b], v);
  }
}

// Stage 2 (one workgroup per row): sum the copies, find the bin of the K-th entry.
__global__ __launch_bounds__(kSelThreads) void select_thresh_kernel(SelArgs a) {
  __shared__ SelShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;
  if (K == n) {  // every entry wins (also n == 0)
    if (tid == 0) a.info[row] = RowInfo{0u, 0u, (uint32_t)n, 0u};
    return;
  }
  uint32_t h[kBinsPerThread] = {};
  const uint32_t* gh = a.ghist + (int64_t)row * kHistCopies * kBins + tid * kBinsPerThread;
#pragma unroll
  for (int c = 0; c < kHistCopies; ++c) {
    const uint4* p = reinterpret_cast<const uint4*>(gh + c * kBins);
#pragma unroll
    for (int j = 0; j < kBinsPerThread / 4; ++j) {
      const uint4 v = p[j];
      h[4 * j] += v.x;
      h[4 * j + 1] += v.y;
      h[4 * j + 2] += v.z;
      h[4 * j + 3] += v.w;
    }
  }
  find_digit(h, (uint32_t)K, sh);
  if (tid == 0) a.info[row] = RowInfo{sh.digit, sh.gt, sh.cnt, 0u};
}

// Stage 3: every entry of the chunk in the K-th entry's bin or above goes to the
// chunk's candidate slots (their order there does not matter: the composites are
// ordered later).
template <int PER>
__global__ __launch_bounds__(kSelThreads) void select_filter_kernel(SelArgs a) {
  __shared__ SelShared sh;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int lo = blockIdx.x * (PER * kSelThreads);
  const int64_t slot = (int64_t)row * a.chunks + blockIdx.x;
  if (lo >= n) {
    if (tid == 0) a.ccnt[slot] = 0u;
    return;
  }
  const float* src = a.scores + (int64_t)row * a.score_stride;
  const uint32_t bin = a.info[row].bin;
  // entry lo + t * PER + i of the chunk sits in register i of thread t
  uint32_t key[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lo + i * kSelThreads + tid;
    key[i] = e < n ? ord_key(src[e]) : 0u;
    mine += (e < n && (key[i] >> (32 - kDigit)) >= bin);
  }
  uint32_t pos = block_suffix(mine, sh);
  if (tid == 0) a.ccnt[slot] = pos + mine;
  uint64_t* cd = a.cand + slot * a.chunk;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lo + i * kSelThreads + tid;
    if (e < n && (key[i] >> (32 - kDigit)) >= bin) cd[pos++] = composite(key[i], (uint32_t)e);
  }
}

// Stage 4 (one workgroup per row): exact selection among the candidates, sort,
// output.  The candidates are read through a flat index over the chunks' slots.
__global__ __launch_bounds__(kSelThreads) void select_final_kernel(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;
  const RowInfo info = a.info[row];
  int C = K == n ? n : (int)(info.above + info.cnt);
  FinishLds f = carve(smem, a.top_k);
  // LDS after the finishing buffers: chunk offsets [chunks + 1], then candidates
  uint32_t* off = f.hist + kBins + 4;
  uint64_t* lc = reinterpret_cast<uint64_t*>(off + ((a.chunks + 4) & ~3));
  const uint32_t* cnt = a.ccnt + (int64_t)row * a.chunks;
  const uint64_t* cd = a.cand + (int64_t)row * a.chunks * a.chunk;
  if (tid == 0) sh.fill = 0u;
  // exclusive prefix of the chunk counts (sequential per 256-chunk block)
  {
    uint32_t carry = 0;
    for (int c0 = 0; c0 < a.chunks; c0 += kSelThreads) {
      const int c = c0 + tid;
      const uint32_t v = c < a.chunks ? cnt[c] : 0u;
      // inclusive prefix within the block of 256 through the suffix helper
      const uint32_t above = block_suffix(v, sh);
      __syncthreads();
      const uint32_t total = sh.wsum[0] + sh.wsum[1] + sh.wsum[2] + sh.wsum[3];
      if (c < a.chunks) off[c] = carry + (total - above - v);
      carry += total;
      __syncthreads();
    }
    if (tid == 0) off[a.chunks] = carry;
    __syncthreads();
    if ((uint32_t)C > carry) C = (int)carry;  // the chunk counts sum to C; never read past them
  }
  // flat candidate i: chunk = last c with off[c] <= i
  auto fetch = [&](int i) -> uint64_t {
    int lo = 0, hi = a.chunks;  // off[lo] <= i < off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= (uint32_t)i) lo = mid; else hi = mid;
    }
    return cd[(int64_t)lo * a.chunk + (i - (int)off[lo])];
  };
  const bool in_lds = C <= a.cand_lds;
  if (in_lds) {
    for (int i = tid; i < C; i += kSelThreads) lc[i] = fetch(i);
    __syncthreads();
  }
  auto get = [&](int i) -> uint64_t { return in_lds ? lc[i] : fetch(i); };
  uint64_t thr = 0ull;
  if (K < C) {
    auto each = [&](auto&& fn) {
      for (int i = tid; i < C; i += kSelThreads) fn(get(i));
    };
    const uint64_t mask = (uint64_t)(kBins - 1) << kTopShift;
    thr = radix_select(each, (uint64_t)info.bin << kTopShift, mask, (uint32_t)K - info.above, kTopShift - 1,
                       f.hist, sh);
  }
  for (int i0 = 0; i0 < C; i0 += kSelThreads) {
    const int i = i0 + tid;
    const uint64_t c = i < C ? get(i) : 0ull;
    const bool sel = i < C && c >= thr;
    const uint64_t m = __ballot(sel);
    uint32_t wb = 0;
    if (lane == 0 && m) wb = atomicAdd(&sh.fill, (uint32_t)__popcll(m));
    wb = __shfl(wb, 0);
    const uint32_t at = wb + __popcll(m & ((1ull << lane) - 1ull));
    if (sel && at < (uint32_t)K) f.sortbuf[at] = c;  // exactly K are selected
  }
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  finish_row(f.sortbuf, f.grp, f.hist, K, a.top_k, oi, os, sh);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------------ host planning

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the long-row pipeline: histogram copies | row info | chunk counts |
// candidate slots.
struct WsLayout {
  size_t hist, info, ccnt, cand, total;
};

static WsLayout ws_layout(int rows, int chunks, int chunk) {
  WsLayout l;
  l.hist = 0;
  l.info = round256((size_t)rows * kHistCopies * kBins * 4);
  l.ccnt = round256(l.info + (size_t)rows * sizeof(RowInfo));
  l.cand = round256(l.ccnt + (size_t)rows * chunks * 4);
  l.total = round256(l.cand + (size_t)rows * chunks * chunk * 8);
  return l;
}

constexpr size_t kFinalLdsBudget = 160 * 1024;

bool plan_select(int rows, int n_cols, int top_k, SelectPlan* p) {
  if (top_k < 1 || top_k > kMaxTopK) return false;
  p->rows = rows;
  p->n_cols = n_cols;
  p->top_k = top_k;
  p->lds = finish_lds_bytes(top_k);
  p->cand_lds = 0;
  if (n_cols <= kRowMax) {
    p->two_pass = 0;
    p->per = n_cols <= 1024 ? 4 : n_cols <= 2048 ? 8 : n_cols <= 4096 ? 16 : 32;
    p->chunks = 1;
    p->bytes = 0;
  } else {
    p->two_pass = 1;
    const int64_t big = (int64_t)rows * ((n_cols + 4095) / 4096);
    p->per = big >= 1024 ? 16 : 8;
    const int chunk = p->per * kSelThreads;
    p->chunks = (n_cols + chunk - 1) / chunk;
    p->bytes = ws_layout(rows, p->chunks, chunk).total;
    const size_t fixed = p->lds + (size_t)4 * ((p->chunks + 4) & ~3);
    if (fixed > kFinalLdsBudget) return false;
    size_t c = (kFinalLdsBudget - fixed) / 8;
    if (c > 12288) c = 12288;
    p->cand_lds = (int)c;
    p->lds = fixed + (size_t)8 * p->cand_lds;
  }
  return true;
}

// Workspace bytes of the plan (device independent); at least 256 when supported.
size_t select_workspace_bytes(int rows, int n_cols, int top_k) {
  SelectPlan p;
  if (!plan_select(rows, n_cols, top_k, &p)) return 0;
  return p.bytes > 256 ? p.bytes : 256;
}

template <typename K>
static hipError_t set_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int PER>
static hipError_t launch_rows(const SelArgs& a, const SelectPlan& p, hipStream_t st) {
  hipError_t e = set_lds(select_rows_kernel<PER>, p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_rows_kernel<PER>, dim3(p.rows), dim3(kSelThreads), p.lds, st, a);
  return hipGetLastError();
}

template <int PER>
static hipError_t launch_pipeline(const SelArgs& a, const SelectPlan& p, void* ws, size_t hist_bytes,
                                  hipStream_t st) {
  hipError_t e = set_lds(select_final_kernel, p.lds);
  if (e != hipSuccess) return e;
  const int64_t n16 = (int64_t)(hist_bytes / 16);
  int blocks = (int)((n16 + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<uint4*>(ws), n16);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid(p.chunks, p.rows);
  hipLaunchKernelGGL(select_hist_kernel<PER>, grid, dim3(kSelThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_thresh_kernel, dim3(p.rows), dim3(kSelThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_filter_kernel<PER>, grid, dim3(kSelThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_final_kernel, dim3(p.rows), dim3(kSelThreads), p.lds, st, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectPlan& p, const float* scores, int64_t score_stride,
                         const int32_t* valid_lens, int64_t first_pos, int ratio, int32_t* out_idx,
                         float* out_scores, void* ws, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  SelArgs a{};
  a.scores = scores;
  a.score_stride = score_stride;
  a.valid_lens = valid_lens;
  a.first_pos = first_pos;
  a.ratio = ratio;
  a.n_cols = p.n_cols;
  a.top_k = p.top_k;
  a.out_idx = out_idx;
  a.out_scores = out_scores;
  if (!p.two_pass) {
    switch (p.per) {
      case 4: return launch_rows<4>(a, p, st);
      case 8: return launch_rows<8>(a, p, st);
      case 16: return launch_rows<16>(a, p, st);
      default: return launch_rows<32>(a, p, st);
    }
  }
  a.chunk = p.per * kSelThreads;
  a.chunks = p.chunks;
  a.cand_lds = p.cand_lds;
  const WsLayout l = ws_layout(p.rows, p.chunks, a.chunk);
  unsigned char* w = static_cast<unsigned char*>(ws);
  a.ghist = reinterpret_cast<uint32_t*>(w + l.hist);
  a.info = reinterpret_cast<RowInfo*>(w + l.info);
  a.ccnt = reinterpret_cast<uint32_t*>(w + l.ccnt);
  a.cand = reinterpret_cast<uint64_t*>(w + l.cand);
  return p.per == 16 ? launch_pipeline<16>(a, p, w, l.info, st) : launch_pipeline<8>(a, p, w, l.info, st);
}

}  // namespace salb
