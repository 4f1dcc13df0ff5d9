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
//   * many rows (256 or more) of up to 32768 entries: one workgroup per row as well,
//     1024 threads with 16 entries each in registers up to 16384 entries, 512 threads
//     with 64 each beyond (one histogram pass, then an LDS candidate list);
//   * longer rows run as a pipeline of three launches (kernel boundaries order
//     them; no grid-wide fences, which write back the whole L2 on this chip):
//     every workgroup of a (chunk, row) grid adds its chunk's LDS histogram of the
//     top 12 order-key bits (its nonzero bins) into one of eight global copies (one
//     per XCD, so contended atomics stay in one L2), which the call zeroes first (a
//     clearing launch, or the scorer launch that precedes the select in the fused
//     path);
//     the (chunk, row) grid then finds the bin holding the K-th entry from the
//     copies (scanning down from the row's highest bin) and writes every entry at
//     or above that bin to the chunk's own candidate slots; one workgroup per row
//     (512 threads when rows are few, 256 when they are many) loads those
//     candidates (about K plus one bin's worth) into registers, selects the K
//     winners exactly and sorts them.
//   * the sort buckets the winners on the 12 highest bits where they differ and
//     ranks each against its bucket (a sorting network if a bucket is crowded).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

constexpr int kDigit = 12;
constexpr int kRankSortMax = 64;  // winners sorted by a plain rank count up to this many
constexpr int kBins = 1 << kDigit;       // 4096 histogram bins
constexpr int kTopShift = 64 - kDigit;   // first digit: the score's top 12 order bits
constexpr int kRowThreads = 256;         // one-workgroup rows
constexpr int kChunkThreads = 256;       // histogram and filter chunks of long rows
constexpr int kFinalThreads = 512;       // the finishing workgroup of a long row when rows are few
constexpr int kFinalPer = 16;            // candidates per finishing thread held in registers
constexpr int kFinalThreadsMany = 256;   // ... and when rows are many (more rows in flight per CU)
constexpr int kFinalPerMany = 16;
constexpr int kFewRows = 256;
constexpr int kRowMax = 32 * kRowThreads;  // 8192: one-workgroup rows
// Wider one-workgroup rows (1024 threads: 16 entries each in registers, or up to
// 32768 entries in LDS) once there are enough rows to fill the GPU with one workgroup
// per row: the row is read once, with no global histogram or candidate pass.
constexpr int kRowThreadsWide = 1024;
constexpr int kRowMaxWide = 32 * kRowThreadsWide;  // 32768
constexpr int kWideRowsMin = 256;
constexpr int kRowThreadsReg = 512;    // many rows of up to 32768 entries: 64 per thread in registers
constexpr int kBucketMax = 48;           // crowded bucket: sorting network instead
constexpr int kHistCopies = kXcds;       // one global histogram per XCD
constexpr int kMaxWaves = 1024 / kWave;  // widest workgroup of the select kernels

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
  int cand_cap;      // LDS candidate slots of a one-workgroup row kept in LDS
  // long-row pipeline
  int chunk;         // entries per chunk workgroup
  int chunks;        // chunks per row
  uint32_t* ghist;   // [rows][kHistCopies][kBins], zeroed by the call before stage 1
  uint32_t* gmax;    // [rows][kHistCopies] highest bin seen, zeroed with ghist
  RowInfo* info;     // [rows]
  uint32_t* ccount;  // [rows][chunks] candidates per chunk
  uint64_t* cand;    // [rows][chunks][chunk] candidate slots
  // sub-tile select
  const uint32_t* tmax;  // [rows][tmax_stride] order-key maximum of each 16-entry sub-tile
  int64_t tmax_stride;
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
  uint32_t wsum[kMaxWaves];
  uint64_t wred[2 * kMaxWaves];
  uint32_t digit, gt, cnt, fill;
};

// Wave scans and reductions through DPP: shifts within 16-lane rows, then the row
// broadcasts that carry the last lane of a row into the rows after it.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the lanes of the wave.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Maximum over the lanes of the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp_or_zero<0x111, 0xf>(x));
  x = max(x, dpp_or_zero<0x112, 0xf>(x));
  x = max(x, dpp_or_zero<0x114, 0xf>(x));
  x = max(x, dpp_or_zero<0x118, 0xf>(x));
  x = max(x, dpp_or_zero<0x142, 0xa>(x));
  x = max(x, dpp_or_zero<0x143, 0xc>(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint64_t wave_max64(uint64_t x) {
  const uint32_t hi = (uint32_t)(x >> 32);
  const uint32_t mhi = wave_max(hi);
  const uint32_t mlo = wave_max(hi == mhi ? (uint32_t)x : 0u);
  return ((uint64_t)mhi << 32) | mlo;
}

// Sum of v over the threads with a larger index.  Two calls must be separated by a
// barrier after the first call's result is used.
template <int NT>
__device__ __forceinline__ uint32_t block_suffix(uint32_t v, SelShared& sh) {
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_prefix_sum(v);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  if ((threadIdx.x & 63) == 0) sh.wsum[wave] = tot;
  __syncthreads();
  uint32_t above = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) above += w > wave ? sh.wsum[w] : 0u;
  return above + tot - incl;
}

// block_suffix, and the block-wide maximum and minimum of mx and mn (same barrier).
template <int NT>
__device__ __forceinline__ uint32_t block_suffix_minmax(uint32_t v, uint64_t& mx, uint64_t& mn, SelShared& sh) {
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_prefix_sum(v);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint64_t wmx = wave_max64(mx);
  const uint64_t wmn = ~wave_max64(~mn);
  if ((threadIdx.x & 63) == 0) {
    sh.wsum[wave] = tot;
    sh.wred[wave] = wmx;
    sh.wred[kMaxWaves + wave] = wmn;
  }
  __syncthreads();
  uint32_t above = 0;
  mx = 0ull;
  mn = ~0ull;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    above += w > wave ? sh.wsum[w] : 0u;
    const uint64_t a = sh.wred[w], b = sh.wred[kMaxWaves + w];
    mx = a > mx ? a : mx;
    mn = b < mn ? b : mn;
  }
  return above + tot - incl;
}

// Thread t owns bins [t * BPT, (t + 1) * BPT).
template <int NT>
__device__ __forceinline__ void load_bins(const uint32_t* hist, uint32_t (&h)[kBins / NT]) {
  constexpr int BPT = kBins / NT;
  const uint4* p = reinterpret_cast<const uint4*>(hist + threadIdx.x * BPT);
#pragma unroll
  for (int j = 0; j < BPT / 4; ++j) {
    const uint4 v = p[j];
    h[4 * j] = v.x;
    h[4 * j + 1] = v.y;
    h[4 * j + 2] = v.z;
    h[4 * j + 3] = v.w;
  }
}

template <int NT>
__device__ __forceinline__ void clear_bins(uint32_t* hist) {
  uint4* p = reinterpret_cast<uint4*>(hist);
#pragma unroll
  for (int j = threadIdx.x; j < kBins / 4; j += NT) p[j] = make_uint4(0u, 0u, 0u, 0u);
}

// Digit search over a 4096-bin histogram held as in load_bins: the bin holding
// the rem-th largest counted entry, the count above it and its own count land in
// sh.digit / sh.gt / sh.cnt.  Requires 1 <= rem <= total.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t (&h)[kBins / NT], uint32_t rem, SelShared& sh) {
  constexpr int BPT = kBins / NT;
  uint32_t own = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) own += h[q];
  uint32_t ge = block_suffix<NT>(own, sh);
  // exactly one thread holds the bin where the count from the top reaches rem
  int hit = -1;
  uint32_t hit_gt = 0, hit_cnt = 0;
#pragma unroll
  for (int q = BPT - 1; q >= 0; --q) {
    const bool here = ge < rem && ge + h[q] >= rem;
    hit = here ? q : hit;
    hit_gt = here ? ge : hit_gt;
    hit_cnt = here ? h[q] : hit_cnt;
    ge += h[q];
  }
  if (hit >= 0) {
    sh.digit = threadIdx.x * BPT + hit;
    sh.gt = hit_gt;
    sh.cnt = hit_cnt;
  }
  __syncthreads();
}

// Radix select: the threshold thr such that exactly `rem` of the composites that
// agree with `prefix` on the bits of `mask` are >= thr (those above the prefix are
// already counted out by the caller).  `each(f)` calls f(c) on every composite
// this thread owns.  Digits are 12 bits wide, from bit `top` down.
template <int NT, typename Each>
__device__ uint64_t radix_select(Each each, uint64_t prefix, uint64_t mask, uint32_t rem, int top,
                                 uint32_t* hist, SelShared& sh) {
  for (;;) {
    const int width = top + 1 < kDigit ? top + 1 : kDigit;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    clear_bins<NT>(hist);
    __syncthreads();
    each([&](uint64_t c) {
      if ((c & mask) == prefix) atomicAdd(&hist[(uint32_t)(c >> shift) & dmask], 1u);
    });
    __syncthreads();
    uint32_t h[kBins / NT];
    load_bins<NT>(hist, h);
    find_digit<NT>(h, rem, sh);
    const uint32_t digit = sh.digit, gt = sh.gt, cnt = sh.cnt;
    prefix |= (uint64_t)digit << shift;
    mask |= (uint64_t)dmask << shift;
    rem -= gt;
    if (cnt == rem || shift == 0) return prefix;
    top = shift - 1;
  }
}

// Radix select on 32-bit values: the digit walk for the rem-th largest value, which
// stops at the first digit whose bin holds exactly the remaining count (every value in
// that bin wins) or after the last bit.  On return `thr` has zero bits below the last
// digit taken and `gt_all` counts the values above its bin.  With `whole` set the
// winners are exactly the values >= thr; otherwise thr is the rem-th largest value
// itself and more values equal it than win (ties the caller breaks by index).  Digits
// are 12 bits wide, from bit `top` down.
template <int NT, typename Each>
__device__ void radix_select32(Each each, uint32_t rem, int top, uint32_t* hist, SelShared& sh, uint32_t& thr,
                               uint32_t& gt_all, bool& whole) {
  uint32_t prefix = 0u, mask = 0u;
  gt_all = 0u;
  for (;;) {
    const int width = top + 1 < kDigit ? top + 1 : kDigit;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    clear_bins<NT>(hist);
    __syncthreads();
    each([&](uint32_t r) {
      if ((r & mask) == prefix) atomicAdd(&hist[(r >> shift) & dmask], 1u);
    });
    __syncthreads();
    uint32_t h[kBins / NT];
    load_bins<NT>(hist, h);
    find_digit<NT>(h, rem, sh);
    const uint32_t digit = sh.digit, gt = sh.gt, cnt = sh.cnt;
    prefix |= digit << shift;
    mask |= dmask << shift;
    rem -= gt;
    gt_all += gt;
    if (cnt == rem || shift == 0) {
      thr = prefix;
      whole = cnt == rem;
      return;
    }
    top = shift - 1;
  }
}

// Descending bitonic sort of buf[0, n2) (n2 a power of two) by the whole block.
template <int NT>
__device__ void bitonic_desc(uint64_t* buf, int n2) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += NT) {
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
// to top_k.  Up to kRankSortMax winners each find their place by counting the larger
// ones; more are bucketed by their top bits and ranked within the bucket (a sorting
// network when a bucket is crowded).  mx and mn are the largest and smallest winner;
// grp holds K entries; hist holds kBins + 4 counters.  The kernel ends after it.
template <int NT>
__device__ void finish_row(uint64_t* sortbuf, uint64_t* grp, uint32_t* hist, int K, int top_k, int32_t* oi,
                           float* os, uint64_t mx, uint64_t mn, SelShared& sh, uint32_t kbase = 0u) {
  constexpr int BPT = kBins / NT;
  const int tid = threadIdx.x;
  for (int i = K + tid; i < top_k; i += NT) {
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
  if (K <= 1) {
    if (K == 1 && tid == 0) {
      const uint64_t c = sortbuf[0];
      oi[0] = (int32_t)(~(uint32_t)c);
      if (os) os[0] = ord_to_float((uint32_t)(c >> 32) + kbase);
    }
    return;
  }
  if (K <= kRankSortMax) {
    // Few winners: each one's place is the count of larger winners (composites are
    // distinct), read with broadcast LDS loads -- one pass, no barrier or atomic.
    for (int i = tid; i < K; i += NT) {
      const uint64_t c = sortbuf[i];
      uint32_t r = 0;
      int j = 0;
      for (; j + 4 <= K; j += 4)
        r += (uint32_t)(sortbuf[j] > c) + (uint32_t)(sortbuf[j + 1] > c) + (uint32_t)(sortbuf[j + 2] > c) +
             (uint32_t)(sortbuf[j + 3] > c);
      for (; j < K; ++j) r += (uint32_t)(sortbuf[j] > c);
      oi[r] = (int32_t)(~(uint32_t)c);
      if (os) os[r] = ord_to_float((uint32_t)(c >> 32) + kbase);
    }
    return;
  }
  const int hb = 63 - __clzll(mx ^ mn);  // composites are distinct: mx != mn
  const int bsh = hb >= kDigit - 1 ? hb - (kDigit - 1) : 0;
  const uint64_t base = mn >> bsh;
  clear_bins<NT>(hist);
  if (tid == 0) {
    hist[kBins] = 0u;  // start of the bucket above the top one
    sh.digit = 0u;
  }
  __syncthreads();
  for (int i = tid; i < K; i += NT) atomicAdd(&hist[(uint32_t)((sortbuf[i] >> bsh) - base)], 1u);
  __syncthreads();
  uint32_t h[BPT];
  load_bins<NT>(hist, h);
  uint32_t own = 0, bmax = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    own += h[q];
    bmax = h[q] > bmax ? h[q] : bmax;
  }
  uint32_t start = block_suffix<NT>(own, sh);  // larger buckets come first
#pragma unroll
  for (int q = BPT - 1; q >= 0; --q) {
    hist[tid * BPT + q] = start;
    start += h[q];
  }
  bmax = wave_max(bmax);
  if ((tid & 63) == 0) atomicMax(&sh.digit, bmax);
  __syncthreads();
  if (sh.digit > (uint32_t)kBucketMax) {
    const int n2 = pow2_at_least(K);
    for (int i = K + tid; i < n2; i += NT) sortbuf[i] = 0ull;  // composites are never 0
    __syncthreads();
    bitonic_desc<NT>(sortbuf, n2);
  } else {
    // scatter into buckets; afterwards hist[b] is the end of bucket b and
    // hist[b + 1] its start
    for (int i = tid; i < K; i += NT) {
      const uint64_t c = sortbuf[i];
      grp[atomicAdd(&hist[(uint32_t)((c >> bsh) - base)], 1u)] = c;
    }
    __syncthreads();
    for (int i = tid; i < K; i += NT) {
      const uint64_t c = grp[i];
      const uint32_t b = (uint32_t)((c >> bsh) - base);
      const uint32_t e = hist[b];
      const uint32_t s = hist[b + 1];
      uint32_t r = s, j = s;
      for (; j + 4 <= e; j += 4) {
        const uint64_t g0 = grp[j], g1 = grp[j + 1], g2 = grp[j + 2], g3 = grp[j + 3];
        r += (g0 > c) + (g1 > c) + (g2 > c) + (g3 > c);
      }
      for (; j < e; ++j) r += grp[j] > c;
      sortbuf[r] = c;
    }
    __syncthreads();
  }
  for (int i = tid; i < K; i += NT) {
    const uint64_t c = sortbuf[i];
    oi[i] = (int32_t)(~(uint32_t)c);
    if (os) os[i] = ord_to_float((uint32_t)(c >> 32) + kbase);
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

// Whether a row select may read its rows with 16-byte loads of four consecutive entries:
// rows 16-byte aligned, stride and n_cols multiples of 4 (every vector then lies inside
// its row).
__host__ __forceinline__ bool rows_vec_ok(const SelArgs& a) {
  return a.score_stride % 4 == 0 && a.n_cols % 4 == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
}

// One workgroup per row; entry e of the row sits in register i of thread t with
// e = i * NT + t, or with VEC (16-byte loads, a quarter of the load instructions)
// e = 4 ((i / 4) NT + t) + i % 4.  Coalesced loads either way.
template <int NT, int PER, bool VEC>
__global__ __launch_bounds__(NT, (NT == kRowThreads && PER <= 16) ? 5 : 1) void select_rows_kernel(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelShared sh;
  const int row = gridDim.x - 1 - blockIdx.x;  // causal rows grow with the index: longest first
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;
  const float* src = a.scores + (int64_t)row * a.score_stride;
  FinishLds f = carve(smem, a.top_k);

  // entry of register i, and the first entry any thread holds in register i
  auto ent = [&](int i) { return VEC ? 4 * ((i >> 2) * NT + tid) + (i & 3) : i * NT + tid; };
  auto ent0 = [](int i) { return VEC ? 4 * (i >> 2) * NT : i * NT; };
  // all loads unconditional inside one row-uniform branch, so that they are in flight
  // together: positions past n re-read the row's last quad (or entry), keys 0
  uint32_t key[PER];
  if (n > 0) {
    if constexpr (VEC) {
      static_assert(PER % 4 == 0, "vector rows");
      const int last = (n - 1) & ~3;  // rows and n_cols are 16-byte aligned
      float4v x[PER / 4];
#pragma unroll
      for (int j = 0; j < PER / 4; ++j) {
        const int e0 = 4 * (j * NT + tid);
        x[j] = *reinterpret_cast<const float4v*>(src + (e0 < n ? e0 : last));
      }
#pragma unroll
      for (int j = 0; j < PER / 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) key[4 * j + q] = 4 * (j * NT + tid) + q < n ? ord_key(x[j][q]) : 0u;
    } else {
      float x[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = i * NT + tid;
        x[i] = src[e < n ? e : n - 1];
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) key[i] = i * NT + tid < n ? ord_key(x[i]) : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = 0u;
  }
  // registers past the row's last entry are skipped on a wave-uniform branch: a short
  // row costs passes over its own length, not over the workgroup's capacity
  auto each_key = [&](auto&& fn) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (ent0(i) >= n) break;
      const int e = ent(i);
      if (e < n) fn(key[i], e);
    }
  };
  // The row's keys are taken relative to its smallest one, and the radix starts at the
  // highest bit in which any two differ: the first digit then splits the row's actual
  // range (a row of close scores would otherwise crowd a few bins of the first digit,
  // and its LDS atomics with them).  The walk runs on the 32-bit keys; the entry index
  // only enters when equal scores straddle the K-th position.
  uint32_t kbase = 0u, thr32 = 0u, gt = 0u;
  bool whole = true;  // the winners are exactly the keys >= kbase + thr32
  if (K < n) {
    uint32_t kmx32 = 0u, kmn32 = ~0u;
    each_key([&](uint32_t k, int) {
      kmx32 = k > kmx32 ? k : kmx32;
      kmn32 = k < kmn32 ? k : kmn32;
    });
    uint64_t kmx = kmx32, kmn = kmn32;
    block_suffix_minmax<NT>(0u, kmx, kmn, sh);
    __syncthreads();  // sh is used again below
    kbase = (uint32_t)kmn;
    const uint32_t span = (uint32_t)kmx - kbase;
    const int top = span ? 31 - __clz(span) : 0;
    radix_select32<NT>([&](auto&& fn) { each_key([&](uint32_t k, int) { fn(k - kbase); }); }, (uint32_t)K, top,
                       f.hist, sh, thr32, gt, whole);
  }
  auto each = [&](auto&& fn) { each_key([&](uint32_t k, int e) { fn(composite(k - kbase, (uint32_t)e)); }); };
  uint32_t off;
  uint64_t mx, mn;
  if (whole) {
    // gather the winners on the 32-bit keys; the bounds handed to the sort are widened
    // over the index bits (every winner's composite lies between them)
    uint32_t mine = 0, rmx = 0u, rmn = ~0u;
    each_key([&](uint32_t k, int) {
      const uint32_t r = k - kbase;
      if (r >= thr32) {
        ++mine;
        rmx = r > rmx ? r : rmx;
        rmn = r < rmn ? r : rmn;
      }
    });
    mx = ((uint64_t)rmx << 32) | 0xffffffffull;
    mn = (uint64_t)rmn << 32;
    if (mine == 0) {  // neutral elements for the block reduction
      mx = 0ull;
      mn = ~0ull;
    }
    off = block_suffix_minmax<NT>(mine, mx, mn, sh);
    each_key([&](uint32_t k, int e) {
      if (k - kbase >= thr32 && off < (uint32_t)K) f.sortbuf[off++] = composite(k - kbase, (uint32_t)e);
    });
  } else {
    // equal keys at the K-th position: the lowest indices among them win
    const uint64_t thr = radix_select<NT>(each, (uint64_t)thr32 << 32, 0xffffffff00000000ull, (uint32_t)K - gt,
                                          31, f.hist, sh);
    uint32_t mine = 0;
    mx = 0ull;
    mn = ~0ull;
    each([&](uint64_t c) {
      if (c >= thr) {
        ++mine;
        mx = c > mx ? c : mx;
        mn = c < mn ? c : mn;
      }
    });
    off = block_suffix_minmax<NT>(mine, mx, mn, sh);
    each([&](uint64_t c) {
      if (c >= thr && off < (uint32_t)K) f.sortbuf[off++] = c;  // exactly K are selected
    });
  }
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  finish_row<NT>(f.sortbuf, f.grp, f.hist, K, a.top_k, oi, os, mx, mn, sh, kbase);
}

// Rows of up to 32768 entries when there are many (one 512-thread workgroup per row,
// longest rows first, several workgroups per CU so that one's loads overlap another's
// passes).  The row stays in registers as order keys (64 per thread, coalesced loads:
// four consecutive entries per 16-byte load where the row's alignment allows, else
// entry i NT + t in register i of thread t).  Its range comes from one wave and block
// reduction; one histogram pass over a 12-bit digit of the key relative to the row's
// smallest (the digit spans the row's actual range) finds the bin of the K-th entry;
// the entries from that bin up -- K plus the rest of the bin -- are compacted into an
// LDS candidate list (one LDS atomic per wave and register, the lanes placed by their
// rank in the wave's ballot), where the radix select finishes and the winners are
// gathered.  A bin crowded past the list's capacity falls back to radix passes over
// the row read again from memory.
// VEC: each lane reads four consecutive entries per 16-byte load, register i of thread t
// holding entry 4 ((i / 4) NT + t) + i % 4 (a quarter of the load instructions); only
// for 16-byte aligned rows whose stride and n_cols are multiples of 4, so that every
// vector lies inside its row.
template <int NT, bool VEC>
__global__ __launch_bounds__(NT) void select_rows_reg_kernel(SelArgs a, int rows) {
  constexpr int PF = kRowMaxWide / NT;  // a row's entries per thread
  // entry of register i, and the first entry any thread holds in register i
  auto ent = [&](int i) { return VEC ? 4 * ((i >> 2) * NT + (int)threadIdx.x) + (i & 3) : i * NT + (int)threadIdx.x; };
  auto ent0 = [](int i) { return VEC ? 4 * (i >> 2) * NT : i * NT; };
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelShared sh;
  __shared__ uint32_t s_kmx[NT / kWave], s_kmn[NT / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);
  FinishLds f = carve(smem + (size_t)a.cand_cap * 8, a.top_k);
  const int row = rows - 1 - (int)blockIdx.x;  // causal rows grow with the index: longest first
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;

  const float* src = a.scores + (int64_t)row * a.score_stride;
  uint32_t key[PF];
  {
    const int last = n > 0 ? n - 1 : 0;  // past the valid entries: re-read valid memory
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < PF / 4; ++j) {
        const float4v v = *reinterpret_cast<const float4v*>(src + 4 * min(j * NT + tid, last >> 2));
#pragma unroll
        for (int q = 0; q < 4; ++q) key[4 * j + q] = ord_key(v[q]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PF; ++i) key[i] = ord_key(src[min(i * NT + tid, last)]);
    }
  }
  uint32_t kmx = 0u, kmn = ~0u;
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const bool v = ent(i) < n;
    kmx = v && key[i] > kmx ? key[i] : kmx;
    kmn = v && key[i] < kmn ? key[i] : kmn;
  }
  kmx = wave_max(kmx);
  kmn = ~wave_max(~kmn);
  if (lane == 0) {
    s_kmx[wave] = kmx;
    s_kmn[wave] = kmn;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    kmx = s_kmx[w] > kmx ? s_kmx[w] : kmx;
    kmn = s_kmn[w] < kmn ? s_kmn[w] : kmn;
  }
  const uint32_t kbase = kmn;
  // every valid entry of the row as its composite, read again from memory: only the
  // rare paths use it (a crowded bin past the candidate list, rows no longer than
  // top_k), so the registers of the row are free after the compaction
  auto each_row = [&](auto&& fn) {
    for (int e = tid; e < n; e += NT) fn(composite(ord_key(src[e]) - kbase, (uint32_t)e));
  };
  int C = -1;  // candidates in the list (-1: the whole row is the candidate set)
  auto each_cand = [&](auto&& fn) {
    for (int i = tid; i < C; i += NT) fn(cand[i]);
  };
  uint64_t thr = 0ull;
  if (K < n) {
    const uint32_t span = kmx - kbase;
    const int bits = span ? 32 - __clz(span) : 1;
    const int shift = bits > kDigit ? bits - kDigit : 0;
    clear_bins<NT>(f.hist);
    if (tid == 0) sh.fill = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (ent0(i) >= n) break;
      if (ent(i) < n) atomicAdd(&f.hist[(key[i] - kbase) >> shift], 1u);
    }
    __syncthreads();
    uint32_t h[kBins / NT];
    load_bins<NT>(f.hist, h);
    find_digit<NT>(h, (uint32_t)K, sh);
    const uint32_t b1 = sh.digit, gt = sh.gt, cnt = sh.cnt;
    const uint64_t prefix = (uint64_t)b1 << (32 + shift);
    if (gt + cnt <= (uint32_t)a.cand_cap) {
      const uint32_t kthr = kbase + (b1 << shift);  // smallest key of bin b1
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        if (ent0(i) >= n) break;
        const int e = ent(i);
        const bool pick = e < n && key[i] >= kthr;
        const uint64_t m = __ballot(pick);
        if (m != 0ull) {
          const int leader = __ffsll((unsigned long long)m) - 1;
          uint32_t base = 0u;
          if (lane == leader) base = atomicAdd(&sh.fill, (uint32_t)__popcll(m));
          base = __builtin_amdgcn_readlane(base, leader);
          const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (pick) cand[base + below] = composite(key[i] - kbase, (uint32_t)e);
        }
      }
      __syncthreads();
      C = (int)(gt + cnt);
      if (gt + cnt == (uint32_t)K)
        thr = prefix;  // the bin is taken whole
      else
        thr = radix_select<NT>(each_cand, prefix, (uint64_t)(kBins - 1) << (32 + shift), (uint32_t)K - gt,
                               31 + shift, f.hist, sh);
    } else {
      thr = radix_select<NT>(each_row, prefix, (uint64_t)(kBins - 1) << (32 + shift), (uint32_t)K - gt, 31 + shift,
                             f.hist, sh);
    }
  }
  // gather the winners
  auto each = [&](auto&& fn) {
    if (C >= 0)
      each_cand(fn);
    else
      each_row(fn);
  };
  uint32_t mine = 0;
  uint64_t mx = 0ull, mn = ~0ull;
  each([&](uint64_t c) {
    if (c >= thr) {
      ++mine;
      mx = c > mx ? c : mx;
      mn = c < mn ? c : mn;
    }
  });
  uint32_t off = block_suffix_minmax<NT>(mine, mx, mn, sh);
  each([&](uint64_t c) {
    if (c >= thr && off < (uint32_t)K) f.sortbuf[off++] = c;  // exactly K are selected
  });
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  finish_row<NT>(f.sortbuf, f.grp, f.hist, K, a.top_k, oi, os, mx, mn, sh, kbase);
}

// ------------------------------------------------------------------ sub-tile rows

// Rows of up to 32768 entries whose 16-entry sub-tiles come with their largest order key
// (written by the scorer beside the scores), top_k <= kTileSelMaxK, rows 16-byte aligned
// with a stride that is a multiple of 16: one 256-thread workgroup per row, longest rows
// first.  When K is at most the count of sub-tiles holding valid entries, the K-th largest
// sub-tile maximum bounds the K-th largest entry from below (at least K sub-tiles, hence
// at least K entries, reach it), so every winner lies in a sub-tile whose maximum reaches
// it.  One histogram pass over the maxima (bins spanning their actual range) gives a bound
// T at or below that maximum; only the sub-tiles reaching T are read, and their entries at
// or above T form an LDS candidate list, where the radix select finishes and the winners
// are gathered -- the same winners as a select over the whole row.  A list crowded past
// its capacity (rows of many equal scores) falls back to radix passes over the whole row.
constexpr int kTileSelThreads = 256;
constexpr int kTileSelMaxK = 512;
constexpr int kTileSelCand = 1920;                      // LDS candidate slots (four workgroups per CU)
constexpr int kTileSelTiles = kRowMaxWide / 16;          // sub-tiles of the longest row: 2048

template <int NT>
__global__ __launch_bounds__(NT) void select_tiles_kernel(SelArgs a, int rows) {
  constexpr int MPT = kTileSelTiles / NT;  // sub-tile maxima per thread
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelShared sh;
  __shared__ uint32_t s_kmx[NT / kWave], s_kmn[NT / kWave];
  __shared__ uint32_t s_tiles, s_cands;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);                             // [kTileSelCand]
  uint16_t* tlist = reinterpret_cast<uint16_t*>(cand + kTileSelCand);             // [kTileSelTiles]
  FinishLds f = carve(reinterpret_cast<unsigned char*>(tlist + kTileSelTiles), a.top_k);
  const int row = rows - 1 - (int)blockIdx.x;  // causal rows grow with the index: longest first
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;
  const float* src = a.scores + (int64_t)row * a.score_stride;

  uint32_t kbase = 0u;  // composites hold keys relative to it
  int C = -1;           // candidates in the list (-1: the whole row is the candidate set)
  uint64_t thr = 0ull;
  auto each_row = [&](auto&& fn) {
    for (int e = tid; e < n; e += NT) fn(composite(ord_key(src[e]) - kbase, (uint32_t)e));
  };
  auto each_cand = [&](auto&& fn) {
    for (int i = tid; i < C; i += NT) fn(cand[i]);
  };
  if (K < n) {
    const int nt = (n + 15) >> 4;  // sub-tiles holding valid entries
    const uint32_t* tm = a.tmax + (int64_t)row * a.tmax_stride;
    uint32_t mk[MPT];
#pragma unroll
    for (int i = 0; i < MPT; ++i) {
      const int j = i * NT + tid;
      mk[i] = j < nt ? tm[j] : 0u;
    }
    // range of the maxima
    uint32_t kmx = 0u, kmn = ~0u;
#pragma unroll
    for (int i = 0; i < MPT; ++i) {
      const bool v = i * NT + tid < nt;
      kmx = v && mk[i] > kmx ? mk[i] : kmx;
      kmn = v && mk[i] < kmn ? mk[i] : kmn;
    }
    kmx = wave_max(kmx);
    kmn = ~wave_max(~kmn);
    if (lane == 0) {
      s_kmx[wave] = kmx;
      s_kmn[wave] = kmn;
    }
    if (tid == 0) {
      s_tiles = 0u;
      s_cands = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
      kmx = s_kmx[w] > kmx ? s_kmx[w] : kmx;
      kmn = s_kmn[w] < kmn ? s_kmn[w] : kmn;
    }
    uint32_t T = 0u;  // every winner's key is >= T, and so is its sub-tile's maximum
    if (K <= nt) {
      const uint32_t span = kmx - kmn;
      const int bits = span ? 32 - __clz(span) : 1;
      const int shift = bits > kDigit ? bits - kDigit : 0;
      clear_bins<NT>(f.hist);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MPT; ++i)
        if (i * NT + tid < nt) atomicAdd(&f.hist[(mk[i] - kmn) >> shift], 1u);
      __syncthreads();
      uint32_t h[kBins / NT];
      load_bins<NT>(f.hist, h);
      find_digit<NT>(h, (uint32_t)K, sh);  // the bin of the K-th largest maximum
      T = kmn + (sh.digit << shift);
    }
    // the sub-tiles whose maximum reaches T, listed in LDS (ballot ranks)
#pragma unroll
    for (int i = 0; i < MPT; ++i) {
      const int j = i * NT + tid;
      const bool pick = j < nt && mk[i] >= T;
      const uint64_t m = __ballot(pick);
      if (m != 0ull) {
        const int leader = __ffsll((unsigned long long)m) - 1;
        uint32_t base = 0u;
        if (lane == leader) base = atomicAdd(&s_tiles, (uint32_t)__popcll(m));
        base = __builtin_amdgcn_readlane(base, leader);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (pick) tlist[base + below] = (uint16_t)j;
      }
    }
    __syncthreads();
    const int ct = (int)s_tiles;
    // their entries at or above T: four lanes per sub-tile, 16 bytes each, LB passes of the
    // workgroup's loads in flight at once; the count runs on past the list's capacity, the
    // writes stop at it
    constexpr int LB = 8;
    for (int w0 = 0; w0 < 4 * ct; w0 += LB * NT) {
      float4v xs[LB];
      int es[LB];
#pragma unroll
      for (int b = 0; b < LB; ++b) {
        const int w = w0 + b * NT + tid;
        xs[b] = float4v{0.f, 0.f, 0.f, 0.f};
        es[b] = 0;
        if (w < 4 * ct) {
          es[b] = 16 * (int)tlist[w >> 2] + 4 * (w & 3);
          xs[b] = *reinterpret_cast<const float4v*>(src + es[b]);
        }
      }
#pragma unroll
      for (int bq = 0; bq < 4 * LB; ++bq) {
        const int b = bq >> 2, q = bq & 3;
        if (w0 + b * NT >= 4 * ct) break;  // uniform: the passes past the list hold nothing
        const int w = w0 + b * NT + tid;
        const int e = es[b] + q;
        const uint32_t key = ord_key(xs[b][q]);
        const bool pick = w < 4 * ct && e < n && key >= T;
        const uint64_t m = __ballot(pick);
        if (m != 0ull) {
          const int leader = __ffsll((unsigned long long)m) - 1;
          uint32_t base = 0u;
          if (lane == leader) base = atomicAdd(&s_cands, (uint32_t)__popcll(m));
          base = __builtin_amdgcn_readlane(base, leader);
          const uint32_t below =
              __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (pick && base + below < (uint32_t)kTileSelCand) cand[base + below] = composite(key - T, (uint32_t)e);
        }
      }
    }
    __syncthreads();
    const uint32_t nc = s_cands;
    if (nc <= (uint32_t)kTileSelCand) {
      C = (int)nc;  // >= K: every winner is listed
      kbase = T;
      const uint32_t rel = kmx - T;  // the largest relative key among the candidates
      const int rbits = rel ? 32 - __clz(rel) : 1;
      thr = radix_select<NT>(each_cand, 0ull, 0ull, (uint32_t)K, 31 + rbits, f.hist, sh);
    } else {
      thr = radix_select<NT>(each_row, 0ull, 0ull, (uint32_t)K, 63, f.hist, sh);
    }
  }
  // gather the winners
  auto each = [&](auto&& fn) {
    if (C >= 0)
      each_cand(fn);
    else
      each_row(fn);
  };
  uint32_t mine = 0;
  uint64_t mx = 0ull, mn = ~0ull;
  each([&](uint64_t c) {
    if (c >= thr) {
      ++mine;
      mx = c > mx ? c : mx;
      mn = c < mn ? c : mn;
    }
  });
  uint32_t off = block_suffix_minmax<NT>(mine, mx, mn, sh);
  each([&](uint64_t c) {
    if (c >= thr && off < (uint32_t)K) f.sortbuf[off++] = c;  // exactly K are selected
  });
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  finish_row<NT>(f.sortbuf, f.grp, f.hist, K, a.top_k, oi, os, mx, mn, sh, kbase);
}

// ------------------------------------------------------------------ long rows

// A chunk's PER entries per thread from lo on, as order keys (0 past n): entry
// lo + i NT + t in register i of thread t, or with VEC (16-byte loads of four
// consecutive entries, a quarter of the load instructions) lo + 4 ((i / 4) NT + t) + i % 4.
template <int PER, bool VEC>
__device__ __forceinline__ int chunk_ent(int lo, int i) {
  constexpr int NT = kChunkThreads;
  return VEC ? lo + 4 * ((i >> 2) * NT + (int)threadIdx.x) + (i & 3) : lo + i * NT + (int)threadIdx.x;
}

// Every load is unconditional, so that all of them are in flight together (a load in a
// branch gets its own wait before the next one is issued): positions past n re-read the
// row's last entry (or quad), and entry 0 when n is 0 (a chunked row is never empty of
// columns), and their keys are 0.
template <int PER, bool VEC>
__device__ __forceinline__ void load_chunk(const float* src, int lo, int n, uint32_t (&key)[PER]) {
  constexpr int NT = kChunkThreads;
  if constexpr (VEC) {
    static_assert(PER % 4 == 0, "vector chunks");
    const int last = n > 0 ? ((n - 1) & ~3) : 0;  // 16-byte aligned: rows and n_cols are
    float4v x[PER / 4];
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const int e0 = lo + 4 * (j * NT + (int)threadIdx.x);
      x[j] = *reinterpret_cast<const float4v*>(src + (e0 < n ? e0 : last));
    }
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const int e0 = lo + 4 * (j * NT + (int)threadIdx.x);
#pragma unroll
      for (int q = 0; q < 4; ++q) key[4 * j + q] = e0 + q < n ? ord_key(x[j][q]) : 0u;
    }
  } else {
    const int last = n > 0 ? n - 1 : 0;
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lo + i * NT + (int)threadIdx.x;
      x[i] = src[e < n ? e : last];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lo + i * NT + (int)threadIdx.x;
      key[i] = e < n ? ord_key(x[i]) : 0u;
    }
  }
}

// Stage 1: the chunk's histogram of the top 12 order-key bits, added into the
// global copy of the XCD the workgroup runs on (workgroups are dealt to the eight
// XCDs round robin by linear index), and the chunk's highest bin into that copy's
// row maximum.
template <int PER, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void select_hist_kernel(SelArgs a) {
  constexpr int NT = kChunkThreads;
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint32_t top_bin;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int lo = blockIdx.x * (PER * NT);
  if (lo >= n) return;
  const float* src = a.scores + (int64_t)row * a.score_stride;
  uint32_t key[PER];  // every load in flight before the first LDS atomic
  load_chunk<PER, VEC>(src, lo, n, key);
  clear_bins<NT>(hist);
  if (tid == 0) top_bin = 0u;
  __syncthreads();
  uint32_t mk = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = chunk_ent<PER, VEC>(lo, i);
    if (e < n) {
      const uint32_t b = key[i] >> (32 - kDigit);
      atomicAdd(&hist[b], 1u);
      mk = b > mk ? b : mk;
    }
  }
  mk = wave_max(mk);
  if ((tid & 63) == 0) atomicMax(&top_bin, mk);
  __syncthreads();
  // every nonzero bin is flushed (a chunk's scores occupy few bins)
  const int copy = (blockIdx.y * gridDim.x + blockIdx.x) % kHistCopies;
  uint32_t* gh = a.ghist + ((int64_t)row * kHistCopies + copy) * kBins;
#pragma unroll
  for (int q = 0; q < kBins / NT; ++q) {
    const int b = q * NT + tid;
    const uint32_t v = hist[b];
    if (v) atomicAdd(&gh[b], v);
  }
  if (tid == 0) atomicMax(&a.gmax[(int64_t)row * kHistCopies + copy], top_bin);
}

// Stage 2: each workgroup finds the bin of its row's K-th entry from the copies,
// scanning down from the row's highest bin (the bins above it are empty), then
// writes every entry of its chunk in that bin or above to the chunk's own
// candidate slots (their order does not matter: the composites are ordered later)
// and the chunk's count to ccount.  The first chunk of the row also records the
// bin for the last stage.
template <int PER, bool VEC>
__global__ __launch_bounds__(kChunkThreads) void select_filter_kernel(SelArgs a) {
  constexpr int NT = kChunkThreads;
  __shared__ SelShared sh;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int lo = blockIdx.x * (PER * NT);
  const int64_t slot = (int64_t)row * gridDim.x + blockIdx.x;
  if (lo >= n && blockIdx.x != 0) {
    if (tid == 0) a.ccount[slot] = 0u;
    return;
  }
  const int K = n < a.top_k ? n : a.top_k;
  // the chunk's scores are loaded first: their latency overlaps the search for the bin
  const float* src = a.scores + (int64_t)row * a.score_stride;
  uint32_t key[PER];
  load_chunk<PER, VEC>(src, lo, n, key);
  RowInfo info{0u, 0u, (uint32_t)n, 0u};  // K == n: every entry is a candidate
  if (K < n) {
    const uint32_t* gm = a.gmax + (int64_t)row * kHistCopies;
    uint32_t mb = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) mb = max(mb, gm[c]);
    mb = min(mb, (uint32_t)(kBins - 1));  // a bin index; never scan past the histogram
    const uint32_t* gh = a.ghist + (int64_t)row * kHistCopies * kBins;
    uint32_t carry = 0;
    if (tid == 0) sh.digit = ~0u;
    for (int base = 0; base <= (int)mb; base += NT) {
      const int b = (int)mb - base - tid;  // thread t: the t-th bin down from the top
      uint32_t v = 0;
      if (b >= 0) {
#pragma unroll
        for (int c = 0; c < kHistCopies; ++c) v += gh[c * kBins + b];
      }
      const uint32_t below_me = block_suffix<NT>(v, sh);  // bins under this one, in this block
      uint32_t total = 0;
#pragma unroll
      for (int w = 0; w < NT / kWave; ++w) total += sh.wsum[w];
      const uint32_t above = carry + (total - below_me - v);
      if (above < (uint32_t)K && above + v >= (uint32_t)K) {
        sh.digit = (uint32_t)b;
        sh.gt = above;
        sh.cnt = v;
      }
      carry += total;
      __syncthreads();
      if (sh.digit != ~0u) break;
    }
    info = RowInfo{sh.digit, sh.gt, sh.cnt, 0u};
  }
  if (blockIdx.x == 0 && tid == 0) a.info[row] = info;
  if (lo >= n) {
    if (tid == 0) a.ccount[slot] = 0u;
    return;
  }
  const uint32_t bin = info.bin;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = chunk_ent<PER, VEC>(lo, i);
    mine += (e < n && (key[i] >> (32 - kDigit)) >= bin);
  }
  uint32_t pos = block_suffix<NT>(mine, sh);
  if (tid == 0) a.ccount[slot] = pos + mine;
  uint64_t* cd = a.cand + slot * (PER * NT);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = chunk_ent<PER, VEC>(lo, i);
    if (e < n && (key[i] >> (32 - kDigit)) >= bin && pos < (uint32_t)(PER * NT))
      cd[pos++] = composite(key[i], (uint32_t)e);
  }
}

// Stage 3 (one workgroup per row): exact selection among the candidates, sort,
// output.  Up to kFinalPer candidates per thread are held in registers, fetched
// through an LDS map from list position to chunk; longer lists (rows crowded with
// equal scores) are read chunk by chunk at every pass.
template <int NT, int PER>
__global__ __launch_bounds__(NT) void select_final_kernel(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = row_valid(a, row);
  const int K = n < a.top_k ? n : a.top_k;
  const RowInfo info = a.info[row];
  const int nch = a.chunks;
  FinishLds f = carve(smem, a.top_k);
  uint32_t* off = f.hist + kBins + 4;                                   // [nch + 1]
  uint16_t* owner = reinterpret_cast<uint16_t*>(off + ((nch + 4) & ~3));  // [NT * PER]
  const uint32_t* cnt = a.ccount + (int64_t)row * nch;
  const uint64_t* cd = a.cand + (int64_t)row * nch * a.chunk;
  const uint32_t first = tid < nch ? cnt[tid] : 0u;
  // exclusive prefix of the chunk counts, 1024 chunks at a time
  uint32_t carry = 0;
  for (int c0 = 0; c0 < nch; c0 += NT) {
    const int c = c0 + tid;
    const uint32_t v = c0 == 0 ? first : c < nch ? cnt[c] : 0u;
    const uint32_t above = block_suffix<NT>(v, sh);
    uint32_t total = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) total += sh.wsum[w];
    if (c < nch) off[c] = carry + (total - above - v);
    carry += total;
    __syncthreads();
  }
  if (tid == 0) off[nch] = carry;
  int C = K == n ? n : (int)(info.above + info.cnt);
  if ((uint32_t)C > carry) C = (int)carry;  // the two agree; never read past the slots
  const bool in_regs = C <= NT * PER;
  uint64_t v[PER];
  if (in_regs) {
    __syncthreads();
    for (int c = tid >> 6; c < nch; c += NT / kWave) {
      const uint32_t o = off[c], e = min(off[c + 1], (uint32_t)C);
      for (uint32_t i = o + (tid & 63); i < e; i += kWave) owner[i] = (uint16_t)c;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = r * NT + tid;
      uint64_t x = 0ull;
      if (i < C) {
        const int c = owner[i];
        const int j = i - (int)off[c];  // in [0, count of chunk c)
        x = (j >= 0 && j < a.chunk) ? cd[(int64_t)c * a.chunk + j] : 0ull;
      }
      v[r] = x;
    }
  } else {
    __syncthreads();
  }
  auto each = [&](auto&& fn) {
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        if (r * NT >= C) break;  // wave-uniform: only the registers that hold candidates
        if (r * NT + tid < C) fn(v[r]);
      }
    } else {
      for (int c = 0; c < nch; ++c) {
        const int m = (int)(off[c + 1] - off[c]);
        for (int i = tid; i < m; i += NT) fn(cd[(int64_t)c * a.chunk + i]);
      }
    }
  };
  uint64_t thr = 0ull;
  if (K < C) {
    const uint64_t mask = (uint64_t)(kBins - 1) << kTopShift;
    thr = radix_select<NT>(each, (uint64_t)info.bin << kTopShift, mask, (uint32_t)K - info.above, kTopShift - 1,
                           f.hist, sh);
  }
  uint32_t mine = 0;
  uint64_t mx = 0ull, mn = ~0ull;
  each([&](uint64_t c) {
    if (c >= thr) {
      ++mine;
      mx = c > mx ? c : mx;
      mn = c < mn ? c : mn;
    }
  });
  uint32_t pos = block_suffix_minmax<NT>(mine, mx, mn, sh);
  each([&](uint64_t c) {
    if (c >= thr && pos < (uint32_t)K) f.sortbuf[pos++] = c;  // exactly K are selected
  });
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)row * a.top_k;
  float* os = a.out_scores ? a.out_scores + (int64_t)row * a.top_k : nullptr;
  finish_row<NT>(f.sortbuf, f.grp, f.hist, K, a.top_k, oi, os, mx, mn, sh);
}

// Zeroes n16 16-byte words (the histogram copies and row maxima of the long-row
// pipeline) ahead of its first stage.
__global__ __launch_bounds__(256) void select_clear_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------------ host planning

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the long-row pipeline: histogram copies and row maxima (zeroed by
// each call before its first stage) | row info | chunk counts | candidate slots.
// Every region is written by the call before it is read: the workspace carries
// nothing from one call to the next.
struct WsLayout {
  size_t hist, gmax, info, ccount, cand, total;
};

static WsLayout ws_layout(int rows, int chunks, int chunk) {
  WsLayout l;
  l.hist = 0;
  l.gmax = (size_t)rows * kHistCopies * kBins * 4;
  l.info = round256(l.gmax + (size_t)rows * kHistCopies * 4);
  l.ccount = round256(l.info + (size_t)rows * sizeof(RowInfo));
  l.cand = round256(l.ccount + (size_t)rows * chunks * 4);
  l.total = round256(l.cand + (size_t)rows * chunks * chunk * 8);
  return l;
}

constexpr size_t kLdsMax = 160 * 1024;
constexpr size_t kStaticLdsReserve = 1024;  // static LDS of the one-workgroup row kernels
// dynamic LDS of a register-row workgroup: two per CU
constexpr size_t kRegRowLds = kLdsMax / 2 - kStaticLdsReserve;

bool plan_select(int rows, int n_cols, int top_k, SelectPlan* p) {
  if (top_k < 1 || top_k > kMaxTopK) return false;
  p->rows = rows;
  p->n_cols = n_cols;
  p->top_k = top_k;
  p->lds = finish_lds_bytes(top_k);
  p->cand_cap = 0;
  if (n_cols <= kRowMax) {
    p->two_pass = 0;
    p->row_nt = kRowThreads;
    p->per = n_cols <= 1024 ? 4 : n_cols <= 2048 ? 8 : n_cols <= 4096 ? 16 : 32;
    p->chunks = 1;
    p->bytes = 0;
  } else if (rows >= kWideRowsMin && n_cols <= 16 * kRowThreadsWide) {
    p->two_pass = 0;  // 1024 threads x 16 registers
    p->row_nt = kRowThreadsWide;
    p->per = 16;
    p->chunks = 1;
    p->bytes = 0;
  } else if (rows >= kWideRowsMin && n_cols <= kRowMaxWide &&
             p->lds + (size_t)16 * top_k <= kRegRowLds) {
    // one workgroup per row, the row in registers; the LDS candidate list takes what
    // two workgroups per CU leave (at least twice top_k)
    p->two_pass = 0;
    p->row_nt = kRowThreadsReg;
    p->per = 0;
    const size_t cap = (kRegRowLds - p->lds) / 8;
    p->cand_cap = (int)(cap < (size_t)kRowMaxWide ? cap : (size_t)kRowMaxWide) & ~1;  // keeps 16-byte alignment
    p->lds += (size_t)p->cand_cap * 8;
    p->chunks = 1;
    p->bytes = 0;
  } else {
    p->two_pass = 1;
    // entries per chunk thread: 16 for many long rows, 4 for very few (more chunks in
    // flight: one 32768-entry row 15.3 -> 14.5 us), else 8
    const int64_t units4k = (int64_t)rows * ((n_cols + 4095) / 4096);
    p->per = units4k >= 1024 ? 16 : units4k < 64 ? 4 : 8;
    const int chunk = p->per * kChunkThreads;
    p->chunks = (n_cols + chunk - 1) / chunk;
    p->bytes = ws_layout(rows, p->chunks, chunk).total;
    // the finishing workgroup also holds the chunk offsets and the position map
    p->final_nt = rows > kFewRows ? kFinalThreadsMany : kFinalThreads;
    const int per = rows > kFewRows ? kFinalPerMany : kFinalPer;
    p->lds += (size_t)4 * ((p->chunks + 4) & ~3) + (size_t)2 * p->final_nt * per;
    if (p->lds > kLdsMax) return false;
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
  return ensure_lds(reinterpret_cast<const void*>(kernel), bytes);
}

template <int NT, int PER>
static hipError_t launch_rows(const SelArgs& a, const SelectPlan& p, hipStream_t st) {
  const bool vec = rows_vec_ok(a);
  hipError_t e = vec ? set_lds(select_rows_kernel<NT, PER, true>, p.lds) : set_lds(select_rows_kernel<NT, PER, false>, p.lds);
  if (e != hipSuccess) return e;
  if (vec)
    hipLaunchKernelGGL((select_rows_kernel<NT, PER, true>), dim3(p.rows), dim3(NT), p.lds, st, a);
  else
    hipLaunchKernelGGL((select_rows_kernel<NT, PER, false>), dim3(p.rows), dim3(NT), p.lds, st, a);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_rows_reg(const SelArgs& a, const SelectPlan& p, hipStream_t st) {
  const bool vec = rows_vec_ok(a);
  hipError_t e = vec ? set_lds(select_rows_reg_kernel<NT, true>, p.lds) : set_lds(select_rows_reg_kernel<NT, false>, p.lds);
  if (e != hipSuccess) return e;
  if (vec)
    hipLaunchKernelGGL((select_rows_reg_kernel<NT, true>), dim3(p.rows), dim3(NT), p.lds, st, a, p.rows);
  else
    hipLaunchKernelGGL((select_rows_reg_kernel<NT, false>), dim3(p.rows), dim3(NT), p.lds, st, a, p.rows);
  return hipGetLastError();
}

template <int PER>
static hipError_t launch_pipeline(const SelArgs& a, const SelectPlan& p, bool counters_zeroed, hipStream_t st) {
  hipError_t e = p.final_nt == kFinalThreads ? set_lds(select_final_kernel<kFinalThreads, kFinalPer>, p.lds)
                                              : set_lds(select_final_kernel<kFinalThreadsMany, kFinalPerMany>, p.lds);
  if (e != hipSuccess) return e;
  if (!counters_zeroed) {
    const int64_t n16 = (int64_t)select_counter_bytes(p) / 16;
    const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 2048);
    hipLaunchKernelGGL(select_clear_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<uint4*>(a.ghist), n16);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid(p.chunks, p.rows);
  if (rows_vec_ok(a)) {
    hipLaunchKernelGGL((select_hist_kernel<PER, true>), grid, dim3(kChunkThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((select_filter_kernel<PER, true>), grid, dim3(kChunkThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((select_hist_kernel<PER, false>), grid, dim3(kChunkThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((select_filter_kernel<PER, false>), grid, dim3(kChunkThreads), 0, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.final_nt == kFinalThreads)
    hipLaunchKernelGGL((select_final_kernel<kFinalThreads, kFinalPer>), dim3(p.rows), dim3(kFinalThreads), p.lds, st,
                       a);
  else
    hipLaunchKernelGGL((select_final_kernel<kFinalThreadsMany, kFinalPerMany>), dim3(p.rows),
                       dim3(kFinalThreadsMany), p.lds, st, a);
  return hipGetLastError();
}

// Bytes at the start of the workspace that the long-row pipeline needs zeroed before
// its first stage (the histogram copies and row maxima); 0 for the one-workgroup rows.
size_t select_counter_bytes(const SelectPlan& p) {
  if (!p.two_pass) return 0;
  return ws_layout(p.rows, p.chunks, p.per * kChunkThreads).info;
}

bool tile_select_fits(int n_cols, int top_k) {
  return n_cols >= 1 && n_cols <= kRowMaxWide && top_k >= 1 && top_k <= kTileSelMaxK;
}

hipError_t launch_select_tiles(const float* scores, int64_t score_stride, const uint32_t* tmax, int64_t tmax_stride,
                               int64_t first_pos, int ratio, int rows, int n_cols, int top_k, int32_t* out_idx,
                               float* out_scores, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  SelArgs a{};
  a.scores = scores;
  a.score_stride = score_stride;
  a.first_pos = first_pos;
  a.ratio = ratio;
  a.n_cols = n_cols;
  a.top_k = top_k;
  a.out_idx = out_idx;
  a.out_scores = out_scores;
  a.tmax = tmax;
  a.tmax_stride = tmax_stride;
  const size_t lds = (size_t)kTileSelCand * 8 + (size_t)kTileSelTiles * 2 + finish_lds_bytes(top_k);
  hipError_t e = set_lds(select_tiles_kernel<kTileSelThreads>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((select_tiles_kernel<kTileSelThreads>), dim3(rows), dim3(kTileSelThreads), lds, st, a, rows);
  return hipGetLastError();
}

hipError_t launch_select(const SelectPlan& p, const float* scores, int64_t score_stride,
                         const int32_t* valid_lens, int64_t first_pos, int ratio, int32_t* out_idx,
                         float* out_scores, void* ws, bool counters_zeroed, hipStream_t st) {
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
  a.cand_cap = p.cand_cap;
  if (!p.two_pass) {
    if (p.row_nt == kRowThreadsReg) return launch_rows_reg<kRowThreadsReg>(a, p, st);
    if (p.row_nt == kRowThreadsWide) return launch_rows<kRowThreadsWide, 16>(a, p, st);
    switch (p.per) {
      case 4: return launch_rows<kRowThreads, 4>(a, p, st);
      case 8: return launch_rows<kRowThreads, 8>(a, p, st);
      case 16: return launch_rows<kRowThreads, 16>(a, p, st);
      default: return launch_rows<kRowThreads, 32>(a, p, st);
    }
  }
  a.chunk = p.per * kChunkThreads;
  a.chunks = p.chunks;
  const WsLayout l = ws_layout(p.rows, p.chunks, a.chunk);
  unsigned char* w = static_cast<unsigned char*>(ws);
  a.ghist = reinterpret_cast<uint32_t*>(w + l.hist);
  a.gmax = reinterpret_cast<uint32_t*>(w + l.gmax);
  a.info = reinterpret_cast<RowInfo*>(w + l.info);
  a.ccount = reinterpret_cast<uint32_t*>(w + l.ccount);
  a.cand = reinterpret_cast<uint64_t*>(w + l.cand);
  if (p.per == 4) return launch_pipeline<4>(a, p, counters_zeroed, st);
  return p.per == 16 ? launch_pipeline<16>(a, p, counters_zeroed, st) : launch_pipeline<8>(a, p, counters_zeroed, st);
}

}  // namespace salb
