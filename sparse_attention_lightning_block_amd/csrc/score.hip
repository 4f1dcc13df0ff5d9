// Lightning-indexer scorers for gfx950.
//
//   I[t, s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[t,s,:] )
// ([listing] "nvfp4-megamoe-kernel -- .../indexer_score_topk.cu": header comment, eq. 16,
// and the scoring loop of its main kernel), with the NVFP4 keys of a paged pool
// resolved through a per-query block table (same page, main kernel).
//
// The scorers share the work decomposition -- a workgroup owns one query row (or a
// group of four) and a contiguous chunk of its logical keys; chunks are spread over
// the XCDs so that all rows of one chunk run on the same XCD (shared pages hit one
// L2):
//
//  * the MFMA scorers (IDX_PREC_MFMA) run the head x key contraction on the fp16
//    matrix cores.  A 16x16x32 MFMA takes 16 heads (M) x 32 dims (K) of q from
//    registers and 32 dims x 16 keys (N) of decoded NVFP4 keys.  The K order inside
//    an instruction is a fixed permutation of the head dims applied to both
//    operands, chosen so that every lane's key slice is contiguous.  The epilogue
//    applies ReLU, the head weights and the per-page global scale to the fp32
//    accumulators, reduces the heads in the lane and then over the lane quarters with
//    row swaps on the VALU (four 16-key steps together: three swaps), and writes the
//    four steps' 64 scores in one store.  q is prescaled per head by a power of two so that its fp16
//    rounding is relative (11 bits); the inverse power is folded into the head
//    weight, which keeps the result identical up to that rounding.
//      - score_mfma_split_kernel (fewer than four rows): every wave streams its own
//        keys of the row through a ring of eight raw steps; each lane decodes its
//        16-byte slice of one key straight into the B operand (no LDS trip).
//      - score_mfma_group_kernel (four rows or more): four rows per workgroup (eight
//        from sixteen rows on), one per wave; when the rows resolve the chunk to the
//        same pages, each 64-key tile is decoded once into LDS (every thread decodes
//        a 1/G slice of a key) and read by all the waves.
//  * score_f32mfma_kernel (IDX_PREC_FP32, D 64/128): the same contraction in fp32 on
//    the fp32 matrix cores, for results within ~1e-5 relative; score_f32_kernel (D 256):
//    one key per lane, fp32 FMAs with q read through the scalar cache.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "nvfp4.hpp"

// Workgroups to aim for when cutting rows into key chunks (build-time tunables).
#ifndef SALB_GROUP_WGS
#define SALB_GROUP_WGS 256
#endif
#ifndef SALB_SPLIT_WGS
#define SALB_SPLIT_WGS 1024
#endif
// LDS for the block-table entries of a balanced group-scorer segment.
constexpr int kBalancePidBytes = 48 * 1024;
// Rows per workgroup of the group scorer once a call has sixteen rows or more (4 or 8).
#ifndef SALB_GROUP_ROWS
#define SALB_GROUP_ROWS 8
#endif

namespace salb {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float load_q(const void* q, int bf16, int64_t i) {
  if (bf16) {
    uint32_t b = reinterpret_cast<const uint16_t*>(q)[i];
    return __uint_as_float(b << 16);
  }
  return reinterpret_cast<const float*>(q)[i];
}

// The words a launch zeroes besides its scores, spread over the whole grid (every
// workgroup runs this before any early exit).
__device__ __forceinline__ void zero_side_words(const ScoreArgs& a, int nt) {
  if (a.zero_n16 == 0) return;
  const int64_t step = (int64_t)gridDim.x * nt;
  for (int64_t i = (int64_t)blockIdx.x * nt + threadIdx.x; i < a.zero_n16; i += step)
    a.zero_ptr[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Power-of-two exponent j with max|x| * 2^j in [2^14, 2^15) (0 for zero/non-finite).
__device__ __forceinline__ int prescale_exp(float mx) {
  if (!(mx > 0.0f) || !(mx < 3.0e38f)) return 0;
  int e;
  frexpf(mx, &e);
  int j = 15 - e;
  return j < -100 ? -100 : (j > 100 ? 100 : j);
}

// ------------------------------------------------------------------ MFMA scorer

// Raw bytes of a DIMS-dim slice of one key: DIMS/2 code bytes and its E4M3 scale
// bytes (DIMS/16 of them; an 8-dim slice shares its 16-dim group's byte).
template <int DIMS>
struct Slice {
  uint32_t w[DIMS / 8];
  uint32_t sc;
};

template <int DIMS>
__device__ __forceinline__ void load_slice(Slice<DIMS>& r, const uint8_t* codes, const uint8_t* scales) {
  if constexpr (DIMS == 8) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(codes);
    r.sc = *scales;
  } else if constexpr (DIMS == 16) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(codes);
    r.w[0] = v[0];
    r.w[1] = v[1];
    r.sc = *scales;
  } else if constexpr (DIMS == 32) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes);
    r.w[0] = v[0];
    r.w[1] = v[1];
    r.w[2] = v[2];
    r.w[3] = v[3];
    r.sc = *reinterpret_cast<const uint16_t*>(scales);
  } else {
    static_assert(DIMS == 64, "slice width");
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(codes);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(codes + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.w[i] = v0[i];
      r.w[4 + i] = v1[i];
    }
    r.sc = *reinterpret_cast<const uint32_t*>(scales);
  }
}

// Eight fp16 code values of step kk (dims 8 kk .. 8 kk + 7) of a raw slice; the sign
// of the page's global scale is folded into the exact fp16 group scale
// (ReLU(g x) = |g| ReLU(sign(g) x)).
template <int DIMS>
__device__ __forceinline__ half8v decode_slice(const Slice<DIMS>& r, int kk, float sgn) {
  const _Float16 sh = (_Float16)(e4m3_to_f32((r.sc >> (8 * (kk >> 1))) & 0xffu) * sgn);
  const half2v s2 = {sh, sh};
  return decode8_f16(r.w[kk], s2);
}

// A lane's quarter of a key in the streaming scorer.
template <int D>
using Raw = Slice<D / 4>;

template <int D>
__device__ __forceinline__ void load_raw(Raw<D>& r, const uint8_t* codes, const uint8_t* scales) {
  load_slice<D / 4>(r, codes, scales);
}

template <int D>
__device__ __forceinline__ half8v decode_step(const Raw<D>& r, int kk, float sgn) {
  return decode_slice<D / 4>(r, kk, sgn);
}

// Work tile of a workgroup over (key chunk, row unit): with enough chunks per row,
// chunks are grouped by XCD (units sharing pages hit one L2); otherwise units are
// spread round-robin over the XCDs, highest (longest causal) rows first.
__device__ __forceinline__ XcdTile score_tile(const ScoreArgs& a, int units) {
  if (a.swizzle) return xcd_tile(blockIdx.x, units);
  XcdTile t;
  t.chunk = (int)blockIdx.x / units;
  t.row = units - 1 - ((int)blockIdx.x % units);
  return t;
}

// Raw query of row t as loaded: lane (col, quarter) holds, for M-tile mt and K-step kk,
// q[16 mt + col][quarter * D/4 + 8 kk .. + 8] (eight bf16 in raw[mt][kk][0], or eight
// fp32 in raw[mt][kk][0..1]), and the weights of accumulator rows 16 mt + 4 quarter + i.
// Issuing these loads apart from the conversion lets the page loads of the segment go
// out while they are in flight.  Queries past T get zeros.
template <int MT, int D>
struct QueryRaw {
  u32x4 q[MT][D / 32][2];
  float w[MT][4];
};

template <int MT, int D>
__device__ __forceinline__ void issue_query(const ScoreArgs& a, int t, int lane, QueryRaw<MT, D>& r) {
  constexpr int KW = D / 32;
  const int col = lane & 15, quarter = lane >> 4;
  const bool has = t < a.T;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + col;
    const bool hv = has && h < a.H;
    const int64_t base = ((int64_t)t * a.H + h) * D + quarter * (D / 4);
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      r.q[mt][kk][0] = u32x4{0u, 0u, 0u, 0u};
      r.q[mt][kk][1] = u32x4{0u, 0u, 0u, 0u};
      if (hv) {
        if (a.q_bf16) {
          r.q[mt][kk][0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + base + kk * 8);
        } else {
          const float* src = reinterpret_cast<const float*>(a.q) + base + kk * 8;
          r.q[mt][kk][0] = *reinterpret_cast<const u32x4*>(src);
          r.q[mt][kk][1] = *reinterpret_cast<const u32x4*>(src + 4);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hr = mt * 16 + quarter * 4 + i;
      r.w[mt][i] = (has && hr < a.H) ? a.w[(int64_t)t * a.H + hr] : 0.0f;
    }
  }
}

// A operands (per-head power-of-two prescaled fp16 q) and accumulator-row weights from
// the raw query.  Row i of accumulator quarter q of tile mt is head 16 mt + 4 q + i; the
// head's max over its D dims spans the four quarter lanes.
template <int MT, int D>
__device__ __forceinline__ void convert_query(const ScoreArgs& a, const QueryRaw<MT, D>& r,
                                              half8v (&A)[MT][D / 32], float (&wr)[MT][4], int lane) {
  constexpr int KW = D / 32;
  const int quarter = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float v[KW][8];
    float mx = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      if (a.q_bf16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[kk][2 * e] = __uint_as_float(r.q[mt][kk][0][e] << 16);
          v[kk][2 * e + 1] = __uint_as_float(r.q[mt][kk][0][e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[kk][e] = __uint_as_float(r.q[mt][kk][0][e]);
          v[kk][4 + e] = __uint_as_float(r.q[mt][kk][1][e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[kk][e]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int j = prescale_exp(mx);  // exponent of head 16 mt + col
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      half8v hv8;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv8[e] = (_Float16)ldexpf(v[kk][e], j);
      A[mt][kk] = hv8;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jr = __shfl(j, quarter * 4 + i);
      wr[mt][i] = ldexpf(r.w[mt][i], -jr);
    }
  }
}

template <int MT, int D>
__device__ __forceinline__ void load_query(const ScoreArgs& a, int t, int lane, half8v (&A)[MT][D / 32],
                                           float (&wr)[MT][4]) {
  QueryRaw<MT, D> r;
  issue_query<MT, D>(a, t, lane, r);
  convert_query<MT, D>(a, r, A, wr, lane);
}

template <int MT>
__device__ __forceinline__ void zero_acc(float4v (&acc)[MT]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = float4v{0.f, 0.f, 0.f, 0.f};
}

// Head reduction of one 16-key step: in-lane over 4*MT heads, then across the four
// lane quarters; every lane ends with the total of its key column (lane & 15).
template <int MT>
__device__ __forceinline__ float head_part(const float4v (&acc)[MT], const float (&wr)[MT][4]) {
  float part = 0.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(wr[mt][i], relu_bits(acc[mt][i]), part);
  return part;
}

template <int MT>
__device__ __forceinline__ float head_sum(const float4v (&acc)[MT], const float (&wr)[MT][4]) {
  return row_sum4(head_part<MT>(acc, wr));
}

// Head reduction and store of one step: lanes 0..15 store its 16 scores (keys below
// s_vend only).
template <int MT>
__device__ __forceinline__ void epilogue(const float4v (&acc)[MT], const float (&wr)[MT][4], float gabs, int s0,
                                         int s_vend, float* out_row, int lane) {
  const float part = head_sum<MT>(acc, wr);
  const int s = s0 + (lane & 15);
  if (lane < 16 && s < s_vend) out_row[s] = gabs * part;
}

// One wave streams the 16-key steps first, first + stride, ... of [s_begin, s_vend)
// for one query, decoding each lane's key slice straight into the B operand.  Loads
// run seven steps ahead (ring of eight raw buffers); the epilogue of step i-1 is issued
// beside the MFMAs of step i (two accumulator sets).  pid/pgs hold the page ids and
// global scales of the logical blocks from lb0 on.
template <int MT, int D, bool UPAGE>
__device__ __forceinline__ void wave_stream(const ScoreArgs& a, const half8v (&A)[MT][D / 32],
                                            const float (&wr)[MT][4], const int* pid, const float* pgs, int lb0,
                                            int s_begin, int s_vend, int first, int stride, float* out_row,
                                            int lane) {
  constexpr int KW = D / 32;
  // the wave's bounds in scalar registers: every branch and trip count below is scalar
  s_begin = __builtin_amdgcn_readfirstlane(s_begin);
  s_vend = __builtin_amdgcn_readfirstlane(s_vend);
  first = __builtin_amdgcn_readfirstlane(first);
  stride = __builtin_amdgcn_readfirstlane(stride);
  const int n_vg = (s_vend - s_begin + 15) >> 4;
  if (first >= n_vg) return;
  const int col = lane & 15, quarter = lane >> 4;
  const uint32_t lane_codes = (uint32_t)(quarter * (D / 8));
  const uint32_t lane_scales = (uint32_t)(quarter * (D / 64));

  auto load_step = [&](int gi, Raw<D>& r, float& g) {
    const int gc = min(gi, n_vg - 1);  // past the end: re-read valid memory, result unused
    const int s0 = s_begin + gc * 16;
    const int s = min(s0 + col, s_vend - 1);
    if constexpr (UPAGE) {
      const uint32_t lb = div_epb((uint32_t)s0, a.epb_magic);
      const int li = (int)lb - lb0;
      const int p = __builtin_amdgcn_readfirstlane(pid[li]);
      g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(pgs[li])));
      const uint32_t slot = (uint32_t)s - lb * (uint32_t)a.epb;
      const uint8_t* kb = a.keys + (int64_t)p * a.epb * (D / 2);
      const uint8_t* sb = a.kscale + (int64_t)p * a.epb * (D / 16);
      load_raw<D>(r, kb + (slot * (D / 2) + lane_codes), sb + (slot * (D / 16) + lane_scales));
    } else {
      const uint32_t lb = div_epb((uint32_t)s, a.epb_magic);
      const int li = (int)lb - lb0;
      const int p = pid[li];
      g = pgs[li];
      const int64_t e = (int64_t)p * a.epb + (int64_t)((uint32_t)s - lb * (uint32_t)a.epb);
      load_raw<D>(r, a.keys + e * (D / 2) + lane_codes, a.kscale + e * (D / 16) + lane_scales);
    }
  };
  auto compute = [&](const Raw<D>& r, float g, float4v (&acc)[MT]) {
    const float sgn = g < 0.0f ? -1.0f : 1.0f;
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      const half8v B = decode_step<D>(r, kk, sgn);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][kk], B, kk == 0 ? float4v{0.f, 0.f, 0.f, 0.f} : acc[mt],
                                                         0, 0, 0);
    }
  };

  // ring of raw steps: step i lives in slot i % kRing from its load, kRing - 1 steps
  // ahead of its MFMAs, until its decode
  constexpr int kRing = 8;
  Raw<D> R[kRing];
  float G[kRing];
  float4v AC0[MT], AC1[MT];
  zero_acc<MT>(AC1);
  int gi = first;
  // issued in ring order (the scheduler may not reorder them): the waits in the loop
  // count on step u's loads being older than those of the steps after it
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) {
    load_step(gi + u * stride, R[u], G[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Four steps make a group: each step leaves its in-lane head sum times the key's
  // |global scale| in p[q] (q = its place in the group), and once the group is complete
  // the four are reduced over the lane quarters together, so that lane (col, q) ends
  // with key col of step q and the group leaves in one store.  sg is the first key of
  // the group's step 0 (a value past s_vend masks the whole store: nothing pending yet).
  float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
  float g_last = 0.0f;  // |global scale| of the last step's key (its ring slot is reloaded first)
  int sg = 0x3fffffff;
  auto flush = [&]() {
    const float sc = row_transpose_sum4(p0, p1, p2, p3);
    const int s = sg + quarter * stride * 16 + col;
    if (s < s_vend) out_row[s] = sc;
  };
  // kRing steps per trip and a single exit (the trip count): steps past this wave's last
  // only reload the ring.  A loop left from the middle of its body would reach its header
  // on paths with other loads outstanding, and the waits placed there would drain the ring.
  const int n_mine = (n_vg - first + stride - 1) / stride;  // >= 1
  const int n_trips = (n_mine + kRing - 1) / kRing;
  for (int trip = 0; trip < n_trips; ++trip) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      load_step(gi + (kRing - 1) * stride, R[(u + kRing - 1) % kRing], G[(u + kRing - 1) % kRing]);
      if (gi < n_vg) {
        // step u multiplies into AC0 when u is even, into AC1 when odd, beside the head
        // sum of the step before it
        float prev;
        if (u & 1) {
          compute(R[u], G[u], AC1);
          prev = g_last * head_part<MT>(AC0, wr);
        } else {
          compute(R[u], G[u], AC0);
          prev = g_last * head_part<MT>(AC1, wr);
        }
        switch ((u + 3) & 3) {
          case 0: p0 = prev; break;
          case 1: p1 = prev; break;
          case 2: p2 = prev; break;
          default: p3 = prev; break;
        }
        if ((u & 3) == 0) {  // the step before completed a group
          flush();
          sg = s_begin + gi * 16;
        }
        g_last = fabsf(G[u]);
      }
      gi += stride;
    }
  }
  // the last step's head sum (its accumulators by the parity of its ring slot), then
  // its group; the group's places past it hold keys past s_vend and are masked
  const int u_last = (n_mine - 1) % kRing;
  const float pl = g_last * ((u_last & 1) ? head_part<MT>(AC1, wr) : head_part<MT>(AC0, wr));
  const int q_last = u_last & 3;
  p0 = q_last == 0 ? pl : p0;
  p1 = q_last == 1 ? pl : p1;
  p2 = q_last == 2 ? pl : p2;
  p3 = q_last == 3 ? pl : p3;
  flush();
}

// Loads the page ids and global scales of logical blocks lb0 .. lb0 + n - 1 of row t.
__device__ __forceinline__ void load_pages(const ScoreArgs& a, int t, int lb0, int n, int* pid, float* pgs, int i0,
                                           int step) {
  const int32_t* bt_row = a.bt + (int64_t)t * a.bt_stride;
  for (int i = i0; i < n; i += step) {
    const int p = bt_row[lb0 + i];
    pid[i] = p;
    pgs[i] = a.gscale[p];
  }
}

// Split scorer: one query per workgroup, the chunk's 16-key steps dealt round-robin
// to the four waves.  Used when there are fewer than four query rows.
template <int MT, int D, bool UPAGE>
__global__ __launch_bounds__(256) void score_mfma_split_kernel(ScoreArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* pid = reinterpret_cast<int*>(smem);
  float* pgs = reinterpret_cast<float*>(pid + a.pid_cap);
  zero_side_words(a, 256);

  const XcdTile tile = score_tile(a, a.T);
  if (tile.chunk >= a.n_chunks) return;
  const int t = tile.row;
  const int valid = a.valid_lens[t];
  const int s_begin = tile.chunk * a.chunk;
  const int s_lim = a.write_tail ? a.n_cols : valid;
  if (s_begin >= s_lim) return;
  const int s_end = min(s_begin + a.chunk, s_lim);
  const int s_vend = min(s_end, valid);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* out_row = a.scores + (int64_t)t * a.score_stride;
  for (int s = max(s_vend, s_begin) + tid; s < s_end; s += 256) out_row[s] = -INFINITY;
  if (s_vend <= s_begin) return;

  const int lb0 = (int)div_epb((uint32_t)s_begin, a.epb_magic);
  const int npages = (int)div_epb((uint32_t)(s_vend - 1), a.epb_magic) - lb0 + 1;
  load_pages(a, t, lb0, npages, pid, pgs, tid, 256);
  half8v A[MT][D / 32];
  float wr[MT][4];
  load_query<MT, D>(a, t, lane, A, wr);
  __syncthreads();
  wave_stream<MT, D, UPAGE>(a, A, wr, pid, pgs, lb0, s_begin, s_vend, wave, 4, out_row, lane);
}

// Group scorer: a workgroup scores four query rows (one per wave) over one chunk of
// keys.  For up to 256 rows, the rows are grouped by decreasing valid length, so the
// four rows of a workgroup end at about the same key.  When the four rows resolve the
// chunk to the same pages (one sequence; checked at run time) each 64-key tile is
// decoded ONCE into LDS as fp16 MFMA B operands and read by all four waves -- a
// quarter of the decode work and of the key traffic per row -- and the decode of tile
// j+1 is spread between the MFMA steps of tile j.  Otherwise every wave streams its
// own row.
template <int MT, int D, bool UPAGE, int G>
__global__ __launch_bounds__(64 * G) void score_mfma_group_kernel(ScoreArgs a) {
  constexpr int NT = 64 * G;  // one wave per row of the group
  constexpr int KW = D / 32;
  constexpr int SD = D / G;   // dims of a key each staging thread loads and decodes
  constexpr int SW = SD / 8;  // its eight-dim steps
  constexpr int LG = G == 8 ? 3 : 2;
  static_assert(G == 4 || G == 8, "group size");
  constexpr int BLD = D + 8;  // LDS row of one decoded key (halves), padded against bank conflicts
  constexpr int TILE = 64;
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* bbuf = reinterpret_cast<_Float16*>(smem);                          // [2][TILE][BLD]
  float* gbuf = reinterpret_cast<float*>(smem + 2 * TILE * BLD * 2);           // [2][TILE]
  int* pid = reinterpret_cast<int*>(gbuf + 2 * TILE);                          // [G][pid_cap]
  float* pgs = reinterpret_cast<float*>(pid + G * a.pid_cap);                  // [G][pid_cap]
  __shared__ int s_vend_w[G];
  __shared__ int s_mismatch;
  __shared__ int s_valid[256];
  __shared__ int s_order[256];
  const int units = (a.T + G - 1) / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  zero_side_words(a, NT);

  // Scores of this wave's row t over keys [s_begin, s_cap); with tail, the part of
  // that range past the row's valid length gets -inf.  Every wave of the workgroup
  // calls it with the same key range.
  auto run_segment = [&](int t, const int s_begin, const int s_cap, const bool tail) {
    // one row per wave: keep the row and its bounds in scalar registers, so that every
    // branch on them below is a scalar branch
    t = __builtin_amdgcn_readfirstlane(t);
    const bool has = t < a.T;
    // the query loads go out first: they need only the row, and the valid length, the
    // block table and the global scales are fetched under them
    QueryRaw<MT, D> qraw;
    issue_query<MT, D>(a, t, lane, qraw);
    const int valid = has ? a.valid_lens[t] : 0;
    const int s_end = !has ? s_begin : tail ? min(s_cap, a.n_cols) : max(s_begin, min(s_cap, valid));
    const int s_vend = max(s_begin, min(s_end, valid));
    float* out_row = a.scores + (int64_t)(has ? t : 0) * a.score_stride;
    for (int s = s_vend + lane; s < s_end; s += 64) out_row[s] = -INFINITY;

    // pages of each row (loads issued before the query's); the row reaching furthest leads
    const int lb0 = (int)div_epb((uint32_t)s_begin, a.epb_magic);
    const int np = s_vend > s_begin ? (int)div_epb((uint32_t)(s_vend - 1), a.epb_magic) - lb0 + 1 : 0;
    int* mypid = pid + wave * a.pid_cap;
    float* mypgs = pgs + wave * a.pid_cap;
    const int32_t* bt_row = a.bt + (int64_t)t * a.bt_stride;
    const int p_first = lane < np ? bt_row[lb0 + lane] : 0;
    // global scales of the first 64 pages (entry 0 of the pool stands in for lanes past
    // the row's pages), then the query conversion
    const float g_first = a.gscale[lane < np ? p_first : 0];
    half8v A[MT][KW];
    float wr[MT][4];
    convert_query<MT, D>(a, qraw, A, wr, lane);
    if (lane < np) {
      mypid[lane] = p_first;
      mypgs[lane] = g_first;
    }
    for (int i = lane + 64; i < np; i += 64) {
      const int p = bt_row[lb0 + i];
      mypid[i] = p;
      mypgs[i] = a.gscale[p];
    }
    if (lane == 0) s_vend_w[wave] = s_vend;
    if (tid == 0) s_mismatch = 0;
    __syncthreads();
    int lead = 0, vmax = s_vend_w[0];
#pragma unroll
    for (int w = 1; w < G; ++w)
      if (s_vend_w[w] > vmax) { vmax = s_vend_w[w]; lead = w; }
    if (vmax <= s_begin) return;  // no key of this chunk is valid for any of the rows
    {
      const int* lp = pid + lead * a.pid_cap;
      bool diff = false;
      for (int i = lane; i < np; i += 64) diff |= mypid[i] != lp[i];
      if (__ballot(diff) != 0ull && lane == 0) s_mismatch = 1;
    }
    __syncthreads();

    if (s_mismatch) {  // rows of different sequences: each wave streams its own row
      wave_stream<MT, D, UPAGE>(a, A, wr, mypid, mypgs, lb0, s_begin, s_vend, 0, 1, out_row, lane);
      return;
    }

    // ---- shared pages: decode each 64-key tile once into LDS
    const int* lpid = pid + lead * a.pid_cap;
    const float* lpgs = pgs + lead * a.pid_cap;
    const int n_tiles = (vmax - s_begin + TILE - 1) / TILE;
    // staging: key kt of the tile, slice qs (dims qs*SD .. qs*SD + SD - 1) of it.  Each
    // group of eight lanes writes eight different keys (same slice), whose LDS rows start
    // on distinct bank groups (the row pitch is an odd number of 16-byte granules):
    // conflict-free writes.
    const int kt = (tid & 7) | ((tid >> (3 + LG)) << 3), qs = (tid >> 3) & (G - 1);
    // Raw tiles in flight: tile i lives in ring slot i % 4 from its load (issued four
    // tiles ahead, so that about 18 KB per workgroup are in flight) until its decode,
    // one tile before it is used.  Loads and decodes past the last tile touch valid
    // memory and a free buffer; their results are unused.
    Slice<SD> R0, R1, R2, R3;
    float G0 = 0.0f, G1 = 0.0f, G2 = 0.0f, G3 = 0.0f;
    auto load_tile = [&](int j, Slice<SD>& raw, float& graw) {
      const int s = min(s_begin + j * TILE + kt, vmax - 1);
      const uint32_t lb = div_epb((uint32_t)s, a.epb_magic);
      const int p = lpid[(int)lb - lb0];
      graw = lpgs[(int)lb - lb0];
      const int64_t e = (int64_t)p * a.epb + (int64_t)((uint32_t)s - lb * (uint32_t)a.epb);
      load_slice<SD>(raw, a.keys + e * (D / 2) + qs * (SD / 2), a.kscale + e * (D / 16) + (qs * SD) / 16);
    };
    // Steps [k0, k1) of this thread's slice of a raw tile into LDS buffer buf.
    auto decode_part = [&](int buf, const Slice<SD>& raw, float graw, int k0, int k1) {
      const float sgn = graw < 0.0f ? -1.0f : 1.0f;
      _Float16* dst = bbuf + (buf * TILE + kt) * BLD + qs * SD;
#pragma unroll
      for (int kk = k0; kk < k1; ++kk) *reinterpret_cast<half8v*>(dst + kk * 8) = decode_slice<SD>(raw, kk, sgn);
      if (k1 == SW && qs == 0) gbuf[buf * TILE + kt] = fabsf(graw);
    };

    const int col = lane & 15, quarter = lane >> 4;
    float4v AC0[MT], AC1[MT];
    zero_acc<MT>(AC1);
    // Each step leaves one in-lane head sum per lane (its quarter's heads, key column
    // lane & 15); the four steps of a tile are reduced over the quarters together, so
    // that lane l ends with key l of the tile (step = lane quarter) and the tile leaves
    // in one 256-byte store.  Step 3 of a tile is reduced at the start of the next one,
    // beside its MFMAs.
    int t_prev = 0x3fffffff;  // previous tile (none yet: its store is masked off)
    float g_prev = 0.0f;      // |global scale| of key t_prev + lane
    float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f;
    // B operands of step k, read from LDS one step before their MFMAs: the reads of
    // step k+1 are in flight while step k multiplies (only step 0 of a tile, which
    // follows the barrier, waits for its own reads).
    half8v BA[KW], BB[KW];
    auto read_b = [&](int buf, int k, half8v (&B)[KW]) {
      const _Float16* src = bbuf + (buf * TILE + k * 16 + col) * BLD + quarter * (D / 4);
#pragma unroll
      for (int kk = 0; kk < KW; ++kk) B[kk] = *reinterpret_cast<const half8v*>(src + kk * 8);
    };
    auto mfma_step = [&](const half8v (&B)[KW], float4v (&acc)[MT]) {
#pragma unroll
      for (int kk = 0; kk < KW; ++kk)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              A[mt][kk], B[kk], kk == 0 ? float4v{0.f, 0.f, 0.f, 0.f} : acc[mt], 0, 0, 0);
    };
    // Interleave a step's MFMAs with the other work of its block: one MFMA and two VALU
    // instructions at a time, with the next step's B reads spread over the first MFMAs.
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < KW * MT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < KW) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    };
    auto flush_prev = [&]() {
      const float sc = row_transpose_sum4(p0, p1, p2, head_part<MT>(AC1, wr));
      if (t_prev + lane < s_vend) out_row[t_prev + lane] = g_prev * sc;
    };
    // One tile: score tile j from LDS while decoding tile j+1 from its ring slot (`nx`)
    // into the other buffer and reloading this tile's slot (`mine`) four tiles ahead.
    auto run_tile = [&](int j, Slice<SD>& mine, float& gmine, const Slice<SD>& nx, float gnx) {
      __syncthreads();  // tile j decoded; the other buffer is free again
      const int buf = j & 1;
      const int t0 = s_begin + j * TILE;
      // Rows done before the tile (a wave-uniform, scalar condition) skip its MFMAs but
      // still share the decode and the loads, which run in one fixed order on every
      // path: the outstanding loads are then the same wherever the waits are placed.
      const bool act = t0 < s_vend;
      float g_lane = 0.0f;
      if (act) {
        g_lane = gbuf[buf * TILE + lane];
        read_b(buf, 0, BA);
        read_b(buf, 1, BB);
        mfma_step(BA, AC0);
        flush_prev();
        interleave();
      }
      decode_part(buf ^ 1, nx, gnx, 0, SW / 2);
      if (act) {
        read_b(buf, 2, BA);
        mfma_step(BB, AC1);
        p0 = head_part<MT>(AC0, wr);
        interleave();
      }
      decode_part(buf ^ 1, nx, gnx, SW / 2, SW);
      if (act) {
        read_b(buf, 3, BB);
        mfma_step(BA, AC0);
        p1 = head_part<MT>(AC1, wr);
        interleave();
      }
      load_tile(j + 4, mine, gmine);
      if (act) {
        mfma_step(BB, AC1);
        p2 = head_part<MT>(AC0, wr);
        interleave();
        t_prev = t0;
        g_prev = g_lane;
      }
    };

    load_tile(0, R0, G0);
    load_tile(1, R1, G1);
    load_tile(2, R2, G2);
    load_tile(3, R3, G3);
    decode_part(0, R0, G0, 0, SW);
    for (int j = 0; j < n_tiles; j += 4) {
      run_tile(j, R0, G0, R1, G1);
      if (j + 1 >= n_tiles) break;
      run_tile(j + 1, R1, G1, R2, G2);
      if (j + 2 >= n_tiles) break;
      run_tile(j + 2, R2, G2, R3, G3);
      if (j + 3 >= n_tiles) break;
      run_tile(j + 3, R3, G3, R0, G0);
    }
    flush_prev();
  };

  int64_t lo = 0, hi = 0;  // balanced: this workgroup's stretch of the total weight
  auto unit_tiles = [&](int u, int& n, int& m) {
    n = (s_valid[s_order[u * G]] + TILE - 1) / TILE;
    m = (G > 4 && u * G + 4 < a.T) ? (s_valid[s_order[u * G + 4]] + TILE - 1) / TILE : 0;
  };
  if (a.balance) {
    // Balanced split (at most 256 rows).  Rows are ranked by valid length (clamped to
    // n_cols) and cut into units of G, so that each unit holds rows of similar length.
    // A unit's 64-key tiles up to its longest row weigh 2, plus 1 while five rows or
    // more are still active (those tiles keep two waves busy on some SIMD); the grid
    // splits the total weight evenly, every workgroup one contiguous stretch of it,
    // which may run over a few units.
    for (int i = tid; i < a.T; i += NT) s_valid[i] = min(max(a.valid_lens[i], 0), a.n_cols);
    __syncthreads();
    if (tid < a.T) {
      const int v = s_valid[tid];
      int rank = 0;
      for (int i = 0; i < a.T; ++i) {
        const int vi = s_valid[i];
        rank += (vi > v) || (vi == v && i < tid);
      }
      s_order[rank] = tid;
    }
    __syncthreads();
    int64_t total = 0;
    for (int u = 0; u < units; ++u) {
      int n, m;
      unit_tiles(u, n, m);
      total += 2 * n + m;
    }
    lo = total * blockIdx.x / gridDim.x;
    hi = total * (blockIdx.x + 1) / gridDim.x;
  }
  // first tile of a unit whose weight offset is at least y
  auto tile_at = [](int64_t y, int n, int m) {
    const int64_t j = y <= 3 * (int64_t)m ? (y + 2) / 3 : m + (y - 3 * (int64_t)m + 1) / 2;
    return (int)(j < n ? j : n);
  };
  // Segments in turn, through one call site: the chunk of the chunked split (which
  // also writes its rows' tails), or each unit's part of the balanced stretch.
  int u_next = 0;
  int64_t base = 0;
  for (;;) {
    int t, s_begin, s_cap;
    bool tail;
    if (!a.balance) {
      if (u_next++ > 0) break;
      const XcdTile tile = score_tile(a, units);
      if (tile.chunk >= a.n_chunks) break;
      t = tile.row * G + wave;
      s_begin = tile.chunk * a.chunk;
      s_cap = s_begin + a.chunk;
      tail = a.write_tail != 0;
    } else {
      int j0 = 0, j1 = 0, u = u_next;
      for (; u < units && base < hi; ++u) {
        int n, m;
        unit_tiles(u, n, m);
        const int64_t w = 2 * n + m;
        if (base + w > lo) {
          j0 = tile_at(max(lo - base, (int64_t)0), n, m);
          j1 = tile_at(min(hi - base, w), n, m);
        }
        base += w;
        if (j1 > j0) break;
      }
      if (!(j1 > j0)) break;
      u_next = u + 1;
      t = u * G + wave < a.T ? s_order[u * G + wave] : a.T;
      s_begin = j0 * TILE;
      s_cap = min(j1 * TILE, s_valid[s_order[u * G]]);
      tail = false;
    }
    run_segment(t, s_begin, s_cap, tail);
    __syncthreads();  // the LDS of a segment is reused by the next one
  }
  if (!a.balance) return;
  // the rows' -inf tails [valid, n_cols), split evenly over the grid
  if (a.write_tail) {
    int64_t tails = 0;
    for (int r = 0; r < a.T; ++r) tails += a.n_cols - s_valid[r];
    const int64_t t0 = tails * blockIdx.x / gridDim.x, t1 = tails * (blockIdx.x + 1) / gridDim.x;
    int64_t c = 0;
    for (int r = 0; r < a.T && c < t1; ++r) {
      const int len = a.n_cols - s_valid[r];
      const int64_t a0 = max(t0, c), a1 = min(t1, c + len);
      if (a1 > a0) {
        float* row = a.scores + (int64_t)r * a.score_stride + s_valid[r];
        for (int64_t i = a0 - c + tid; i < a1 - c; i += NT) row[i] = -INFINITY;
      }
      c += len;
    }
  }
}

// ------------------------------------------------------------------ FP32 scorer

template <int D, int HM, int QBF16>
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreArgs a) {
  zero_side_words(a, 256);
  const XcdTile tile = score_tile(a, a.T);
  if (tile.chunk >= a.n_chunks) return;
  const int t = tile.row;
  const int valid = a.valid_lens[t];
  const int s = tile.chunk * a.chunk + (int)threadIdx.x;
  const int s_lim = a.write_tail ? a.n_cols : valid;
  if (s >= s_lim) return;
  float* out_row = a.scores + (int64_t)t * a.score_stride;
  if (s >= valid) {
    out_row[s] = -INFINITY;
    return;
  }
  const int32_t* bt_row = a.bt + (int64_t)t * a.bt_stride;
  const uint32_t lb = div_epb((uint32_t)s, a.epb_magic);
  const int p = bt_row[lb];
  const int64_t e = (int64_t)p * a.epb + (s - (int)lb * a.epb);
  const float g = a.gscale[p];
  const uint8_t* kp = a.keys + e * (D / 2);
  const uint8_t* sp = a.kscale + e * (D / 16);
  const int64_t qbase = (int64_t)t * a.H * D;

  float acc[HM];
#pragma unroll
  for (int h = 0; h < HM; ++h) acc[h] = 0.0f;
  for (int gi = 0; gi < D / 16; ++gi) {
    const u32x2 wv = *reinterpret_cast<const u32x2*>(kp + gi * 8);
    const float sc = e4m3_to_f32(sp[gi]);
    float kv[16];
    decode8_f32(wv[0], sc, kv);
    decode8_f32(wv[1], sc, kv + 8);
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      if (h < a.H) {
        float part = 0.0f;
        const int64_t qo = qbase + (int64_t)h * D + gi * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) part = fmaf(load_q(a.q, QBF16, qo + i), kv[i], part);
        acc[h] += part;
      }
    }
  }
  float score = 0.0f;
#pragma unroll
  for (int h = 0; h < HM; ++h)
    if (h < a.H) score = fmaf(a.w[(int64_t)t * a.H + h], fmaxf(g * acc[h], 0.0f), score);
  out_row[s] = score;
}

// FP32 scores on the fp32 matrix cores (IDX_PREC_FP32 at D 64 or 128, up to 64 heads):
// every wave streams 16-key steps of one row.  v_mfma_f32_16x16x4_f32 takes 16 heads x
// 4 dims of q (A) and 4 dims x 16 keys of exact NVFP4 code values (B), fp32 products and
// sums.  Lane (c, g) = (lane % 16, lane / 16) holds, in both operands, the dims
// [g D/4, (g + 1) D/4): MFMA step s takes dim g D/4 + s from every lane group, so each
// lane decodes one contiguous D/8-byte slice of its key (key c of the step).  The
// epilogue is the vector kernel's, w * max(g * dot, 0) per head: lane (c, g) holds heads
// 16 mt + 4 g + i of key c, summed in the lane and then over the four lane groups.
template <int MT, int D>
__global__ __launch_bounds__(256) void score_f32mfma_kernel(ScoreArgs a) {
  constexpr int KS = D / 4;   // MFMA steps = dims per lane group
  constexpr int NB = D / 8;   // code bytes of a lane's slice
  constexpr int NG = KS / 16; // 16-dim scale groups in it
  static_assert(D == 64 || D == 128, "head dim");
  zero_side_words(a, 256);
  const XcdTile tile = score_tile(a, a.T);
  if (tile.chunk >= a.n_chunks) return;
  const int t = tile.row;
  const int valid = a.valid_lens[t];
  const int s_begin = tile.chunk * a.chunk;
  const int s_lim = a.write_tail ? a.n_cols : valid;
  if (s_begin >= s_lim) return;
  const int s_end = min(s_begin + a.chunk, s_lim);
  const int s_vend = min(s_end, valid);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  float* out_row = a.scores + (int64_t)t * a.score_stride;
  for (int s = max(s_vend, s_begin) + tid; s < s_end; s += 256) out_row[s] = -INFINITY;
  if (s_vend <= s_begin) return;

  // A operands q[16 mt + c][g KS + s] and the weights of accumulator rows 16 mt + 4 g + i
  float qa[MT][KS];
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = 16 * mt + c;
    const int64_t base = ((int64_t)t * a.H + h) * D + g * KS;
#pragma unroll
    for (int s = 0; s < KS; s += 8) {
      if (h >= a.H) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qa[mt][s + e] = 0.0f;
      } else if (a.q_bf16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + base + s);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qa[mt][s + 2 * e] = __uint_as_float(v[e] << 16);
          qa[mt][s + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
        }
      } else {
        const float* src = reinterpret_cast<const float*>(a.q) + base + s;
        const float4v v0 = *reinterpret_cast<const float4v*>(src);
        const float4v v1 = *reinterpret_cast<const float4v*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qa[mt][s + e] = v0[e];
          qa[mt][s + 4 + e] = v1[e];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hr = 16 * mt + 4 * g + i;
      wr[mt][i] = hr < a.H ? a.w[(int64_t)t * a.H + hr] : 0.0f;
    }
  }
  const int32_t* bt_row = a.bt + (int64_t)t * a.bt_stride;
  // Step i of this wave covers keys s_begin + 16 wave + 64 i + (0..15).  Its loads run
  // ahead of the matrix work: the table entry two steps ahead, the codes, the scales and
  // the global scale one step ahead (keys past the valid end re-read the last valid one;
  // their scores are not stored).
  const int w0 = __builtin_amdgcn_readfirstlane(s_begin + 16 * wave);
  const int n_steps = w0 < s_vend ? (s_vend - w0 + 63) / 64 : 0;
  struct KeyRaw {
    uint32_t words[NB / 4];
    uint32_t sc;  // the slice's NG scale bytes
    float gs;
  };
  auto key_of = [&](int i) { return min(w0 + 64 * i + c, s_vend - 1); };
  auto entry_of = [&](int i) { return bt_row[div_epb((uint32_t)key_of(i), a.epb_magic)]; };
  auto load_key = [&](int i, int p, KeyRaw& r) {
    const int s = key_of(i);
    const uint32_t lb = div_epb((uint32_t)s, a.epb_magic);
    const int64_t e = (int64_t)p * a.epb + (s - (int)lb * a.epb);
    const uint8_t* kp = a.keys + e * (D / 2) + g * NB;
    const uint8_t* sp = a.kscale + e * (D / 16) + g * NG;
    if constexpr (NB == 16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(kp);
#pragma unroll
      for (int k = 0; k < 4; ++k) r.words[k] = v[k];
      r.sc = *reinterpret_cast<const uint16_t*>(sp);
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(kp);
      r.words[0] = v[0];
      r.words[1] = v[1];
      r.sc = *sp;
    }
    r.gs = a.gscale[p];
  };
  auto compute_store = [&](int i, const KeyRaw& r) {
    float kb[KS];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float sc = e4m3_to_f32((r.sc >> (8 * j)) & 0xffu);
      decode8_f32(r.words[2 * j], sc, kb + 16 * j);
      decode8_f32(r.words[2 * j + 1], sc, kb + 16 * j + 8);
    }
    float4v acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[mt][k], kb[k], acc[mt], 0, 0, 0);
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) part = fmaf(wr[mt][q], fmaxf(r.gs * acc[mt][q], 0.0f), part);
    part = row_sum4(part);
    // every lane stores its column's total; columns past the valid end were computed on
    // the last valid key (clamped above), so they write that key's own score to its slot
    out_row[key_of(i)] = part;
  };
  if (n_steps == 0) return;
  // two steps per trip and a single exit; the loads are issued in pipeline order
  const int pa = entry_of(0);
  int pb = entry_of(1);  // table entry of step i + 1
  int pc = entry_of(2);  // ... of step i + 2
  __builtin_amdgcn_sched_barrier(0);
  KeyRaw r0;  // step i
  load_key(0, pa, r0);
  __builtin_amdgcn_sched_barrier(0);
  // (the scheduling barriers keep each step's loads ahead of the matrix work before them)
  for (int i = 0; i < n_steps; i += 2) {
    KeyRaw r1;
    load_key(i + 1, pb, r1);
    const int pd = entry_of(i + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute_store(i, r0);
    __builtin_amdgcn_sched_barrier(0);
    load_key(i + 2, pc, r0);
    pc = entry_of(i + 4);
    pb = pd;
    __builtin_amdgcn_sched_barrier(0);
    compute_store(i + 1, r1);  // past the last step: its scores are not stored
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------ debug dequant

template <int D>
__global__ __launch_bounds__(256) void debug_dequant_kernel(const uint8_t* keys, const uint8_t* kscale,
                                                           const float* gscale, const int32_t* bt_row,
                                                           int n, int epb, uint64_t magic, int mode,
                                                           float* out) {
  const int s = blockIdx.x;
  if (s >= n) return;
  const uint32_t lb = div_epb((uint32_t)s, magic);
  const int p = bt_row[lb];
  const int64_t e = (int64_t)p * epb + (s - (int)lb * epb);
  const float g = gscale[p];
  const int d0 = threadIdx.x * 8;  // eight elements per thread
  if (d0 >= D) return;
  const uint32_t word = *reinterpret_cast<const uint32_t*>(keys + e * (D / 2) + d0 / 2);
  const uint32_t sb = kscale[e * (D / 16) + d0 / 16];
  float v[8];
  if (mode == 2) {
    const half8v h = decode8_f16(word, splat_scale_f16(sb));
    const u32x4 u = __builtin_bit_cast(u32x4, h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xffffu));
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
    }
  } else {
    decode8_f32(word, e4m3_to_f32(sb), v);
    if (mode == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * g;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) out[(int64_t)s * D + d0 + i] = v[i];
}

// ------------------------------------------------------------------ launchers

template <int MT, int D, int G>
static void launch_group(const ScoreArgs& a, int blocks, hipStream_t st) {
  const size_t lds = (size_t)2 * 64 * (D + 8) * 2 + 2 * 64 * 4 + (size_t)G * a.pid_cap * 8;
  if (a.epb % 16 == 0)
    hipLaunchKernelGGL((score_mfma_group_kernel<MT, D, true, G>), dim3(blocks), dim3(64 * G), lds, st, a);
  else
    hipLaunchKernelGGL((score_mfma_group_kernel<MT, D, false, G>), dim3(blocks), dim3(64 * G), lds, st, a);
}

template <int MT, int D>
static hipError_t launch_mfma_t(const ScoreArgs& a, int blocks, int group, hipStream_t st) {
  if (group == 8) {
    launch_group<MT, D, 8>(a, blocks, st);
  } else if (group == 4) {
    launch_group<MT, D, 4>(a, blocks, st);
  } else {
    const size_t lds = (size_t)a.pid_cap * 8;
    if (a.epb % 16 == 0)
      hipLaunchKernelGGL((score_mfma_split_kernel<MT, D, true>), dim3(blocks), dim3(256), lds, st, a);
    else
      hipLaunchKernelGGL((score_mfma_split_kernel<MT, D, false>), dim3(blocks), dim3(256), lds, st, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_d(const ScoreArgs& a, int blocks, int group, hipStream_t st) {
  const int mt = (a.H + 15) / 16;
  switch (mt) {
    case 1: return launch_mfma_t<1, D>(a, blocks, group, st);
    case 2: return launch_mfma_t<2, D>(a, blocks, group, st);
    case 3: return launch_mfma_t<3, D>(a, blocks, group, st);
    default: return launch_mfma_t<4, D>(a, blocks, group, st);
  }
}

template <int D, int QB>
static hipError_t launch_f32_q(const ScoreArgs& a, int blocks, hipStream_t st) {
  if (a.H <= 8) {
    hipLaunchKernelGGL((score_f32_kernel<D, 8, QB>), dim3(blocks), dim3(256), 0, st, a);
  } else if (a.H <= 16) {
    hipLaunchKernelGGL((score_f32_kernel<D, 16, QB>), dim3(blocks), dim3(256), 0, st, a);
  } else if (a.H <= 32) {
    hipLaunchKernelGGL((score_f32_kernel<D, 32, QB>), dim3(blocks), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((score_f32_kernel<D, 64, QB>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32_d(const ScoreArgs& a, int blocks, hipStream_t st) {
  return a.q_bf16 ? launch_f32_q<D, 1>(a, blocks, st) : launch_f32_q<D, 0>(a, blocks, st);
}

template <int D>
static hipError_t launch_f32mfma_d(const ScoreArgs& a, int blocks, hipStream_t st) {
  switch ((a.H + 15) / 16) {
    case 1: hipLaunchKernelGGL((score_f32mfma_kernel<1, D>), dim3(blocks), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((score_f32mfma_kernel<2, D>), dim3(blocks), dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((score_f32mfma_kernel<3, D>), dim3(blocks), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((score_f32mfma_kernel<4, D>), dim3(blocks), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

// The FP32 path runs on the fp32 matrix cores for D 64/128 and up to 64 heads.
static bool f32_uses_mfma(const ScoreArgs& a) { return (a.D == 64 || a.D == 128) && a.H <= 64; }

// Keys per workgroup: enough workgroups to fill the chip a few times over
// (`target`), multiples of 64, between 256 and 4096, and few enough block-table
// entries per chunk (<= 500) for the LDS page lists.
static int chunk_keys(int units, int n_cols, int epb, int target) {
  int64_t n_chunks = (target + units - 1) / units;
  if (n_chunks < 1) n_chunks = 1;
  int64_t c = ((int64_t)n_cols + n_chunks - 1) / n_chunks;
  c = (c + 63) / 64 * 64;
  if (c < 256) c = 256;
  if (c > 4096) c = 4096;
  const int64_t cap = (int64_t)500 * epb / 64 * 64;
  if (c > cap) c = cap < 64 ? 64 : cap;
  return (int)c;
}

hipError_t launch_score_rows(ScoreArgs a, int precision, hipStream_t st) {
  // rows per workgroup of the group scorer (0: the one-row split scorer)
  const int group = precision != 1 ? 0 : a.T >= 16 ? SALB_GROUP_ROWS : a.T >= 4 ? 4 : 0;
  const int units = group ? (a.T + group - 1) / group : a.T;
  if (precision == 1) {
    a.chunk = chunk_keys(units, a.n_cols, a.epb, group ? SALB_GROUP_WGS : SALB_SPLIT_WGS);
    a.pid_cap = a.chunk / a.epb + 2;
  } else if (f32_uses_mfma(a)) {
    a.chunk = chunk_keys(units, a.n_cols, a.epb, SALB_SPLIT_WGS);
    a.pid_cap = 0;
  } else {
    a.chunk = 256;
    a.pid_cap = 0;
  }
  a.n_chunks = (a.n_cols + a.chunk - 1) / a.chunk;
  a.swizzle = a.n_chunks >= kXcds;
  const int64_t per_unit = a.swizzle ? (int64_t)((a.n_chunks + kXcds - 1) / kXcds) * kXcds : a.n_chunks;
  int64_t blocks = per_unit * units;
  a.balance = 0;
  if (group && a.T >= 16 && a.T <= 256) {
    // balanced split (from 16 rows on; fewer rows keep the chunked split, which has
    // the shorter start-up): the grid shares the rows' weighted 64-key tiles evenly.  Tiles
    // weigh 2 or 3, so a workgroup's stretch of one unit spans at most half its share
    // of the weight plus two tiles; the grid grows until that fits the LDS page slots.
    a.balance = 1;
    const int64_t tiles = (int64_t)units * ((a.n_cols + 63) / 64);
    const int64_t weight = tiles * (group == 8 ? 3 : 2);
    const int64_t max_pid = (int64_t)kBalancePidBytes / (group * 8);
    const int64_t max_tiles = std::max<int64_t>(3, (max_pid - 2) * a.epb / 64);
    int64_t nw = std::max<int64_t>(1, std::min<int64_t>(SALB_GROUP_WGS, tiles));
    auto seg_tiles = [&](int64_t n) { return (weight + n - 1) / n / 2 + 2; };
    if (seg_tiles(nw) > max_tiles) nw = (weight + 2 * (max_tiles - 2) - 1) / (2 * (max_tiles - 2));
    a.pid_cap = (int)(seg_tiles(nw) * 64 / a.epb + 2);
    blocks = nw;
  }
  // T >= 1 and n_cols >= 1 here (the entry points return before), so blocks >= 1 and
  // the launch also zeroes the side words it was given
  if (blocks <= 0) return hipErrorInvalidConfiguration;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (precision == 1) {
    switch (a.D) {
      case 64: return launch_mfma_d<64>(a, (int)blocks, group, st);
      case 128: return launch_mfma_d<128>(a, (int)blocks, group, st);
      default: return launch_mfma_d<256>(a, (int)blocks, group, st);
    }
  }
  if (f32_uses_mfma(a))
    return a.D == 64 ? launch_f32mfma_d<64>(a, (int)blocks, st) : launch_f32mfma_d<128>(a, (int)blocks, st);
  switch (a.D) {
    case 64: return launch_f32_d<64>(a, (int)blocks, st);
    case 128: return launch_f32_d<128>(a, (int)blocks, st);
    default: return launch_f32_d<256>(a, (int)blocks, st);
  }
}

hipError_t launch_debug_dequant(const uint8_t* keys, const uint8_t* kscale, const float* gscale,
                                const int32_t* bt_row, int n, int D, int epb, int mode, float* out,
                                hipStream_t st) {
  const uint64_t magic = host_epb_magic(epb);
  switch (D) {
    case 64:
      hipLaunchKernelGGL((debug_dequant_kernel<64>), dim3(n), dim3(64), 0, st, keys, kscale, gscale, bt_row, n,
                         epb, magic, mode, out);
      break;
    case 128:
      hipLaunchKernelGGL((debug_dequant_kernel<128>), dim3(n), dim3(64), 0, st, keys, kscale, gscale, bt_row, n,
                         epb, magic, mode, out);
      break;
    default:
      hipLaunchKernelGGL((debug_dequant_kernel<256>), dim3(n), dim3(64), 0, st, keys, kscale, gscale, bt_row, n,
                         epb, magic, mode, out);
      break;
  }
  return hipGetLastError();
}

}  // namespace salb
