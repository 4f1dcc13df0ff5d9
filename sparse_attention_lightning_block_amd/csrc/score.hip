// Lightning-indexer scorers for gfx950.
//
//   I[t, s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[t,s,:] )
// ([listing] "nvfp4-megamoe-kernel -- .../indexer_score_topk.cu": header comment, eq. 16,
// and the scoring loop of its main kernel), with the NVFP4 keys of a paged pool
// resolved through a per-query block table (same page, main kernel).
//
// Two scorers share the work decomposition -- a workgroup owns one query row and a
// contiguous chunk of that row's logical keys; chunks are spread over the XCDs so
// that all rows of one chunk run on the same XCD (shared pages hit one L2):
//
//  * score_mfma_kernel (IDX_PREC_MFMA): the head x key contraction on the fp16
//    matrix cores.  A 16x16x32 MFMA takes 16 heads (M) x 32 dims (K) of q from
//    registers and 32 dims x 16 keys (N) of decoded NVFP4 keys; each lane decodes
//    its own 16-byte slice of one key straight into the B operand (no LDS trip).
//    The K order inside an instruction is a fixed permutation of the head dims
//    applied to both operands, chosen so that every lane's slice is contiguous.
//    The epilogue applies ReLU, the head weights and the per-page global scale to
//    the fp32 accumulators, reduces the 64 heads (in-lane, then two lane swaps)
//    and writes one score per key.  q is prescaled per head by a power of two so
//    that its fp16 rounding is relative (11 bits); the inverse power is folded
//    into the head weight, which keeps the result identical up to that rounding.
//  * score_f32_kernel (IDX_PREC_FP32): one key per lane, fp32 FMAs with q read
//    through the scalar cache, for results within ~1e-5 relative.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"
#include "nvfp4.hpp"

namespace salb {

// ------------------------------------------------------------------ helpers

template <int D>
struct KeySlice {
  // One lane's share of one key for the MFMA operand: D/4 consecutive dims
  // (D/8 bytes of codes) and their D/64 scale bytes.
  static constexpr int kWords = D / 32;
  uint32_t w[kWords];
  uint32_t sc;
};

template <int D>
__device__ __forceinline__ void load_slice(KeySlice<D>& ks, const uint8_t* __restrict__ keys,
                                           const uint8_t* __restrict__ kscale, int64_t e, int quarter) {
  const uint8_t* kp = keys + e * (D / 2) + quarter * (D / 8);
  const uint8_t* sp = kscale + e * (D / 16) + quarter * (D / 64);
  if constexpr (D == 64) {
    u32x2 v = *reinterpret_cast<const u32x2*>(kp);
    ks.w[0] = v[0];
    ks.w[1] = v[1];
    ks.sc = *sp;
  } else if constexpr (D == 128) {
    u32x4 v = *reinterpret_cast<const u32x4*>(kp);
    ks.w[0] = v[0];
    ks.w[1] = v[1];
    ks.w[2] = v[2];
    ks.w[3] = v[3];
    ks.sc = *reinterpret_cast<const uint16_t*>(sp);
  } else {
    u32x4 v0 = *reinterpret_cast<const u32x4*>(kp);
    u32x4 v1 = *reinterpret_cast<const u32x4*>(kp + 16);
    ks.w[0] = v0[0];
    ks.w[1] = v0[1];
    ks.w[2] = v0[2];
    ks.w[3] = v0[3];
    ks.w[4] = v1[0];
    ks.w[5] = v1[1];
    ks.w[6] = v1[2];
    ks.w[7] = v1[3];
    ks.sc = *reinterpret_cast<const uint32_t*>(sp);
  }
}

__device__ __forceinline__ float load_q(const void* q, int bf16, int64_t i) {
  if (bf16) {
    uint32_t b = reinterpret_cast<const uint16_t*>(q)[i];
    return __uint_as_float(b << 16);
  }
  return reinterpret_cast<const float*>(q)[i];
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

template <int MT, int D>
__global__ __launch_bounds__(256) void score_mfma_kernel(ScoreArgs a) {
  constexpr int HP = MT * 16;     // padded head count
  constexpr int QLD = D + 8;      // padded LDS row (halves)
  constexpr int KW = D / 32;      // K-steps of 32 dims
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* qh = reinterpret_cast<_Float16*>(smem);                       // [HP][QLD]
  float* wsc = reinterpret_cast<float*>(smem + HP * QLD * 2);              // [HP]
  int* pid = reinterpret_cast<int*>(wsc + HP);                             // [pid_cap]
  float* pgs = reinterpret_cast<float*>(pid + a.pid_cap);                  // [pid_cap]

  const XcdTile tile = xcd_tile(blockIdx.x, a.T);
  if (tile.chunk >= a.n_chunks) return;
  const int t = tile.row;
  const int valid = a.valid_lens[t];
  const int s_begin = tile.chunk * a.chunk;
  const int s_lim = a.write_tail ? a.n_cols : valid;
  if (s_begin >= s_lim) return;
  const int s_end = min(s_begin + a.chunk, s_lim);
  const int s_vend = min(s_end, valid);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float* out_row = a.scores + (int64_t)t * a.score_stride;

  // -- pages of this chunk
  int lb0 = div_epb((uint32_t)s_begin, a.epb_magic);
  int npages = 0;
  if (s_vend > s_begin) npages = (int)div_epb((uint32_t)(s_vend - 1), a.epb_magic) - lb0 + 1;
  const int32_t* bt_row = a.bt + (int64_t)t * a.bt_stride;
  for (int i = tid; i < npages; i += 256) {
    int p = bt_row[lb0 + i];
    pid[i] = p;
    pgs[i] = a.gscale[p];
  }

  // -- q[t] -> LDS as per-head prescaled fp16, and the matching head weights
  const int64_t qbase = (int64_t)t * a.H * D;
  for (int h = wave; h < HP; h += 4) {
    constexpr int PER = D / 64;
    float v[PER];
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      v[i] = (h < a.H) ? load_q(a.q, a.q_bf16, qbase + (int64_t)h * D + lane * PER + i) : 0.0f;
      mx = fmaxf(mx, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const int j = prescale_exp(mx);
#pragma unroll
    for (int i = 0; i < PER; ++i) qh[h * QLD + lane * PER + i] = (_Float16)ldexpf(v[i], j);
    if (lane == 0) wsc[h] = (h < a.H) ? ldexpf(a.w[(int64_t)t * a.H + h], -j) : 0.0f;
  }
  __syncthreads();

  // -- A operands (q) and the accumulator-row weights, per wave
  const int quarter = lane >> 4;  // which D/4 slice of a key / q row this lane holds
  const int col = lane & 15;
  half8v A[MT][KW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int kk = 0; kk < KW; ++kk)
      A[mt][kk] = *reinterpret_cast<const half8v*>(qh + (mt * 16 + col) * QLD + quarter * (D / 4) + kk * 8);
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[mt][i] = wsc[mt * 16 + quarter * 4 + i];

  // -- stream the chunk, 16 keys per wave step
  const int n_groups = (s_end - s_begin + 15) >> 4;
  KeySlice<D> cur, nxt;
  float g_cur = 0.0f, g_nxt = 0.0f;
  bool in_cur = false, in_nxt = false;

  auto fetch = [&](int gi, KeySlice<D>& ks, float& g, bool& in) {
    const int s = s_begin + gi * 16 + col;
    in = s < s_vend;
    if (in) {
      const uint32_t lb = div_epb((uint32_t)s, a.epb_magic);
      const int li = (int)lb - lb0;
      const int p = pid[li];
      g = pgs[li];
      const int64_t e = (int64_t)p * a.epb + (s - (int)lb * a.epb);
      load_slice<D>(ks, a.keys, a.kscale, e, quarter);
    } else {
#pragma unroll
      for (int i = 0; i < KW; ++i) ks.w[i] = 0u;
      ks.sc = 0u;
      g = 0.0f;
    }
  };

  int gi = wave;
  if (gi < n_groups) fetch(gi, cur, g_cur, in_cur);
  for (; gi < n_groups; gi += 4) {
    const int s0 = s_begin + gi * 16;
    const bool has_next = gi + 4 < n_groups;
    if (has_next) fetch(gi + 4, nxt, g_nxt, in_nxt);

    if (s0 < s_vend) {
      float4v acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KW; ++kk) {
        const half2v s2 = splat_scale_f16((cur.sc >> (8 * (kk >> 1))) & 0xffu);
        const half8v B = decode8_f16(cur.w[kk], s2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][kk], B, acc[mt], 0, 0, 0);
      }
      // ReLU(g * dot) = |g| * ReLU(sign(g) * dot): the page scale leaves the ReLU.
      float part = 0.0f;
      float gabs = g_cur;
      if (__ballot(g_cur < 0.0f) == 0ull) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wr[mt][i], fmaxf(acc[mt][i], 0.0f), part);
      } else {
        const float sg = g_cur < 0.0f ? -1.0f : 1.0f;
        gabs = fabsf(g_cur);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wr[mt][i], fmaxf(acc[mt][i] * sg, 0.0f), part);
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const int s = s0 + col;
      if (lane < 16 && s < s_end) out_row[s] = in_cur ? gabs * part : -INFINITY;
    } else {
      const int s = s0 + col;
      if (lane < 16 && s < s_end) out_row[s] = -INFINITY;
    }
    if (has_next) {
      cur = nxt;
      g_cur = g_nxt;
      in_cur = in_nxt;
    }
  }
}

// ------------------------------------------------------------------ FP32 scorer

template <int D, int HM, int QBF16>
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreArgs a) {
  const XcdTile tile = xcd_tile(blockIdx.x, a.T);
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

template <int MT, int D>
static hipError_t launch_mfma_t(const ScoreArgs& a, int blocks, hipStream_t st) {
  constexpr int HP = MT * 16;
  const size_t lds = (size_t)HP * (D + 8) * 2 + HP * 4 + (size_t)a.pid_cap * 8;
  hipLaunchKernelGGL((score_mfma_kernel<MT, D>), dim3(blocks), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_d(const ScoreArgs& a, int blocks, hipStream_t st) {
  const int mt = (a.H + 15) / 16;
  switch (mt) {
    case 1: return launch_mfma_t<1, D>(a, blocks, st);
    case 2: return launch_mfma_t<2, D>(a, blocks, st);
    case 3: return launch_mfma_t<3, D>(a, blocks, st);
    default: return launch_mfma_t<4, D>(a, blocks, st);
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

// Keys per workgroup for the MFMA scorer: about a thousand workgroups of work,
// at least 512 keys (so the per-workgroup q staging stays small) and at most 4096.
static int mfma_chunk(int T, int n_cols) {
  const int64_t work = (int64_t)T * n_cols;
  int64_t c = (work / 1024 + 63) / 64 * 64;
  if (c < 512) c = 512;
  if (c > 4096) c = 4096;
  return (int)c;
}

hipError_t launch_score_rows(ScoreArgs a, int precision, hipStream_t st) {
  if (precision == 1) {
    a.chunk = mfma_chunk(a.T, a.n_cols);
    a.pid_cap = a.chunk / a.epb + 2;
  } else {
    a.chunk = 256;
    a.pid_cap = 0;
  }
  a.n_chunks = (a.n_cols + a.chunk - 1) / a.chunk;
  const int64_t padded = (int64_t)((a.n_chunks + kXcds - 1) / kXcds) * kXcds;
  const int64_t blocks = padded * a.T;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (precision == 1) {
    switch (a.D) {
      case 64: return launch_mfma_d<64>(a, (int)blocks, st);
      case 128: return launch_mfma_d<128>(a, (int)blocks, st);
      default: return launch_mfma_d<256>(a, (int)blocks, st);
    }
  }
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
