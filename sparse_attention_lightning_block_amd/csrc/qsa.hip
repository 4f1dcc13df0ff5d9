// QSA block-pooled indexer variant for gfx950 ([qsa.rs] "metrale_model_layers/layers/ops/qsa.rs":
// doc comments of qsa_block_pool, qsa_qprep / qsa_qprep_rows, qsa_score and qsa_score_rows).
//
//  * block pool: mean of `ratio` raw bf16 keys -> RMSNorm scaled by (1 + w) -> RoPE at
//    the block's first token position; one workgroup per pooled block, 16-byte loads.
//  * query prep: per (row, head) RMSNorm scaled by (1 + w) -> RoPE at first_pos + row.
//  * row scores: sum_h ReLU(q_h . k_b) / sqrt(hd), -inf past the row's complete blocks;
//    on the fp16 matrix cores (hd 64 or 128 with 16, 32 or 64 heads), else in fp32.
//
// RoPE pairs dimension i with i + rot/2 (i < rot/2) and rotates by
// pos * theta^(-2i/rot).  The page gives rot and theta but no pairing; the half
// split is this library's convention.  At the positions of long prefills
// (~5e5) an fp32 angle would be off by ~0.03 rad, so the angle, its sine and
// cosine and the rotation are evaluated in fp64 (once per position and pair).
// theta^(-2i/rot) is formed as exp2(-2i/rot * log2(theta)): within a few units in the
// last place of the fp64 power (~1e-9 rad of angle at 5e5), and far fewer registers.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Cosine and sine of a RoPE angle (fp64).  The angle is first reduced by the nearest
// multiple of 2*pi, with 2*pi split into three doubles and each product taken by an fma
// (exact to ~3e-16 rad for angles below 2^32), so that the library sine and cosine see
// |x| <= ~3.4: at long-prefill positions the raw angle reaches ~5e5 rad, where they
// would take their slow large-argument reduction.
__device__ __forceinline__ void rope_cos_sin(double angle, double& c, double& s) {
  constexpr double kInv2Pi = 0.15915494309189535;
  constexpr double k2PiHi = 0x1.921fb54442d18p+2;
  constexpr double k2PiMid = 0x1.1a62633145c07p-52;
  constexpr double k2PiLo = -0x1.f1976b7ed8fbcp-108;
  const double k = rint(angle * kInv2Pi);
  double r = fma(-k, k2PiHi, angle);
  r = fma(-k, k2PiMid, r);
  r = fma(-k, k2PiLo, r);
  sincos(r, &s, &c);
}

// ------------------------------------------------------------------ block pool

// Eight pooled blocks per 256-thread workgroup, 32 threads per block.  Thread j of a
// block owns the 8-dim column group j % CG of the raw rows r = j / CG (mod 32 / CG):
// every 16-byte load of the block is in flight at once.  The column sums meet
// through lane swaps, the RMSNorm sum of squares through a reduction over the
// column groups, and the rotation pairs through LDS.  The rotation angle and its
// sine and cosine are evaluated in fp64 (at long-prefill positions an fp32 angle is
// off by ~0.03 rad), once per (block, pair).
constexpr int kPoolTPB = 32;                  // threads per pooled block
constexpr int kPoolNBW = 256 / kPoolTPB;      // blocks per 256-thread group

// LDS of one 256-thread pooling group: the normalised block rows and the rotation
// pairs' cosines and sines.
template <int HD>
struct PoolLds {
  float xs[kPoolNBW][HD];
  double cs[kPoolNBW][HD / 2][2];
};

// The pooling of one 256-thread group (group index grp: blocks first_block + 8 grp ..
// + 7 below n_new).  Every thread of the workgroup calls it (it holds one barrier).
template <int HD, typename OutT>
__device__ __forceinline__ void pool_group(const uint16_t* __restrict__ raw, const float* __restrict__ kw,
                                           OutT* __restrict__ out, uint32_t first_block, uint32_t n_new,
                                           uint32_t ratio, int rot, float theta, float eps, uint32_t grp, int tid,
                                           PoolLds<HD>& lds) {
  constexpr int TPB = kPoolTPB;     // threads per block
  constexpr int NBW = kPoolNBW;     // blocks per group
  constexpr int CG = HD / 8;        // 16-byte column groups per raw row
  constexpr int RC = TPB / CG;      // raw-row classes (threads per column group)
  static_assert(RC >= 1 && TPB % CG == 0, "head_dim");
  constexpr int B = RC >= 4 ? 4 : 8;  // raw rows per thread in flight
  auto& xs = lds.xs;
  auto& cs = lds.cs;
  const int bi = tid / TPB, j = tid % TPB;
  const int cg = j % CG, rc = j / CG;
  const uint32_t nb_local = grp * NBW + bi;
  const bool live = nb_local < n_new;
  // blocks past n_new re-read the last new block and store nothing
  const uint32_t b = first_block + (live ? nb_local : n_new - 1);
  const uint16_t* base = raw + (int64_t)b * ratio * HD + cg * 8;
  // Raw rows r0 + u RC + rc (u < B) of this thread's column group: all B loads are issued
  // before any is used; rows past the block re-read its last row and add nothing.
  auto load_batch = [&](uint32_t r0, u32x4 (&v)[B]) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t r = min(r0 + (uint32_t)(u * RC + rc), ratio - 1);
      v[u] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * HD);
    }
  };
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add_batch = [&](uint32_t r0, const u32x4 (&v)[B]) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool ok = r0 + (uint32_t)(u * RC + rc) < ratio;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = acc[2 * i] + __uint_as_float(v[u][i] << 16);
        const float hi = acc[2 * i + 1] + __uint_as_float(v[u][i] & 0xffff0000u);
        acc[2 * i] = ok ? lo : acc[2 * i];
        acc[2 * i + 1] = ok ? hi : acc[2 * i + 1];
      }
    }
  };
  u32x4 v[B];
  load_batch(0, v);
  float wk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wk[i] = kw[cg * 8 + i];
  __builtin_amdgcn_sched_barrier(0);
  const int half = rot >> 1;
  if (live) {  // the rotation angles while the loads are in flight (dead blocks skip them)
    for (int i = j; i < half; i += TPB) {
      const double inv_freq = exp2(-2.0 * (double)i / (double)rot * log2((double)theta));
      double sn, c;
      rope_cos_sin((double)b * (double)ratio * inv_freq, c, sn);
      cs[bi][i][0] = c;
      cs[bi][i][1] = sn;
    }
  }
  add_batch(0, v);
  const uint32_t n_more = (ratio - 1) / (uint32_t)(B * RC);  // further batches, uniform
  for (uint32_t p = 1; p <= n_more; ++p) {
    load_batch(p * B * RC, v);
    add_batch(p * B * RC, v);
  }
  // sum the raw-row classes (lanes j ^ CG, j ^ 2 CG, ... of the same block)
#pragma unroll
  for (int off = CG; off < TPB; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off);
  float m[8], ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m[i] = acc[i] / (float)ratio;
    ss += m[i] * m[i];
  }
  // sum of squares over the column groups (lanes j ^ 1 .. j ^ CG/2)
#pragma unroll
  for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss / (float)HD + eps);
  if (rc == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[bi][cg * 8 + i] = m[i] * inv * (1.0f + wk[i]);
  }
  __syncthreads();
  if (live && rc == 0) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = cg * 8 + i;
      if (d < half) {
        const double a = xs[bi][d], bb = xs[bi][d + half];
        o[i] = (float)(a * cs[bi][d][0] - bb * cs[bi][d][1]);
      } else if (d < rot) {
        const double a = xs[bi][d - half], bb = xs[bi][d];
        o[i] = (float)(a * cs[bi][d - half][1] + bb * cs[bi][d - half][0]);
      } else {
        o[i] = xs[bi][d];
      }
    }
    OutT* dst = out + (int64_t)b * HD + cg * 8;
    if constexpr (sizeof(OutT) == 4) {
      *reinterpret_cast<float4v*>(dst) = float4v{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<float4v*>(dst + 4) = float4v{o[4], o[5], o[6], o[7]};
    } else {  // fp16 storage: each fp32 result rounded to nearest even
      half8v h;
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (_Float16)o[i];
      *reinterpret_cast<half8v*>(dst) = h;
    }
  }
}

template <int HD, typename OutT>
__global__ __launch_bounds__(256) void block_pool_kernel(const uint16_t* __restrict__ raw,
                                                         const float* __restrict__ kw, OutT* __restrict__ out,
                                                         uint32_t first_block, uint32_t n_new, uint32_t ratio,
                                                         int rot, float theta, float eps) {
  __shared__ PoolLds<HD> lds;
  pool_group<HD, OutT>(raw, kw, out, first_block, n_new, ratio, rot, theta, eps, blockIdx.x, threadIdx.x, lds);
}

// ------------------------------------------------------------------ query prep

// A row is cut into slices of SL 16-byte chunks (SL a multiple of 64 chunks, so a slice
// holds whole heads), one workgroup per (row, slice) and one chunk per thread: thread t
// owns the 8 dims of chunk s SL + t, and a head's HD / 8 chunks sit in consecutive lanes
// of one wave, so the head's RMSNorm sum of squares is a lane-swap tree with no LDS or
// barrier.  The chunk and norm-weight loads are issued before the rotation angles are
// evaluated (fp64, once per pair and workgroup), so the angle work overlaps their
// latency; the normalised values meet their rotation partners through LDS after the
// one barrier, and each chunk leaves as 16-byte stores.  The arithmetic of a chunk does
// not depend on the slicing or the workgroup size, so every launch shape gives the same
// bits.  A decode row spreads over several CUs; a prefill keeps many slices in flight
// per CU.

// The prep of chunks [s SL, s SL + SL) of row r by threads [0, SL) of the workgroup
// (the others only take part in the barrier).  smem: qprep_lds_bytes(SL, hd).
template <int HD, typename OutT, int SL>
__device__ __forceinline__ void qprep_slice(const uint16_t* __restrict__ qk, const float* __restrict__ qw,
                                            OutT* __restrict__ out, uint32_t r, uint32_t s, uint32_t first_pos,
                                            uint32_t qkw, uint32_t n_heads, int rot, float theta, float eps,
                                            int tid, unsigned char* smem) {
  constexpr int CG = HD / 8;  // chunks per head
  static_assert(SL % 64 == 0 && 64 % CG == 0, "whole heads per wave");
  const int n_chunks = (int)n_heads * CG;
  float* xs = reinterpret_cast<float*>(smem);           // [SL * 8] normalised values of the slice
  double* cs = reinterpret_cast<double*>(xs + SL * 8);  // [HD / 2][2] cosine, sine
  const int c = (int)s * SL + tid;                      // this thread's chunk
  const bool mine = tid < SL && c < n_chunks;
  const int d0 = (tid % CG) * 8;                        // its dims d0 .. d0 + 7 of its head
  const int half = rot >> 1;
  // lanes past the row re-read its last chunk and store nothing
  const u32x4 v = *reinterpret_cast<const u32x4*>(qk + (int64_t)r * qkw + 8 * min(c, n_chunks - 1));
  float wq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wq[i] = qw[d0 + i];
  __builtin_amdgcn_sched_barrier(0);
  if (tid < SL) {  // the row's rotation angles, while the loads are in flight
    const double pos = (double)first_pos + (double)r;
    for (int i = tid; i < half; i += SL) {
      const double inv_freq = exp2(-2.0 * (double)i / (double)rot * log2((double)theta));
      double sn, cn;
      rope_cos_sin(pos * inv_freq, cn, sn);
      cs[2 * i] = cn;
      cs[2 * i + 1] = sn;
    }
  }
  float x[8], ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
#pragma unroll
  for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off);
  const float hv = 1.0f / sqrtf(ss / (float)HD + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x[i] * hv * (1.0f + wq[i]);
  if (mine) {
    float* xd = xs + 8 * tid;
#pragma unroll
    for (int i = 0; i < 8; ++i) xd[i] = x[i];
  }
  __syncthreads();
  if (!mine) return;
  const float* xh = xs + (tid / CG) * HD;  // this thread's head in the slice
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = d0 + i;
    if (d < half) {
      const double a = x[i], bb = xh[d + half];
      o[i] = (float)(a * cs[2 * d] - bb * cs[2 * d + 1]);
    } else if (d < rot) {
      const double a = xh[d - half], bb = x[i];
      o[i] = (float)(a * cs[2 * (d - half) + 1] + bb * cs[2 * (d - half)]);
    } else {
      o[i] = x[i];
    }
  }
  OutT* dc = out + (int64_t)r * n_chunks * 8 + 8 * c;
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<float4v*>(dc) = float4v{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<float4v*>(dc + 4) = float4v{o[4], o[5], o[6], o[7]};
  } else {  // fp16 storage: each fp32 result rounded to nearest even
    half8v h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)o[i];
    *reinterpret_cast<half8v*>(dc) = h;
  }
}

// One (row, slice) per workgroup of SL threads: workgroup g takes row g / n_slices.
template <int HD, typename OutT, int SL>
__global__ __launch_bounds__(SL) void qprep_rows_kernel(const uint16_t* __restrict__ qk,
                                                        const float* __restrict__ qw, OutT* __restrict__ out,
                                                        uint32_t first_pos, uint32_t qkw, uint32_t n_heads,
                                                        uint32_t n_slices, int rot, float theta, float eps) {
  extern __shared__ __align__(16) unsigned char smem[];
  qprep_slice<HD, OutT, SL>(qk, qw, out, blockIdx.x / n_slices, blockIdx.x % n_slices, first_pos, qkw, n_heads, rot,
                            theta, eps, threadIdx.x, smem);
}

// A decode step's inputs in one launch: workgroups [0, rows n_slices) prepare the query
// rows, kQprepDecodeSlice chunks each; the others pool the new blocks, one 256-thread
// group each (the same arithmetic as qprep_rows_kernel and block_pool_kernel, so the
// outputs are bit-identical to theirs).
constexpr int kQprepDecodeSlice = 128;

template <int HD>
__global__ __launch_bounds__(256) void decode_prep_kernel(
    const uint16_t* __restrict__ raw, const float* __restrict__ kw, float* __restrict__ block_keys,
    uint32_t first_block, uint32_t n_new, uint32_t ratio, const uint16_t* __restrict__ qk,
    const float* __restrict__ qw, float* __restrict__ q_out, uint32_t rows, uint32_t n_slices, uint32_t first_pos,
    uint32_t qkw, uint32_t n_heads, int rot, float theta, float eps) {
  extern __shared__ __align__(16) unsigned char smem[];
  const uint32_t n_q = rows * n_slices;
  if (blockIdx.x < n_q) {  // uniform over the workgroup
    qprep_slice<HD, float, kQprepDecodeSlice>(qk, qw, q_out, blockIdx.x / n_slices, blockIdx.x % n_slices,
                                              first_pos, qkw, n_heads, rot, theta, eps, threadIdx.x, smem);
    return;
  }
  pool_group<HD, float>(raw, kw, block_keys, first_block, n_new, ratio, rot, theta, eps, blockIdx.x - n_q,
                        threadIdx.x, *reinterpret_cast<PoolLds<HD>*>(smem));
}

// ------------------------------------------------------------------ row scores (fp32)

// One block key per lane; q[r] read through the scalar cache.
template <int HD>
__global__ __launch_bounds__(256) void qsa_score_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ keys,
                                                            float* __restrict__ scores, uint32_t nb,
                                                            uint32_t first_pos, uint32_t stride, uint32_t ratio,
                                                            uint32_t n_heads) {
  const uint32_t r = blockIdx.y;
  const uint32_t bidx = blockIdx.x * 256 + threadIdx.x;
  if (bidx >= nb) return;
  uint64_t nvalid = ((uint64_t)first_pos + r + 1) / ratio;
  float* out = scores + (int64_t)r * stride;
  if (bidx >= nvalid) {
    out[bidx] = -INFINITY;
    return;
  }
  const float* k = keys + (int64_t)bidx * HD;
  float kv[HD];
#pragma unroll
  for (int d = 0; d < HD; d += 4) {
    const float4v v = *reinterpret_cast<const float4v*>(k + d);
    kv[d] = v[0];
    kv[d + 1] = v[1];
    kv[d + 2] = v[2];
    kv[d + 3] = v[3];
  }
  const float* qr = q + (int64_t)r * n_heads * HD;
  float sum = 0.0f;
  for (uint32_t h = 0; h < n_heads; ++h) {
    float dot = 0.0f;
#pragma unroll
    for (int d = 0; d < HD; ++d) dot = fmaf(qr[h * HD + d], kv[d], dot);
    sum += fmaxf(dot, 0.0f);
  }
  out[bidx] = sum * (1.0f / sqrtf((float)HD));
}

// ------------------------------------------------------------------ row scores (MFMA)

// Q[rows*heads, hd] x K[blocks, hd]^T on the fp16 matrix cores (16x16x32), then
// ReLU, the head sum and 1/sqrt(hd).  A wave holds 64 consecutive (row, head) pairs
// of q as A operands (RPW = 64 / NH rows); a workgroup of 8 waves (RPG rows) streams
// its key chunk in 64-key tiles converted to fp16 in LDS.  Every key tile is read
// by the workgroup once for all its rows, so the key traffic per score is 1/RPG of
// a key; the loads of tile j+2 are in flight (in registers) while tile j is
// multiplied and tile j+1 waits in registers for its LDS buffer.  The chunks are
// dealt so that all workgroups of one chunk run on one XCD: the chunk's keys (2 MB
// at 32768 blocks) stay in that XCD's L2.  q and the keys come out of RMSNorm, so
// their fp16 roundings are relative (2^-11) and the products stay far inside the
// fp16 range; the accumulation is fp32.
//
// With TMAX the scorer also writes, for every row and 16-block sub-tile (a 16-lane row of
// the wave), the largest order key of the sub-tile's stored scores (blocks past nb count
// as key 0, the order key of NaN, which no score undercuts): the per-sub-tile bound a
// select uses to skip most of a row.
constexpr int kQsaThreads = 512;

// Maximum over the lanes of each 16-lane row, left in the row's last lane (row shifts
// with 0 shifted in: 0 is below every order key that matters).
__device__ __forceinline__ uint32_t row_max_last(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
  return x;
}

// row_max_last of N values, the N chains interleaved step by step (each DPP read then
// follows its source's write by N - 1 independent instructions instead of wait states).
template <int N>
__device__ __forceinline__ void row_max_last_n(uint32_t (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = max(x[i], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x[i], 0x111, 0xf, 0xf, false));
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = max(x[i], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x[i], 0x112, 0xf, 0xf, false));
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = max(x[i], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x[i], 0x114, 0xf, 0xf, false));
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = max(x[i], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x[i], 0x118, 0xf, 0xf, false));
}

template <int HD, int NH, typename InT, bool TMAX>
__global__ __launch_bounds__(kQsaThreads) void qsa_score_mfma_kernel(const InT* __restrict__ q,
                                                                     const InT* __restrict__ keys,
                                                                     float* __restrict__ scores, uint32_t rows,
                                                                     uint32_t nb, uint32_t first_pos,
                                                                     uint32_t stride, uint32_t ratio,
                                                                     uint32_t chunk, uint32_t n_groups,
                                                                     float out_scale, uint32_t* __restrict__ tmax,
                                                                     uint32_t tstride) {
  constexpr int NT = kQsaThreads;
  constexpr int NW = NT / 64;     // waves
  constexpr int KW = HD / 32;     // K steps of 32 dims
  constexpr int RPW = 64 / NH;    // rows per wave
  constexpr int RPG = NW * RPW;   // rows per workgroup
  constexpr int MTR = NH / 16;    // M tiles per row
  constexpr int TILE = 64;
  constexpr int BLD = HD + 8;     // halves per LDS key row (padding against bank conflicts)
  constexpr int LPK = NT / TILE;  // loader threads per key
  constexpr int FPL = HD / LPK;   // floats each loader thread converts per tile
  static_assert(FPL % 8 == 0, "loader slice");
  __shared__ __align__(16) _Float16 kb[2][TILE * BLD];

  const XcdTile xt = xcd_tile((int)blockIdx.x, (int)n_groups);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int quarter = lane >> 4, col = lane & 15;
  const int64_t c0 = (int64_t)xt.chunk * chunk;
  const int64_t c1 = c0 + chunk < (int64_t)nb ? c0 + chunk : (int64_t)nb;
  if (c0 >= c1) return;
  const int r0 = xt.row * RPG;
  // valid blocks grow with the row: the group's last row bounds the keys to score
  const int r_last = min(r0 + RPG, (int)rows) - 1;
  auto valid_of = [&](int r) -> int64_t {
    const int64_t v = ((int64_t)first_pos + r + 1) / ratio;
    return v < (int64_t)nb ? v : (int64_t)nb;
  };
  const int64_t vmax = valid_of(r_last);
  const int64_t kend = c1 < vmax ? c1 : vmax;  // keys [c0, kend) are multiplied
  // keys of the chunk past every row's valid count: -inf (and, with TMAX, the maxima of
  // the sub-tiles past the last 64-key tile multiplied below: the order key of -inf)
  {
    const int64_t from = kend > c0 ? kend : c0;
    const int64_t tfrom = kend > c0 ? c0 + (kend - c0 + 63) / 64 * 64 : c0;
    for (int rr = 0; rr < RPG; ++rr) {
      const int r = r0 + rr;
      if (r >= (int)rows) break;
      for (int64_t s = from + tid; s < c1; s += NT) scores[(int64_t)r * stride + s] = -INFINITY;
      if constexpr (TMAX)
        for (int64_t s = tfrom + 16 * tid; s < c1; s += 16 * NT) tmax[(int64_t)r * tstride + (s >> 4)] = ord_key(-INFINITY);
    }
  }
  if (kend <= c0) return;

  // A operands: (row, head) pair m = wave * 64 + 16 * mt + col of the group
  half8v A[4][KW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int mm = 16 * mt + col;
    const int r = r0 + wave * RPW + mm / NH;
    const int h = mm % NH;
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      half8v a;
      if (r < (int)rows) {
        const InT* src = q + ((int64_t)r * NH + h) * HD + 32 * kk + 8 * quarter;
        if constexpr (sizeof(InT) == 2) {
          a = *reinterpret_cast<const half8v*>(src);
        } else {
          const float4v x0 = *reinterpret_cast<const float4v*>(src);
          const float4v x1 = *reinterpret_cast<const float4v*>(src + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = (_Float16)x0[e];
            a[4 + e] = (_Float16)x1[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (_Float16)0.0f;
      }
      A[mt][kk] = a;
    }
  }
  // per row of the wave: its output row (a row past the last one writes nothing) and
  // the end of its valid keys relative to the chunk start, key offsets are 32-bit
  float* orow[RPW];
  uint32_t* trow[RPW];  // with TMAX: the row's sub-tile maxima from the chunk start on
  int vrel[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = r0 + wave * RPW + rr;
    orow[rr] = r < (int)rows ? scores + (int64_t)r * stride + c0 : nullptr;
    trow[rr] = TMAX && r < (int)rows ? tmax + (int64_t)r * tstride + (c0 >> 4) : nullptr;  // c0: a multiple of 64
    vrel[rr] = r < (int)rows ? (int)(valid_of(r) - c0) : 0;
  }
  const int crel = (int)(c1 - c0);

  // tile loader: thread t converts FPL floats of key t / LPK
  // each group of eight lanes converts the same part of eight different keys, whose
  // LDS rows start on distinct bank groups: conflict-free tile writes
  static_assert(LPK == 8 && NT % 64 == 0, "loader map");
  const int lk = (tid & 7) | ((tid >> 6) << 3), lpart = (tid >> 3) & 7;
  // keys past kend are clamped onto the last one (their scores are masked at the store).
  // A loader thread's slice is FPL elements: FPL / 4 float4 loads of fp32 keys
  // (converted on the way into LDS), or FPL / 8 16-byte loads of fp16 keys (copied).
  constexpr int SV = sizeof(InT) == 4 ? FPL / 4 : FPL / 8;  // 16-byte vectors per slice
  typedef u32x4 Stage[SV];
  const InT* kbase = keys + lpart * FPL;
  auto load_tile = [&](int64_t k0, Stage& st) {
    const int64_t kk = min(k0 + lk, kend - 1);
    const InT* src = kbase + kk * HD;
#pragma unroll
    for (int j = 0; j < SV; ++j) st[j] = *reinterpret_cast<const u32x4*>(src + (16 / sizeof(InT)) * j);
  };
  auto store_tile = [&](int buf, const Stage& st) {
    _Float16* dst = &kb[buf][lk * BLD + lpart * FPL];
#pragma unroll
    for (int j = 0; j < FPL / 8; ++j) {
      if constexpr (sizeof(InT) == 2) {
        *reinterpret_cast<u32x4*>(dst + 8 * j) = st[j];
      } else {
        half8v h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = (_Float16)__uint_as_float(st[2 * j][e]);
          h[4 + e] = (_Float16)__uint_as_float(st[2 * j + 1][e]);
        }
        *reinterpret_cast<half8v*>(dst + 8 * j) = h;
      }
    }
  };
  // multiply one LDS tile, reduce the heads, write the scores
  auto do_tile = [&](int buf, int64_t k0) {
    float4v acc[4][4];
    // every B operand of the tile is read from LDS up front; the compiler places the
    // waits, so the later reads complete under the first MFMAs
    half8v B[KW][4];
#pragma unroll
    for (int kk = 0; kk < KW; ++kk)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        B[kk][nt] = *reinterpret_cast<const half8v*>(&kb[buf][(16 * nt + col) * BLD + 32 * kk + 8 * quarter]);
#pragma unroll
    for (int kk = 0; kk < KW; ++kk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              A[mt][kk], B[kk][nt], kk == 0 ? float4v{0.0f, 0.0f, 0.0f, 0.0f} : acc[mt][nt], 0, 0, 0);
    // ReLU and head sum: lane (quarter, col) holds heads 4*quarter + i of each M tile
    // for key 16 * nt + col.  The in-lane sums of the four N tiles are then reduced over
    // the quarters so that quarter q keeps N tile q: lane (quarter, col) ends with key
    // 16 * quarter + col of the tile, for each row.
    const int key = (int)(k0 - c0) + 16 * quarter + col;
    uint32_t tk[RPW];  // with TMAX: each row's order key of its stored score
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      float x[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        x[nt] = 0.0f;
#pragma unroll
        for (int j = 0; j < MTR; ++j) {
          const float4v a = acc[rr * MTR + j][nt];
          x[nt] += relu_bits(a[0]) + relu_bits(a[1]) + relu_bits(a[2]) + relu_bits(a[3]);
        }
      }
      const float v = row_transpose_sum4(x[0], x[1], x[2], x[3]);
      const float sv = key < vrel[rr] ? v * out_scale : -INFINITY;
      if (orow[rr] != nullptr && key < crel) orow[rr][key] = sv;
      if constexpr (TMAX) {
        // the order key of the stored score: a score here is +0 or more, or NaN (only from
        // non-finite inputs: key 0), or the -inf of a masked block (key ~bits(-inf))
        const uint32_t sb = __float_as_uint(sv);
        const uint32_t k = key >= vrel[rr] ? ~0xff800000u : sb > 0x7f800000u ? 0u : (sb | 0x80000000u);
        tk[rr] = trow[rr] != nullptr && key < crel ? k : 0u;
      }
    }
    if constexpr (TMAX) {
      // the maximum of sub-tile (k0 + 16 quarter) / 16 of each row, in the last lane
      // (col 15) of the quarter, which stores all of the wave's rows in one branch
      row_max_last_n<RPW>(tk);
      const int st0 = (int)(k0 - c0) + 16 * quarter;  // the sub-tile's first block, relative to c0
      if (col == 15 && st0 < crel) {
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
          if (trow[rr] != nullptr) trow[rr][st0 >> 4] = tk[rr];
      }
    }
  };

  // two register stages: tile j + 2 loads while tile j multiplies and tile j + 1
  // waits for its LDS buffer.  Two tiles per trip and a single exit: the loads are
  // unconditional (past the last tile they re-read the clamped last key), so every path
  // into the loop header has the same loads outstanding and the waits there only wait
  // for the tile they need.
  Stage sa, sb;
  load_tile(c0, sa);
  load_tile(c0 + TILE, sb);
  store_tile(0, sa);
  __syncthreads();
  const int n_tiles = (int)((kend - c0 + TILE - 1) / TILE);
  for (int j = 0; j < n_tiles; j += 2) {
    const int64_t k0 = c0 + (int64_t)j * TILE;
    // tile j is in buffer 0, tile j + 1 in sb
    load_tile(k0 + 2 * TILE, sa);
    do_tile(0, k0);
    store_tile(1, sb);
    __syncthreads();
    // tile j + 1 is in buffer 1, tile j + 2 in sa
    load_tile(k0 + 3 * TILE, sb);
    if (j + 1 < n_tiles) do_tile(1, k0 + TILE);
    store_tile(0, sa);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ decode scores

// Zeroes n16 16-byte words at p over the whole grid (a fused score + top-k call clears
// the select's counters in its score launch instead of a launch of its own).
__device__ __forceinline__ void zero_words(uint4* p, int64_t n16) {
  if (n16 == 0) return;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += step)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// One decode query against n_blocks block keys ([qsa.rs] qsa_score), fp32.  A 256-thread
// workgroup takes 64 consecutive blocks, one per lane, whose key stays in registers;
// the four waves split the heads (wave w takes heads w, w + 4, ...), reading the query
// from LDS (every lane the same address: broadcast reads), and the four partial head
// sums meet in LDS.  Four independent accumulators per dot product keep the FMA chains
// short.  One query is far below the MFMA ridge (2 * heads flops per key byte), so the
// VALU does the arithmetic.
template <int HD>
__global__ __launch_bounds__(256) void qsa_decode_score_kernel(const float* __restrict__ q,
                                                               const float* __restrict__ keys,
                                                               float* __restrict__ scores, uint32_t nb,
                                                               uint32_t n_heads, float out_scale,
                                                               uint4* __restrict__ zero_ptr, int64_t zero_n16) {
  zero_words(zero_ptr, zero_n16);
  extern __shared__ __align__(16) float qs[];  // [n_heads * HD]
  __shared__ float part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (uint32_t i = tid * 4; i < n_heads * HD; i += 1024)
    *reinterpret_cast<float4v*>(qs + i) = *reinterpret_cast<const float4v*>(q + i);
  const uint32_t b = blockIdx.x * 64 + lane;
  const uint32_t bc = b < nb ? b : nb - 1;  // lanes past the last block re-read it; not stored
  float k[HD];
  const float* kp = keys + (int64_t)bc * HD;
#pragma unroll
  for (int d = 0; d < HD; d += 4) {
    const float4v v = *reinterpret_cast<const float4v*>(kp + d);
    k[d] = v[0];
    k[d + 1] = v[1];
    k[d + 2] = v[2];
    k[d + 3] = v[3];
  }
  __syncthreads();
  float acc = 0.0f;
  for (uint32_t h = wave; h < n_heads; h += 4) {
    const float* qh = qs + h * HD;
    float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
#pragma unroll
    for (int d = 0; d < HD; d += 4) {
      const float4v x = *reinterpret_cast<const float4v*>(qh + d);
      d0 = fmaf(x[0], k[d], d0);
      d1 = fmaf(x[1], k[d + 1], d1);
      d2 = fmaf(x[2], k[d + 2], d2);
      d3 = fmaf(x[3], k[d + 3], d3);
    }
    acc += fmaxf((d0 + d1) + (d2 + d3), 0.0f);
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && b < nb) scores[b] = ((part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane])) * out_scale;
}

// The same scores on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: fp32 products and
// fp32 accumulation), for head counts that are a multiple of 16 (at most 64) and hd 64 or
// 128.  Each wave takes UPW units of 16 consecutive blocks and computes the 16-head x
// 16-block tiles S^T[h, b] = q[h, :] . k[b, :].  Lane l (column c = l % 16, lane group
// g = l / 16) holds, in both operands, the dims [g * HD/4, (g + 1) * HD/4): MFMA step s
// takes dim g * HD/4 + s from every group, so the steps and the four groups together
// cover each dim once.  The A operand is head m * 16 + c of the query, the B operand
// block b0 + c; the result leaves block b0 + c in lane column c with heads 4g .. 4g + 3
// of the tile in its four values.  ReLU, the sum over those heads and the head tiles in
// the lane, then the sum over the four lane groups; ×1/√hd.  Loads: each lane reads
// 128-byte (hd 128) runs of its block and of the query, all issued before the first MFMA.
template <int HD, int MT, int UPW>
__global__ __launch_bounds__(256) void qsa_decode_score_mfma_kernel(const float* __restrict__ q,
                                                                    const float* __restrict__ keys,
                                                                    float* __restrict__ scores, uint32_t nb,
                                                                    float out_scale, uint4* __restrict__ zero_ptr,
                                                                    int64_t zero_n16, uint32_t* __restrict__ tmax) {
  zero_words(zero_ptr, zero_n16);
  constexpr int KS = HD / 4;  // MFMA steps = dims per lane group
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const uint32_t units = (nb + 15) / 16;
  const uint32_t u0 = (blockIdx.x * 4 + wave) * UPW;
  if (u0 >= units) return;  // a whole wave leaves; the kernel has no barrier
  float kb[UPW][KS];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const uint32_t b = (u0 + u) * 16 + c;
    const float* src = keys + (int64_t)(b < nb ? b : nb - 1) * HD + g * KS;  // past the end: re-read, not stored
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const float4v v = *reinterpret_cast<const float4v*>(src + s);
      kb[u][s] = v[0];
      kb[u][s + 1] = v[1];
      kb[u][s + 2] = v[2];
      kb[u][s + 3] = v[3];
    }
  }
  float qa[MT][KS];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float* src = q + (m * 16 + c) * HD + g * KS;
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const float4v v = *reinterpret_cast<const float4v*>(src + s);
      qa[m][s] = v[0];
      qa[m][s + 1] = v[1];
      qa[m][s + 2] = v[2];
      qa[m][s + 3] = v[3];
    }
  }
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    float4v acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[m][s], kb[u][s], acc[m], 0, 0, 0);
    float part = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
      part += (fmaxf(acc[m][0], 0.0f) + fmaxf(acc[m][1], 0.0f)) + (fmaxf(acc[m][2], 0.0f) + fmaxf(acc[m][3], 0.0f));
    part = row_sum4(part);
    const uint32_t b = (u0 + u) * 16 + c;
    if (g == 0 && b < nb) scores[b] = part * out_scale;
    if (tmax != nullptr) {  // uniform: the unit's largest order key (every 16-lane row holds the unit)
      const uint32_t m = row_max_last(b < nb ? ord_key(part * out_scale) : 0u);
      if (lane == 15 && (u0 + u) * 16 < nb) tmax[u0 + u] = m;
    }
  }
}

// ------------------------------------------------------------------ launchers

template <typename OutT>
hipError_t launch_block_pool(const uint16_t* raw, const float* kw, OutT* out, uint32_t first_block,
                             uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot, float theta,
                             float eps, hipStream_t st) {
  const dim3 grid((n_new + 7) / 8);
  switch (hd) {
    case 64:
      hipLaunchKernelGGL((block_pool_kernel<64, OutT>), grid, dim3(256), 0, st, raw, kw, out, first_block, n_new, ratio,
                         (int)rot, theta, eps);
      break;
    case 128:
      hipLaunchKernelGGL((block_pool_kernel<128, OutT>), grid, dim3(256), 0, st, raw, kw, out, first_block, n_new, ratio,
                         (int)rot, theta, eps);
      break;
    default:
      hipLaunchKernelGGL((block_pool_kernel<256, OutT>), grid, dim3(256), 0, st, raw, kw, out, first_block, n_new, ratio,
                         (int)rot, theta, eps);
      break;
  }
  return hipGetLastError();
}

static size_t qprep_lds_bytes(uint32_t slice, uint32_t hd) { return (size_t)32 * slice + (size_t)8 * hd; }

template <int HD>
static hipError_t launch_decode_prep_hd(const uint16_t* raw, const float* kw, float* block_keys, uint32_t first_block,
                                        uint32_t n_new, uint32_t ratio, const uint16_t* qk, const float* qw,
                                        float* q_out, uint32_t rows, uint32_t first_pos, uint32_t qkw,
                                        uint32_t n_heads, uint32_t rot, float theta, float eps, hipStream_t st) {
  const uint32_t n_slices = (n_heads * (HD / 8) + kQprepDecodeSlice - 1) / kQprepDecodeSlice;
  const size_t pool_lds = sizeof(PoolLds<HD>);
  const size_t q_lds = qprep_lds_bytes(kQprepDecodeSlice, HD);
  const size_t lds = q_lds > pool_lds ? q_lds : pool_lds;
  const uint32_t grid = rows * n_slices + (n_new + kPoolNBW - 1) / kPoolNBW;
  hipLaunchKernelGGL((decode_prep_kernel<HD>), dim3(grid), dim3(256), lds, st, raw, kw, block_keys, first_block, n_new,
                     ratio, qk, qw, q_out, rows, n_slices, first_pos, qkw, n_heads, (int)rot, theta, eps);
  return hipGetLastError();
}

hipError_t launch_decode_prep(const uint16_t* raw, const float* kw, float* block_keys, uint32_t first_block,
                              uint32_t n_new, uint32_t ratio, const uint16_t* qk, const float* qw, float* q_out,
                              uint32_t rows, uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd,
                              uint32_t rot, float theta, float eps, hipStream_t st) {
  switch (hd) {
    case 64:
      return launch_decode_prep_hd<64>(raw, kw, block_keys, first_block, n_new, ratio, qk, qw, q_out, rows, first_pos,
                                       qkw, n_heads, rot, theta, eps, st);
    case 128:
      return launch_decode_prep_hd<128>(raw, kw, block_keys, first_block, n_new, ratio, qk, qw, q_out, rows,
                                        first_pos, qkw, n_heads, rot, theta, eps, st);
    default:
      return launch_decode_prep_hd<256>(raw, kw, block_keys, first_block, n_new, ratio, qk, qw, q_out, rows,
                                        first_pos, qkw, n_heads, rot, theta, eps, st);
  }
}

// Slices of 256 chunks when the rows alone fill the chip several times over, else of 128
// (a short decode batch spreads over more CUs).
template <int HD, typename OutT>
static hipError_t launch_qprep_rows_hd(const uint16_t* qk, const float* qw, OutT* out, uint32_t rows,
                                       uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t rot, float theta,
                                       float eps, hipStream_t st) {
  const uint32_t n_chunks = n_heads * (HD / 8);
  if ((uint64_t)rows * ((n_chunks + 255) / 256) >= 1024) {
    const uint32_t n_slices = (n_chunks + 255) / 256;
    hipLaunchKernelGGL((qprep_rows_kernel<HD, OutT, 256>), dim3(rows * n_slices), dim3(256),
                       qprep_lds_bytes(256, HD), st, qk, qw, out, first_pos, qkw, n_heads, n_slices, (int)rot, theta,
                       eps);
  } else {
    const uint32_t n_slices = (n_chunks + 127) / 128;
    hipLaunchKernelGGL((qprep_rows_kernel<HD, OutT, 128>), dim3(rows * n_slices), dim3(128),
                       qprep_lds_bytes(128, HD), st, qk, qw, out, first_pos, qkw, n_heads, n_slices, (int)rot, theta,
                       eps);
  }
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_qprep_rows(const uint16_t* qk, const float* qw, OutT* out, uint32_t rows,
                             uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot,
                             float theta, float eps, hipStream_t st) {
  switch (hd) {
    case 64:
      return launch_qprep_rows_hd<64, OutT>(qk, qw, out, rows, first_pos, qkw, n_heads, rot, theta, eps, st);
    case 128:
      return launch_qprep_rows_hd<128, OutT>(qk, qw, out, rows, first_pos, qkw, n_heads, rot, theta, eps, st);
    default:
      return launch_qprep_rows_hd<256, OutT>(qk, qw, out, rows, first_pos, qkw, n_heads, rot, theta, eps, st);
  }
}

template <int HD, int NH, typename InT>
static hipError_t launch_qsa_mfma(const InT* q, const InT* keys, float* scores, uint32_t rows, uint32_t nb,
                                  uint32_t first_pos, uint32_t stride, uint32_t ratio, hipStream_t st,
                                  uint32_t* tmax = nullptr, uint32_t tstride = 0) {
  constexpr uint32_t kRowsPerGroup = (kQsaThreads / 64) * (64 / NH);
  const uint32_t n_groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  // one key chunk per XCD (a multiple of the 64-key tile)
  uint32_t chunk = (nb + kXcds - 1) / kXcds;
  chunk = (chunk + 63) / 64 * 64;
  const dim3 grid(n_groups * kXcds);
  if (tmax)
    hipLaunchKernelGGL((qsa_score_mfma_kernel<HD, NH, InT, true>), grid, dim3(kQsaThreads), 0, st, q, keys, scores, rows, nb,
                     first_pos, stride, ratio, chunk, n_groups, 1.0f / sqrtf((float)HD), tmax, tstride);
  else
    hipLaunchKernelGGL((qsa_score_mfma_kernel<HD, NH, InT, false>), grid, dim3(kQsaThreads), 0, st, q, keys, scores, rows, nb,
                     first_pos, stride, ratio, chunk, n_groups, 1.0f / sqrtf((float)HD), nullptr, 0u);
  return hipGetLastError();
}

template <int HD, int MT>
static hipError_t launch_decode_mfma(const float* q, const float* keys, float* scores, uint32_t nb, float sc,
                                     uint4* zero_ptr, int64_t zero_n16, uint32_t* tmax, hipStream_t st) {
  // two 16-block units per wave once that still leaves a wave per SIMD (1024 SIMDs)
  const uint32_t units = (nb + 15) / 16;
  if (units >= 2048) {
    const dim3 grid((units + 7) / 8);
    hipLaunchKernelGGL((qsa_decode_score_mfma_kernel<HD, MT, 2>), grid, dim3(256), 0, st, q, keys, scores, nb, sc,
                       zero_ptr, zero_n16, tmax);
  } else {
    const dim3 grid((units + 3) / 4);
    hipLaunchKernelGGL((qsa_decode_score_mfma_kernel<HD, MT, 1>), grid, dim3(256), 0, st, q, keys, scores, nb, sc,
                       zero_ptr, zero_n16, tmax);
  }
  return hipGetLastError();
}

bool qsa_decode_uses_mfma(uint32_t n_heads, uint32_t hd) {
  return (hd == 64 || hd == 128) && n_heads % 16 == 0 && n_heads >= 16 && n_heads <= 64;
}

hipError_t launch_qsa_decode_score(const float* q, const float* keys, float* scores, uint32_t nb, uint32_t n_heads,
                                   uint32_t hd, uint4* zero_ptr, int64_t zero_n16, hipStream_t st, uint32_t* tmax) {
  if (tmax != nullptr && !qsa_decode_uses_mfma(n_heads, hd)) return hipErrorInvalidValue;  // maxima: matrix-core kernel only
  const float sc = 1.0f / sqrtf((float)hd);
  if (qsa_decode_uses_mfma(n_heads, hd)) {
    const uint32_t mt = n_heads / 16;
    if (hd == 64) {
      switch (mt) {
        case 1: return launch_decode_mfma<64, 1>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
        case 2: return launch_decode_mfma<64, 2>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
        case 3: return launch_decode_mfma<64, 3>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
        default: return launch_decode_mfma<64, 4>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
      }
    }
    switch (mt) {
      case 1: return launch_decode_mfma<128, 1>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
      case 2: return launch_decode_mfma<128, 2>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
      case 3: return launch_decode_mfma<128, 3>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
      default: return launch_decode_mfma<128, 4>(q, keys, scores, nb, sc, zero_ptr, zero_n16, tmax, st);
    }
  }
  const dim3 grid((nb + 63) / 64);
  const size_t lds = (size_t)n_heads * hd * 4;
  hipError_t e;
  switch (hd) {
    case 64:
      if ((e = ensure_lds(reinterpret_cast<const void*>(qsa_decode_score_kernel<64>), lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(qsa_decode_score_kernel<64>, grid, dim3(256), lds, st, q, keys, scores, nb, n_heads, sc,
                         zero_ptr, zero_n16);
      break;
    case 128:
      if ((e = ensure_lds(reinterpret_cast<const void*>(qsa_decode_score_kernel<128>), lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(qsa_decode_score_kernel<128>, grid, dim3(256), lds, st, q, keys, scores, nb, n_heads, sc,
                         zero_ptr, zero_n16);
      break;
    default:
      if ((e = ensure_lds(reinterpret_cast<const void*>(qsa_decode_score_kernel<256>), lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(qsa_decode_score_kernel<256>, grid, dim3(256), lds, st, q, keys, scores, nb, n_heads, sc,
                         zero_ptr, zero_n16);
      break;
  }
  return hipGetLastError();
}

bool qsa_score_uses_mfma(int precision, uint32_t n_heads, uint32_t hd) {
  return precision == 1 && (hd == 64 || hd == 128) && (n_heads == 16 || n_heads == 32 || n_heads == 64);
}

template hipError_t launch_block_pool<float>(const uint16_t*, const float*, float*, uint32_t, uint32_t, uint32_t,
                                             uint32_t, uint32_t, float, float, hipStream_t);
template hipError_t launch_block_pool<_Float16>(const uint16_t*, const float*, _Float16*, uint32_t, uint32_t,
                                                uint32_t, uint32_t, uint32_t, float, float, hipStream_t);
template hipError_t launch_qprep_rows<float>(const uint16_t*, const float*, float*, uint32_t, uint32_t, uint32_t,
                                             uint32_t, uint32_t, uint32_t, float, float, hipStream_t);
template hipError_t launch_qprep_rows<_Float16>(const uint16_t*, const float*, _Float16*, uint32_t, uint32_t,
                                                uint32_t, uint32_t, uint32_t, uint32_t, float, float, hipStream_t);

// fp16 q and block keys (the storage of qsa_qprep_rows_f16 / qsa_block_pool_f16): the
// matrix-core scorer only, which rounds fp32 inputs to exactly these values itself.
hipError_t launch_qsa_score_f16(const _Float16* q, const _Float16* keys, float* scores, uint32_t rows, uint32_t nb,
                                uint32_t first_pos, uint32_t stride, uint32_t ratio, uint32_t n_heads, uint32_t hd,
                                hipStream_t st, uint32_t* tmax, uint32_t tstride) {
  if (hd == 64) {
    switch (n_heads) {
      case 16: return launch_qsa_mfma<64, 16>(q, keys, scores, rows, nb, first_pos, stride, ratio, st, tmax, tstride);
      case 32: return launch_qsa_mfma<64, 32>(q, keys, scores, rows, nb, first_pos, stride, ratio, st, tmax, tstride);
      default: return launch_qsa_mfma<64, 64>(q, keys, scores, rows, nb, first_pos, stride, ratio, st, tmax, tstride);
    }
  }
  switch (n_heads) {
    case 16: return launch_qsa_mfma<128, 16>(q, keys, scores, rows, nb, first_pos, stride, ratio, st, tmax, tstride);
    case 32: return launch_qsa_mfma<128, 32>(q, keys, scores, rows, nb, first_pos, stride, ratio, st, tmax, tstride);
    default: return launch_qsa_mfma<128, 64>(q, keys, scores, rows, nb, first_pos, stride, ratio, st, tmax, tstride);
  }
}

hipError_t launch_qsa_score(const float* q, const float* keys, float* scores, uint32_t rows, uint32_t nb,
                            uint32_t first_pos, uint32_t stride, uint32_t ratio, uint32_t n_heads, uint32_t hd,
                            int precision, hipStream_t st) {
  if (qsa_score_uses_mfma(precision, n_heads, hd)) {
    if (hd == 64) {
      switch (n_heads) {
        case 16: return launch_qsa_mfma<64, 16>(q, keys, scores, rows, nb, first_pos, stride, ratio, st);
        case 32: return launch_qsa_mfma<64, 32>(q, keys, scores, rows, nb, first_pos, stride, ratio, st);
        default: return launch_qsa_mfma<64, 64>(q, keys, scores, rows, nb, first_pos, stride, ratio, st);
      }
    }
    switch (n_heads) {
      case 16: return launch_qsa_mfma<128, 16>(q, keys, scores, rows, nb, first_pos, stride, ratio, st);
      case 32: return launch_qsa_mfma<128, 32>(q, keys, scores, rows, nb, first_pos, stride, ratio, st);
      default: return launch_qsa_mfma<128, 64>(q, keys, scores, rows, nb, first_pos, stride, ratio, st);
    }
  }
  const dim3 grid((nb + 255) / 256, rows);
  switch (hd) {
    case 64:
      hipLaunchKernelGGL(qsa_score_f32_kernel<64>, grid, dim3(256), 0, st, q, keys, scores, nb, first_pos, stride,
                         ratio, n_heads);
      break;
    case 128:
      hipLaunchKernelGGL(qsa_score_f32_kernel<128>, grid, dim3(256), 0, st, q, keys, scores, nb, first_pos, stride,
                         ratio, n_heads);
      break;
    default:
      hipLaunchKernelGGL(qsa_score_f32_kernel<256>, grid, dim3(256), 0, st, q, keys, scores, nb, first_pos, stride,
                         ratio, n_heads);
      break;
  }
  return hipGetLastError();
}

}  // namespace salb
