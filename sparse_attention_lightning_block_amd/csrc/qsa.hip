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
// cosine and the rotation are evaluated in fp64.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Sum over the block (blockDim.x <= 256, a multiple of 64).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) s += red[w];
  __syncthreads();
  return s;
}

// Rotate the pairs (i, i + rot/2) of x (in LDS, fp32) at position pos; thread d < rot/2
// writes both members of its pair into `out`.
__device__ __forceinline__ void rope_pair(const float* x, float* out_row, int d, int hd, int rot, double pos,
                                          double theta) {
  const int half = rot >> 1;
  if (d < half) {
    const double inv_freq = pow(theta, -2.0 * (double)d / (double)rot);
    double s, c;
    sincos(pos * inv_freq, &s, &c);
    const double a = x[d], b = x[d + half];
    out_row[d] = (float)(a * c - b * s);
    out_row[d + half] = (float)(a * s + b * c);
  } else if (d >= rot && d < hd) {
    out_row[d] = x[d];
  }
}

// ------------------------------------------------------------------ block pool

template <int HD>
__global__ __launch_bounds__(256) void block_pool_kernel(const uint16_t* __restrict__ raw,
                                                         const float* __restrict__ kw, float* __restrict__ out,
                                                         uint32_t first_block, uint32_t ratio, int rot,
                                                         float theta, float eps) {
  constexpr int CG = HD / 8;        // 16-byte column groups per row
  constexpr int RL = 256 / CG;      // rows handled in parallel
  __shared__ float part[RL][HD];
  __shared__ float xs[HD];
  __shared__ float red[4];
  const uint32_t b = first_block + blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rl = tid / CG;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* base = raw + (int64_t)b * ratio * HD;
  for (uint32_t r = rl; r < ratio; r += RL) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + (int64_t)r * HD + cg * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rl][cg * 8 + i] = acc[i];
  __syncthreads();
  float m = 0.0f;
  if (tid < HD) {
    for (int r = 0; r < RL; ++r) m += part[r][tid];
    m = m / (float)ratio;
  }
  const float ss = block_sum(tid < HD ? m * m : 0.0f, red);
  const float inv = 1.0f / sqrtf(ss / (float)HD + eps);
  if (tid < HD) xs[tid] = m * inv * (1.0f + kw[tid]);
  __syncthreads();
  rope_pair(xs, out + (int64_t)b * HD, tid, HD, rot, (double)b * (double)ratio, (double)theta);
}

// ------------------------------------------------------------------ query prep

template <int HD>
__global__ __launch_bounds__(HD) void qprep_rows_kernel(const uint16_t* __restrict__ qk,
                                                        const float* __restrict__ qw, float* __restrict__ out,
                                                        uint32_t first_pos, uint32_t qkw, uint32_t n_heads,
                                                        int rot, float theta, float eps) {
  __shared__ float xs[HD];
  __shared__ float red[4];
  const uint32_t r = blockIdx.x, h = blockIdx.y;
  const int d = threadIdx.x;
  const float x = bf16_to_f32(qk[(int64_t)r * qkw + (int64_t)h * HD + d]);
  const float ss = block_sum(x * x, red);
  const float inv = 1.0f / sqrtf(ss / (float)HD + eps);
  xs[d] = x * inv * (1.0f + qw[d]);
  __syncthreads();
  rope_pair(xs, out + ((int64_t)r * n_heads + h) * HD, d, HD, rot, (double)first_pos + (double)r, (double)theta);
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
// of q as A operands (RPW = 64 / NH rows); a workgroup (4 waves, RPG rows) streams
// its key chunk in 64-key tiles converted to fp16 in LDS (two buffers: the next
// tile's loads are in flight while the current one is multiplied).  The chunks are
// dealt so that all workgroups of one chunk run on one XCD: the chunk's keys (2 MB
// at 32768 blocks) stay in that XCD's L2.  q and the keys come out of RMSNorm, so
// their fp16 roundings are relative (2^-11) and the products stay far inside the
// fp16 range; the accumulation is fp32.
template <int HD, int NH>
__global__ __launch_bounds__(256) void qsa_score_mfma_kernel(const float* __restrict__ q,
                                                             const float* __restrict__ keys,
                                                             float* __restrict__ scores, uint32_t rows,
                                                             uint32_t nb, uint32_t first_pos, uint32_t stride,
                                                             uint32_t ratio, uint32_t chunk, uint32_t n_groups,
                                                             float out_scale) {
  constexpr int KW = HD / 32;     // K steps of 32 dims
  constexpr int RPW = 64 / NH;    // rows per wave
  constexpr int RPG = 4 * RPW;    // rows per workgroup
  constexpr int MTR = NH / 16;    // M tiles per row
  constexpr int TILE = 64;
  constexpr int BLD = HD + 8;     // halves per LDS key row (padding against bank conflicts)
  constexpr int LPK = 4;          // loader threads per key
  constexpr int FPL = HD / LPK;   // floats each loader thread converts per tile
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
  // keys of the chunk past every row's valid count: -inf
  for (int rr = 0; rr < RPG; ++rr) {
    const int r = r0 + rr;
    if (r >= (int)rows) break;
    const int64_t from = kend > c0 ? kend : c0;
    for (int64_t s = from + tid; s < c1; s += 256) scores[(int64_t)r * stride + s] = -INFINITY;
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
        const float* src = q + ((int64_t)r * NH + h) * HD + 32 * kk + 8 * quarter;
        const float4v x0 = *reinterpret_cast<const float4v*>(src);
        const float4v x1 = *reinterpret_cast<const float4v*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (_Float16)x0[e];
          a[4 + e] = (_Float16)x1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (_Float16)0.0f;
      }
      A[mt][kk] = a;
    }
  }
  int64_t vrow[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = r0 + wave * RPW + rr;
    vrow[rr] = r < (int)rows ? valid_of(r) : 0;
  }

  // tile loader: thread t converts FPL floats of key t / LPK
  const int lk = tid / LPK, lpart = tid % LPK;
  float4v stage[FPL / 4];
  auto load_tile = [&](int64_t k0) {
    const int64_t kk = k0 + lk;
    if (kk < kend) {
      const float* src = keys + kk * HD + lpart * FPL;
#pragma unroll
      for (int j = 0; j < FPL / 4; ++j) stage[j] = *reinterpret_cast<const float4v*>(src + 4 * j);
    } else {
#pragma unroll
      for (int j = 0; j < FPL / 4; ++j) stage[j] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  auto store_tile = [&](int buf) {
    _Float16* dst = &kb[buf][lk * BLD + lpart * FPL];
#pragma unroll
    for (int j = 0; j < FPL / 8; ++j) {
      half8v h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = (_Float16)stage[2 * j][e];
        h[4 + e] = (_Float16)stage[2 * j + 1][e];
      }
      *reinterpret_cast<half8v*>(dst + 8 * j) = h;
    }
  };

  load_tile(c0);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  for (int64_t k0 = c0; k0 < kend; k0 += TILE) {
    const bool more = k0 + TILE < kend;
    if (more) load_tile(k0 + TILE);
    float4v acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      half8v B[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        B[nt] = *reinterpret_cast<const half8v*>(&kb[buf][(16 * nt + col) * BLD + 32 * kk + 8 * quarter]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][kk], B[nt], acc[mt][nt], 0, 0, 0);
    }
    // ReLU and head sum: lane (quarter, col) holds heads 4*quarter + i of each M tile
    // for key 16 * nt + col; the four quarters are then summed across lanes.
    float s[4][RPW];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        float x = 0.0f;
#pragma unroll
        for (int j = 0; j < MTR; ++j) {
          const float4v a = acc[rr * MTR + j][nt];
          x += fmaxf(a[0], 0.0f) + fmaxf(a[1], 0.0f) + fmaxf(a[2], 0.0f) + fmaxf(a[3], 0.0f);
        }
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        s[nt][rr] = x;
      }
    }
    // lane (quarter, col) writes key 16 * quarter + col of the tile for each row
    const int64_t key = k0 + 16 * quarter + col;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = r0 + wave * RPW + rr;
      float v = s[0][rr];
#pragma unroll
      for (int nt = 1; nt < 4; ++nt) v = quarter == nt ? s[nt][rr] : v;
      if (r < (int)rows && key < c1) scores[(int64_t)r * stride + key] = key < vrow[rr] ? v * out_scale : -INFINITY;
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_block_pool(const uint16_t* raw, const float* kw, float* out, uint32_t first_block,
                             uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot, float theta,
                             float eps, hipStream_t st) {
  switch (hd) {
    case 64:
      hipLaunchKernelGGL(block_pool_kernel<64>, dim3(n_new), dim3(256), 0, st, raw, kw, out, first_block, ratio,
                         (int)rot, theta, eps);
      break;
    case 128:
      hipLaunchKernelGGL(block_pool_kernel<128>, dim3(n_new), dim3(256), 0, st, raw, kw, out, first_block, ratio,
                         (int)rot, theta, eps);
      break;
    default:
      hipLaunchKernelGGL(block_pool_kernel<256>, dim3(n_new), dim3(256), 0, st, raw, kw, out, first_block, ratio,
                         (int)rot, theta, eps);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_qprep_rows(const uint16_t* qk, const float* qw, float* out, uint32_t rows,
                             uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot,
                             float theta, float eps, hipStream_t st) {
  switch (hd) {
    case 64:
      hipLaunchKernelGGL(qprep_rows_kernel<64>, dim3(rows, n_heads), dim3(64), 0, st, qk, qw, out, first_pos, qkw,
                         n_heads, (int)rot, theta, eps);
      break;
    case 128:
      hipLaunchKernelGGL(qprep_rows_kernel<128>, dim3(rows, n_heads), dim3(128), 0, st, qk, qw, out, first_pos,
                         qkw, n_heads, (int)rot, theta, eps);
      break;
    default:
      hipLaunchKernelGGL(qprep_rows_kernel<256>, dim3(rows, n_heads), dim3(256), 0, st, qk, qw, out, first_pos,
                         qkw, n_heads, (int)rot, theta, eps);
      break;
  }
  return hipGetLastError();
}

template <int HD, int NH>
static hipError_t launch_qsa_mfma(const float* q, const float* keys, float* scores, uint32_t rows, uint32_t nb,
                                  uint32_t first_pos, uint32_t stride, uint32_t ratio, hipStream_t st) {
  constexpr uint32_t kRowsPerGroup = 4 * (64 / NH);
  const uint32_t n_groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  // one key chunk per XCD (a multiple of the 64-key tile)
  uint32_t chunk = (nb + kXcds - 1) / kXcds;
  chunk = (chunk + 63) / 64 * 64;
  const dim3 grid(n_groups * kXcds);
  hipLaunchKernelGGL((qsa_score_mfma_kernel<HD, NH>), grid, dim3(256), 0, st, q, keys, scores, rows, nb, first_pos,
                     stride, ratio, chunk, n_groups, 1.0f / sqrtf((float)HD));
  return hipGetLastError();
}

bool qsa_score_uses_mfma(int precision, uint32_t n_heads, uint32_t hd) {
  return precision == 1 && (hd == 64 || hd == 128) && (n_heads == 16 || n_heads == 32 || n_heads == 64);
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
