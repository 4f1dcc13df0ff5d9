// QSA block-pooled indexer variant for gfx950 ([qsa.rs] "metrale_model_layers/layers/ops/qsa.rs":
// doc comments of qsa_block_pool, qsa_qprep / qsa_qprep_rows, qsa_score and qsa_score_rows).
//
//  * block pool: mean of `ratio` raw bf16 keys -> RMSNorm scaled by (1 + w) -> RoPE at
//    the block's first token position; one workgroup per pooled block, 16-byte loads.
//  * query prep: per (row, head) RMSNorm scaled by (1 + w) -> RoPE at first_pos + row.
//  * row scores: sum_h ReLU(q_h . k_b) / sqrt(hd), -inf past the row's complete blocks.
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

hipError_t launch_qsa_score(const float* q, const float* keys, float* scores, uint32_t rows, uint32_t nb,
                            uint32_t first_pos, uint32_t stride, uint32_t ratio, uint32_t n_heads, uint32_t hd,
                            int precision, hipStream_t st) {
  (void)precision;
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
