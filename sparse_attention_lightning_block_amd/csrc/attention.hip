// Block-sparse prefill attention for gfx950 ([qsa.rs] "metrale_model_layers/layers/ops/qsa.rs",
// qsa_prefill_attn): for prefill row r at position pos = first_pos + r and query head h,
//   out[r, h] = sum_j softmax_j(inv_sqrt_d * q[r, h] . k_j) v_j
// over the positions of the row's listed complete blocks (0 <= b < floor((pos+1)/ratio))
// and of its incomplete tail [ratio * floor((pos+1)/ratio), pos], read from the paged
// bf16 K/V cache; query head h reads KV head h / (nq / nkv).
//
// One 256-thread workgroup per (row, KV head).  The row's attended positions are listed
// once in LDS (as cache rows); the four waves take 32-position steps in turn, each with
// its own online softmax, and meet in LDS at the end.  Per step and wave:
//  * S^T = K Q^T on the bf16 matrix cores (16x16x32): A = 16 positions' keys straight
//    from the cache, B = the group's query heads (N = 16, heads past the group are
//    zero).  Lane (quarter g, column c) ends with head c's scores of positions
//    4g .. 4g+3 of each 16-position tile -- exactly the 8 values it must supply, as the
//    B operand P^T, to the next product;
//  * O^T += V^T P^T on the fp16 matrix cores (16x16x32, K = the step's 32 positions in
//    the order above): A = V^T from the wave's LDS slab, where the step's values were
//    written transposed (position-contiguous per dim) as fp16 (exact for bf16 values in
//    fp16's range), B = P^T in fp16 (P in [0, 1]).  Lane (g, c) then holds head c's
//    output dims 16 nt + 4 g + i, so the softmax rescaling of a head's accumulators
//    stays in its lanes.
// Softmax in base 2 (scores times inv_sqrt_d * log2(e), v_exp_f32), fp32 throughout.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kAttnStep = 32;             // positions per wave step
constexpr int kVPitch = kAttnStep + 4;    // halves per dim row of a V^T slab (padded)

struct AttnArgs {
  const uint16_t* q;      // [rows, nq, hd] bf16
  const uint16_t* k;      // [pages, block_size, nkv, hd] bf16
  const uint16_t* v;
  const int32_t* bt;      // block table of the sequence
  const int32_t* lists;   // [rows, topk]
  float* out;             // [rows, nq, hd]
  int rows, topk, ratio, block_size, nq, nkv, group;
  int64_t first_pos;
  float scale2;           // inv_sqrt_d * log2(e)
  int tok_cap;            // LDS slots for a row's attended positions
};

// Max and sum over the four lanes of a head (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads) void prefill_attn_kernel(AttnArgs a) {
  constexpr int KW = HD / 32;   // K steps of the score product
  constexpr int NTO = HD / 16;  // output dim tiles
  extern __shared__ __align__(16) unsigned char smem[];
  int* tok_row = reinterpret_cast<int*>(smem);                                   // [tok_cap] cache rows
  int* blist = tok_row + a.tok_cap;                                               // [topk] listed blocks
  const size_t slab_off = ((size_t)(a.tok_cap + a.topk) * 4 + 15) & ~(size_t)15;
  _Float16* vslab = reinterpret_cast<_Float16*>(smem + slab_off);                // [waves][HD][kVPitch]
  __shared__ int s_wcnt[kAttnWaves];
  __shared__ float s_m[kAttnWaves][16], s_l[kAttnWaves][16];

  const int r = blockIdx.x / a.nkv, kvh = blockIdx.x % a.nkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quarter = lane >> 4;
  const int64_t pos = a.first_pos + r;
  const int64_t nb64 = (pos + 1) / a.ratio;

  // ---- the row's listed complete blocks, in list order
  int n_list = 0;
  for (int base = 0; base < a.topk; base += kAttnThreads) {
    const int i = base + tid;
    int b = -1;
    bool ok = false;
    if (i < a.topk) {
      b = a.lists[(int64_t)r * a.topk + i];
      ok = b >= 0 && (int64_t)b < nb64;
    }
    const uint64_t m = __ballot(ok);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wcnt[wave] = __popcll(m);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      woff += w < wave ? s_wcnt[w] : 0;
      tot += s_wcnt[w];
    }
    if (ok) blist[n_list + woff + before] = b;
    n_list += tot;
    __syncthreads();
  }
  // ---- attended positions as cache rows: the listed blocks, then the tail
  const int64_t tail0 = nb64 * a.ratio;
  const int n_tail = (int)(pos + 1 - tail0);
  const int n_tok = n_list * a.ratio + n_tail;
  for (int t = tid; t < n_tok; t += kAttnThreads) {
    int64_t s;
    if (t < n_list * a.ratio) {
      const int j = t / a.ratio;
      s = (int64_t)blist[j] * a.ratio + (t - j * a.ratio);
    } else {
      s = tail0 + (t - n_list * a.ratio);
    }
    const int64_t lb = s / a.block_size;
    tok_row[t] = a.bt[lb] * a.block_size + (int)(s - lb * a.block_size);
  }
  __syncthreads();

  // ---- the group's query heads as the B operand of S^T (head c = col; zeros past the group)
  bf16x8 qb[KW];
  {
    const bool hv = col < a.group;
    const int h = kvh * a.group + (hv ? col : 0);
    const uint16_t* qp = a.q + ((int64_t)r * a.nq + h) * HD + quarter * 8;
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) {
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (hv) x = *reinterpret_cast<const u32x4*>(qp + kk * 32);
      qb[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int64_t row_elems = (int64_t)a.nkv * HD;
  const uint16_t* kbase = a.k + (int64_t)kvh * HD + quarter * 8;
  const uint16_t* vbase = a.v + (int64_t)kvh * HD;
  _Float16* vt = vslab + (size_t)wave * HD * kVPitch;
  float m = -INFINITY, l = 0.0f;   // running max (base 2) and partial sum of head col
  float4v O[NTO];
#pragma unroll
  for (int nt = 0; nt < NTO; ++nt) O[nt] = float4v{0.f, 0.f, 0.f, 0.f};

  const int n_steps = (n_tok + kAttnStep - 1) / kAttnStep;
  for (int st = wave; st < n_steps; st += kAttnWaves) {
    const int v0 = st * kAttnStep;
    // keys of positions v0 + 16 t2 + col as A operands (clamped past the end: masked below)
    bf16x8 ka[2][KW];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int t = min(v0 + 16 * t2 + col, n_tok - 1);
      const uint16_t* kp = kbase + (int64_t)tok_row[t] * row_elems;
#pragma unroll
      for (int kk = 0; kk < KW; ++kk) ka[t2][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + kk * 32));
    }
    // the step's values, transposed into the wave's slab as fp16: HD units (8 groups of
    // 4 positions x HD/8 chunks of 8 dims), HD/64 per lane; unit u covers positions
    // 4 (u % 8) .. + 3 and dims 8 (u / 8) .. + 7
    static_assert(HD % 64 == 0, "units per lane");
#pragma unroll
    for (int j = 0; j < HD / 64; ++j) {
      const int u = lane + kWave * j;
      const int tg = u & 7, dc = u >> 3;
      u32x4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = min(v0 + 4 * tg + i, n_tok - 1);
        raw[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)tok_row[t] * row_elems + dc * 8);
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        _Float16 h4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = raw[i][d >> 1];
          h4[i] = (_Float16)__uint_as_float((d & 1) ? (w & 0xffff0000u) : (w << 16));
        }
        typedef _Float16 half4v __attribute__((__vector_size__(4 * sizeof(_Float16))));
        half4v hv = {h4[0], h4[1], h4[2], h4[3]};
        *reinterpret_cast<half4v*>(vt + (dc * 8 + d) * kVPitch + 4 * tg) = hv;
      }
    }
    // S^T: lane (quarter, col) gets positions 16 t2 + 4 quarter + i of head col
    float s[2][4];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KW; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t2][kk], qb[kk], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = v0 + 16 * t2 + 4 * quarter + i;
        s[t2][i] = t < n_tok ? acc[i] * a.scale2 : -INFINITY;
      }
    }
    // online softmax of head col over the step
    float tmax = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[t2][i]);
    tmax = quad_max(tmax);
    const float m_new = fmaxf(m, tmax);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? exp2f(m - m_new) : 1.0f;
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t2][i] = live ? exp2f(s[t2][i] - m_new) : 0.0f;
        psum += p[t2][i];
      }
    l = l * alpha + psum;
    m = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int nt = 0; nt < NTO; ++nt) O[nt] *= alpha;
    }
    half8v pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (_Float16)p[0][i];
      pb[4 + i] = (_Float16)p[1][i];
    }
    // O^T += V^T P^T: A for dim tile nt = slab rows 16 nt + col, positions 4 quarter .. +3
    // and 16 + 4 quarter .. +3 (the K order of pb)
#pragma unroll
    for (int nt = 0; nt < NTO; ++nt) {
      const _Float16* src = vt + (nt * 16 + col) * kVPitch + 4 * quarter;
      typedef _Float16 half4v __attribute__((__vector_size__(4 * sizeof(_Float16))));
      const half4v lo = *reinterpret_cast<const half4v*>(src);
      const half4v hi = *reinterpret_cast<const half4v*>(src + 16);
      half8v va;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        va[i] = lo[i];
        va[4 + i] = hi[i];
      }
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, O[nt], 0, 0, 0);
    }
  }

  // ---- combine the four waves: head col's max, sum and output dims 16 nt + 4 quarter + i
  const float l_tot = row_sum4(l);
  __syncthreads();  // the slabs and the position list are free again
  float* s_o = reinterpret_cast<float*>(smem);  // [waves][16][HD]
  if (quarter == 0) {
    s_m[wave][col] = m;
    s_l[wave][col] = l_tot;
  }
#pragma unroll
  for (int nt = 0; nt < NTO; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[((size_t)wave * 16 + col) * HD + nt * 16 + 4 * quarter + i] = O[nt][i];
  __syncthreads();
  for (int idx = tid; idx < a.group * HD; idx += kAttnThreads) {
    const int h = idx / HD, d = idx - h * HD;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float num = 0.0f, den = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = s_m[w][h] == -INFINITY ? 0.0f : exp2f(s_m[w][h] - mx);
        num += f * s_o[((size_t)w * 16 + h) * HD + d];
        den += f * s_l[w][h];
      }
    }
    a.out[((int64_t)r * a.nq + kvh * a.group + h) * HD + d] = den > 0.0f ? num / den : 0.0f;
  }
}

size_t prefill_attn_lds_bytes(int topk, int ratio, int hd) {
  const size_t tok_cap = (size_t)topk * ratio + ratio;
  const size_t head = ((tok_cap + topk) * 4 + 15) & ~(size_t)15;
  const size_t slabs = (size_t)kAttnWaves * hd * kVPitch * 2;
  const size_t combine = (size_t)kAttnWaves * 16 * hd * 4;
  const size_t body = head + slabs;
  return body > combine ? body : combine;
}

hipError_t launch_prefill_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* bt,
                               const int32_t* lists, float* out, int rows, int64_t first_pos, int topk, int ratio,
                               int block_size, int nq, int nkv, int hd, float inv_sqrt_d, hipStream_t st) {
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.bt = bt;
  a.lists = lists;
  a.out = out;
  a.rows = rows;
  a.topk = topk;
  a.ratio = ratio;
  a.block_size = block_size;
  a.nq = nq;
  a.nkv = nkv;
  a.group = nq / nkv;
  a.first_pos = first_pos;
  a.scale2 = inv_sqrt_d * 1.4426950408889634f;
  a.tok_cap = topk * ratio + ratio;
  const size_t lds = prefill_attn_lds_bytes(topk, ratio, hd);
  const dim3 grid((unsigned)((int64_t)rows * nkv));
  hipError_t e;
  if (hd == 64) {
    if ((e = ensure_lds(reinterpret_cast<const void*>(prefill_attn_kernel<64>), lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_attn_kernel<64>, grid, dim3(kAttnThreads), lds, st, a);
  } else {
    if ((e = ensure_lds(reinterpret_cast<const void*>(prefill_attn_kernel<128>), lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_attn_kernel<128>, grid, dim3(kAttnThreads), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace salb
