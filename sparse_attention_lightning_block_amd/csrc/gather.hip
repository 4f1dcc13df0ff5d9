// Selected-entry gathers for gfx950: the top-k indices turned into dense tiles.
//
//  * gather_kv ([commits] "nvfp4-megamoe-kernel -- commit graph of dsv4/kernels/indexer",
//    c2f705a21a, gather_kv.cu): for every (query t, slot i) with s = topk_idx[t, i] >= 0,
//    the entry is resolved through the query's block table, its FP8 E4M3 part times its
//    fp32 group scale is rounded once to bf16, and its bf16 RoPE part is copied: a dense
//    [T, top_k, d_nope + d_rope] bf16 tile.  Slots with index -1 get zeros.
//  * qsa_gather ([qsa.rs] "metrale_model_layers/layers/ops/qsa.rs", qsa_gather): the
//    selected positions' K and V rows ([nkv, hd] each) copied into [n_sel, nkv, hd].
//
// Both are pure data movement, bound by HBM.  The FP8 gather's work is a flat list of
// (output row, 16-byte chunk) items, one per thread: the grid covers every item (up to
// 16384 workgroups; beyond that a grid-stride loop), so that the chains of dependent
// loads (index, block-table entry, data) of many threads are in flight at once -- more
// threads with one chain each measured faster than fewer threads with four, and faster
// than one wave per row (its 40 busy lanes of 64 carry all of a row's conversions).  The
// QSA gather, a plain copy, takes one wave per selected position: the position and its
// table entry are loaded once per row, and every lane copies 16-byte chunks.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace salb {

constexpr int kGatherThreads = 256;
constexpr int kGatherItems = 1;  // items per thread and pass of the FP8 gather

// One rounding of the exact product a * s to bfloat16 (round to nearest, ties to even).
// p = RN32(a * s) and e = a * s - p (exact through the fma) decide it: bfloat16's ties
// sit on fp32 values, and when p lands exactly on one the sign of e says on which side
// the exact product lies; elsewhere rounding p is rounding the product, since the exact
// value is within half an fp32 spacing of p and cannot cross a tie point that is not p.
// (Exact for products in the normal fp32 range; a and s are finite.)
__device__ __forceinline__ uint32_t bf16_of_product(float a, float s) {
  const float p = a * s;
  const float e = fmaf(a, s, -p);
  const uint32_t b = __float_as_uint(p);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u | ((b >> 16) & 0x8000u);  // NaN
  if ((b & 0xffffu) == 0x8000u && e != 0.0f) {
    // on a tie: round away from zero iff the exact product is larger in magnitude
    const bool up = (e > 0.0f) == (p > 0.0f);
    return (b >> 16) + (up ? 1u : 0u);
  }
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

struct GatherKvArgs {
  const uint8_t* fp8;
  const float* scale;
  const uint16_t* rope;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* idx;
  uint16_t* out;
  int64_t n_items;  // T * top_k * cpr
  int top_k, epb, n_cols;
  int d_nope, d_rope, group;
  int cpr_nope, cpr;  // chunks per row: d_nope / 16 FP8 chunks, then d_rope / 8 rope chunks
  uint64_t epb_magic;
};

// Rows per wave and pass of the QSA gather (its waves copy whole rows).
constexpr int kRowsPerWave = 2;

__global__ __launch_bounds__(kGatherThreads) void gather_kv_kernel(GatherKvArgs a) {
  const int64_t step = (int64_t)gridDim.x * kGatherThreads;
  for (int64_t base = (int64_t)blockIdx.x * kGatherThreads + threadIdx.x; base < a.n_items;
       base += step * kGatherItems) {
    int64_t item[kGatherItems];
    int64_t row[kGatherItems];
    int chunk[kGatherItems];
    int s[kGatherItems];
#pragma unroll
    for (int u = 0; u < kGatherItems; ++u) {
      item[u] = base + u * step;
      const int64_t it = item[u] < a.n_items ? item[u] : 0;
      row[u] = it / a.cpr;
      chunk[u] = (int)(it - row[u] * a.cpr);
      s[u] = item[u] < a.n_items ? a.idx[row[u]] : -1;
    }
    int64_t ent[kGatherItems];
#pragma unroll
    for (int u = 0; u < kGatherItems; ++u) {
      ent[u] = -1;
      if (s[u] >= 0 && s[u] < a.n_cols) {  // -1 (and anything outside the table) is padding
        const int t = (int)(row[u] / a.top_k);
        const uint32_t lb = div_epb((uint32_t)s[u], a.epb_magic);
        const int p = a.bt[(int64_t)t * a.bt_stride + lb];
        ent[u] = (int64_t)p * a.epb + (int64_t)((uint32_t)s[u] - lb * (uint32_t)a.epb);
      }
    }
    u32x4 raw[kGatherItems];
    float sc[kGatherItems];
#pragma unroll
    for (int u = 0; u < kGatherItems; ++u) {
      raw[u] = u32x4{0u, 0u, 0u, 0u};
      sc[u] = 0.0f;
      if (ent[u] >= 0) {
        if (chunk[u] < a.cpr_nope) {
          raw[u] = *reinterpret_cast<const u32x4*>(a.fp8 + ent[u] * a.d_nope + chunk[u] * 16);
          sc[u] = a.scale[ent[u] * (a.d_nope / a.group) + (chunk[u] * 16) / a.group];
        } else {
          raw[u] = *reinterpret_cast<const u32x4*>(a.rope + ent[u] * a.d_rope + (chunk[u] - a.cpr_nope) * 8);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherItems; ++u) {
      if (item[u] >= a.n_items) continue;
      uint16_t* dst = a.out + row[u] * (a.d_nope + a.d_rope);
      if (chunk[u] < a.cpr_nope) {
        // 16 E4M3 codes -> 16 bf16, two 16-byte stores
        u32x4 o0, o1;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
          const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[u][wv], false);
          const float2v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[u][wv], true);
          const uint32_t w0 = bf16_of_product(lo[0], sc[u]) | (bf16_of_product(lo[1], sc[u]) << 16);
          const uint32_t w1 = bf16_of_product(hi[0], sc[u]) | (bf16_of_product(hi[1], sc[u]) << 16);
          if (wv < 2) {
            o0[2 * wv] = w0;
            o0[2 * wv + 1] = w1;
          } else {
            o1[2 * (wv - 2)] = w0;
            o1[2 * (wv - 2) + 1] = w1;
          }
        }
        if (ent[u] < 0) o0 = o1 = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(dst + chunk[u] * 16) = o0;
        *reinterpret_cast<u32x4*>(dst + chunk[u] * 16 + 8) = o1;
      } else {
        *reinterpret_cast<u32x4*>(dst + a.d_nope + (chunk[u] - a.cpr_nope) * 8) = raw[u];
      }
    }
  }
}

struct QsaGatherArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* sel;
  uint16_t* k_out;
  uint16_t* v_out;
  int64_t n_items;  // n_sel
  int block_size, row_elems, cpr;  // row_elems = nkv * hd; cpr = row_elems / 8
};

// One wave per selected position, kRowsPerWave at a time: the position's table entry
// is loaded once (the same address in every lane), and the lanes copy the K and V rows
// in 16-byte chunks.
__global__ __launch_bounds__(kGatherThreads) void qsa_gather_kernel(QsaGatherArgs a) {
  constexpr int WPB = kGatherThreads / 64;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * WPB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n_rows = a.n_items;  // n_sel
  const int64_t step = (int64_t)gridDim.x * WPB * kRowsPerWave;
  for (int64_t r0 = wave * kRowsPerWave; r0 < n_rows; r0 += step) {
    int64_t src[kRowsPerWave];
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
      const int64_t r = r0 + u < n_rows ? r0 + u : n_rows - 1;  // past the end: re-read the last, not stored
      const uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane(a.sel[r]);
      const uint32_t lb = pos / (uint32_t)a.block_size;
      const int64_t phys = __builtin_amdgcn_readfirstlane(a.bt[lb]);
      src[u] = (phys * a.block_size + (pos - lb * (uint32_t)a.block_size)) * a.row_elems;
    }
    for (int c = lane; c < a.cpr; c += 64) {
      u32x4 xk[kRowsPerWave], xv[kRowsPerWave];
#pragma unroll
      for (int u = 0; u < kRowsPerWave; ++u) {
        xk[u] = *reinterpret_cast<const u32x4*>(a.k + src[u] + c * 8);
        xv[u] = *reinterpret_cast<const u32x4*>(a.v + src[u] + c * 8);
      }
#pragma unroll
      for (int u = 0; u < kRowsPerWave; ++u) {
        if (r0 + u >= n_rows) continue;
        const int64_t dst = (r0 + u) * a.row_elems + c * 8;
        *reinterpret_cast<u32x4*>(a.k_out + dst) = xk[u];
        *reinterpret_cast<u32x4*>(a.v_out + dst) = xv[u];
      }
    }
  }
}

// Workgroups for one item per thread (at most 16384; beyond that a grid-stride loop).
static unsigned gather_grid(int64_t n_items) {
  const int64_t want = (n_items + (int64_t)kGatherThreads * kGatherItems - 1) / ((int64_t)kGatherThreads * kGatherItems);
  return (unsigned)(want < 16384 ? (want > 0 ? want : 1) : 16384);
}

// Workgroups for one wave per kRowsPerWave rows (at most 16384; beyond that the waves
// loop over the rows).
static unsigned gather_rows_grid(int64_t n_rows) {
  const int64_t waves = (n_rows + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t want = (waves + kGatherThreads / 64 - 1) / (kGatherThreads / 64);
  return (unsigned)(want < 16384 ? (want > 0 ? want : 1) : 16384);
}

hipError_t launch_gather_kv(const uint8_t* fp8, const float* scale, const uint16_t* rope, const int32_t* bt,
                            int64_t bt_stride, const int32_t* idx, int T, int top_k, int epb, int max_lb,
                            int d_nope, int d_rope, int group, uint16_t* out, hipStream_t st) {
  GatherKvArgs a{};
  a.fp8 = fp8;
  a.scale = scale;
  a.rope = rope;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.idx = idx;
  a.out = out;
  a.top_k = top_k;
  a.epb = epb;
  a.n_cols = max_lb * epb;
  a.d_nope = d_nope;
  a.d_rope = d_rope;
  a.group = group;
  a.cpr_nope = d_nope / 16;
  a.cpr = a.cpr_nope + d_rope / 8;
  a.n_items = (int64_t)T * top_k * a.cpr;
  a.epb_magic = host_epb_magic(epb);
  hipLaunchKernelGGL(gather_kv_kernel, dim3(gather_grid(a.n_items)), dim3(kGatherThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_qsa_gather(const uint16_t* k, const uint16_t* v, const int32_t* bt, const int32_t* sel,
                             uint16_t* k_out, uint16_t* v_out, int n_sel, int block_size, int nkv, int hd,
                             hipStream_t st) {
  QsaGatherArgs a{};
  a.k = k;
  a.v = v;
  a.bt = bt;
  a.sel = sel;
  a.k_out = k_out;
  a.v_out = v_out;
  a.block_size = block_size;
  a.row_elems = nkv * hd;
  a.cpr = a.row_elems / 8;
  a.n_items = n_sel;  // selected positions, one wave each
  hipLaunchKernelGGL(qsa_gather_kernel, dim3(gather_rows_grid(a.n_items)), dim3(kGatherThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace salb
