// Shared device/host helpers for the gfx950 indexer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

namespace salb {

typedef _Float16 half2v __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef _Float16 half8v __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float float4v __attribute__((__vector_size__(4 * sizeof(float))));
typedef float float2v __attribute__((__vector_size__(2 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs; workgroup b is dispatched to XCD b % 8

// ---------------------------------------------------------------------------
// Total order used by every top-k: score descending, ties by lower index.
// A float maps to a 32-bit key whose unsigned order is the float order, with
// -0.0 merged into +0.0 and NaN mapped to the smallest key.  The 64-bit
// composite (key << 32) | ~index is unique per entry and its unsigned order is
// exactly the selection order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of ord_key on its image; key 0 (every NaN) gives the canonical quiet NaN.
__device__ __forceinline__ float ord_to_float(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint32_t)(~idx);
}

// ReLU through the integer max: a negative float (sign bit set) is a negative int32,
// so max(bits, 0) gives +0.0 for it and leaves non-negative values unchanged.  One
// VALU op, with no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum over the four 16-lane rows of a wave, for every lane position within a row
// (the xor-16 and xor-32 butterflies).  gfx950's row-swap permutes exchange rows
// between two registers on the VALU: swapping x with itself and adding the pair
// gives the butterfly without an LDS round trip.
__device__ __forceinline__ float row_sum4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over all 64 lanes, the same total in every lane: butterflies within quads and
// 16-lane rows through DPP (quad permutes, then the half-row and row mirrors, which
// pair a lane with one holding the other quad's or half's sum), then across the rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return row_sum4(x);
}

// Four values per lane, x0..x3; lane i of row r (lanes 16 r .. 16 r + 15) returns the
// sum of x_r over lane i of all four rows -- four butterflies' worth of sums, each
// kept by one row, in three row swaps.  The 32-lane swap of (x0, x2) leaves the lower
// half with x0 of both halves and the upper half with x2 of both; likewise (x1, x3);
// the 16-lane swap of those two then pairs rows 0/1 and 2/3.
__device__ __forceinline__ float row_transpose_sum4(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x1), __float_as_uint(x3), false, false);
  const float y02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float y13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(y02), __float_as_uint(y13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Exact floor(s / epb) for s < 2^24 and epb <= 2^16: m = ceil(2^40 / epb).
__device__ __forceinline__ uint32_t div_epb(uint32_t s, uint64_t magic) {
  return (uint32_t)(((uint64_t)s * magic) >> 40);
}

inline uint64_t host_epb_magic(int epb) {
  return (((uint64_t)1 << 40) + (uint64_t)epb - 1) / (uint64_t)epb;
}

// Reverse of the XCD round-robin: blocks b with equal b % 8 share an XCD (and its
// L2).  Work item (chunk, row) is assigned so that each XCD walks chunks
// c = xcd, xcd + 8, ... and, for each of them, all rows: rows that read the same
// pages (shared block tables) do so from the same L2 at about the same time.
struct XcdTile {
  int chunk;
  int row;
};

__device__ __forceinline__ XcdTile xcd_tile(int b, int rows) {
  int xcd = b & (kXcds - 1);
  int j = b >> 3;
  XcdTile t;
  t.row = j % rows;
  t.chunk = (j / rows) * kXcds + xcd;
  return t;
}

// Raises a kernel's dynamic-LDS limit (needed above 64 KiB) once: later calls return
// without touching the runtime, so launches made while a stream is captured into a
// graph issue no attribute calls.
inline hipError_t ensure_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> raised;
  std::lock_guard<std::mutex> lock(mu);
  auto it = raised.find(fn);
  if (it != raised.end() && it->second >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) raised[fn] = bytes;
  return e;
}

}  // namespace salb
