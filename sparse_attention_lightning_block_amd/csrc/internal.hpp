// Internal interfaces between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace salb {

struct ScoreArgs {
  const void* q;
  int q_bf16;
  const float* w;
  const uint8_t* keys;
  const uint8_t* kscale;
  const float* gscale;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* valid_lens;
  int T, H, D, epb, max_lb;
  uint64_t epb_magic;
  float* scores;
  int64_t score_stride;
  int n_cols;
  int write_tail;  // 1: s in [valid, n_cols) gets -inf
  // 16-byte words the launch zeroes besides its scores (the select counters of the
  // fused path, so that the select needs no clearing launch of its own)
  uint4* zero_ptr;
  int64_t zero_n16;
  // filled by the launcher
  int chunk;       // keys per workgroup
  int n_chunks;
  int pid_cap;     // LDS slots for the chunk's block-table entries
  int swizzle;     // 1: chunk-major XCD grouping (see score_tile)
  int balance;     // 1: group scorer work split evenly over the grid by weighted tiles
};

hipError_t launch_score_rows(ScoreArgs a, int precision, hipStream_t st);
hipError_t launch_debug_dequant(const uint8_t* keys, const uint8_t* kscale, const float* gscale,
                                const int32_t* bt_row, int n, int D, int epb, int mode, float* out,
                                hipStream_t st);

// Checks valid lengths and the block-table entries they use (validate.hip); waits for
// the result.  host_status[0]: first bad row (-1 none), [1]: first bad row*max_lb+block.
hipError_t validate_pages(const int32_t* bt, int64_t bt_stride, const int32_t* valid_lens, int T, int max_lb, int epb,
                          int cap, int n_pages, int64_t* dev_status, int64_t host_status[2], hipStream_t st);

// Per-row top-k (topk.hip).
constexpr int kMaxTopK = 8192;

struct SelectPlan {
  int rows, n_cols, top_k;
  int two_pass;   // 0: one workgroup per row; 1: histogram + filter grid over (chunk, row)
  int row_nt;     // threads of the one-workgroup rows (two_pass == 0)
  int cand_cap;   // LDS candidate slots of a one-workgroup row kept in LDS (per == 0)
  int per;        // entries per thread (a row, or a chunk of the two-pass grid)
  int chunks;     // chunks per row (two-pass)
  int final_nt;   // threads of the finishing workgroup (two-pass)
  size_t lds;     // dynamic LDS of a workgroup that finishes a row
  size_t bytes;   // workspace bytes
};

bool plan_select(int rows, int n_cols, int top_k, SelectPlan* p);
// counters_zeroed: the first select_counter_bytes(p) bytes of ws were zeroed by an
// earlier launch of this call on the same stream (else the select zeroes them itself).
// The sub-tile select (rows of at most 32768 entries whose 16-entry sub-tiles come with
// their largest order key; top_k <= 512; rows 16-byte aligned, stride a multiple of 16).
bool tile_select_fits(int n_cols, int top_k);
hipError_t launch_select_tiles(const float* scores, int64_t score_stride, const uint32_t* tmax, int64_t tmax_stride,
                               int64_t first_pos, int ratio, int rows, int n_cols, int top_k, int32_t* out_idx,
                               float* out_scores, hipStream_t st);
hipError_t launch_select(const SelectPlan& p, const float* scores, int64_t score_stride,
                         const int32_t* valid_lens, int64_t first_pos, int ratio, int32_t* out_idx,
                         float* out_scores, void* ws, bool counters_zeroed, hipStream_t st);
size_t select_counter_bytes(const SelectPlan& p);
size_t select_workspace_bytes(int rows, int n_cols, int top_k);  // 0 if unsupported

// Selected-entry gathers (gather.hip).
hipError_t launch_gather_kv(const uint8_t* fp8, const float* scale, const uint16_t* rope, const int32_t* bt,
                            int64_t bt_stride, const int32_t* idx, int T, int top_k, int epb, int max_lb,
                            int d_nope, int d_rope, int group, uint16_t* out, hipStream_t st);
hipError_t launch_qsa_gather(const uint16_t* k, const uint16_t* v, const int32_t* bt, const int32_t* sel,
                             uint16_t* k_out, uint16_t* v_out, int n_sel, int block_size, int nkv, int hd,
                             hipStream_t st);

// Block-sparse prefill attention (attention.hip).
size_t prefill_attn_lds_bytes(int topk, int ratio, int hd);
hipError_t launch_prefill_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* bt,
                               const int32_t* lists, float* out, int rows, int64_t first_pos, int topk, int ratio,
                               int block_size, int nq, int nkv, int hd, float inv_sqrt_d, hipStream_t st);

// QSA (qsa.hip).
// OutT float or _Float16 (fp16 storage, each fp32 result rounded to nearest even)
template <typename OutT>
hipError_t launch_block_pool(const uint16_t* raw, const float* kw, OutT* out, uint32_t first_block,
                             uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot, float theta,
                             float eps, hipStream_t st);
template <typename OutT>
hipError_t launch_qprep_rows(const uint16_t* qk, const float* qw, OutT* out, uint32_t rows,
                             uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot,
                             float theta, float eps, hipStream_t st);
// The query rows' prep and the new blocks' pooling (fp32 outputs) in one launch.
hipError_t launch_decode_prep(const uint16_t* raw, const float* kw, float* block_keys, uint32_t first_block,
                              uint32_t n_new, uint32_t ratio, const uint16_t* qk, const float* qw, float* q_out,
                              uint32_t rows, uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd,
                              uint32_t rot, float theta, float eps, hipStream_t st);
// tmax (nullable): [rows][tstride] order-key maxima of the 16-block sub-tiles.
hipError_t launch_qsa_score_f16(const _Float16* q, const _Float16* keys, float* scores, uint32_t rows, uint32_t nb,
                                uint32_t first_pos, uint32_t stride, uint32_t ratio, uint32_t n_heads, uint32_t hd,
                                hipStream_t st, uint32_t* tmax = nullptr, uint32_t tstride = 0);
bool qsa_score_uses_mfma(int precision, uint32_t n_heads, uint32_t hd);
// zero_ptr / zero_n16: 16-byte words the launch also zeroes (0 words: none)
// Whether the decode scores run on the fp32 matrix cores (the kernel that can also write
// the 16-block sub-tile maxima).
bool qsa_decode_uses_mfma(uint32_t n_heads, uint32_t hd);
hipError_t launch_qsa_decode_score(const float* q, const float* keys, float* scores, uint32_t nb, uint32_t n_heads,
                                   uint32_t hd, uint4* zero_ptr, int64_t zero_n16, hipStream_t st, uint32_t* tmax = nullptr);
hipError_t launch_qsa_score(const float* q, const float* keys, float* scores, uint32_t rows, uint32_t nb,
                            uint32_t first_pos, uint32_t stride, uint32_t ratio, uint32_t n_heads, uint32_t hd,
                            int precision, hipStream_t st);

}  // namespace salb
