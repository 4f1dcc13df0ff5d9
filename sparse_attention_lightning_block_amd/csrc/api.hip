// C ABI of the gfx950 indexer library: argument checks, workspace layout, dispatch.
// Every check runs on the host before any HIP call; see include/indexer.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/indexer.h"
#include "common.hpp"
#include "internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return IDX_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(IDX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxCols = 1 << 24;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Checks shared by the paged scorers.
int check_paged(const void* q, int q_dtype, const float* w, const uint8_t* keys, const uint8_t* scale,
                const float* gscale, const int32_t* bt, int64_t bt_stride, const int32_t* valid_lens, int T, int H,
                int D, int epb, int max_lb, int n_pages, int precision) {
  if (T < 0) return fail(IDX_ERR_SHAPE, "T = %d must be >= 0", T);
  if (!q || !w || !keys || !scale || !gscale || !bt || !valid_lens)
    return fail(IDX_ERR_NULL, "q, w, keys_fp4, key_scale, key_gscale, block_table and valid_lens are required");
  if (q_dtype != IDX_DTYPE_F32 && q_dtype != IDX_DTYPE_BF16) return fail(IDX_ERR_UNSUPPORTED, "q_dtype %d", q_dtype);
  if (precision != IDX_PREC_FP32 && precision != IDX_PREC_MFMA)
    return fail(IDX_ERR_UNSUPPORTED, "precision %d", precision);
  if (D != 64 && D != 128 && D != 256) return fail(IDX_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128, 256)", D);
  if (H < 1 || H > 64) return fail(IDX_ERR_UNSUPPORTED, "n_heads %d (supported: 1..64)", H);
  if (epb < 1 || epb > 65536) return fail(IDX_ERR_SHAPE, "entries_per_block %d (supported: 1..65536)", epb);
  if (max_lb < 1) return fail(IDX_ERR_SHAPE, "max_lb %d must be >= 1", max_lb);
  if (n_pages < 1) return fail(IDX_ERR_SHAPE, "n_pages %d must be >= 1", n_pages);
  if (bt_stride < max_lb) return fail(IDX_ERR_SHAPE, "bt_stride %lld < max_lb %d", (long long)bt_stride, max_lb);
  if ((int64_t)max_lb * epb >= kMaxCols)
    return fail(IDX_ERR_UNSUPPORTED, "max_lb * epb = %lld (supported: < 2^24)", (long long)max_lb * epb);
  if (!aligned(keys, 16)) return fail(IDX_ERR_SHAPE, "keys_fp4 must be 16-byte aligned");
  if (!aligned(scale, 4)) return fail(IDX_ERR_SHAPE, "key_scale must be 4-byte aligned");
  if (!aligned(q, q_dtype == IDX_DTYPE_F32 ? 4 : 2) || !aligned(w, 4) || !aligned(gscale, 4) || !aligned(bt, 4) ||
      !aligned(valid_lens, 4))
    return fail(IDX_ERR_SHAPE, "q, w, key_gscale, block_table and valid_lens must be naturally aligned");
  return IDX_OK;
}

salb::ScoreArgs make_args(const void* q, int q_dtype, const float* w, const uint8_t* keys, const uint8_t* scale,
                          const float* gscale, const int32_t* bt, int64_t bt_stride, const int32_t* valid_lens,
                          int T, int H, int D, int epb, int max_lb) {
  salb::ScoreArgs a{};
  a.q = q;
  a.q_bf16 = q_dtype == IDX_DTYPE_BF16;
  a.w = w;
  a.keys = keys;
  a.kscale = scale;
  a.gscale = gscale;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.valid_lens = valid_lens;
  a.T = T;
  a.H = H;
  a.D = D;
  a.epb = epb;
  a.max_lb = max_lb;
  a.epb_magic = salb::host_epb_magic(epb);
  return a;
}

// IDX_F_VALIDATE: the metadata check, run to completion before anything else is
// launched.  dev_status: 16 bytes of device memory the call may overwrite.
int validate_if_asked(unsigned flags, const int32_t* bt, int64_t bt_stride, const int32_t* valid_lens, int T,
                      int max_lb, int epb, int cap, int n_pages, void* dev_status, hipStream_t stream) {
  if (!(flags & IDX_F_VALIDATE)) return IDX_OK;
  int64_t st[2] = {-1, -1};
  hipError_t e = salb::validate_pages(bt, bt_stride, valid_lens, T, max_lb, epb, cap, n_pages,
                                      static_cast<int64_t*>(dev_status), st, stream);
  if (e != hipSuccess) return hip_fail(e, "validation");
  if (st[0] >= 0) return fail(IDX_ERR_DATA, "valid_lens[%lld] is outside [0, %d]", (long long)st[0], cap);
  if (st[1] >= 0)
    return fail(IDX_ERR_DATA, "block_table[%lld][%lld] names a page outside [0, %d)", (long long)(st[1] / max_lb),
                (long long)(st[1] % max_lb), n_pages);
  return IDX_OK;
}

int check_flags(unsigned flags) {
  if (flags & ~(unsigned)IDX_F_VALIDATE) return fail(IDX_ERR_UNSUPPORTED, "flags 0x%x", flags);
  return IDX_OK;
}

}  // namespace

// Workspace of indexer_score_topk_noalloc: one copy per GPU, held from the library's
// load until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns for the current device
// may be handed to kernels.
static __device__ __align__(256) unsigned char scratch[IDX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up once per device (with that
// device current) and kept; NULL with the HIP error in *err on failure.
void* scratch_on_current_device(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

const char* indexer_last_error(void) { return g_err.c_str(); }

int indexer_score_rows(const void* q, int q_dtype, const float* w, const uint8_t* keys_fp4,
                       const uint8_t* key_scale, const float* key_gscale, const int32_t* block_table,
                       int64_t bt_stride, const int32_t* valid_lens, int T, int H, int D, int epb, int max_lb,
                       int n_pages, int precision, unsigned flags, float* scores, int64_t score_stride,
                       int n_cols, hipStream_t stream) {
  int rc = check_paged(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride, valid_lens, T, H, D,
                       epb, max_lb, n_pages, precision);
  if (rc) return rc;
  if ((rc = check_flags(flags))) return rc;
  if (!scores) return fail(IDX_ERR_NULL, "scores is required");
  if (n_cols < 0 || n_cols >= kMaxCols) return fail(IDX_ERR_SHAPE, "n_cols %d out of range [0, 2^24)", n_cols);
  if (score_stride < n_cols) return fail(IDX_ERR_SHAPE, "score_stride < n_cols");
  if (!aligned(scores, 4)) return fail(IDX_ERR_SHAPE, "scores must be 4-byte aligned");
  if (T == 0 || n_cols == 0) return ok();
  if (flags & IDX_F_VALIDATE) {
    if (!aligned(scores, 8)) return fail(IDX_ERR_SHAPE, "IDX_F_VALIDATE needs 8-byte aligned scores");
    if ((int64_t)(T - 1) * score_stride + n_cols < 4)
      return fail(IDX_ERR_SHAPE, "IDX_F_VALIDATE needs a scores buffer of at least 4 floats");
    const int cap = (int64_t)max_lb * epb < n_cols ? max_lb * epb : n_cols;
    if ((rc = validate_if_asked(flags, block_table, bt_stride, valid_lens, T, max_lb, epb, cap, n_pages, scores,
                                stream)))
      return rc;
  }
  salb::ScoreArgs a = make_args(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride, valid_lens,
                                T, H, D, epb, max_lb);
  a.scores = scores;
  a.score_stride = score_stride;
  a.n_cols = n_cols;
  a.write_tail = 1;
  hipError_t e = salb::launch_score_rows(a, precision, stream);
  if (e != hipSuccess) return hip_fail(e, "score kernel launch");
  return ok();
}

size_t indexer_topk_workspace_size(int rows, int n_cols, int top_k) {
  if (rows <= 0 || n_cols <= 0 || top_k <= 0 || n_cols >= kMaxCols) return 0;
  return salb::select_workspace_bytes(rows, n_cols, top_k);
}

static int check_select(int rows, int n_cols, int top_k, int64_t score_stride, int ratio) {
  if (rows < 0) return fail(IDX_ERR_SHAPE, "rows %d must be >= 0", rows);
  if (n_cols < 0 || n_cols >= kMaxCols) return fail(IDX_ERR_SHAPE, "n_cols %d out of range [0, 2^24)", n_cols);
  if (top_k < 1 || top_k > salb::kMaxTopK)
    return fail(IDX_ERR_UNSUPPORTED, "top_k %d (supported: 1..%d)", top_k, salb::kMaxTopK);
  if (score_stride < n_cols) return fail(IDX_ERR_SHAPE, "score_stride < n_cols");
  if (ratio < 0) return fail(IDX_ERR_SHAPE, "ratio %d must be >= 0", ratio);
  return IDX_OK;
}

int indexer_topk_select(const float* scores, int64_t score_stride, const int32_t* valid_lens, int64_t first_pos,
                        int ratio, int rows, int n_cols, int top_k, int32_t* topk_idx, float* topk_scores,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_select(rows, n_cols, top_k, score_stride, ratio);
  if (rc) return rc;
  if (!topk_idx) return fail(IDX_ERR_NULL, "topk_idx is required");
  if (rows == 0) return ok();
  if (!scores && n_cols > 0) return fail(IDX_ERR_NULL, "scores is required");
  salb::SelectPlan p;
  if (!salb::plan_select(rows, n_cols > 0 ? n_cols : 1, top_k, &p))
    return fail(IDX_ERR_UNSUPPORTED, "top_k %d is not supported", top_k);
  if (p.bytes > 0 && (!workspace || workspace_bytes < p.bytes))
    return fail(IDX_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", p.bytes, workspace_bytes);
  if (workspace && !aligned(workspace, 256)) return fail(IDX_ERR_SHAPE, "workspace must be 256-byte aligned");
  if (n_cols == 0) {
    // no candidates: every slot is padding
    p.n_cols = 0;
  }
  hipError_t e = salb::launch_select(p, scores, score_stride, valid_lens, first_pos, ratio, topk_idx, topk_scores,
                                     workspace, false, stream);
  if (e != hipSuccess) return hip_fail(e, "select kernel launch");
  return ok();
}

size_t indexer_score_topk_workspace_size(int T, int max_lb, int epb, int top_k) {
  if (T <= 0 || max_lb <= 0 || epb <= 0 || top_k <= 0) return 0;
  const int64_t n_cols = (int64_t)max_lb * epb;
  if (n_cols >= kMaxCols) return 0;
  const size_t stride = round_up((size_t)n_cols, 64);
  const size_t scores = round_up((size_t)T * stride * 4, 256);
  return scores + salb::select_workspace_bytes(T, (int)n_cols, top_k);
}

int indexer_score_topk(const void* q, int q_dtype, const float* w, const uint8_t* keys_fp4,
                       const uint8_t* key_scale, const float* key_gscale, const int32_t* block_table,
                       int64_t bt_stride, const int32_t* valid_lens, int T, int H, int D, int epb, int max_lb,
                       int n_pages, int top_k, int precision, unsigned flags, int32_t* topk_idx,
                       float* topk_scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_paged(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride, valid_lens, T, H, D,
                       epb, max_lb, n_pages, precision);
  if (rc) return rc;
  if ((rc = check_flags(flags))) return rc;
  const int n_cols = max_lb * epb;
  rc = check_select(T, n_cols, top_k, n_cols, 0);
  if (rc) return rc;
  if (!topk_idx) return fail(IDX_ERR_NULL, "topk_idx is required");
  if (T == 0) return ok();
  salb::SelectPlan p;
  if (!salb::plan_select(T, n_cols, top_k, &p))
    return fail(IDX_ERR_UNSUPPORTED, "top_k %d is not supported", top_k);
  const size_t stride = round_up((size_t)n_cols, 64);
  const size_t score_bytes = round_up((size_t)T * stride * 4, 256);
  const size_t need = score_bytes + p.bytes;
  if (!workspace || workspace_bytes < need)
    return fail(IDX_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(IDX_ERR_SHAPE, "workspace must be 256-byte aligned");
  if ((rc = validate_if_asked(flags, block_table, bt_stride, valid_lens, T, max_lb, epb, n_cols, n_pages, workspace,
                              stream)))
    return rc;
  float* sc = static_cast<float*>(workspace);
  salb::ScoreArgs a = make_args(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride, valid_lens,
                                T, H, D, epb, max_lb);
  a.scores = sc;
  a.score_stride = (int64_t)stride;
  a.n_cols = n_cols;
  a.write_tail = 0;
  // the scorer launch also zeroes the select's histogram counters (no clearing launch)
  unsigned char* sel_ws = static_cast<unsigned char*>(workspace) + score_bytes;
  a.zero_ptr = reinterpret_cast<uint4*>(sel_ws);
  a.zero_n16 = (int64_t)(salb::select_counter_bytes(p) / 16);
  hipError_t e = salb::launch_score_rows(a, precision, stream);
  if (e != hipSuccess) return hip_fail(e, "score kernel launch");
  e = salb::launch_select(p, sc, (int64_t)stride, valid_lens, 0, 0, topk_idx, topk_scores, sel_ws, true, stream);
  if (e != hipSuccess) return hip_fail(e, "select kernel launch");
  return ok();
}

int indexer_score_topk_noalloc(const void* q, int q_dtype, const float* w, const uint8_t* keys_fp4,
                               const uint8_t* key_scale, const float* key_gscale, const int32_t* block_table,
                               int64_t bt_stride, const int32_t* valid_lens, int T, int H, int D, int epb,
                               int max_lb, int n_pages, int top_k, int precision, unsigned flags,
                               int32_t* topk_idx, float* topk_scores, hipStream_t stream) {
  // the size rule first, on the host: no HIP call for a call that cannot fit
  if (T > 0 && max_lb > 0 && epb > 0 && top_k > 0) {
    const size_t need = indexer_score_topk_workspace_size(T, max_lb, epb, top_k);
    if (need > (size_t)IDX_NOALLOC_SCRATCH_BYTES)
      return fail(IDX_ERR_WORKSPACE, "the call needs %zu bytes of scratch; the no-alloc entry holds %llu", need,
                  (unsigned long long)IDX_NOALLOC_SCRATCH_BYTES);
  }
  int rc = check_paged(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride, valid_lens, T, H, D,
                       epb, max_lb, n_pages, precision);
  if (rc) return rc;
  if (T == 0) return indexer_score_topk(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride,
                                        valid_lens, T, H, D, epb, max_lb, n_pages, top_k, precision, flags, topk_idx,
                                        topk_scores, nullptr, 0, stream);
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (!ws) return hip_fail(e, "no-alloc scratch address");
  return indexer_score_topk(q, q_dtype, w, keys_fp4, key_scale, key_gscale, block_table, bt_stride, valid_lens, T, H,
                            D, epb, max_lb, n_pages, top_k, precision, flags, topk_idx, topk_scores, ws,
                            (size_t)IDX_NOALLOC_SCRATCH_BYTES, stream);
}

int indexer_gather_kv(const uint8_t* kv_fp8, const float* kv_scale, const uint16_t* kv_rope,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* topk_idx, int T, int top_k,
                      int epb, int max_lb, int n_pages, int d_nope, int d_rope, int group, uint16_t* out,
                      hipStream_t stream) {
  if (T < 0 || top_k < 1) return fail(IDX_ERR_SHAPE, "T = %d, top_k = %d: need T >= 0 and top_k >= 1", T, top_k);
  if (!block_table || !topk_idx || !out || (d_nope > 0 && (!kv_fp8 || !kv_scale)) || (d_rope > 0 && !kv_rope))
    return fail(IDX_ERR_NULL, "block_table, topk_idx, out and the pool arrays of nonzero width are required");
  if (epb < 1 || epb > 65536) return fail(IDX_ERR_SHAPE, "entries_per_block %d (supported: 1..65536)", epb);
  if (max_lb < 1 || n_pages < 1) return fail(IDX_ERR_SHAPE, "max_lb and n_pages must be >= 1");
  if (bt_stride < max_lb) return fail(IDX_ERR_SHAPE, "bt_stride %lld < max_lb %d", (long long)bt_stride, max_lb);
  if ((int64_t)max_lb * epb >= kMaxCols)
    return fail(IDX_ERR_UNSUPPORTED, "max_lb * epb = %lld (supported: < 2^24)", (long long)max_lb * epb);
  if (d_nope < 0 || d_nope % 16 || d_rope < 0 || d_rope % 8 || d_nope + d_rope < 8)
    return fail(IDX_ERR_UNSUPPORTED, "d_nope %d must be a multiple of 16 and d_rope %d of 8 (sum >= 8)", d_nope,
                d_rope);
  if (d_nope > 0 && (group < 16 || group % 16 || d_nope % group))
    return fail(IDX_ERR_UNSUPPORTED, "group %d must be a multiple of 16 dividing d_nope %d", group, d_nope);
  if (!aligned(kv_fp8, 16) || !aligned(kv_rope, 16) || !aligned(out, 16) || !aligned(kv_scale, 4) ||
      !aligned(block_table, 4) || !aligned(topk_idx, 4))
    return fail(IDX_ERR_SHAPE, "kv_fp8, kv_rope and out must be 16-byte aligned");
  if (T == 0) return ok();
  hipError_t e = salb::launch_gather_kv(kv_fp8, kv_scale, kv_rope, block_table, bt_stride, topk_idx, T, top_k, epb,
                                        max_lb, d_nope, d_rope, group, out, stream);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

int qsa_gather(const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* block_table, const int32_t* sel,
               uint16_t* k_out, uint16_t* v_out, uint32_t n_sel, uint32_t block_size, uint32_t nkv, uint32_t hd,
               hipStream_t stream) {
  if (!k_cache || !v_cache || !block_table || !sel || !k_out || !v_out)
    return fail(IDX_ERR_NULL, "k_cache, v_cache, block_table, sel, k_out and v_out are required");
  if (block_size < 1) return fail(IDX_ERR_SHAPE, "block_size must be >= 1");
  if (nkv < 1 || hd < 1 || ((uint64_t)nkv * hd) % 8 || (uint64_t)nkv * hd > (1u << 20))
    return fail(IDX_ERR_UNSUPPORTED, "nkv * hd = %llu must be a multiple of 8 (at most 2^20)",
                (unsigned long long)nkv * hd);
  if (n_sel > 0x7fffffffu) return fail(IDX_ERR_SHAPE, "n_sel too large");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) ||
      !aligned(block_table, 4) || !aligned(sel, 4))
    return fail(IDX_ERR_SHAPE, "caches and outputs must be 16-byte aligned");
  if (n_sel == 0) return ok();
  hipError_t e = salb::launch_qsa_gather(k_cache, v_cache, block_table, sel, k_out, v_out, (int)n_sel,
                                         (int)block_size, (int)nkv, (int)hd, stream);
  if (e != hipSuccess) return hip_fail(e, "QSA gather launch");
  return ok();
}

int qsa_prefill_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* block_table,
                     const int32_t* lists, float* attn_out, uint32_t rows, uint32_t first_pos, uint32_t topk,
                     uint32_t ratio, uint32_t block_size, uint32_t nq, uint32_t nkv, uint32_t hd, float inv_sqrt_d,
                     hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !attn_out || (topk > 0 && !lists))
    return fail(IDX_ERR_NULL, "q, k_cache, v_cache, block_table, attn_out and (for topk > 0) lists are required");
  if (hd != 64 && hd != 128) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128)", hd);
  if (nkv < 1 || nq < nkv || nq % nkv || nq / nkv > 16)
    return fail(IDX_ERR_UNSUPPORTED, "nq %u / nkv %u: nkv must divide nq with at most 16 query heads per KV head", nq,
                nkv);
  if (ratio < 1 || block_size < 1) return fail(IDX_ERR_SHAPE, "ratio and block_size must be >= 1");
  if (topk > 65536 || (uint64_t)topk * ratio + ratio > (1u << 24))
    return fail(IDX_ERR_UNSUPPORTED, "topk %u * ratio %u too large", topk, ratio);
  if ((uint64_t)rows * nkv > 0x7fffffffull || (uint64_t)first_pos + rows > 0x7fffffffull)
    return fail(IDX_ERR_SHAPE, "rows / positions out of range");
  const size_t lds = salb::prefill_attn_lds_bytes((int)topk, (int)ratio, (int)hd);
  if (lds > 160 * 1024 - 2048)
    return fail(IDX_ERR_UNSUPPORTED, "topk %u * ratio %u positions do not fit the workgroup's LDS", topk, ratio);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(attn_out, 4) ||
      !aligned(block_table, 4) || !aligned(lists, 4))
    return fail(IDX_ERR_SHAPE, "q and the caches must be 16-byte aligned");
  if (rows == 0) return ok();
  hipError_t e = salb::launch_prefill_attn(q, k_cache, v_cache, block_table, lists, attn_out, (int)rows, first_pos,
                                           (int)topk, (int)ratio, (int)block_size, (int)nq, (int)nkv, (int)hd,
                                           inv_sqrt_d, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return ok();
}

extern "C++" {
static int block_pool_check(const uint16_t* raw_keys, const float* k_norm_w, const void* block_keys,
                            uint32_t first_block, uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot) {
  if (!raw_keys || !k_norm_w || !block_keys) return fail(IDX_ERR_NULL, "raw_keys, k_norm_w and block_keys are required");
  if (hd != 64 && hd != 128 && hd != 256) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128, 256)", hd);
  if (rot > hd || (rot & 1)) return fail(IDX_ERR_SHAPE, "rot %u must be even and <= hd", rot);
  if (ratio < 1) return fail(IDX_ERR_SHAPE, "ratio must be >= 1");
  if ((uint64_t)first_block + n_new > 0x7fffffffull) return fail(IDX_ERR_SHAPE, "block range too large");
  if (!aligned(raw_keys, 16) || !aligned(block_keys, 16) || !aligned(k_norm_w, 4))
    return fail(IDX_ERR_SHAPE, "raw_keys and block_keys must be 16-byte aligned");
  return IDX_OK;
}

// Workgroups per query row at the smallest slice the query prep launches (128 chunks of
// 8 dims): bounds the launch grid.
static uint64_t qprep_slices(uint32_t n_heads, uint32_t hd) { return ((uint64_t)n_heads * hd / 8 + 127) / 128; }

static int qprep_check(const uint16_t* qk, const float* q_norm_w, const void* q_out, uint32_t qkw, uint32_t n_heads,
                       uint32_t hd, uint32_t rot) {
  if (!qk || !q_norm_w || !q_out) return fail(IDX_ERR_NULL, "qk, q_norm_w and q_out are required");
  if (hd != 64 && hd != 128 && hd != 256) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128, 256)", hd);
  if (rot > hd || (rot & 1)) return fail(IDX_ERR_SHAPE, "rot %u must be even and <= hd", rot);
  if (n_heads < 1 || n_heads > 65535) return fail(IDX_ERR_SHAPE, "n_heads %u out of range", n_heads);
  if ((uint64_t)n_heads * hd > qkw) return fail(IDX_ERR_SHAPE, "qkw %u < n_heads * hd", qkw);
  if ((uint64_t)n_heads * hd > 32768)
    return fail(IDX_ERR_UNSUPPORTED, "n_heads * hd = %llu (supported: <= 32768)", (unsigned long long)n_heads * hd);
  if (qkw % 8 != 0 || !aligned(qk, 16) || !aligned(q_out, 16) || !aligned(q_norm_w, 4))
    return fail(IDX_ERR_SHAPE, "qk and q_out must be 16-byte aligned and qkw a multiple of 8");
  return IDX_OK;
}

template <typename OutT>
static int block_pool_impl(const uint16_t* raw_keys, const float* k_norm_w, OutT* block_keys, uint32_t first_block,
                           uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot, float theta, float eps,
                           hipStream_t stream) {
  int rc;
  if ((rc = block_pool_check(raw_keys, k_norm_w, block_keys, first_block, n_new, ratio, hd, rot)) != IDX_OK) return rc;
  if (n_new == 0) return ok();
  hipError_t e = salb::launch_block_pool<OutT>(raw_keys, k_norm_w, block_keys, first_block, n_new, ratio, hd, rot,
                                               theta, eps, stream);
  if (e != hipSuccess) return hip_fail(e, "block pool launch");
  return ok();
}
}  // extern "C++"

int qsa_block_pool(const uint16_t* raw_keys, const float* k_norm_w, float* block_keys, uint32_t first_block,
                   uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot, float theta, float eps,
                   hipStream_t stream) {
  return block_pool_impl<float>(raw_keys, k_norm_w, block_keys, first_block, n_new, ratio, hd, rot, theta, eps,
                                stream);
}

int qsa_block_pool_f16(const uint16_t* raw_keys, const float* k_norm_w, uint16_t* block_keys, uint32_t first_block,
                       uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot, float theta, float eps,
                       hipStream_t stream) {
  return block_pool_impl<_Float16>(raw_keys, k_norm_w, reinterpret_cast<_Float16*>(block_keys), first_block, n_new,
                                   ratio, hd, rot, theta, eps, stream);
}

extern "C++" {
template <typename OutT>
static int qprep_rows_impl(const uint16_t* qk, const float* q_norm_w, OutT* q_out, uint32_t rows, uint32_t first_pos,
                           uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot, float theta, float eps,
                           hipStream_t stream) {
  int rc;
  if ((rc = qprep_check(qk, q_norm_w, q_out, qkw, n_heads, hd, rot)) != IDX_OK) return rc;
  if ((uint64_t)rows * qprep_slices(n_heads, hd) > 0x7fffffffull)
    return fail(IDX_ERR_SHAPE, "rows %u too large", rows);
  if (rows == 0) return ok();
  hipError_t e = salb::launch_qprep_rows<OutT>(qk, q_norm_w, q_out, rows, first_pos, qkw, n_heads, hd, rot, theta,
                                               eps, stream);
  if (e != hipSuccess) return hip_fail(e, "query prep launch");
  return ok();
}
}  // extern "C++"

int qsa_qprep_rows(const uint16_t* qk, const float* q_norm_w, float* q_out, uint32_t rows, uint32_t first_pos,
                   uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot, float theta, float eps,
                   hipStream_t stream) {
  return qprep_rows_impl<float>(qk, q_norm_w, q_out, rows, first_pos, qkw, n_heads, hd, rot, theta, eps, stream);
}

int qsa_qprep_rows_f16(const uint16_t* qk, const float* q_norm_w, uint16_t* q_out, uint32_t rows, uint32_t first_pos,
                       uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot, float theta, float eps,
                       hipStream_t stream) {
  return qprep_rows_impl<_Float16>(qk, q_norm_w, reinterpret_cast<_Float16*>(q_out), rows, first_pos, qkw, n_heads,
                                   hd, rot, theta, eps, stream);
}

int qsa_decode_prep(const uint16_t* raw_keys, const float* k_norm_w, float* block_keys, uint32_t first_block,
                    uint32_t n_new, uint32_t ratio, const uint16_t* qk, const float* q_norm_w, float* q_out,
                    uint32_t rows, uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot,
                    float theta, float eps, hipStream_t stream) {
  int rc;
  if ((rc = block_pool_check(raw_keys, k_norm_w, block_keys, first_block, n_new, ratio, hd, rot)) != IDX_OK) return rc;
  if ((rc = qprep_check(qk, q_norm_w, q_out, qkw, n_heads, hd, rot)) != IDX_OK) return rc;
  if ((uint64_t)rows * qprep_slices(n_heads, hd) + (n_new + 7) / 8 > 0x7fffffffull)
    return fail(IDX_ERR_SHAPE, "rows %u too large", rows);
  if (n_new == 0 && rows == 0) return ok();
  hipError_t e = salb::launch_decode_prep(raw_keys, k_norm_w, block_keys, first_block, n_new, ratio, qk, q_norm_w,
                                          q_out, rows, first_pos, qkw, n_heads, hd, rot, theta, eps, stream);
  if (e != hipSuccess) return hip_fail(e, "decode prep launch");
  return ok();
}

int qsa_qprep(const uint16_t* q_in, const float* q_norm_w, float* q_out, uint32_t n_heads, uint32_t hd,
              uint32_t rot, uint32_t pos, float theta, float eps, hipStream_t stream) {
  if (!q_in || !q_norm_w || !q_out) return fail(IDX_ERR_NULL, "q_in, q_norm_w and q_out are required");
  if (n_heads < 1 || n_heads > 65535) return fail(IDX_ERR_SHAPE, "n_heads %u out of range", n_heads);
  if (hd != 64 && hd != 128 && hd != 256) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128, 256)", hd);
  // one row of qsa_qprep_rows at position pos, read from a projection row of n_heads * hd
  return qsa_qprep_rows(q_in, q_norm_w, q_out, 1, pos, n_heads * hd, n_heads, hd, rot, theta, eps, stream);
}

int qsa_score(const float* q, const float* block_keys, float* scores, uint32_t n_blocks, uint32_t n_heads,
              uint32_t hd, hipStream_t stream) {
  if (!q || !block_keys || (!scores && n_blocks > 0))
    return fail(IDX_ERR_NULL, "q, block_keys and (for n_blocks > 0) scores are required");
  if (hd != 64 && hd != 128 && hd != 256) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128, 256)", hd);
  if (n_heads < 1 || n_heads > 64) return fail(IDX_ERR_UNSUPPORTED, "n_heads %u (supported: 1..64)", n_heads);
  if (n_blocks > 0x7fffffffu) return fail(IDX_ERR_SHAPE, "n_blocks too large");
  if (!aligned(q, 16) || !aligned(block_keys, 16) || !aligned(scores, 4))
    return fail(IDX_ERR_SHAPE, "q and block_keys must be 16-byte aligned");
  if (n_blocks == 0) return ok();
  hipError_t e = salb::launch_qsa_decode_score(q, block_keys, scores, n_blocks, n_heads, hd, nullptr, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "QSA decode score launch");
  return ok();
}

// qsa_score_topk's workspace: the scores then the general select's buffers, or (on the
// matrix-core scorer, when the sub-tile select takes the shape) the scores padded to whole
// 16-block sub-tiles then the sub-tile maxima.  The size covers both.
static size_t decode_tiles_bytes(uint32_t n_blocks) {
  return round_up((size_t)((n_blocks + 15) & ~15u) * 4, 256) + round_up((size_t)((n_blocks + 15) / 16) * 4, 256);
}

size_t qsa_score_topk_workspace_size(uint32_t n_blocks, int top_k) {
  if (n_blocks == 0 || n_blocks > 0x7fffffffu || top_k <= 0) return 0;
  salb::SelectPlan p;
  if (!salb::plan_select(1, (int)n_blocks, top_k, &p)) return 0;
  const size_t rows_path = round_up((size_t)n_blocks * 4, 256) + p.bytes;
  const size_t tiles_path = salb::tile_select_fits((int)n_blocks, top_k) ? decode_tiles_bytes(n_blocks) : 0;
  return rows_path > tiles_path ? rows_path : tiles_path;
}

int qsa_score_topk(const float* q, const float* block_keys, uint32_t n_blocks, uint32_t n_heads, uint32_t hd,
                   int top_k, int32_t* topk_idx, float* topk_scores, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  if (!q || !block_keys || !topk_idx) return fail(IDX_ERR_NULL, "q, block_keys and topk_idx are required");
  if (hd != 64 && hd != 128 && hd != 256) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128, 256)", hd);
  if (n_heads < 1 || n_heads > 64) return fail(IDX_ERR_UNSUPPORTED, "n_heads %u (supported: 1..64)", n_heads);
  if (n_blocks > 0x7fffffffu || (int64_t)n_blocks >= kMaxCols)
    return fail(IDX_ERR_UNSUPPORTED, "n_blocks %u (supported: < 2^24)", n_blocks);
  if (!aligned(q, 16) || !aligned(block_keys, 16)) return fail(IDX_ERR_SHAPE, "q and block_keys must be 16-byte aligned");
  int rc = check_select(1, (int)n_blocks, top_k, (int64_t)n_blocks, 0);
  if (rc) return rc;
  if (n_blocks == 0) {  // no block: every slot is padding (the select alone writes it)
    return indexer_topk_select(nullptr, 0, nullptr, 0, 0, 1, 0, top_k, topk_idx, topk_scores, workspace,
                               workspace_bytes, stream);
  }
  if (salb::qsa_decode_uses_mfma(n_heads, hd) && salb::tile_select_fits((int)n_blocks, top_k)) {
    // the scorer records the 16-block sub-tile maxima; the sub-tile select reads only the
    // sub-tiles that can hold a winner (one launch for the select, no counters to clear)
    const size_t need = decode_tiles_bytes(n_blocks);
    if (!workspace || workspace_bytes < need)
      return fail(IDX_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace_bytes);
    if (!aligned(workspace, 256)) return fail(IDX_ERR_SHAPE, "workspace must be 256-byte aligned");
    const uint32_t s16 = (n_blocks + 15) & ~15u;
    float* sc = static_cast<float*>(workspace);
    uint32_t* tm = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) + round_up((size_t)s16 * 4, 256));
    hipError_t e = salb::launch_qsa_decode_score(q, block_keys, sc, n_blocks, n_heads, hd, nullptr, 0, stream, tm);
    if (e != hipSuccess) return hip_fail(e, "QSA decode score launch");
    e = salb::launch_select_tiles(sc, s16, tm, s16 / 16, 0, 0, 1, (int)n_blocks, top_k, topk_idx, topk_scores, stream);
    if (e != hipSuccess) return hip_fail(e, "select kernel launch");
    return ok();
  }
  salb::SelectPlan p;
  if (!salb::plan_select(1, (int)n_blocks, top_k, &p)) return fail(IDX_ERR_UNSUPPORTED, "top_k %d is not supported", top_k);
  const size_t score_bytes = round_up((size_t)n_blocks * 4, 256);
  const size_t need = score_bytes + p.bytes;
  if (!workspace || workspace_bytes < need)
    return fail(IDX_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(IDX_ERR_SHAPE, "workspace must be 256-byte aligned");
  float* sc = static_cast<float*>(workspace);
  unsigned char* sel_ws = static_cast<unsigned char*>(workspace) + score_bytes;
  // the score launch also zeroes the select's counters (no clearing launch)
  hipError_t e = salb::launch_qsa_decode_score(q, block_keys, sc, n_blocks, n_heads, hd, reinterpret_cast<uint4*>(sel_ws),
                                               (int64_t)(salb::select_counter_bytes(p) / 16), stream);
  if (e != hipSuccess) return hip_fail(e, "QSA decode score launch");
  e = salb::launch_select(p, sc, (int64_t)n_blocks, nullptr, 0, 0, topk_idx, topk_scores, sel_ws, true, stream);
  if (e != hipSuccess) return hip_fail(e, "select kernel launch");
  return ok();
}

int qsa_score_rows(const float* q, const float* block_keys, float* scores, uint32_t rows, uint32_t n_blocks_max,
                   uint32_t first_pos, uint32_t score_stride, uint32_t ratio, uint32_t n_heads, uint32_t hd,
                   int precision, hipStream_t stream) {
  if (!q || !block_keys || !scores) return fail(IDX_ERR_NULL, "q, block_keys and scores are required");
  if (hd != 64 && hd != 128 && hd != 256) return fail(IDX_ERR_UNSUPPORTED, "hd %u (supported: 64, 128, 256)", hd);
  if (n_heads < 1 || n_heads > 64) return fail(IDX_ERR_UNSUPPORTED, "n_heads %u (supported: 1..64)", n_heads);
  if (ratio < 1) return fail(IDX_ERR_SHAPE, "ratio must be >= 1");
  if (score_stride < n_blocks_max) return fail(IDX_ERR_SHAPE, "score_stride < n_blocks_max");
  if (n_blocks_max >= (uint32_t)kMaxCols) return fail(IDX_ERR_UNSUPPORTED, "n_blocks_max must be < 2^24");
  if (precision != IDX_PREC_FP32 && precision != IDX_PREC_MFMA)
    return fail(IDX_ERR_UNSUPPORTED, "precision %d", precision);
  if (!aligned(q, 16) || !aligned(block_keys, 16) || !aligned(scores, 4))
    return fail(IDX_ERR_SHAPE, "q and block_keys must be 16-byte aligned");
  if (rows == 0 || n_blocks_max == 0) return ok();
  hipError_t e = salb::launch_qsa_score(q, block_keys, scores, rows, n_blocks_max, first_pos, score_stride, ratio,
                                        n_heads, hd, precision, stream);
  if (e != hipSuccess) return hip_fail(e, "QSA score launch");
  return ok();
}

int qsa_score_rows_f16(const uint16_t* q, const uint16_t* block_keys, float* scores, uint32_t rows,
                       uint32_t n_blocks_max, uint32_t first_pos, uint32_t score_stride, uint32_t ratio,
                       uint32_t n_heads, uint32_t hd, hipStream_t stream) {
  if (!q || !block_keys || !scores) return fail(IDX_ERR_NULL, "q, block_keys and scores are required");
  if (hd != 64 && hd != 128) return fail(IDX_ERR_UNSUPPORTED, "hd %u (fp16 inputs: 64 or 128)", hd);
  if (n_heads != 16 && n_heads != 32 && n_heads != 64)
    return fail(IDX_ERR_UNSUPPORTED, "n_heads %u (fp16 inputs: 16, 32 or 64)", n_heads);
  if (ratio < 1) return fail(IDX_ERR_SHAPE, "ratio must be >= 1");
  if (score_stride < n_blocks_max) return fail(IDX_ERR_SHAPE, "score_stride < n_blocks_max");
  if (n_blocks_max >= (uint32_t)kMaxCols) return fail(IDX_ERR_UNSUPPORTED, "n_blocks_max must be < 2^24");
  if (!aligned(q, 16) || !aligned(block_keys, 16) || !aligned(scores, 4))
    return fail(IDX_ERR_SHAPE, "q and block_keys must be 16-byte aligned");
  if (rows == 0 || n_blocks_max == 0) return ok();
  hipError_t e = salb::launch_qsa_score_f16(reinterpret_cast<const _Float16*>(q),
                                            reinterpret_cast<const _Float16*>(block_keys), scores, rows, n_blocks_max,
                                            first_pos, score_stride, ratio, n_heads, hd, stream);
  if (e != hipSuccess) return hip_fail(e, "QSA score launch");
  return ok();
}

static int score_f16_check(const uint16_t* q, const uint16_t* block_keys, const float* scores, uint32_t n_heads,
                           uint32_t hd, uint32_t ratio) {
  if (!q || !block_keys || !scores) return fail(IDX_ERR_NULL, "q, block_keys and scores are required");
  if (hd != 64 && hd != 128) return fail(IDX_ERR_UNSUPPORTED, "hd %u (fp16 inputs: 64 or 128)", hd);
  if (n_heads != 16 && n_heads != 32 && n_heads != 64)
    return fail(IDX_ERR_UNSUPPORTED, "n_heads %u (fp16 inputs: 16, 32 or 64)", n_heads);
  if (ratio < 1 || ratio > 0x7fffffffu) return fail(IDX_ERR_SHAPE, "ratio must be >= 1");
  if (!aligned(q, 16) || !aligned(block_keys, 16)) return fail(IDX_ERR_SHAPE, "q and block_keys must be 16-byte aligned");
  return IDX_OK;
}

int qsa_score_rows_f16_tmax(const uint16_t* q, const uint16_t* block_keys, float* scores, uint32_t* tile_max,
                            uint32_t rows, uint32_t n_blocks_max, uint32_t first_pos, uint32_t score_stride,
                            uint32_t tile_stride, uint32_t ratio, uint32_t n_heads, uint32_t hd, hipStream_t stream) {
  int rc = score_f16_check(q, block_keys, scores, n_heads, hd, ratio);
  if (rc) return rc;
  if (!tile_max) return fail(IDX_ERR_NULL, "tile_max is required");
  if (score_stride < n_blocks_max) return fail(IDX_ERR_SHAPE, "score_stride < n_blocks_max");
  if (tile_stride < (n_blocks_max + 15) / 16) return fail(IDX_ERR_SHAPE, "tile_stride < ceil(n_blocks_max / 16)");
  if (n_blocks_max >= (uint32_t)kMaxCols) return fail(IDX_ERR_UNSUPPORTED, "n_blocks_max must be < 2^24");
  if (!aligned(scores, 4) || !aligned(tile_max, 4)) return fail(IDX_ERR_SHAPE, "scores and tile_max must be 4-byte aligned");
  if (rows == 0 || n_blocks_max == 0) return ok();
  hipError_t e = salb::launch_qsa_score_f16(reinterpret_cast<const _Float16*>(q),
                                            reinterpret_cast<const _Float16*>(block_keys), scores, rows, n_blocks_max,
                                            first_pos, score_stride, ratio, n_heads, hd, stream, tile_max, tile_stride);
  if (e != hipSuccess) return hip_fail(e, "QSA score launch");
  return ok();
}

int qsa_select_tiles(const float* scores, int64_t score_stride, const uint32_t* tile_max, int64_t tile_stride,
                     int64_t first_pos, int ratio, int rows, int n_cols, int top_k, int32_t* topk_idx,
                     float* topk_scores, hipStream_t stream) {
  int rc = check_select(rows, n_cols, top_k, score_stride, ratio);
  if (rc) return rc;
  if (!topk_idx) return fail(IDX_ERR_NULL, "topk_idx is required");
  if (ratio < 1) return fail(IDX_ERR_SHAPE, "ratio must be >= 1 (the causal valid count)");
  if (rows == 0) return ok();
  if (!scores || !tile_max) return fail(IDX_ERR_NULL, "scores and tile_max are required");
  if (!salb::tile_select_fits(n_cols, top_k))
    return fail(IDX_ERR_UNSUPPORTED, "n_cols %d / top_k %d (supported: 1..32768 / 1..512)", n_cols, top_k);
  if (score_stride % 4 != 0 || score_stride < (int64_t)((n_cols + 15) & ~15) || !aligned(scores, 16))
    return fail(IDX_ERR_SHAPE, "scores must be 16-byte aligned, score_stride a multiple of 4 and >= n_cols rounded up to 16");
  if (tile_stride < (n_cols + 15) / 16 || !aligned(tile_max, 4)) return fail(IDX_ERR_SHAPE, "tile_stride < ceil(n_cols / 16)");
  hipError_t e = salb::launch_select_tiles(scores, score_stride, tile_max, tile_stride, first_pos, ratio, rows, n_cols,
                                           top_k, topk_idx, topk_scores, stream);
  if (e != hipSuccess) return hip_fail(e, "select kernel launch");
  return ok();
}

// Workspace of qsa_score_select_f16: the scores (row stride n_blocks rounded up to 16),
// then either the sub-tile maxima (the sub-tile select) or the general select's buffers.
struct ScoreSelectLayout {
  uint32_t sstride, tstride;
  size_t scores, tmax, select, total;
  bool tiles;
};

static bool score_select_layout(uint32_t rows, uint32_t n_blocks, int top_k, ScoreSelectLayout* l) {
  l->sstride = (n_blocks + 15u) & ~15u;
  l->tstride = l->sstride / 16;
  l->tiles = salb::tile_select_fits((int)n_blocks, top_k);
  l->scores = 0;
  l->tmax = round_up((size_t)rows * l->sstride * 4, 256);
  if (l->tiles) {
    l->select = l->tmax;
    l->total = l->tmax + round_up((size_t)rows * l->tstride * 4, 256);
    return true;
  }
  salb::SelectPlan p;
  if (!salb::plan_select((int)rows, (int)n_blocks, top_k, &p)) return false;
  l->select = l->tmax;
  l->total = l->tmax + p.bytes;
  return true;
}

size_t qsa_score_select_f16_workspace_size(uint32_t rows, uint32_t n_blocks, int top_k) {
  if (rows == 0 || n_blocks == 0 || (int64_t)n_blocks >= kMaxCols || rows > 0x7fffffffu || top_k <= 0) return 0;
  ScoreSelectLayout l;
  if (!score_select_layout(rows, n_blocks, top_k, &l)) return 0;
  return l.total;
}

int qsa_score_select_f16(const uint16_t* q, const uint16_t* block_keys, uint32_t rows, uint32_t n_blocks,
                         uint32_t first_pos, uint32_t ratio, uint32_t n_heads, uint32_t hd, int top_k,
                         int32_t* topk_idx, float* topk_scores, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!q || !block_keys || !topk_idx) return fail(IDX_ERR_NULL, "q, block_keys and topk_idx are required");
  if (hd != 64 && hd != 128) return fail(IDX_ERR_UNSUPPORTED, "hd %u (fp16 inputs: 64 or 128)", hd);
  if (n_heads != 16 && n_heads != 32 && n_heads != 64)
    return fail(IDX_ERR_UNSUPPORTED, "n_heads %u (fp16 inputs: 16, 32 or 64)", n_heads);
  if (ratio < 1 || ratio > 0x7fffffffu) return fail(IDX_ERR_SHAPE, "ratio must be >= 1");
  if (rows > 0x7fffffffu) return fail(IDX_ERR_SHAPE, "rows %u out of range", rows);
  if ((int64_t)n_blocks >= kMaxCols) return fail(IDX_ERR_UNSUPPORTED, "n_blocks must be < 2^24");
  int rc = check_select((int)rows, (int)n_blocks, top_k, (int64_t)n_blocks, (int)ratio);
  if (rc) return rc;
  if (!aligned(q, 16) || !aligned(block_keys, 16)) return fail(IDX_ERR_SHAPE, "q and block_keys must be 16-byte aligned");
  if (rows == 0) return ok();
  if (n_blocks == 0)  // no block: every slot is padding (the select alone writes it)
    return indexer_topk_select(nullptr, 0, nullptr, first_pos, (int)ratio, (int)rows, 0, top_k, topk_idx, topk_scores,
                               workspace, workspace_bytes, stream);
  ScoreSelectLayout l;
  if (!score_select_layout(rows, n_blocks, top_k, &l)) return fail(IDX_ERR_UNSUPPORTED, "top_k %d is not supported", top_k);
  if (!workspace || workspace_bytes < l.total)
    return fail(IDX_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", l.total, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(IDX_ERR_SHAPE, "workspace must be 256-byte aligned");
  unsigned char* w = static_cast<unsigned char*>(workspace);
  float* sc = reinterpret_cast<float*>(w + l.scores);
  uint32_t* tm = l.tiles ? reinterpret_cast<uint32_t*>(w + l.tmax) : nullptr;
  hipError_t e = salb::launch_qsa_score_f16(reinterpret_cast<const _Float16*>(q),
                                            reinterpret_cast<const _Float16*>(block_keys), sc, rows, n_blocks,
                                            first_pos, l.sstride, ratio, n_heads, hd, stream, tm, l.tstride);
  if (e != hipSuccess) return hip_fail(e, "QSA score launch");
  if (l.tiles) {
    e = salb::launch_select_tiles(sc, l.sstride, tm, l.tstride, first_pos, (int)ratio, (int)rows, (int)n_blocks, top_k,
                                  topk_idx, topk_scores, stream);
  } else {
    salb::SelectPlan p;
    salb::plan_select((int)rows, (int)n_blocks, top_k, &p);
    e = salb::launch_select(p, sc, l.sstride, nullptr, first_pos, (int)ratio, topk_idx, topk_scores, w + l.select,
                            false, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "select kernel launch");
  return ok();
}

int indexer_debug_dequant(const uint8_t* keys_fp4, const uint8_t* key_scale, const float* key_gscale,
                          const int32_t* block_table_row, int n, int D, int epb, int n_pages, int mode, float* out,
                          hipStream_t stream) {
  if (!keys_fp4 || !key_scale || !key_gscale || !block_table_row || !out)
    return fail(IDX_ERR_NULL, "all pointers are required");
  if (D != 64 && D != 128 && D != 256) return fail(IDX_ERR_UNSUPPORTED, "head_dim %d", D);
  if (epb < 1 || epb > 65536 || n_pages < 1) return fail(IDX_ERR_SHAPE, "epb / n_pages out of range");
  if (n < 0 || n >= kMaxCols) return fail(IDX_ERR_SHAPE, "n out of range");
  if (mode < 0 || mode > 2) return fail(IDX_ERR_UNSUPPORTED, "mode %d", mode);
  if (!aligned(keys_fp4, 16) || !aligned(key_scale, 4)) return fail(IDX_ERR_SHAPE, "misaligned key arrays");
  if (n == 0) return ok();
  hipError_t e = salb::launch_debug_dequant(keys_fp4, key_scale, key_gscale, block_table_row, n, D, epb, mode, out,
                                            stream);
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return ok();
}

}  // extern "C"
