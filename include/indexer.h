/*
 * Lightning-indexer score + top-k for MI355X (gfx950): the C ABI.
 *
 * Pages this library implements (cited by title and section):
 *  [listing] "nvfp4-megamoe-kernel -- dsv4/kernels/indexer/indexer_score_topk.cu":
 *            header comment (eq. 16), NVFP4 notes, dequant_fp4_scalar, heap_insert,
 *            the main kernel (paged pool, block table, valid lengths, final sort)
 *            and its PyTorch binding (argument list and shapes).
 *  [commits] "nvfp4-megamoe-kernel -- commit graph of dsv4/kernels/indexer":
 *            79ef87f9a9 (E2M1 encoding table), e74c84458c (E2M1 magnitude LUT),
 *            c2f705a21a (score_topk launcher: q in BF16 or FP32).
 *  [qsa.rs]  "metrale_model_layers/layers/ops/qsa.rs": doc comments and argument
 *            lists of qsa_block_pool, qsa_qprep_rows, qsa_score_rows(_tc), and the
 *            module comment on per-row prefill selection passes.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers the caller allocates; the library never
 *    allocates, frees or synchronises.  All work is enqueued on `stream`
 *    (NULL = the null stream) and the call returns without waiting.
 *  - Inputs are read-only and must not alias outputs.  Outputs are overwritten
 *    completely (including -1 / -inf padding).
 *  - Return value: IDX_OK or an IDX_ERR_* code.  Argument checks run on the host
 *    before any HIP call; on failure nothing is launched and
 *    indexer_last_error() describes the problem.  Device faults surface at the
 *    caller's next synchronisation.  A call with no rows to process returns
 *    IDX_OK without launching anything ([qsa.rs] qsa_block_pool: no launch when
 *    there is no work).
 *  - Out-of-range data (a valid length beyond the table, a page id outside the
 *    pool) is undefined behaviour unless the call is made with IDX_F_VALIDATE,
 *    which checks it first and returns IDX_ERR_DATA (see the flags below).
 *  - Workspaces are scratch: every call writes each part of its workspace before
 *    reading it, so a workspace needs no initialisation and may serve calls of any
 *    shape in turn (the size rule of each call still applies).  Calls that share a
 *    workspace must be ordered (one stream, or synchronised).
 */
#ifndef SALB_INDEXER_H
#define SALB_INDEXER_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define IDX_OK 0
#define IDX_ERR_NULL 1         /* a required pointer is NULL */
#define IDX_ERR_SHAPE 2        /* inconsistent or out-of-range sizes */
#define IDX_ERR_WORKSPACE 3    /* workspace missing or smaller than the *_workspace_size() value */
#define IDX_ERR_UNSUPPORTED 4  /* a size or mode this build does not implement */
#define IDX_ERR_HIP 5          /* a HIP runtime call failed (message in indexer_last_error) */
#define IDX_ERR_DATA 6         /* IDX_F_VALIDATE found a valid length or page id out of range */

/* flags of the paged scorers */
#define IDX_F_VALIDATE 1u      /* check valid_lens and the block-table entries they use before
                                  any scoring: a one-workgroup check kernel, then a
                                  synchronisation of `stream` (so the call blocks and must not
                                  be captured into a graph); on bad data nothing else is
                                  launched and IDX_ERR_DATA names the first bad row or entry.
                                  Without it such data is undefined behaviour. */

/* element type of q */
#define IDX_DTYPE_F32 0
#define IDX_DTYPE_BF16 1

/* arithmetic of the dot products */
#define IDX_PREC_FP32 0   /* fp32 products and sums (the fp32 matrix cores at D 64/128, vector
                             FMAs at D 256); scores within ~1e-5 relative of the exact value */
#define IDX_PREC_MFMA 1   /* fp16 matrix cores with fp32 accumulation; q rounded to 11 bits
                             after a per-head power-of-two prescale, NVFP4 code values exact */

/* Human-readable description of the last error on the calling thread ("" if none). */
const char* indexer_last_error(void);

/*
 * indexer_score_rows -- the lightning-indexer scores of every (query, key) pair.
 *
 * [listing] header comment (eq. 16) and main kernel:
 *     scores[t, s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[t,s,:] )    for s < valid_lens[t]
 *     scores[t, s] = -inf                                          for valid_lens[t] <= s < n_cols
 * with one key vector per logical entry s, shared by all heads:
 *     p = block_table[t * bt_stride + s / epb],  e = p * epb + s % epb,
 *     k[t,s,d] = E2M1(nibble d of keys_fp4[e]) * E4M3(key_scale[e, d/16]) * key_gscale[p]
 * nibble d is the low nibble of byte d/2 for even d and the high nibble for odd d
 * ([listing] dequant_fp4_scalar); E2M1 magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6 with
 * bit 3 as sign ([commits] 79ef87f9a9, e74c84458c); E4M3 is the OCP FP8 format.
 *
 *  q           [T, H, D] fp32 or bf16 (q_dtype), contiguous
 *  w           [T, H] fp32, contiguous (any sign)
 *  keys_fp4    [n_pages, epb, D/2] uint8, contiguous
 *  key_scale   [n_pages, epb, D/16] uint8 (E4M3 bytes), contiguous
 *  key_gscale  [n_pages] fp32 (any sign)
 *  block_table [T, max_lb] int32 with row stride bt_stride >= max_lb; entries at
 *              logical blocks >= ceil(valid_lens[t]/epb) are never read
 *  valid_lens  [T] int32, each in [0, min(n_cols, max_lb*epb)]
 *  scores      [T, n_cols] fp32 output with row stride score_stride >= n_cols
 * Supported: D in {64, 128, 256}; 1 <= H <= 64; 1 <= epb <= 65536; n_cols < 2^24.
 * precision: IDX_PREC_FP32 or IDX_PREC_MFMA.
 * flags: 0 or IDX_F_VALIDATE (the check uses the first 16 bytes of `scores` as its
 *        status word; scores must then be 8-byte aligned).
 */
int indexer_score_rows(const void* q, int q_dtype, const float* w,
                       const uint8_t* keys_fp4, const uint8_t* key_scale, const float* key_gscale,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* valid_lens,
                       int T, int H, int D, int epb, int max_lb, int n_pages,
                       int precision, unsigned flags, float* scores, int64_t score_stride, int n_cols,
                       hipStream_t stream);

/*
 * indexer_topk_select -- per-row top-k of a score matrix.
 *
 * For each row r, the candidates are the entries s in [0, valid_r); they are
 * ranked by score descending, equal scores by increasing index (the order of the
 * [listing]'s heap comparator and final selection sort; -0.0 equals 0.0, NaN
 * ranks below every number).  The first K_r = min(top_k, valid_r) ranked indices
 * go to topk_idx[r, 0:K_r] and the remaining slots hold -1 ([listing]: heap
 * pre-filled with -1); topk_scores (optional, may be NULL) receives the matching
 * scores and -inf in padded slots.
 *
 * valid_r is valid_lens[r] if valid_lens != NULL; otherwise, if ratio > 0,
 * min(n_cols, floor((first_pos + r + 1) / ratio)) -- the count of complete
 * blocks of a prefill row at position first_pos + r ([qsa.rs] qsa_score_rows);
 * otherwise n_cols.
 *
 *  scores      [rows, n_cols] fp32, row stride score_stride >= n_cols
 *  topk_idx    [rows, top_k] int32 output (logical indices s)
 *  topk_scores [rows, top_k] fp32 output or NULL
 *  workspace   device scratch of indexer_topk_workspace_size(...) bytes, 256-byte
 *              aligned, owned by the caller; no initialisation needed (rows longer
 *              than 8192 entries zero its histogram counters with one small launch
 *              ahead of the select).  May be NULL when the size is 0.
 * Supported: 1 <= top_k <= 8192, n_cols < 2^24.
 */
size_t indexer_topk_workspace_size(int rows, int n_cols, int top_k);
int indexer_topk_select(const float* scores, int64_t score_stride, const int32_t* valid_lens,
                        int64_t first_pos, int ratio, int rows, int n_cols, int top_k,
                        int32_t* topk_idx, float* topk_scores,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * indexer_score_topk -- the fused hot path: Selected[t] = TopK(I[t, :], top_k)
 * ([listing] header comment, eq. 16; main kernel and its binding).
 *
 * Arguments as for indexer_score_rows (with n_cols = max_lb * epb) and
 * indexer_topk_select; the scores live only in the workspace.
 *  topk_idx    [T, top_k] int32 output: logical entry indices s, -1 padded
 *  topk_scores [T, top_k] fp32 output or NULL
 *  flags       0 or IDX_F_VALIDATE
 *  workspace   device scratch of indexer_score_topk_workspace_size(...) bytes, 256-byte
 *              aligned, no initialisation needed: it holds the [T, max_lb*epb] score
 *              matrix and the select's buffers; the scorer launch also zeroes the
 *              select's histogram counters.
 */
size_t indexer_score_topk_workspace_size(int T, int max_lb, int epb, int top_k);
int indexer_score_topk(const void* q, int q_dtype, const float* w,
                       const uint8_t* keys_fp4, const uint8_t* key_scale, const float* key_gscale,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* valid_lens,
                       int T, int H, int D, int epb, int max_lb, int n_pages, int top_k,
                       int precision, unsigned flags, int32_t* topk_idx, float* topk_scores,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * indexer_score_topk_noalloc -- indexer_score_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, which lives instead in
 * a scratch array of IDX_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends.  Results are those of indexer_score_topk.
 *  - Calls whose indexer_score_topk_workspace_size(T, max_lb, epb, top_k) exceeds the
 *    scratch return IDX_ERR_WORKSPACE before any HIP call.
 *  - The scratch of the current device (hipGetDevice) is used; `stream` must belong to
 *    that device.  Its address is looked up once per device; no call allocates or
 *    frees anything.
 *  - All calls on one GPU share its scratch: calls that overlap in time on one GPU
 *    (different streams, or threads without ordering) race and give undefined results.
 *    Each call initialises what it reads, so calls of any shapes may follow each other.
 */
#define IDX_NOALLOC_SCRATCH_BYTES (128ull << 20)
int indexer_score_topk_noalloc(const void* q, int q_dtype, const float* w,
                               const uint8_t* keys_fp4, const uint8_t* key_scale, const float* key_gscale,
                               const int32_t* block_table, int64_t bt_stride, const int32_t* valid_lens,
                               int T, int H, int D, int epb, int max_lb, int n_pages, int top_k,
                               int precision, unsigned flags, int32_t* topk_idx, float* topk_scores,
                               hipStream_t stream);

/*
 * indexer_gather_kv -- the selected entries as a dense bf16 tile ([commits] c2f705a21a,
 * gather_kv.cu: FP8 + BF16 split entries of a paged pool, resolved through the block
 * table, dequantised to one dense [T, top_k, head_dim] bf16 tile).
 *
 * For t < T and i < top_k, with s = topk_idx[t, i]:
 *   s in [0, max_lb*epb): p = block_table[t * bt_stride + s / epb], e = p * epb + s % epb,
 *     out[t, i, d]          = bf16(E4M3(kv_fp8[e, d]) * kv_scale[e, d / group])  d < d_nope
 *     out[t, i, d_nope + j] = kv_rope[e, j]                                      j < d_rope
 *   otherwise (the -1 padding of a top-k): out[t, i, :] = 0.
 * bf16(x) is one round-to-nearest-even of the exact product (for products in the normal
 * fp32 range; the product is never rounded to fp32 first).
 *  kv_fp8    [n_pages, epb, d_nope] uint8 OCP E4M3 codes, 16-byte aligned
 *  kv_scale  [n_pages, epb, d_nope / group] fp32
 *  kv_rope   [n_pages, epb, d_rope] bf16 (uint16 bit patterns), 16-byte aligned
 *  out       [T, top_k, d_nope + d_rope] bf16 output, 16-byte aligned
 * Page ids outside [0, n_pages) among the entries selected are undefined behaviour (the
 * indices come from indexer_score_topk, which only returns entries below valid_lens).
 * Supported: d_nope a multiple of 16, group a multiple of 16 dividing it, d_rope a
 * multiple of 8, 1 <= epb <= 65536, max_lb * epb < 2^24.
 */
int indexer_gather_kv(const uint8_t* kv_fp8, const float* kv_scale, const uint16_t* kv_rope,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* topk_idx,
                      int T, int top_k, int epb, int max_lb, int n_pages, int d_nope, int d_rope, int group,
                      uint16_t* out, hipStream_t stream);

/*
 * qsa_gather -- selected tokens' K/V rows into contiguous scratch ([qsa.rs] qsa_gather):
 *   k_out[i, :, :] = k_cache[block_table[sel[i] / block_size], sel[i] % block_size, :, :]
 *   v_out[i, :, :] = v_cache[...same...]                                       i < n_sel
 *  k_cache, v_cache [n_blocks, block_size, nkv, hd] 2-byte elements (bf16), 16-byte aligned
 *  block_table      [>= max(sel) / block_size + 1] int32 (one sequence)
 *  sel              [n_sel] int32 token positions; outside the table is undefined behaviour
 *  k_out, v_out     [n_sel, nkv, hd] outputs, 16-byte aligned
 * A bit copy.  Supported: nkv * hd a multiple of 8.
 */
int qsa_gather(const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* block_table, const int32_t* sel,
               uint16_t* k_out, uint16_t* v_out, uint32_t n_sel, uint32_t block_size, uint32_t nkv, uint32_t hd,
               hipStream_t stream);

/*
 * qsa_prefill_attn -- block-sparse prefill attention over the selected blocks
 * ([qsa.rs] qsa_prefill_attn: per row and query head, attention over exactly the blocks
 * of the row's list plus the incomplete tail, read from the paged cache):
 *   row r at pos = first_pos + r has nb = floor((pos + 1) / ratio) complete blocks;
 *   it attends positions [ratio*b, ratio*b + ratio) of every list entry 0 <= b < nb
 *   (-1 and other entries are skipped) and the tail [ratio*nb, pos];
 *   attn_out[r, h, :] = sum_j softmax_j(inv_sqrt_d * q[r, h] . k_j) * v_j,
 *   with k_j, v_j of KV head h / (nq / nkv) at cache page block_table[j / block_size],
 *   slot j % block_size; a row that attends nothing gets zeros.
 * Scores and the softmax in fp32 (q . k from bf16 inputs on the matrix cores), the
 * probabilities rounded to fp16 for the value product.
 *  q           [rows, nq, hd] bf16 (uint16 bit patterns), 16-byte aligned
 *  k_cache,    [pages, block_size, nkv, hd] bf16, 16-byte aligned
 *  v_cache
 *  block_table [> (first_pos + rows - 1) / block_size] int32 (one sequence); the cache
 *              rows it names, page * block_size + slot, must be below 2^31
 *  lists       [rows, topk] int32 (a top-k of complete blocks, -1 padded); NULL if topk = 0
 *  attn_out    [rows, nq, hd] fp32 output
 * Supported: hd 64 or 128; nkv dividing nq with nq / nkv <= 16; topk * ratio small
 * enough for a workgroup's LDS (about 25000 positions at hd 128).
 */
int qsa_prefill_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* block_table,
                     const int32_t* lists, float* attn_out, uint32_t rows, uint32_t first_pos, uint32_t topk,
                     uint32_t ratio, uint32_t block_size, uint32_t nq, uint32_t nkv, uint32_t hd, float inv_sqrt_d,
                     hipStream_t stream);

/*
 * qsa_block_pool -- pooled QSA block keys ([qsa.rs] qsa_block_pool).
 *
 * For b in [first_block, first_block + n_new):
 *     m = mean(raw_keys[ratio*b .. ratio*b + ratio - 1, :])
 *     n = m / sqrt(mean(m^2) + eps) * (1 + k_norm_w)
 *     block_keys[b, :] = RoPE(n, position ratio*b) on dims [0, rot)
 * RoPE pairs dim i with i + rot/2 (i < rot/2) at angle pos * theta^(-2i/rot),
 * the angle formed in fp64; dims >= rot are copied.
 *  raw_keys   [>= ratio*(first_block+n_new), hd] bf16 (uint16 bit patterns)
 *  k_norm_w   [hd] fp32
 *  block_keys [>= first_block+n_new, hd] fp32 output (only the n_new rows are written)
 * raw_keys and block_keys 16-byte aligned.
 * Supported: hd in {64, 128, 256}, rot even and <= hd, ratio >= 1.
 */
int qsa_block_pool(const uint16_t* raw_keys, const float* k_norm_w, float* block_keys,
                   uint32_t first_block, uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot,
                   float theta, float eps, hipStream_t stream);

/*
 * qsa_block_pool_f16 -- qsa_block_pool with fp16 block keys: each fp32 result rounded to
 * nearest even, the values the matrix-core scorer multiplies (qsa_score_rows_f16 reads
 * them as they are; qsa_score_rows with IDX_PREC_MFMA rounds fp32 keys to the same
 * values).  block_keys [>= first_block+n_new, hd] fp16 (uint16 bit patterns), 16-byte
 * aligned; everything else as qsa_block_pool.
 */
int qsa_block_pool_f16(const uint16_t* raw_keys, const float* k_norm_w, uint16_t* block_keys,
                       uint32_t first_block, uint32_t n_new, uint32_t ratio, uint32_t hd, uint32_t rot,
                       float theta, float eps, hipStream_t stream);

/*
 * qsa_qprep_rows -- prefill query prep ([qsa.rs] qsa_qprep_rows, qsa_qprep).
 *
 * For row r and head h: x = qk[r, h*hd .. h*hd+hd-1];
 *     q_out[r, h, :] = RoPE(x / sqrt(mean(x^2) + eps) * (1 + q_norm_w), first_pos + r)
 *  qk       [rows, qkw] bf16 (uint16 bit patterns), qkw >= n_heads*hd, qkw a multiple
 *           of 8, 16-byte aligned
 *  q_norm_w [hd] fp32
 *  q_out    [rows, n_heads, hd] fp32 output, 16-byte aligned
 * RoPE as in qsa_block_pool.
 * Supported: hd in {64, 128, 256}, rot even and <= hd, n_heads * hd <= 32768, and
 * rows * ceil(n_heads * hd / 1024) < 2^31 (the launch grid; IDX_ERR_SHAPE otherwise).
 */
int qsa_qprep_rows(const uint16_t* qk, const float* q_norm_w, float* q_out,
                   uint32_t rows, uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd,
                   uint32_t rot, float theta, float eps, hipStream_t stream);

/*
 * qsa_qprep_rows_f16 -- qsa_qprep_rows with fp16 output (each fp32 result rounded to
 * nearest even; the query values the matrix-core scorer multiplies).  q_out
 * [rows, n_heads, hd] fp16 (uint16 bit patterns), 16-byte aligned.
 */
int qsa_qprep_rows_f16(const uint16_t* qk, const float* q_norm_w, uint16_t* q_out,
                       uint32_t rows, uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd,
                       uint32_t rot, float theta, float eps, hipStream_t stream);

/*
 * qsa_qprep -- one decode query ([qsa.rs] qsa_qprep): per head h,
 *     q_out[h, :] = RoPE(x / sqrt(mean(x^2) + eps) * (1 + q_norm_w), pos),  x = q_in[h*hd .. h*hd+hd-1]
 * i.e. qsa_qprep_rows for one row at position pos, read from a projection of n_heads * hd.
 *  q_in   [n_heads * hd] bf16 (uint16 bit patterns), 16-byte aligned
 *  q_out  [n_heads, hd] fp32 output, 16-byte aligned
 */
int qsa_qprep(const uint16_t* q_in, const float* q_norm_w, float* q_out, uint32_t n_heads, uint32_t hd,
              uint32_t rot, uint32_t pos, float theta, float eps, hipStream_t stream);

/*
 * qsa_decode_prep -- a decode step's inputs in one launch: qsa_block_pool of blocks
 * [first_block, first_block + n_new) into block_keys and qsa_qprep_rows of rows
 * [0, rows) (positions first_pos + r) into q_out, both fp32.  The arguments, layouts,
 * checks and results are those of the two calls, bit for bit (the same arithmetic);
 * the two write disjoint outputs, so one launch replaces two.  Returns IDX_OK without a
 * launch when n_new and rows are both 0.
 */
int qsa_decode_prep(const uint16_t* raw_keys, const float* k_norm_w, float* block_keys, uint32_t first_block,
                    uint32_t n_new, uint32_t ratio, const uint16_t* qk, const float* q_norm_w, float* q_out,
                    uint32_t rows, uint32_t first_pos, uint32_t qkw, uint32_t n_heads, uint32_t hd, uint32_t rot,
                    float theta, float eps, hipStream_t stream);

/*
 * qsa_score -- decode scores of one query over n_blocks blocks ([qsa.rs] qsa_score):
 *     scores[b] = sum_h ReLU(q[h,:] . block_keys[b,:]) / sqrt(hd)     b < n_blocks
 * (every block given is scored; the caller passes the query's complete blocks).  fp32
 * arithmetic, within ~1e-5 relative of the exact value: on the fp32 matrix cores
 * (fp32 products and accumulation) when n_heads is 16, 32, 48 or 64 and hd is 64 or
 * 128, else on the vector ALUs.
 *  q          [n_heads, hd] fp32, 16-byte aligned
 *  block_keys [>= n_blocks, hd] fp32, 16-byte aligned
 *  scores     [n_blocks] fp32 output (may be NULL when n_blocks is 0: nothing is launched)
 * Supported: hd in {64, 128, 256}, 1 <= n_heads <= 64.
 */
int qsa_score(const float* q, const float* block_keys, float* scores, uint32_t n_blocks, uint32_t n_heads,
              uint32_t hd, hipStream_t stream);

/*
 * qsa_score_topk -- qsa_score of one decode query over n_blocks blocks, then the top_k
 * of those scores as indexer_topk_select of one row with every block valid: the same
 * indices and scores, bit for bit, as the two calls.  The scores live in the workspace.
 * On the matrix-core scorer (16..64 heads in steps of 16, hd 64 or 128) with n_blocks <=
 * 32768 and top_k <= 512, the score launch also records the largest order key of every
 * 16-block sub-tile and one select launch reads only the sub-tiles that can hold a winner
 * (as qsa_select_tiles); otherwise the score launch clears the general select's counters.
 * top_k slots past n_blocks get -1 (and -inf).
 *  workspace  >= qsa_score_topk_workspace_size(n_blocks, top_k) bytes, 256-byte aligned,
 *             any contents (NULL allowed when the size is 0)
 * Errors as qsa_score and indexer_topk_select; IDX_ERR_WORKSPACE when it is too small.
 */
size_t qsa_score_topk_workspace_size(uint32_t n_blocks, int top_k);
int qsa_score_topk(const float* q, const float* block_keys, uint32_t n_blocks, uint32_t n_heads, uint32_t hd,
                   int top_k, int32_t* topk_idx, float* topk_scores, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * qsa_score_rows -- QSA block scores ([qsa.rs] qsa_score, qsa_score_rows, qsa_score_rows_tc):
 *     scores[r, b] = sum_h ReLU(q[r,h,:] . block_keys[b,:]) / sqrt(hd)   for b < nb_r
 *     scores[r, b] = -inf                                              for nb_r <= b < n_blocks_max
 * with nb_r = min(n_blocks_max, floor((first_pos + r + 1) / ratio)).
 *  q          [rows, n_heads, hd] fp32
 *  block_keys [n_blocks_max, hd] fp32
 *  scores     [rows, n_blocks_max] fp32 output, row stride score_stride >= n_blocks_max
 * Supported: hd in {64, 128, 256}, 1 <= n_heads <= 64; precision IDX_PREC_FP32 or IDX_PREC_MFMA.
 * IDX_PREC_MFMA runs on the fp16 matrix cores (q and keys rounded to fp16, fp32
 * accumulation; within 2e-3 of the row's largest score) when hd is 64 or 128 and
 * n_heads is 16, 32 or 64, and on the fp32 path (~1e-5 relative) otherwise.  The fp16
 * rounding takes the values as they are, with no prescale: it assumes every |q| and
 * |block_keys| element is below 65504 and that elements below 2^-14 (fp16's normal
 * range) carry a negligible share of a score -- which holds for the RMSNorm outputs of
 * qsa_block_pool and qsa_qprep_rows (elements of order sqrt(hd) * |1 + w|).  Other
 * inputs belong on IDX_PREC_FP32.
 */
int qsa_score_rows(const float* q, const float* block_keys, float* scores,
                   uint32_t rows, uint32_t n_blocks_max, uint32_t first_pos, uint32_t score_stride,
                   uint32_t ratio, uint32_t n_heads, uint32_t hd, int precision, hipStream_t stream);

/*
 * qsa_score_rows_f16 -- qsa_score_rows on the fp16 matrix cores from fp16 q [rows, n_heads,
 * hd] and block keys [n_blocks_max, hd] (uint16 bit patterns, 16-byte aligned), as
 * written by qsa_qprep_rows_f16 and qsa_block_pool_f16: the same scores, bit for bit, as
 * qsa_score_rows with IDX_PREC_MFMA on the fp32 tensors those calls round, with half the
 * query and key bytes.  Supported: hd in {64, 128}, n_heads in {16, 32, 64}.
 */
int qsa_score_rows_f16(const uint16_t* q, const uint16_t* block_keys, float* scores,
                       uint32_t rows, uint32_t n_blocks_max, uint32_t first_pos, uint32_t score_stride,
                       uint32_t ratio, uint32_t n_heads, uint32_t hd, hipStream_t stream);

/*
 * qsa_score_select_f16 -- the QSA prefill's row scores and their top-k in one call
 * ([qsa.rs] qsa_score_rows_tc and the causal valid count of qsa_score_rows): qsa_score_rows_f16 of
 * rows [0, rows) over blocks [0, n_blocks) followed by indexer_topk_select with the valid
 * count floor((first_pos + r + 1) / ratio), bit-identical to the two calls (indices and
 * scores, ties included); the scores live only in the workspace.  For n_blocks <= 32768
 * and top_k <= 512 the score launch also records the largest order key of every 16-block
 * sub-tile, and the select reads only the sub-tiles whose maximum reaches the K-th
 * largest sub-tile maximum (no winner lies elsewhere); otherwise the general select runs.
 *  q, block_keys   as qsa_score_rows_f16 (fp16 bit patterns, 16-byte aligned)
 *  topk_idx        [rows, top_k] int32 output (block indices, -1 past the valid count)
 *  topk_scores     [rows, top_k] fp32 output or NULL (-inf past the valid count)
 *  workspace       device scratch of qsa_score_select_f16_workspace_size(rows, n_blocks,
 *                  top_k) bytes, 256-byte aligned, no initialisation needed
 * Errors as qsa_score_rows_f16 and indexer_topk_select; IDX_ERR_WORKSPACE when it is too small.
 */
/*
 * The two halves of qsa_score_select_f16, for callers that keep the scores:
 *
 * qsa_score_rows_f16_tmax -- qsa_score_rows_f16, and for every row r < rows and 16-block
 * sub-tile s < ceil(n_blocks_max / 16) the largest order key of the sub-tile's stored
 * scores into tile_max[r * tile_stride + s] (uint32; the order key maps a score's bits to
 * an unsigned integer in score order, -0 as +0, every NaN to 0, the lowest; blocks past
 * n_blocks_max count as 0).  tile_stride >= ceil(n_blocks_max / 16).
 *
 * qsa_select_tiles -- indexer_topk_select with the causal valid count (ratio >= 1) over
 * those scores and tile maxima: the same output, bit for bit, reading only the sub-tiles
 * that can hold a winner.  Supported: n_cols <= 32768, top_k <= 512; scores 16-byte
 * aligned with score_stride a multiple of 4 and >= n_cols rounded up to 16 (whole
 * sub-tiles are read); no workspace.
 */
int qsa_score_rows_f16_tmax(const uint16_t* q, const uint16_t* block_keys, float* scores, uint32_t* tile_max,
                            uint32_t rows, uint32_t n_blocks_max, uint32_t first_pos, uint32_t score_stride,
                            uint32_t tile_stride, uint32_t ratio, uint32_t n_heads, uint32_t hd, hipStream_t stream);
int qsa_select_tiles(const float* scores, int64_t score_stride, const uint32_t* tile_max, int64_t tile_stride,
                     int64_t first_pos, int ratio, int rows, int n_cols, int top_k, int32_t* topk_idx,
                     float* topk_scores, hipStream_t stream);

size_t qsa_score_select_f16_workspace_size(uint32_t rows, uint32_t n_blocks, int top_k);
int qsa_score_select_f16(const uint16_t* q, const uint16_t* block_keys, uint32_t rows, uint32_t n_blocks,
                         uint32_t first_pos, uint32_t ratio, uint32_t n_heads, uint32_t hd, int top_k,
                         int32_t* topk_idx, float* topk_scores, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * indexer_debug_dequant -- test hook for the NVFP4 decoders used by the scorers.
 *
 * For the first n logical entries of one block-table row (addressing as in
 * indexer_score_rows), writes out[s, d] (fp32, [n, D]):
 *   mode 0: the exact code value E2M1 * E4M3 from the fp32 decoder,
 *   mode 1: the fp32 rounding of code value * key_gscale[p] from the fp32 decoder,
 *   mode 2: the code value from the fp16 matrix-core operand decoder, widened to fp32.
 */
int indexer_debug_dequant(const uint8_t* keys_fp4, const uint8_t* key_scale, const float* key_gscale,
                          const int32_t* block_table_row, int n, int D, int epb, int n_pages,
                          int mode, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SALB_INDEXER_H */
