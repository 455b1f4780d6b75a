/*
 * mla_decode.h - C ABI of the MI355X (gfx950) single-token MLA decode library.
 *
 * Operation (kernelindex.com "kernelbot-amd-mixed-mla-695854", the chunked
 * torch attention fallback; "kernelbot-amd-mixed-mla-668813", the module
 * constants): DeepSeek-style multi-head latent attention decode with one query
 * token per request, 16 query heads sharing a single latent KV head of width
 * 576 (512 latent + 64 rope).  For request b and head h
 *
 *     out[b,h,:] = bf16( softmax_t( q[b,h,:] . k_t / sqrt(576) ) @ v_t )
 *
 * where k_t is the dequantised 576-wide cache row of token t and v_t its first
 * 512 entries.  The work is split over the KV sequence (split-K "flash
 * decoding", page 668813's mxfp4 stage-1/stage-2 kernels): stage 1 produces a
 * normalised partial output and a base-2 log-sum-exp per (request, split,
 * head); stage 2 merges the splits.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers unless stated otherwise; the
 *     caller allocates and owns every buffer (the library allocates nothing and
 *     keeps no state between calls; calls on different streams with disjoint
 *     outputs and workspaces may run concurrently).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; nothing synchronises with the host.
 *   - Return value: MLA_OK (0) or a negative MLA_ERR_* code.  Argument errors
 *     are detected on the host before anything is enqueued.  Device-resident
 *     contents (indptr monotonicity, page ids in range) are not checked on the
 *     hot path: a gathered row past the cache is clamped to its last row (so
 *     a corrupt page id gives wrong values, never an access outside the
 *     cache), while kv_indptr / page_indptr entries that index past the page
 *     table are undefined behaviour, as for an out-of-range pointer.
 *     mla_check_tables checks host copies of the tables against the cache
 *     size before they are uploaded.
 *   - bf16 values are raw IEEE bfloat16 bit patterns (uint16).
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 3  /* 3: q_dtypes MLA_Q_BF16_FP8_STATIC and MLA_Q_BF16_MXFP4 */

/* Fixed MLA geometry (page 668813 module constants). */
#define MLA_NUM_HEADS 16
#define MLA_HEAD_DIM_QK 576      /* 512 latent + 64 rope */
#define MLA_HEAD_DIM_V 512       /* V = first 512 latent dims */
#define MLA_MXFP4_ROW_BYTES 288  /* 576 e2m1 codes, two per byte */
#define MLA_MXFP4_ROW_SCALES 18  /* one e8m0 per 32 elements */

/* Element formats. */
#define MLA_DTYPE_BF16 0         /* IEEE bfloat16 */
#define MLA_DTYPE_FP8_E4M3FN 1   /* OCP fp8 e4m3fn with one fp32 per-tensor scale */
#define MLA_DTYPE_MXFP4 2        /* OCP MX e2m1 + e8m0 per 32 elements */
/* Split cache (mla_decode_mixed): K from an mxfp4 cache, V from an fp8 cache
 * on the same rows.  Accepted as kv_dtype by mla_choose_num_splits only. */
#define MLA_KV_MXFP4_K_FP8_V 3

/* q_dtype only, with the fp8 cache: Q arrives as bf16 [batch,R,576] and the
 * stage-1 workgroups quantise it to e4m3fn themselves, code for code as
 * mla_quantize_fp8 with dynamic == 0 and the static per-tensor scale
 * *q_scale (device float[1]), before decoding it as fp8 Q.  Page 600081's
 * fp8 route takes such a static Q scale (`STATIC_Q_ABSMAX`) so that no amax
 * pass is needed per call; here the quantiser's separate launch goes too.
 * For every finite Q the output is bit-identical to mla_quantize_fp8
 * followed by the decode with MLA_DTYPE_FP8_E4M3FN (NaN elements of Q give
 * unspecified codes there and here). */
#define MLA_Q_BF16_FP8_STATIC 4

/* q_dtype only, with the mxfp4 cache: Q arrives as bf16 [batch,R,576] and the
 * stage-1 workgroups quantise it to mxfp4 themselves (e2m1 codes with one
 * e8m0 scale per 32 elements), code for code and scale for scale as
 * mla_quantize_mxfp4, before decoding it as mxfp4 Q; q_scale is NULL.  Page
 * 668813's mxfp4 route quantises Q to mxfp4 on every call.  The output is
 * bit-identical to mla_quantize_mxfp4 followed by the decode with
 * MLA_DTYPE_MXFP4 (NaN elements of Q give unspecified codes there and here). */
#define MLA_Q_BF16_MXFP4 5

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_NULL (-1)        /* a required pointer is NULL */
#define MLA_ERR_DTYPE (-2)       /* unsupported (q, kv) format pair */
#define MLA_ERR_ARG (-3)         /* a size/count is out of range */
#define MLA_ERR_ALIGN (-4)       /* a buffer is not 16-byte aligned */
#define MLA_ERR_WORKSPACE (-5)   /* workspace missing or too small */
#define MLA_ERR_LAUNCH (-6)      /* the HIP runtime rejected a launch */
#define MLA_ERR_DEVICE (-7)      /* no usable gfx950 device */

#define MLA_MAX_SPLITS 256
#define MLA_MAX_Q_ROWS 1024      /* query rows per request (q_seq_len x heads), multiple of 16 */

/*
 * mla_decode - split-K MLA decode of `batch` single-token requests.
 *
 * q          [batch,16,576] bf16            (q_dtype = MLA_DTYPE_BF16,
 *                                            MLA_Q_BF16_FP8_STATIC or
 *                                            MLA_Q_BF16_MXFP4), or
 *            [batch,16,576] e4m3fn bytes    (q_dtype = MLA_DTYPE_FP8_E4M3FN), or
 *            [batch,16,288] packed e2m1     (q_dtype = MLA_DTYPE_MXFP4).
 * q_scale    NULL for bf16 and MLA_Q_BF16_MXFP4; device float[1] per-tensor scale for fp8 (the value
 *            a code is multiplied by) and for MLA_Q_BF16_FP8_STATIC (the
 *            static scale Q is quantised with); device uint8 e8m0
 *            [batch*16, 18] for mxfp4.
 * kv_cache   physical cache rows: [num_kv_rows,576] bf16 | [num_kv_rows,576]
 *            e4m3fn | [num_kv_rows,288] packed e2m1 (byte i: element 2i in the
 *            low nibble, 2i+1 in the high nibble; page 668813's stage-1 kernel).
 * kv_scale   NULL for bf16; device float[1] for fp8; device uint8 e8m0
 *            [num_kv_rows,18] for mxfp4, whose allocation must cover at least
 *            ceil(18*num_kv_rows/16)*16 bytes (rows are read as aligned dwords).
 * kv_indptr  device int32[batch+1], token offsets: request b has
 *            kv_indptr[b+1]-kv_indptr[b] >= 0 tokens.
 * page_table device int32 physical page ids.
 * page_indptr NULL: one table over the concatenated token stream - token t of
 *            request b is logical position g = kv_indptr[b] + t and lives in row
 *            page_table[g / page_size] * page_size + g % page_size.
 *            Non-NULL (device int32[batch]): per-request tables - token t of
 *            request b lives in row page_table[page_indptr[b] + t / page_size]
 *            * page_size + t % page_size.
 * page_size  >= 1 rows per page.
 * num_splits 1..MLA_MAX_SPLITS chunks per request (ceil(L/S) tokens each, the
 *            last ones possibly short or empty).  1 writes `out` directly from
 *            stage 1 and needs no workspace.
 * out        [batch,16,512] bf16, round-to-nearest-even of the fp32 result.
 * workspace  device scratch of at least mla_workspace_bytes(batch, num_splits)
 *            bytes (may be NULL when that is 0); contents on entry are ignored.
 *
 * Supported (q, kv) pairs: (bf16,bf16), (bf16,fp8), (fp8,fp8), (bf16 quantised
 * to fp8 in the call, fp8), (bf16,mxfp4), (mxfp4,mxfp4), (bf16 quantised to
 * mxfp4 in the call, mxfp4); anything else returns MLA_ERR_DTYPE.  q, kv_cache, out and
 * workspace must be 16-byte aligned.
 */
int mla_decode(const void* q, int32_t q_dtype, const void* q_scale,
               const void* kv_cache, int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows,
               const int32_t* kv_indptr, int32_t batch,
               const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
               int32_t num_splits, void* out, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * mla_decode_noalloc - mla_decode with no workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The split partials live in a
 * static device array of MLA_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; its address is looked up on
 * the first call on a device.  The call allocates nothing and calls no
 * allocating routine.  Every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (different streams, or concurrent host threads
 * enqueueing before the previous call has run) race on it and must be
 * serialised by the caller; no part of it needs to start at zero (each call
 * writes every partial it reads).  Arguments, output and errors as for
 * mla_decode, plus MLA_ERR_WORKSPACE when mla_workspace_bytes(batch,
 * num_splits) exceeds MLA_NOALLOC_SCRATCH_BYTES (e.g. batch 256 at 4 splits)
 * and MLA_ERR_DEVICE when the array's device address cannot be looked up.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int mla_decode_noalloc(const void* q, int32_t q_dtype, const void* q_scale,
                       const void* kv_cache, int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows,
                       const int32_t* kv_indptr, int32_t batch,
                       const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                       int32_t num_splits, void* out, void* stream);

/*
 * mla_validate - the host-side argument checks of mla_decode, with the same
 * arguments, returning the status mla_decode would return before launching.
 * Makes no HIP call and touches no device memory (usable without a GPU).
 */
int mla_validate(const void* q, int32_t q_dtype, const void* q_scale,
                 const void* kv_cache, int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows,
                 const int32_t* kv_indptr, int32_t batch,
                 const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                 int32_t num_splits, void* out, void* workspace, size_t workspace_bytes);

/*
 * mla_check_tables - host check of the index tables a decode call will read
 * (pure host code, no HIP call): every token a request covers must map to a
 * physical row inside the cache, by the paging rule given for mla_decode.
 *
 * kv_indptr_host   host int32[batch+1], non-negative and nondecreasing.
 * page_table_host  host int32[page_table_len] (may be NULL when that is 0).
 * page_indptr_host NULL (one table over the token stream) or host
 *                  int32[batch] (per-request tables, non-negative starts).
 * page_size        >= 1; num_kv_rows >= 0 cache rows.
 * bad_request      optional out: the first request whose tokens fail (or -1
 *                  for a size error or when every check passes).
 *
 * Returns MLA_OK; MLA_ERR_NULL for a missing table; MLA_ERR_ARG for
 * batch < 0, page_size < 1, negative sizes, decreasing or negative offsets,
 * a page-table index past page_table_len, or a page id whose rows fall
 * outside [0, num_kv_rows).  Cost: one pass over the pages the requests
 * touch.
 */
int mla_check_tables(const int32_t* kv_indptr_host, int32_t batch, const int32_t* page_table_host,
                     int64_t page_table_len, const int32_t* page_indptr_host, int32_t page_size,
                     int64_t num_kv_rows, int32_t* bad_request);

/* Bytes of workspace mla_decode needs: fp32 partial outputs [batch,S,16,512]
 * plus base-2 log-sum-exps [batch,S,16]; 0 when num_splits == 1.  Returns 0
 * for invalid arguments too (batch < 1 or num_splits outside 1..MLA_MAX_SPLITS). */
size_t mla_workspace_bytes(int32_t batch, int32_t num_splits);

/*
 * mla_choose_num_splits - split count for `batch` requests of about
 * `kv_len` tokens with Q in q_dtype over a cache in kv_dtype (any MLA_DTYPE_*
 * code, or MLA_KV_MXFP4_K_FP8_V for the split cache; unknown codes count as
 * bf16 Q / fp8 cache) on a device with `num_cus` compute units (0 = 256,
 * MI355X).  On the tuned grid (batch 4/32/64/256 x kv_len 1024/8192 x the five
 * supported format pairs, MI355X) it returns the measured fastest S, from a
 * table written by mla_latent_kv_13_amd/tune.py.  Elsewhere an occupancy cost
 * model decides: ceil(batch*S / num_cus) rounds of one workgroup per CU, each
 * streaming its chunk rounded up to 128 tokens, plus for S > 1 the partial
 * outputs, a second launch and a per-split stage-2 latency.  (Page 695854's
 * split selectors and page 668813's split tables pick S per shape for the
 * same reasons.)  Returns a value in 1..MLA_MAX_SPLITS; pure host code.
 */
int32_t mla_choose_num_splits(int32_t batch, int32_t kv_len, int32_t q_dtype, int32_t kv_dtype, int32_t num_cus);

/*
 * mla_recommend_page_size - page size for a cache serving `batch` requests of
 * about `kv_len` tokens, Q in q_dtype over a cache in kv_dtype, on `num_cus`
 * compute units (0 = 256).  On the tuned grid (as mla_choose_num_splits) it
 * returns the measured fastest page size of {1, 2, 4, ..., 64}; elsewhere a
 * model: the largest power of two up to 16 that is at most a quarter of
 * kv_len.  (Page 668813's page-size table and page 600081's selector pick 1
 * for short and 8 for long sequences.)  The kernels accept any page size
 * >= 1; pure host code.
 */
int32_t mla_recommend_page_size(int32_t batch, int32_t kv_len, int32_t q_dtype, int32_t kv_dtype, int32_t num_cus);

/*
 * mla_decode_rows - mla_decode for q_rows query rows per request: q_seq_len
 * query tokens x num_heads heads (multi-token decode, or more than 16 heads),
 * flattened row-major into q [batch, q_rows, 576] (mxfp4: [batch, q_rows,
 * 288] with e8m0 q_scale [batch*q_rows, 18]; the in-call quantisation modes
 * MLA_Q_BF16_FP8_STATIC and MLA_Q_BF16_MXFP4 take bf16 rows as mla_decode
 * does); out is [batch, q_rows, 512].
 * Every row attends to its request's whole cache with no mask, as page
 * 695854's chunked torch fallback treats q_seq_len x num_heads rows (its
 * aiter route takes q_seq_len 4 with 16, 32 or 64 heads).  q_rows is a
 * multiple of 16 in 16..MLA_MAX_Q_ROWS; the kernels run one workgroup per
 * 16-row group, the groups sharing a token range back to back so the cache
 * is re-read from the cache hierarchy rather than HBM.  Workspace:
 * mla_workspace_bytes_rows(batch, q_rows, num_splits).  q_rows == 16 is
 * mla_decode.  Errors as mla_decode, plus MLA_ERR_ARG for a bad q_rows.
 */
int mla_decode_rows(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows,
                    const void* kv_cache, int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows,
                    const int32_t* kv_indptr, int32_t batch,
                    const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                    int32_t num_splits, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of mla_decode_rows (0 when num_splits == 1 or arguments
 * are out of range); mla_workspace_bytes(b, s) == mla_workspace_bytes_rows(b, 16, s). */
size_t mla_workspace_bytes_rows(int32_t batch, int32_t q_rows, int32_t num_splits);

/*
 * Work lists for ragged batches.  With one split count for the whole batch a
 * long request's splits outlast everything else; a work list instead cuts
 * every request into items of about the same token count, so one launch is
 * balanced whatever the length mix.  Page 668813's fp8 route and page
 * 695854's default route build the same kind of plan with aiter's metadata
 * builder (get_mla_metadata_v1: per-CU work items, per-request reduce
 * ranges, an fp32 partial array); this plan is built on the host.
 *
 * mla_plan_worklist - host planner (pure host code, no HIP call).
 *   kv_indptr_host  host int32[batch+1] token offsets, nondecreasing.
 *   num_cus         compute units (0 = 256).
 *   max_items       capacity of items_host, >= batch.
 *   items_host      out: int32[max_items][4] = {request, first token within
 *                   the request, token count, slot}; slot indexes the item's
 *                   partial in the workspace, or is -1 when its request is a
 *                   single item (stage 1 then writes `out` directly).
 *   req_host        out: int32[batch][2] = {first slot, number of items}.
 *   num_items, num_slots  out: items written and partial slots used.
 * The chunk is the smallest multiple of 128 tokens (at least 256, grown in
 * steps of about 1/8 from T / (R * num_cus), T the total token count) whose
 * items fit R = ceil(batch / num_cus) rounds of one workgroup per CU, then
 * doubled if needed until the items fit in max_items.  A request of L tokens becomes n = ceil(L /
 * chunk) items, item j covering tokens [floor(jL/n), floor((j+1)L/n)); an
 * empty request one item of 0 tokens.  Items are listed request by request.
 * Returns MLA_OK, MLA_ERR_NULL, or MLA_ERR_ARG (batch < 0, max_items < batch,
 * decreasing offsets).
 */
int mla_plan_worklist(const int32_t* kv_indptr_host, int32_t batch, int32_t num_cus, int32_t max_items,
                      int32_t* items_host, int32_t* req_host, int32_t* num_items, int32_t* num_slots);

/* Bytes of workspace a plan with num_slots partial slots needs for q_rows
 * query rows per request (fp32 partial O [num_slots,q_rows,512] then base-2
 * LSE [num_slots,q_rows]); 0 for 0 slots or a bad q_rows. */
size_t mla_worklist_workspace_bytes(int32_t num_slots, int32_t q_rows);

/*
 * mla_decode_worklist - mla_decode over a plan from mla_plan_worklist: one
 * stage-1 workgroup per item, then stage 2 merges the slots of every request
 * with more than one item.  items (int32[num_items][4]) and req
 * (int32[batch][2]) are device copies of the planner's arrays; the other
 * arguments are as for mla_decode_rows, with num_splits replaced by the plan
 * and workspace sized by mla_worklist_workspace_bytes(num_slots, q_rows).  Errors as for
 * mla_decode, plus MLA_ERR_NULL for a missing plan array and MLA_ERR_ARG for
 * num_items < batch or num_slots < 0.  The device-resident plan is not
 * checked, like kv_indptr.
 */
int mla_decode_worklist(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows,
                        const void* kv_cache, int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows,
                        const int32_t* kv_indptr, int32_t batch,
                        const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                        const int32_t* items, int32_t num_items, const int32_t* req, int32_t num_slots,
                        void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_mixed - decode over a split cache (page 695854, its triton and
 * sage mxfp4 q=1 routes): the logits use the mxfp4 cache's keys (all 576
 * dims) and the outputs the fp8 cache's values (dims 0..511 of its rows), the
 * two caches holding the same tokens in the same physical rows:
 *
 *     out[b,h,:] = bf16( softmax_t( q[b,h,:] . kmx_t / sqrt(576) ) @ vfp8_t[0:512] )
 *
 * q, q_scale   bf16 [batch,q_rows,576] (q_dtype MLA_DTYPE_BF16, q_scale NULL)
 *              or packed e2m1 [batch,q_rows,288] with e8m0 [batch*q_rows,18]
 *              (MLA_DTYPE_MXFP4, as page 695854 quantises Q for these routes).
 * k_cache      [num_kv_rows,288] packed e2m1, k_scale e8m0 [num_kv_rows,18]
 *              (allocation padded as for mla_decode's mxfp4 kv_scale).
 * v_cache      [num_kv_rows,576] e4m3fn (only bytes 0..511 of a row are
 *              read), v_scale device float[1].
 * The other arguments are as for mla_decode_rows (q_rows, paging, splits,
 * workspace of mla_workspace_bytes_rows(batch, q_rows, num_splits)).  Errors
 * as for mla_decode_rows; MLA_ERR_DTYPE for a q_dtype other than bf16 or
 * mxfp4, MLA_ERR_NULL for a missing v_cache / v_scale, MLA_ERR_ALIGN for a
 * v_cache that is not 16-byte or a v_scale that is not 4-byte aligned.
 */
int mla_decode_mixed(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows,
                     const void* k_cache, const void* k_scale, const void* v_cache, const void* v_scale,
                     int64_t num_kv_rows, const int32_t* kv_indptr, int32_t batch,
                     const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                     int32_t num_splits, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* The host-side argument checks of mla_decode_mixed (no HIP call). */
int mla_validate_mixed(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows,
                       const void* k_cache, const void* k_scale, const void* v_cache, const void* v_scale,
                       int64_t num_kv_rows, const int32_t* kv_indptr, int32_t batch,
                       const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                       int32_t num_splits, void* out, void* workspace, size_t workspace_bytes);

/*
 * mla_quantize_fp8 - OCP e4m3fn per-tensor quantisation of n bf16 values
 * (page 668813, the naive per-tensor fp8 quantiser): with dynamic != 0 the
 * scale is max(max|x|, 1e-12) / 448 computed on the device and written to
 * *scale (device float[1]); with dynamic == 0 *scale is read as given.  Each
 * code is the nearest e4m3fn value to clamp(x / scale, -448, 448) (fp32
 * division, ties to even).  NaN inputs are ignored by the amax.
 */
int mla_quantize_fp8(const void* src_bf16, int64_t n, uint8_t* dst, float* scale, int32_t dynamic,
                     void* stream);

/*
 * mla_quantize_mxfp4 - OCP MX mxfp4 quantisation of rows of `cols` bf16 values
 * (cols a positive multiple of 32): per 32-element block the e8m0 scale is
 * floor(log2(amax)) - 2 + 127 clamped to [0,254] (0 for an all-zero block) and
 * each element is the nearest e2m1 value to x / 2^(e-127), ties to even,
 * saturating at +-6.  packed: [rows, cols/2] (element 2i in the low nibble);
 * scales: [rows, cols/32].
 */
int mla_quantize_mxfp4(const void* src_bf16, int64_t rows, int64_t cols, uint8_t* packed,
                       uint8_t* scales, void* stream);

/*
 * mla_stream_read - measurement helper, not part of the decode path.  Reads
 * `bytes` bytes (a multiple of 16) of the device buffer `src` (16-byte
 * aligned) once with 16-byte non-temporal loads spread over up to 131072
 * workgroups, folding them into one word that is written to `sink` (device,
 * 4 bytes) only if it equals a fixed improbable value.  Enqueued on `stream`;
 * its duration is the streaming-read ceiling of the device for a buffer of
 * that size.  Returns MLA_ERR_ARG for a negative or unaligned size,
 * MLA_ERR_NULL, MLA_ERR_ALIGN or MLA_ERR_LAUNCH; 0 bytes is a no-op.
 */
int mla_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Human-readable text for a status code (static storage). */
const char* mla_status_string(int status);

/* MLA_ABI_VERSION of the loaded library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H_ */
