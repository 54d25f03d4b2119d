/*
 * verify_attn.h -- C ABI of the MI355X (gfx950) split-KV target-verify
 * attention library (speculative decoding, topk = 1).
 *
 * The operation is the one sglang's "verify_splitkv.py" defines (module
 * docstring; kernels _verify_prefix_stage1 and _verify_combine_stage2; entry
 * verify_splitkv_fwd): each sequence b has a prefix of n_b tokens in a paged
 * KV pool and l_ext draft tokens.  Draft query row i of query head h attends
 *   - to every prefix token (no mask), score = sm_scale * k_scale *
 *     <cast_to_pool_dtype(q), K_pool[row]>, value = v_scale * V_pool[row];
 *   - to the draft tokens j <= i of its own sequence (causal), score =
 *     sm_scale * <q, K_ext[j]>, value = V_ext[j] (no cast, no scale);
 * with one softmax over both.  Query heads are grouped contiguously per KV
 * head (kv_head = h / (h_q / h_kv)).
 *
 * Execution: two kernels on the caller's stream.  The prefix pass splits every
 * sequence's prefix into ranges processed in parallel; each range writes a
 * normalised partial output and its log-sum-exp into the caller's workspace.
 * The combine pass merges the ranges by log-sum-exp, computes the small causal
 * draft block and merges the two.  No call allocates, synchronises, or reads
 * device memory on the host, so every call may be captured into a HIP graph.
 *
 * Pointers: every tensor pointer is a device pointer (HIP device memory of the
 * current device).  The caller owns every buffer; the library keeps no
 * reference after a call returns.  Element strides are in elements of the
 * tensor's own type; the last dimension of every tensor must be contiguous.
 *
 * Errors: every entry point returns VA_OK (0) or a negative va_status_t and
 * does nothing else on error.  verify_attn_last_error() gives a message for
 * the most recent error on the calling thread.
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VA_API __attribute__((visibility("default")))

/* Element type of the prefix pool (k_buf, v_buf).  q, k_ext, v_ext and out
 * are always bf16.  FP8_E4M3FN is the OCP 8-bit format (bias 7, max 448). */
typedef enum {
    VA_DTYPE_BF16 = 0,
    VA_DTYPE_FP8_E4M3FN = 1
} va_dtype_t;

typedef enum {
    VA_OK = 0,
    VA_ERR_NULL_ARG = -1,   /* a required pointer is NULL */
    VA_ERR_BATCH = -2,      /* bs < 1 */
    VA_ERR_HEADS = -3,      /* h_q or h_kv < 1, or h_q % h_kv != 0 */
    VA_ERR_HEAD_DIM = -4,   /* head dims not in {64,128,256}, or neither equal nor a factor 2 apart */
    VA_ERR_DTYPE = -5,      /* kv_dtype not a va_dtype_t */
    VA_ERR_EXTEND = -6,     /* l_ext < 1, or q_rows != bs * l_ext (ragged extend) */
    VA_ERR_STRIDE = -7,     /* stride not positive, rows overlap, or row start not 16-B aligned */
    VA_ERR_SCALE = -8,      /* sm_scale, k_scale or v_scale not finite or <= 0 */
    VA_ERR_WORKSPACE = -9,  /* workspace NULL or smaller than the plan's size */
    VA_ERR_SPLIT = -10,     /* split_tokens not a multiple of 64, or both split fields set */
    VA_ERR_ALIGN = -11,     /* a tensor base pointer is not 16-byte aligned */
    VA_ERR_DEVICE = -12,    /* a HIP runtime call failed (device query or launch) */
    VA_ERR_SIZE = -13       /* a size is negative or exceeds the kernels' index range */
} va_status_t;

/* Static problem description: shapes, strides and the pool dtype.  Every
 * field is a host value; nothing here is read from device memory.
 *   q      [q_rows, h_q,  head_dim]    bf16     strides q_stride[0..1]
 *   k_ext  [q_rows, h_kv, head_dim]    bf16     strides kext_stride[0..1]
 *   v_ext  [q_rows, h_kv, v_head_dim]  bf16     strides vext_stride[0..1]
 *   k_buf  [pool,   h_kv, head_dim]    kv_dtype strides kbuf_stride[0..1]
 *   v_buf  [pool,   h_kv, v_head_dim]  kv_dtype strides vbuf_stride[0..1]
 *   out    [q_rows, h_q,  v_head_dim]  bf16     strides out_stride[0..1]
 * head_dim and v_head_dim are separate, as verify_splitkv.py keeps them
 * (VerifySplitKV(..., head_dim, v_head_dim, ...); BLOCK_DV in
 * _verify_prefix_stage1): both in {64, 128, 256}, equal or one twice the
 * other.
 * num_kv_indices is the length of kv_indices: a static shape, which may be
 * the capacity of a buffer sized for the largest batch (as a captured graph
 * replays it) rather than the batch's own total; every kv_indptr entry must
 * lie in [0, num_kv_indices].
 * Splitting (both 0 = the library's heuristic: the grid holds one range per
 * resident prefix workgroup, at least one per sequence and at most
 * ceil(num_kv_indices / 64) -- for a batch with more sequences than that,
 * about one range per MiB of K/V per KV head -- and the kernels pick the
 * range size from kv_indptr on every launch: the smallest multiple of 64
 * tokens whose ranges fit that grid, or whole sequences for a batch past
 * the resident workgroups whose prefixes are within 1/8 of equal, with the
 * MiB-range bound taken for the tokens kv_indptr holds; so the split follows
 * the lengths actually passed, whatever the capacity of kv_indices):
 *   split_tokens > 0 : every prefix is cut into ranges of split_tokens tokens
 *                      (a multiple of 64), one work item each;
 *   n_splits > 0     : the pages' rule -- every prefix is cut into n_splits
 *                      ranges of ceil(ceil(n_b / n_splits) / 32) * 32 tokens;
 *                      ranges past the end are empty.
 * The result does not depend on the split beyond floating-point rounding. */
typedef struct {
    int32_t bs;
    int32_t h_q;
    int32_t h_kv;
    int32_t head_dim;
    int32_t v_head_dim;
    int32_t kv_dtype;
    int64_t q_rows;
    int64_t num_kv_indices;
    int64_t q_stride[2];
    int64_t kext_stride[2];
    int64_t vext_stride[2];
    int64_t kbuf_stride[2];
    int64_t vbuf_stride[2];
    int64_t out_stride[2];
    int32_t split_tokens;
    int32_t n_splits;
} va_desc_t;

/* Launch plan derived from a descriptor (pure function of the descriptor,
 * l_ext and the CU count; identical for every call with the same inputs, so a
 * workspace sized once stays valid, as graph capture needs). */
typedef struct {
    int32_t mode;            /* 0: heuristic (range size fitted on the device); 1: n_splits equal
                                ranges per sequence; 2: ranges of split_tokens tokens; 3: the
                                heuristic for a batch past the resident workgroups (rounds) */
    int32_t split_tokens;    /* mode 2: tokens per range; modes 0, 3: the size num_kv_indices tokens in
                                equal prefixes would get (where the kernels guess each range starts) */
    int32_t n_splits;        /* ranges per sequence (mode 1) */
    int32_t rows;            /* query rows per KV head: (h_q / h_kv) * l_ext */
    int32_t row_chunks;      /* rows are processed in chunks of at most 64 */
    int32_t tile_tokens;     /* prefix tokens per LDS tile in the prefix kernel */
    int64_t range_slots;     /* ranges (partial-output slots) per KV head the grid holds */
    int64_t prefix_blocks;   /* grid of the prefix kernel (workgroups of 256 or 512 threads) */
    int64_t combine_blocks;  /* grid of the combine kernel (one 64-thread workgroup per output row) */
    size_t workspace_bytes;  /* bytes of workspace the two passes need */
    size_t partial_bytes;    /* of which: bf16 partial outputs (the fp32 log-sum-exps follow) */
    size_t table_offset;     /* then, from this offset: each sequence's first range and range count */
} va_plan_t;

/* Validate a descriptor (host only; no HIP call).
 * Mirrors can_handle() in verify_splitkv.py, which accepts only causal topk=1
 * verify with a constant extend length: bs >= 1, h_q % h_kv == 0, supported
 * head dims, q_rows == bs * l_ext.  Returns VA_OK or the first failing code. */
VA_API int verify_attn_check(const va_desc_t *desc, int32_t l_ext);

/* Compute the launch plan.  num_cus > 0 uses that CU count (pure host);
 * num_cus <= 0 queries the current HIP device once and caches it per device.
 * The static split heuristic needs only shapes (no device read), the
 * capture-safety constraint stated in verify_splitkv.py's choose_n_splits. */
VA_API int verify_attn_plan(const va_desc_t *desc, int32_t l_ext, int32_t num_cus,
                            va_plan_t *plan);

/* Workspace size in bytes for (desc, l_ext) on a device with num_cus CUs
 * (num_cus <= 0: the current device).  Equals plan.workspace_bytes.  The
 * workspace holds the partial outputs and log-sum-exps of the prefix ranges,
 * the role of VerifySplitKV's att_out / att_lse scratch in verify_splitkv.py,
 * which that class sizes once by max_bs so that its address stays fixed.  In
 * the same spirit the size never decreases as bs or num_kv_indices grow (all
 * other fields equal): a workspace sized for the largest call serves every
 * smaller one. */
VA_API int verify_attn_workspace_bytes(const va_desc_t *desc, int32_t l_ext, int32_t num_cus,
                                       size_t *bytes);

/* Full verify attention: the prefix pass then the combine pass, both on
 * `stream` (a hipStream_t; NULL = the default stream).  The operation of
 * verify_splitkv_fwd / VerifySplitKV.__call__ in sglang's verify_splitkv.py
 * (stage 1 _verify_prefix_stage1 over the split prefix, stage 2
 * _verify_combine_stage2 for the range merge, the causal draft block and the
 * final merge), with the arguments of its problem statement.
 *   q, k_ext, v_ext   draft queries / keys / values (bf16, layouts above)
 *   k_buf, v_buf      prefix pool (desc->kv_dtype)
 *   qo_indptr [bs+1]  int32; must equal b * l_ext (constant extend length)
 *   kv_indptr [bs+1]  int32; non-decreasing prefix offsets into kv_indices
 *   kv_indices        int64 pool row of every prefix token, each in [0, pool)
 *   sm_scale          softmax scale (1/sqrt(head_dim) is the usual value)
 *   k_scale, v_scale  pool dequant multipliers on prefix scores / prefix values
 *   out               bf16 output, written in full (rounded to nearest even)
 *   workspace         device buffer of at least verify_attn_workspace_bytes(),
 *                     256-byte aligned; caller-owned, contents not preserved
 * Ownership: the library keeps no pointer after the call; calls that share a
 * workspace must not overlap in time (same stream, or synchronised).
 * The qo_indptr / kv_indptr / kv_indices preconditions are not checked on the
 * host (that would need a device read); violating them is undefined. */
VA_API int verify_attn_run(const void *q, const void *k_ext, const void *v_ext,
                           const void *k_buf, const void *v_buf,
                           const int32_t *qo_indptr, const int32_t *kv_indptr,
                           const int64_t *kv_indices, int32_t l_ext,
                           float sm_scale, float k_scale, float v_scale, void *out,
                           const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                           void *stream);

/* verify_attn_run without a workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the partial outputs and log-sum-exps live in a device array
 * the library owns, 32 MiB per GPU (kept until the process ends), instead of
 * the caller's workspace.  Arguments, results and errors as for
 * verify_attn_run; a call whose plan needs more than the array holds
 * (plan.workspace_bytes > 32 MiB: e.g. several hundred sequences of many
 * query rows) returns VA_ERR_WORKSPACE and launches nothing.  No call
 * allocates: the array's address on a device is resolved once, by the first
 * call on that device (make that call outside graph capture).  Every call on
 * a GPU shares that GPU's array and leaves its contents behind; calls that
 * overlap in time on one GPU (different streams, or different threads) race
 * on it and give undefined results. */
VA_API int verify_attn_run_noalloc(const void *q, const void *k_ext, const void *v_ext,
                                   const void *k_buf, const void *v_buf,
                                   const int32_t *qo_indptr, const int32_t *kv_indptr,
                                   const int64_t *kv_indices, int32_t l_ext,
                                   float sm_scale, float k_scale, float v_scale, void *out,
                                   const va_desc_t *desc, void *stream);

/* Prefix pass only (the pages' _verify_prefix_stage1): writes, for every range
 * and query row, the v_scale-multiplied normalised partial output (bf16) and
 * its natural log-sum-exp into the workspace; an empty range writes output 0
 * and log-sum-exp -inf.  Arguments as for verify_attn_run. */
VA_API int verify_attn_prefix(const void *q, const void *k_buf, const void *v_buf,
                              const int32_t *qo_indptr, const int32_t *kv_indptr,
                              const int64_t *kv_indices, int32_t l_ext,
                              float sm_scale, float k_scale, float v_scale,
                              const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Combine pass only (the pages' _verify_combine_stage2): log-sum-exp merge of
 * the ranges written by verify_attn_prefix, the causal draft block, the final
 * two-way merge and the bf16 store into out.  Arguments as for verify_attn_run. */
VA_API int verify_attn_combine(const void *q, const void *k_ext, const void *v_ext,
                               const int32_t *qo_indptr, const int32_t *kv_indptr,
                               int32_t l_ext, float sm_scale, void *out,
                               const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Page-table prefix (page_size > 1; the unified-verify block table of sglang's
 * aiter_backend.py, which views the pool as [pages, page_size, H_KV, D]): as
 * verify_attn_run / verify_attn_prefix, but the prefix rows come from
 * block_table (int32, row b at block_table + b * block_table_stride) instead
 * of kv_indices: token t < n_b of sequence b is pool row
 *   block_table[b * block_table_stride + t / page_size] * page_size
 *     + t % page_size
 * of k_buf / v_buf (whose desc strides are per token row).  kv_indptr still
 * gives the prefix lengths n_b = kv_indptr[b+1] - kv_indptr[b], and
 * desc->num_kv_indices their host-known total.  page_size >= 1; page ids and
 * table bounds are not checked (device data). */
VA_API int verify_attn_run_paged(const void *q, const void *k_ext, const void *v_ext,
                                 const void *k_buf, const void *v_buf,
                                 const int32_t *qo_indptr, const int32_t *kv_indptr,
                                 const int32_t *block_table, int64_t block_table_stride,
                                 int32_t page_size, int32_t l_ext,
                                 float sm_scale, float k_scale, float v_scale, void *out,
                                 const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                                 void *stream);

VA_API int verify_attn_prefix_paged(const void *q, const void *k_buf, const void *v_buf,
                                    const int32_t *qo_indptr, const int32_t *kv_indptr,
                                    const int32_t *block_table, int64_t block_table_stride,
                                    int32_t page_size, int32_t l_ext,
                                    float sm_scale, float k_scale, float v_scale,
                                    const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Tree verify (topk > 1): as verify_attn_run / verify_attn_combine, but the
 * draft block follows a tree mask instead of the causal rule.  Layout of the
 * mask as sglang's aiter_backend.py builds it for extend attention with
 * skip_prefix_custom_mask: sequence b's mask is a row-major byte array of
 * l_ext rows x (n_b + l_ext) columns starting at byte offset mask_indptr[b]
 * (int64, bs + 1 entries), n_b = kv_indptr[b+1] - kv_indptr[b]; the first n_b
 * columns (the prefix) are not read -- the prefix stays fully visible -- and
 * draft key j is visible to draft row i when byte n_b + j of row i is
 * nonzero.  A row that sees no key at all is written as 0.  l_ext <= 64
 * (VA_ERR_EXTEND otherwise).  The prefix pass is unchanged. */
VA_API int verify_attn_run_tree(const void *q, const void *k_ext, const void *v_ext,
                                const void *k_buf, const void *v_buf,
                                const int32_t *qo_indptr, const int32_t *kv_indptr,
                                const int64_t *kv_indices, int32_t l_ext,
                                float sm_scale, float k_scale, float v_scale,
                                const uint8_t *custom_mask, const int64_t *mask_indptr, void *out,
                                const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                                void *stream);

VA_API int verify_attn_combine_tree(const void *q, const void *k_ext, const void *v_ext,
                                    const int32_t *qo_indptr, const int32_t *kv_indptr,
                                    int32_t l_ext, float sm_scale,
                                    const uint8_t *custom_mask, const int64_t *mask_indptr,
                                    void *out, const va_desc_t *desc, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Draft K/V append into the pool, the step before verify (sglang
 * aiter_backend.py: set_kv_buffer at out_cache_loc, and
 * launch_reshape_and_cache_flash, which fuses the bf16 -> fp8 cast with the
 * paged write).  Row i of k [n_tokens, h_kv, head_dim] and v [n_tokens, h_kv,
 * v_head_dim] (bf16; strides desc->kext_stride / vext_stride) is written to
 * pool row out_cache_loc[i] (int64, each in [0, pool)) of k_buf / v_buf
 * (desc->kv_dtype, strides desc->kbuf_stride / vbuf_stride).  A bf16 pool
 * receives the bits unchanged (scales ignored); an fp8 pool receives the
 * E4M3FN code of x / scale, the quotient one correctly rounded fp32 division,
 * rounded to nearest even and saturating at +-448.  Rows named twice: one of
 * the writes survives (unordered).  Uses desc->h_kv, head_dim, v_head_dim,
 * kv_dtype and the four strides only.  n_tokens = 0 is a no-op. */
VA_API int verify_attn_append_kv(const void *k, const void *v, const int64_t *out_cache_loc,
                                 int64_t n_tokens, float k_scale, float v_scale,
                                 void *k_buf, void *v_buf, const va_desc_t *desc, void *stream);

/* kv_indices from the request-to-token table, as sglang's aiter_backend.py
 * builds them for verify (kv_indptr = running sum of the lengths, then
 * create_flashinfer_kv_indices_triton): for request b < bs and i < seq_lens[b],
 *   kv_indices[kv_indptr[b] + i] =
 *       req_to_token[req_pool_indices[b] * req_to_token_stride + start_b + i]
 * with start_b = kv_start_idx[b] (or 0 when kv_start_idx is NULL).  Writes
 * kv_indptr [bs + 1] (int32, kv_indptr[0] = 0) too.  req_to_token is int32,
 * req_pool_indices int64, seq_lens and kv_start_idx int32.  capacity is the
 * length of kv_indices (normally the host-known total of seq_lens); entries
 * beyond it are not written.  One kernel launch; no host synchronisation. */
VA_API int verify_attn_build_kv_indices(const int32_t *req_to_token, int64_t req_to_token_stride,
                                        const int64_t *req_pool_indices, const int32_t *seq_lens,
                                        const int32_t *kv_start_idx, int32_t bs, int64_t capacity,
                                        int32_t *kv_indptr, int64_t *kv_indices, void *stream);

/* Static text for a status code. */
VA_API const char *verify_attn_strerror(int code);

/* Message for the most recent error on the calling thread ("" if none). */
VA_API const char *verify_attn_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
VA_API int verify_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
