// va_plan.cpp -- host-side validation, static split planning and error state.
//
// Validation mirrors can_handle() in sglang's verify_splitkv.py: only shapes
// and host scalars are inspected, never tensor values, because the verify
// step runs inside captured HIP graphs where a device->host read is not
// allowed.  The split plan is likewise a pure function of static shapes and
// the CU count (choose_n_splits in the same file is the pages' version of
// this idea: a split count from the average prefix length).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "va_internal.h"

namespace va {

namespace {
thread_local char g_last_error[512] = {0};

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

// Byte strides of a row/head must keep 16-byte row starts (the kernels move
// data in 16-byte vectors).
bool aligned_strides(const int64_t s[2], int elem_bytes)
{
    return (s[0] * elem_bytes) % 16 == 0 && (s[1] * elem_bytes) % 16 == 0;
}
}  // namespace

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

void clear_error() { g_last_error[0] = 0; }

const char *last_error() { return g_last_error; }

int check_desc(const va_desc_t *d, int32_t l_ext)
{
    if (!d)
        return fail(VA_ERR_NULL_ARG, "descriptor is NULL");
    if (d->bs < 1)
        return fail(VA_ERR_BATCH, "bs = %d; need at least one sequence", d->bs);
    if (d->h_q < 1 || d->h_kv < 1 || d->h_q % d->h_kv != 0)
        return fail(VA_ERR_HEADS, "h_q = %d, h_kv = %d; need h_q a positive multiple of h_kv",
                    d->h_q, d->h_kv);
    if (!supported_head_dims(d->head_dim, d->v_head_dim))
        return fail(VA_ERR_HEAD_DIM,
                    "head_dim = %d, v_head_dim = %d; supported: both in {64,128,256}, equal or one twice the other",
                    d->head_dim, d->v_head_dim);
    if (d->kv_dtype != VA_DTYPE_BF16 && d->kv_dtype != VA_DTYPE_FP8_E4M3FN)
        return fail(VA_ERR_DTYPE, "kv_dtype = %d is not a va_dtype_t", d->kv_dtype);
    if (l_ext < 1)
        return fail(VA_ERR_EXTEND, "l_ext = %d; need at least one draft token", l_ext);
    if (d->q_rows != (int64_t)d->bs * l_ext)
        return fail(VA_ERR_EXTEND, "q_rows = %lld but bs * l_ext = %lld (ragged extend is not supported)",
                    (long long)d->q_rows, (long long)d->bs * l_ext);
    if (d->num_kv_indices < 0)
        return fail(VA_ERR_SIZE, "num_kv_indices = %lld is negative", (long long)d->num_kv_indices);
    if (d->num_kv_indices > INT32_MAX)
        return fail(VA_ERR_SIZE, "num_kv_indices = %lld exceeds the int32 range of kv_indptr",
                    (long long)d->num_kv_indices);
    const int64_t *in_strides[5] = {d->q_stride, d->kext_stride, d->vext_stride, d->kbuf_stride,
                                    d->vbuf_stride};
    for (int i = 0; i < 5; ++i)
        if (in_strides[i][0] < 0 || in_strides[i][1] < 0)
            return fail(VA_ERR_STRIDE, "negative input stride");
    const int kv_bytes = d->kv_dtype == VA_DTYPE_FP8_E4M3FN ? 1 : 2;
    if (!aligned_strides(d->q_stride, 2) || !aligned_strides(d->kext_stride, 2) ||
        !aligned_strides(d->vext_stride, 2) || !aligned_strides(d->out_stride, 2) ||
        !aligned_strides(d->kbuf_stride, kv_bytes) || !aligned_strides(d->vbuf_stride, kv_bytes))
        return fail(VA_ERR_STRIDE, "every row and head stride must be a multiple of 16 bytes");
    if (d->kbuf_stride[0] * kv_bytes > (int64_t)UINT32_MAX || d->vbuf_stride[0] * kv_bytes > (int64_t)UINT32_MAX)
        return fail(VA_ERR_STRIDE, "pool row stride above 4 GiB");
    // The output is written: its rows must not overlap.
    if (d->out_stride[1] < d->v_head_dim || d->out_stride[0] < (int64_t)d->h_q * d->out_stride[1])
        return fail(VA_ERR_STRIDE, "out strides (%lld, %lld) make output rows overlap",
                    (long long)d->out_stride[0], (long long)d->out_stride[1]);
    if (d->split_tokens < 0 || d->n_splits < 0)
        return fail(VA_ERR_SPLIT, "negative split_tokens / n_splits");
    if (d->split_tokens > 0 && d->n_splits > 0)
        return fail(VA_ERR_SPLIT, "set at most one of split_tokens and n_splits");
    if (d->split_tokens % kSplitQuantum != 0)
        return fail(VA_ERR_SPLIT, "split_tokens = %d is not a multiple of %d", d->split_tokens,
                    kSplitQuantum);
    clear_error();
    return VA_OK;
}

int current_device_cus(int32_t *cus)
{
    static std::atomic<int32_t> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(VA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) {
        int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return VA_OK;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0)
        return fail(VA_ERR_DEVICE, "hipDeviceGetAttribute(CU count): %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64)
        cache[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return VA_OK;
}

int make_plan(const va_desc_t *d, int32_t l_ext, int32_t num_cus, va_plan_t *plan)
{
    if (!plan)
        return fail(VA_ERR_NULL_ARG, "plan is NULL");
    int rc = check_desc(d, l_ext);
    if (rc != VA_OK)
        return rc;
    if (num_cus <= 0) {
        rc = current_device_cus(&num_cus);
        if (rc != VA_OK)
            return rc;
    }
    va_plan_t p;
    memset(&p, 0, sizeof(p));
    const int64_t group = d->h_q / d->h_kv;
    const int64_t rows = group * l_ext;
    if (rows > INT32_MAX / 2)
        return fail(VA_ERR_SIZE, "rows per KV head (%lld) too large", (long long)rows);
    p.rows = (int32_t)rows;
    p.row_chunks = (int32_t)((rows + kRowChunk - 1) / kRowChunk);
    const int kv_elem_bytes = d->kv_dtype == VA_DTYPE_FP8_E4M3FN ? 1 : 2;
    p.tile_tokens = tile_tokens_for(d->head_dim, d->v_head_dim, kv_elem_bytes);
    const int64_t T = d->num_kv_indices;
    int64_t ranges;  // prefix workgroups per (KV head, row chunk)
    if (d->n_splits > 0) {
        p.mode = 1;
        p.n_splits = d->n_splits;
        ranges = (int64_t)d->bs * d->n_splits;
    } else if (d->split_tokens > 0) {
        // every prefix cut into ranges of exactly c tokens:
        // sum_b ceil(n_b / c) <= floor((T + bs * (c - 1)) / c)
        p.mode = 2;
        const int64_t c = d->split_tokens;
        p.split_tokens = (int32_t)c;
        ranges = (T + (int64_t)d->bs * (c - 1)) / c;
    } else {
        // One range per resident prefix workgroup, at least one per sequence
        // and (for short batches) no more than T / 64 rounded up: ranges are
        // at least kSplitQuantum tokens.  The count does not depend on T
        // beyond that cap, so a kv_indices buffer sized for the largest batch
        // (graph capture) keeps the full grid, and the workspace never
        // shrinks as T or bs grow.  The kernels fit the range size to the
        // lengths in kv_indptr on every launch.  split_tokens is only the
        // size T tokens in equal prefixes would get: the kernels' guess for
        // where each range starts, so that its first index copies can go out
        // before kv_indptr has been read.
        p.mode = 0;
        const int64_t units = (int64_t)d->h_kv * p.row_chunks;
        const int qb = query_blocks_for(rows < kRowChunk ? (int)rows : kRowChunk);
        const int64_t target = (int64_t)prefix_resident_per_cu(qb) * num_cus;
        int64_t c = (T * units + target - 1) / target;
        c = align_up(c < kSplitQuantum ? kSplitQuantum : c, kSplitQuantum);
        p.split_tokens = (int32_t)std::min<int64_t>(c, (int64_t)1 << 30);
        const int64_t resident = target / units;  // ranges per (KV head, row chunk) resident at once
        ranges = T > 0 ? std::max<int64_t>(std::min<int64_t>(resident, (T + kSplitQuantum - 1) / kSplitQuantum),
                                           d->bs)
                       : 0;
        if (d->bs > resident) {
            // More sequences than resident workgroups: the grid runs in rounds,
            // and with one range per sequence a ragged batch ends on a few long
            // sequences.  Allow ranges of about kRoundRangeBytes of K/V per KV
            // head, so that the dispatcher balances the rounds (mode 3: the
            // kernels keep whole sequences when the prefixes are near equal).
            p.mode = 3;
            const int64_t c_round = round_range_tokens(d->head_dim, d->v_head_dim, kv_elem_bytes);
            ranges = std::max<int64_t>(ranges, (T + c_round - 1) / c_round);
        }
    }
    p.range_slots = ranges;
    const int64_t slots = p.range_slots * d->h_kv;
    p.prefix_blocks = ranges * d->h_kv * p.row_chunks;
    // one wavefront per output row
    p.combine_blocks = ((int64_t)d->bs * d->h_kv * rows + kCombineRowsPerBlock - 1) / kCombineRowsPerBlock;
    if (p.prefix_blocks > INT32_MAX || p.combine_blocks > INT32_MAX || p.range_slots > INT32_MAX)
        return fail(VA_ERR_SIZE, "grid too large (%lld prefix workgroups)", (long long)p.prefix_blocks);
    const int64_t o_bytes = align_up(slots * rows * d->v_head_dim * 2, 256);  // bf16 partials
    const int64_t l_bytes = align_up(slots * rows * 4, 256);
    // each sequence's first range and range count (the prefix pass writes
    // them for the combine pass, which loads its sequence's entry
    // unconditionally, so the table is there even when no prefix pass runs)
    const int64_t t_bytes = align_up((int64_t)d->bs * 8, 256);
    p.partial_bytes = (size_t)o_bytes;
    p.table_offset = (size_t)(o_bytes + l_bytes);
    p.workspace_bytes = (size_t)(o_bytes + l_bytes + t_bytes);
    *plan = p;
    clear_error();
    return VA_OK;
}

}  // namespace va

extern "C" {

VA_API int verify_attn_check(const va_desc_t *desc, int32_t l_ext)
{
    return va::check_desc(desc, l_ext);
}

VA_API int verify_attn_plan(const va_desc_t *desc, int32_t l_ext, int32_t num_cus, va_plan_t *plan)
{
    return va::make_plan(desc, l_ext, num_cus, plan);
}

VA_API int verify_attn_workspace_bytes(const va_desc_t *desc, int32_t l_ext, int32_t num_cus,
                                       size_t *bytes)
{
    if (!bytes)
        return va::fail(VA_ERR_NULL_ARG, "bytes is NULL");
    va_plan_t p;
    int rc = va::make_plan(desc, l_ext, num_cus, &p);
    if (rc == VA_OK)
        *bytes = p.workspace_bytes;
    return rc;
}

VA_API const char *verify_attn_strerror(int code)
{
    switch (code) {
    case VA_OK: return "ok";
    case VA_ERR_NULL_ARG: return "required pointer is NULL";
    case VA_ERR_BATCH: return "batch size must be >= 1";
    case VA_ERR_HEADS: return "h_q must be a positive multiple of h_kv";
    case VA_ERR_HEAD_DIM: return "unsupported head dims (need both in {64,128,256}, equal or one twice the other)";
    case VA_ERR_DTYPE: return "unsupported pool dtype";
    case VA_ERR_EXTEND: return "l_ext < 1 or q_rows != bs * l_ext";
    case VA_ERR_STRIDE: return "invalid stride";
    case VA_ERR_SCALE: return "scales must be finite and > 0";
    case VA_ERR_WORKSPACE: return "workspace missing or too small";
    case VA_ERR_SPLIT: return "invalid split override";
    case VA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case VA_ERR_DEVICE: return "HIP runtime error";
    case VA_ERR_SIZE: return "size out of range";
    default: return "unknown status";
    }
}

VA_API const char *verify_attn_last_error(void) { return va::last_error(); }

VA_API int verify_attn_version(void) { return 300; }

}  // extern "C"
