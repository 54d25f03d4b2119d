// va_api.cpp -- C entry points that run the two passes on the caller's stream.
//
// The flow is the pages' VerifySplitKV.__call__ (sglang verify_splitkv.py):
// prefix pass into partials (bf16 normalised outputs, fp32 log-sum-exps; the
// pages keep fp32 outputs), then the fused combine / draft / merge pass.
// Differences: the partial buffer is the caller's workspace (the pages cache
// one per shape, sized by the largest batch), scales are host floats that are
// validated instead of silently replaced by 1.0, and failures are status codes
// instead of a False that sends the caller to another kernel.
#include <cmath>
#include <cstdint>

#include "va_internal.h"

namespace va {
namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_scales(float sm_scale, float k_scale, float v_scale)
{
    const float s[3] = {sm_scale, k_scale, v_scale};
    for (float x : s)
        if (!std::isfinite(x) || !(x > 0.0f)) {
            set_error("scales must be finite and > 0 (sm_scale=%g k_scale=%g v_scale=%g)",
                      (double)sm_scale, (double)k_scale, (double)v_scale);
            return VA_ERR_SCALE;
        }
    return VA_OK;
}

int check_ptrs(const void *const *ptrs, int n)
{
    for (int i = 0; i < n; ++i) {
        if (!ptrs[i]) {
            set_error("argument pointer %d is NULL", i);
            return VA_ERR_NULL_ARG;
        }
    }
    return VA_OK;
}

int check_align(const void *const *ptrs, int n)
{
    for (int i = 0; i < n; ++i)
        if (!aligned16(ptrs[i])) {
            set_error("tensor pointer %d is not 16-byte aligned", i);
            return VA_ERR_ALIGN;
        }
    return VA_OK;
}

int check_workspace(const va_plan_t &plan, const void *ws, size_t ws_bytes)
{
    if (plan.workspace_bytes == 0)
        return VA_OK;
    if (!ws || ws_bytes < plan.workspace_bytes) {
        set_error("workspace %p of %zu bytes; the plan needs %zu", ws, ws_bytes, plan.workspace_bytes);
        return VA_ERR_WORKSPACE;
    }
    if (((uintptr_t)ws & 255u) != 0) {
        set_error("workspace must be 256-byte aligned");
        return VA_ERR_ALIGN;
    }
    return VA_OK;
}

int prefix_impl(const void *q, const void *k_buf, const void *v_buf, const int32_t *qo_indptr,
                const int32_t *kv_indptr, const int64_t *kv_indices, int32_t l_ext, float sm_scale,
                float k_scale, float v_scale, const va_desc_t *desc, const va_plan_t &plan,
                void *workspace, void *stream, const int32_t *block_table = nullptr,
                int64_t bt_stride = 0, int32_t page_size = 1)
{
    if (plan.prefix_blocks == 0)
        return VA_OK;  // no prefix token anywhere: the combine pass sees zero ranges
    PrefixParams p;
    p.block_table = block_table;
    p.bt_s0 = bt_stride;
    p.page_size = page_size;
    p.q = (const uint16_t *)q;
    p.k_buf = (const uint8_t *)k_buf;
    p.v_buf = (const uint8_t *)v_buf;
    p.qo_indptr = qo_indptr;
    p.kv_indptr = kv_indptr;
    p.kv_indices = kv_indices;
    p.part_o = (uint16_t *)workspace;
    p.part_lse = (float *)((char *)workspace + plan.partial_bytes);
    p.seq_ranges = (int32_t *)((char *)workspace + plan.table_offset);
    const int eb = desc->kv_dtype == VA_DTYPE_FP8_E4M3FN ? 1 : 2;
    p.q_s0 = desc->q_stride[0];
    p.q_s1 = desc->q_stride[1];
    p.kb_s0 = (uint32_t)(desc->kbuf_stride[0] * eb);
    p.kb_s1 = desc->kbuf_stride[1] * eb;
    p.vb_s0 = (uint32_t)(desc->vbuf_stride[0] * eb);
    p.vb_s1 = desc->vbuf_stride[1] * eb;
    p.qk_scale_log2 = (float)((double)sm_scale * (double)k_scale * 1.4426950408889634);
    p.v_scale = v_scale;
    p.bs = desc->bs;
    p.h_kv = desc->h_kv;
    p.group = desc->h_q / desc->h_kv;
    p.l_ext = l_ext;
    p.rows = plan.rows;
    p.row_chunks = plan.row_chunks;
    p.mode = plan.mode;
    p.split_tokens = plan.split_tokens > 0 ? plan.split_tokens : 1;
    p.n_splits = plan.n_splits > 0 ? plan.n_splits : 1;
    p.total_tokens = (int32_t)desc->num_kv_indices;  // < 2^31, checked by the planner
    const int qb = query_blocks_for(plan.rows < kRowChunk ? plan.rows : kRowChunk);
    int e = launch_prefix(p, desc->head_dim, desc->v_head_dim, desc->kv_dtype == VA_DTYPE_FP8_E4M3FN, qb,
                          plan.prefix_blocks, stream);
    if (e != 0) {
        set_error("prefix kernel launch: %s", hip_error_string(e));
        return VA_ERR_DEVICE;
    }
    return VA_OK;
}

int combine_impl(const void *q, const void *k_ext, const void *v_ext, const int32_t *qo_indptr,
                 const int32_t *kv_indptr, int32_t l_ext, float sm_scale, void *out,
                 const va_desc_t *desc, const va_plan_t &plan, void *workspace, void *stream,
                 const uint8_t *mask = nullptr, const int64_t *mask_indptr = nullptr)
{
    CombineParams c;
    c.mask = mask;
    c.mask_indptr = mask_indptr;
    c.q = (const uint16_t *)q;
    c.k_ext = (const uint16_t *)k_ext;
    c.v_ext = (const uint16_t *)v_ext;
    c.qo_indptr = qo_indptr;
    c.kv_indptr = kv_indptr;
    c.part_o = (const uint16_t *)workspace;
    c.part_lse = (const float *)((const char *)workspace + plan.partial_bytes);
    c.seq_ranges = (const int32_t *)((const char *)workspace + plan.table_offset);
    c.out = (uint16_t *)out;
    c.q_s0 = desc->q_stride[0];
    c.q_s1 = desc->q_stride[1];
    c.ke_s0 = desc->kext_stride[0];
    c.ke_s1 = desc->kext_stride[1];
    c.ve_s0 = desc->vext_stride[0];
    c.ve_s1 = desc->vext_stride[1];
    c.o_s0 = desc->out_stride[0];
    c.o_s1 = desc->out_stride[1];
    c.sm_scale = sm_scale;
    c.bs = desc->bs;
    c.h_kv = desc->h_kv;
    c.group = desc->h_q / desc->h_kv;
    c.l_ext = l_ext;
    c.rows = plan.rows;
    c.mode = plan.mode;
    c.split_tokens = plan.split_tokens > 0 ? plan.split_tokens : 1;
    c.n_splits = plan.n_splits > 0 ? plan.n_splits : 1;
    // preload depths from static shapes: ranges per sequence the grid allows
    // on average (a batch may exceed it; the kernel then loops) and draft rows
    const int64_t per_seq = plan.mode == 1 ? plan.n_splits : (plan.range_slots + desc->bs - 1) / desc->bs;
    const int pre = per_seq <= 8 ? 8 : 32;
    const int pre_d = l_ext == 1 ? 1 : (l_ext <= 4 ? 4 : 8);
    int e = launch_combine(c, desc->head_dim, desc->v_head_dim, pre, pre_d, plan.combine_blocks, stream);
    if (e != 0) {
        set_error("combine kernel launch: %s", hip_error_string(e));
        return VA_ERR_DEVICE;
    }
    return VA_OK;
}

// Page-table arguments of the *_paged entry points.
int check_paged(const va_desc_t *desc, const int32_t *block_table, int64_t bt_stride, int32_t page_size)
{
    if (page_size < 1) {
        set_error("page_size = %d; need >= 1", page_size);
        return VA_ERR_SIZE;
    }
    if (bt_stride < 0) {
        set_error("block table stride %lld is negative", (long long)bt_stride);
        return VA_ERR_STRIDE;
    }
    if (desc->num_kv_indices > 0 && !block_table) {
        set_error("block_table is NULL");
        return VA_ERR_NULL_ARG;
    }
    return VA_OK;
}

// Tree-mask arguments of the *_tree entry points.
int check_tree(const uint8_t *mask, const int64_t *mask_indptr, int32_t l_ext)
{
    const void *ptrs[2] = {mask, mask_indptr};
    int rc = check_ptrs(ptrs, 2);
    if (rc != VA_OK)
        return rc;
    if (l_ext > kMaxTreeDrafts) {
        set_error("l_ext = %d; the tree-mask path takes at most %d draft tokens", l_ext, kMaxTreeDrafts);
        return VA_ERR_EXTEND;
    }
    return VA_OK;
}

}  // namespace
}  // namespace va

extern "C" {

VA_API int verify_attn_prefix(const void *q, const void *k_buf, const void *v_buf,
                              const int32_t *qo_indptr, const int32_t *kv_indptr,
                              const int64_t *kv_indices, int32_t l_ext, float sm_scale,
                              float k_scale, float v_scale, const va_desc_t *desc, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    int rc = va::check_desc(desc, l_ext);  // host checks first: no device query on bad input
    if (rc != VA_OK)
        return rc;
    // kv_indices may be NULL only when there is no prefix token at all
    const void *ptrs[6] = {q, k_buf, v_buf, qo_indptr, kv_indptr,
                           desc->num_kv_indices > 0 ? (const void *)kv_indices : (const void *)q};
    if ((rc = va::check_ptrs(ptrs, 6)) != VA_OK)
        return rc;
    const void *al[3] = {q, k_buf, v_buf};
    if ((rc = va::check_align(al, 3)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, k_scale, v_scale)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    return va::prefix_impl(q, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext, sm_scale,
                           k_scale, v_scale, desc, plan, workspace, stream);
}

VA_API int verify_attn_combine(const void *q, const void *k_ext, const void *v_ext,
                               const int32_t *qo_indptr, const int32_t *kv_indptr, int32_t l_ext,
                               float sm_scale, void *out, const va_desc_t *desc, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    int rc = va::check_desc(desc, l_ext);  // host checks first: no device query on bad input
    if (rc != VA_OK)
        return rc;
    const void *ptrs[6] = {q, k_ext, v_ext, qo_indptr, kv_indptr, out};
    if ((rc = va::check_ptrs(ptrs, 6)) != VA_OK)
        return rc;
    const void *al[4] = {q, k_ext, v_ext, out};
    if ((rc = va::check_align(al, 4)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, 1.0f, 1.0f)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    return va::combine_impl(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc, plan,
                            workspace, stream);
}

VA_API int verify_attn_run(const void *q, const void *k_ext, const void *v_ext, const void *k_buf,
                           const void *v_buf, const int32_t *qo_indptr, const int32_t *kv_indptr,
                           const int64_t *kv_indices, int32_t l_ext, float sm_scale, float k_scale,
                           float v_scale, void *out, const va_desc_t *desc, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    int rc = va::check_desc(desc, l_ext);  // host checks first: no device query on bad input
    if (rc != VA_OK)
        return rc;
    const void *ptrs[9] = {q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr,
                           desc->num_kv_indices > 0 ? (const void *)kv_indices : (const void *)q, out};
    if ((rc = va::check_ptrs(ptrs, 9)) != VA_OK)
        return rc;
    const void *al[6] = {q, k_ext, v_ext, k_buf, v_buf, out};
    if ((rc = va::check_align(al, 6)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, k_scale, v_scale)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    rc = va::prefix_impl(q, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext, sm_scale, k_scale,
                         v_scale, desc, plan, workspace, stream);
    if (rc != VA_OK)
        return rc;
    return va::combine_impl(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc, plan,
                            workspace, stream);
}

VA_API int verify_attn_run_noalloc(const void *q, const void *k_ext, const void *v_ext, const void *k_buf,
                                   const void *v_buf, const int32_t *qo_indptr, const int32_t *kv_indptr,
                                   const int64_t *kv_indices, int32_t l_ext, float sm_scale, float k_scale,
                                   float v_scale, void *out, const va_desc_t *desc, void *stream)
{
    int rc = va::check_desc(desc, l_ext);  // host checks first: no device query on bad input
    if (rc != VA_OK)
        return rc;
    const void *ptrs[9] = {q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr,
                           desc->num_kv_indices > 0 ? (const void *)kv_indices : (const void *)q, out};
    if ((rc = va::check_ptrs(ptrs, 9)) != VA_OK)
        return rc;
    const void *al[6] = {q, k_ext, v_ext, k_buf, v_buf, out};
    if ((rc = va::check_align(al, 6)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, k_scale, v_scale)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if (plan.workspace_bytes > va::kNoAllocScratchBytes) {
        va::set_error("the call needs %zu bytes of partials; verify_attn_run_noalloc holds at most %zu "
                      "(use verify_attn_run with a workspace)",
                      plan.workspace_bytes, va::kNoAllocScratchBytes);
        return VA_ERR_WORKSPACE;
    }
    void *ws = nullptr;
    if ((rc = va::noalloc_scratch(&ws)) != VA_OK)
        return rc;
    rc = va::prefix_impl(q, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext, sm_scale, k_scale,
                         v_scale, desc, plan, ws, stream);
    if (rc != VA_OK)
        return rc;
    return va::combine_impl(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc, plan, ws,
                            stream);
}

VA_API int verify_attn_combine_tree(const void *q, const void *k_ext, const void *v_ext,
                                    const int32_t *qo_indptr, const int32_t *kv_indptr, int32_t l_ext,
                                    float sm_scale, const uint8_t *custom_mask, const int64_t *mask_indptr,
                                    void *out, const va_desc_t *desc, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    int rc = va::check_desc(desc, l_ext);  // host checks first: no device query on bad input
    if (rc != VA_OK)
        return rc;
    const void *ptrs[6] = {q, k_ext, v_ext, qo_indptr, kv_indptr, out};
    if ((rc = va::check_ptrs(ptrs, 6)) != VA_OK)
        return rc;
    if ((rc = va::check_tree(custom_mask, mask_indptr, l_ext)) != VA_OK)
        return rc;
    const void *al[4] = {q, k_ext, v_ext, out};
    if ((rc = va::check_align(al, 4)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, 1.0f, 1.0f)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    return va::combine_impl(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc, plan,
                            workspace, stream, custom_mask, mask_indptr);
}

VA_API int verify_attn_run_tree(const void *q, const void *k_ext, const void *v_ext, const void *k_buf,
                                const void *v_buf, const int32_t *qo_indptr, const int32_t *kv_indptr,
                                const int64_t *kv_indices, int32_t l_ext, float sm_scale, float k_scale,
                                float v_scale, const uint8_t *custom_mask, const int64_t *mask_indptr,
                                void *out, const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                                void *stream)
{
    int rc = va::check_desc(desc, l_ext);  // host checks first: no device query on bad input
    if (rc != VA_OK)
        return rc;
    const void *ptrs[9] = {q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr,
                           desc->num_kv_indices > 0 ? (const void *)kv_indices : (const void *)q, out};
    if ((rc = va::check_ptrs(ptrs, 9)) != VA_OK)
        return rc;
    if ((rc = va::check_tree(custom_mask, mask_indptr, l_ext)) != VA_OK)
        return rc;
    const void *al[6] = {q, k_ext, v_ext, k_buf, v_buf, out};
    if ((rc = va::check_align(al, 6)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, k_scale, v_scale)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    rc = va::prefix_impl(q, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext, sm_scale, k_scale,
                         v_scale, desc, plan, workspace, stream);
    if (rc != VA_OK)
        return rc;
    return va::combine_impl(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc, plan,
                            workspace, stream, custom_mask, mask_indptr);
}

VA_API int verify_attn_prefix_paged(const void *q, const void *k_buf, const void *v_buf,
                                    const int32_t *qo_indptr, const int32_t *kv_indptr,
                                    const int32_t *block_table, int64_t block_table_stride,
                                    int32_t page_size, int32_t l_ext, float sm_scale, float k_scale,
                                    float v_scale, const va_desc_t *desc, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    int rc = va::check_desc(desc, l_ext);
    if (rc != VA_OK)
        return rc;
    const void *ptrs[5] = {q, k_buf, v_buf, qo_indptr, kv_indptr};
    if ((rc = va::check_ptrs(ptrs, 5)) != VA_OK)
        return rc;
    if ((rc = va::check_paged(desc, block_table, block_table_stride, page_size)) != VA_OK)
        return rc;
    const void *al[3] = {q, k_buf, v_buf};
    if ((rc = va::check_align(al, 3)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, k_scale, v_scale)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    return va::prefix_impl(q, k_buf, v_buf, qo_indptr, kv_indptr, nullptr, l_ext, sm_scale, k_scale,
                           v_scale, desc, plan, workspace, stream, block_table, block_table_stride,
                           page_size);
}

VA_API int verify_attn_run_paged(const void *q, const void *k_ext, const void *v_ext, const void *k_buf,
                                 const void *v_buf, const int32_t *qo_indptr, const int32_t *kv_indptr,
                                 const int32_t *block_table, int64_t block_table_stride, int32_t page_size,
                                 int32_t l_ext, float sm_scale, float k_scale, float v_scale, void *out,
                                 const va_desc_t *desc, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    int rc = va::check_desc(desc, l_ext);
    if (rc != VA_OK)
        return rc;
    const void *ptrs[8] = {q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, out};
    if ((rc = va::check_ptrs(ptrs, 8)) != VA_OK)
        return rc;
    if ((rc = va::check_paged(desc, block_table, block_table_stride, page_size)) != VA_OK)
        return rc;
    const void *al[6] = {q, k_ext, v_ext, k_buf, v_buf, out};
    if ((rc = va::check_align(al, 6)) != VA_OK)
        return rc;
    if ((rc = va::check_scales(sm_scale, k_scale, v_scale)) != VA_OK)
        return rc;
    va_plan_t plan;
    if ((rc = va::make_plan(desc, l_ext, 0, &plan)) != VA_OK)
        return rc;
    if ((rc = va::check_workspace(plan, workspace, workspace_bytes)) != VA_OK)
        return rc;
    rc = va::prefix_impl(q, k_buf, v_buf, qo_indptr, kv_indptr, nullptr, l_ext, sm_scale, k_scale, v_scale,
                         desc, plan, workspace, stream, block_table, block_table_stride, page_size);
    if (rc != VA_OK)
        return rc;
    return va::combine_impl(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc, plan,
                            workspace, stream);
}

}  // extern "C"
