// va_aux_api.cpp -- C entry points of the draft K/V append and the kv_indices
// build (kernels in va_aux.hip).  Host-side validation of shapes, strides and
// scalars only; device data (locations, table entries) is not inspected.
#include <cmath>
#include <cstdint>

#include "va_internal.h"

extern "C" {

VA_API int verify_attn_append_kv(const void *k, const void *v, const int64_t *out_cache_loc,
                                 int64_t n_tokens, float k_scale, float v_scale, void *k_buf, void *v_buf,
                                 const va_desc_t *desc, void *stream)
{
    using namespace va;
    if (!desc) {
        set_error("descriptor is NULL");
        return VA_ERR_NULL_ARG;
    }
    if (desc->h_kv < 1) {
        set_error("h_kv = %d", desc->h_kv);
        return VA_ERR_HEADS;
    }
    const int d = desc->head_dim, dv = desc->v_head_dim;
    if (!supported_head_dims(d, dv)) {
        set_error("head_dim = %d, v_head_dim = %d; supported: both in {64,128,256}, equal or one twice the other",
                  d, dv);
        return VA_ERR_HEAD_DIM;
    }
    if (desc->kv_dtype != VA_DTYPE_BF16 && desc->kv_dtype != VA_DTYPE_FP8_E4M3FN) {
        set_error("kv_dtype = %d is not a va_dtype_t", desc->kv_dtype);
        return VA_ERR_DTYPE;
    }
    if (n_tokens < 0) {
        set_error("n_tokens = %lld is negative", (long long)n_tokens);
        return VA_ERR_SIZE;
    }
    const bool fp8 = desc->kv_dtype == VA_DTYPE_FP8_E4M3FN;
    if (fp8 && (!std::isfinite(k_scale) || !(k_scale > 0.0f) || !std::isfinite(v_scale) || !(v_scale > 0.0f))) {
        set_error("scales must be finite and > 0 (k_scale=%g v_scale=%g)", (double)k_scale, (double)v_scale);
        return VA_ERR_SCALE;
    }
    const int eb = fp8 ? 1 : 2;
    const int64_t *s4[4] = {desc->kext_stride, desc->vext_stride, desc->kbuf_stride, desc->vbuf_stride};
    const int es[4] = {2, 2, eb, eb};
    for (int i = 0; i < 4; ++i)
        if (s4[i][0] < 0 || s4[i][1] < 0 || (s4[i][0] * es[i]) % 16 != 0 || (s4[i][1] * es[i]) % 16 != 0) {
            set_error("every row and head stride must be non-negative and a multiple of 16 bytes");
            return VA_ERR_STRIDE;
        }
    if (n_tokens == 0)
        return VA_OK;
    if (!k || !v || !out_cache_loc || !k_buf || !v_buf) {
        set_error("a tensor pointer is NULL");
        return VA_ERR_NULL_ARG;
    }
    const void *al[4] = {k, v, k_buf, v_buf};
    for (const void *p : al)
        if (((uintptr_t)p & 15u) != 0) {
            set_error("tensor pointer not 16-byte aligned");
            return VA_ERR_ALIGN;
        }
    if (n_tokens * desc->h_kv > (int64_t)INT32_MAX * 4) {
        set_error("n_tokens too large");
        return VA_ERR_SIZE;
    }
    AppendParams p;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.loc = out_cache_loc;
    p.k_buf = (uint8_t *)k_buf;
    p.v_buf = (uint8_t *)v_buf;
    p.n = n_tokens;
    p.h_kv = desc->h_kv;
    p.k_s0 = desc->kext_stride[0];
    p.k_s1 = desc->kext_stride[1];
    p.v_s0 = desc->vext_stride[0];
    p.v_s1 = desc->vext_stride[1];
    p.kb_s0 = desc->kbuf_stride[0] * eb;
    p.kb_s1 = desc->kbuf_stride[1] * eb;
    p.vb_s0 = desc->vbuf_stride[0] * eb;
    p.vb_s1 = desc->vbuf_stride[1] * eb;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    const int e = launch_append(p, d, dv, fp8, stream);
    if (e != 0) {
        set_error("append kernel launch: %s", hip_error_string(e));
        return VA_ERR_DEVICE;
    }
    clear_error();
    return VA_OK;
}

VA_API int verify_attn_build_kv_indices(const int32_t *req_to_token, int64_t req_to_token_stride,
                                        const int64_t *req_pool_indices, const int32_t *seq_lens,
                                        const int32_t *kv_start_idx, int32_t bs, int64_t capacity,
                                        int32_t *kv_indptr, int64_t *kv_indices, void *stream)
{
    using namespace va;
    if (bs < 1) {
        set_error("bs = %d; need at least one request", bs);
        return VA_ERR_BATCH;
    }
    if (req_to_token_stride < 0 || capacity < 0) {
        set_error("negative stride or capacity");
        return VA_ERR_SIZE;
    }
    if (!req_to_token || !req_pool_indices || !seq_lens || !kv_indptr || (capacity > 0 && !kv_indices)) {
        set_error("a required pointer is NULL");
        return VA_ERR_NULL_ARG;
    }
    BuildIndicesParams p;
    p.req_to_token = req_to_token;
    p.rt_stride = req_to_token_stride;
    p.req_pool_indices = req_pool_indices;
    p.seq_lens = seq_lens;
    p.kv_start_idx = kv_start_idx;
    p.kv_indptr = kv_indptr;
    p.kv_indices = kv_indices;
    p.capacity = capacity;
    p.bs = bs;
    // enough workgroups per request to spread long requests over the CUs
    int64_t parts = (capacity + (int64_t)bs * 4096 - 1) / ((int64_t)bs * 4096);
    p.parts = (int32_t)(parts < 1 ? 1 : (parts > 64 ? 64 : parts));
    if ((int64_t)bs * p.parts > INT32_MAX) {
        set_error("bs too large");
        return VA_ERR_SIZE;
    }
    const int e = launch_build_kv_indices(p, stream);
    if (e != 0) {
        set_error("kv_indices kernel launch: %s", hip_error_string(e));
        return VA_ERR_DEVICE;
    }
    clear_error();
    return VA_OK;
}

}  // extern "C"
