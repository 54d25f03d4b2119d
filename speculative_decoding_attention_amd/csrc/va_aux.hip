// va_aux.hip -- gfx950 kernels around the verify attention: the draft K/V
// append into the paged pool (with the bf16 -> E4M3FN quantization of an fp8
// pool) and the kv_indices build from the request-to-token table.
//
// Append (sglang aiter_backend.py: set_kv_buffer, and
// launch_reshape_and_cache_flash, which fuses the fp8 cast with the paged
// write): one wavefront per (token, KV head) row; the K row and the V row are
// each read once (16-bit lanes) and written once to pool row out_cache_loc[i].
// An fp8 pool stores the E4M3FN code of x / scale: the quotient is one
// correctly rounded fp32 division, v_cvt_pk_fp8_f32 rounds it to nearest even
// on the OCP grid, and a clamp to +-448 first makes the cast saturate (the
// instruction alone turns overflow into NaN).  A bf16 pool receives the bits.
//
// kv_indices build (create_flashinfer_kv_indices_triton as aiter_backend.py
// calls it, with kv_indptr the running sum of the request lengths): request b
// copies req_to_token[req_pool_indices[b], start_b + i] for i < seq_lens[b] to
// kv_indices[kv_indptr[b] + i] (int32 -> int64); each workgroup of a request
// forms kv_indptr[b] itself from seq_lens[0..b), so one launch writes both.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "va_internal.h"

namespace va {

namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float clamp_e4m3_range(float x)
{
    return x != x ? x : fminf(fmaxf(x, -448.0f), 448.0f);
}

// 4 bf16 values (one 8-byte lane load) -> 4 E4M3FN codes of x / scale
__device__ __forceinline__ uint32_t quantize4(uint32_t lo, uint32_t hi, float scale)
{
    const float x0 = clamp_e4m3_range(__fdiv_rn(bf16_bits_to_f32(lo & 0xffffu), scale));
    const float x1 = clamp_e4m3_range(__fdiv_rn(bf16_bits_to_f32(lo >> 16), scale));
    const float x2 = clamp_e4m3_range(__fdiv_rn(bf16_bits_to_f32(hi & 0xffffu), scale));
    const float x3 = clamp_e4m3_range(__fdiv_rn(bf16_bits_to_f32(hi >> 16), scale));
    const int d = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, d, true);
}

__device__ __forceinline__ float quantize1(uint32_t h, float scale)
{
    return clamp_e4m3_range(__fdiv_rn(bf16_bits_to_f32(h), scale));
}

// one row of D elements: bf16 source, bf16 or fp8 destination; lane covers
// D / 64 consecutive elements
template <int D, bool FP8>
__device__ __forceinline__ void append_row(const uint16_t *src, uint8_t *dst, float scale, int lane)
{
    constexpr int VPL = D / 64;
    const int c0 = lane * VPL;
    if constexpr (VPL == 4) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t w = *(const u32x2_t *)(src + c0);
        if constexpr (FP8)
            *(uint32_t *)(dst + c0) = quantize4(w[0], w[1], scale);
        else
            *(u32x2_t *)(dst + 2 * c0) = w;
    } else if constexpr (VPL == 2) {
        const uint32_t w = *(const uint32_t *)(src + c0);
        if constexpr (FP8) {
            const int d = __builtin_amdgcn_cvt_pk_fp8_f32(quantize1(w & 0xffffu, scale), quantize1(w >> 16, scale),
                                                          0, false);
            *(uint16_t *)(dst + c0) = (uint16_t)(d & 0xffff);
        } else {
            *(uint32_t *)(dst + 2 * c0) = w;
        }
    } else {
        const uint16_t h = src[c0];
        if constexpr (FP8)
            dst[c0] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(quantize1(h, scale), 0.0f, 0, false) & 0xff);
        else
            *(uint16_t *)(dst + 2 * c0) = h;
    }
}

template <int D, int DV, bool FP8>
__global__ __launch_bounds__(kAuxThreads) void append_kernel(const AppendParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kAuxThreads / 64) + (threadIdx.x >> 6);
    if (row >= p.n * p.h_kv)
        return;  // padding wave of the last workgroup
    const int64_t i = row / p.h_kv;
    const int g = (int)(row % p.h_kv);
    const int64_t t = p.loc[i];
    append_row<D, FP8>(p.k + i * p.k_s0 + (int64_t)g * p.k_s1, p.k_buf + t * p.kb_s0 + (int64_t)g * p.kb_s1,
                       p.k_scale, lane);
    append_row<DV, FP8>(p.v + i * p.v_s0 + (int64_t)g * p.v_s1, p.v_buf + t * p.vb_s0 + (int64_t)g * p.vb_s1,
                        p.v_scale, lane);
}

// grid: bs * parts workgroups; part q of request b copies tokens q, q + parts *
// kAuxThreads, ... in blocks of kAuxThreads
__global__ __launch_bounds__(kAuxThreads) void build_kv_indices_kernel(const BuildIndicesParams p)
{
    __shared__ int64_t s_part[kAuxThreads / 64];
    const int b = (int)(blockIdx.x / p.parts);
    const int part = (int)(blockIdx.x % p.parts);
    // kv_indptr[b] = sum of seq_lens[0..b)
    int64_t acc = 0;
    for (int j = threadIdx.x; j < b; j += kAuxThreads)
        acc += p.seq_lens[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0)
        s_part[threadIdx.x >> 6] = acc;
    __syncthreads();
    int64_t base = 0;
#pragma unroll
    for (int w = 0; w < kAuxThreads / 64; ++w)
        base += s_part[w];
    const int32_t n = p.seq_lens[b];
    if (part == 0 && threadIdx.x == 0) {
        if (b == 0)
            p.kv_indptr[0] = 0;
        p.kv_indptr[b + 1] = (int32_t)(base + n);
    }
    const int32_t *src = p.req_to_token + p.req_pool_indices[b] * p.rt_stride + (p.kv_start_idx ? p.kv_start_idx[b] : 0);
    for (int64_t i = (int64_t)part * kAuxThreads + threadIdx.x; i < n; i += (int64_t)p.parts * kAuxThreads) {
        const int64_t o = base + i;
        if (o < p.capacity)  // never write past the caller's kv_indices
            p.kv_indices[o] = (int64_t)src[i];
    }
}

}  // namespace

int launch_append(const AppendParams &p, int head_dim, int v_head_dim, bool kv_fp8, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const int64_t rows = p.n * p.h_kv;
    dim3 grid((unsigned)((rows + kAuxThreads / 64 - 1) / (kAuxThreads / 64))), block(kAuxThreads);
#define VA_APPEND(D, DV)                                                               \
    if (kv_fp8)                                                                        \
        hipLaunchKernelGGL((append_kernel<D, DV, true>), grid, block, 0, s, p);        \
    else                                                                               \
        hipLaunchKernelGGL((append_kernel<D, DV, false>), grid, block, 0, s, p);
    // the head-dim pairs of the verify kernels (the host checks)
    switch (head_dim * 1000 + v_head_dim) {
    case 64064: VA_APPEND(64, 64) break;
    case 64128: VA_APPEND(64, 128) break;
    case 128064: VA_APPEND(128, 64) break;
    case 128128: VA_APPEND(128, 128) break;
    case 128256: VA_APPEND(128, 256) break;
    case 256128: VA_APPEND(256, 128) break;
    case 256256: VA_APPEND(256, 256) break;
    default: return (int)hipErrorInvalidValue;
    }
#undef VA_APPEND
    return (int)hipGetLastError();
}

int launch_build_kv_indices(const BuildIndicesParams &p, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((unsigned)((int64_t)p.bs * p.parts)), block(kAuxThreads);
    hipLaunchKernelGGL(build_kv_indices_kernel, grid, block, 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace va
