// va_kernels.hip -- gfx950 kernels of split-KV target-verify attention.
//
// Prefix kernel (the pages' _verify_prefix_stage1, sglang verify_splitkv.py):
// one workgroup of 4 wavefronts per (prefix range, KV head, row chunk).  All
// query rows that share a KV head -- the GQA group times the l_ext draft rows
// -- form one tile of up to 64 rows, so every K/V byte of the range is read
// from HBM once for the whole group (the pages launch one program per query
// head and re-read the range per head).  K/V rows are gathered through
// kv_indices with 16-byte coalesced loads into registers one tile ahead,
// converted to bf16 if the pool is fp8, and staged in double-buffered LDS.
// Scores S^T = K Q^T and the update O^T += V^T P^T run on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the softmax is the online
// (running max / running sum) recurrence of the pages, in base 2.  k_scale is
// folded into the score scale; v_scale multiplies the range's output.
//
// Combine kernel (the pages' _verify_combine_stage2): one wavefront per
// (sequence, KV head, query row): log-sum-exp merge of the ranges, the causal
// draft block in fp32 (no pool cast, no scales), the final two-way merge and a
// round-to-nearest-even bf16 store.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "va_internal.h"

namespace va {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ conversions ---
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// OCP E4M3FN byte -> bf16 bits (exact: every E4M3FN value is a bf16 value).
// Exponent field e >= 1: 2^(e-7) * (1 + m/8) -> bf16 exponent e + 120.
// e == 0: subnormal m * 2^-9.  0x7f / 0xff: NaN.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t b)
{
    const uint32_t em = b & 0x7fu;
    uint32_t r = (em >= 8u) ? (em << 4) + 0x3c00u
                            : (__float_as_uint((float)em * 0x1p-9f) >> 16);
    r = (em == 0x7fu) ? 0x7fc0u : r;
    return ((b & 0x80u) << 8) | r;
}

// Round a real to the nearest E4M3FN value (ties to even), saturating at
// +-448.  Grid spacing is 2^(k-3) in [2^k, 2^(k+1)), 2^-9 below 2^-6.
__device__ __forceinline__ float round_to_e4m3(float x)
{
    const float a = fabsf(x);
    if (a != a)
        return x;
    float r;
    if (!(a < 448.0f)) {
        r = 448.0f;
    } else if (a < 0x1p-6f) {
        r = rintf(a * 512.0f) * 0x1p-9f;
    } else {
        int e;
        frexpf(a, &e);  // a = f * 2^e, f in [0.5, 1): binade k = e - 1
        r = ldexpf(rintf(ldexpf(a, 4 - e)), e - 4);
    }
    return copysignf(r, x);
}

__device__ __forceinline__ u32x4_t fp8x16_to_bf16_lo(u32x4_t v)
{
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t x = v[w];
        o[2 * w + 0] = e4m3_to_bf16(x & 0xffu) | (e4m3_to_bf16((x >> 8) & 0xffu) << 16);
        o[2 * w + 1] = e4m3_to_bf16((x >> 16) & 0xffu) | (e4m3_to_bf16(x >> 24) << 16);
    }
    return o;
}

__device__ __forceinline__ u32x4_t fp8x16_to_bf16_hi(u32x4_t v)
{
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t x = v[2 + w];
        o[2 * w + 0] = e4m3_to_bf16(x & 0xffu) | (e4m3_to_bf16((x >> 8) & 0xffu) << 16);
        o[2 * w + 1] = e4m3_to_bf16((x >> 16) & 0xffu) | (e4m3_to_bf16(x >> 24) << 16);
    }
    return o;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ range lookup ---
// Ranges of the batch are numbered sequence by sequence.  Mode 0: sequence b
// owns ceil(n_b / split_tokens) ranges of split_tokens tokens (the last one
// shorter).  Mode 1 (the pages' rule): n_splits ranges of
// ceil(ceil(n_b / n_splits) / 32) * 32 tokens, empty past the end.
struct Range {
    int32_t b;
    int32_t start;
    int32_t end;
    bool valid;
};

// Number of mode-0 ranges of sequences [0, b_end), and the whole-wave lookup
// of the sequence that owns range `target` (both use the same wave scan).
__device__ __forceinline__ Range locate_range(const int32_t *kv_indptr, int32_t bs, int32_t mode,
                                              int32_t split_tokens, int32_t n_splits,
                                              int64_t cidx)
{
    Range r = {0, 0, 0, false};
    if (mode == 1) {
        const int64_t b = cidx / n_splits;
        if (b >= bs)
            return r;
        const int32_t s = (int32_t)(cidx % n_splits);
        const int32_t n = kv_indptr[b + 1] - kv_indptr[b];
        const int32_t per = ((n + n_splits - 1) / n_splits + kEvenSplitGranule - 1) /
                            kEvenSplitGranule * kEvenSplitGranule;
        r.b = (int32_t)b;
        r.start = s * per;
        r.end = min(r.start + per, n);
        r.valid = true;
        return r;
    }
    const int lane = threadIdx.x & 63;
    int64_t cum = 0;
    for (int32_t b0 = 0; b0 < bs; b0 += 64) {
        const int32_t b = b0 + lane;
        const int32_t n = b < bs ? kv_indptr[b + 1] - kv_indptr[b] : 0;
        const int32_t nch = (n + split_tokens - 1) / split_tokens;
        int32_t incl = nch;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(incl, off);
            if (lane >= off)
                incl += y;
        }
        const int32_t total = __shfl(incl, 63);
        if (cidx < cum + total) {
            const uint64_t hit = __ballot(cum + incl > cidx);
            const int first = __ffsll((unsigned long long)hit) - 1;
            const int32_t excl = __shfl(incl - nch, first);
            const int32_t nf = __shfl(n, first);
            const int32_t c = (int32_t)(cidx - cum - excl);
            r.b = b0 + first;
            r.start = c * split_tokens;
            r.end = min(r.start + split_tokens, nf);
            r.valid = true;
            return r;
        }
        cum += total;
    }
    return r;
}

// First range index and range count of sequence b (whole-wave call).
__device__ __forceinline__ void ranges_of(const int32_t *kv_indptr, int32_t bs, int32_t mode,
                                          int32_t split_tokens, int32_t n_splits, int32_t b,
                                          int32_t *base, int32_t *count)
{
    if (mode == 1) {
        *base = b * n_splits;
        *count = n_splits;
        return;
    }
    const int lane = threadIdx.x & 63;
    int32_t acc = 0;
    for (int32_t b0 = 0; b0 < b; b0 += 64) {
        const int32_t bb = b0 + lane;
        const int32_t n = bb < b ? kv_indptr[bb + 1] - kv_indptr[bb] : 0;
        int32_t nch = (n + split_tokens - 1) / split_tokens;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            nch += __shfl_xor(nch, off);
        acc += nch;
    }
    const int32_t n = kv_indptr[b + 1] - kv_indptr[b];
    *base = acc;
    *count = (n + split_tokens - 1) / split_tokens;
}

// ----------------------------------------------------------- prefix kernel ---
// LDS tile layouts (bf16 rows of D elements, 16-byte chunks):
//   K: chunk c of token row t lives at chunk c ^ (t & 7) -- the score MFMA
//      reads 16 consecutive rows at one chunk, which this spreads over banks;
//   V: chunk c of token row t lives at chunk c ^ (((t >> 2) & 3) << 1) -- the
//      transposed 16-bit reads of the value MFMA touch rows 4 apart.
// P tile: for value step ks (32 tokens) and row block rb, lane l's 8 bf16
// B-operand values sit at ((ks * MB + rb) * 64 + l) * 16.
template <bool FP8, int D, int MB>
__global__ __launch_bounds__(kThreads) void prefix_kernel(const PrefixParams p)
{
    constexpr int TN = tile_tokens_for(D);
    constexpr int E = FP8 ? 1 : 2;          // pool bytes per element
    constexpr int GCH = D * E / 16;         // 16-byte chunks per pool row
    constexpr int ROWB = D * 2;             // LDS bytes per bf16 row
    constexpr int CPT = TN * GCH / kThreads;  // staged chunks per thread per tile
    constexpr int RSTEP = kThreads / GCH;   // row step between a thread's chunks
    constexpr int NTB = TN / 16;            // 16-token score blocks per tile
    constexpr int NKS_QK = D / 32;          // k-steps of the score MFMA
    constexpr int NKS_PV = TN / 32;         // k-steps of the value MFMA
    constexpr int NP = NTB * MB;            // score blocks per tile
    constexpr int PPW = NP >= 4 ? NP / 4 : 1;  // score blocks per wave
    constexpr int QKW = NP >= 4 ? 4 : NP;   // waves that compute scores
    constexpr int DW = D / 4;               // output columns per wave
    constexpr int DB = DW / 16;             // 16-column blocks per wave
    static_assert(CPT >= 1 && CPT * kThreads == TN * GCH, "tile/thread mismatch");
    static_assert(MB == 1 || MB == 2 || MB == 4, "row blocks");

    __shared__ __attribute__((aligned(16))) uint8_t s_k[2][TN * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[2][TN * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[NKS_PV * MB * 64 * 16];
    __shared__ float s_max[4][16];
    __shared__ float s_sum[4][16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // ---- work item: (range, KV head, row chunk) ----
    const int64_t blk = blockIdx.x;
    const int rc = (int)(blk % p.row_chunks);
    const int64_t t1 = blk / p.row_chunks;
    const int kvh = (int)(t1 % p.h_kv);
    const int64_t cidx = t1 / p.h_kv;
    const Range rg = locate_range(p.kv_indptr, p.bs, p.mode, p.split_tokens, p.n_splits, cidx);
    if (!rg.valid)
        return;  // surplus slot of the static grid: never read by the combine pass
    const int64_t slot = cidx * p.h_kv + kvh;
    const int rows = p.rows;
    const int row0 = rc * kRowChunk;
    float *po = p.part_o + slot * (int64_t)rows * D;
    float *pl = p.part_lse + slot * (int64_t)rows;

    if (rg.start >= rg.end) {
        // Empty range: output 0 and log-sum-exp -inf, so the merge weight is
        // exactly 0 and no stale value can leak in.
        const int nr = min(rows - row0, MB * 16);
        for (int e = tid; e < nr * D; e += kThreads)
            po[(int64_t)(row0 + e / D) * D + (e % D)] = 0.0f;
        if (tid < nr)
            pl[row0 + tid] = -INFINITY;
        return;
    }

    const int64_t kv0 = (int64_t)p.kv_indptr[rg.b] + rg.start;
    const int len = rg.end - rg.start;
    const int nt = (len + TN - 1) / TN;
    const int qo = p.qo_indptr[rg.b];

    // ---- this wave's score blocks and its query operand ----
    const int pair0 = wave * PPW;
    const int rbw = pair0 / NTB;  // row block of this wave's score blocks
    const int tb0 = pair0 % NTB;  // first token block
    const bool qk_active = wave < QKW;
    bf16x8_t qreg[NKS_QK];
    {
        const int r = row0 + rbw * 16 + col;
        const bool rv = qk_active && r < rows;
        const int hg = rv ? r / p.l_ext : 0;
        const int di = rv ? r % p.l_ext : 0;
        const uint16_t *qrow = p.q + (int64_t)(qo + di) * p.q_s0 + (int64_t)(kvh * p.group + hg) * p.q_s1;
#pragma unroll
        for (int ks = 0; ks < NKS_QK; ++ks) {
            u32x4_t raw = {0u, 0u, 0u, 0u};
            if (rv)
                raw = *(const u32x4_t *)(qrow + ks * 32 + grp * 8);
            if (FP8) {
                // the prefix dot product uses q rounded to the pool dtype
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t lo = f32_to_bf16_rne(round_to_e4m3(bf16_to_f32(raw[w] & 0xffffu)));
                    const uint32_t hi = f32_to_bf16_rne(round_to_e4m3(bf16_to_f32(raw[w] >> 16)));
                    raw[w] = lo | (hi << 16);
                }
            }
            qreg[ks] = as_bf16x8(raw);
        }
    }

    // ---- staging: this thread's rows and chunk of every tile ----
    const int s_ch = tid % GCH;
    const int s_row0 = tid / GCH;
    const uint8_t *kbase = p.k_buf + (int64_t)kvh * p.kb_s1 + s_ch * 16;
    const uint8_t *vbase = p.v_buf + (int64_t)kvh * p.vb_s1 + s_ch * 16;
    u32x4_t stk[CPT], stv[CPT];
    int64_t sidx[CPT];

    auto load_idx = [&](int t) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int tok = t * TN + s_row0 + j * RSTEP;
            sidx[j] = (t < nt && tok < len) ? p.kv_indices[kv0 + tok] : -1;
        }
    };
    auto load_data = [&]() {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if (sidx[j] >= 0) {
                stk[j] = *(const u32x4_t *)(kbase + sidx[j] * p.kb_s0);
                stv[j] = *(const u32x4_t *)(vbase + sidx[j] * p.vb_s0);
            } else {
                stk[j] = u32x4_t{0u, 0u, 0u, 0u};
                stv[j] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int row = s_row0 + j * RSTEP;
            uint8_t *kr = s_k[buf] + row * ROWB;
            uint8_t *vr = s_v[buf] + row * ROWB;
            const int kz = row & 7;
            const int vz = ((row >> 2) & 3) << 1;
            if (FP8) {
                const int c0 = 2 * s_ch, c1 = 2 * s_ch + 1;
                *(u32x4_t *)(kr + ((c0 ^ kz) << 4)) = fp8x16_to_bf16_lo(stk[j]);
                *(u32x4_t *)(kr + ((c1 ^ kz) << 4)) = fp8x16_to_bf16_hi(stk[j]);
                *(u32x4_t *)(vr + ((c0 ^ vz) << 4)) = fp8x16_to_bf16_lo(stv[j]);
                *(u32x4_t *)(vr + ((c1 ^ vz) << 4)) = fp8x16_to_bf16_hi(stv[j]);
            } else {
                *(u32x4_t *)(kr + ((s_ch ^ kz) << 4)) = stk[j];
                *(u32x4_t *)(vr + ((s_ch ^ vz) << 4)) = stv[j];
            }
        }
    };

    // ---- running softmax state (lane's row in each row block: 16*rb + col) ----
    float m_run[MB], l_run[MB];
    f32x4_t oacc[DB][MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            oacc[db][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // prologue: tile 0 into LDS, tile 1 in flight, indices of tile 2 loaded
    load_idx(0);
    load_data();
    store_tile(0);
    load_idx(1);
    load_data();
    load_idx(2);
    __syncthreads();

    const float qk_scale = p.qk_scale_log2;
    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        const uint8_t *K = s_k[buf];
        const uint8_t *V = s_v[buf];

        // ---- scores of this wave's blocks: S^T[token][row] ----
        f32x4_t sc[PPW];
        if (qk_active) {
            float lmax = -INFINITY;
#pragma unroll
            for (int pp = 0; pp < PPW; ++pp) {
                const int tb = tb0 + pp;
                const int krow = tb * 16 + col;
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS_QK; ++ks) {
                    const int ch = (ks * 4 + grp) ^ (krow & 7);
                    const u32x4_t a = *(const u32x4_t *)(K + krow * ROWB + (ch << 4));
                    acc = mfma16x16x32(as_bf16x8(a), qreg[ks], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = t * TN + tb * 16 + grp * 4 + i;
                    const float v = tok < len ? acc[i] * qk_scale : -INFINITY;
                    acc[i] = v;
                    lmax = fmaxf(lmax, v);
                }
                sc[pp] = acc;
            }
            lmax = fmaxf(lmax, __shfl_xor(lmax, 16));
            lmax = fmaxf(lmax, __shfl_xor(lmax, 32));
            if (grp == 0)
                s_max[wave][col] = lmax;
        }
        __syncthreads();

        // ---- tile max per row, running-state rescale factors ----
        float alpha[MB];
        float m_w = 0.0f;  // new running max of this wave's score row block
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            float mt = -INFINITY;
#pragma unroll
            for (int w = 0; w < QKW; ++w)
                if ((w * PPW) / NTB == rb)
                    mt = fmaxf(mt, s_max[w][col]);
            const float mn = fmaxf(m_run[rb], mt);
            alpha[rb] = exp2f(m_run[rb] - mn);
            m_run[rb] = mn;
            if (rb == rbw)
                m_w = mn;
        }

        // ---- probabilities (bf16) into LDS, partial row sums ----
        if (qk_active) {
            float lsum = 0.0f;
#pragma unroll
            for (int pp = 0; pp < PPW; ++pp) {
                const int tb = tb0 + pp;
                uint32_t h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h[i] = f32_to_bf16_rne(exp2f(sc[pp][i] - m_w));
                    lsum += bf16_to_f32(h[i]);
                }
                const u32x2_t w2 = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                *(u32x2_t *)(s_p + (((tb >> 1) * MB + rbw) * 64 + lane) * 16 + (tb & 1) * 8) = w2;
            }
            lsum += __shfl_xor(lsum, 16);
            lsum += __shfl_xor(lsum, 32);
            if (grp == 0)
                s_sum[wave][col] = lsum;
        }
        __syncthreads();

        // ---- O^T[dv][row] = alpha * O^T + V^T P^T over this wave's columns ----
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            float ts = 0.0f;
#pragma unroll
            for (int w = 0; w < QKW; ++w)
                if ((w * PPW) / NTB == rb)
                    ts += s_sum[w][col];
            l_run[rb] = l_run[rb] * alpha[rb] + ts;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db][rb] *= alpha[rb];
        }
#pragma unroll
        for (int ks = 0; ks < NKS_PV; ++ks) {
            bf16x8_t pb[MB];
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
                pb[rb] = as_bf16x8(*(const u32x4_t *)(s_p + ((ks * MB + rb) * 64 + lane) * 16));
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dv = wave * DW + db * 16 + col;
                const int cch = dv >> 3;
                const int cin = (dv & 7) * 2;
                uint32_t w4[4];
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {
                    uint32_t pair = 0;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int i = 2 * i2 + hh;
                        const int tok = ks * 32 + (i >> 2) * 16 + grp * 4 + (i & 3);
                        const int pc = cch ^ (((tok >> 2) & 3) << 1);
                        const uint32_t v = *(const uint16_t *)(V + tok * ROWB + (pc << 4) + cin);
                        pair |= v << (16 * hh);
                    }
                    w4[i2] = pair;
                }
                const bf16x8_t a = as_bf16x8(u32x4_t{w4[0], w4[1], w4[2], w4[3]});
#pragma unroll
                for (int rb = 0; rb < MB; ++rb)
                    oacc[db][rb] = mfma16x16x32(a, pb[rb], oacc[db][rb]);
            }
        }

        // ---- next tile: registers -> LDS, then the loads two tiles ahead ----
        if (t + 1 < nt) {
            store_tile(buf ^ 1);
            load_data();
            load_idx(t + 3);
        }
        __syncthreads();
    }

    // ---- epilogue: normalised, v_scale-multiplied partial and its lse ----
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        const int r = row0 + rb * 16 + col;
        if (r < rows) {
            const float inv = p.v_scale / l_run[rb];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dv = wave * DW + db * 16 + grp * 4;
                const f32x4_t o = oacc[db][rb] * inv;
                *(f32x4_t *)(po + (int64_t)r * D + dv) = o;
            }
            if (wave == 0 && grp == 0)
                pl[r] = (m_run[rb] + log2f(l_run[rb])) * kLn2;
        }
    }
}

// ---------------------------------------------------------- combine kernel ---
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombineParams p)
{
    constexpr int VPL = D / 64;  // elements of D / Dv per lane
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t total = (int64_t)p.bs * p.h_kv * p.rows;
    if (gw >= total)
        return;
    const int r = (int)(gw % p.rows);
    const int64_t t = gw / p.rows;
    const int kvh = (int)(t % p.h_kv);
    const int b = (int)(t / p.h_kv);
    const int hg = r / p.l_ext;
    const int di = r % p.l_ext;
    const int h = kvh * p.group + hg;
    const int qo = p.qo_indptr[b];
    const int d0 = lane * VPL;

    // ---- (a) log-sum-exp merge of the prefix ranges ----
    int32_t base, count;
    ranges_of(p.kv_indptr, p.bs, p.mode, p.split_tokens, p.n_splits, b, &base, &count);
    float acc[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        acc[v] = 0.0f;
    float m = -INFINITY, den = 0.0f;
    for (int s = 0; s < count; ++s) {
        const int64_t slot = (int64_t)(base + s) * p.h_kv + kvh;
        const float lse = p.part_lse[slot * p.rows + r];
        if (lse == -INFINITY)
            continue;  // empty range
        const float *o = p.part_o + (slot * p.rows + r) * D + d0;
        float ov[VPL];
        if constexpr (VPL == 4) {
            const f32x4_t x = *(const f32x4_t *)o;
            ov[0] = x[0];
            ov[1] = x[1];
            ov[2] = x[2];
            ov[3] = x[3];
        } else {
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                ov[v] = o[v];
        }
        const float mn = fmaxf(m, lse);
        const float a = expf(m - mn);
        const float w = expf(lse - mn);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            acc[v] = acc[v] * a + w * ov[v];
        den = den * a + w;
        m = mn;
    }
    float op[VPL];
    const float lse_p = den > 0.0f ? m + logf(den) : -INFINITY;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        op[v] = den > 0.0f ? acc[v] / den : 0.0f;

    // ---- (b) causal draft block: keys j <= di, fp32, no cast, no scales ----
    float qv[VPL];
    {
        const uint16_t *qr = p.q + (int64_t)(qo + di) * p.q_s0 + (int64_t)h * p.q_s1 + d0;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            qv[v] = bf16_to_f32(qr[v]);
    }
    float od[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        od[v] = 0.0f;
    float md = -INFINITY, dd = 0.0f;
    for (int j = 0; j <= di; ++j) {
        const uint16_t *kr = p.k_ext + (int64_t)(qo + j) * p.ke_s0 + (int64_t)kvh * p.ke_s1 + d0;
        const uint16_t *vr = p.v_ext + (int64_t)(qo + j) * p.ve_s0 + (int64_t)kvh * p.ve_s1 + d0;
        float dot = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            dot += qv[v] * bf16_to_f32(kr[v]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            dot += __shfl_xor(dot, off);
        const float s = dot * p.sm_scale;
        const float mn = fmaxf(md, s);
        const float a = expf(md - mn);
        const float w = expf(s - mn);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            od[v] = od[v] * a + w * bf16_to_f32(vr[v]);
        dd = dd * a + w;
        md = mn;
    }
    const float lse_d = md + logf(dd);

    // ---- (c) final merge of prefix and draft, bf16 store ----
    const float mm = fmaxf(lse_p, lse_d);
    const float wp = expf(lse_p - mm);
    const float wd = expf(lse_d - mm);
    const float inv = 1.0f / (wp + wd);
    uint16_t *orow = p.out + (int64_t)(qo + di) * p.o_s0 + (int64_t)h * p.o_s1 + d0;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        orow[v] = (uint16_t)f32_to_bf16_rne((op[v] * wp + (od[v] / dd) * wd) * inv);
}

// ----------------------------------------------------------------- launch ---
template <bool FP8, int D>
static int launch_prefix_mb(const PrefixParams &p, int mb, int64_t blocks, hipStream_t s)
{
    dim3 grid((unsigned)blocks), block(kThreads);
    switch (mb) {
    case 1: hipLaunchKernelGGL((prefix_kernel<FP8, D, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((prefix_kernel<FP8, D, 2>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((prefix_kernel<FP8, D, 4>), grid, block, 0, s, p); break;
    }
    return (int)hipGetLastError();
}

int launch_prefix(const PrefixParams &p, int head_dim, bool kv_fp8, int row_blocks, int64_t blocks,
                  void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (kv_fp8) {
        switch (head_dim) {
        case 64: return launch_prefix_mb<true, 64>(p, row_blocks, blocks, s);
        case 128: return launch_prefix_mb<true, 128>(p, row_blocks, blocks, s);
        default: return launch_prefix_mb<true, 256>(p, row_blocks, blocks, s);
        }
    }
    switch (head_dim) {
    case 64: return launch_prefix_mb<false, 64>(p, row_blocks, blocks, s);
    case 128: return launch_prefix_mb<false, 128>(p, row_blocks, blocks, s);
    default: return launch_prefix_mb<false, 256>(p, row_blocks, blocks, s);
    }
}

int launch_combine(const CombineParams &p, int head_dim, int64_t blocks, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((unsigned)blocks), block(kThreads);
    switch (head_dim) {
    case 64: hipLaunchKernelGGL((combine_kernel<64>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((combine_kernel<128>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((combine_kernel<256>), grid, block, 0, s, p); break;
    }
    return (int)hipGetLastError();
}

const char *hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace va
