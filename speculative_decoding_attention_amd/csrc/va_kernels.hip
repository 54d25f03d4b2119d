// va_kernels.hip -- gfx950 kernels of split-KV target-verify attention.
//
// Prefix kernel (the pages' _verify_prefix_stage1, sglang verify_splitkv.py):
// one workgroup per (prefix range, KV head, chunk of <= 64 query rows).  All
// query rows that share a KV head -- the GQA group times the l_ext draft rows
// -- are one or two 32-row MFMA column blocks, so every K/V byte of the range
// is read from HBM once for the whole group (the pages launch one program per
// query head and re-read the range per head).  K/V rows are gathered through
// kv_indices straight into an LDS ring with global_load_lds_dwordx4.  Scores
// run on v_mfma_f32_32x32x16_bf16 (fp8 pools: the 32x32x64 fp8 MFMA on the raw
// E4M3FN pool bytes); the softmax is the online running-max / running-sum
// recurrence of the pages in base 2 with k_scale folded into the score scale;
// P V runs on the bf16 MFMA with V^T from the transposing LDS reads (fp8 V is
// widened to bf16 by the hardware conversion).  Each range writes its
// normalised, v_scale-multiplied output (bf16) and natural log-sum-exp.
//
// Combine kernel (the pages' _verify_combine_stage2): one wavefront per
// (sequence, KV head, query row): log-sum-exp merge of the ranges, the causal
// draft block in fp32 (no pool cast, no scales), the final two-way merge and a
// round-to-nearest-even bf16 store.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "va_internal.h"

namespace va {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------- cross-lane steps ---
// Reductions and scans over the 64 lanes of a wave without LDS round trips:
// DPP row permutations inside each 16-lane row (quad_perm, row_shr,
// row_half_mirror, row_mirror), then v_readlane of one lane per row for what
// crosses rows.  A lane whose DPP source lies outside its row reads 0 (the
// old value, with bound_ctrl off).
enum : int {
    kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
    kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
    kDppRowShr1 = 0x111,       // row_shr:1
    kDppRowShr2 = 0x112,
    kDppRowShr4 = 0x114,
    kDppRowShr8 = 0x118,
    kDppRowMirror = 0x140,     // lane 15 - i of the row
    kDppRowHalfMirror = 0x141  // lane 7 - i of the half row
};

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}

// value of lane `l` (wave-uniform l) in every lane
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// sum / max over the 64 lanes, the same value in every lane
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp_f<kDppQuadXor1>(x);
    x += dpp_f<kDppQuadXor2>(x);
    x += dpp_f<kDppRowHalfMirror>(x);
    x += dpp_f<kDppRowMirror>(x);  // every lane holds its row's sum
    return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}

__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_f<kDppRowMirror>(x));
    return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

__device__ __forceinline__ int wave_max_i(int x)
{
    x = max(x, dpp_i<kDppQuadXor1>(x));
    x = max(x, dpp_i<kDppQuadXor2>(x));
    x = max(x, dpp_i<kDppRowHalfMirror>(x));
    x = max(x, dpp_i<kDppRowMirror>(x));
    return max(max(lane_i(x, 0), lane_i(x, 16)), max(lane_i(x, 32), lane_i(x, 48)));
}

__device__ __forceinline__ int wave_sum_i(int x)
{
    x += dpp_i<kDppQuadXor1>(x);
    x += dpp_i<kDppQuadXor2>(x);
    x += dpp_i<kDppRowHalfMirror>(x);
    x += dpp_i<kDppRowMirror>(x);
    return (lane_i(x, 0) + lane_i(x, 16)) + (lane_i(x, 32) + lane_i(x, 48));
}

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

// q (bf16, exact in f32) -> nearest E4M3FN value, ties to even, saturating at
// +-448.  v_cvt_pk_fp8_f32 rounds to nearest even on the OCP grid but turns
// values beyond 448 into NaN, so finite inputs are clamped first (NaN stays
// NaN).
__device__ __forceinline__ float clamp_e4m3_range(float x)
{
    return x != x ? x : fminf(fmaxf(x, -448.0f), 448.0f);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ range lookup ---
// Ranges are numbered sequence by sequence; range r of the batch and KV head
// h writes partial slot r * h_kv + h.
//   mode 0 (fitted): sequence b of n_b tokens is cut into ceil(n_b / c)
//     ranges of c tokens (the last one shorter), c = 64 k with k the smallest
//     positive integer for which the batch needs at most `cap` ranges, cap
//     being the ranges per (KV head, row chunk) the grid holds (never fewer
//     than bs, so k = max ceil(n_b / 64), one range per sequence, always
//     fits).  k comes from the lengths in kv_indptr on every launch, so the
//     split follows the batch actually passed whatever the length of
//     kv_indices: a buffer sized for the largest batch, as a captured graph
//     replays it with other lengths, splits the same as an exact one.
//   mode 1 (the pages' rule): sequence b owns ranges b * n_splits ..
//     + n_splits - 1 of ceil(ceil(n_b / n_splits) / 32) * 32 tokens, empty
//     past the end.
//   mode 2 (explicit): as mode 0 with c = split_tokens.
//   mode 3 (fitted, in rounds): mode 0 for a batch with more sequences than
//     the CUs hold prefix workgroups; the grid allows ranges of about 1 MiB of
//     K/V per KV head, and a batch of (nearly) equal prefixes keeps one range
//     per sequence.
struct Range {
    int32_t b;
    int32_t start;    // token range [start, end) of sequence b's prefix
    int32_t end;
    int32_t kv_base;  // kv_indptr[b]
    int32_t qo;       // qo_indptr[b]
    int32_t seq_ranges;  // ranges of sequence b (modes 0, 2, 3)
    bool valid;
};

// Index pointers of the sequences b0 + 64 c + lane, c < NC, each clamped to
// the last sequence so that every load is in bounds and unconditional (the
// compiler then issues all of them before the first wait).  One group holds
// 64 NC sequences in registers: NC = 1 serves batches of up to 64 sequences,
// NC = 8 up to 512, from a single load round; larger batches walk further
// groups, each loaded again where it is needed.
template <int NC>
struct SeqGroup {
    int32_t k0[NC], k1[NC], q0[NC];  // kv_indptr[b], kv_indptr[b + 1], qo_indptr[b]
};

template <int NC>
__device__ __forceinline__ SeqGroup<NC> load_group(const int32_t *kv_indptr, const int32_t *qo_indptr,
                                                    int32_t bs, int32_t b0)
{
    SeqGroup<NC> g;
    const int32_t lane = (int32_t)(threadIdx.x & 63);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int32_t b = min(b0 + 64 * c + lane, bs - 1);
        g.k0[c] = kv_indptr[b];
        g.k1[c] = kv_indptr[b + 1];
        g.q0[c] = qo_indptr[b];
    }
    return g;
}

// prefix length of sequence b0 + 64 c + lane (0 past the batch)
template <int NC>
__device__ __forceinline__ uint32_t seq_len(const SeqGroup<NC> &g, int c, int32_t b0, int32_t bs)
{
    return b0 + 64 * c + (int32_t)(threadIdx.x & 63) < bs ? (uint32_t)(g.k1[c] - g.k0[c]) : 0u;
}

// Division by a wave-uniform k >= 1.  With m = floor((2^32 - 1) / k), taken
// once per k, x * m / 2^32 falls below x / k by x (1 + (2^32 - 1) mod k) /
// (k 2^32) < 1 for every 32-bit x, so floor(x m / 2^32) is floor(x / k) or
// one less, and one comparison of the remainder settles it: a multiply-high
// and a correction per lane instead of a full division.
struct UniformDiv {
    uint32_t k, m;
};

__device__ __forceinline__ UniformDiv uniform_div(uint32_t k) { return UniformDiv{k, 0xffffffffu / k}; }

__device__ __forceinline__ uint32_t div_floor(uint32_t x, const UniformDiv &d)
{
    const uint32_t q = __umulhi(x, d.m);
    return x - q * d.k >= d.k ? q + 1u : q;
}

// ranges of 64 k tokens that cover a prefix of n tokens
__device__ __forceinline__ uint32_t ranges_for(uint32_t n, const UniformDiv &d)
{
    return div_floor(((n + 63u) >> 6) + d.k - 1u, d);
}

// number of ranges of 64 k tokens the whole batch needs (whole-wave call)
template <int NC>
__device__ __forceinline__ uint32_t batch_ranges(const int32_t *kv_indptr, const int32_t *qo_indptr, int32_t bs,
                                                 uint32_t k, const SeqGroup<NC> &first)
{
    const UniformDiv d = uniform_div(k);
    uint32_t t = 0;
    for (int32_t b0 = 0; b0 < bs; b0 += 64 * NC) {
        const SeqGroup<NC> g = b0 == 0 ? first : load_group<NC>(kv_indptr, qo_indptr, bs, b0);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            t += ranges_for(seq_len(g, c, b0, bs), d);
    }
    return (uint32_t)wave_sum_i((int32_t)t);
}

// Mode 0: the range size in units of 64 tokens (whole-wave call).  With
// m_b = ceil(n_b / 64) and M their sum, count(k) = sum_b ceil(m_b / k) is at
// least M / k and at most M / k + bs, so the answer lies in
// [ceil(M / cap), ceil(M / (cap - bs))] (when cap > bs) and never above
// max m_b; a binary search over whole-batch counts takes it from there.
// `count` receives the number of ranges when it is known on the way (else
// cap, an upper bound).  In rounds (mode 3, a batch past the resident
// workgroups) the planner's grid holds max(bs, ceil(T / round_tokens))
// ranges for the T of num_kv_indices; the fit takes that bound for the T the
// batch really has, so a kv_indices buffer of larger capacity splits the
// batch exactly as one of its own length, and a workgroup whose slot `cidx`
// lies past the bound leaves before the search.
template <int NC>
__device__ __forceinline__ uint32_t fitted_range_units(const int32_t *kv_indptr, const int32_t *qo_indptr,
                                                       int32_t bs, int32_t cap, bool rounds, uint32_t round_tokens,
                                                       int64_t cidx, const SeqGroup<NC> &first, uint32_t &count)
{
    uint32_t ms = 0, mx = 0, nz = 0, ns = 0;
    for (int32_t b0 = 0; b0 < bs; b0 += 64 * NC) {
        const SeqGroup<NC> g = b0 == 0 ? first : load_group<NC>(kv_indptr, qo_indptr, bs, b0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint32_t n = seq_len(g, c, b0, bs);
            const uint32_t m = (n + 63u) >> 6;
            ms += m;
            mx = max(mx, m);
            nz += m > 0u ? 1u : 0u;
            ns += n;
        }
    }
    const uint32_t msum = (uint32_t)wave_sum_i((int32_t)ms);
    uint32_t ucap = (uint32_t)cap;
    if (rounds) {
        const uint32_t tokens = (uint32_t)wave_sum_i((int32_t)ns);
        ucap = min(ucap, max((uint32_t)bs, (tokens + round_tokens - 1u) / round_tokens));
    }
    count = ucap;
    if (msum == 0 || cidx >= (int64_t)ucap)
        return 1u;  // no prefix token, or no range for this slot: any size
    // A batch past the resident workgroups runs in rounds.  When its prefixes
    // are (nearly) equal, whole sequences fill the rounds evenly and each
    // extra round would start all its workgroups at once, unhidden: keep one
    // range per sequence (it always fits: cap >= bs).
    if (rounds) {
        const uint32_t mmax = (uint32_t)wave_max_i((int32_t)mx);
        const uint32_t nonempty = (uint32_t)wave_sum_i((int32_t)nz);
        if ((uint64_t)mmax * nonempty <= (uint64_t)msum + msum / 8u) {
            count = nonempty;  // the workgroups of the other slots leave at once
            return mmax;
        }
    }
    uint32_t lo = max((msum + ucap - 1u) / ucap, 1u);
    const uint32_t nlo = batch_ranges(kv_indptr, qo_indptr, bs, lo, first);
    if (nlo <= ucap) {
        count = nlo;
        return lo;  // every uniform batch whose lengths are multiples of the size
    }
    uint32_t hi = (uint32_t)wave_max_i((int32_t)mx);
    if (ucap > (uint32_t)bs)
        hi = min(hi, (msum + (ucap - (uint32_t)bs) - 1u) / (ucap - (uint32_t)bs));
    while (lo + 1u < hi) {  // count(lo) > cap >= count(hi)
        const uint32_t mid = lo + (hi - lo) / 2u;
        const uint32_t n = batch_ranges(kv_indptr, qo_indptr, bs, mid, first);
        if (n <= ucap) {
            hi = mid;
            count = n;
        } else {
            lo = mid;
        }
    }
    return hi;
}

// Range size of modes 0, 2 and 3 in units of 64 tokens; `count` as for
// fitted_range_units.
template <int NC>
__device__ __forceinline__ uint32_t range_units(const int32_t *kv_indptr, const int32_t *qo_indptr, int32_t bs,
                                                int32_t mode, int32_t split_tokens, int32_t cap,
                                                uint32_t round_tokens, int64_t cidx, const SeqGroup<NC> &first,
                                                uint32_t &count)
{
    if (mode == 2) {
        count = (uint32_t)cap;
        return (uint32_t)split_tokens >> 6;
    }
    return fitted_range_units<NC>(kv_indptr, qo_indptr, bs, cap, mode == 3, round_tokens, cidx, first, count);
}

// Mode 1: range `cidx` -> its sequence, token range and index pointers.
__device__ __forceinline__ Range locate_range(const int32_t *kv_indptr, const int32_t *qo_indptr,
                                              int32_t bs, int32_t n_splits, int64_t cidx)
{
    Range r = {0, 0, 0, 0, 0, 0, false};
    const int64_t b = cidx / n_splits;
    if (b >= bs)
        return r;
    const int32_t s = (int32_t)(cidx % n_splits);
    const int32_t k0 = kv_indptr[b];
    const int32_t n = kv_indptr[b + 1] - k0;
    const int32_t per = ((n + n_splits - 1) / n_splits + kEvenSplitGranule - 1) /
                        kEvenSplitGranule * kEvenSplitGranule;
    r.b = (int32_t)b;
    r.start = s * per;
    r.end = min(r.start + per, n);
    r.kv_base = k0;
    r.qo = qo_indptr[b];
    r.valid = true;
    return r;
}

// inclusive prefix sum over the lanes
__device__ __forceinline__ int wave_scan_incl(int x)
{
    x += dpp_i<kDppRowShr1>(x);
    x += dpp_i<kDppRowShr2>(x);
    x += dpp_i<kDppRowShr4>(x);
    x += dpp_i<kDppRowShr8>(x);  // prefix within the row
    const int t0 = lane_i(x, 15), t1 = lane_i(x, 31), t2 = lane_i(x, 47);
    const int lane = threadIdx.x & 63;
    return x + (lane >= 16 ? t0 : 0) + (lane >= 32 ? t1 : 0) + (lane >= 48 ? t2 : 0);
}

// Modes 0, 2 and 3: range `cidx` -> its sequence, token range and index
// pointers, for ranges of 64 k tokens numbered sequence by sequence (`count`:
// a bound on the number of ranges; slots past it hold none).
template <int NC>
__device__ __forceinline__ Range locate_split_range(const int32_t *kv_indptr, const int32_t *qo_indptr,
                                                    int32_t bs, uint32_t k, int64_t cidx, uint32_t count,
                                                    const SeqGroup<NC> &first)
{
    Range r = {0, 0, 0, 0, 0, 0, false};
    if (cidx >= (int64_t)count)
        return r;
    const UniformDiv d = uniform_div(k);
    const int32_t c_tok = (int32_t)(k << 6);
    int64_t cum = 0;
    for (int32_t b0 = 0; b0 < bs; b0 += 64 * NC) {
        const SeqGroup<NC> g = b0 == 0 ? first : load_group<NC>(kv_indptr, qo_indptr, bs, b0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint32_t n = seq_len(g, c, b0, bs);
            const int32_t nch = (int32_t)ranges_for(n, d);
            const int32_t incl = wave_scan_incl(nch);
            const int32_t total = lane_i(incl, 63);
            if (cidx < cum + total) {
                const uint64_t hit = __ballot(cum + incl > cidx);
                const int h = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
                const int32_t ci = (int32_t)(cidx - cum - lane_i(incl - nch, h));
                r.b = b0 + 64 * c + h;
                r.start = ci * c_tok;
                r.end = min(r.start + c_tok, lane_i((int32_t)n, h));
                r.kv_base = lane_i(g.k0[c], h);
                r.qo = lane_i(g.q0[c], h);
                r.seq_ranges = lane_i(nch, h);
                r.valid = true;
                return r;
            }
            cum += total;
        }
    }
    return r;
}

// ----------------------------------------------------------- prefix kernel ---
// Asynchronous global -> LDS copies.  global_load_lds_dwordx{1,4} writes lane
// l's 4 / 16 bytes to LDS at M0 + 4l / 16l and counts in vmcnt like any load
// (loads retire in issue order).  They are issued from inline asm so that the
// compiler inserts no waits of its own for them; every wait is explicit.
__device__ __forceinline__ uint32_t lds_offset(const void *p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lds_base), "v"(g) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(lds_base), "v"(g) : "memory", "m0");
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier for LDS data only: this wave's LDS operations are complete
// (lgkmcnt 0) before it arrives.  Copies into LDS are covered by wait_vm first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// K rows have D elements, V rows DV; the larger of the two sizes the tile and
// the ring, so each stage holds a K region and a V region of TN rows of the
// larger row size (the smaller operand leaves the end of its region unused).
template <bool FP8, int D, int DV, int NQB>
struct PrefixGeom {
    static constexpr int NW = prefix_waves(NQB);
    static constexpr int E = FP8 ? 1 : 2;               // pool bytes per element
    static constexpr int DM = D > DV ? D : DV;
    static constexpr int ROWB_K = D * E;                // pool bytes per K row
    static constexpr int ROWB_V = DV * E;               // pool bytes per V row
    static constexpr int ROWB_M = DM * E;
    static constexpr int TN0 = 16384 / ROWB_M;
    static constexpr int TN = TN0 > 128 ? 128 : TN0;    // tokens per tile (K+V <= 32 KB)
    static constexpr int LCH_K = ROWB_K / 16;           // 16-byte chunks per K row
    static constexpr int LCH_V = ROWB_V / 16;
    static constexpr int RPI_K = 64 / LCH_K;            // K rows per wave-wide copy
    static constexpr int RPI_V = 64 / LCH_V;
    static constexpr int NBUF = prefix_ring_stages(NQB);  // tiles in the LDS ring
    static constexpr int STAGE_K = TN * ROWB_M;         // K region; the V region follows
    static constexpr int STAGE = 2 * STAGE_K;
    static constexpr int NIKW_K = TN * LCH_K / (64 * NW);  // K copies per wave per tile
    static constexpr int NIKW_V = TN * LCH_V / (64 * NW);  // V copies per wave per tile
    static constexpr int NCP = NIKW_K + NIKW_V;
    static constexpr int RW = TN / NW;                  // rows each wave copies per tile
    static constexpr int NIDX = 3;                      // index slots per wave
    static_assert(NIKW_K >= 1 && NIKW_K * 64 * NW == TN * LCH_K, "K tile / copy geometry");
    static_assert(NIKW_V >= 1 && NIKW_V * 64 * NW == TN * LCH_V, "V tile / copy geometry");
    static_assert(NIKW_K * RPI_K == RW && NIKW_V * RPI_V == RW, "K and V copies cover the same rows");
    static_assert(2 * RW <= 64, "one index copy per wave per tile");
    static_assert(TN == tile_tokens_for(D, DV, E), "host and kernel tile rules agree");
};

// LDS layouts (per ring stage; rows of raw pool bytes, 16-byte chunks; the
// 64 LDS banks span 256 bytes):
//   K: chunk c of token row t sits at chunk c ^ kswz(t).  bf16: kswz(t) =
//      t & 15 (t & 7 for 8-chunk rows): the score MFMA reads 16 consecutive
//      rows at one chunk per LDS cycle, which this puts on 16 different bank
//      groups.  fp8 rows are 64..256 bytes, so rows 256 / row_bytes apart
//      share their banks: kswz(t) = (t / (256 / row_bytes)) mod chunks spreads
//      every such set of rows over distinct chunks.
//   V: chunk c of token row t sits at chunk c ^ vswz(t).  bf16 values are read
//      with the 16-bit transposing read: 32 lanes cover 4 consecutive rows x 4
//      chunks, so vswz(t) = (t & 3) << 2 moves each row to its own group of 4
//      chunks ((t & 1) << 2 for 8-chunk rows).  fp8 values are read with the
//      8-bit transposing read (16 rows x 32 bytes per instruction) and use
//      the fp8 K rule.
// The copies choose, for every LDS chunk, the pool chunk that belongs there.
//
// Work split: a wave computes the scores of all query rows of its block for a
// 32-token sub-tile (32x32 MFMA: tokens x 32 query rows), keeps its own
// running max / sum, and accumulates its share of the output columns.  When a
// tile holds several sub-tiles (short rows: fp8, D <= 128) the waves of a
// block take different sub-tiles and all columns, so no score is computed
// twice; with one sub-tile per tile (bf16, D = 256) they share its scores and
// split the columns.  The score C-layout of one 32 x 32 block is exactly the
// B operand of two value MFMA k-steps, so probabilities never leave registers
// and a tile needs a single barrier.  The running max is raised only when a row's
// new maximum exceeds it by more than 2^8 (the rescale of the accumulators is
// then skipped for most tiles); probabilities stay below 2^8, far inside the
// range of bf16 and fp32.
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 x fp8 (format 0: OCP E4M3FN on both operands), E8M0 scales 127 = 1.0
__device__ __forceinline__ f32x16_t mfma32x32x64_fp8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Two E4M3FN codes (bytes 0,1 or, with HIGH, 2,3 of w) -> two bf16 (exact),
// packed.
template <bool HIGH>
__device__ __forceinline__ uint32_t cvt_e4m3x2_bf16(int w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}

// value of lane l ^ 32
__device__ __forceinline__ float swap_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Both shapes keep two waves on every SIMD (two 4-wave workgroups, or one
// 8-wave workgroup, per CU), so the launch bound holds the kernel to 256
// registers per lane.
// The leading scalar arguments are what the first memory round trip needs
// (the range lookup); they are preloaded into SGPRs at wave launch, so the
// kv_indptr loads issue without waiting for the kernel-argument fetch.  The
// same fields are also in p.
template <bool FP8, int D, int DV, int NQB>
__global__ __launch_bounds__(prefix_waves(NQB) * 64, 2) void prefix_kernel(
    const int32_t *kv_indptr, const int32_t *qo_indptr, const int64_t *kv_indices, int32_t bs, int32_t mode,
    int32_t split_tokens, int32_t total_tokens, int32_t h_kv, int32_t row_chunks, int32_t n_splits,
    const PrefixParams p)
{
    using G = PrefixGeom<FP8, D, DV, NQB>;
    constexpr int NW = G::NW;
    constexpr int TN = G::TN;
    constexpr int ROWB_K = G::ROWB_K;
    constexpr int ROWB_V = G::ROWB_V;
    constexpr int LCH_K = G::LCH_K;
    constexpr int LCH_V = G::LCH_V;
    constexpr int NBUF = G::NBUF;
    constexpr int NCP = G::NCP;
    constexpr int RW = G::RW;
    constexpr int NKS = D / 16;             // k-steps of the score MFMA
    constexpr int NSUB = TN / 32;           // 32-token sub-tiles per tile
    constexpr int GW = NW / NQB;            // waves per query block
    // The waves of a query block split a tile's sub-tiles TS ways and the
    // output columns CS ways (TS * CS = GW).  Each wave keeps its own running
    // max / sum; the TS token shares are merged after the last tile.
    constexpr int TS = GW < NSUB ? GW : NSUB;
    constexpr int CS = GW / TS;
    constexpr int DWV = DV / CS;            // output columns per wave
    constexpr int DBW = DWV / 32;           // 32-column blocks per wave
    static_assert(TS * CS == GW && NSUB % TS == 0, "work split");
    constexpr int KSWZ = (LCH_K < 16 ? LCH_K : 16) - 1;
    constexpr int VSWZ8 = (LCH_V < 16 ? LCH_V : 16) - 1;
    constexpr int VSWZ_ROWS = LCH_V >= 16 ? 3 : 1;  // bf16: rows whose 4-chunk groups differ
    // fp8: log2(256 / row bytes)
    constexpr int SW8_SHIFT_K = ROWB_K >= 256 ? 0 : (ROWB_K == 128 ? 1 : 2);
    constexpr int SW8_SHIFT_V = ROWB_V >= 256 ? 0 : (ROWB_V == 128 ? 1 : 2);
    auto kswz = [](int r) { return FP8 ? ((r >> SW8_SHIFT_K) & KSWZ) : (r & KSWZ); };
    auto vswz = [](int r) { return FP8 ? ((r >> SW8_SHIFT_V) & VSWZ8) : ((r & VSWZ_ROWS) << 2); };
    constexpr float kRescale = 8.0f;        // log2 headroom before the max is raised
    static_assert(NQB == 1 || NQB == 2, "query blocks");
    static_assert(NQB * 32 * D * 2 <= G::STAGE, "query tile fits one ring stage");
    static_assert(TN % 32 == 0 && DWV % 32 == 0, "tile / column geometry");
    // after tile t's copies, the next two steps issue 2 index copies and up to
    // 2 * NCP tile copies
    constexpr int VM_TWO_AHEAD = 2 + 2 * NCP;
    constexpr int VM_ONE_AHEAD = 2 + NCP;
    constexpr int VM_NONE_AHEAD = 2;

    __shared__ __attribute__((aligned(1024))) uint8_t s_ring[NBUF * G::STAGE];
    __shared__ __attribute__((aligned(16))) int64_t s_idx[NW][G::NIDX][RW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;   // token (A) / query row (B, C) within a 32 block
    const int half = lane >> 5;  // k half of the operands

    // ---- work item: (range, KV head, row chunk) ----
    const uint32_t blk = blockIdx.x;
    const int rc = (int)(blk % (uint32_t)row_chunks);
    const uint32_t t1 = blk / (uint32_t)row_chunks;
    const int kvh = (int)(t1 % (uint32_t)h_kv);
    const int64_t cidx = t1 / (uint32_t)h_kv;
    const int row0 = rc * kRowChunk;
    const uint32_t ring = lds_offset(s_ring);
    const uint32_t idx_base = lds_offset(&s_idx[wave][0][0]);
    const bool paged = kv_indices == nullptr;  // prefix rows through a page table

    // The piece being processed: tokens [pstart, pstart + len) of sequence pb,
    // whose first token sits at kv_indices position kv0.  Index entries
    // kv0 .. kv0 + fetch - 1 may be read (fetch >= len); tokens past len are
    // masked out of the scores and their K/V copies read pool row 0.
    int64_t kv0 = 0;
    int len = 0, fetch = 1, pb = 0, pstart = 0, qo = 0;

    // ---- copy issue: index slots, K/V tiles, query tile ----
    auto issue_idx = [&](int k) {
        // rows wave*RW .. +RW of tile k: the two dwords of the int64 index, or
        // the token's page id in both lanes of the pair
        if (lane < 2 * RW) {
            int tok = k * TN + wave * RW + (lane >> 1);
            tok = tok < fetch ? tok : fetch - 1;
            const uint32_t dst = __builtin_amdgcn_readfirstlane(idx_base + (k % G::NIDX) * RW * 8);
            if (paged)
                dma4(p.block_table + (int64_t)pb * p.bt_s0 + (pstart + tok) / p.page_size, dst);
            else
                dma4((const uint32_t *)(kv_indices + kv0 + tok) + (lane & 1), dst);
        }
    };
    const uint8_t *kbase = p.k_buf + (int64_t)kvh * p.kb_s1;
    const uint8_t *vbase = p.v_buf + (int64_t)kvh * p.vb_s1;
    auto issue_tile = [&](int k) {
        const int64_t *ix = &s_idx[wave][k % G::NIDX][0];
        // this wave's rows wave*RW .. +RW sit at byte wave*RW*row_bytes of
        // each region; one wave-wide copy moves 1 KB (RPI rows)
        const uint32_t st = ring + (k % NBUF) * G::STAGE;
        auto pool_row = [&](int rl) {
            const int tok = k * TN + wave * RW + rl;
            uint64_t t = (uint64_t)ix[rl];
            if (paged)  // pool row = page id * page_size + position in the page
                t = (uint64_t)(uint32_t)t * (uint32_t)p.page_size + (uint32_t)((pstart + tok) % p.page_size);
            return tok < len ? t : (uint64_t)0;
        };
        // every copy's pool row first: the copies are asm with a memory
        // clobber, so an index read between them would be read again; K and V
        // rows of equal size share their rows
        constexpr bool SAME = LCH_K == LCH_V;
        uint64_t tk[G::NIKW_K], tv[G::NIKW_V];
#pragma unroll
        for (int i = 0; i < G::NIKW_K; ++i)
            tk[i] = pool_row(i * G::RPI_K + lane / LCH_K);
#pragma unroll
        for (int i = 0; i < G::NIKW_V; ++i)
            tv[i] = SAME ? tk[i < G::NIKW_K ? i : 0] : pool_row(i * G::RPI_V + lane / LCH_V);
#pragma unroll
        for (int i = 0; i < (G::NIKW_K > G::NIKW_V ? G::NIKW_K : G::NIKW_V); ++i) {
            if (i < G::NIKW_K) {
                const int rl = i * G::RPI_K + lane / LCH_K;  // row within this wave's rows
                const int pc = lane % LCH_K;                 // LDS chunk within the row
                dma16(kbase + tk[i] * p.kb_s0 + ((pc ^ kswz(wave * RW + rl)) << 4),
                      __builtin_amdgcn_readfirstlane(st + wave * RW * ROWB_K + i * 1024));
            }
            if (i < G::NIKW_V) {
                const int rl = i * G::RPI_V + lane / LCH_V;
                const int pc = lane % LCH_V;
                dma16(vbase + tv[i] * p.vb_s0 + ((pc ^ vswz(wave * RW + rl)) << 4),
                      __builtin_amdgcn_readfirstlane(st + G::STAGE_K + wave * RW * ROWB_V + i * 1024));
            }
        }
    };
    // query tile -> ring stage NBUF-1: bf16 rows of D, chunk c of local row r
    // at chunk c ^ qswz(r).  Each lane later reads its own row, so without the
    // swizzle the 32 rows (a multiple of 256 bytes apart for D >= 128) would
    // all hit the same LDS banks.
    constexpr int QCH = D / 8;                    // 16-byte chunks per query row
    constexpr int QI = NQB * 32 * QCH / 64;       // wave-wide copies for the tile
    constexpr int QPW = QI / NW;                  // of which each wave issues
    static_assert(QI % NW == 0, "query copies split evenly over the waves");
    constexpr int QSW_SHIFT = D * 2 >= 256 ? 0 : (D * 2 == 128 ? 1 : 2);  // rows sharing 256 bytes
    constexpr int QSW_MASK = (QCH < 16 ? QCH : 16) - 1;
    auto qswz = [](int r) { return (r >> QSW_SHIFT) & QSW_MASK; };
    auto issue_query = [&]() {
        const int rows = p.rows;
#pragma unroll
        for (int k = 0; k < QPW; ++k) {
            const int i = wave + k * NW;
            const int e = i * 64 + lane;
            const int r = row0 + e / QCH;             // query row of this chunk
            const int rr = r < rows ? r : row0;       // padding rows copy a valid row
            const int hg = rr / p.l_ext, di = rr % p.l_ext;
            const int ch = (e % QCH) ^ qswz(e / QCH);  // source chunk of this LDS chunk
            const uint16_t *src = p.q + (int64_t)(qo + di) * p.q_s0 +
                                  (int64_t)(kvh * p.group + hg) * p.q_s1 + ch * 8;
            dma16(src, __builtin_amdgcn_readfirstlane(ring + (NBUF - 1) * G::STAGE + i * 1024));
        }
    };

    // ---- range ----
    // Modes 0, 2 and 3 cut every prefix into ranges of c tokens; split_tokens
    // is c itself (mode 2) or the planner's estimate of it (modes 0 and 3: the
    // size that num_kv_indices tokens in equal prefixes would get).  If every prefix is
    // a multiple of it, range cidx starts at kv_indices position
    // cidx * split_tokens: its first three index copies go out before the
    // index pointers are read, and are used if the range really starts there.
    // Mode 1 (the pages' rule): range cidx is split cidx % n_splits of
    // sequence cidx / n_splits.
    int64_t P0 = -1;
    int early_fetch = 0;
    auto early_copies = [&]() {
        if (mode != 1 && !paged) {
            const int64_t g0 = cidx * (int64_t)split_tokens;
            if (g0 < total_tokens) {
                P0 = g0;
                kv0 = g0;
                fetch = (int)min((int64_t)split_tokens, (int64_t)total_tokens - g0);
                early_fetch = fetch;
                issue_idx(0);
                issue_idx(1);
                issue_idx(2);
            }
        }
        // the remaining kernel arguments while those loads are in flight (the
        // scheduling barrier keeps the early copies ahead of their wait;
        // row_chunks stays live so that no register of the argument loads is
        // reused early)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::"s"(p.q), "s"(p.k_buf), "s"(p.v_buf), "s"(p.kb_s1), "s"(p.vb_s1), "s"(p.kb_s0),
                     "s"(p.vb_s0), "s"(p.q_s0), "s"(p.q_s1), "s"(p.group), "s"(p.l_ext), "s"(p.rows),
                     "s"(p.row_chunks)
                     : "memory");
    };
    const int32_t range_cap = (int32_t)(gridDim.x / (uint32_t)(h_kv * row_chunks));  // ranges per (KV head, chunk)
    constexpr uint32_t kRoundTokens = (uint32_t)round_range_tokens(D, DV, FP8 ? 1 : 2);
    Range rg;
    if (mode == 1) {
        early_copies();
        rg = locate_range(kv_indptr, qo_indptr, bs, n_splits, cidx);
    } else if (bs <= 64) {
        const SeqGroup<1> first = load_group<1>(kv_indptr, qo_indptr, bs, 0);
        early_copies();
        uint32_t count;
        const uint32_t k = range_units<1>(kv_indptr, qo_indptr, bs, mode, split_tokens, range_cap, kRoundTokens,
                                          cidx, first, count);
        rg = locate_split_range<1>(kv_indptr, qo_indptr, bs, k, cidx, count, first);
    } else {
        const SeqGroup<8> first = load_group<8>(kv_indptr, qo_indptr, bs, 0);
        early_copies();
        uint32_t count;
        const uint32_t k = range_units<8>(kv_indptr, qo_indptr, bs, mode, split_tokens, range_cap, kRoundTokens,
                                          cidx, first, count);
        rg = locate_split_range<8>(kv_indptr, qo_indptr, bs, k, cidx, count, first);
    }
    const int rows = p.rows;
    if (!rg.valid) {
        wait_vm<0>();  // early index copies of a surplus slot of the static grid
        return;        // (never read by the combine pass)
    }
    // the first range of each sequence records where the sequence's ranges
    // sit, for the combine pass (modes 0, 2 and 3; mode 1 needs no table)
    if (mode != 1 && kvh == 0 && rc == 0 && rg.start == 0 && tid == 0)
        ((i32x2_t *)p.seq_ranges)[rg.b] = i32x2_t{(int32_t)cidx, rg.seq_ranges};
    const int64_t slot = cidx * h_kv + kvh;
    uint16_t *po = p.part_o + slot * (int64_t)rows * DV;
    float *pl = p.part_lse + slot * (int64_t)rows;
    if (rg.start >= rg.end) {
        // Empty range (mode 1 past the end): output 0 and log-sum-exp -inf, so
        // the merge weight is exactly 0 and no stale value can leak in.
        const int nr = min(rows - row0, NQB * 32);
        for (int e = tid; e < nr * DV; e += NW * 64)
            po[(int64_t)(row0 + e / DV) * DV + (e % DV)] = 0;
        if (tid < nr)
            pl[row0 + tid] = -INFINITY;
        return;
    }
    pb = rg.b;
    pstart = rg.start;
    len = rg.end - rg.start;
    fetch = len;
    kv0 = (int64_t)rg.kv_base + rg.start;
    qo = rg.qo;
    // the early index copies are this range's if it starts at P0 and they
    // cover every token of tiles 0..2
    const bool ready = kv0 == P0 && min(len, 3 * TN) <= early_fetch;
    const int nt = (len + TN - 1) / TN;


    // prologue: index slots 0..2, the query tile, then steps
    // j = 0 .. NBUF-2, step j = [tile j][index copy of tile j+2].  Loads
    // retire in order, so "slot j has landed" is "at most the loads issued
    // after it are outstanding" (loads between them that were already
    // awaited only make a wait stricter).
    static_assert(NBUF == 2 || NBUF == 4, "wait counts are written for 2- or 4-stage rings");
    if (!ready) {
        issue_idx(0);
        issue_idx(1);
        issue_idx(2);
    }
    issue_query();
    wait_vm<QPW + 2>();  // index slot 0: then slots 1, 2 and the query copies
    issue_tile(0);
    if constexpr (NBUF == 4) {
        issue_idx(3);
        if (1 < nt) {
            wait_vm<QPW + NCP + 2>();  // index slot 1: then slot 2, query, tile 0, slot 3
            issue_tile(1);
        }
        issue_idx(4);
        if (2 < nt) {
            wait_vm<QPW + 2 * NCP + 2>();  // index slot 2: then query, tile 0, slot 3, tile 1, slot 4
            issue_tile(2);
        }
        // the query tile: then min(nt, 3) tiles and index slots 3, 4
        if (nt >= 3)
            wait_vm<2 + 3 * NCP>();
        else if (nt == 2)
            wait_vm<2 + 2 * NCP>();
        else
            wait_vm<2 + NCP>();
    } else {
        wait_vm<NCP>();  // the query tile: then tile 0
    }
    lds_barrier();

    // ---- this wave's query block (waves qbw*GW .. +GW share it) ----
    const int qbw = wave / GW;   // query block of this wave
    const int wg = wave % GW;    // wave within the block's group
    const int ts = wg % TS;      // token share: sub-tiles ts, ts + TS, ...
    const int cs = wg / TS;      // column share: columns cs * DWV .. + DWV

    // ---- query operand (B: col = query row, k = d) ----
    // bf16: k-step ks holds d = 16 ks + 8 half + 0..7.  fp8: E4M3FN codes of q
    // rounded to the pool dtype (the prefix dot product uses that q); k-step j
    // of the 32x32x64 MFMA holds d = 64 j + 32 half + 0..31, and the K operand
    // uses the same d, so the k order inside the instruction does not matter.
    constexpr int NQR = FP8 ? D / 64 : NKS;
    typedef typename std::conditional<FP8, i32x8_t, bf16x8_t>::type qop_t;
    qop_t qreg[NQR];
    {
        // every local row holds a valid query row (padding rows a copy of the
        // chunk's first row), and a padding row's outputs are never stored
        const int rl = qbw * 32 + l32;
        const uint8_t *qrow = s_ring + (NBUF - 1) * G::STAGE + rl * D * 2;
        const int qz = qswz(rl);
        if constexpr (FP8) {
#pragma unroll
            for (int j = 0; j < NQR; ++j) {
                i32x8_t codes;
#pragma unroll
                for (int c = 0; c < 4; ++c) {  // 16-byte chunk of 8 bf16 values
                    const u32x4_t raw = *(const u32x4_t *)(qrow + ((8 * j + 4 * half + c) ^ qz) * 16);
#pragma unroll
                    for (int w = 0; w < 2; ++w) {  // 4 codes per dword
                        const float x0 = clamp_e4m3_range(bf16_to_f32(raw[2 * w] & 0xffffu));
                        const float x1 = clamp_e4m3_range(bf16_to_f32(raw[2 * w] >> 16));
                        const float x2 = clamp_e4m3_range(bf16_to_f32(raw[2 * w + 1] & 0xffffu));
                        const float x3 = clamp_e4m3_range(bf16_to_f32(raw[2 * w + 1] >> 16));
                        const int d = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
                        codes[2 * c + w] = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, d, true);
                    }
                }
                qreg[j] = codes;
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                qreg[ks] = as_bf16x8(*(const u32x4_t *)(qrow + ((ks * 2 + half) ^ qz) * 16));
            }
        }
    }

    // ---- running state: lane's query row is 32*qbw + l32 ----
    float m_ref = -INFINITY, l_part = 0.0f;
    f32x16_t oacc[DBW];
#pragma unroll
    for (int db = 0; db < DBW; ++db)
        oacc[db] = f32x16_t{};

    const float qk_scale = p.qk_scale_log2;
    for (int t = 0; t < nt; ++t) {
        // tile t's copies by this wave are complete; then everyone's are
        if constexpr (NBUF == 4) {
            const int after = nt - 1 - t;
            if (after >= 2)
                wait_vm<VM_TWO_AHEAD>();
            else if (after == 1)
                wait_vm<VM_ONE_AHEAD>();
            else
                wait_vm<VM_NONE_AHEAD>();
        } else {
            wait_vm<0>();  // tile t was the last copy issued
        }
        lds_barrier();

        // step j = t + NBUF - 1 into the stage tile t-1 used (everyone is past it)
        {
            const int j = t + NBUF - 1;
            issue_idx(j + 2);
            if (j < nt) {
                wait_vm<2 * NCP + 2>();  // index slot j, copied two steps ago
                issue_tile(j);
            }
        }

        const uint8_t *K = s_ring + (t % NBUF) * G::STAGE;
        const uint8_t *V = K + G::STAGE_K;

        // one 32-token sub-tile; tokens past the range are masked only in the
        // (at most one) sub-tile that straddles the end.  `masked` is a bool
        // (fp8 pools: one body with the mask as a branch inside it) or a
        // std::bool_constant (bf16 pools: a masked and an unmasked body).  Two
        // bodies make the compiler copy the output accumulators in and out of
        // every tile to reconcile their register assignments (64 moves a tile
        // on fp8 D=128), which the issue-bound fp8 loop pays for; the
        // memory-bound bf16 loop measured faster with two bodies all the same.
        auto sub_tile = [&](const int sub, auto masked) {
            const int tok0 = t * TN + sub * 32;  // first token of the sub-tile

            // ---- scores S^T[token][query row] of this wave's block, 32 x 32 ----
            // two accumulators (even / odd k-steps) halve the chain of dependent
            // MFMAs
            f32x16_t sc = {}, sc2 = {};
            const int krow = sub * 32 + l32;
#pragma unroll
            for (int ks = 0; ks < NQR; ++ks) {
                if constexpr (FP8) {
                    // d = 64 ks + 32 half + 0..31: chunks 4 ks + 2 half, +1
                    const int c0 = 4 * ks + 2 * half;
                    const u32x4_t lo = *(const u32x4_t *)(K + krow * ROWB_K + ((c0 ^ kswz(krow)) << 4));
                    const u32x4_t hi = *(const u32x4_t *)(K + krow * ROWB_K + (((c0 + 1) ^ kswz(krow)) << 4));
                    const i32x8_t a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    if (ks & 1)
                        sc2 = mfma32x32x64_fp8(a, qreg[ks], sc2);
                    else
                        sc = mfma32x32x64_fp8(a, qreg[ks], sc);
                } else {
                    const int ch = (ks * 2 + half) ^ kswz(krow);
                    const bf16x8_t a = as_bf16x8(*(const u32x4_t *)(K + krow * ROWB_K + (ch << 4)));
                    if (ks & 1)
                        sc2 = mfma32x32x16(a, qreg[ks], sc2);
                    else
                        sc = mfma32x32x16(a, qreg[ks], sc);
                }
            }
            sc += sc2;

            // ---- softmax: lane holds 16 of the row's 32 tokens, lane^32 the rest ----
            bool mask_now;
            if constexpr (std::is_same<decltype(masked), bool>::value)
                mask_now = masked;
            else
                mask_now = decltype(masked)::value;
            if (mask_now) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int tok = tok0 + 8 * (v >> 2) + 4 * half + (v & 3);
                    sc[v] = tok < len ? sc[v] : -INFINITY;
                }
            }
            float mx = sc[0];
#pragma unroll
            for (int v = 1; v < 16; ++v)
                mx = fmaxf(mx, sc[v]);
            mx = fmaxf(mx, swap_halves(mx)) * qk_scale;  // row max, log2 units
            const bool grow = mx > m_ref + kRescale;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                // raise the reference (all lanes of the wave)
                const float mn = fmaxf(m_ref, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
                m_ref = mn;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < DBW; ++db)
                    oacc[db] *= alpha;
            }
            const float mneg = -m_ref;
            float rs = 0.0f;
            uint32_t pk[8];
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v], qk_scale, mneg));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v + 1], qk_scale, mneg));
                rs += e0 + e1;
                pk[v >> 1] = pack_bf16x2(e0, e1);
            }
            l_part += rs;

            // ---- O^T[dv][query row] += V^T P^T over this wave's columns ----
            {
#pragma unroll
                for (int db = 0; db < DBW; ++db) {
                    const int cb = cs * DWV + db * 32;  // first column of the block
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {    // 16 tokens per value k-step
                        u32x4_t a;
                        if constexpr (FP8) {
                            // 8-bit transposing read: in each 16-lane group,
                            // input lane 2t+u points at row R(t), columns
                            // c0 + 8u .. +7; output lane j receives column
                            // c0 + j of rows R(0..7), here the k-slots of the
                            // value operand (tokens 4*half + {0..3, 8..11})
                            const int g16 = lane & 15;
                            const int t8 = g16 >> 1;
                            const int col = cb + 16 * ((lane >> 4) & 1) + 8 * (g16 & 1);
                            const int tok = sub * 32 + kh * 16 + 4 * half + (t8 < 4 ? t8 : t8 + 4);
                            const int pc = (col >> 4) ^ vswz(tok);
                            const i32x2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                (__attribute__((address_space(3))) i32x2_t *)(V + tok * ROWB_V + (pc << 4) + (col & 15)));
                            // E4M3FN -> bf16 is exact; the hardware conversion
                            // decodes the OCP format
                            a = u32x4_t{cvt_e4m3x2_bf16<false>(raw[0]), cvt_e4m3x2_bf16<true>(raw[0]),
                                        cvt_e4m3x2_bf16<false>(raw[1]), cvt_e4m3x2_bf16<true>(raw[1])};
                        } else {
                            // transposing reads: input lane 4t+u of each 16-lane
                            // group points at row T(t), columns 4u..4u+3; output
                            // lane j receives column j of rows T(0..3)
                            const int g16 = lane & 15;
                            const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
#pragma unroll
                            for (int r = 0; r < 2; ++r) {
                                const int tok = sub * 32 + kh * 16 + 8 * r + 4 * half + (g16 >> 2);
                                const int pc = (col >> 3) ^ vswz(tok);
                                const uint8_t *src = V + tok * ROWB_V + (pc << 4) + (col & 7) * 2;
                                const i16x4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                    (__attribute__((address_space(3))) i16x4_t *)(src));
                                const u32x2_t w2 = __builtin_bit_cast(u32x2_t, v4);
                                a[2 * r] = w2[0];
                                a[2 * r + 1] = w2[1];
                            }
                        }
                        const u32x4_t bop = {pk[4 * kh], pk[4 * kh + 1], pk[4 * kh + 2], pk[4 * kh + 3]};
                        oacc[db] = mfma32x32x16(as_bf16x8(a), as_bf16x8(bop), oacc[db]);
                    }
                }
            }
        };
#pragma unroll
        for (int i = 0; i < NSUB / TS; ++i) {
            const int sub = ts + i * TS;
            const int tok0 = t * TN + sub * 32;
            if (tok0 >= len)
                break;  // rest of the last tile is past the range
            if constexpr (FP8)
                sub_tile(sub, tok0 + 32 > len);
            else if (tok0 + 32 > len)
                sub_tile(sub, std::true_type{});
            else
                sub_tile(sub, std::false_type{});
        }
    }
    wait_vm<0>();  // trailing index copies
    float lrow = l_part + swap_halves(l_part);

    // ---- merge the token shares ----
    // Slots live in the ring, free once every wave is past the last tile.  The
    // 32-column block db of a column share belongs to the wave whose token
    // share is db mod TS: every wave publishes its (max, sum) and the blocks
    // it does not own, then merges and stores the blocks it owns, so the LDS
    // reads and the stores spread over all waves.  A share that saw no token
    // has max -inf and weight exactly 0; share 0 always saw the range's first
    // token, so the merged max is finite.
    if constexpr (TS > 1) {
        // (max, sum) per share: [NQB][CS][TS][2][32] floats; blocks: [NQB][CS]
        // [DBW][TS - 1 sources][32 rows][OST] words of bf16 pairs (the shares
        // travel rounded to bf16, as the partial outputs leave the kernel; the
        // owner's own share stays fp32), rows padded to 18 words so that the
        // 8-byte accesses of 16 lanes fall on distinct banks
        constexpr int OST = 18;
        constexpr int BLK = 32 * OST;
        constexpr int ML = NQB * CS * TS * 64;
        static_assert((ML + NQB * CS * DBW * (TS - 1) * BLK) * 4 <= NBUF * G::STAGE, "merge slots fit the ring");
        float *ml = (float *)s_ring + (qbw * CS + cs) * TS * 64;
        uint32_t *ob = (uint32_t *)s_ring + ML + (qbw * CS + cs) * DBW * (TS - 1) * BLK;
        lds_barrier();
        if (half == 0) {
            ml[ts * 64 + l32] = m_ref;
            ml[ts * 64 + 32 + l32] = lrow;
        }
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
            const int owner = db % TS;
            if (owner != ts) {  // source slot of this share in the owner's list
                uint32_t *dst = ob + (db * (TS - 1) + (ts < owner ? ts : ts - 1)) * BLK + l32 * OST + 2 * half;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *(u32x2_t *)(dst + 4 * g4) = u32x2_t{pack_bf16x2(oacc[db][4 * g4], oacc[db][4 * g4 + 1]),
                                                         pack_bf16x2(oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3])};
            }
        }
        lds_barrier();
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < TS; ++k)
            mx = fmaxf(mx, ml[k * 64 + l32]);
        float lsum = 0.0f;
#pragma unroll
        for (int k = 0; k < TS; ++k)
            lsum += __builtin_amdgcn_exp2f(ml[k * 64 + l32] - mx) * ml[k * 64 + 32 + l32];
        // weights of this wave's share and of the other shares, in slot order
        const float a_own = __builtin_amdgcn_exp2f(m_ref - mx);
        float a_src[TS - 1];
#pragma unroll
        for (int k = 0; k < TS - 1; ++k)
            a_src[k] = __builtin_amdgcn_exp2f(ml[(k < ts ? k : k + 1) * 64 + l32] - mx);
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
            if (db % TS != ts)
                continue;
            // every source block's reads first, then the sums: with the reads
            // interleaved, the compiler kept two of them in flight at a time
            u32x2_t o[TS - 1][4];
#pragma unroll
            for (int k = 0; k < TS - 1; ++k) {
                const uint32_t *src = ob + (db * (TS - 1) + k) * BLK + l32 * OST + 2 * half;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    o[k][g4] = *(const u32x2_t *)(src + 4 * g4);
            }
            oacc[db] *= a_own;
#pragma unroll
            for (int k = 0; k < TS - 1; ++k)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t w = o[k][g4][e >> 1];
                        oacc[db][4 * g4 + e] += a_src[k] * __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
                    }
        }
        lrow = lsum;
        m_ref = mx;
    }

    // ---- epilogue: normalised, v_scale-multiplied partial (bf16) and its lse;
    // each wave stores the column blocks it owns ----
    const int r = row0 + qbw * 32 + l32;
    if (r < rows) {
        const float inv = p.v_scale / lrow;
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
            if (db % TS != ts)
                continue;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int dv = cs * DWV + db * 32 + 8 * g4 + 4 * half;
                const u32x2_t o = {pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                                   pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
                *(u32x2_t *)(po + (int64_t)r * DV + dv) = o;
            }
        }
        if (ts == 0 && cs == 0 && half == 0)
            pl[r] = (m_ref + __log2f(lrow)) * kLn2;
    }
}

// ---------------------------------------------------------- combine kernel ---
// One wavefront per output row (sequence b, KV head, query row r).  Loads are issued in two dependent
// rounds: the index pointers, then every range's log-sum-exp (one per lane),
// the first PRE partial outputs, the query row and the first PRE_D draft rows
// at once.  Then: (a) log-sum-exp merge of the ranges, (b) the draft block in
// fp32 (query not cast, no k/v scale) over the visible draft keys -- causal,
// or a tree mask (aiter_backend.py's custom_mask / mask_indptr with the prefix
// columns skipped), (c) the final two-way merge and a round-to-nearest-even
// bf16 store.  A row that sees no key at all is written as 0.
template <int VPL>
__device__ __forceinline__ void load_bf16_row(const uint16_t *src, float (&dst)[VPL])
{
    if constexpr (VPL == 4) {
        const u32x2_t w = *(const u32x2_t *)src;
        dst[0] = bf16_to_f32(w[0] & 0xffffu);
        dst[1] = bf16_to_f32(w[0] >> 16);
        dst[2] = bf16_to_f32(w[1] & 0xffffu);
        dst[3] = bf16_to_f32(w[1] >> 16);
    } else if constexpr (VPL == 2) {
        const uint32_t w = *(const uint32_t *)src;
        dst[0] = bf16_to_f32(w & 0xffffu);
        dst[1] = bf16_to_f32(w >> 16);
    } else {
        dst[0] = bf16_to_f32(*src);
    }
}

// PRE (partial rows per load batch) and PRE_D (draft rows loaded in the
// second round) are the host's choice from static shapes: every load of a
// batch is issued, and lanes past the sequence's ranges or draft rows re-read
// a valid row, so depths beyond what the batch needs only move duplicate
// bytes (a decode step has one or two ranges and one draft row per sequence).
template <int D, int DV, int PRE, int PRE_D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const int32_t *kv_indptr, const int32_t *qo_indptr, int32_t bs, int32_t mode, int32_t split_tokens,
    int32_t n_splits, int32_t h_kv, int32_t rows, const CombineParams p)
{  // leading arguments preloaded into SGPRs, as for the prefix kernel
    constexpr int VPL = D / 64;    // elements of a query / key row per lane
    constexpr int VPLV = DV / 64;  // elements of a value / output row per lane
    static_assert(PRE >= 1 && PRE <= 64 && PRE_D >= 1 && PRE_D <= 64, "preload depths");

    const int lane = threadIdx.x & 63;
    // the plan keeps bs * h_kv * rows below 2^31
    const uint32_t gr = blockIdx.x * kCombineRowsPerBlock + (threadIdx.x >> 6);
    if (gr >= (uint32_t)(bs * h_kv * rows))
        return;  // padding wave of the last workgroup
    const int r = (int)(gr % (uint32_t)rows);
    const uint32_t t = gr / (uint32_t)rows;
    const int kvh = (int)(t % (uint32_t)h_kv);
    const int b = (int)(t / (uint32_t)h_kv);
    const int hg = r / p.l_ext;
    const int di = r % p.l_ext;
    const int h = kvh * p.group + hg;
    const int d0 = lane * VPL;    // this lane's query / key elements
    const int dv0 = lane * VPLV;  // this lane's value / output elements

    // ---- first load round: where this sequence's rows and ranges are ----
    const int qo = qo_indptr[b];
    // modes 0, 2 and 3: the prefix pass recorded the sequence's first range and
    // range count (only for sequences with a prefix; an empty one has none)
    const int32_t k0 = kv_indptr[b], k1 = kv_indptr[b + 1];
    const i32x2_t tab = ((const i32x2_t *)p.seq_ranges)[b];
    asm volatile("" ::"s"(p.q), "s"(p.k_ext), "s"(p.v_ext), "s"(p.part_o), "s"(p.part_lse), "s"(p.q_s0),
                 "s"(p.q_s1), "s"(p.ke_s0), "s"(p.ke_s1), "s"(p.ve_s0), "s"(p.ve_s1), "s"(p.group), "s"(p.l_ext)
                 : "memory");
    const int32_t base = mode == 1 ? b * n_splits : tab[0];
    const int32_t count = mode == 1 ? n_splits : (k1 > k0 ? tab[1] : 0);
    const int L = p.l_ext;
    int64_t mrow = 0;  // this row's tree-mask bytes for the draft keys
    if (p.mask)
        mrow = p.mask_indptr[b] + (int64_t)di * (k1 - k0 + L) + (k1 - k0);

    // ---- second load round: log-sum-exps, partial outputs, query row, draft rows ----
    const int64_t lse_step = (int64_t)p.h_kv * p.rows;  // next range, same head and row
    const float *lse_row = p.part_lse + ((int64_t)base * p.h_kv + kvh) * p.rows + r;
    const uint16_t *o_row = p.part_o + (((int64_t)base * p.h_kv + kvh) * p.rows + r) * DV + dv0;
    const int64_t o_step = lse_step * DV;
    // Every load below is unconditional: a lane or slot past the sequence's
    // ranges re-reads a valid address (the query row, the sequence's first
    // draft value row, or the last range) and gets weight 0, so the compiler
    // issues all loads before the first wait.
    const uint16_t *q_row = p.q + (int64_t)(qo + di) * p.q_s0 + (int64_t)h * p.q_s1;
    const uint16_t *v_row0 = p.v_ext + (int64_t)qo * p.ve_s0 + (int64_t)kvh * p.ve_s1 + dv0;
    const int last = count > 0 ? count - 1 : 0;
    float lse0 = *(lane < count ? lse_row + lane * lse_step : (const float *)q_row);  // range s = lane
    lse0 = lane < count ? lse0 : -INFINITY;
    float ov[PRE][VPLV];
#pragma unroll
    for (int i = 0; i < PRE; ++i)
        load_bf16_row<VPLV>(count > 0 ? o_row + (i < count ? i : last) * o_step : v_row0, ov[i]);
    float qv[VPL];
    load_bf16_row<VPL>(q_row + d0, qv);
    // visible draft keys j < 64 as bits: mask bytes (one lane per key) or j <= di
    uint64_t vis;
    if (p.mask) {
        const uint8_t byte = p.mask[mrow + (lane < L ? lane : 0)];
        vis = __ballot(lane < L && byte != 0);
    } else {
        vis = di >= 63 ? ~0ull : ((2ull << di) - 1);
    }
    float kd[PRE_D][VPL], vd[PRE_D][VPLV];
#pragma unroll
    for (int j = 0; j < PRE_D; ++j) {
        const int jj = j < L ? j : 0;  // rows past the sequence's drafts are loaded but unused
        load_bf16_row<VPL>(p.k_ext + (int64_t)(qo + jj) * p.ke_s0 + (int64_t)kvh * p.ke_s1 + d0, kd[j]);
        load_bf16_row<VPLV>(p.v_ext + (int64_t)(qo + jj) * p.ve_s0 + (int64_t)kvh * p.ve_s1 + dv0, vd[j]);
    }

    // ---- (a) prefix ranges ----
    float m = lse0;
    for (int s = 64 + lane; s < count; s += 64)
        m = fmaxf(m, lse_row[s * lse_step]);
    m = wave_max(m);
    float den = 0.0f;
    float acc[VPLV];
#pragma unroll
    for (int v = 0; v < VPLV; ++v)
        acc[v] = 0.0f;
    if (m > -INFINITY) {  // an empty range (lse -inf) has weight 0 and output 0
        float e = lane < count ? __expf(lse0 - m) : 0.0f;
        for (int s = 64 + lane; s < count; s += 64)
            e += __expf(lse_row[s * lse_step] - m);
        den = wave_sum(e);
        // ranges in batches of PRE: every load of a batch is issued before
        // any is used; lanes hold the log-sum-exps of 64 ranges at a time
        // lane l holds the weight of range (s0 & ~63) + l (0 past count)
        float w_c = lane < count ? __expf(lse0 - m) : 0.0f;
        for (int s0 = 0; s0 < count; s0 += PRE) {
            if (s0 > 0) {
                if ((s0 & 63) == 0) {
                    const int sl = s0 + lane;
                    const float lse_c = lse_row[(sl < count ? sl : last) * lse_step];
                    w_c = sl < count ? __expf(lse_c - m) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < PRE; ++i)
                    load_bf16_row<VPLV>(o_row + (s0 + i < count ? s0 + i : last) * o_step, ov[i]);
            }
#pragma unroll
            for (int i = 0; i < PRE; ++i) {
                const float w = lane_f(w_c, (s0 & 63) + i);
#pragma unroll
                for (int v = 0; v < VPLV; ++v)
                    acc[v] += w * ov[i][v];
            }
        }
    }

    // ---- (b) visible draft keys: fp32, query not cast, no k/v scale ----
    float sj[PRE_D];
#pragma unroll
    for (int j = 0; j < PRE_D; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            dot += qv[v] * kd[j][v];
        sj[j] = dot;
    }
#pragma unroll
    for (int j = 0; j < PRE_D; ++j)
        sj[j] = wave_sum(sj[j]);
    float md = -INFINITY;
#pragma unroll
    for (int j = 0; j < PRE_D; ++j) {
        sj[j] *= p.sm_scale;
        if ((vis >> j) & 1)
            md = fmaxf(md, sj[j]);
    }
    float dd = 0.0f;
    float od[VPLV];
#pragma unroll
    for (int v = 0; v < VPLV; ++v)
        od[v] = 0.0f;
#pragma unroll
    for (int j = 0; j < PRE_D; ++j) {
        if ((vis >> j) & 1) {
            const float w = __expf(sj[j] - md);
            dd += w;
#pragma unroll
            for (int v = 0; v < VPLV; ++v)
                od[v] += w * vd[j][v];
        }
    }
    // draft rows beyond the preloaded ones (l_ext > PRE_D): online update
    const int jend = p.mask ? L : di + 1;
    for (int j = PRE_D; j < jend; ++j) {
        if (p.mask && !((vis >> j) & 1))
            continue;
        float kj[VPL], vj[VPLV];
        load_bf16_row<VPL>(p.k_ext + (int64_t)(qo + j) * p.ke_s0 + (int64_t)kvh * p.ke_s1 + d0, kj);
        load_bf16_row<VPLV>(p.v_ext + (int64_t)(qo + j) * p.ve_s0 + (int64_t)kvh * p.ve_s1 + dv0, vj);
        float dot = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            dot += qv[v] * kj[v];
        const float s = wave_sum(dot) * p.sm_scale;
        const float mn = fmaxf(md, s);
        const float a = __expf(md - mn);
        const float w = __expf(s - mn);
#pragma unroll
        for (int v = 0; v < VPLV; ++v)
            od[v] = od[v] * a + w * vj[v];
        dd = dd * a + w;
        md = mn;
    }

    // ---- (c) final merge of the prefix and draft parts; bf16 store ----
    // out = (acc + e^(m_d - M) * od) / (den + e^(m_d - M) * dd) with the prefix
    // terms taken relative to e^(m - M), M the larger of m and m_d
    const float mm = fmaxf(m, md);
    const float wp = den > 0.0f ? __expf(m - mm) : 0.0f;
    const float wd = dd > 0.0f ? __expf(md - mm) : 0.0f;
    const float tot = wp * den + wd * dd;
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
    uint16_t *orow = p.out + (int64_t)(qo + di) * p.o_s0 + (int64_t)h * p.o_s1 + dv0;
    uint32_t ob[VPLV];
#pragma unroll
    for (int v = 0; v < VPLV; ++v)
        ob[v] = f32_to_bf16_rne((wp * acc[v] + wd * od[v]) * inv);
    if constexpr (VPLV == 4)
        *(u32x2_t *)orow = u32x2_t{ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16)};
    else if constexpr (VPLV == 2)
        *(uint32_t *)orow = ob[0] | (ob[1] << 16);
    else
        orow[0] = (uint16_t)ob[0];
}

// ----------------------------------------------------------------- launch ---
template <bool FP8, int D, int DV>
static int launch_prefix_qb(const PrefixParams &p, int qblocks, int64_t blocks, hipStream_t s)
{
    dim3 grid((unsigned)blocks), block(prefix_waves(qblocks) * 64);
#define VA_PREFIX_ARGS p.kv_indptr, p.qo_indptr, p.kv_indices, p.bs, p.mode, p.split_tokens, p.total_tokens, \
                       p.h_kv, p.row_chunks, p.n_splits, p
    if (qblocks == 1)
        hipLaunchKernelGGL((prefix_kernel<FP8, D, DV, 1>), grid, block, 0, s, VA_PREFIX_ARGS);
    else
        hipLaunchKernelGGL((prefix_kernel<FP8, D, DV, 2>), grid, block, 0, s, VA_PREFIX_ARGS);
#undef VA_PREFIX_ARGS
    return (int)hipGetLastError();
}

template <bool FP8>
static int launch_prefix_dims(const PrefixParams &p, int head_dim, int v_head_dim, int qblocks, int64_t blocks,
                              hipStream_t s)
{
    // (head_dim, v_head_dim): equal, or one twice the other (the host checks)
    switch (head_dim * 1000 + v_head_dim) {
    case 64064: return launch_prefix_qb<FP8, 64, 64>(p, qblocks, blocks, s);
    case 64128: return launch_prefix_qb<FP8, 64, 128>(p, qblocks, blocks, s);
    case 128064: return launch_prefix_qb<FP8, 128, 64>(p, qblocks, blocks, s);
    case 128128: return launch_prefix_qb<FP8, 128, 128>(p, qblocks, blocks, s);
    case 128256: return launch_prefix_qb<FP8, 128, 256>(p, qblocks, blocks, s);
    case 256128: return launch_prefix_qb<FP8, 256, 128>(p, qblocks, blocks, s);
    case 256256: return launch_prefix_qb<FP8, 256, 256>(p, qblocks, blocks, s);
    default: return (int)hipErrorInvalidValue;
    }
}

int launch_prefix(const PrefixParams &p, int head_dim, int v_head_dim, bool kv_fp8, int qblocks, int64_t blocks,
                  void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    return kv_fp8 ? launch_prefix_dims<true>(p, head_dim, v_head_dim, qblocks, blocks, s)
                  : launch_prefix_dims<false>(p, head_dim, v_head_dim, qblocks, blocks, s);
}

template <int D, int DV, int PRE>
static void launch_combine_d(const CombineParams &p, int pre_d, dim3 grid, dim3 block, hipStream_t s)
{
#define VA_COMBINE_ARGS p.kv_indptr, p.qo_indptr, p.bs, p.mode, p.split_tokens, p.n_splits, p.h_kv, p.rows, p
    if (pre_d == 1)
        hipLaunchKernelGGL((combine_kernel<D, DV, PRE, 1>), grid, block, 0, s, VA_COMBINE_ARGS);
    else if (pre_d == 4)
        hipLaunchKernelGGL((combine_kernel<D, DV, PRE, 4>), grid, block, 0, s, VA_COMBINE_ARGS);
    else
        hipLaunchKernelGGL((combine_kernel<D, DV, PRE, 8>), grid, block, 0, s, VA_COMBINE_ARGS);
#undef VA_COMBINE_ARGS
}

template <int D, int DV>
static void launch_combine_pre(const CombineParams &p, int pre, int pre_d, dim3 grid, dim3 block, hipStream_t s)
{
    if (pre == 8)
        launch_combine_d<D, DV, 8>(p, pre_d, grid, block, s);
    else
        launch_combine_d<D, DV, 32>(p, pre_d, grid, block, s);
}

int launch_combine(const CombineParams &p, int head_dim, int v_head_dim, int pre, int pre_d, int64_t blocks,
                   void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((unsigned)blocks), block(kCombineThreads);
    switch (head_dim * 1000 + v_head_dim) {
    case 64064: launch_combine_pre<64, 64>(p, pre, pre_d, grid, block, s); break;
    case 64128: launch_combine_pre<64, 128>(p, pre, pre_d, grid, block, s); break;
    case 128064: launch_combine_pre<128, 64>(p, pre, pre_d, grid, block, s); break;
    case 128128: launch_combine_pre<128, 128>(p, pre, pre_d, grid, block, s); break;
    case 128256: launch_combine_pre<128, 256>(p, pre, pre_d, grid, block, s); break;
    case 256128: launch_combine_pre<256, 128>(p, pre, pre_d, grid, block, s); break;
    case 256256: launch_combine_pre<256, 256>(p, pre, pre_d, grid, block, s); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

const char *hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace va
