// va_internal.h -- internal definitions shared by the host side and the HIP
// kernels of the verify-attention library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "verify_attn.h"

namespace va {

// Rows of one KV head's query tile are processed in chunks of at most this
// many rows (2 MFMA column blocks of 32).
constexpr int kRowChunk = 64;
// Granule of the pages' equal-split rule (ranges are rounded up to it).
constexpr int kEvenSplitGranule = 32;
// The combine kernel runs one wavefront per output row, one row per
// workgroup (the rows then spread over every CU).
constexpr int kCombineThreads = 64;
constexpr int kCombineRowsPerBlock = kCombineThreads / 64;
// Prefix kernel shape.  A workgroup is one group of 4 waves per 32-row query
// block.  One query block: 4 waves and a 2-tile LDS ring of K/V tiles
// (<= 32 KB each), two workgroups per CU (their tiles differ, so no score work
// is repeated).  Two query blocks: 8 waves and a 4-tile ring, one workgroup
// per CU.  The split heuristic aims for that many resident workgroups per CU.
constexpr int prefix_waves(int qblocks) { return qblocks == 1 ? 4 : 8; }
constexpr int prefix_ring_stages(int qblocks) { return qblocks == 1 ? 2 : 4; }
constexpr int prefix_resident_per_cu(int qblocks) { return qblocks == 1 ? 2 : 1; }
// Draft tokens a tree mask may cover (the combine kernel keeps a row's
// visibility in one 64-bit ballot).
constexpr int kMaxTreeDrafts = 64;
// Smallest range the heuristic chooses; ranges are multiples of this.
constexpr int kSplitQuantum = 64;
// When a batch has more sequences than the CUs hold prefix workgroups, ranges
// of about this many K/V bytes per KV head let the dispatcher balance the
// rounds of workgroups (1024 tokens at bf16 D = Dv = 256).
constexpr int64_t kRoundRangeBytes = int64_t(1) << 20;
// Those ranges in tokens (a multiple of kSplitQuantum, at least one): the
// planner sizes the grid with it and the kernels bound their fit with it.
constexpr int round_range_tokens(int head_dim, int v_head_dim, int elem_bytes)
{
    const int64_t c = kRoundRangeBytes / ((int64_t)(head_dim + v_head_dim) * elem_bytes) / kSplitQuantum * kSplitQuantum;
    return c >= kSplitQuantum ? (int)c : kSplitQuantum;
}
// Size of the library-owned device array verify_attn_run_noalloc keeps its
// partials in (va_noalloc.hip): the headline and 64k-prefix workloads need
// 8.5 MB of it on MI355X.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// Prefix tokens per LDS tile: as many as keep a tile within 32 KB when K and
// V rows both had the larger head dim, at most 128 (bf16 D=256: 32; fp8
// D=128: 128).
constexpr int tile_tokens_for(int head_dim, int v_head_dim, int elem_bytes)
{
    const int dm = head_dim > v_head_dim ? head_dim : v_head_dim;
    return 16384 / (dm * elem_bytes) > 128 ? 128 : 16384 / (dm * elem_bytes);
}

// Head-dim pairs the kernels are built for: both in {64, 128, 256}, equal
// or one twice the other.
constexpr bool supported_head_dims(int head_dim, int v_head_dim)
{
    const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
    const bool dv_ok = v_head_dim == 64 || v_head_dim == 128 || v_head_dim == 256;
    return d_ok && dv_ok &&
           (head_dim == v_head_dim || head_dim == 2 * v_head_dim || v_head_dim == 2 * head_dim);
}

// 32-row query blocks (MFMA column blocks) per row chunk: 1 or 2.
inline int query_blocks_for(int rows_in_chunk) { return rows_in_chunk <= 32 ? 1 : 2; }

struct PrefixParams {
    const uint16_t *q;
    const uint8_t *k_buf;  // byte pointers: the pool is bf16 or fp8
    const uint8_t *v_buf;
    const int32_t *qo_indptr;
    const int32_t *kv_indptr;
    const int64_t *kv_indices;
    // page-table prefix (NULL: kv_indices): token t of sequence b is pool row
    // block_table[b * bt_s0 + t / page_size] * page_size + t % page_size
    const int32_t *block_table;
    int64_t bt_s0;
    int32_t page_size;
    uint16_t *part_o;  // [range_slots * h_kv, rows, D] bf16 (round to nearest even)
    float *part_lse;   // [range_slots * h_kv, rows]    fp32 (natural log)
    int32_t *seq_ranges;  // [bs][2]: first range and range count of each sequence (modes 0, 2, 3)
    int64_t q_s0, q_s1;        // elements
    uint32_t kb_s0, vb_s0;     // pool row strides, bytes (< 2^32, checked on the host)
    int64_t kb_s1, vb_s1;      // pool head strides, bytes
    float qk_scale_log2;       // sm_scale * k_scale * log2(e)
    float v_scale;
    int32_t bs, h_kv, group, l_ext, rows, row_chunks;
    int32_t mode, split_tokens, n_splits;  // plan.mode (0 fitted, 1 n_splits, 2 explicit size)
    int32_t total_tokens;  // num_kv_indices
};

struct CombineParams {
    const uint16_t *q;
    const uint16_t *k_ext;
    const uint16_t *v_ext;
    const int32_t *qo_indptr;
    const int32_t *kv_indptr;
    const uint16_t *part_o;
    const float *part_lse;
    const int32_t *seq_ranges;  // written by the prefix pass (modes 0, 2, 3)
    uint16_t *out;
    const uint8_t *mask;          // tree mask bytes, or NULL for the causal draft block
    const int64_t *mask_indptr;   // [bs + 1] byte offsets of each sequence's mask
    int64_t q_s0, q_s1, ke_s0, ke_s1, ve_s0, ve_s1, o_s0, o_s1;  // elements
    float sm_scale;
    int32_t bs, h_kv, group, l_ext, rows;
    int32_t mode, split_tokens, n_splits;
};

// Threads per workgroup of the append and kv_indices kernels (va_aux.hip).
constexpr int kAuxThreads = 256;

struct AppendParams {
    const uint16_t *k;        // [n, h_kv, D] bf16
    const uint16_t *v;        // [n, h_kv, Dv] bf16
    const int64_t *loc;       // [n] pool rows
    uint8_t *k_buf;           // pool bytes (bf16 or E4M3FN)
    uint8_t *v_buf;
    int64_t n;
    int32_t h_kv;
    int64_t k_s0, k_s1, v_s0, v_s1;      // elements
    int64_t kb_s0, kb_s1, vb_s0, vb_s1;  // bytes
    float k_scale, v_scale;
};

struct BuildIndicesParams {
    const int32_t *req_to_token;
    int64_t rt_stride;               // elements per req_to_token row
    const int64_t *req_pool_indices;
    const int32_t *seq_lens;
    const int32_t *kv_start_idx;     // or NULL
    int32_t *kv_indptr;              // [bs + 1] out
    int64_t *kv_indices;             // [capacity] out
    int64_t capacity;
    int32_t bs, parts;               // parts: workgroups per request
};

int launch_append(const AppendParams &p, int head_dim, int v_head_dim, bool kv_fp8, void *stream);
int launch_build_kv_indices(const BuildIndicesParams &p, void *stream);

// Launchers (defined in va_kernels.hip).  Return a hipError_t value.
int launch_prefix(const PrefixParams &p, int head_dim, int v_head_dim, bool kv_fp8, int qblocks,
                  int64_t blocks, void *stream);
// pre: partial rows per load batch (8 or 32); pre_d: draft rows preloaded (1, 4 or 8)
int launch_combine(const CombineParams &p, int head_dim, int v_head_dim, int pre, int pre_d, int64_t blocks,
                   void *stream);
const char *hip_error_string(int err);

// Host-side validation and planning (defined in va_plan.cpp).
int check_desc(const va_desc_t *d, int32_t l_ext);
int make_plan(const va_desc_t *d, int32_t l_ext, int32_t num_cus, va_plan_t *plan);
int current_device_cus(int32_t *cus);
// Address of the current device's copy of the verify_attn_run_noalloc array
// (va_noalloc.hip), resolved once per device.
int noalloc_scratch(void **ptr);
void set_error(const char *fmt, ...);
void clear_error();

}  // namespace va
