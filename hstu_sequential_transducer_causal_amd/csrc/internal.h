// internal.h -- host-side interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hstu {

// Jagged tile work list.  One item covers BM query rows of one sequence
// (all heads share the item list; the head is the fastest-varying index of
// the flattened work index item * H + h).  Its key tiles (BN keys each) are
// [0, a_end) followed by [kb_begin, kb_end); every other key tile of the row
// block has no visible pair and is skipped.
struct WorkItem {
    int32_t b;
    int32_t qt;
    int32_t a_end;
    int32_t kb;  // kb_begin | kb_end << 16
};

constexpr int kMaxSeqLen = 65536;
constexpr int kMaxPosBuckets = 8192;

// Rows per timestamp block: the attention core's key tile and its wave's
// query-row slice.
constexpr int kTsBlock = 32;

// Workspace carve-up of the scheduler and the timestamp preparation (all
// offsets 256-byte aligned).
struct SchedLayout {
    size_t off_ctrl;   // int32[64]: [0] item count, [1] work cursor of the persistent kernel
    size_t off_qscan;  // int32[B + 1] exclusive prefix of query tiles per sequence
    size_t off_bscan;  // int32[B + 1] exclusive prefix of 32-row timestamp blocks per sequence
    size_t off_items;  // WorkItem[cap]
    size_t off_stats;  // uint32x2[cap_blk]: encoded timestamp range of each 32-row block
    size_t off_enc;    // uint32[num_rows]: encoded timestamp of each row
    size_t cap;        // item capacity = B * ceil(max_seq_len / BM)
    size_t cap_blk;    // block capacity = B * ceil(max_seq_len / 32)
    size_t bytes;      // total
};

SchedLayout sched_layout(int B, int max_seq_len, int tile_m, int64_t num_rows, size_t base_offset);

struct SchedArgs {
    int B;
    int max_seq_len;   // bound on every sequence length (sizes the cost histogram)
    int64_t cap;       // item capacity of `items`
    int cand_only;     // M-FALCON: only the query tiles that hold candidate rows
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    int tile_m, tile_n;
    int32_t* ctrl;
    int32_t* qscan;
    int32_t* bscan;
    WorkItem* items;
};

// Per-row timestamp code e = 2 (t - t_first) + 2^31 (t_first: the sequence's
// first row) and, per 32-row block of a sequence, the range [min e, max e];
// a block with some |t - t_first| >= 2^30 gets the range {0xffffffff, 0}.
struct TsPrepArgs {
    int B;
    const int32_t* offsets;
    const int32_t* lengths;
    const int64_t* ts;
    const int32_t* bscan;
    uint32_t* enc;
    uint32_t* stats;     // pairs (min, max)
    int64_t cap_blk;
};

hipError_t launch_ts_prep(const TsPrepArgs& a, hipStream_t stream);

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream);

// Attention core, bf16 with MFMA, d_qk = d_v = 128.
constexpr int kBf16TileM = 128;
constexpr int kBf16TileN = 32;

// Attention core, fp32 (VALU), d in {32, 64}.
constexpr int kF32TileM = 64;
constexpr int kF32TileN = 64;

struct AttnCoreArgs {
    int H, d;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    const void* q; int64_t q_stride;
    const void* k; int64_t k_stride;
    const void* v; int64_t v_stride;
    const int64_t* ts;
    const float* rab_pos; int P; int rp_head_stride;
    const float* rab_time; int NT; int rt_head_stride;
    float alpha;
    int act;
    void* o; int64_t o_stride;
    const WorkItem* items;
    const int32_t* ctrl;   // [0] = item count
    int32_t* cursor;       // persistent work cursor (zeroed by the scheduler)
    const int32_t* bscan;  // timestamp blocks (bf16 core only)
    const uint32_t* stats;
    const uint32_t* enc;
    int64_t num_rows;
    hipEvent_t ev_begin, ev_end;   // optional: stamped at the kernel's own start and end
};

hipError_t launch_attn_bf16(const AttnCoreArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnCoreArgs& a, hipStream_t stream);

// LayerNorm(O_row) * U_row epilogue, optionally scored against w for the
// candidate rows (M-FALCON).
struct LnGateArgs {
    int B;
    int64_t num_rows;
    int width;            // H * d_v
    int dtype;            // HSTU_F32 / HSTU_BF16
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    const void* o; int64_t o_stride;
    const void* u; int64_t u_stride;
    void* y; int64_t y_stride;   // may be NULL when scores are requested
    float eps;
    const float* w;       // NULL: no scores
    float* scores; int score_stride;
};

hipError_t launch_ln_gate(const LnGateArgs& a, hipStream_t stream);

// bf16 GEMMs of the layer: C[M, N] = A[M, K] * B[N, K]^T (both K-contiguous).
struct GemmArgs {
    int64_t M;
    int N, K;
    const void* a; int64_t lda;
    const void* b; int64_t ldb;
    const float* bias;       // [N] or NULL
    const void* residual;    // [M, N] bf16 or NULL (added after the bias)
    int64_t ldr;
    void* c; int64_t ldc;
    int silu;                // apply SiLU to the result
};

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream);

int device_cu_count();

}  // namespace hstu
