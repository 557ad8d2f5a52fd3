// internal.h -- host-side interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hstu {

// Jagged tile work list.  One entry (a piece) covers BM query rows of one
// sequence (all heads share the list; the head is the fastest-varying index
// of the flattened work index piece * H + h).  The row block's key tiles (BN
// keys each) are [0, a_end) followed by [kb_begin, kb_end) -- every other key
// tile of the block has no visible pair -- and the piece takes positions
// [p0, p1) of that list.  A block whose list is long next to the work per
// workgroup is split into several pieces ("split-K": without a softmax the
// partial sums over key ranges simply add); each piece then writes fp32
// partial sums to partial slot (slot + k), and the LN(O) * U epilogue -- or,
// without one, a combine pass -- adds them up.
struct WorkItem {
    int32_t b;
    int32_t qt;
    int32_t a_end;
    int32_t kb;     // kb_begin | kb_end << 16
    int32_t pr;     // p0 | p1 << 16
    int32_t slot;   // first partial slot of the block, or -1: not split (O written directly)
    int32_t k;      // piece index within the block
    int32_t n;      // pieces of the block
};

// The sequence of a work item, as the scheduler saw it (written next to the
// item, so that a kernel fetching the item does not wait a second round trip
// for the sequence's offsets): first row, length, history rows.
struct ItemSeq {
    int32_t row0;
    int32_t L;
    int32_t n;
    int32_t pad;
};

// Checks of the batch structure the kernels read from device memory without a
// host copy: offsets[0] >= 0, offsets non-decreasing, offsets[B] <= num_rows,
// 0 <= lengths[b] <= offsets[b+1] - offsets[b], every length <= max_seq_len,
// 0 <= ncand[b] <= length.  Runs one workgroup, copies the first failure back
// and synchronises the stream: *first = 8 b + check (check 1..6 in the order
// above), or -1 for none.  The result lives in a device variable of the
// library (one per GPU), so calls on one GPU must not overlap.
struct ValidateArgs {
    int B;
    int64_t num_rows;
    int max_seq_len;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    int packed = 0;   // (layer calls) also offsets[0] == 0 and offsets[B] == num_rows
};
hipError_t validate_batch(const ValidateArgs& a, hipStream_t stream, int64_t* first);

// A split row block: its pieces' partial sums sit in slots slot .. slot+n-1.
struct SplitBlock {
    int32_t b;
    int32_t qt;
    int32_t slot;
    int32_t n;
};

// Partial slots (one per split piece and head, BM x d fp32 each) a call may use.
constexpr int kMaxPartialSlots = 1024;
// Pieces are never shorter than this many key tiles.
constexpr int kMinPieceTiles = 8;

constexpr int kMaxSeqLen = 65536;
constexpr int kMaxPosBuckets = 8192;

// Rows per timestamp block: the attention core's key tile and its wave's
// query-row slice.
constexpr int kTsBlock = 32;
// The bf16 attention core pulls work per accelerator die (XCD, each with its
// own L2): kXcds cursors in the control block, one 128-byte line apart.
constexpr int kXcds = 8;
constexpr int kXcdCursor = 32;
constexpr int kXcdStride = 32;
constexpr int kCtrlInts = kXcdCursor + kXcds * kXcdStride;

// Workspace carve-up of the scheduler and the timestamp preparation (all
// offsets 256-byte aligned).
struct SchedLayout {
    size_t off_ctrl;   // int32[kCtrlInts]: [0] piece count, [1] work cursor of the persistent
                       // kernel, [2] split-block count, [kXcdCursor + kXcdStride x] the bf16
                       // core's cursor of accelerator die (XCD) x
    size_t off_qscan;  // int32[B + 1] exclusive prefix of query tiles per sequence
    size_t off_items;  // WorkItem[cap_pieces]
    size_t off_item_seq;   // ItemSeq[cap_pieces]
    size_t off_split;  // SplitBlock[cap]
    size_t off_part;   // float[part_slots][BM][d]: partial sums of split pieces
    size_t off_stats;  // uint32x2[cap_blk]: encoded timestamp range of 32-row block j of
                       // sequence b at index b * nblk + j
    size_t off_enc;    // uint32[num_rows]: encoded timestamp of each row
    size_t off_rowmap; // int32[num_rows]: split map of each row (see AttnCoreArgs::rowmap)
    size_t cap;        // row-block capacity = B * ceil(max_seq_len / BM)
    size_t cap_pieces; // piece capacity = cap + part_slots / H
    size_t cap_blk;    // block capacity = B * nblk
    int nblk;          // 32-row blocks per sequence = ceil(max_seq_len / 32)
    int part_slots;    // partial slots (split pieces x heads); 0: no splitting
    size_t bytes;      // total
};

// split_d: head dim of the partial slots (0 disables splitting).
SchedLayout sched_layout(int B, int H, int max_seq_len, int tile_m, int split_d, int64_t num_rows,
                         size_t base_offset, int max_part_slots = kMaxPartialSlots);

struct SchedArgs {
    int B;
    int max_seq_len;   // bound on every sequence length (sizes the cost histogram)
    int64_t cap;       // row-block capacity (split-block list)
    int64_t cap_pieces;   // piece capacity of `items`
    int cand_only;     // M-FALCON: only the query tiles that hold candidate rows
    int kv_mode;       // items are blocks of tile_m keys with their tile_n-row query tiles
    int H;
    int slots;         // workgroups of the attention core (the work per workgroup sets the piece size)
    int part_slots;    // partial slots available (0: no splitting)
    SplitBlock* split;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    int tile_m, tile_n;
    int32_t* ctrl;
    int32_t* qscan;
    WorkItem* items;
    ItemSeq* item_seq = nullptr;   // NULL: not written
    // Timestamp codes (bf16 core; enc == NULL skips them): per row
    // e = 2 (t - t_first) + 2^31 (t_first: the sequence's first row) and,
    // per 32-row block, the range [min e, max e]; a block with some
    // |t - t_first| >= 2^30 gets the range {0xffffffff, 0}.
    const int64_t* ts;
    uint32_t* enc;
    uint32_t* stats;     // pairs (min, max), block j of sequence b at b * nblk + j
    int nblk;
    int64_t cap_blk;
    // cross mode: the rows are candidates, each item's key tiles are the
    // whole history of its sequence (kv_offsets), and the codes count from
    // the history's first event (ref_offsets, ref_ts); skip_list: codes only
    const int32_t* kv_offsets = nullptr;
    const int32_t* ref_offsets = nullptr;
    const int64_t* ref_ts = nullptr;
    int skip_list = 0;
};

// Work list and timestamp codes, in one launch.
hipError_t launch_sched(const SchedArgs& a, hipStream_t stream);
// The gradients' preparation in one launch: two work lists (only the first
// may ask for timestamp codes) and gbase[b], the index of sequence b's first
// 32x32 G block (B entries).
hipError_t launch_sched_pair(const SchedArgs& a, const SchedArgs& b, int64_t* gbase, hipStream_t stream);

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
    const ItemSeq* item_seq = nullptr;   // NULL: read the sequence offsets instead
    const int32_t* ctrl;   // [0] = item count
    int32_t* cursor;       // persistent work cursor (zeroed by the scheduler)
    float* partial;        // partial slots of split pieces (bf16 core only)
    // bf16 core only: per row of every row block it computes, -1 (O written)
    // or, for a split block, slot | pieces << 16 | (row within block) << 23
    int32_t* rowmap;
    int nblk;              // timestamp blocks per sequence in `stats`
    const uint32_t* stats;
    const uint32_t* enc;
    int64_t num_rows;
    hipEvent_t ev_begin, ev_end;   // optional: stamped at the kernel's own start and end
    // cross mode (bf16 core; q_offsets != NULL): queries, their timestamps,
    // codes and block ranges in their own row space; offsets, ts, enc and
    // stats above are the keys' (a history cache), every key visible
    const int32_t* q_offsets = nullptr;
    const int64_t* ts_q = nullptr;
    const uint32_t* enc_q = nullptr;
    const uint32_t* stats_q = nullptr;
    int nblk_q = 0;
};

hipError_t launch_attn_bf16(const AttnCoreArgs& a, hipStream_t stream);

// Workgroups of the persistent bf16 attention core.
int attn_bf16_slots();

// Sums the partial slots of every split row block into its bf16 O rows.
struct CombineArgs {
    int H, d, BM;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ctrl;        // [2] = split-block count
    const SplitBlock* split;
    const float* partial;
    void* o; int64_t o_stride;
    int64_t max_blocks;         // capacity of the split-block list
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnCoreArgs& a, hipStream_t stream);

// Gradients of the bf16 attention core (d = 128): dQ by a query-major pass
// over the forward's work list (which also writes one table-gradient partial
// row per work item), dK and dV by a key-major pass over a list built with
// kv_mode, then the partial rows summed in work order.
struct AttnBwdArgs {
    int H;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    const void* q; int64_t q_stride;
    const void* k; int64_t k_stride;
    const void* v; int64_t v_stride;
    const void* dout; int64_t dout_stride;
    const int64_t* ts;
    const float* rab_pos; int P; int rp_head_stride;
    const float* rab_time; int NT; int rt_head_stride;
    float alpha;
    int act;
    void* dq; int64_t dq_stride;
    void* dk; int64_t dk_stride;
    void* dv; int64_t dv_stride;
    float* drab_pos;             // [P] or [H][P]; NULL: not computed
    float* drab_time;            // [NT] or [H][NT]; NULL: not computed
    const WorkItem* q_items;  int32_t* q_ctrl;    // query-major list (with its per-die cursors)
    const WorkItem* kv_items; int32_t* kv_ctrl;   // key-major list
    int nblk;
    const uint32_t* stats;
    const uint32_t* enc;
    int64_t num_rows;
    float* rab_part;             // [work][P + NT]
    float* rab_part2;            // [heads][chunks][P + NT]
    // G = dLoss/dS of every 32x32 block (query tile q, key tile k <= q) that
    // holds a visible pair, fp32, written by the dK/dV kernel and read by the
    // dQ kernel: block (b, q, k) of head h at ((gbase[b] + q (q + 1) / 2 + k)
    // * H + h) * 1024 floats, gbase the per-sequence prefix of
    // ceil(L / 32) (ceil(L / 32) + 1) / 2; blocks at or past gcap are
    // neither written nor read.
    float* gbuf;
    int64_t* gbase;              // [B]
    int64_t gcap;
    // K of every 32-key tile and head in the order the dQ kernel's G K reads
    // it (8 KiB each, tile kt of sequence b and head h at (b H + h) nblk + kt),
    // written by the dK/dV kernel
    void* kp;
    int B;
    hipEvent_t ev_dq_begin, ev_dq_end, ev_dkv_begin, ev_dkv_end;   // optional
};

size_t attn_bwd_rab_part_floats(int64_t cap, int H, int P, int NT);
size_t attn_bwd_rab_part2_floats(int H, int P, int NT);
// Blocks of G a batch can hold at most (every sequence no longer than
// max_seq_len, num_rows rows in all).
int64_t attn_bwd_g_blocks(int B, int max_seq_len, int64_t num_rows);
// The dQ kernel keeps four per-wave histograms of the table gradients in LDS;
// the dK/dV kernel keeps the position table next to its tile ring.
bool attn_bwd_tables_fit(int P, int NT);
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t stream);

// Gradients of Y = LayerNorm(O) * U (rows of width H * d_v, bf16): dO and dU.
struct LnGateBwdArgs {
    int B;
    int64_t num_rows;
    int width;
    const int32_t* offsets;
    const int32_t* lengths;
    const void* o; int64_t o_stride;
    const void* u; int64_t u_stride;
    const void* dy; int64_t dy_stride;
    void* dout; int64_t dout_stride;
    void* du; int64_t du_stride;
    float eps;
};

hipError_t launch_ln_gate_bwd(const LnGateBwdArgs& a, hipStream_t stream);

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
    void* o; int64_t o_stride;     // read, and written for split rows
    const void* u; int64_t u_stride;
    void* y; int64_t y_stride;   // may be NULL when scores are requested
    float eps;
    const float* w;       // NULL: no scores
    float* scores; int score_stride;
    // bf16 with split row blocks: rows whose map entry is >= 0 sum their
    // block's partial slots (BM x d fp32 each, head-major per piece) and
    // write that sum to O before normalising it.  NULL: O holds every row.
    const int32_t* rowmap;
    const float* partial;
    int H, d, BM;
    int cand_only;        // the core computed only candidate-row blocks: map only those rows
    // cross mode (bf16, d = 128): every row is a candidate scored against a
    // history cache; its own key adds alpha SiLU(q.k + rab_pos[0] +
    // rab_time[0]) v per head to O (written back) before the LayerNorm
    int cross = 0;
    const void* sq = nullptr; int64_t sqs = 0;
    const void* sk = nullptr; int64_t sks = 0;
    const void* sv = nullptr; int64_t svs = 0;
    const float* rab_pos = nullptr; int rp_hs = 0;
    const float* rab_time = nullptr; int rt_hs = 0;
    float alpha = 0.0f;
    // optional events stamped with the start / end of the launch
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
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
    void* c_pre = nullptr;   // with silu: also the value before it (bf16), or NULL
    int64_t ldcp = 0;
};

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream);

// Weight gradients: C[M, N] (fp32) = sum_t A[t, M] B[t, N] over T tokens,
// A and B bf16 token-major; M, N multiples of 128.  The tokens are split over
// `splits` workgroup layers whose fp32 partials ([splits][M][N]) are added
// in split order.
struct GemmTnArgs {
    const void* a; int64_t lda;
    const void* b; int64_t ldb;
    int64_t T;
    int M, N;
    int splits;
    float* part;
    float* c;
};
int gemm_tn_splits(int64_t T, int M, int N);
hipError_t launch_gemm_tn(const GemmTnArgs& g, hipStream_t stream);

// Column sums of a bf16 [T, C] matrix (fixed order), partials [64][C].
size_t colsum_part_floats(int C);
hipError_t launch_colsum(const void* x, int64_t ld, int64_t T, int C, float* part, float* out, hipStream_t stream);
// dZ (.)= SiLU'(P), elementwise over `count` bf16 values (count % 8 == 0).
hipError_t launch_silu_grad(void* dz, const void* pre, int64_t count, hipStream_t stream);
// out[c][r] = in[r][c], bf16.
hipError_t launch_transpose(const void* in, int R, int C, void* out, hipStream_t stream);

// Stochastic length: kept rows of every sequence (min(cap_b, L_b) by
// smallest Philox key, in order) and the gather of their rows.
constexpr int kSlMaxTensors = 8;
struct SlArgs {
    int B;
    int64_t num_rows;
    const int32_t* offsets;
    int cap;
    const int32_t* caps;
    uint64_t seed, step;
    int32_t* out_offsets;
    int64_t* out_index;
    int num_tensors;
    const void* src[kSlMaxTensors]; int64_t src_stride[kSlMaxTensors];
    void* dst[kSlMaxTensors]; int64_t dst_stride[kSlMaxTensors];
    int row_bytes[kSlMaxTensors];
};
hipError_t launch_stochastic_length(const SlArgs& a, hipStream_t stream);

int device_cu_count();

}  // namespace hstu
