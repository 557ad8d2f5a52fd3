// attn_bwd.hip -- gradients of the attention core for gfx950: bf16 inputs,
// fp32 accumulation, d_qk = d_v = 128.
//
// The forward ("生成式推荐（一）：HSTU", sections "高性能自注意力Encoder：HSTU"
// and "Pointwise aggregated attention") computes, per head and visible pair
// (i, j) of a jagged sequence,
//   S_ij = <Q_i, K_j> + rab_pos[pb(i, j)] + rab_time[tb(i, j)],
//   O_i  = alpha * sum_j SiLU(S_ij) V_j.
// With dO = dLoss/dO given, the chain rule gives
//   dV_j += alpha SiLU(S_ij) dO_i,
//   G_ij  = alpha <dO_i, V_j> SiLU'(S_ij)            (= dLoss/dS_ij),
//   dQ_i += G_ij K_j,   dK_j += G_ij Q_i,
//   drab_pos[pb(i, j)] += G_ij,   drab_time[tb(i, j)] += G_ij,
// with SiLU'(x) = s + SiLU(x) (1 - s), s = sigmoid(x) (identity: 1).
//
// Two persistent kernels, with no atomics on the gradients of Q, K and V;
// both pull their work lists per accelerator die (entry f H + k runs head
// (k - b) mod H, so a die meets the same sequence-heads' operands in its L2):
//   * attn_bwd_dkv_kernel (first): one work item = 128 keys x 1 head (a
//     key-major work list: the 32-row query tiles that see the keys).  Per
//     query tile: S = Q K^T and dO V^T with K and V in registers, then
//     dV += A^T dO and dK += G^T Q (A = SiLU(S) masked).  It also stores, for
//     the dQ kernel, G of every 32 x 32 block holding a visible pair (fp32, in
//     its own register order: lane = key, 16 queries per lane) and its K
//     fragments in the order G K reads them.  A tile feeds two products that
//     read it in different orders (rows as M, and rows as the contraction); it
//     is staged twice, in the two swizzles those reads are conflict-free in.
//     Tiles arrive by direct-to-LDS buffer loads two tiles ahead of use (a
//     3-stage ring).  The relative bias takes the forward's block-uniform
//     shortcuts (a constant time bucket, a fully clamped position bucket) and
//     otherwise reads per element.
//   * attn_bwd_dq_kernel (second): one work item = 128 query rows x 1 head
//     (the forward's work list); each wave streams its 32-row tile's G blocks
//     and K fragments (buffer loads, fixed counts per step), turns each G
//     block over with two identity MFMAs (lane = key to lane = query) and
//     accumulates dQ += G K.  The exact fp32 G is also summed by position and
//     time bucket into per-wave LDS histograms, written as one partial row per
//     work item and added up in a fixed order by rab_grad_partial_kernel and
//     rab_grad_final_kernel (so the table gradients do not depend on which
//     workgroup took which item).  LDS float atomics are slow, so the common
//     cases avoid them per element: a block of history rows sums its 63
//     position diagonals through a skewed LDS scratch, a block of candidate
//     rows (one position) sums its key columns across the lanes, and a block
//     spanning at most four time buckets sums them in registers; one atomic
//     per bucket then adds each sum.
#include <hip/hip_ext.h>

#include "internal.h"
#include "hstu_device.h"
#include "tile_ops.h"
#include "tile_stream.h"

namespace hstu {

namespace {

constexpr int HD = 128;
constexpr int kThreads = 256;
constexpr int kBlk = 128;          // query rows (dq) or keys (dkv) per work item
constexpr int kStages = 3;         // tiles t .. t+2 in flight
constexpr int kDiagPitch = 36;     // floats per column of the dQ kernel's diagonal scratch

struct BwdParams {
    int H;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    const uint16_t* q; int64_t qs;
    const uint16_t* k; int64_t ks;
    const uint16_t* v; int64_t vs;
    const uint16_t* g; int64_t gs;          // dO
    const int64_t* ts;
    const float* rab_pos; int P; int rp_hs;
    const float* rab_time; int NT; int rt_hs;
    float alpha;
    int act;                                // 0: SiLU, 1: identity
    uint16_t* dq; int64_t dqs;
    uint16_t* dk; int64_t dks;
    uint16_t* dv; int64_t dvs;
    const WorkItem* items;
    const int32_t* ctrl;
    int nblk;
    const uint32_t* stats;
    const uint32_t* enc;
    float* rab_part;                        // [work][P + NT] (dq kernel)
    float* gbuf;                            // G blocks (written by dK/dV, read by dQ)
    const int64_t* gbase;
    int64_t gcap;
    uint16_t* kp;                           // K fragments for G K (written by dK/dV, read by dQ)
};

// Small LDS state after the tile ring.
struct Small {
    uint32_t codes[kStages][64];   // the streamed tile's 32 row codes (the loads write 64 lanes)
    float tt_fast[32];             // by leading-zero count of 2|dt| + 1
    float tt_wide[65];             // by bit length of |dt|
    int32_t item[8];
    int32_t work;
};

template <int kTiles>
__device__ __forceinline__ Small& small_of(uint8_t* smem) {
    return *reinterpret_cast<Small*>(smem + kTiles * kStages * kTileBytes);
}
template <int kTiles>
__device__ __forceinline__ float* ptab_of(uint8_t* smem) {
    return reinterpret_cast<float*>(smem + kTiles * kStages * kTileBytes + ((sizeof(Small) + 15) & ~size_t(15)));
}

// Wave 0 only: the 32 row codes of tile `tile` (lanes 32-63 write zeros).
__device__ __forceinline__ void issue_codes(const u32x4& wrs, int64_t enc_row0, Small& s, int stage, int tile,
                                            int L, int lane) {
    const int j = tile * 32 + lane;
    uint32_t off = 0x80000000u;   // out of range: lands as 0
    if (lane < 32 && j < L) off = (uint32_t)(enc_row0 + 4 * (int64_t)j);
    dma4(wrs, uniu(lds_addr(s.codes[0]) + (uint32_t)(stage * 64 * 4)), off);
}

__device__ __forceinline__ void wait_tile(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
        case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// Keeps a value loaded before the tile loop out of the loop's wait counts:
// its load is waited for here, once.
template <typename T>
__device__ __forceinline__ void settle(T& x) { asm volatile("" : "+v"(x)); }

// Bias tables of head h into LDS: rab_pos in bucket order, and the time
// table by leading-zero count of 2|dt| + 1 and by bit length of |dt|.
__device__ __forceinline__ void load_tables(const BwdParams& p, int h, float* ptab, Small& s, int tid) {
    const float* rp = p.rab_pos + (int64_t)h * p.rp_hs;
    const float* rt = p.rab_time + (int64_t)h * p.rt_hs;
    for (int e = tid; e < p.P; e += kThreads) ptab[e] = rp[e];
    if (tid < 32) s.tt_fast[tid] = rt[min(p.NT - 1, 31 - tid)];
    if (tid < 65) s.tt_wide[tid] = rt[min(p.NT - 1, tid)];
}

// Time buckets of one 32 x 32 block from the two 32-row blocks' code ranges:
// the bucket (as a leading-zero count) is the same for every pair when the
// range of gaps stays within one power of two.
struct TimeBlock {
    bool wide;       // some gap needs 64-bit arithmetic
    bool constant;   // one bucket for the block
    int cz;          // its leading-zero count (the block's smallest gap)
    int czhi;        // leading-zero count of its largest gap (<= cz)
};

__device__ __forceinline__ TimeBlock time_block(uint32_t amn, uint32_t amx, uint32_t bmn, uint32_t bmx) {
    TimeBlock t;
    t.wide = amn > amx || bmn > bmx;
    const uint32_t lo = amn >= bmx ? amn - bmx : (bmn >= amx ? bmn - amx : 0u);
    const uint32_t hi = max(amx >= bmn ? amx - bmn : 0u, bmx >= amn ? bmx - amn : 0u);
    const int czlo = (int)clz_gap(lo), czhi = (int)clz_gap(hi);
    t.constant = !t.wide && czlo == czhi;
    t.cz = czlo;
    t.czhi = czhi;
    return t;
}

// Floats per copy of the dK/dV kernel's padded position table (P + 128,
// rounded up to a multiple of 4).
__host__ __device__ __forceinline__ int ptab2_width(int P) { return (P + 128 + 3) & ~3; }

// Activation value and slope: SiLU (x s, s + x s (1 - s) with s = sigmoid(x))
// or the identity (x, 1).
__device__ __forceinline__ void act_and_slope(float x, bool silu, float& a, float& slope) {
    if (silu) {
        const float e = __builtin_amdgcn_exp2f(-x * kLog2e);
        const float sg = __builtin_amdgcn_rcpf(1.0f + e);
        a = x * sg;
        slope = sg + a * (1.0f - sg);
    } else {
        a = x;
        slope = 1.0f;
    }
}

// 16 values (the 32x32 accumulator's order) -> two A operands of 16-long
// contraction chunks.
__device__ __forceinline__ void pack_a(const float (&x)[16], bf16x8 (&pa)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(x[8 * c + 2 * e], x[8 * c + 2 * e + 1]);
        pa[c] = __builtin_bit_cast(bf16x8, pk);
    }
}

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p, bool valid) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (valid) z = *reinterpret_cast<const u32x4*>(p);
    return __builtin_bit_cast(bf16x8, z);
}

// Sum over the wave's 64 lanes, complete in lane 63 (DPP row shifts, then
// the row broadcasts 15 and 31; no LDS traffic).  Fixed order, so the same
// inputs give the same bits.
__device__ __forceinline__ float wave_total(float v) {
    auto dpp = [](float x, int ctrl_id) -> float {
        int xi = __builtin_bit_cast(int, x);
        int r;
        switch (ctrl_id) {
            case 0: r = __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xF, 0xF, true); break;   // row_shr:1
            case 1: r = __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xF, 0xF, true); break;   // row_shr:2
            case 2: r = __builtin_amdgcn_update_dpp(0, xi, 0x114, 0xF, 0xF, true); break;   // row_shr:4
            case 3: r = __builtin_amdgcn_update_dpp(0, xi, 0x118, 0xF, 0xF, true); break;   // row_shr:8
            case 4: r = __builtin_amdgcn_update_dpp(0, xi, 0x142, 0xA, 0xF, false); break;  // row_bcast:15
            default: r = __builtin_amdgcn_update_dpp(0, xi, 0x143, 0xC, 0xF, false); break; // row_bcast:31
        }
        return __builtin_bit_cast(float, r);
    };
    v = v + dpp(v, 0);
    v = v + dpp(v, 1);
    v = v + dpp(v, 2);
    v = v + dpp(v, 3);
    v = v + dpp(v, 4);
    v = v + dpp(v, 5);
    return v;
}

// Block code ranges through the scalar cache (uniform addresses): these loads
// count in lgkmcnt, so waiting for them never waits for the tile loads.
typedef const __attribute__((address_space(4))) u32x2* StatsPtr;
__device__ __forceinline__ StatsPtr stats_ptr(const uint32_t* p) { return (StatsPtr)(uintptr_t)p; }

// The accelerator die (XCD) the calling workgroup runs on.
__device__ __forceinline__ int xcd_id() {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
    return (int)(xcc & (kXcds - 1));
}

// Next entry of the longest-first list for a workgroup on die my_xcd: the
// die's own share (entries my_xcd, my_xcd + 8, ...) through its cursor, then
// the other dies' remaining entries; total_work when none is left.  Entry
// f H + k is row block f of head (k - b) mod H (head_of): a die then runs the
// blocks of a few sequence-heads, whose K, V, Q and dO meet in its L2.
__device__ __forceinline__ int pull_entry(const int32_t* ctrl, int total_work, int my_xcd) {
    for (int k = 0; k < kXcds; ++k) {
        const int x = (my_xcd + k) & (kXcds - 1);
        int32_t* cur = const_cast<int32_t*>(ctrl) + kXcdCursor + kXcdStride * x;
        // a queue seen exhausted is skipped with a load, not an atomic
        if (k > 0 && __hip_atomic_load(cur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * kXcds + x >= total_work)
            continue;
        const int w = atomicAdd(cur, 1) * kXcds + x;
        if (w < total_work) return w;
    }
    return total_work;
}
__device__ __forceinline__ int head_of(int w, int b, int H) { return (w % H + H - b % H) % H; }

// Item fetch (thread 0), then shared.
__device__ __forceinline__ void fetch_item(const BwdParams& p, Small& s, int total_work, int tid, int my_xcd) {
    if (tid == 0) {
        const int w = pull_entry(p.ctrl, total_work, my_xcd);
        s.work = w;
        if (w < total_work) {
            const WorkItem it = p.items[w / p.H];
            s.item[0] = it.b; s.item[1] = it.qt; s.item[2] = it.a_end; s.item[3] = it.kb;
            s.item[4] = it.pr;
        }
    }
    lds_sync();
}

// ---------------------------------------------------------------------------
// dQ and the table gradients (query-major), from the G blocks and the K
// fragments the dK/dV kernel stored
// ---------------------------------------------------------------------------
// A block of G arrives as the dK/dV kernel held it: lane = key b (l % 32),
// the 16 values of queries a = 8 (r / 4) + 4 (l / 32) + r % 4.  The table
// gradients are summed in that order, from the exact fp32 values.  dQ
// contracts over keys, so for G K the block is turned over first, by two
// MFMAs against the identity: packed to bf16 it is an A operand with the keys
// as rows and the queries as the contraction, and its product with the
// identity on the queries is the block with the queries as columns (lane =
// query, the 16 values of keys 8 (r / 4) + 4 (l / 32) + r % 4), whose packed
// accumulator is the A operand of G K, exactly bf16(G) (transpose_identity).
__device__ __forceinline__ int64_t tri(int q) { return (int64_t)q * (q + 1) / 2; }

// A G block is stored when it holds a visible pair: k <= q, and history keys
// in the key tile or the diagonal tile (candidate keys are seen by their own
// row alone).
__device__ __forceinline__ bool g_block_live(int q, int k, int n) { return k <= q && (32 * k < n || k == q); }

// The K fragments of one 32-key tile and head as G K reads them (B operand
// of chunk c, column block nb, at fragment 4 c + nb): lane l holds column
// 32 nb + l % 32 at keys 16 c + 8 (e / 4) + 4 (l / 32) + e % 4.  8 KiB per
// tile, 1 KiB per fragment, lane-major.
constexpr int kKpBytes = 8 * 64 * 16;

__global__ void __launch_bounds__(kThreads, 2) attn_bwd_dq_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int32_t item[8];
    __shared__ __attribute__((aligned(16))) uint32_t qcodes[4][32];   // each wave's 32 query codes
    // one histogram per wave ([P] position, then [NT] time buckets), so that
    // the order of the additions into each does not depend on how the waves
    // interleave; added in wave order at the end of the item
    const int hw = (p.P + p.NT + 3) & ~3;
    float* hist_all = reinterpret_cast<float*>(smem);
    // per wave, a scratch in which a block's G is written skewed (column
    // a - b + 31, row a for query a and key b; kDiagPitch floats per
    // column), so that each column holds one diagonal and its 32 entries are
    // read with 8 16-byte loads.  Only the band a <= column <= a + 31 is ever
    // written; the rest stays zero from the start.
    float* scratch_all = hist_all + 4 * hw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int l32 = lane & 31;
    const int h2 = lane >> 5;
    const int total_work = p.ctrl[0] * p.H;
    const int P = p.P, NT = p.NT;
    bf16x8 idf[2];
    transpose_identity(lane, idf);

    float* hist = hist_all + wave * hw;
    float* scratch = scratch_all + wave * (64 * kDiagPitch);
    for (int e = tid; e < 4 * hw + 4 * 64 * kDiagPitch; e += kThreads) hist_all[e] = 0.0f;

    const int my_xcd = xcd_id();
    for (;;) {
        if (tid == 0) {
            const int w = pull_entry(p.ctrl, total_work, my_xcd);
            item[0] = w;
            if (w < total_work) {
                const WorkItem it = p.items[w / p.H];
                item[1] = it.b; item[2] = it.qt; item[3] = it.a_end; item[4] = it.kb; item[5] = it.pr;
            }
        }
        lds_sync();
        const int w = uni(item[0]);
        if (w >= total_work) break;
        const int b = uni(item[1]), qt = uni(item[2]), a_end = uni(item[3]);
        const int kb_begin = uni(item[4]) & 0xffff;
        const int ntiles = uni(item[5]) >> 16;
        const int h = head_of(w, b, p.H);
        const int64_t row0 = uni(p.offsets[b]);
        const int L = uni(p.lengths ? p.lengths[b] : p.offsets[b + 1] - (int)row0);
        const int n = uni(p.ncand ? L - p.ncand[b] : L);
        const int bbase = b * p.nblk;
        auto tile_of = [&](int pos) { return pos < a_end ? pos : kb_begin + (pos - a_end); };

        // ---- this wave's query tile q: G blocks of its row (one buffer
        //      range from block (q, 0) on), K fragments of the sequence and
        //      head, key codes of the sequence.  Blocks the wave does not read
        //      (past its diagonal, candidates of other rows, past the list's
        //      end) are loaded from out of range and arrive as zeros without a
        //      memory access, so that every step issues the same loads and the
        //      compiler's waits count exactly.
        const int q = qt * (kBlk / 32) + wave;
        const int wrow0 = q * 32;
        const bool wave_rows = wrow0 < L;
        __amdgpu_buffer_rsrc_t grs, krs, ers;
        {
            const int64_t blk0 = wave_rows ? p.gbase[b] + tri(q) : 0;
            const int64_t room = max((int64_t)0, min((int64_t)(q + 1), p.gcap - blk0));
            grs = __builtin_amdgcn_make_buffer_rsrc(p.gbuf + blk0 * p.H * 1024, (short)0,
                                                    wave_rows ? (int)(room * p.H * 4096) : 0, 0x00020000);
            krs = __builtin_amdgcn_make_buffer_rsrc(p.kp + ((int64_t)b * p.H + h) * p.nblk * (kKpBytes / 2),
                                                    (short)0, p.nblk * kKpBytes, 0x00020000);
            ers = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.enc) + row0, (short)0, L * 4,
                                                    0x00020000);
        }
        auto g_live = [&](int pos) { return pos < ntiles && wave_rows && g_block_live(q, tile_of(pos), n); };
        auto load_g = [&](int pos, f32x16& g, uint32_t& kcode) {
            const bool live = g_live(pos);
            const uint32_t off = live ? (uint32_t)((tile_of(pos) * p.H + h) * 4096 + lane * 64) : 0x80000000u;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(grs, off + 16 * m, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) g[4 * m + e] = x[e];
            }
            kcode = __builtin_amdgcn_raw_buffer_load_b32(ers, live ? (uint32_t)((tile_of(pos) * 32 + l32) * 4) : 0x80000000u, 0, 0);
        };
        auto load_k = [&](int pos, u32x4 (&kf)[2][4]) {
            const uint32_t off = g_live(pos) ? (uint32_t)(tile_of(pos) * kKpBytes + lane * 16) : 0x80000000u;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    kf[c][nb] = __builtin_amdgcn_raw_buffer_load_b128(krs, off + (4 * c + nb) * 1024, 0, 0);
        };

        // the codes of this wave's 32 queries, read back by groups of four
        if (lane < 32) qcodes[wave][lane] = __builtin_amdgcn_raw_buffer_load_b32(ers, (uint32_t)((wrow0 + lane) * 4), 0, 0);
        const int64_t t_first = p.ts[row0];
        const int qblk = bbase + q;
        uint32_t rmin = wave_rows ? p.stats[2 * qblk] : 0x80000000u;
        uint32_t rmax = wave_rows ? p.stats[2 * qblk + 1] : 0x80000000u;
        rmin = uniu(rmin);
        rmax = uniu(rmax);
        const int prow_min = uni(min(wrow0, n));

        f32x16 dqa[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqa[nb][r] = 0.0f;

        const StatsPtr kstats = stats_ptr(p.stats);

        // table-gradient histogram updates of one block, G as stored (lane =
        // key j0 + l32, element r = query wrow0 + 8 (r / 4) + 4 h2 + r % 4,
        // invisible pairs already zero)
        auto hist_block = [&](int kt, const f32x16& gv, uint32_t kcode) {
            const int j0 = kt * 32;
            const int j = j0 + l32;
            const u32x2 kr = kstats[bbase + kt];
            const TimeBlock tb = time_block(rmin, rmax, kr[0], kr[1]);
            const bool pos_clamped = prow_min - min(j0 + 31, n) >= P - 1;
            const bool tconst = tb.constant;
            const int tlo = min(NT - 1, 31 - tb.cz);
            const int thi = min(NT - 1, 31 - tb.czhi);
            const bool few = !tb.constant && !tb.wide && thi - tlo < 4;
            // time bucket of element r (keys and queries in time order: along
            // r the buckets do not decrease)
            uint32_t tb4[4] = {0u, 0u, 0u, 0u};
            if (!tconst) {
                int64_t tj64 = 0;
                if (tb.wide) tj64 = j < L ? p.ts[row0 + j] : t_first;
                u32x4 qc[4];   // queries 8 q + 4 h2 + 0..3
                if (!tb.wide) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) qc[g4] = *reinterpret_cast<const u32x4*>(&qcodes[wave][8 * g4 + 4 * h2]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int tbr;
                    if (!tb.wide) {
                        tbr = min(NT - 1, 31 - (int)__builtin_clz(sad_u32(qc[r >> 2][r & 3], kcode, 1u)));
                    } else {
                        const int i = wrow0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                        const int64_t ti = i < L ? p.ts[row0 + i] : t_first;
                        const int64_t dt = ti - tj64;
                        const uint64_t ad = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
                        tbr = min(NT - 1, bit_length_u64(ad));
                    }
                    tb4[r >> 2] |= (uint32_t)tbr << (8 * (r & 3));
                }
            }
            auto tbv = [&](int r) { return (int)((tb4[r >> 2] >> (8 * (r & 3))) & 0xffu); };
            // block sums (cross-lane, no LDS)
            // (a block spanning few time buckets sums buckets tlo+1 .. thi
            // per element and takes bucket tlo as the rest of the total)
            float gsum = 0.0f;
            float tsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < 16; ++r) gsum += gv[r];
            if (few) {
                const int nk = thi - tlo;   // 1 .. 3
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int k = tbv(r) - tlo;
                    tsum[1] += (k == 1) ? gv[r] : 0.0f;
                    if (nk >= 2) {
                        tsum[2] += (k == 2) ? gv[r] : 0.0f;
                        tsum[3] += (k == 3) ? gv[r] : 0.0f;
                    }
                }
            }
            const bool colwise = !pos_clamped && wrow0 >= n;
            float csum = 0.0f;
            if (colwise) csum = gsum;   // (before the wave reduction below)
            if (pos_clamped || tconst || few) gsum = wave_total(gsum);
            if (few) {
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    if (tlo + k <= thi) tsum[k] = wave_total(tsum[k]);
                tsum[0] = ((gsum - tsum[1]) - tsum[2]) - tsum[3];
            }
            // Position buckets.  When the wave's rows are all history rows,
            // the bucket of a visible pair is min(i - j, P - 1): the block's 63
            // diagonals, summed through the skewed scratch with plain LDS
            // writes and reads, take one atomic each (LDS float atomics are
            // slow).  When they are all candidate rows (all at position n),
            // the bucket min(n - min(j, n), P - 1) depends on the key alone,
            // which is this lane's: its 16 values, and the other half-wave's
            // 16 of the same key, make one sum.  Otherwise per element.
            const bool diag = !pos_clamped && wrow0 + 31 < n;
            if (diag) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int a = 8 * (r >> 2) + 4 * h2 + (r & 3);
                    scratch[(a + 31 - l32) * kDiagPitch + a] = gv[r];
                }
                // lane u sums column u: diagonal a - b = u - 31
                float dsum = 0.0f;
                const f32x4* col = reinterpret_cast<const f32x4*>(scratch + lane * kDiagPitch);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const f32x4 x = col[k];
                    dsum += x[0];
                    dsum += x[1];
                    dsum += x[2];
                    dsum += x[3];
                }
                const int pb = wrow0 - j0 + lane - 31;
                if (lane < 63 && pb >= 0 && dsum != 0.0f) atomicAdd(&hist[min(pb, P - 1)], dsum);
            } else if (colwise) {
                csum += __shfl_xor(csum, 32, 64);
                const int pb = n - min(j, n);
                if (lane < 32 && csum != 0.0f) atomicAdd(&hist[min(pb, P - 1)], csum);
            } else if (!pos_clamped) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (gv[r] != 0.0f) {
                        const int i = wrow0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                        atomicAdd(&hist[min(max(min(i, n) - min(j, n), 0), P - 1)], gv[r]);
                    }
                }
            }
            if (!tconst && !few) {
                // buckets come in runs along r: one atomic per run
                float run = 0.0f;
                int rb = tbv(0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int bk = tbv(r);
                    if (bk != rb) {
                        if (run != 0.0f) atomicAdd(&hist[P + rb], run);
                        run = 0.0f;
                        rb = bk;
                    }
                    run += gv[r];
                }
                if (run != 0.0f) atomicAdd(&hist[P + rb], run);
            }
            // one lane adds the block sums to this wave's own histogram:
            // plain read-add-writes (an atomic at a uniform address becomes a
            // scan over the active lanes)
            if (lane == 63) {
                if (pos_clamped) hist[P - 1] += gsum;
                if (tconst) hist[P + tlo] += gsum;
                if (few) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (tlo + k <= thi) hist[P + tlo + k] += tsum[k];
                }
            }
        };

        // ---- the tiles: G and the key codes two tiles ahead (two register
        //      sets), the K fragments one tile ahead, loaded after this
        //      tile's G K (the loads are issued in the order they are needed)
        f32x16 gA, gB;
        uint32_t kcA, kcB;
        u32x4 kf[2][4];
        load_g(0, gA, kcA);
        load_k(0, kf);
        load_g(1, gB, kcB);

        auto step = [&](int t, f32x16& g, uint32_t& kcode) {
            const int kt = tile_of(t);
            const bool live = g_live(t);
            if (live) {
                hist_block(kt, g, kcode);
                float gl[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) gl[r] = g[r];
                bf16x8 hi[2];
                pack_a(gl, hi);
                f32x16 gt;
#pragma unroll
                for (int r = 0; r < 16; ++r) gt[r] = 0.0f;
                gt = mfma32(hi[0], idf[0], gt);
                gt = mfma32(hi[1], idf[1], gt);
                float gq[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) gq[r] = gt[r];
                bf16x8 pg[2];
                pack_a(gq, pg);
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        dqa[nb] = mfma32(pg[c], __builtin_bit_cast(bf16x8, kf[c][nb]), dqa[nb]);
            }
            load_k(t + 1, kf);
            load_g(t + 2, g, kcode);
        };

        int t = 0;
        for (; t + 1 < ntiles; t += 2) {
            step(t, gA, kcA);
            step(t + 1, gB, kcB);
        }
        if (t < ntiles) step(t, gA, kcA);

        // ---- (gradient rows are written once: non-temporal stores)
        // ---- dQ = alpha * acc for rows < L; lane holds column nb*32 + l32 at
        //      rows wrow0 + 8 (r / 4) + 4 h2 + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ro = wrow0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (ro < L) {
                uint16_t* op = p.dq + (row0 + ro) * p.dqs + h * HD + l32;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) __builtin_nontemporal_store(f32_to_bf16_bits(p.alpha * dqa[nb][r]), op + nb * 32);
            }
        }
        // ---- this item's table-gradient histogram -> its partial row
        lds_sync();
        // (row (w / H) H + h: the reduction takes a head's rows in list order)
        float* part = p.rab_part + ((int64_t)(w / p.H) * p.H + h) * (P + NT);
        for (int e = tid; e < P + NT; e += kThreads) {
            part[e] = ((hist_all[e] + hist_all[hw + e]) + hist_all[2 * hw + e]) + hist_all[3 * hw + e];
            hist_all[e] = hist_all[hw + e] = hist_all[2 * hw + e] = hist_all[3 * hw + e] = 0.0f;
        }
        lds_sync();   // histogram cleared before the next item
    }
}

// ---------------------------------------------------------------------------
// dK and dV (key-major)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads, 1) attn_bwd_dkv_kernel(BwdParams p, const void* ws_base, uint32_t ws_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* ring_q = smem;                               // Q, kswz: A operand of S = Q K^T
    uint8_t* ring_qt = smem + kStages * kTileBytes;       // Q, vswz: B operand of dK += G^T Q
    uint8_t* ring_g = smem + 2 * kStages * kTileBytes;    // dO, kswz: A operand of dO V^T
    uint8_t* ring_gt = smem + 3 * kStages * kTileBytes;   // dO, vswz: B operand of dV += A^T dO
    Small& s = small_of<4>(smem);
    float* ptab = ptab_of<4>(smem);
    // the position table padded for blocks of history rows: copy c holds
    // T[x - c] at x, T[u] = rab_pos[clamp(u - 32, 0, P - 1)]
    const int pw = ptab2_width(p.P);
    float* ptab2 = ptab + ((p.P + 3) & ~3);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int l32 = lane & 31;
    const int h2 = lane >> 5;
    const int total_work = p.ctrl[0] * p.H;
    const bool shared_tables = (p.rp_hs == 0) && (p.rt_hs == 0);
    const bool silu = p.act == 0;
    const int P = p.P;
    const int per_tile = uni(wave == 0 ? 9 : 8);
    const u32x4 wrs = make_rsrc(ws_base, ws_bytes);
    const int64_t enc_base = (const uint8_t*)p.enc - (const uint8_t*)ws_base;
    int loaded_head = -1;

    const int my_xcd = xcd_id();
    for (;;) {
        fetch_item(p, s, total_work, tid, my_xcd);
        const int w = uni(s.work);
        if (w >= total_work) break;
        const int b = uni(s.item[0]), kblock = uni(s.item[1]);
        const int kbw = uni(s.item[3]);
        const int rt_begin = kbw & 0xffff;
        const int ntiles = uni(s.item[4]) >> 16;
        const int h = head_of(w, b, p.H);
        const int64_t row0 = uni(p.offsets[b]);
        const int L = uni(p.lengths ? p.lengths[b] : p.offsets[b + 1] - (int)row0);
        const int n = uni(p.ncand ? L - p.ncand[b] : L);
        const int bbase = b * p.nblk;

        if (loaded_head < 0 || (!shared_tables && loaded_head != h)) {
            load_tables(p, h, ptab, s, tid);
            const float* rp = p.rab_pos + (int64_t)h * p.rp_hs;
            for (int e = tid; e < 2 * pw; e += kThreads) {
                const int c = e >= pw ? 1 : 0;
                const int u = e - c * pw - c;
                ptab2[e] = rp[min(max(u - 32, 0), P - 1)];
            }
            loaded_head = h;
            lds_wait();
        }
        const float pos_far = p.rab_pos[(int64_t)h * p.rp_hs + P - 1];

        const TileSrc sq = tile_src(p.q + row0 * p.qs + h * HD, p.qs, L, lane, wave, false);
        const TileSrc sqt = tile_src(p.q + row0 * p.qs + h * HD, p.qs, L, lane, wave, true);
        const TileSrc sg = tile_src(p.g + row0 * p.gs + h * HD, p.gs, L, lane, wave, false);
        const TileSrc sgt = tile_src(p.g + row0 * p.gs + h * HD, p.gs, L, lane, wave, true);
        const int64_t enc_row0 = enc_base + 4 * row0;
        auto issue = [&](int stage, int tile) {
            issue_part(sq, ring_q, stage, tile, wave);
            issue_part(sqt, ring_qt, stage, tile, wave);
            issue_part(sg, ring_g, stage, tile, wave);
            issue_part(sgt, ring_gt, stage, tile, wave);
            if (wave == 0) issue_codes(wrs, enc_row0, s, stage, tile, L, lane);
        };
#pragma unroll
        for (int pre = 0; pre < kStages - 1; ++pre)
            if (pre < ntiles) issue(pre, rt_begin + pre);

        // ---- this wave's 32 keys: K and V as B operands (lane = key)
        const int k0w = kblock * kBlk + wave * 32;
        const int j = k0w + l32;
        const bool key_valid = j < L;
        bf16x8 kf[8], vf[8];
        {
            const uint16_t* kp = p.k + (row0 + j) * p.ks + h * HD + h2 * 8;
            const uint16_t* vp = p.v + (row0 + j) * p.vs + h * HD + h2 * 8;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                kf[kc] = load_frag(kp + kc * 16, key_valid);
                vf[kc] = load_frag(vp + kc * 16, key_valid);
            }
        }
        const int64_t t_first = p.ts[row0];
        int64_t tj64 = key_valid ? p.ts[row0 + j] : t_first;
        uint32_t ej = key_valid ? p.enc[row0 + j] : 0x80000000u;
        const bool wave_keys = k0w < L;
        const int kblk = bbase + kblock * (kBlk / 32) + wave;
        uint32_t kmn = wave_keys ? p.stats[2 * kblk] : 0x80000000u;
        uint32_t kmx = wave_keys ? p.stats[2 * kblk + 1] : 0x80000000u;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) {
            settle(kf[kc]);
            settle(vf[kc]);
        }
        settle(tj64);
        settle(ej);
        settle(kmn);
        settle(kmx);
        kmn = uniu(kmn);
        kmx = uniu(kmx);
        const int pkey = min(j, n);
        const int pkey_max = uni(min(k0w + 31, n));
        // G blocks of this wave's key tile kw: block (q, kw) of the sequence
        // at gblk0 + q (q + 1) / 2
        const int kw = kblock * (kBlk / 32) + wave;
        const int64_t gblk0 = uni(p.gbase[b]) + kw;
        // this key tile's K as the dQ kernel's G K reads it: the B operand
        // with the features as columns and the keys as the contraction,
        // turned over from kf (keys as rows) by two MFMAs per 32-feature
        // block against the identity on the features (exact), then packed
        if (wave_keys) {
            bf16x8 ik[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 z = {0u, 0u, 0u, 0u};
                if ((l32 >> 4) == c && ((l32 >> 3) & 1) == h2) {
                    const int e = l32 & 7;
                    z[e >> 1] = 0x3F80u << (16 * (e & 1));
                }
                ik[c] = __builtin_bit_cast(bf16x8, z);
            }
            uint8_t* kpd = reinterpret_cast<uint8_t*>(p.kp) + (((int64_t)b * p.H + h) * p.nblk + kw) * kKpBytes +
                           lane * 16;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                f32x16 c32;
#pragma unroll
                for (int r = 0; r < 16; ++r) c32[r] = 0.0f;
                c32 = mfma32(kf[2 * nb], ik[0], c32);
                c32 = mfma32(kf[2 * nb + 1], ik[1], c32);
                float cf[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) cf[r] = c32[r];
                bf16x8 pk[2];
                pack_a(cf, pk);
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pk[c]),
                                                reinterpret_cast<u32x4*>(kpd + (4 * c + nb) * 1024));
            }
        }

        f32x16 dka[4], dva[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dka[nb][r] = 0.0f;
                dva[nb][r] = 0.0f;
            }

        const StatsPtr rstats = stats_ptr(p.stats);
        // ---- software pipeline over the query tiles: step t builds S(t)
        //      (bias as the initial accumulator) and dP(t) = dO V^T while the
        //      activation, slope and G of tile t-1 run on the VALU between
        //      those MFMAs; then dV += A^T dO and dK += G^T Q for tile t-1.
        //      The transposed fragments of tile t are read into registers at
        //      the end of step t, so its stage may be refilled after the next
        //      barrier.
        const uint32_t a_off = k_lane_offset(lane), t_off = v_lane_offset(lane);
        u32x4 trq[2][4], trg[2][4];   // Q^T and dO^T fragments of the tile being finished
        struct Tile {
            float cadd;
            int r0;
            bool full;
        };

        auto sync = [&](int t) {
            wait_tile(t + 1 < ntiles ? per_tile : 0);   // tile t has landed (t+1 may be in flight)
            lds_sync();                                   // and every wave is done with tile t-1's stage
            if (t + kStages - 1 < ntiles) issue((t + kStages - 1) % kStages, rt_begin + t + kStages - 1);
        };

        // bias of tile t into sacc (position, then time per element when the
        // block needs it); the block-uniform rest goes into the returned cadd
        auto prep = [&](int t, f32x16& sacc, bf16x8 (&qa)[8], bf16x8 (&ga)[8]) -> Tile {
            const int rt = rt_begin + t;
            const int r0 = rt * 32;
            const int stage = t % kStages;
            const u32x2 rr = rstats[bbase + rt];
            const TimeBlock tb = time_block(rr[0], rr[1], kmn, kmx);
            const bool pos_clamped = min(r0, n) - pkey_max >= P - 1;
            const bool hist_rows = r0 + 31 < n;
            Tile st;
            st.r0 = r0;
            st.full = (r0 + 31 < L) && (k0w + 31 < n) && (k0w + 31 <= r0);
            st.cadd = 0.0f;
            if (pos_clamped) st.cadd += pos_far;
            if (tb.constant) st.cadd += s.tt_fast[tb.cz];
            if (pos_clamped) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
            } else if (hist_rows) {
                // rows i = r0 + c (c = 8q + 4h2 + t): entries x0 + 8q + t of
                // the padded table, two per 8-byte read
                const int x0 = min(max(r0 - pkey + 32 + 4 * h2, 0), pw - 32);
                const int c = x0 & 1;
                const float* pp = ptab2 + c * pw + (x0 + c);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const float2 pv = *reinterpret_cast<const float2*>(pp + 8 * q + 2 * t2);
                        sacc[4 * q + 2 * t2] = pv.x;
                        sacc[4 * q + 2 * t2 + 1] = pv.y;
                    }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = r0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    sacc[r] = ptab[min(max(min(i, n) - pkey, 0), P - 1)];
                }
            }
            const uint8_t* q_lds = ring_q + stage * kTileBytes;
            const uint8_t* g_lds = ring_g + stage * kTileBytes;
            uint32_t ao = a_off;
            asm volatile("" : "+v"(ao));
            const uint32_t qb = lds_addr(q_lds) + ao, gb = lds_addr(g_lds) + ao;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                qa[kc] = lds_read_b128(qb ^ (uint32_t)(kc << 5));
                ga[kc] = lds_read_b128(gb ^ (uint32_t)(kc << 5));
            }
            if (!tb.constant) {
                const uint32_t* codes = s.codes[stage];
                if (!tb.wide) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int c = 8 * (r >> 2) + 4 * h2 + (r & 3);
                        sacc[r] += s.tt_fast[__builtin_clz(sad_u32(codes[c], ej, 1u))];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = r0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                        const int64_t ti = i < L ? p.ts[row0 + i] : t_first;
                        const int64_t dt = ti - tj64;
                        const uint64_t ad = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
                        sacc[r] += s.tt_wide[bit_length_u64(ad)];
                    }
                }
            }
            return st;
        };

        // activation, slope and G of element r of a finished S / dP
        auto act_elem = [&](const f32x16& sacc, const f32x16& gacc, float cadd, int r, float (&av)[16],
                            float (&gv)[16]) {
            float a, slope;
            act_and_slope(sacc[r] + cadd, silu, a, slope);
            av[r] = a;
            gv[r] = gacc[r] * slope;
        };

        // mask (blocks with invisible pairs), pack, dV += A^T dO, dK += G^T Q
        auto finish = [&](const Tile& st, float (&av)[16], float (&gv)[16]) {
            if (!st.full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = st.r0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    const bool vis = (i < L) & (j < L) & ((i < n) ? (j <= i) : ((j < n) | (j == i)));
                    av[r] = vis ? av[r] : 0.0f;
                    gv[r] = vis ? gv[r] : 0.0f;
                }
            }
            // G of a block the dQ kernel reads, as this lane holds it
            const int qt32 = st.r0 >> 5;
            const int64_t gblk = gblk0 + tri(qt32);
            if (wave_keys && g_block_live(qt32, kw, n) && gblk < p.gcap) {
                f32x4* dst = reinterpret_cast<f32x4*>(p.gbuf + (gblk * p.H + h) * 1024 + lane * 16);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    __builtin_nontemporal_store(f32x4{gv[4 * m], gv[4 * m + 1], gv[4 * m + 2], gv[4 * m + 3]}, dst + m);
            }
            bf16x8 pa[2], pg[2];
            pack_a(av, pa);
            pack_a(gv, pg);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    dva[nb] = mfma32(pa[c], __builtin_bit_cast(bf16x8, trg[c][nb]), dva[nb]);
                    dka[nb] = mfma32(pg[c], __builtin_bit_cast(bf16x8, trq[c][nb]), dka[nb]);
                }
        };

        auto read_tr = [&](int t) {
            const int stage = t % kStages;
            uint32_t to = t_off;
            asm volatile("" : "+v"(to));
            read_v_tile(lds_addr(ring_gt + stage * kTileBytes), to, trg);
            read_v_tile(lds_addr(ring_qt + stage * kTileBytes), to, trq);
        };

        auto step = [&](int t, f32x16& sC, f32x16& gC, const Tile& stC, f32x16& sN, f32x16& gN) -> Tile {
            sync(t);
            bf16x8 qa[8], ga[8];
            const Tile stN = prep(t, sN, qa, ga);
#pragma unroll
            for (int r = 0; r < 16; ++r) gN[r] = 0.0f;
            float av[16], gv[16];
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                gN = mfma32(ga[kc], vf[kc], gN);
                act_elem(sC, gC, stC.cadd, 2 * kc, av, gv);
                sN = mfma32(qa[kc], kf[kc], sN);
                act_elem(sC, gC, stC.cadd, 2 * kc + 1, av, gv);
            }
#pragma unroll
            for (int kc = 0; kc < 16; ++kc) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // then VALU
            }
            finish(stC, av, gv);
            read_tr(t);
            return stN;
        };

        if (ntiles > 0) {
            f32x16 sA, gA, sB, gB;
            Tile stA, stB;
            {
                sync(0);
                bf16x8 qa[8], ga[8];
                stA = prep(0, sA, qa, ga);
#pragma unroll
                for (int r = 0; r < 16; ++r) gA[r] = 0.0f;
#pragma unroll
                for (int kc = 0; kc < 8; ++kc) {
                    gA = mfma32(ga[kc], vf[kc], gA);
                    sA = mfma32(qa[kc], kf[kc], sA);
                }
                read_tr(0);
            }
            int t = 1;
            for (; t + 1 < ntiles; t += 2) {
                stB = step(t, sA, gA, stA, sB, gB);
                stA = step(t + 1, sB, gB, stB, sA, gA);
            }
            if (t < ntiles) {
                stB = step(t, sA, gA, stA, sB, gB);
                sA = sB;
                gA = gB;
                stA = stB;
            }
            float av[16], gv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) act_elem(sA, gA, stA.cadd, r, av, gv);
            finish(stA, av, gv);
        }

        // ---- dK, dV = alpha * acc for keys < L; lane holds column nb*32 +
        //      l32 at keys k0w + 8 (r / 4) + 4 h2 + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ko = k0w + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (ko < L) {
                uint16_t* kp = p.dk + (row0 + ko) * p.dks + h * HD + l32;
                uint16_t* vp = p.dv + (row0 + ko) * p.dvs + h * HD + l32;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    __builtin_nontemporal_store(f32_to_bf16_bits(p.alpha * dka[nb][r]), kp + nb * 32);
                    __builtin_nontemporal_store(f32_to_bf16_bits(p.alpha * dva[nb][r]), vp + nb * 32);
                }
            }
        }
        lds_barrier();   // this item's LDS use is over before the next item starts
    }
}

// Table gradients, in two fixed-order passes over the partial rows (one per
// work item w, head w % H).  Pass 1: chunk c of kChunks sums its rows (of
// head h, or all heads for a shared table) for one column e, in row order
// with four interleaved accumulators added in a fixed order at the end.
// Pass 2: the chunks in order, times alpha.
constexpr int kChunks = 64;

__global__ void __launch_bounds__(256) rab_grad_partial_kernel(const float* part, const int32_t* ctrl, int H,
                                                               int width, int P, int per_head_pos,
                                                               int per_head_time, float* part2) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y;
    const int h = blockIdx.z;
    if (e >= width) return;
    const bool per_head = e < P ? per_head_pos != 0 : per_head_time != 0;
    const int step = per_head ? H : 1;
    const int nrows = per_head ? (ctrl[0] * H - h + H - 1) / H : ctrl[0] * H;   // rows of this head
    const int per_chunk = (nrows + kChunks - 1) / kChunks;
    const int r0 = c * per_chunk, r1 = min(nrows, r0 + per_chunk);
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    int r = r0;
    const int64_t base = per_head ? h : 0;
    for (; r + 4 <= r1; r += 4) {
        a0 += part[(base + (int64_t)(r + 0) * step) * width + e];
        a1 += part[(base + (int64_t)(r + 1) * step) * width + e];
        a2 += part[(base + (int64_t)(r + 2) * step) * width + e];
        a3 += part[(base + (int64_t)(r + 3) * step) * width + e];
    }
    for (; r < r1; ++r) a0 += part[(base + (int64_t)r * step) * width + e];
    part2[((int64_t)h * kChunks + c) * width + e] = (a0 + a1) + (a2 + a3);
}

__global__ void __launch_bounds__(256) rab_grad_final_kernel(const float* part2, int width, int P, int NT,
                                                             int per_head_pos, int per_head_time, float alpha,
                                                             float* drab_pos, float* drab_time) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int h = blockIdx.y;
    if (e >= width) return;
    const bool is_pos = e < P;
    const bool per_head = is_pos ? per_head_pos != 0 : per_head_time != 0;
    if (!per_head && h > 0) return;
    float* dst = is_pos ? drab_pos : drab_time;
    if (!dst) return;
    float acc = 0.0f;
    for (int c = 0; c < kChunks; ++c) acc += part2[((int64_t)h * kChunks + c) * width + e];
    const int idx = is_pos ? e : e - P;
    dst[(per_head ? h * (is_pos ? P : NT) : 0) + idx] = alpha * acc;
}

size_t smem_bytes(int tiles, int P, int NT, bool hist) {
    size_t b = (size_t)tiles * kStages * kTileBytes + ((sizeof(Small) + 15) & ~size_t(15));
    if (hist)   // the dQ kernel: histograms and diagonal scratch only
        return sizeof(float) * 4 * ((size_t)((P + NT + 3) & ~3) + 64 * kDiagPitch);
    else        // the dK/dV kernel: the table and its padded copies
        b += sizeof(float) * ((size_t)((P + 3) & ~3) + 2 * (size_t)ptab2_width(P));
    return b;
}

BwdParams make_params(const AttnBwdArgs& a) {
    BwdParams p;
    p.H = a.H;
    p.offsets = a.offsets; p.lengths = a.lengths; p.ncand = a.ncand;
    p.q = static_cast<const uint16_t*>(a.q); p.qs = a.q_stride;
    p.k = static_cast<const uint16_t*>(a.k); p.ks = a.k_stride;
    p.v = static_cast<const uint16_t*>(a.v); p.vs = a.v_stride;
    p.g = static_cast<const uint16_t*>(a.dout); p.gs = a.dout_stride;
    p.ts = a.ts;
    p.rab_pos = a.rab_pos; p.P = a.P; p.rp_hs = a.rp_head_stride;
    p.rab_time = a.rab_time; p.NT = a.NT; p.rt_hs = a.rt_head_stride;
    p.alpha = a.alpha;
    p.act = a.act;
    p.dq = static_cast<uint16_t*>(a.dq); p.dqs = a.dq_stride;
    p.dk = static_cast<uint16_t*>(a.dk); p.dks = a.dk_stride;
    p.dv = static_cast<uint16_t*>(a.dv); p.dvs = a.dv_stride;
    p.nblk = a.nblk;
    p.stats = a.stats;
    p.enc = a.enc;
    p.rab_part = a.rab_part;
    p.gbuf = a.gbuf;
    p.gbase = a.gbase;
    p.gcap = a.gcap;
    p.kp = static_cast<uint16_t*>(a.kp);
    return p;
}

}  // namespace

bool attn_bwd_tables_fit(int P, int NT) {
    return smem_bytes(1, P, NT, true) <= 160 * 1024 && smem_bytes(4, P, NT, false) <= 160 * 1024;
}

int64_t attn_bwd_g_blocks(int B, int max_seq_len, int64_t num_rows) {
    // sum over sequences of m (m + 1) / 2, m = ceil(L / 32) <= M: at most
    // (M + 1) / 2 per 32-row tile, and at most num_rows / 32 + B tiles
    const int64_t M = (max(max_seq_len, 0) + 31) / 32;
    const int64_t by_tiles = ((M + 1) * (num_rows / 32 + 1 + B) + 1) / 2;
    const int64_t by_seqs = (int64_t)B * (M * (M + 1) / 2);
    return min(by_tiles, by_seqs);
}

size_t attn_bwd_rab_part_floats(int64_t cap, int H, int P, int NT) {
    return (size_t)cap * (size_t)H * (size_t)(P + NT);
}

size_t attn_bwd_rab_part2_floats(int H, int P, int NT) { return (size_t)H * kChunks * (size_t)(P + NT); }

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t stream) {
    const int grid = device_cu_count();
    const void* ws_base = a.stats;
    const size_t span = (size_t)((const uint8_t*)(a.enc + a.num_rows) - (const uint8_t*)a.stats);
    const uint32_t wsb = (uint32_t)(span > 0x7fffffffu ? 0x7fffffffu : span);

    hipError_t e;

    // dK, dV and the G blocks, then dQ and the table gradients from G
    BwdParams pk = make_params(a);
    pk.items = a.kv_items; pk.ctrl = a.kv_ctrl;
    const size_t smk = smem_bytes(4, a.P, a.NT, false);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_bwd_dkv_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smk);
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL(attn_bwd_dkv_kernel, dim3(grid), dim3(kThreads), smk, stream, a.ev_dkv_begin,
                          a.ev_dkv_end, 0, pk, ws_base, wsb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    BwdParams pq = make_params(a);
    pq.items = a.q_items; pq.ctrl = a.q_ctrl;
    const size_t smq = smem_bytes(1, a.P, a.NT, true);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_bwd_dq_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smq);
    if (e != hipSuccess) return e;
    // two workgroups per CU when their LDS allows it
    const int qgrid = smq <= 80 * 1024 ? 2 * grid : grid;
    hipExtLaunchKernelGGL(attn_bwd_dq_kernel, dim3(qgrid), dim3(kThreads), smq, stream, a.ev_dq_begin,
                          a.ev_dq_end, 0, pq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (a.drab_pos || a.drab_time) {
        const int width = a.P + a.NT;
        const int hy = (a.rp_head_stride > 0 || a.rt_head_stride > 0) ? a.H : 1;
        const unsigned gx = (unsigned)((width + 255) / 256);
        hipLaunchKernelGGL(rab_grad_partial_kernel, dim3(gx, kChunks, (unsigned)hy), dim3(256), 0, stream,
                           a.rab_part, a.q_ctrl, a.H, width, a.P, a.rp_head_stride > 0 ? 1 : 0,
                           a.rt_head_stride > 0 ? 1 : 0, a.rab_part2);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(rab_grad_final_kernel, dim3(gx, (unsigned)hy), dim3(256), 0, stream, a.rab_part2,
                           width, a.P, a.NT, a.rp_head_stride > 0 ? 1 : 0, a.rt_head_stride > 0 ? 1 : 0,
                           a.alpha, a.drab_pos, a.drab_time);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace hstu
