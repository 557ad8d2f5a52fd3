// attn_bf16.hip -- attention core of the HSTU layer for gfx950, bf16 inputs,
// fp32 accumulation, d_qk = d_v = 128.
//
// Per head h and visible pair (i, j) of a jagged sequence:
//   S_ij = <Q_i, K_j> + rab_pos[pb(i, j)] + rab_time[tb(i, j)]
//   O_i  = alpha * sum_j SiLU(S_ij) V_j
// ("生成式推荐（一）：HSTU", sections "高性能自注意力Encoder：HSTU" and
// "Pointwise aggregated attention": SiLU in place of softmax, no
// normalisation over the sequence, a relative bias from position and time.)
//
// Design: one workgroup = 4 waves = one work item of 128 query rows x 1 head;
// each wave owns 32 query rows; key tiles of 32 keys; v_mfma_f32_32x32x16_bf16.
//
//   * S^T = K Q^T per 32-key tile: in the accumulator lane l holds query row
//     (l % 32) against 16 keys, which after bias + SiLU + bf16 packing are
//     directly the A operand of O += A V.  Q stays in registers.
//   * K and V tiles are staged row-major into a 4-stage LDS ring by buffer
//     loads that write LDS directly (no registers, no VALU; rows past the
//     sequence end fall outside the buffer's range and arrive as zeros), three
//     tiles ahead of their use.  V is read transposed by ds_read_b64_tr_b16,
//     so the B operand of A V needs no shuffle.
//   * Timestamps arrive pre-encoded (a small preparation kernel): per row
//     e = 2 (t - t_first) + 2^31, exact when |t - t_first| < 2^30, and per
//     32-row block the range [min e, max e] (or a "wide" mark).
//   * The relative bias is the MFMA's initial accumulator, chosen per 32 x 32
//     block with wave-uniform (scalar) tests:
//       - time bucket constant over the block (from the row and key blocks'
//         ranges): no per-element time work; the constant folds into the first
//         FMA of the activation;
//       - position bucket clamped over the whole block: no position reads;
//       - otherwise position entries come from a reversed LDS table (2 shifted
//         copies, so a lane reads 2 entries with one 8-byte load) and the time
//         bucket per element: |e_i - e_j| + 1 = 2|dt| + 1 is one v_sad_u32 and
//         its leading-zero count c = 31 - bit_length(|dt|) indexes a 32-entry
//         LDS table;
//       - blocks outside the 2^30 range use 64-bit arithmetic.
//   * SiLU in exp2 form: t = -log2(e) (S + c), A' = t / (1 + 2^t); the factor
//     -ln 2 that turns A' into SiLU(S) is folded into alpha.
//   * Blocks whose pairs are all visible skip the mask; the others select
//     (never multiply) so that padding and masked garbage cannot leak.
//   * Software pipeline over the key tiles: while S(t) is being built (its
//     LDS reads, bias, and the dependent chain of 8 QK^T MFMAs), the
//     activation of S(t-1) runs on the VALU between those MFMAs, and then
//     O += A(t-1) V(t-1) is issued; V(t) is read into registers at the end of
//     the step.  Fragment addresses are one per-lane base XOR constants, so
//     the loop keeps two address registers and never touches scratch (a
//     scratch reload would wait for every tile load in flight).
//   * Persistent grid: workgroups pull items (longest first) from the
//     scheduler's list through atomic cursors until it is exhausted, one
//     cursor per accelerator die (XCD, each with its own L2): die x takes
//     every 8th entry, and an entry's head is rotated by its sequence, so the
//     row blocks of a sequence-head meet in one L2 (HBM reads of the K/V
//     re-reads fall by 43 %) while the dies get equal shares of the
//     cost-sorted list; a die out of work helps the others.
#include <hip/hip_ext.h>

#include "internal.h"
#include "hstu_device.h"
#include "tile_ops.h"

namespace hstu {

namespace {

constexpr int BM = kBf16TileM;   // 128 query rows per item
constexpr int BN = kBf16TileN;   // 32 keys per tile
constexpr int HD = 128;          // head dim
constexpr int kThreads = 256;
constexpr int kStages = 4;       // LDS ring depth: tiles t .. t+3 in flight


struct Params {
    int H;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    const uint16_t* q; int64_t qs;
    const uint16_t* k; int64_t ks;
    const uint16_t* v; int64_t vs;
    const int64_t* ts;
    const float* rab_pos; int P; int rp_hs;
    const float* rab_time; int NT; int rt_hs;
    float alpha;
    uint16_t* o; int64_t os;
    const WorkItem* items;
    const int32_t* ctrl;
    int32_t* cursor;
    float* partial;
    int32_t* rowmap;
    int nblk;
    const uint32_t* stats;
    const uint32_t* enc;
    int pos_copy;   // floats per shifted copy of the reversed position table
    // cross mode: queries (and O) in their own row space; the fields above
    // then describe the keys (a history cache)
    const int32_t* q_offsets;
    const int64_t* ts_q;
    const uint32_t* enc_q;
    const uint32_t* stats_q;
    int nblk_q;
};

struct Smem {
    uint8_t k[kStages][BN * kRowBytes];   // [32 keys][128 d], 16-B chunk c of row r at c ^ (r & 15)
    uint8_t v[kStages][BN * kRowBytes];   // [32 keys][128 d], 16-B chunk c of row r at c ^ 4 (r & 3)
    uint32_t tsk[kStages][64];            // [0..31] key codes, [32..33] key block range
    float tt_fast[32];                    // by leading-zero count of 2|dt| + 1
    float tt_wide[65];                    // by bit length of |dt|
    int32_t item[8];
    int32_t work;
};

// Per-item state of the tile loads.  Wave w fills key rows 8w .. 8w+7 of the
// K and V tiles with 2 buffer loads each: lane l of load m writes 16 bytes at
// row 8w + 4m + l/16, physical chunk l % 16, so it fetches the logical chunk
// that the swizzle puts there.  Wave 0 also loads the 32 key codes with one
// 4-byte-per-lane load.
struct TileDma {
    u32x4 krs, vrs, wrs;
    uint32_t koff[2], voff[2];
    uint32_t ktile, vtile;        // bytes per key tile in K and V
    uint32_t code_off;            // lane < 32: byte offset of the sequence's code `lane`; else out of range
};

// The three parts of a tile's loads go out at different points of the
// previous tiles' work, so that no wave stalls long on a full load queue.
__device__ __forceinline__ void issue_k(const TileDma& d, Smem& s, int stage, int kt, int wave) {
    const uint32_t kl = lds_addr(s.k[0]) + (uint32_t)(stage * (BN * kRowBytes) + 2 * wave * 1024);
    const uint32_t ksoff = uniu((uint32_t)kt * d.ktile);
#pragma unroll
    for (int m = 0; m < 2; ++m) dma16(d.krs, uniu(kl + m * 1024), d.koff[m], ksoff);
}
__device__ __forceinline__ void issue_v(const TileDma& d, Smem& s, int stage, int kt, int wave) {
    const uint32_t vl = lds_addr(s.v[0]) + (uint32_t)(stage * (BN * kRowBytes) + 2 * wave * 1024);
    const uint32_t vsoff = uniu((uint32_t)kt * d.vtile);
#pragma unroll
    for (int m = 0; m < 2; ++m) dma16(d.vrs, uniu(vl + m * 1024), d.voff[m], vsoff);
}
// Wave 0 only: the tile's 32 key codes (lanes 32-63 write zeros; codes of
// keys past the sequence end are other rows' or zeros, and those keys are
// masked).  The lane's offset is fixed per item, the tile is the scalar offset.
__device__ __forceinline__ void issue_codes(const TileDma& d, Smem& s, int stage, int kt) {
    const uint32_t lds = uniu(lds_addr(s.tsk[0]) + (uint32_t)(stage * 64 * 4));
    const uint32_t soff = uniu((uint32_t)kt * (uint32_t)(BN * 4));
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(d.code_off), "s"(d.wrs), "s"(soff),
                 "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void issue_tile(const TileDma& d, Smem& s, int stage, int kt, int L, int wave,
                                           int lane) {
    issue_k(d, s, stage, kt, wave);
    issue_v(d, s, stage, kt, wave);
    if (wave == 0) issue_codes(d, s, stage, kt);
}

// kCross: the queries are candidates in their own buffers, each seeing every
// key of its sequence's history (position n, no mask beyond the key count);
// their own key is added by the epilogue.
template <bool kSilu, bool kCross>
__global__ void __launch_bounds__(kThreads, 2) attn_bf16_kernel(Params p, const void* ws_base, uint32_t ws_bytes) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    Smem& s = *reinterpret_cast<Smem*>(smem_raw);
    float* ptab = reinterpret_cast<float*>(smem_raw + ((sizeof(Smem) + 15) & ~size_t(15)));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int l32 = lane & 31;
    const int h2 = lane >> 5;            // which 8-wide k slice / 4-key group of the lane
    const int total_work = p.ctrl[0] * p.H;
    const bool shared_tables = (p.rp_hs == 0) && (p.rt_hs == 0);
    const int P = p.P;
    const int Dhi = P + 63;              // position difference of reversed-table entry 0
    const int CS = p.pos_copy;
    const float kNegLog2e = -kLog2e;
    const float alpha_eff = kSilu ? -p.alpha * 0.69314718055994531f : p.alpha;
    const int per_tile = uni(wave == 0 ? 5 : 4);   // buffer loads per tile of this wave
    const u32x4 wrs = make_rsrc(ws_base, ws_bytes);
    const int64_t enc_base = (const uint8_t*)p.enc - (const uint8_t*)ws_base;
    // key block ranges through the scalar cache (uniform addresses)
    const __attribute__((address_space(4))) u32x2* kstats =
        (const __attribute__((address_space(4))) u32x2*)(uintptr_t)p.stats;
    int loaded_head = -1;
    // the accelerator die (XCD) this workgroup runs on
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
    const int my_xcd = (int)(xcc & (kXcds - 1));

    for (;;) {
        if (tid == 0) {
            // die x takes the entries x, x + 8, x + 16, ... of the
            // longest-first list (an equal share of a cost-sorted list); an
            // entry's head is rotated by its sequence (below), so a die runs
            // the row blocks of a few sequence-heads, whose K/V then meet in
            // its L2, and different dies read different heads' columns; a die
            // out of work takes the others' remaining entries
            int w = total_work;
            for (int k = 0; k < kXcds; ++k) {
                const int x = (my_xcd + k) & (kXcds - 1);
                int32_t* cur = p.cursor + kXcdStride * x;
                // a queue seen exhausted is skipped with a load, not an atomic
                if (k > 0 && __hip_atomic_load(cur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * kXcds + x >=
                                 total_work)
                    continue;
                const int ww = atomicAdd(cur, 1) * kXcds + x;
                if (ww < total_work) {
                    w = ww;
                    break;
                }
            }
            s.work = w;
            if (w < total_work) {
                const WorkItem it = p.items[w / p.H];
                s.item[0] = it.b; s.item[1] = it.qt; s.item[2] = it.a_end; s.item[3] = it.kb;
                s.item[4] = it.pr; s.item[5] = it.slot; s.item[6] = it.k; s.item[7] = it.n;
            }
        }
        lds_sync();
        const int w = uni(s.work);
        if (w >= total_work) break;
        const int b = uni(s.item[0]), qt = uni(s.item[1]), a_end = uni(s.item[2]);
        const int kbw = uni(s.item[3]);
        const int kb_begin = kbw & 0xffff;
        const int prw = uni(s.item[4]);
        const int p0 = prw & 0xffff, p1 = prw >> 16;   // this piece's positions in the tile list
        const int slot = uni(s.item[5]), piece = uni(s.item[6]), npieces = uni(s.item[7]);
        const int h = (w % p.H + p.H - b % p.H) % p.H;   // head order rotated by the sequence

        // wave-uniform by construction; readfirstlane lets the compiler keep
        // them (and the buffer descriptors built from them) in SGPRs
        const int64_t row0 = uni(p.offsets[b]);
        const int L = uni(p.lengths ? p.lengths[b] : p.offsets[b + 1] - (int)row0);
        const int n = kCross ? L : uni(p.ncand ? L - p.ncand[b] : L);
        const int bbase = b * p.nblk;
        // query rows: the sequence's own, or (cross) the candidates'
        const int64_t row0q = kCross ? (int64_t)uni(p.q_offsets[b]) : row0;
        const int Lq = kCross ? uni(p.q_offsets[b + 1] - (int)row0q) : L;

        // ---- bias tables (reloaded only when they differ by head)
        if (loaded_head < 0 || (!shared_tables && loaded_head != h)) {
            const float* rp = p.rab_pos + (int64_t)h * p.rp_hs;
            const float* rt = p.rab_time + (int64_t)h * p.rt_hs;
            // copy c holds Rv[w - c], Rv[u] = rab_pos[clamp(Dhi - u, 0, P-1)]
            for (int e = tid; e < 2 * CS; e += kThreads) {
                const int c = e / CS;
                const int u = e - c * CS - c;
                const int dd = min(max(Dhi - u, 0), P - 1);
                ptab[e] = rp[dd];
            }
            if (tid < 32) s.tt_fast[tid] = rt[min(p.NT - 1, 31 - tid)];
            if (tid < 65) s.tt_wide[tid] = rt[min(p.NT - 1, tid)];
            loaded_head = h;
            lds_wait();   // visible to all after the first tile's barrier
        }

        // ---- tile loads: the first kStages - 1 tiles go out before this
        //      item's other global reads, so that all of them share one latency
        TileDma dma;
        {
            const uint16_t* kb0 = p.k + row0 * p.ks + h * HD;
            const uint16_t* vb0 = p.v + row0 * p.vs + h * HD;
            dma.krs = make_rsrc(kb0, (uint32_t)(L * p.ks * 2));
            dma.vrs = make_rsrc(vb0, (uint32_t)(L * p.vs * 2));
            dma.wrs = wrs;
            const int pc = lane & 15;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int rr = 8 * wave + 4 * m + (lane >> 4);
                dma.koff[m] = (uint32_t)(rr * p.ks * 2 + ((pc ^ (rr & 15)) << 4));
                dma.voff[m] = (uint32_t)(rr * p.vs * 2 + ((pc ^ ((rr & 3) << 2)) << 4));
            }
            dma.ktile = (uint32_t)(BN * p.ks * 2);
            dma.vtile = (uint32_t)(BN * p.vs * 2);
            dma.code_off = lane < 32 ? (uint32_t)(enc_base + 4 * (row0 + lane)) : 0x80000000u;
        }
        const int ntiles = p1 - p0;
        auto tile_of = [&](int it) {
            const int pos = p0 + it;
            return pos < a_end ? pos : kb_begin + (pos - a_end);
        };
#pragma unroll
        for (int pre = 0; pre < kStages - 1; ++pre)
            if (pre < ntiles) issue_tile(dma, s, pre, tile_of(pre), L, wave, lane);

        // ---- this wave's 32 query rows
        const int wrow0 = qt * BM + wave * 32;
        const int i = wrow0 + l32;               // this lane's query row
        const bool row_valid = i < Lq;
        bf16x8 qf[8];
        {
            const uint16_t* qp = p.q + (row0q + i) * p.qs + h * HD + h2 * 8;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                u32x4 z = {0u, 0u, 0u, 0u};
                if (row_valid) z = *reinterpret_cast<const u32x4*>(qp + kc * 16);
                qf[kc] = __builtin_bit_cast(bf16x8, z);
            }
        }
        // (cross: a user without history has no keys, and no rows to read)
        const int64_t t_first = (!kCross || L > 0) ? p.ts[row0] : 0;
        const int64_t ti64 = row_valid ? (kCross ? p.ts_q[row0q + i] : p.ts[row0 + i]) : t_first;
        uint32_t tie = row_valid ? (kCross ? p.enc_q[row0q + i] : p.enc[row0 + i]) : 0x80000000u;
        const int qblk = (kCross ? b * p.nblk_q : bbase) + qt * (BM / 32) + wave;   // this wave's 32-row block
        const uint32_t* qstats = kCross ? p.stats_q : p.stats;
        const bool wave_rows = wrow0 < Lq;
        uint32_t rmin = wave_rows ? qstats[2 * qblk] : 0x80000000u;
        uint32_t rmax = wave_rows ? qstats[2 * qblk + 1] : 0x80000000u;
        rmin = uniu(rmin);
        rmax = uniu(rmax);
        const bool rows_wide = rmin > rmax;
        const int prow = kCross ? n : min(i, n);
        // visibility of row i (rows past L see nothing): keys j <= vis_lim,
        // and j == vis_self for a candidate row (cross: every history key)
        const int vis_lim = kCross ? (i < Lq ? n - 1 : -1) : (i >= L ? -1 : (i < n ? i : n - 1));
        const int vis_self = kCross ? -1 : ((i >= n && i < L) ? i : -1);
        const bool cand_rows = kCross ? false : wrow0 + 31 >= n;   // the block holds candidate rows
        const int prow_min = kCross ? n : uni(min(wrow0, n));
        // time table by leading-zero count, one entry per lane (lanes 32-63
        // repeat 0-31), read with readlane for block-uniform buckets
        int ttv = __builtin_bit_cast(int, p.rab_time[(int64_t)h * p.rt_hs + min(p.NT - 1, 31 - l32)]);
        float pos_far = p.rab_pos[(int64_t)h * p.rp_hs + P - 1];   // every clamped difference
        // These item-level loads complete here: a value still in flight at
        // the loop entry would make the compiler wait for every load (the
        // tile loads included) at its first use in each iteration.
        asm volatile("" : "+v"(pos_far), "+v"(ttv), "+v"(tie), "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]), "+v"(qf[4]),
                     "+v"(qf[5]), "+v"(qf[6]), "+v"(qf[7]));

        f32x16 oacc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.0f;

        // ---- software pipeline over the key tiles.  Iteration it builds
        //      S(it) while it finishes tile it-1: the activation of S(it-1)
        //      runs on the VALU while S(it)'s LDS reads are in flight, then
        //      the MFMAs of S(it) = K Q^T and of O += A(it-1) V(it-1) go out
        //      interleaved (two independent chains keep the matrix pipe
        //      busy), and V(it) is read into registers for the next iteration.
        u32x2 krange_next = {0u, 0u};
        if (!kCross || ntiles > 0) krange_next = kstats[bbase + tile_of(0)];
        u32x4 vf[2][4];
        const uint32_t koff_lane = k_lane_offset(lane), voff_lane = v_lane_offset(lane);
        const uint32_t ptab_lds = lds_addr(ptab);
        const int prow4 = prow - 4 * h2;   // the position term's row part for this lane's keys

        // the barrier of tile it (its loads have landed, every wave is done
        // with tile it-1's stage: V(it-1) was read before it), then the K
        // part of tile it+3's loads into that stage
        auto tile_sync = [&](int it) {
            const int later = min(kStages - 2, ntiles - 1 - it);
            wait_vmcnt(later * per_tile);
            lds_sync();
            if (it + kStages - 1 < ntiles)
                issue_k(dma, s, (it + kStages - 1) & (kStages - 1), tile_of(it + kStages - 1), wave);
        };

        // bias of tile it (as the initial accumulator, plus a constant) and
        // its K fragments; the time part follows in time_bias (after other
        // work has covered the LDS latency of the codes)
        struct TileFacts {
            bool wide;
            int czlo, czhi, j0;
        };
        auto tile_bias = [&](int it, f32x16& acc, float& cadd, bf16x8 (&kf)[8]) -> TileFacts {
            const int kt = tile_of(it);
            const int j0 = kt * BN;
            const int stage = it & (kStages - 1);
            const uint8_t* k_lds = s.k[stage];

            // block-uniform facts (scalar; the key block's code range was
            // loaded one tile ahead)
            const uint32_t kmn = uniu(krange_next[0]), kmx = uniu(krange_next[1]);
            if (it + 1 < ntiles) krange_next = kstats[bbase + tile_of(it + 1)];
            const bool wide = rows_wide || kmn > kmx;
            const uint32_t lo = rmin >= kmx ? rmin - kmx : (kmn >= rmax ? kmn - rmax : 0u);
            const uint32_t hi = max(rmax >= kmn ? rmax - kmn : 0u, kmx >= rmin ? kmx - rmin : 0u);
            const int czlo = (int)clz_gap(lo), czhi = (int)clz_gap(hi);   // czhi <= czlo
            const bool pos_clamped = prow_min - (j0 + 31) >= P - 1;

            // LDS reads: position entries when needed, then K (the key codes,
            // when needed, are read by time_bias)
            // position bias: lane (row i, keys j0 + 8q + 4h2 + t) reads
            // reversed-table entries u0 + 8q + t; a block whose differences
            // all clamp takes rab_pos[P-1] as a constant
            cadd = 0.0f;
            if (pos_clamped) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
                cadd = pos_far;
            } else {
                // entries u0 + 8q + t, u0 = Dhi - x, from copy c = u0 & 1 at
                // float index c * (CS + 1) + u0: one base, immediate offsets
                const int x = min(max(prow4 - j0, 0), P + 26);
                const int u0 = Dhi - x;
                const uint32_t pa = ptab_lds + 4u * (uint32_t)u0 + (uint32_t)(u0 & 1) * (4u * (uint32_t)CS + 4u);
                typedef float f32x2v __attribute__((ext_vector_type(2)));
                typedef __attribute__((address_space(3))) const f32x2v lds_f2;
                const lds_f2* pp = (const lds_f2*)(uintptr_t)pa;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const f32x2v pv = pp[4 * q + t2];
                        acc[4 * q + 2 * t2] = pv[0];
                        acc[4 * q + 2 * t2 + 1] = pv[1];
                    }
                }
            }
            uint32_t ko = koff_lane;
            asm volatile("" : "+v"(ko));   // recomputed per tile: keeps one register live, not eight
            const uint32_t kb = lds_addr(k_lds) + ko;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) kf[kc] = lds_read_b128(kb ^ (uint32_t)(kc << 5));
            return TileFacts{wide, czlo, czhi, j0};
        };
        auto time_bias = [&](int it, const TileFacts& f, f32x16& acc, float& cadd) {
                const bool wide = f.wide;
                const int czlo = f.czlo, czhi = f.czhi, j0 = f.j0;
                const uint32_t* tsk = s.tsk[it & (kStages - 1)];
                u32x4 codes[4];
                if (!wide && czlo != czhi) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) codes[q] = *reinterpret_cast<const u32x4*>(&tsk[8 * q + 4 * h2]);
                }
                // time bias: constant over the block (most blocks), one of two
                // buckets split at a power of two, or per element
                if (!wide && czlo - czhi <= 1) {
                    const float tlo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ttv, czlo));
                    if (czlo == czhi) {
                        cadd += tlo;
                    } else {
                        // |e_i - e_j| + 1 < 2^(32 - czlo) exactly when the bucket is czlo
                        const float thi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ttv, czhi));
                        uint32_t thr = 1u << (32 - czlo);
                        asm volatile("" : "+s"(thr));   // opaque: one compare per element, not a shift and a compare
#pragma unroll
                        for (int q = 0; q < 4; ++q)
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                acc[4 * q + t] += sad_u32(tie, codes[q][t], 1u) >= thr ? thi : tlo;
                    }
                } else if (!wide) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            acc[4 * q + t] += s.tt_fast[__builtin_clz(sad_u32(tie, codes[q][t], 1u))];
                } else {
                    const int64_t* tsb = p.ts + row0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int j = j0 + 8 * q + 4 * h2 + t;
                            const int64_t tj = j < L ? tsb[j] : t_first;
                            const int64_t dt = ti64 - tj;
                            const uint64_t ad = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
                            acc[4 * q + t] += s.tt_wide[bit_length_u64(ad)];
                        }
                    }
                }
        };

        // activation of element r of S(it) (in place)
        auto act_one = [&](f32x16& acc, float c2, int r) {
            if (kSilu) {
                const float t = __builtin_fmaf(acc[r], kNegLog2e, c2);
                const float e = __builtin_amdgcn_exp2f(t);
                acc[r] = t * __builtin_amdgcn_rcpf(1.0f + e);
            } else {
                acc[r] = acc[r] + c2;
            }
        };
        auto act_const = [&](float cadd) { return kSilu ? cadd * kNegLog2e : cadd; };

        // mask of the activated S(it), packed to bf16: the A operand of
        // O += A V for the tile's two 16-key chunks
        auto tile_pack = [&](int it, const f32x16& a_in, u32x4 (&pk)[2]) {
            const int j0 = tile_of(it) * BN;
            const bool full = (j0 + 32 <= n) && (kCross || j0 + 31 <= wrow0);
            float a[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = a_in[r];
            if (!full) {
                // key j = j0 + 4h2 + c (c = 8q + t) is visible when j <=
                // vis_lim (causal history, or all history for a candidate) or
                // j == vis_self (a candidate's own key)
                const int jb = j0 + 4 * h2;
                const int xl = vis_lim - jb, xs = vis_self - jb;
                if (cand_rows) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            a[4 * q + t] = ((xl >= 8 * q + t) | (xs == 8 * q + t)) ? a[4 * q + t] : 0.0f;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int t = 0; t < 4; ++t) a[4 * q + t] = xl >= 8 * q + t ? a[4 * q + t] : 0.0f;
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[c][e] = pack_bf16x2(a[8 * c + 2 * e], a[8 * c + 2 * e + 1]);
        };

        // the V and key-code parts of tile it+3's loads
        auto issue_rest = [&](int it) {
            if (it + kStages - 1 < ntiles) {
                const int st3 = (it + kStages - 1) & (kStages - 1), kt3 = tile_of(it + kStages - 1);
                issue_v(dma, s, st3, kt3, wave);
                if (wave == 0) issue_codes(dma, s, st3, kt3);
            }
        };

        auto read_v = [&](int it) {
            uint32_t vo = voff_lane;
            asm volatile("" : "+v"(vo));
            read_v_tile(lds_addr(s.v[it & (kStages - 1)]), vo, vf);
        };

        // one pipeline step: S(it) into accN while tile it-1 (S in accC)
        // is finished
        auto step = [&](int it, f32x16& accC, float caddC, f32x16& accN, float& caddN) {
            tile_sync(it);
            bf16x8 kf[8];
            const TileFacts f = tile_bias(it, accN, caddN, kf);
            const float c2 = act_const(caddC);
            // the first activations cover the LDS latency of this tile's reads
#pragma unroll
            for (int r = 0; r < 4; ++r) act_one(accC, c2, r);
            time_bias(it, f, accN, caddN);
            issue_rest(it);
            // S(it) = K Q^T: a dependent chain of 8 MFMAs, each followed by
            // the activation of 1.5 elements of S(it-1)
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                accN = mfma32(kf[kc], qf[kc], accN);
                if (kc < 6) {
                    act_one(accC, c2, 4 + 2 * kc);
                    act_one(accC, c2, 5 + 2 * kc);
                }
            }
#pragma unroll
            for (int kc = 0; kc < 6; ++kc) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // then VALU
            }
            u32x4 pk[2];
            tile_pack(it - 1, accC, pk);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    oacc[nb] = mfma32(__builtin_bit_cast(bf16x8, pk[c]), __builtin_bit_cast(bf16x8, vf[c][nb]), oacc[nb]);
            read_v(it);
        };

        // The tile list runs over keys in increasing order, so the tiles past
        // the one holding this wave's last valid row hold no pair its rows
        // see (a history row sees keys up to itself, a candidate the history
        // and itself): the wave computes the first nuse tiles of the piece and
        // only keeps the ring going (barriers and its share of the loads) for
        // the rest.
        int nuse = ntiles;
        if (wrow0 >= Lq) {
            nuse = 0;
        } else if (!kCross) {
            const int kt_last = min(wrow0 + 31, L - 1) / BN;
            const int pos_last = kt_last < a_end ? kt_last : a_end + (kt_last - kb_begin);
            nuse = min(ntiles, max(0, pos_last + 1 - p0));
        }
        nuse = uni(nuse);

        if (nuse > 0) {
            f32x16 accA, accB;
            float caddA = 0.0f, caddB = 0.0f;
            // prologue: S(0), V(0)
            {
                tile_sync(0);
                bf16x8 kf[8];
                const TileFacts f = tile_bias(0, accA, caddA, kf);
                time_bias(0, f, accA, caddA);
                issue_rest(0);
#pragma unroll
                for (int kc = 0; kc < 8; ++kc) accA = mfma32(kf[kc], qf[kc], accA);
                read_v(0);
            }
            int it = 1;
            for (; it + 1 < nuse; it += 2) {
                step(it, accA, caddA, accB, caddB);
                step(it + 1, accB, caddB, accA, caddA);
            }
            if (it < nuse) {
                step(it, accA, caddA, accB, caddB);
                accA = accB;
                caddA = caddB;
                ++it;
            }
            // epilogue: finish the last tile
            {
                const float c2 = act_const(caddA);
#pragma unroll
                for (int r = 0; r < 16; ++r) act_one(accA, c2, r);
            }
            u32x4 pk[2];
            tile_pack(nuse - 1, accA, pk);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    oacc[nb] = mfma32(__builtin_bit_cast(bf16x8, pk[c]), __builtin_bit_cast(bf16x8, vf[c][nb]), oacc[nb]);
        }
        for (int it = nuse; it < ntiles; ++it) {
            tile_sync(it);
            issue_rest(it);
        }

        // ---------- O = alpha * acc, rows < L only: bf16 into O (non-temporal:
        //            the epilogue reads it once, and the tiles the other items
        //            still read keep the caches), or fp32 into the piece's
        //            partial slot when the row block is split
        // lane holds O[row 8 (r / 4) + 4 h2 + r % 4][d = nb * 32 + l32]
        if (slot < 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ro = wrow0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                if (ro < Lq) {
                    uint16_t* op = p.o + (row0q + ro) * p.os + h * HD + l32;
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) __builtin_nontemporal_store(f32_to_bf16_bits(alpha_eff * oacc[nb][r]), op + nb * 32);
                }
            }
        } else {
            float* pp = p.partial + ((int64_t)(slot + piece) * p.H + h) * (BM * HD);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wave * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                if (qt * BM + lr < Lq) {
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) pp[lr * HD + nb * 32 + l32] = alpha_eff * oacc[nb][r];
                }
            }
        }
        // the row map tells the epilogue which rows to sum from partial slots
        if (p.rowmap && h == 0 && piece == 0 && lane < 32) {
            const int lr = wave * 32 + lane;
            if (qt * BM + lr < Lq)
                p.rowmap[row0q + qt * BM + lr] = slot < 0 ? -1 : (slot | (npieces << 16) | (lr << 23));
        }
        lds_barrier();   // this item's LDS use is over before the next item starts
    }
}

}  // namespace

int attn_bf16_slots() { return device_cu_count() * 2; }

hipError_t launch_attn_bf16(const AttnCoreArgs& a, hipStream_t stream) {
    Params p;
    p.H = a.H;
    p.offsets = a.offsets; p.lengths = a.lengths; p.ncand = a.ncand;
    p.q = static_cast<const uint16_t*>(a.q); p.qs = a.q_stride;
    p.k = static_cast<const uint16_t*>(a.k); p.ks = a.k_stride;
    p.v = static_cast<const uint16_t*>(a.v); p.vs = a.v_stride;
    p.ts = a.ts;
    p.rab_pos = a.rab_pos; p.P = a.P; p.rp_hs = a.rp_head_stride;
    p.rab_time = a.rab_time; p.NT = a.NT; p.rt_hs = a.rt_head_stride;
    p.alpha = a.alpha;
    p.o = static_cast<uint16_t*>(a.o); p.os = a.o_stride;
    p.items = a.items; p.ctrl = a.ctrl;
    p.cursor = const_cast<int32_t*>(a.ctrl) + kXcdCursor;   // the per-XCD cursors
    p.stats = a.stats; p.enc = a.enc;
    p.partial = a.partial; p.rowmap = a.rowmap; p.nblk = a.nblk;
    p.pos_copy = ((a.P + 128 + 4) + 3) & ~3;
    p.q_offsets = a.q_offsets; p.ts_q = a.ts_q; p.enc_q = a.enc_q; p.stats_q = a.stats_q; p.nblk_q = a.nblk_q;
    const bool cross = a.q_offsets != nullptr;
    const size_t smem = ((sizeof(Smem) + 15) & ~size_t(15)) + sizeof(float) * 2 * size_t(p.pos_copy);
    const void* fn = cross ? (a.act == 0 ? reinterpret_cast<const void*>(attn_bf16_kernel<true, true>)
                                         : reinterpret_cast<const void*>(attn_bf16_kernel<false, true>))
                           : (a.act == 0 ? reinterpret_cast<const void*>(attn_bf16_kernel<true, false>)
                                         : reinterpret_cast<const void*>(attn_bf16_kernel<false, false>));
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    const int grid = attn_bf16_slots();
    // one buffer resource covers the block ranges and the row codes
    const void* ws_base = a.stats;
    const size_t span = (size_t)((const uint8_t*)(a.enc + a.num_rows) - (const uint8_t*)a.stats);
    const uint32_t wsb = (uint32_t)(span > 0x7fffffffu ? 0x7fffffffu : span);
    if (cross) {
        if (a.act == 0)
            hipExtLaunchKernelGGL((attn_bf16_kernel<true, true>), dim3(grid), dim3(kThreads), smem, stream,
                                  a.ev_begin, a.ev_end, 0, p, ws_base, wsb);
        else
            hipExtLaunchKernelGGL((attn_bf16_kernel<false, true>), dim3(grid), dim3(kThreads), smem, stream,
                                  a.ev_begin, a.ev_end, 0, p, ws_base, wsb);
    } else if (a.act == 0) {
        hipExtLaunchKernelGGL((attn_bf16_kernel<true, false>), dim3(grid), dim3(kThreads), smem, stream,
                              a.ev_begin, a.ev_end, 0, p, ws_base, wsb);
    } else {
        hipExtLaunchKernelGGL((attn_bf16_kernel<false, false>), dim3(grid), dim3(kThreads), smem, stream,
                              a.ev_begin, a.ev_end, 0, p, ws_base, wsb);
    }
    return hipGetLastError();
}

}  // namespace hstu
