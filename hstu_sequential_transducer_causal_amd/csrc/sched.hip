// sched.hip -- jagged tile scheduler.
//
// Builds, on the device and from the sequence offsets alone, the list of
// work items of the attention core: one item per (sequence, block of BM
// query rows), carrying the key-tile ranges that hold at least one visible
// pair.  Processing real lengths instead of padded ones is the point of the
// jagged kernel described on "Meta HSTU: как действия пользователя стали
// основой большой рекомендательной модели" (section "Разная длина истории
// превращается в выигрыш по ресурсам"); the M-FALCON mask ("生成式推荐（一）：
// HSTU", section "M-FALCON") lets candidate rows skip the key tiles that
// hold only other candidates.
//
// Key tiles of the query rows [q0, q1) of a sequence with n history rows:
//   q1 <= n (history only):   [0, ceil(q1 / BN))
//   otherwise:                [0, ceil(n / BN)) for the history columns, plus
//                             the tiles of the candidates' own diagonal
//                             [max(q0, n) / BN, ceil(q1 / BN)) beyond it.
// In key-major mode (the key and value gradients) an item is a block of BM
// keys instead, with the one range of BN-row query tiles that see them.
//
// Items are written longest first (counting sort on the number of key
// tiles) so that the persistent attention kernel, which takes items in list
// order, balances its CUs like a longest-processing-time schedule.
//
// One workgroup of 1024 threads runs the whole build (a few microseconds next
// to the attention core); the launch's other workgroups encode the timestamps
// (prep_kernel).  The gradients build their two lists and the G-block prefix
// in one launch (prep_pair_kernel).  The batch validator (validate_batch)
// lives here too.
#include <algorithm>

#include "internal.h"
#include "hstu_device.h"

namespace hstu {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBins = kMaxSeqLen / 32 + 2;  // cost <= number of key tiles of a sequence
// Batches of up to this many sequences keep their per-sequence data in LDS
// (the binary searches below then never wait on memory); larger ones use the
// workspace copies.
constexpr int kLdsSeq = 4096;
// Up to this many row blocks keep their cost (key tiles) in LDS between the
// passes; longer lists recompute it.
constexpr int kLdsItems = 8192;
// 32-row timestamp blocks per workgroup of the timestamp role.
constexpr int kTsPerGroup = kThreads / 32;

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Tile sizes are powers of two (launch_sched checks): tiles of 2^s rows.
struct TileShift {
    int m, n;   // log2 of the query (or key-major block) tile and the key tile
};
__device__ __forceinline__ int ceil_tiles(int x, int s) { return (x + (1 << s) - 1) >> s; }   // x >= 0
inline bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

struct Ranges {
    int a_end, kb_begin, kb_end;
};

__device__ __forceinline__ Ranges tile_ranges(int L, int n, int qt, TileShift ts, bool kv_mode, bool cross) {
    if (cross) {
        // candidate rows against a history cache of n keys: all of them
        Ranges r;
        r.a_end = ceil_tiles(n, ts.n);
        r.kb_begin = r.kb_end = r.a_end;
        return r;
    }
    if (kv_mode) {
        // key block [k0, k1): the 32-row query tiles from k0's on -- to the
        // end for a block holding history keys (every later row and every
        // candidate sees them), to k1 for a block of candidates only (each is
        // seen by itself alone)
        const int k0 = qt << ts.m, k1 = min(k0 + (1 << ts.m), L);
        Ranges r;
        r.a_end = 0;
        r.kb_begin = k0 >> ts.n;
        r.kb_end = ceil_tiles(k0 < n ? L : k1, ts.n);
        return r;
    }
    int q0 = qt << ts.m;
    int q1 = min(q0 + (1 << ts.m), L);
    Ranges r;
    if (q1 <= n) {
        r.a_end = ceil_tiles(q1, ts.n);
        r.kb_begin = r.kb_end = r.a_end;
    } else {
        r.a_end = ceil_tiles(n, ts.n);
        r.kb_begin = max(max(q0, n) >> ts.n, r.a_end);
        r.kb_end = max(ceil_tiles(q1, ts.n), r.kb_begin);
    }
    return r;
}

struct SchedSmem {
    int hist[kMaxBins];
    int wave_tot[kWaves];
    long long wave_sum[kWaves];
    int wave_max[kWaves];
    int carry, carry2;
    int qscan[kLdsSeq + 1];
    int len[kLdsSeq];
    int nhist[kLdsSeq];          // history rows n_b
    int row0[kLdsSeq];           // first row offsets[b]
    uint16_t cost[kLdsItems];
};

// Exclusive scan of one value per thread over the workgroup; also returns
// the workgroup total.  All threads must call it.
__device__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        int s = wave_tot[i];
        before += (i < w) ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

// Workgroup sum (64-bit) and maximum of one value per thread; all threads
// must call it.
__device__ long long block_sum_max(long long v, int m, SchedSmem& s, int& mx) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        v += __shfl_xor(v, o, 64);
        m = max(m, __shfl_xor(m, o, 64));
    }
    if (lane == 0) {
        s.wave_sum[w] = v;
        s.wave_max[w] = m;
    }
    __syncthreads();
    long long t = 0;
    int tm = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        t += s.wave_sum[i];
        tm = max(tm, s.wave_max[i]);
    }
    __syncthreads();
    mx = tm;
    return t;
}

__device__ __forceinline__ int seq_length(const SchedArgs& a, int b) {
    return a.lengths ? a.lengths[b] : a.offsets[b + 1] - a.offsets[b];
}

__device__ __forceinline__ int seq_history(const SchedArgs& a, int b, int L) {
    if (a.kv_offsets) return a.kv_offsets[b + 1] - a.kv_offsets[b];   // cross: the history cache
    return a.ncand ? L - a.ncand[b] : L;
}

// First query tile of a sequence in the work list: 0, or with cand_only the
// tile holding the first candidate row.
__device__ __forceinline__ int first_tile(const SchedArgs& a, int n, int sm) { return a.cand_only ? n >> sm : 0; }

// Query tiles of a sequence in the work list (with cand_only, none for a
// sequence without candidates).
__device__ __forceinline__ int tile_count(const SchedArgs& a, int L, int n, int sm) {
    if (a.cand_only && L <= n) return 0;
    return ceil_tiles(L, sm) - first_tile(a, n, sm);
}

// Pieces of a row block of c key tiles at piece size `chunk` (a block is
// split only when it exceeds 1.5 chunks: a little over the mean work per
// workgroup does not hold up the grid's end, while the split costs partial
// traffic), and the end (exclusive, in list positions) of piece k;
// piece_end(c, n, -1) = 0.
__device__ __forceinline__ int pieces_of(int c, int chunk) {
    return 2 * (int64_t)c > 3 * (int64_t)chunk ? min(ceil_div(c, chunk), 64) : 1;
}
__device__ __forceinline__ int piece_end(int c, int n, int k) { return (int)(((int64_t)c * (k + 1)) / n); }

// Sequence of flat query tile f: the last b with qscan[b] <= f.
template <typename Ptr>
__device__ __forceinline__ int find_seq(Ptr qscan, int B, int f) {
    int lo = 0, hi = B;  // qscan[lo] <= f < qscan[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (qscan[mid] <= f) lo = mid; else hi = mid;
    }
    return lo;
}

// Workgroup 0 of the preparation launch: the work list.
__device__ void build_work_list(const SchedArgs& a, SchedSmem& s) {
    const int tid = threadIdx.x;
    const TileShift tsh = {__builtin_ctz((unsigned)a.tile_m), __builtin_ctz((unsigned)a.tile_n)};
    const bool in_lds = a.B <= kLdsSeq;
    // costs (key tiles of an item) lie in [0, ceil(max_seq_len / BN)]
    const int nbins = min(kMaxBins, ceil_tiles(a.max_seq_len, tsh.n) + 2);

    for (int i = tid; i < nbins; i += kThreads) s.hist[i] = 0;
    if (tid == 0) s.carry = 0;
    __syncthreads();

    // 1. query tiles per sequence -> exclusive prefix qscan[0..B]
    for (int base = 0; base < a.B; base += kThreads) {
        const int b = base + tid;
        int nq = 0;
        if (b < a.B) {
            const int L = seq_length(a, b);
            const int n = seq_history(a, b, L);
            nq = tile_count(a, L, n, tsh.m);
            if (in_lds) {
                s.len[b] = L;
                s.nhist[b] = n;
                s.row0[b] = a.offsets[b];
            }
        }
        int total;
        const int ex = block_exclusive_scan(nq, s.wave_tot, total);
        const int carry = s.carry;
        if (b < a.B) {
            a.qscan[b] = carry + ex;
            if (in_lds) s.qscan[b] = carry + ex;
        }
        __syncthreads();
        if (tid == 0) s.carry = carry + total;
        __syncthreads();
    }
    const int nitems = s.carry;
    if (tid == 0) {
        a.qscan[a.B] = nitems;
        if (in_lds) s.qscan[a.B] = nitems;
    }
    __syncthreads();
    const bool cost_in_lds = in_lds && nitems <= kLdsItems;

    // the row block of flat query tile f
    auto item_of = [&](int f, int& b, int& qt) -> Ranges {
        int L, n;
        if (in_lds) {
            b = find_seq(s.qscan, a.B, f);
            qt = f - s.qscan[b];
            L = s.len[b];
            n = s.nhist[b];
        } else {
            b = find_seq(a.qscan, a.B, f);
            qt = f - a.qscan[b];
            L = seq_length(a, b);
            n = seq_history(a, b, L);
        }
        qt += first_tile(a, n, tsh.m);
        return tile_ranges(L, n, qt, tsh, a.kv_mode != 0, a.kv_offsets != nullptr);
    };
    auto cost_of = [](const Ranges& r) { return r.a_end + (r.kb_end - r.kb_begin); };
    auto cost_at = [&](int f) {
        if (cost_in_lds) return (int)s.cost[f];
        int b, qt;
        return cost_of(item_of(f, b, qt));
    };

    // 2. costs, their total (key tiles over all blocks) and maximum
    long long work;
    int max_cost;
    {
        long long mine = 0;
        int mx = 0;
        for (int f = tid; f < nitems; f += kThreads) {
            int b, qt;
            const int c = cost_of(item_of(f, b, qt));
            if (cost_in_lds) s.cost[f] = (uint16_t)c;
            mine += c;
            mx = max(mx, c);
        }
        work = block_sum_max(mine, mx, s, max_cost);   // (its barriers publish s.cost)
    }

    // 3. piece size: only blocks longer than the mean work per workgroup --
    //    which would hold up the persistent grid's end -- are split, within
    //    the partial-slot budget
    int chunk = 1 << 30;
    if (a.part_slots > 0 && a.slots > 0) {
        const unsigned long long units = (unsigned long long)work * (unsigned long long)a.H;
        // (a 32-bit division when it fits: the 64-bit one is a long routine)
        const unsigned long long per_slot =
            units < (1ull << 31) ? (unsigned long long)(((uint32_t)units + (uint32_t)a.slots - 1u) / (uint32_t)a.slots)
                                 : (units + a.slots - 1) / (unsigned long long)a.slots;
        chunk = max(kMinPieceTiles, (int)min(per_slot, 1ull << 20));
        for (int round = 0; round < 24 && pieces_of(max_cost, chunk) > 1; ++round) {
            int mine = 0;
            for (int f = tid; f < nitems; f += kThreads) {
                const int np = pieces_of(cost_at(f), chunk);
                mine += np > 1 ? np : 0;
            }
            int unused;
            const long long sp = block_sum_max(mine, 0, s, unused);
            if (sp * a.H <= a.part_slots) break;
            chunk *= 2;
        }
        if (pieces_of(max_cost, chunk) > 1) {
            // (the budget loop ended without fitting: cannot happen for
            // lengths within max_seq_len, but never overrun the slots)
            int mine = 0;
            for (int f = tid; f < nitems; f += kThreads) {
                const int np = pieces_of(cost_at(f), chunk);
                mine += np > 1 ? np : 0;
            }
            int unused;
            if (block_sum_max(mine, 0, s, unused) * a.H > a.part_slots) chunk = 1 << 30;
        }
    }
    const bool any_split = pieces_of(max_cost, chunk) > 1;

    // 4. histogram of piece costs
    for (int f = tid; f < nitems; f += kThreads) {
        const int c = cost_at(f);
        const int np = any_split ? pieces_of(c, chunk) : 1;
        if (np == 1) {
            atomicAdd(&s.hist[min(c, nbins - 1)], 1);
        } else {
            for (int k = 0; k < np; ++k)
                atomicAdd(&s.hist[min(piece_end(c, np, k) - piece_end(c, np, k - 1), nbins - 1)], 1);
        }
    }
    __syncthreads();

    // 5. start position of each cost bin, largest cost first: one wave scans
    //    the bins in that order (lane l takes positions [l per, l per + per),
    //    position p being bin nbins - 1 - p)
    if (tid < 64) {
        const int per = (nbins + 63) / 64;
        int sum = 0;
        for (int k = 0; k < per; ++k) {
            const int pos = tid * per + k;
            if (pos < nbins) sum += s.hist[nbins - 1 - pos];
        }
        int x = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (tid >= o) x += y;
        }
        int run = x - sum;
        for (int k = 0; k < per; ++k) {
            const int pos = tid * per + k;
            if (pos < nbins) {
                const int c = s.hist[nbins - 1 - pos];
                s.hist[nbins - 1 - pos] = run;
                run += c;
            }
        }
        if (tid == 63) s.carry = x;
    }
    __syncthreads();
    const int npieces = s.carry;

    // 6. scatter the pieces into their bins; split blocks get consecutive
    //    partial slots and an entry in the split-block list
    if (tid == 0) {
        s.carry = 0;    // split blocks so far
        s.carry2 = 0;   // partial slots so far
    }
    __syncthreads();
    for (int base = 0; base < nitems; base += kThreads) {
        const int f = base + tid;
        int b = 0, qt = 0, c = 0, np = 1;
        Ranges r = {0, 0, 0};
        ItemSeq sq = {0, 0, 0, 0};
        if (f < nitems) {
            r = item_of(f, b, qt);
            c = cost_of(r);
            np = any_split ? pieces_of(c, chunk) : 1;
            if (a.item_seq) {
                sq.row0 = in_lds ? s.row0[b] : a.offsets[b];
                sq.L = in_lds ? s.len[b] : seq_length(a, b);
                sq.n = in_lds ? s.nhist[b] : seq_history(a, b, sq.L);
            }
        }
        int sx = 0, px = 0, nsplit = 0, nslots = 0;
        if (any_split) {
            // one scan of (split blocks << 17 | their slots): at most 1024
            // blocks of at most 64 pieces in a pass
            int tot;
            const int packed = np > 1 ? (1 << 17) | np : 0;
            const int ex = block_exclusive_scan(packed, s.wave_tot, tot);
            sx = ex >> 17;
            px = ex & 0x1ffff;
            nsplit = tot >> 17;
            nslots = tot & 0x1ffff;
        }
        const int scarry = s.carry, pcarry = s.carry2;
        if (f < nitems) {
            const int slot = np > 1 ? pcarry + px : -1;
            if (np > 1 && scarry + sx < a.cap) {
                SplitBlock sb;
                sb.b = b; sb.qt = qt; sb.slot = slot; sb.n = np;
                a.split[scarry + sx] = sb;
            }
            for (int k = 0; k < np; ++k) {
                const int p0 = piece_end(c, np, k - 1), p1 = piece_end(c, np, k);
                const int pos = atomicAdd(&s.hist[min(p1 - p0, nbins - 1)], 1);
                WorkItem it;
                it.b = b;
                it.qt = qt;
                it.a_end = r.a_end;
                it.kb = r.kb_begin | (r.kb_end << 16);
                it.pr = p0 | (p1 << 16);
                it.slot = slot;
                it.k = k;
                it.n = np;
                if (pos < a.cap_pieces) {   // (lengths within max_seq_len always fit)
                    a.items[pos] = it;
                    if (a.item_seq) a.item_seq[pos] = sq;
                }
            }
        }
        if (any_split) {
            __syncthreads();
            if (tid == 0) {
                s.carry = scarry + nsplit;
                s.carry2 = pcarry + nslots;
            }
            __syncthreads();
        }
    }
    if (tid == 0) {
        a.ctrl[0] = (int)min((int64_t)npieces, a.cap_pieces);
        a.ctrl[1] = 0;
        a.ctrl[2] = any_split ? (int)min((int64_t)s.carry, a.cap) : 0;
        for (int x = 0; x < kXcds; ++x) a.ctrl[kXcdCursor + kXcdStride * x] = 0;
    }
}

// Workgroups 1.. of the preparation launch: per row the timestamp code
// e = 2 (t - t_first) + 2^31 (t_first: the sequence's first row) and, per
// 32-row block (sequence b, block j at index b * nblk + j), the code range
// [min e, max e]; a block with some |t - t_first| >= 2^30 gets the range
// {0xffffffff, 0}.  One half-wave per block.
__device__ void encode_timestamps(const SchedArgs& a, int first_block) {
    const int lane = threadIdx.x & 63;
    const int64_t g = ((int64_t)blockIdx.x - first_block) * kTsPerGroup + (threadIdx.x >> 5);
    const int b = (int)(g / a.nblk);
    const int j0 = (int)(g - (int64_t)b * a.nblk) * kTsBlock;
    bool active = g < a.cap_blk;
    int64_t row0 = 0;
    int L = 0;
    if (active) {
        row0 = a.offsets[b];
        L = seq_length(a, b);
        active = j0 < L;
    }
    uint32_t mn = 0xffffffffu, mx = 0u;
    bool narrow = true;
    const int j = j0 + (lane & 31);
    if (active && j < L) {
        // codes relative to the sequence's first event, or to its history's
        // first event when the rows are candidates scored against a cache
        int64_t t_first = a.ts[row0];
        if (a.ref_offsets && a.ref_offsets[b + 1] > a.ref_offsets[b]) t_first = a.ref_ts[a.ref_offsets[b]];
        const int64_t d = a.ts[row0 + j] - t_first;
        narrow = d > -(int64_t(1) << 30) && d < (int64_t(1) << 30);
        const uint32_t e = uint32_t(int32_t(d) * 2) + 0x80000000u;
        a.enc[row0 + j] = e;
        mn = e;
        mx = e;
    }
    int nar = narrow ? 1 : 0;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, m, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, m, 64));
        nar &= __shfl_xor(nar, m, 64);
    }
    if (active && (lane & 31) == 0) {
        a.stats[2 * g] = nar ? mn : 0xffffffffu;
        a.stats[2 * g + 1] = nar ? mx : 0u;
    }
}

// One launch prepares everything the attention core reads besides the
// inputs: workgroup 0 builds the work list while the others (bf16 core
// only) encode the timestamps.
__global__ void __launch_bounds__(kThreads) prep_kernel(SchedArgs a) {
    __shared__ SchedSmem s;
    if (blockIdx.x == 0) {
        if (!a.skip_list) build_work_list(a, s);
    } else {
        encode_timestamps(a, 1);
    }
}

// Where each sequence's 32x32 blocks of dLoss/dS start in the gradients' G
// buffer: the exclusive prefix over sequences of T(ceil(L / 32)), T(n) =
// n (n + 1) / 2, the blocks on and below the diagonal of an L x L causal
// mask cut into 32-row and 32-column blocks.
__device__ void g_block_prefix(const SchedArgs& a, int64_t* gbase) {
    __shared__ int64_t sums[kThreads];
    const int tid = threadIdx.x;
    const int per = (a.B + kThreads - 1) / kThreads;
    const int b0 = min(a.B, tid * per), b1 = min(a.B, b0 + per);
    auto blocks_of = [&](int b) {
        const int L = a.lengths ? a.lengths[b] : a.offsets[b + 1] - a.offsets[b];
        const int64_t n = (max(L, 0) + 31) / 32;
        return n * (n + 1) / 2;
    };
    int64_t mine = 0;
    for (int b = b0; b < b1; ++b) mine += blocks_of(b);
    sums[tid] = mine;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
        const int64_t x = tid >= d ? sums[tid - d] : 0;
        __syncthreads();
        sums[tid] += x;
        __syncthreads();
    }
    int64_t run = sums[tid] - mine;
    for (int b = b0; b < b1; ++b) {
        gbase[b] = run;
        run += blocks_of(b);
    }
}

// The gradients' preparation in one launch: workgroups 0 and 1 build the two
// work lists, workgroup 2 the G-block prefix, the others encode the
// timestamps of the first list's rows.
__global__ void __launch_bounds__(kThreads) prep_pair_kernel(SchedArgs a, SchedArgs b, int64_t* gbase) {
    __shared__ SchedSmem s;
    if (blockIdx.x == 0) {
        build_work_list(a, s);
    } else if (blockIdx.x == 1) {
        build_work_list(b, s);
    } else if (blockIdx.x == 2) {
        g_block_prefix(a, gbase);
    } else {
        encode_timestamps(a, 3);
    }
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

SchedLayout sched_layout(int B, int H, int max_seq_len, int tile_m, int split_d, int64_t num_rows,
                         size_t base, int max_part_slots) {
    SchedLayout l;
    l.cap = size_t(B) * size_t((max_seq_len + tile_m - 1) / tile_m);
    l.nblk = (max_seq_len + kTsBlock - 1) / kTsBlock;
    l.cap_blk = size_t(B) * size_t(l.nblk);
    // partial slots: at most max_part_slots (<= kMaxPartialSlots), and no
    // more than 8 per row block and head
    l.part_slots = split_d > 0 && H > 0
                       ? (int)std::min<size_t>(size_t(std::max(0, std::min(max_part_slots, kMaxPartialSlots))),
                                               l.cap * size_t(H) * 8)
                       : 0;
    l.cap_pieces = l.cap + (H > 0 ? size_t(l.part_slots) / size_t(H) : 0);
    l.off_ctrl = align256(base);
    l.off_qscan = align256(l.off_ctrl + kCtrlInts * sizeof(int32_t));
    l.off_items = align256(l.off_qscan + (size_t(B) + 1) * sizeof(int32_t));
    l.off_item_seq = align256(l.off_items + l.cap_pieces * sizeof(WorkItem));
    l.off_split = align256(l.off_item_seq + l.cap_pieces * sizeof(ItemSeq));
    l.off_part = align256(l.off_split + l.cap * sizeof(SplitBlock));
    l.off_stats = align256(l.off_part + size_t(l.part_slots) * size_t(tile_m) * size_t(split_d) * sizeof(float));
    l.off_enc = align256(l.off_stats + l.cap_blk * 2 * sizeof(uint32_t));
    l.off_rowmap = align256(l.off_enc + size_t(num_rows) * sizeof(uint32_t));
    l.bytes = align256(l.off_rowmap + (split_d > 0 ? size_t(num_rows) * sizeof(int32_t) : 0));
    return l;
}

hipError_t launch_sched_pair(const SchedArgs& a, const SchedArgs& b, int64_t* gbase, hipStream_t stream) {
    if (a.skip_list || b.skip_list || b.enc || !gbase) return hipErrorInvalidValue;
    if (!pow2(a.tile_m) || !pow2(a.tile_n) || !pow2(b.tile_m) || !pow2(b.tile_n)) return hipErrorInvalidValue;
    const int64_t ts_groups = a.enc ? (a.cap_blk + kTsPerGroup - 1) / kTsPerGroup : 0;
    hipLaunchKernelGGL(prep_pair_kernel, dim3((unsigned)(3 + ts_groups)), dim3(kThreads), 0, stream, a, b, gbase);
    return hipGetLastError();
}

namespace {

__device__ int64_t g_validate_first;   // first failure of the last validate_batch on this GPU

__global__ void __launch_bounds__(256) validate_batch_kernel(ValidateArgs a) {
    __shared__ unsigned long long first;
    if (threadIdx.x == 0) first = ~0ull;
    __syncthreads();
    for (int b = threadIdx.x; b < a.B; b += 256) {
        const int64_t o0 = a.offsets[b], o1 = a.offsets[b + 1];
        int check = 0;
        int64_t L = o1 - o0;
        if (b == 0 && o0 < 0) check = 1;
        else if (o1 < o0) check = 2;
        else if (b == a.B - 1 && o1 > a.num_rows) check = 3;
        else if (a.packed && ((b == 0 && o0 != 0) || (b == a.B - 1 && o1 != a.num_rows))) check = 7;
        else {
            if (a.lengths) {
                const int64_t l = a.lengths[b];
                if (l < 0 || l > L) check = 4;
                L = l;
            }
            if (check == 0 && L > a.max_seq_len) check = 5;
            if (check == 0 && a.ncand) {
                const int64_t c = a.ncand[b];
                if (c < 0 || c > L) check = 6;
            }
        }
        if (check) atomicMin(&first, (unsigned long long)(8 * (int64_t)b + check));
    }
    __syncthreads();
    if (threadIdx.x == 0) g_validate_first = first == ~0ull ? -1 : (int64_t)first;
}

}  // namespace

hipError_t validate_batch(const ValidateArgs& a, hipStream_t stream, int64_t* first) {
    *first = -1;
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(validate_batch_kernel, dim3(1), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess)
        e = hipMemcpyFromSymbolAsync(first, HIP_SYMBOL(g_validate_first), sizeof(int64_t), 0,
                                     hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return e;
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream) {
    if (!pow2(a.tile_m) || !pow2(a.tile_n)) return hipErrorInvalidValue;
    const int64_t ts_groups = a.enc ? (a.cap_blk + kTsPerGroup - 1) / kTsPerGroup : 0;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(1 + ts_groups)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

namespace {

__device__ __forceinline__ void combine_one(const CombineArgs& a, int64_t t, int per_row, int64_t per_block) {
    const int64_t sb_i = t / per_block;
    const int64_t rem = t - sb_i * per_block;
    const int h = (int)(rem / (a.BM * per_row));
    const int lr = (int)(rem / per_row) % a.BM;
    const int c8 = (int)(rem % per_row) * 8;
    const SplitBlock sb = a.split[sb_i];
    const int64_t row0 = a.offsets[sb.b];
    const int L = a.lengths ? a.lengths[sb.b] : a.offsets[sb.b + 1] - (int)row0;
    const int r = sb.qt * a.BM + lr;
    if (r >= L) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < sb.n; ++k) {
        const float* src = a.partial + ((int64_t)(sb.slot + k) * a.H + h) * a.BM * a.d + (int64_t)lr * a.d + c8;
        const float4 x0 = *reinterpret_cast<const float4*>(src);
        const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
        acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
        acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
    }
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    uint16_t* dst = static_cast<uint16_t*>(a.o) + (row0 + r) * a.o_stride + h * a.d + c8;
    *reinterpret_cast<u32x4*>(dst) = pk;
}

// Grid-stride over (split block, head, row, 8 columns): the sum of the
// block's partial slots, rounded to bf16 into O (rows past L are skipped).
// With no split block every thread exits at once.
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    const int per_row = a.d / 8;
    const int64_t per_block = (int64_t)a.H * a.BM * per_row;
    const int64_t nsb = min((int64_t)a.ctrl[2], a.max_blocks);
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < nsb * per_block; t += (int64_t)gridDim.x * 256)
        combine_one(a, t, per_row, per_block);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    if (a.max_blocks <= 0) return hipSuccess;
    const int64_t threads = a.max_blocks * a.H * a.BM * (a.d / 8);
    const int64_t blocks = std::min<int64_t>((threads + 255) / 256, (int64_t)device_cu_count());
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hstu
