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
//
// Items are written longest first (counting sort on the number of key
// tiles) so that the persistent attention kernel, which takes items in list
// order, balances its CUs like a longest-processing-time schedule.
//
// One workgroup of 1024 threads runs the whole build; it is a few
// microseconds of work next to the attention core.
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

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct Ranges {
    int a_end, kb_begin, kb_end;
};

__device__ __forceinline__ Ranges tile_ranges(int L, int n, int qt, int BM, int BN) {
    int q0 = qt * BM;
    int q1 = min(q0 + BM, L);
    Ranges r;
    if (q1 <= n) {
        r.a_end = ceil_div(q1, BN);
        r.kb_begin = r.kb_end = r.a_end;
    } else {
        r.a_end = ceil_div(n, BN);
        r.kb_begin = max(max(q0, n) / BN, r.a_end);
        r.kb_end = max(ceil_div(q1, BN), r.kb_begin);
    }
    return r;
}

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

__device__ __forceinline__ int seq_length(const SchedArgs& a, int b) {
    return a.lengths ? a.lengths[b] : a.offsets[b + 1] - a.offsets[b];
}

__device__ __forceinline__ int seq_history(const SchedArgs& a, int b, int L) {
    return a.ncand ? L - a.ncand[b] : L;
}

// First query tile of a sequence in the work list: 0, or with cand_only the
// tile holding the first candidate row.
__device__ __forceinline__ int first_tile(const SchedArgs& a, int n, int BM) { return a.cand_only ? n / BM : 0; }

// Query tiles of a sequence in the work list (with cand_only, none for a
// sequence without candidates).
__device__ __forceinline__ int tile_count(const SchedArgs& a, int L, int n, int BM) {
    if (a.cand_only && L <= n) return 0;
    return ceil_div(L, BM) - first_tile(a, n, BM);
}

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

__global__ void __launch_bounds__(kThreads) sched_kernel(SchedArgs a) {
    __shared__ int hist[kMaxBins];
    __shared__ int wave_tot[kWaves];
    __shared__ int carry_s, bcarry_s;
    __shared__ int qscan_s[kLdsSeq + 1];
    __shared__ int len_s[kLdsSeq];
    __shared__ int hist_s[kLdsSeq];   // history rows n_b
    const int tid = threadIdx.x;
    const int BM = a.tile_m, BN = a.tile_n;
    const bool in_lds = a.B <= kLdsSeq;
    // costs (key tiles of an item) lie in [0, ceil(max_seq_len / BN)]
    const int nbins = min(kMaxBins, ceil_div(a.max_seq_len, BN) + 2);

    for (int i = tid; i < nbins; i += kThreads) hist[i] = 0;
    if (tid == 0) {
        carry_s = 0;
        bcarry_s = 0;
    }
    __syncthreads();

    // 1. query tiles and 32-row timestamp blocks per sequence -> exclusive
    //    prefixes qscan[0..B] and bscan[0..B]
    for (int base = 0; base < a.B; base += kThreads) {
        int b = base + tid;
        int nq = 0, nblk = 0;
        if (b < a.B) {
            const int L = seq_length(a, b);
            const int n = seq_history(a, b, L);
            nq = tile_count(a, L, n, BM);
            nblk = ceil_div(L, kTsBlock);
            if (in_lds) {
                len_s[b] = L;
                hist_s[b] = n;
            }
        }
        int total, btotal;
        int ex = block_exclusive_scan(nq, wave_tot, total);
        int bex = block_exclusive_scan(nblk, wave_tot, btotal);
        int carry = carry_s, bcarry = bcarry_s;
        if (b < a.B) {
            a.qscan[b] = carry + ex;
            a.bscan[b] = bcarry + bex;
            if (in_lds) qscan_s[b] = carry + ex;
        }
        __syncthreads();
        if (tid == 0) {
            carry_s = carry + total;
            bcarry_s = bcarry + btotal;
        }
        __syncthreads();
    }
    const int nitems = carry_s;
    if (tid == 0) {
        a.qscan[a.B] = nitems;
        a.bscan[a.B] = bcarry_s;
        if (in_lds) qscan_s[a.B] = nitems;
    }
    __syncthreads();

    // the item of flat query tile f
    auto item_of = [&](int f, int& b, int& qt) -> Ranges {
        int L, n;
        if (in_lds) {
            b = find_seq(qscan_s, a.B, f);
            qt = f - qscan_s[b];
            L = len_s[b];
            n = hist_s[b];
        } else {
            b = find_seq(a.qscan, a.B, f);
            qt = f - a.qscan[b];
            L = seq_length(a, b);
            n = seq_history(a, b, L);
        }
        qt += first_tile(a, n, BM);
        return tile_ranges(L, n, qt, BM, BN);
    };

    // 2. histogram of item costs (key tiles per item)
    for (int f = tid; f < nitems; f += kThreads) {
        int b, qt;
        const Ranges r = item_of(f, b, qt);
        atomicAdd(&hist[min(r.a_end + (r.kb_end - r.kb_begin), nbins - 1)], 1);
    }
    __syncthreads();

    // 3. start position of each cost bin, largest cost first
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < nbins; base += kThreads) {
        int bin = nbins - 1 - (base + tid);
        int c = bin >= 0 ? hist[bin] : 0;
        int total;
        int ex = block_exclusive_scan(c, wave_tot, total);
        int carry = carry_s;
        if (bin >= 0) hist[bin] = carry + ex;
        __syncthreads();
        if (tid == 0) carry_s = carry + total;
        __syncthreads();
    }

    // 4. scatter the items into their bins
    for (int f = tid; f < nitems; f += kThreads) {
        int b, qt;
        const Ranges r = item_of(f, b, qt);
        int pos = atomicAdd(&hist[min(r.a_end + (r.kb_end - r.kb_begin), nbins - 1)], 1);
        WorkItem it;
        it.b = b;
        it.qt = qt;
        it.a_end = r.a_end;
        it.kb = r.kb_begin | (r.kb_end << 16);
        if (pos < a.cap) a.items[pos] = it;   // (lengths within max_seq_len always fit)
    }
    if (tid == 0) {
        a.ctrl[0] = (int)min((int64_t)nitems, a.cap);
        a.ctrl[1] = 0;
    }
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// One wave per two 32-row blocks (lanes 0-31 and 32-63).
__global__ void __launch_bounds__(256) ts_prep_kernel(TsPrepArgs a) {
    __shared__ int bscan_s[kLdsSeq + 1];
    const bool in_lds = a.B <= kLdsSeq;
    if (in_lds)
        for (int i = threadIdx.x; i <= a.B; i += 256) bscan_s[i] = a.bscan[i];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t f = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
    const int nblk = in_lds ? bscan_s[a.B] : a.bscan[a.B];
    const bool active = f < nblk && f < a.cap_blk;
    uint32_t mn = 0xffffffffu, mx = 0u;
    bool narrow = true;
    int64_t fi = 0;
    if (active) {
        fi = f;
        const int b = in_lds ? find_seq(bscan_s, a.B, (int)f) : find_seq(a.bscan, a.B, (int)f);
        const int64_t row0 = a.offsets[b];
        const int L = a.lengths ? a.lengths[b] : a.offsets[b + 1] - (int)row0;
        const int j = ((int)f - (in_lds ? bscan_s[b] : a.bscan[b])) * kTsBlock + (lane & 31);
        if (j < L) {
            const int64_t t_first = a.ts[row0];
            const int64_t d = a.ts[row0 + j] - t_first;
            narrow = d > -(int64_t(1) << 30) && d < (int64_t(1) << 30);
            const uint32_t e = uint32_t(int32_t(d) * 2) + 0x80000000u;
            a.enc[row0 + j] = e;
            mn = e;
            mx = e;
        }
    }
    int nar = narrow ? 1 : 0;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, m, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, m, 64));
        nar &= __shfl_xor(nar, m, 64);
    }
    if (active && (lane & 31) == 0) {
        a.stats[2 * fi] = nar ? mn : 0xffffffffu;
        a.stats[2 * fi + 1] = nar ? mx : 0u;
    }
}

}  // namespace

SchedLayout sched_layout(int B, int max_seq_len, int tile_m, int64_t num_rows, size_t base) {
    SchedLayout l;
    l.off_ctrl = align256(base);
    l.off_qscan = align256(l.off_ctrl + 64 * sizeof(int32_t));
    l.off_bscan = align256(l.off_qscan + (size_t(B) + 1) * sizeof(int32_t));
    l.off_items = align256(l.off_bscan + (size_t(B) + 1) * sizeof(int32_t));
    l.cap = size_t(B) * size_t((max_seq_len + tile_m - 1) / tile_m);
    l.cap_blk = size_t(B) * size_t((max_seq_len + kTsBlock - 1) / kTsBlock);
    l.off_stats = align256(l.off_items + l.cap * sizeof(WorkItem));
    l.off_enc = align256(l.off_stats + l.cap_blk * 2 * sizeof(uint32_t));
    l.bytes = align256(l.off_enc + size_t(num_rows) * sizeof(uint32_t));
    return l;
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_ts_prep(const TsPrepArgs& a, hipStream_t stream) {
    if (a.cap_blk <= 0) return hipSuccess;
    const int64_t blocks = (a.cap_blk + 7) / 8;
    hipLaunchKernelGGL(ts_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hstu
