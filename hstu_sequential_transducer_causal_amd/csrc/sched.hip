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

// Sequence of flat query tile f: the last b with qscan[b] <= f.
__device__ __forceinline__ int find_seq(const int32_t* qscan, int B, int f) {
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
    __shared__ int carry_s;
    const int tid = threadIdx.x;
    const int BM = a.tile_m, BN = a.tile_n;

    for (int i = tid; i < kMaxBins; i += kThreads) hist[i] = 0;
    if (tid == 0) carry_s = 0;
    __syncthreads();

    // 1. query tiles and 32-row timestamp blocks per sequence -> exclusive
    //    prefixes qscan[0..B] and bscan[0..B]
    __shared__ int bcarry_s;
    if (tid == 0) bcarry_s = 0;
    for (int base = 0; base < a.B; base += kThreads) {
        int b = base + tid;
        int nq = 0, nblk = 0;
        if (b < a.B) {
            const int L = seq_length(a, b);
            nq = ceil_div(L, BM);
            nblk = ceil_div(L, kTsBlock);
        }
        int total, btotal;
        int ex = block_exclusive_scan(nq, wave_tot, total);
        int bex = block_exclusive_scan(nblk, wave_tot, btotal);
        int carry = carry_s, bcarry = bcarry_s;
        if (b < a.B) {
            a.qscan[b] = carry + ex;
            a.bscan[b] = bcarry + bex;
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
    }
    __syncthreads();

    // 2. histogram of item costs (key tiles per item)
    for (int f = tid; f < nitems; f += kThreads) {
        int b = find_seq(a.qscan, a.B, f);
        int L = seq_length(a, b);
        Ranges r = tile_ranges(L, seq_history(a, b, L), f - a.qscan[b], BM, BN);
        atomicAdd(&hist[r.a_end + (r.kb_end - r.kb_begin)], 1);
    }
    __syncthreads();

    // 3. start position of each cost bin, largest cost first
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < kMaxBins; base += kThreads) {
        int bin = kMaxBins - 1 - (base + tid);
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
        int b = find_seq(a.qscan, a.B, f);
        int L = seq_length(a, b);
        int qt = f - a.qscan[b];
        Ranges r = tile_ranges(L, seq_history(a, b, L), qt, BM, BN);
        int pos = atomicAdd(&hist[r.a_end + (r.kb_end - r.kb_begin)], 1);
        WorkItem it;
        it.b = b;
        it.qt = qt;
        it.a_end = r.a_end;
        it.kb = r.kb_begin | (r.kb_end << 16);
        a.items[pos] = it;
    }
    if (tid == 0) {
        a.ctrl[0] = nitems;
        a.ctrl[1] = 0;
    }
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// One wave per two 32-row blocks (lanes 0-31 and 32-63).
__global__ void __launch_bounds__(256) ts_prep_kernel(TsPrepArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t f = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
    const int nblk = a.bscan[a.B];
    const bool active = f < nblk && f < a.cap_blk;
    uint32_t mn = 0xffffffffu, mx = 0u;
    bool narrow = true;
    int64_t fi = 0;
    if (active) {
        fi = f;
        const int b = find_seq(a.bscan, a.B, (int)f);
        const int64_t row0 = a.offsets[b];
        const int L = a.lengths ? a.lengths[b] : a.offsets[b + 1] - (int)row0;
        const int j = ((int)f - a.bscan[b]) * kTsBlock + (lane & 31);
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
