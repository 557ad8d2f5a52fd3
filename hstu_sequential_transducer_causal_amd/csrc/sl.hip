// sl.hip -- stochastic length on the device: seeded, order-preserving
// subsampling of long sequences fused with the jagged gather of their rows.
//
// Stochastic length ("行动胜于言语：万亿参数序列转导器用于生成式推荐", section
// "2.1"; the GRs summary page, section 2.1): in training a history longer than
// a cap is replaced by a random subsequence that keeps the events' order, so
// attention costs O(N^alpha d) instead of O(N^2 d).  The sampler (the pages do
// not fix one): event j of sequence b gets the top 32 bits of the first word
// of Philox-4x64-10 (Salmon et al., SC'11) for counter (j, b, step, 0) and key
// (seed, 0x534c); the sequence keeps its min(cap_b, L_b) events with the
// smallest (key, j), in their original order -- every subset of that size is
// equally likely, and the choice is a pure function of (seed, step, b, j).
//
//   sl_offsets_kernel  one workgroup: packed offsets of the kept rows.
//   sl_select_kernel   one workgroup per sequence: a 4-pass radix select
//                      (8 bits per pass, LDS histogram) finds the cap-th
//                      smallest key; a block scan then writes the kept source
//                      rows in order (ties on the threshold key by index).
//                      The keys of a sequence of up to kKeyCache events are
//                      computed once and kept in LDS; longer ones recompute
//                      them in every pass.
//   sl_gather_kernel   copies the kept rows of up to 8 row-major tensors.
#include <algorithm>

#include "internal.h"
#include "hstu_device.h"

namespace hstu {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kSelThreads = 1024;            // the select kernel's workgroup
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kKeyCache = 16384;             // keys kept in LDS (64 KiB)

constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kM1 = 0xCA5A826395121157ull;
constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kW1 = 0xBB67AE8584CAA73Bull;
constexpr uint64_t kDomain = 0x534Cull;

// Sort key of event j of sequence b: Philox-4x64-10, first word, top 32 bits.
__device__ __forceinline__ uint32_t event_key(int j, int b, uint64_t step, uint64_t seed) {
    uint64_t x0 = (uint64_t)j, x1 = (uint64_t)b, x2 = step, x3 = 0;
    uint64_t k0 = seed, k1 = kDomain;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kW0;
            k1 += kW1;
        }
        const uint64_t hi0 = __umul64hi(kM0, x0), lo0 = kM0 * x0;
        const uint64_t hi1 = __umul64hi(kM1, x2), lo1 = kM1 * x2;
        const uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
        x0 = y0;
        x1 = lo1;
        x2 = y2;
        x3 = lo0;
    }
    return (uint32_t)(x0 >> 32);
}

// Exclusive scan of one int per thread over a workgroup of NW waves, with
// the total.
template <int NW>
__device__ int block_scan(int v, int* wave_tot, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int s = wave_tot[i];
        before += i < w ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

__device__ __forceinline__ int cap_of(const SlArgs& a, int b) { return a.caps ? a.caps[b] : a.cap; }

__global__ void __launch_bounds__(kThreads) sl_offsets_kernel(SlArgs a) {
    __shared__ int wave_tot[kWaves];
    __shared__ int carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < a.B; base += kThreads) {
        const int b = base + threadIdx.x;
        int k = 0;
        if (b < a.B) k = max(0, min(cap_of(a, b), a.offsets[b + 1] - a.offsets[b]));
        int total;
        const int ex = block_scan<kWaves>(k, wave_tot, total);
        const int c = carry;
        if (b < a.B) a.out_offsets[b] = c + ex;
        __syncthreads();
        if (threadIdx.x == 0) carry = c + total;
        __syncthreads();
    }
    if (threadIdx.x == 0) a.out_offsets[a.B] = carry;
}

__global__ void __launch_bounds__(kSelThreads) sl_select_kernel(SlArgs a) {
    __shared__ int hist[256];
    __shared__ int wave_tot[kSelWaves];
    __shared__ uint32_t s_prefix, s_mask;
    __shared__ int s_remaining, s_lt, s_eq;
    __shared__ uint32_t keys[kKeyCache];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t off = a.offsets[b];
    const int L = a.offsets[b + 1] - (int)off;
    const int k = max(0, min(cap_of(a, b), L));
    const int64_t out0 = a.out_offsets[b];
    if (k >= L) {
        for (int j = tid; j < L; j += kSelThreads) a.out_index[out0 + j] = off + j;
        return;
    }
    if (k == 0) return;

    const bool cached = L <= kKeyCache;
    if (cached)   // (visible after the first pass's first barrier)
        for (int j = tid; j < L; j += kSelThreads) keys[j] = event_key(j, b, a.step, a.seed);
    auto key_at = [&](int j) { return cached ? keys[j] : event_key(j, b, a.step, a.seed); };

    // the k-th smallest key, 8 bits at a time from the top
    if (tid == 0) {
        s_prefix = 0;
        s_mask = 0;
        s_remaining = k;
    }
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        const uint32_t prefix = s_prefix, mask = s_mask;
        for (int j = tid; j < L; j += kSelThreads) {
            const uint32_t u = key_at(j);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
        }
        __syncthreads();
        // the digit d: the first bin whose count, added to the bins below it,
        // reaches the rank still to find (255 if none does).  One wave: lane l
        // holds bins 4l .. 4l + 3 and their inclusive running total.
        if (tid < 64) {
            const int rem = s_remaining;
            int c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = hist[4 * tid + i];
            const int sum = (c[0] + c[1]) + (c[2] + c[3]);
            int x = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (tid >= o) x += y;
            }
            const unsigned long long reach = __ballot(x >= rem);
            const int owner = reach ? __ffsll((long long)reach) - 1 : 63;
            if (tid == owner) {
                int cum = x - sum, i = 0;
                for (; i < 3; ++i) {
                    if (cum + c[i] >= rem) break;
                    cum += c[i];
                }
                const uint32_t d = (uint32_t)(4 * tid + i);
                s_remaining = rem - cum;
                s_prefix = prefix | (d << shift);
                s_mask = mask | (255u << shift);
            }
        }
        __syncthreads();
    }
    const uint32_t thr = s_prefix;
    const int need_eq = s_remaining;   // events with key == thr to keep (lowest j first)

    // kept events in order: key < thr, or key == thr among the first need_eq
    if (tid == 0) {
        s_lt = 0;   // kept so far
        s_eq = 0;   // key == thr seen so far
    }
    __syncthreads();
    for (int base = 0; base < L; base += kSelThreads) {
        const int j = base + tid;
        uint32_t u = 0xffffffffu;
        bool valid = j < L;
        if (valid) u = key_at(j);
        const bool eq = valid && u == thr;
        int eq_total;
        const int eq_rank = block_scan<kSelWaves>(eq ? 1 : 0, wave_tot, eq_total);
        const int eq_before = s_eq;
        const bool keep = valid && (u < thr || (eq && eq_before + eq_rank < need_eq));
        int kept_total;
        const int pos = block_scan<kSelWaves>(keep ? 1 : 0, wave_tot, kept_total);
        const int kept_before = s_lt;
        if (keep) a.out_index[out0 + kept_before + pos] = off + j;
        __syncthreads();
        if (tid == 0) {
            s_eq = eq_before + eq_total;
            s_lt = kept_before + kept_total;
        }
        __syncthreads();
    }
}

// Rows of tensor blockIdx.y at the kept source rows: 16-byte chunks when the
// rows allow them, else 4-byte words.
__global__ void __launch_bounds__(kThreads) sl_gather_kernel(SlArgs a) {
    const int t = blockIdx.y;
    const int64_t total = a.out_offsets[a.B];
    const char* src = static_cast<const char*>(a.src[t]);
    char* dst = static_cast<char*>(a.dst[t]);
    const int64_t ss = a.src_stride[t], ds = a.dst_stride[t];
    const int rb = a.row_bytes[t];
    const bool wide = (rb % 16 == 0) && (ss % 16 == 0) && (ds % 16 == 0) &&
                      ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 == 0);
    const int unit = wide ? 16 : 4;
    const int per_row = rb / unit;
    const int64_t n = total * per_row;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads) {
        const int64_t r = e / per_row;
        const int c = (int)(e - r * per_row);
        const int64_t sr = a.out_index[r];
        if (wide)
            *reinterpret_cast<u32x4*>(dst + r * ds + c * 16) = *reinterpret_cast<const u32x4*>(src + sr * ss + c * 16);
        else
            *reinterpret_cast<uint32_t*>(dst + r * ds + c * 4) = *reinterpret_cast<const uint32_t*>(src + sr * ss + c * 4);
    }
}

}  // namespace

hipError_t launch_stochastic_length(const SlArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(sl_offsets_kernel, dim3(1), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sl_select_kernel, dim3((unsigned)a.B), dim3(kSelThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.num_tensors <= 0 || a.num_rows <= 0) return e;
    const int64_t blocks = std::min<int64_t>(4 * (int64_t)device_cu_count(), (a.num_rows + 3) / 4 + 1);
    hipLaunchKernelGGL(sl_gather_kernel, dim3((unsigned)blocks, (unsigned)a.num_tensors), dim3(kThreads), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace hstu
