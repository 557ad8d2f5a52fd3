// attn_f32.hip -- fp32 attention core (d_qk = d_v in {32, 64}) for the
// small fp32 workload.  Same definition as the bf16 core:
//   O_i = alpha * sum_{j visible} SiLU(<Q_i, K_j> + rab_pos[pb] + rab_time[tb]) V_j
// ("生成式推荐（一）：HSTU", section "Pointwise aggregated attention").
//
// One wave per work item (64 query rows of one head); each lane owns one
// query row with Q and the accumulator in registers; key tiles of 64 rows are
// staged in LDS and read as broadcasts.  fp32 throughout, accurate expf.
#include <hip/hip_ext.h>

#include "internal.h"
#include "hstu_device.h"

namespace hstu {

namespace {

constexpr int BM = kF32TileM;
constexpr int BN = kF32TileN;

struct Params {
    int H;
    const int32_t* offsets;
    const int32_t* lengths;
    const int32_t* ncand;
    const float* q; int64_t qs;
    const float* k; int64_t ks;
    const float* v; int64_t vs;
    const int64_t* ts;
    const float* rab_pos; int P; int rp_hs;
    const float* rab_time; int NT; int rt_hs;
    float alpha;
    int act;
    float* o; int64_t os;
    const WorkItem* items;
    const int32_t* ctrl;
    int32_t* cursor;
};

template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(Params p) {
    __shared__ float ks[BN][D];
    __shared__ float vs[BN][D];
    __shared__ int64_t tss[BN];
    __shared__ int32_t wsh;
    const int lane = threadIdx.x;
    const int total_work = p.ctrl[0] * p.H;

    for (;;) {
        if (lane == 0) wsh = atomicAdd(p.cursor, 1);
        __syncthreads();
        const int w = wsh;
        __syncthreads();
        if (w >= total_work) break;
        const WorkItem it = p.items[w / p.H];
        const int h = w % p.H;
        const int64_t row0 = p.offsets[it.b];
        const int L = p.lengths ? p.lengths[it.b] : p.offsets[it.b + 1] - (int)row0;
        const int n = p.ncand ? L - p.ncand[it.b] : L;
        const int kb_begin = it.kb & 0xffff, kb_end = it.kb >> 16;
        const float* rp = p.rab_pos + (int64_t)h * p.rp_hs;
        const float* rt = p.rab_time + (int64_t)h * p.rt_hs;

        const int i = it.qt * BM + lane;
        const bool valid = i < L;
        float qr[D], acc[D];
#pragma unroll
        for (int c = 0; c < D; ++c) {
            qr[c] = valid ? p.q[(row0 + i) * p.qs + h * D + c] : 0.0f;
            acc[c] = 0.0f;
        }
        const int64_t ti = valid ? p.ts[row0 + i] : 0;
        const int pi = min(i, n);

        const int p0 = it.pr & 0xffff, p1 = it.pr >> 16;   // (never split: the whole list)
        const int ntiles = p1 - p0;
        for (int t = 0; t < ntiles; ++t) {
            const int pos = p0 + t;
            const int kt = pos < it.a_end ? pos : kb_begin + (pos - it.a_end);
            const int j0 = kt * BN;
            {
                const int j = j0 + lane;
                const bool jv = j < L;
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    ks[lane][c] = jv ? p.k[(row0 + j) * p.ks + h * D + c] : 0.0f;
                    vs[lane][c] = jv ? p.v[(row0 + j) * p.vs + h * D + c] : 0.0f;
                }
                tss[lane] = jv ? p.ts[row0 + j] : 0;
            }
            __syncthreads();
            for (int jj = 0; jj < BN; ++jj) {
                const int j = j0 + jj;
                const bool vis = valid && (j < L) && (i < n ? (j <= i) : (j < n || j == i));
                float s = 0.0f;
#pragma unroll
                for (int c = 0; c < D; ++c) s = fmaf(qr[c], ks[jj][c], s);
                const int pj = min(j, n);
                const int pb = min(max(pi - pj, 0), p.P - 1);
                const int64_t dt = ti - tss[jj];
                const uint64_t ad = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
                const int tb = min(p.NT - 1, bit_length_u64(ad));
                s += vis ? rp[pb] : 0.0f;
                s += vis ? rt[tb] : 0.0f;
                float a = (p.act == 0) ? silu_precise(s) : s;
                a = vis ? a : 0.0f;
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] = fmaf(a, vs[jj][c], acc[c]);
            }
            __syncthreads();
        }
        if (valid) {
#pragma unroll
            for (int c = 0; c < D; ++c) p.o[(row0 + i) * p.os + h * D + c] = p.alpha * acc[c];
        }
    }
}

}  // namespace

hipError_t launch_attn_f32(const AttnCoreArgs& a, hipStream_t stream) {
    Params p;
    p.H = a.H;
    p.offsets = a.offsets; p.lengths = a.lengths; p.ncand = a.ncand;
    p.q = static_cast<const float*>(a.q); p.qs = a.q_stride;
    p.k = static_cast<const float*>(a.k); p.ks = a.k_stride;
    p.v = static_cast<const float*>(a.v); p.vs = a.v_stride;
    p.ts = a.ts;
    p.rab_pos = a.rab_pos; p.P = a.P; p.rp_hs = a.rp_head_stride;
    p.rab_time = a.rab_time; p.NT = a.NT; p.rt_hs = a.rt_head_stride;
    p.alpha = a.alpha; p.act = a.act;
    p.o = static_cast<float*>(a.o); p.os = a.o_stride;
    p.items = a.items; p.ctrl = a.ctrl; p.cursor = a.cursor;
    const int grid = device_cu_count() * 4;
    if (a.d == 32) {
        hipExtLaunchKernelGGL(attn_f32_kernel<32>, dim3(grid), dim3(64), 0, stream,
                              a.ev_begin, a.ev_end, 0, p);
    } else {
        hipExtLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, stream,
                              a.ev_begin, a.ev_end, 0, p);
    }
    return hipGetLastError();
}

}  // namespace hstu
