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
// Design (one workgroup = 4 waves = one work item of 128 query rows x 1 head):
//   * Each wave owns 32 query rows.  It computes S^T = K Q^T with
//     v_mfma_f32_16x16x32_bf16 so that, in the accumulator, lane l holds
//     query row (l % 16) against 4 consecutive keys: after the bias, SiLU,
//     mask and bf16 packing these registers are directly the A operand of
//     the second product O += A V.  Q stays in registers for the whole item.
//   * K tiles (64 keys x 128) are staged row-major in LDS with a 16-byte XOR
//     swizzle; V tiles are transposed while staging (d-major) so that the B
//     operand of A V is two 8-byte LDS reads.  The next tile's global loads
//     are issued before the current tile's math (register prefetch).
//   * The relative bias enters as the MFMA's initial accumulator:
//       position: a per-item LDS table E[u] = rab_pos[clamp(u - 64, 0, P-1)];
//         a lane's 16 bias entries of a 16x16 block sit at fixed offsets
//         from one clamped base index, so no per-element index math;
//       time: timestamps are re-encoded per tile as e = 2 (t - t_first) + 2^31
//         (exact when all |t - t_first| < 2^30, checked per tile), so
//         |e_i - e_j| + 1 = 2|dt| + 1 is one v_sad_u32 and its leading-zero
//         count c = 31 - bit_length(|dt|) indexes a 32-entry LDS table;
//         tiles outside that range use 64-bit arithmetic.
//   * Tiles whose pairs are all visible skip the mask; the others select
//     (never multiply) so that padding and masked garbage cannot leak.
//   * Persistent grid: workgroups pull items (longest first) from the
//     scheduler's list through an atomic cursor until it is exhausted.
#include "internal.h"
#include "hstu_device.h"

namespace hstu {

namespace {

constexpr int BM = kBf16TileM;   // 128 query rows per item
constexpr int BN = kBf16TileN;   // 64 keys per tile
constexpr int HD = 128;          // head dim
constexpr int kThreads = 256;
constexpr int kPosMargin = 64;   // table entries below diff 0
constexpr int kPosExtra = 64;    // table entries beyond P-1 (clamped values)

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
    int act;
    uint16_t* o; int64_t os;
    const WorkItem* items;
    const int32_t* ctrl;
    int32_t* cursor;
};

struct Smem {
    uint8_t k[BN * HD * 2];         // [64 keys][128 d] bf16, 16-B chunks swizzled by key & 15
    uint8_t vt[HD * BN * 2];        // [128 d][64 keys] bf16, 8-B chunks swizzled by d & 14
    uint32_t tsenc[BN];             // 2 (t - t_first) + 2^31
    int64_t ts64[BN];
    float tt_fast[32];              // by leading-zero count of 2|dt|+1
    float tt_wide[65];              // by bit length of |dt|
    int32_t item[4];
    int32_t head;
    int32_t flags;
};


__device__ __forceinline__ bool narrow_delta(int64_t d) {
    return d > -(int64_t(1) << 30) && d < (int64_t(1) << 30);
}

__device__ __forceinline__ uint32_t encode_ts(int64_t d) {
    return uint32_t(int32_t(d) * 2) + 0x80000000u;
}

// Global -> register part of staging one key tile.
struct Prefetch {
    u32x4 kr[4];
    u32x4 vr[4];
    int64_t t;
};

__device__ __forceinline__ void prefetch_tile(const Params& p, Prefetch& pf, int64_t row0, int L, int h,
                                              int j0) {
    const int tid = threadIdx.x;
    const int chunk = tid & 15;
    const int rsub = tid >> 4;   // 0..15
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        int j = j0 + r4 * 16 + rsub;
        u32x4 z = {0u, 0u, 0u, 0u};
        pf.kr[r4] = z;
        if (j < L)
            pf.kr[r4] = *reinterpret_cast<const u32x4*>(p.k + (row0 + j) * p.ks + h * HD + chunk * 8);
    }
    // V: this thread owns keys j0 + 4*rsub + 0..3 at d = 8*chunk .. 8*chunk+7
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int j = j0 + 4 * rsub + r;
        u32x4 z = {0u, 0u, 0u, 0u};
        pf.vr[r] = z;
        if (j < L)
            pf.vr[r] = *reinterpret_cast<const u32x4*>(p.v + (row0 + j) * p.vs + h * HD + chunk * 8);
    }
    pf.t = 0;
    if (tid < BN && j0 + tid < L) pf.t = p.ts[row0 + j0 + tid];
}

// Register -> LDS part of staging; returns this thread's "tile is wide" vote.
__device__ __forceinline__ bool store_tile(Smem& s, const Prefetch& pf, int L, int j0, int64_t t_first) {
    const int tid = threadIdx.x;
    const int chunk = tid & 15;
    const int rsub = tid >> 4;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        int row = r4 * 16 + rsub;
        *reinterpret_cast<u32x4*>(s.k + row * (HD * 2) + ((chunk ^ (row & 15)) << 4)) = pf.kr[r4];
    }
    // transpose 4 keys x 8 d into 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const int sh = (e & 1) * 16;
        uint32_t x0 = (pf.vr[0][w] >> sh) & 0xffffu;
        uint32_t x1 = (pf.vr[1][w] >> sh) & 0xffffu;
        uint32_t x2 = (pf.vr[2][w] >> sh) & 0xffffu;
        uint32_t x3 = (pf.vr[3][w] >> sh) & 0xffffu;
        u32x2 val = {x0 | (x1 << 16), x2 | (x3 << 16)};
        int d = chunk * 8 + e;
        *reinterpret_cast<u32x2*>(s.vt + d * (BN * 2) + ((rsub ^ (d & 14)) << 3)) = val;
    }
    bool wide = false;
    if (tid < BN) {
        int64_t t = (j0 + tid < L) ? pf.t : t_first;
        int64_t dlt = t - t_first;
        wide = !narrow_delta(dlt);
        s.tsenc[tid] = encode_ts(dlt);
        s.ts64[tid] = t;
    }
    return wide;
}

__global__ void __launch_bounds__(kThreads, 2) attn_bf16_kernel(Params p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    Smem& s = *reinterpret_cast<Smem*>(smem_raw);
    float* epos = reinterpret_cast<float*>(smem_raw + sizeof(Smem));   // [P + 128]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c16 = lane & 15;
    const int g = lane >> 4;
    const int total_work = p.ctrl[0] * p.H;
    const bool shared_tables = (p.rp_hs == 0) && (p.rt_hs == 0);
    int loaded_head = -1;

    for (;;) {
        if (tid == 0) {
            int w = atomicAdd(p.cursor, 1);
            s.head = w;
            if (w < total_work) {
                WorkItem it = p.items[w / p.H];
                s.item[0] = it.b; s.item[1] = it.qt; s.item[2] = it.a_end; s.item[3] = it.kb;
            }
        }
        __syncthreads();
        const int w = s.head;
        if (w >= total_work) break;
        const int b = s.item[0], qt = s.item[1], a_end = s.item[2];
        const int kb_begin = s.item[3] & 0xffff, kb_end = s.item[3] >> 16;
        const int h = w % p.H;

        const int64_t row0 = p.offsets[b];
        const int L = p.lengths ? p.lengths[b] : p.offsets[b + 1] - (int)row0;
        const int n = p.ncand ? L - p.ncand[b] : L;
        const int64_t t_first = p.ts[row0];

        // ---- relative-bias tables (per head only when tables differ by head)
        if (loaded_head < 0 || (!shared_tables && loaded_head != h)) {
            const float* rp = p.rab_pos + (int64_t)h * p.rp_hs;
            const float* rt = p.rab_time + (int64_t)h * p.rt_hs;
            const int ne = p.P + kPosMargin + kPosExtra;
            for (int u = tid; u < ne; u += kThreads) {
                int dd = min(max(u - kPosMargin, 0), p.P - 1);
                epos[u] = rp[dd];
            }
            if (tid < 32) s.tt_fast[tid] = rt[min(p.NT - 1, 31 - tid)];
            if (tid < 65) s.tt_wide[tid] = rt[min(p.NT - 1, tid)];
            loaded_head = h;
        }

        // ---- this wave's query rows: Q fragments, timestamps, positions
        const int wrow0 = qt * BM + wave * 32;
        bf16x8 qf[2][4];
        uint32_t tsi[2];
        int64_t ts64i[2];
        int prow[2];
        bool narrow_q = true;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int i = wrow0 + qb * 16 + c16;
            const bool valid = i < L;
            const uint16_t* qp = p.q + (row0 + i) * p.qs + h * HD + g * 8;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 z = {0u, 0u, 0u, 0u};
                if (valid) z = *reinterpret_cast<const u32x4*>(qp + c * 32);
                qf[qb][c] = __builtin_bit_cast(bf16x8, z);
            }
            int64_t t = valid ? p.ts[row0 + i] : t_first;
            narrow_q = narrow_q && narrow_delta(t - t_first);
            tsi[qb] = encode_ts(t - t_first);
            ts64i[qb] = t;
            prow[qb] = min(i, n);
        }

        f32x4 oacc[2][8];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) oacc[qb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int ntiles = a_end + (kb_end - kb_begin);
        Prefetch pf;
        if (ntiles > 0) prefetch_tile(p, pf, row0, L, h, 0 < a_end ? 0 : kb_begin * BN);
        __syncthreads();  // tables visible; previous item's LDS reads done

        for (int it = 0; it < ntiles; ++it) {
            const int kt = it < a_end ? it : kb_begin + (it - a_end);
            const int j0 = kt * BN;
            const bool wide_vote = store_tile(s, pf, L, j0, t_first);
            const int wide = __syncthreads_or(wide_vote ? 1 : 0) || !narrow_q;
            if (it + 1 < ntiles) {
                const int kt1 = (it + 1) < a_end ? (it + 1) : kb_begin + (it + 1 - a_end);
                prefetch_tile(p, pf, row0, L, h, kt1 * BN);
            }

            // Pairs of this wave's rows in this tile: all visible?
            const bool full = (j0 + BN <= n) && (j0 + BN - 1 <= wrow0);

            // ---------------- S^T = K Q^T + bias
            f32x4 sacc[2][4];
            int pbase[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                int x = prow[qb] - (j0 + 4 * g);
                x = min(max(x, 0), p.P + 50);
                pbase[qb] = x + kPosMargin;
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int krow = kb * 16 + c16;
                bf16x8 kf[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kf[c] = *reinterpret_cast<const bf16x8*>(s.k + krow * (HD * 2) + (((4 * c + g) ^ c16) << 4));
                const u32x4 tj = *reinterpret_cast<const u32x4*>(&s.tsenc[kb * 16 + 4 * g]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    f32x4 init;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float tb;
                        if (!wide) {
                            uint32_t x = sad_u32(tsi[qb], tj[r], 1u);
                            tb = s.tt_fast[__builtin_clz(x)];
                        } else {
                            int64_t dt = ts64i[qb] - s.ts64[kb * 16 + 4 * g + r];
                            uint64_t ad = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
                            tb = s.tt_wide[bit_length_u64(ad)];
                        }
                        init[r] = epos[pbase[qb] - 16 * kb - r] + tb;
                    }
                    f32x4 acc = init;
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc = mfma16x16x32(kf[c], qf[qb][c], acc);
                    sacc[qb][kb] = acc;
                }
            }

            // ---------------- activation, mask, pack to bf16 (A operand)
            bf16x8 pa[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int i = wrow0 + qb * 16 + c16;
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    uint32_t wv[4];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int kb = 2 * c2 + hh;
                        float a4[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float sv = sacc[qb][kb][r];
                            float a = (p.act == 0) ? silu_fast(sv) : sv;
                            if (!full) {
                                const int j = j0 + kb * 16 + 4 * g + r;
                                const bool vis = (j < L) && (i < n ? (j <= i) : (j < n || j == i));
                                a = vis ? a : 0.0f;
                            }
                            a4[r] = a;
                        }
                        wv[hh * 2 + 0] = pack_bf16x2(a4[0], a4[1]);
                        wv[hh * 2 + 1] = pack_bf16x2(a4[2], a4[3]);
                    }
                    u32x4 packed = {wv[0], wv[1], wv[2], wv[3]};
                    pa[qb][c2] = __builtin_bit_cast(bf16x8, packed);
                }
            }

            // ---------------- O += A V
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    const int d = nb * 16 + c16;
                    const uint8_t* vrow = s.vt + d * (BN * 2);
                    u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (((c2 * 8 + g) ^ (d & 14)) << 3));
                    u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (((c2 * 8 + 4 + g) ^ (d & 14)) << 3));
                    u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
                    bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) oacc[qb][nb] = mfma16x16x32(pa[qb][c2], vf, oacc[qb][nb]);
                }
            }
            __syncthreads();  // all waves done with this tile's LDS before it is overwritten
        }

        // ---------------- O = alpha * acc, bf16, rows < L only
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = wrow0 + qb * 16 + 4 * g + r;
                if (i < L) {
                    uint16_t* op = p.o + (row0 + i) * p.os + h * HD + c16;
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) op[nb * 16] = f32_to_bf16_bits(p.alpha * oacc[qb][nb][r]);
                }
            }
        }
    }
}

}  // namespace

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
    p.alpha = a.alpha; p.act = a.act;
    p.o = static_cast<uint16_t*>(a.o); p.os = a.o_stride;
    p.items = a.items; p.ctrl = a.ctrl; p.cursor = a.cursor;
    const size_t smem = sizeof(Smem) + sizeof(float) * size_t(a.P + kPosMargin + kPosExtra);
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_bf16_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    const int grid = device_cu_count() * 2;
    hipLaunchKernelGGL(attn_bf16_kernel, dim3(grid), dim3(kThreads), smem, stream, p);
    return hipGetLastError();
}

}  // namespace hstu
