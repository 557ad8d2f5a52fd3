// epilogue.hip -- pointwise transformation gate Y = LayerNorm(O) (.) U, and the
// M-FALCON candidate score <Y, w>.
//
// "生成式推荐（一）：HSTU", section "Pointwise aggregated attention": the
// aggregated attention enters the layer as Norm(A(X)V(X)) (.) U(X), with
// Norm = LayerNorm; "Meta HSTU: как действия пользователя стали основой
// большой рекомендательной модели", section "Что меняется внутри HSTU по
// сравнению с обычным Transformer": normalise, then gate elementwise by U.
// LayerNorm runs over all H*d_v values of a row (biased variance, eps added
// to the variance, no affine parameters).
//
// HBM-bound: 16-byte vector loads, the row held in registers for a two-pass
// (mean, then centred variance) reduction with wavefront shuffles.  The
// common case (bf16, packed, Y wanted, no scores) takes ln_gate_rows_kernel:
// several rows per wave, all their loads issued before any arithmetic.
// Everything else takes ln_gate_kernel (one wave per row), which for batches
// of up to 1024 sequences first copies the batch structure into LDS for its
// rows' sequence searches.  ln_gate_bwd_kernel is the gate's gradient.
//
// Rows of a row block that the bf16 attention core split over key ranges
// arrive as fp32 partial sums: their O is the sum of those, rounded to bf16
// as the core rounds O, and is written to O here before it is normalised.
#include <hip/hip_ext.h>

#include "internal.h"
#include "hstu_device.h"
#include "../../include/hstu.h"

namespace hstu {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

// Largest b in [0, B) with offsets[b] <= row (row must be < offsets[B]).
__device__ __forceinline__ int seq_of_row(const int32_t* off, int B, int64_t row) {
    int lo = 0, hi = B;  // off[lo] <= row < off[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (off[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

// Elements per lane per chunk: 8 (one 16-byte bf16 load or two fp32 loads).
// The bf16 rows are read and written once, so their accesses are
// non-temporal: they do not displace data the next launches read again (the
// attention core measured 2.5 % faster in a loop of forward steps).
template <bool BF16>
struct Vec8 {
    static __device__ __forceinline__ void load(const void* base, int64_t idx, float* x) {
        if constexpr (BF16) {
            u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = __uint_as_float(r[e] << 16);
                x[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
            }
        } else {
            const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
            f32x4 a = p[0], b = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
        }
    }
    static __device__ __forceinline__ void store(void* base, int64_t idx, const float* x) {
        if constexpr (BF16) {
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
            __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx));
        } else {
            f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
            p[0] = f32x4{x[0], x[1], x[2], x[3]};
            p[1] = f32x4{x[4], x[5], x[6], x[7]};
        }
    }
};

// Batches of up to this many sequences have their offsets copied into LDS by
// each workgroup of ln_gate_kernel (one coalesced read), so that the rows'
// sequence searches do not wait on memory at every step.
constexpr int kOffLds = 1024;

template <bool BF16, int NCH>
__global__ void __launch_bounds__(kThreads) ln_gate_kernel(LnGateArgs a) {
    __shared__ int32_t s_off[kOffLds + 1], s_len[kOffLds], s_nc[kOffLds];
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    const bool need_seq = a.lengths || a.ncand || a.cross;
    const bool off_lds = need_seq && a.B > 0 && a.B <= kOffLds;   // (uniform)
    if (off_lds) {
        for (int i = threadIdx.x; i <= a.B; i += kThreads) {
            s_off[i] = a.offsets[i];
            if (i < a.B) {
                if (a.lengths) s_len[i] = a.lengths[i];
                if (a.ncand) s_nc[i] = a.ncand[i];
            }
        }
        __syncthreads();
    }
    const int32_t* off = off_lds ? s_off : a.offsets;
    const int32_t* lens = off_lds ? s_len : a.lengths;
    const int32_t* ncs = off_lds ? s_nc : a.ncand;
    if (a.B <= 0 || row >= a.num_rows) return;
    if (row < off[0] || row >= off[a.B]) return;
    // A packed causal batch needs no sequence lookup: every row in range is a
    // valid history row.
    int b = 0, r = 0, n = 0;
    bool want_score = false;
    if (need_seq) {
        b = seq_of_row(off, a.B, row);
        r = (int)(row - off[b]);
        const int L = a.lengths ? lens[b] : off[b + 1] - off[b];
        if (r >= L) return;  // padding row: never read or written
        n = a.cross ? 0 : (a.ncand ? L - ncs[b] : L);
        want_score = a.w != nullptr && r >= n;
    }
    // (with cand_only only the candidate rows are covered by this call's map)
    const bool mapped = BF16 && a.rowmap != nullptr && (want_score || !a.cand_only);
    if (a.y == nullptr && !want_score && !mapped) return;

    const int W = a.width;
    // the map entry and both operand rows are fetched before any arithmetic
    const int code = mapped ? a.rowmap[row] : -1;
    float x[NCH][8], u[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
            Vec8<BF16>::load(a.o, row * a.o_stride + col, x[c]);
            if (a.y || want_score) Vec8<BF16>::load(a.u, row * a.u_stride + col, u[c]);
        }
    }
    if constexpr (BF16) {
        if (code >= 0) {
            // O of a split row: slot | pieces << 16 | (row within block) << 23
            const int slot = code & 0xffff, np = (code >> 16) & 0x7f, lr = code >> 23;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int col = (c * 64 + lane) * 8;
                if (col < W) {
                    const int h = col / a.d;
                    const int cc = col - h * a.d;
                    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    for (int k = 0; k < np; ++k) {
                        const float* src = a.partial + ((int64_t)(slot + k) * a.H + h) * a.BM * a.d +
                                           (int64_t)lr * a.d + cc;
                        const f32x4 p0 = *reinterpret_cast<const f32x4*>(src);
                        const f32x4 p1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[e] += p0[e];
                            acc[4 + e] += p1[e];
                        }
                    }
                    u32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        r[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
                        x[c][2 * e] = __uint_as_float(r[e] << 16);
                        x[c][2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
                    }
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + row * a.o_stride + col) = r;
                }
            }
        }
        if (a.cross) {
            // the candidate's own key: per head (16 lanes of 8 columns),
            // s = q.k + rab_pos[0] + rab_time[0], O += alpha SiLU(s) v
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int col = (c * 64 + lane) * 8;
                float q8[8], k8[8], v8[8];
                float dot = 0.0f;
                if (col < W) {
                    Vec8<true>::load(a.sq, row * a.sqs + col, q8);
                    Vec8<true>::load(a.sk, row * a.sks + col, k8);
                    Vec8<true>::load(a.sv, row * a.svs + col, v8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) dot = fmaf(q8[e], k8[e], dot);
                }
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) dot += __shfl_xor(dot, m, 64);
                if (col < W) {
                    const int h = col / a.d;
                    const float sv = dot + a.rab_pos[(int64_t)h * a.rp_hs] + a.rab_time[(int64_t)h * a.rt_hs];
                    const float act = a.alpha * silu_fast(sv);
                    u32x4 rr;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        rr[e] = pack_bf16x2(fmaf(act, v8[2 * e], x[c][2 * e]), fmaf(act, v8[2 * e + 1], x[c][2 * e + 1]));
                        x[c][2 * e] = __uint_as_float(rr[e] << 16);
                        x[c][2 * e + 1] = __uint_as_float(rr[e] & 0xffff0000u);
                    }
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + row * a.o_stride + col) = rr;
                }
            }
        }
        if (a.y == nullptr && !want_score) return;
    }
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += x[c][e];
        }
    }
    const float mean = wave_sum(sum) / (float)W;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dlt = x[c][e] - mean;
                sq = fmaf(dlt, dlt, sq);
            }
        }
    }
    const float var = wave_sum(sq) / (float)W;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    float dot = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (x[c][e] - mean) * rstd * u[c][e];
            if (a.y) Vec8<BF16>::store(a.y, row * a.y_stride + col, y);
            if (want_score) {
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf(y[e], a.w[col + e], dot);
            }
        }
    }
    if (want_score) {
        dot = wave_sum(dot);
        if (lane == 0) a.scores[(int64_t)b * a.score_stride + (r - n)] = dot;
    }
}

// The common case -- bf16, a packed causal batch (no padding, no candidates,
// no scores), Y wanted -- with R rows per wave: the map entries and operand
// rows of all R rows are fetched before any arithmetic, so that a wave keeps
// R times more bytes in flight (one row of H*d_v = 512 values is only 2 KB
// of loads).  Split rows (map entry >= 0) take their O from the partial sums
// as in ln_gate_kernel.
template <int NCH, int R>
__global__ void __launch_bounds__(kThreads) ln_gate_rows_kernel(LnGateArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * R;
    const int64_t lo = a.offsets[0], hi = min((int64_t)a.offsets[a.B], a.num_rows);
    const int W = a.width;
    if (row0 >= hi || row0 + R <= lo) return;
    // Loads are unconditional, from rows clamped into [lo, hi) and columns
    // clamped into the row, so that no branch joins in-flight registers;
    // the pairs stay raw bf16 until the last load is issued, which keeps
    // every load of the wave in flight together.
    int code[R];
    u32x4 xr[R][NCH], ur[R][NCH];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t row = min(max(row0 + k, lo), hi - 1);
        code[k] = a.rowmap ? a.rowmap[row] : -1;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int col = (c * 64 + lane) * 8 < W ? (c * 64 + lane) * 8 : 0;
            xr[k][c] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.o) + row * a.o_stride + col));
            ur[k][c] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.u) + row * a.u_stride + col));
        }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t row = row0 + k;
        if (!(row >= lo && row < hi)) continue;
        if (code[k] >= 0) {
            // O of a split row: slot | pieces << 16 | (row within block) << 23
            const int slot = code[k] & 0xffff, np = (code[k] >> 16) & 0x7f, lr = code[k] >> 23;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int col = (c * 64 + lane) * 8;
                if (col < W) {
                    const int h = col / a.d;
                    const int cc = col - h * a.d;
                    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    for (int pc = 0; pc < np; ++pc) {
                        const float* src = a.partial + ((int64_t)(slot + pc) * a.H + h) * a.BM * a.d +
                                           (int64_t)lr * a.d + cc;
                        const f32x4 p0 = *reinterpret_cast<const f32x4*>(src);
                        const f32x4 p1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[e] += p0[e];
                            acc[4 + e] += p1[e];
                        }
                    }
                    u32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
                    xr[k][c] = r;
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + row * a.o_stride + col) = r;
                }
            }
        }
        float x[NCH][8], u[NCH][8];
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if ((c * 64 + lane) * 8 < W)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[c][2 * e] = __uint_as_float(xr[k][c][e] << 16);
                    x[c][2 * e + 1] = __uint_as_float(xr[k][c][e] & 0xffff0000u);
                    u[c][2 * e] = __uint_as_float(ur[k][c][e] << 16);
                    u[c][2 * e + 1] = __uint_as_float(ur[k][c][e] & 0xffff0000u);
                    sum += x[c][2 * e] + x[c][2 * e + 1];
                }
        const float mean = wave_sum(sum) / (float)W;
        float sq = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if ((c * 64 + lane) * 8 < W)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dlt = x[c][e] - mean;
                    sq = fmaf(dlt, dlt, sq);
                }
        const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)W + a.eps);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int col = (c * 64 + lane) * 8;
            if (col < W) {
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (x[c][e] - mean) * rstd * u[c][e];
                Vec8<true>::store(a.y, row * a.y_stride + col, y);
            }
        }
    }
}

// Gradients of Y = LN(O) (.) U for bf16 rows (one wave per row): with
// xhat = (O - mean) rstd,
//   dU = xhat (.) dY,   g = dY (.) U,   dO = rstd (g - mean(g) - xhat mean(g xhat))
// (the derivative of a LayerNorm without affine parameters).  Padding rows
// are skipped.
template <int NCH>
__global__ void __launch_bounds__(kThreads) ln_gate_bwd_kernel(LnGateBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (a.B <= 0 || row >= a.num_rows) return;
    if (row < a.offsets[0] || row >= a.offsets[a.B]) return;
    if (a.lengths) {
        const int b = seq_of_row(a.offsets, a.B, row);
        if ((int)(row - a.offsets[b]) >= a.lengths[b]) return;
    }
    const int W = a.width;
    float x[NCH][8], u[NCH][8], gy[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
            Vec8<true>::load(a.o, row * a.o_stride + col, x[c]);
            Vec8<true>::load(a.u, row * a.u_stride + col, u[c]);
            Vec8<true>::load(a.dy, row * a.dy_stride + col, gy[c]);
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if ((c * 64 + lane) * 8 < W)
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += x[c][e];
    const float mean = wave_sum(sum) / (float)W;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if ((c * 64 + lane) * 8 < W)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dlt = x[c][e] - mean;
                sq = fmaf(dlt, dlt, sq);
            }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)W + a.eps);
    float mg = 0.0f, mgx = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
            float du[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xh = (x[c][e] - mean) * rstd;
                const float g = gy[c][e] * u[c][e];
                du[e] = xh * gy[c][e];
                mg += g;
                mgx = fmaf(g, xh, mgx);
                x[c][e] = xh;
                u[c][e] = g;
            }
            if (a.du) Vec8<true>::store(a.du, row * a.du_stride + col, du);
        }
    }
    mg = wave_sum(mg) / (float)W;
    mgx = wave_sum(mgx) / (float)W;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < W) {
            float d[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) d[e] = rstd * (u[c][e] - mg - x[c][e] * mgx);
            Vec8<true>::store(a.dout, row * a.dout_stride + col, d);
        }
    }
}

template <bool BF16>
hipError_t launch_typed(const LnGateArgs& a, hipStream_t stream) {
    const int nch = (a.width + 511) / 512;
    if (BF16 && a.B > 0 && !a.lengths && !a.ncand && !a.cross && !a.w && a.y && nch <= 2 && !a.cand_only) {
        if (nch == 1) {
            const dim3 g((unsigned)((a.num_rows + 4 * kRowsPerBlock - 1) / (4 * kRowsPerBlock)));
            hipExtLaunchKernelGGL((ln_gate_rows_kernel<1, 4>), g, dim3(kThreads), 0, stream, a.ev_begin, a.ev_end, 0, a);
        } else {
            const dim3 g((unsigned)((a.num_rows + 2 * kRowsPerBlock - 1) / (2 * kRowsPerBlock)));
            hipExtLaunchKernelGGL((ln_gate_rows_kernel<2, 2>), g, dim3(kThreads), 0, stream, a.ev_begin, a.ev_end, 0, a);
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((a.num_rows + kRowsPerBlock - 1) / kRowsPerBlock));
    switch (nch) {
        case 1: hipExtLaunchKernelGGL((ln_gate_kernel<BF16, 1>), grid, dim3(kThreads), 0, stream, a.ev_begin, a.ev_end, 0, a); break;
        case 2: hipExtLaunchKernelGGL((ln_gate_kernel<BF16, 2>), grid, dim3(kThreads), 0, stream, a.ev_begin, a.ev_end, 0, a); break;
        case 3:
        case 4: hipExtLaunchKernelGGL((ln_gate_kernel<BF16, 4>), grid, dim3(kThreads), 0, stream, a.ev_begin, a.ev_end, 0, a); break;
        default: hipExtLaunchKernelGGL((ln_gate_kernel<BF16, 8>), grid, dim3(kThreads), 0, stream, a.ev_begin, a.ev_end, 0, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_gate_bwd(const LnGateBwdArgs& a, hipStream_t stream) {
    if (a.num_rows <= 0 || a.B <= 0) return hipSuccess;
    const int nch = (a.width + 511) / 512;
    const dim3 grid((unsigned)((a.num_rows + kRowsPerBlock - 1) / kRowsPerBlock));
    switch (nch) {
        case 1: hipLaunchKernelGGL((ln_gate_bwd_kernel<1>), grid, dim3(kThreads), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((ln_gate_bwd_kernel<2>), grid, dim3(kThreads), 0, stream, a); break;
        case 3:
        case 4: hipLaunchKernelGGL((ln_gate_bwd_kernel<4>), grid, dim3(kThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL((ln_gate_bwd_kernel<8>), grid, dim3(kThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_ln_gate(const LnGateArgs& a, hipStream_t stream) {
    if (a.num_rows <= 0) return hipSuccess;
    return a.dtype == HSTU_BF16 ? launch_typed<true>(a, stream) : launch_typed<false>(a, stream);
}

}  // namespace hstu
