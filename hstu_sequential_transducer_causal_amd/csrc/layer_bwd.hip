// layer_bwd.hip -- the pieces of the HSTU layer's gradients around the
// attention: weight gradients of f1 and f2 (a contraction over tokens), bias
// gradients (token sums), the slope of the SiLU of phi1, and weight
// transposes for the data gradients.
//
// The layer ("生成式推荐（一）：HSTU", section "高性能自注意力Encoder：HSTU"):
// Z = SiLU(X W1^T + b1) -> U | V | Q | K, attention, Y = LN(O) (.) U,
// X_out = X + Y W2^T + b2.  Its gradients (chain rule, reverse order):
//   dY = dX_out W2,  dW2 = dX_out^T Y,  db2 = sum_t dX_out,
//   (gate and attention) -> dZ = dU | dV | dQ | dK,
//   dP = dZ (.) SiLU'(P), P = X W1^T + b1,
//   dX = dX_out + dP W1,  dW1 = dP^T X,  db1 = sum_t dP.
//
// gemm_tn_kernel: C[m, n] = sum_t A[t, m] B[t, n] for token-major A and B.
// Both operands stream as [32 tokens][128 columns] tiles into an LDS ring and
// are read transposed (ds_read_b64_tr_b16), which puts the tokens in the
// contraction slots of v_mfma_f32_32x32x16_bf16 for both in the same order.
// The token range is split over workgroups (fp32 partials), summed in a fixed
// order by split_sum_kernel.
#include <hip/hip_ext.h>

#include "internal.h"
#include "hstu_device.h"
#include "tile_ops.h"
#include "tile_stream.h"

namespace hstu {

namespace {

constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kSumChunks = 64;
constexpr int kTnWgPerCu = 2;     // gemm_tn_kernel workgroups resident per CU (48 KiB of LDS each)

struct TnParams {
    const uint16_t* a; int64_t lda;   // [T, M]
    const uint16_t* b; int64_t ldb;   // [T, N]
    int64_t T;
    int M, N;
    int splits, tiles_per_split;      // token tiles (32 rows) per split
    float* part;                      // [splits][M][N]
};

// Two 32-column blocks (cb, cb + 1) of the transposed read of a [32][128]
// vswz tile, 16-row chunk c: lane l gets column cb*32 + l % 32 (and the next
// block) at rows 16c + 4 (l / 32) + 0..3 and 16c + 8 + 4 (l / 32) + 0..3.
__device__ __forceinline__ void read_tr_pair(const uint8_t* lds, int c, int lane, int cb, bf16x8 (&f)[2]) {
    const int m = lane & 15;
    const int dsub = ((lane >> 4) & 1) * 16;
    const int row0 = c * 16 + 4 * (lane >> 5) + (m >> 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int col = (cb + i) * 32 + dsub + 4 * (m & 3);
        const int chunk = col >> 3;
        const int within = (col & 7) * 2;
        const u32x2 v0 = ds_read_tr(lds + vswz(row0, chunk) + within);
        const u32x2 v1 = ds_read_tr(lds + vswz(row0 + 8, chunk) + within);
        f[i] = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
    }
}

__device__ __forceinline__ void wait_loads(int n) {
    if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// 128 x 128 output tile per workgroup; wave w computes rows 64 (w / 2) ..,
// columns 64 (w % 2) .. as 2 x 2 blocks of 32 x 32.
__global__ void __launch_bounds__(kThreads, kTnWgPerCu) gemm_tn_kernel(TnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t ring_a[kStages * kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring_b[kStages * kTileBytes];
    const int lane = threadIdx.x & 63;
    const int wave = uni(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 128;
    const int split = blockIdx.z;
    const int64_t ntok_tiles = (p.T + 31) / 32;
    const int t_begin = split * p.tiles_per_split;
    const int t_end = (int)min<int64_t>(ntok_tiles, (int64_t)t_begin + p.tiles_per_split);
    const int ntiles = max(0, t_end - t_begin);
    const int wm = wave >> 1, wn = wave & 1;

    const TileSrc sa = tile_src(p.a + m0, p.lda, (int)p.T, lane, wave, true);
    const TileSrc sb = tile_src(p.b + n0, p.ldb, (int)p.T, lane, wave, true);
    auto issue = [&](int stage, int tile) {
        issue_part(sa, ring_a, stage, tile, wave);
        issue_part(sb, ring_b, stage, tile, wave);
    };
#pragma unroll
    for (int pre = 0; pre < kStages - 1; ++pre)
        if (pre < ntiles) issue(pre, t_begin + pre);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int it = 0; it < ntiles; ++it) {
        const int stage = it % kStages;
        wait_loads(it + 1 < ntiles ? 4 : 0);   // 4 loads per tile and wave
        lds_barrier();
        if (it + kStages - 1 < ntiles) issue((it + kStages - 1) % kStages, t_begin + it + kStages - 1);
        const uint8_t* a_lds = ring_a + stage * kTileBytes;
        const uint8_t* b_lds = ring_b + stage * kTileBytes;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 af[2], bfr[2];
            read_tr_pair(a_lds, c, lane, 2 * wm, af);
            read_tr_pair(b_lds, c, lane, 2 * wn, bfr);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    }

    // lane holds C[row 8 (r / 4) + 4 (l / 32) + r % 4][column l % 32] of each block
    const int l32 = lane & 31, h2 = lane >> 5;
    float* out = p.part + (int64_t)split * p.M * p.N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + (2 * wm + i) * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                const int n = n0 + (2 * wn + j) * 32 + l32;
                out[(int64_t)m * p.N + n] = acc[i][j][r];
            }
}

// out[e] = scale * sum_s part[s][e], in split order.
__global__ void __launch_bounds__(256) split_sum_kernel(const float* part, int64_t count, int splits, float* out) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= count) return;
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s) acc += part[(int64_t)s * count + e];
    out[e] = acc;
}

// Column sums of a bf16 [T, C] matrix in two fixed-order passes: chunk k of
// kSumChunks row ranges per column, then the chunks.
__global__ void __launch_bounds__(256) colsum_partial_kernel(const uint16_t* x, int64_t ld, int64_t T, int C,
                                                             float* part) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    const int k = blockIdx.y;
    if (col >= C) return;
    const int64_t per = (T + kSumChunks - 1) / kSumChunks;
    const int64_t t0 = k * per, t1 = min(T, t0 + per);
    float a0 = 0.0f, a1 = 0.0f;
    int64_t t = t0;
    for (; t + 2 <= t1; t += 2) {
        a0 += bf16_to_f32(x[t * ld + col]);
        a1 += bf16_to_f32(x[(t + 1) * ld + col]);
    }
    if (t < t1) a0 += bf16_to_f32(x[t * ld + col]);
    part[(int64_t)k * C + col] = a0 + a1;
}

__global__ void __launch_bounds__(256) colsum_final_kernel(const float* part, int C, float* out) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= C) return;
    float acc = 0.0f;
    for (int k = 0; k < kSumChunks; ++k) acc += part[(int64_t)k * C + col];
    out[col] = acc;
}

// dP = dZ (.) SiLU'(P) in place on dZ: SiLU'(x) = s (1 + x (1 - s)), s = sigmoid(x).
__global__ void __launch_bounds__(256) silu_grad_kernel(uint16_t* dz, const uint16_t* pre, int64_t count8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count8) return;
    u32x4 g = reinterpret_cast<const u32x4*>(dz)[i];
    const u32x4 x = reinterpret_cast<const u32x4*>(pre)[i];
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float gv[2] = {__uint_as_float(g[e] << 16), __uint_as_float(g[e] & 0xffff0000u)};
        const float xv[2] = {__uint_as_float(x[e] << 16), __uint_as_float(x[e] & 0xffff0000u)};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-xv[h] * kLog2e));
            gv[h] *= s * (1.0f + xv[h] * (1.0f - s));
        }
        r[e] = pack_bf16x2(gv[0], gv[1]);
    }
    reinterpret_cast<u32x4*>(dz)[i] = r;
}

// out[c][r] = in[r][c] for a bf16 [R, C] matrix, 32 x 32 tiles through LDS.
__global__ void __launch_bounds__(256) transpose_kernel(const uint16_t* in, int R, int C, uint16_t* out) {
    __shared__ uint16_t tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 8 rows per pass
    for (int k = ty; k < 32; k += 8)
        if (r0 + k < R && c0 + tx < C) tile[k][tx] = in[(int64_t)(r0 + k) * C + c0 + tx];
    __syncthreads();
    for (int k = ty; k < 32; k += 8)
        if (c0 + k < C && r0 + tx < R) out[(int64_t)(c0 + k) * R + r0 + tx] = tile[tx][k];
}

}  // namespace

int gemm_tn_splits(int64_t T, int M, int N) {
    const int tiles = (M / 128) * (N / 128);
    const int64_t tok_tiles = (T + 31) / 32;
    int s = (kTnWgPerCu * device_cu_count() + tiles - 1) / max(tiles, 1);
    s = (int)std::min<int64_t>(std::max(1, s), std::max<int64_t>(1, tok_tiles));
    return std::min(s, 64);
}

hipError_t launch_gemm_tn(const GemmTnArgs& g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    TnParams p;
    p.a = static_cast<const uint16_t*>(g.a); p.lda = g.lda;
    p.b = static_cast<const uint16_t*>(g.b); p.ldb = g.ldb;
    p.T = g.T; p.M = g.M; p.N = g.N;
    p.splits = g.splits;
    const int64_t tok_tiles = (g.T + 31) / 32;
    p.tiles_per_split = (int)((tok_tiles + g.splits - 1) / g.splits);
    p.part = g.part;
    hipLaunchKernelGGL(gemm_tn_kernel, dim3(g.N / 128, g.M / 128, g.splits), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t count = (int64_t)g.M * g.N;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, g.part, count,
                       g.splits, g.c);
    return hipGetLastError();
}

size_t colsum_part_floats(int C) { return (size_t)kSumChunks * C; }

hipError_t launch_colsum(const void* x, int64_t ld, int64_t T, int C, float* part, float* out, hipStream_t stream) {
    if (C <= 0) return hipSuccess;
    hipLaunchKernelGGL(colsum_partial_kernel, dim3((unsigned)((C + 255) / 256), kSumChunks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), ld, T, C, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, stream, part, C, out);
    return hipGetLastError();
}

hipError_t launch_silu_grad(void* dz, const void* pre, int64_t count, hipStream_t stream) {
    const int64_t n8 = count / 8;
    if (n8 <= 0) return hipSuccess;
    hipLaunchKernelGGL(silu_grad_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint16_t*>(dz), static_cast<const uint16_t*>(pre), n8);
    return hipGetLastError();
}

hipError_t launch_transpose(const void* in, int R, int C, void* out, hipStream_t stream) {
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((C + 31) / 32), (unsigned)((R + 31) / 32)), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(in), R, C, static_cast<uint16_t*>(out));
    return hipGetLastError();
}

}  // namespace hstu
