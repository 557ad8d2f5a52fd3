// gemm.hip -- bf16 MFMA GEMMs of the HSTU layer's pointwise projection f1
// (with the SiLU of phi1 fused) and pointwise transformation f2 (with the
// residual fused): "生成式推荐（一）：HSTU", section
// "高性能自注意力Encoder：HSTU" (f1 and f2 are single linear layers, phi1 =
// SiLU, residual connections between identical layers).
//
//   C[m, n] = epi( sum_k A[m, k] B[n, k] + bias[n] ) (+ R[m, n])
//
// A (activations) and B (weights, out x in) are both K-contiguous, so both
// feed v_mfma_f32_16x16x32_bf16 with 16-byte reads.  128 x 128 block tile,
// BK = 64, 4 waves of 64 x 64, LDS tiles with a 16-byte XOR swizzle and a
// register prefetch of the next K slice.  Requires N % 128 == 0 and
// K % 64 == 0; M is arbitrary (rows are guarded).
#include "internal.h"
#include "hstu_device.h"

namespace hstu {

namespace {

constexpr int TM = 128, TN = 128, TK = 64;
constexpr int kThreads = 256;

struct Params {
    int64_t M;
    int N, K;
    const uint16_t* a; int64_t lda;
    const uint16_t* b; int64_t ldb;
    const float* bias;
    const uint16_t* res; int64_t ldr;
    uint16_t* c; int64_t ldc;
    int silu;
    uint16_t* cp; int64_t ldcp;   // optional pre-activation output
};

// Row r of a [128][64] bf16 tile occupies 128 bytes = 8 chunks of 16 bytes;
// chunk x of row r is stored at position x ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz(int r, int x) { return (r * 8 + (x ^ ((r >> 1) & 7))) << 4; }

__global__ void __launch_bounds__(kThreads, 2) gemm_bf16_kernel(Params p) {
    __shared__ __align__(16) uint8_t sa[TM * TK * 2];
    __shared__ __align__(16) uint8_t sb[TN * TK * 2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c16 = lane & 15;
    const int g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * TM;
    const int n0 = blockIdx.x * TN;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging: thread -> (row = tid / 8 + 32 * it, chunk = tid % 8)
    const int srow = tid >> 3, sch = tid & 7;
    u32x4 ra[4], rb[4];
    auto prefetch = [&](int k0) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = srow + 32 * it;
            const int64_t m = m0 + r;
            u32x4 z = {0u, 0u, 0u, 0u};
            ra[it] = z;
            if (m < p.M) ra[it] = *reinterpret_cast<const u32x4*>(p.a + m * p.lda + k0 + sch * 8);
            rb[it] = *reinterpret_cast<const u32x4*>(p.b + (int64_t)(n0 + r) * p.ldb + k0 + sch * 8);
        }
    };
    prefetch(0);
    for (int k0 = 0; k0 < p.K; k0 += TK) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = srow + 32 * it;
            *reinterpret_cast<u32x4*>(sa + swz(r, sch)) = ra[it];
            *reinterpret_cast<u32x4*>(sb + swz(r, sch)) = rb[it];
        }
        __syncthreads();
        if (k0 + TK < p.K) prefetch(k0 + TK);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + i * 16 + c16;
                af[i] = *reinterpret_cast<const bf16x8*>(sa + swz(r, 4 * kc + g));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wn * 64 + j * 16 + c16;
                bfr[j] = *reinterpret_cast<const bf16x8*>(sb + swz(r, 4 * kc + g));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
        }
        __syncthreads();
    }

    // epilogue: lane holds C[row 4g + r][col c16] of each 16 x 16 block
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + c16;
        const float bias = p.bias ? p.bias[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + 4 * g + r;
                if (m < p.M) {
                    float x = acc[i][j][r] + bias;
                    if (p.cp) p.cp[m * p.ldcp + n] = f32_to_bf16_bits(x);
                    if (p.silu) x = silu_fast(x);
                    if (p.res) x += bf16_to_f32(p.res[m * p.ldr + n]);
                    p.c[m * p.ldc + n] = f32_to_bf16_bits(x);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
    if (g.M <= 0) return hipSuccess;
    Params p;
    p.M = g.M; p.N = g.N; p.K = g.K;
    p.a = static_cast<const uint16_t*>(g.a); p.lda = g.lda;
    p.b = static_cast<const uint16_t*>(g.b); p.ldb = g.ldb;
    p.bias = g.bias;
    p.res = static_cast<const uint16_t*>(g.residual); p.ldr = g.ldr;
    p.c = static_cast<uint16_t*>(g.c); p.ldc = g.ldc;
    p.silu = g.silu;
    p.cp = static_cast<uint16_t*>(g.c_pre); p.ldcp = g.ldcp;
    dim3 grid(g.N / TN, (unsigned)((g.M + TM - 1) / TM));
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hstu
