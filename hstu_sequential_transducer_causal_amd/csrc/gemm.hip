// gemm.hip -- bf16 MFMA GEMMs of the HSTU layer's pointwise projection f1
// (with the SiLU of phi1 fused) and pointwise transformation f2 (with the
// residual fused): "生成式推荐（一）：HSTU", section
// "高性能自注意力Encoder：HSTU" (f1 and f2 are single linear layers, phi1 =
// SiLU, residual connections between identical layers).
//
//   C[m, n] = epi( sum_k A[m, k] B[n, k] + bias[n] ) (+ R[m, n])
//
// A (activations, [M][K]) and B (weights, out x in, [N][K]) are both
// K-contiguous, so a tile row of either is directly an MFMA operand row.
//
// Design (gfx950): a workgroup of 4 waves computes a 256 x 128 tile of C, each
// wave 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16; three workgroups
// share a CU, so one's prologue and epilogue overlap the others' MFMAs.  K
// streams in slices of 32 through a 2-stage LDS ring (24 KiB a stage) filled
// by direct-to-LDS buffer loads issued one slice ahead, so the data never
// passes through registers; rows past M fall outside the buffer's range and
// read as zeros.  A tile row is 64 bytes; its 16-byte chunks are XOR-swizzled
// by (row / 4) % 4, so the 16 rows a 16-lane group reads at one logical chunk
// hit distinct banks.  Per 16-wide K step a wave reads 6 fragments (16 bytes
// a lane) for 8 MFMAs.  The epilogue stages the fp32 tile through the ring in
// passes of 32 rows (72-float row pitch: conflict-free column writes),
// then each lane finishes 8 consecutive columns of a row (bias, optional
// pre-activation copy, SiLU, residual) and writes them with 16-byte stores --
// whole 128-byte lines per 8 lanes.  Tiles are dealt to the dies so that each
// die takes a contiguous run of the strip-major order: the N tiles of one A
// strip share its L2.
//
// Requires N % 128 == 0, K % 32 == 0, row strides that are multiples of 8
// elements and 16-byte aligned matrices; M is arbitrary.
#include "internal.h"
#include "tile_ops.h"

namespace hstu {

namespace {

constexpr int BM = 256, BN = 128, BK = 32;
// Three workgroups per CU (48 KiB of LDS and 160 VGPRs each) with a 2-stage
// ring measured faster than two with 3 stages or one with 4: the latency of
// a tile's first loads and the epilogue's work are hidden by the other
// workgroups rather than by a deeper ring.
constexpr int kWgPerCu = 3;
constexpr int kStages = 2;
constexpr int kAhead = kStages - 1;              // slices in flight ahead of the one computed
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kWaveN = 64;                       // each wave: 128 rows x kWaveN columns of C
constexpr int kBJ = kWaveN / 32;                 // 32x32 blocks across a wave's columns
constexpr int kWavesN = BN / kWaveN;
static_assert(kWaves / kWavesN * 128 == BM, "waves tile the block");
constexpr int kRow = BK * 2;                     // bytes per tile row
constexpr int kABytes = BM * kRow;
constexpr int kBBytes = BN * kRow;
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kSmem = kStages * kStageBytes;
constexpr int kRowsA = BM / kWaves, kRowsB = BN / kWaves;   // tile rows each wave loads
constexpr int kLoadsA = kRowsA / 16, kLoadsB = kRowsB / 16; // 1 KiB loads (16 rows) per wave and slice
constexpr int kLoads = kLoadsA + kLoadsB;
static_assert(kLoads * (kAhead - 1) <= 15, "slice waits fit the vmcnt field");
constexpr int kPitch = kWaveN + 8;               // epilogue staging row pitch (floats): 4 rows = 32 banks
constexpr int kColGroups = kWaveN / 8;           // lanes per staged row (8 columns each)
// epilogue staging: rows of the wave's 128-row tile per pass through the ring
constexpr int kPassRows = kSmem >= kWaves * 128 * kPitch * 4 ? 128
                        : kSmem >= kWaves * 64 * kPitch * 4 ? 64 : 32;
static_assert(kWaves * kPassRows * kPitch * 4 <= kSmem, "a pass of the staged tile fits the ring");

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
    int tiles_n;                  // N / BN
};

// Physical 16-byte chunk of logical chunk x in tile row r (an involution).
__device__ __forceinline__ uint32_t chunk_of(int r, int x) { return (uint32_t)(x ^ ((r >> 2) & 3)); }

// vmcnt(kLoads n): wait until at most n later slices' loads are in flight
// (other counters untouched).
constexpr int vm_field(int n) { return kLoads * n <= 15 ? kLoads * n : 15; }
__device__ __forceinline__ void wait_slice(int n) {
    if (n >= 2)
        __builtin_amdgcn_s_waitcnt(0x0F70 | vm_field(2));
    else if (n == 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | vm_field(1));
    else
        __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }

__global__ void __launch_bounds__(kThreads, kWgPerCu) gemm_bf16_kernel(Params p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int wm = wave / kWavesN, wn = wave % kWavesN;

    // die x (workgroups x, x + 8, ...) takes tiles [x * per + min(x, rem), ...)
    const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
    const int per = nwg / 8, rem = nwg % 8, x = wg % 8;
    const int t = x * per + min(x, rem) + wg / 8;
    const int mt = t / p.tiles_n, nt = t - mt * p.tiles_n;
    const int64_t m0 = (int64_t)mt * BM;
    const int n0 = nt * BN;
    const int rows = (int)min((int64_t)BM, p.M - m0);

    const u32x4 ra = make_rsrc(p.a + m0 * p.lda, (uint32_t)(rows * p.lda * 2));
    const u32x4 rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, (uint32_t)(BN * p.ldb * 2));

    // loads: load m of wave w fills tile rows 16m .. 16m+15 of the wave's
    // share (A: rows kRowsA w + .., B: rows kRowsB w + ..); lane l writes row
    // 16m + l/4 at physical chunk l % 4, so it fetches the logical chunk placed
    // there.  The swizzle does not depend on m; m moves 16 rows (a scalar
    // offset).
    const int q = lane >> 2, pch = lane & 3;
    const int r_a = kRowsA * wave + q, r_b = kRowsB * wave + q;
    const uint32_t voa = (uint32_t)(r_a * p.lda * 2) + (chunk_of(r_a, pch) << 4);
    const uint32_t vob = (uint32_t)(r_b * p.ldb * 2) + (chunk_of(r_b, pch) << 4);
    const uint32_t a16 = uniu((uint32_t)(16 * p.lda * 2)), b16 = uniu((uint32_t)(16 * p.ldb * 2));
    const uint32_t sbase = lds_addr(smem);
    auto issue = [&](int kt) {
        const uint32_t st = sbase + (uint32_t)((kt % kStages) * kStageBytes);
        const uint32_t kb = (uint32_t)kt * (BK * 2);
#pragma unroll
        for (int m = 0; m < kLoadsA; ++m)
            dma16(ra, uniu(st + (uint32_t)((kRowsA * wave + 16 * m) * kRow)), voa, uniu(kb + m * a16));
#pragma unroll
        for (int m = 0; m < kLoadsB; ++m)
            dma16(rb, uniu(st + (uint32_t)(kABytes + (kRowsB * wave + 16 * m) * kRow)), vob, uniu(kb + m * b16));
    };

    // fragments: lane l reads row (block base) + l % 32 at logical chunk
    // 2 s + l / 32 for K step s; the row's swizzle (l % 32 / 4) % 4 is the same
    // in every 32-row block, and chunk 2 s + c is chunk c XOR 2 s, i.e. the
    // address XOR (s << 5)
    const uint32_t qq = (uint32_t)((l32 >> 2) & 3);
    const uint32_t fa = (uint32_t)((wm * 128 + l32) * kRow) + (((uint32_t)h ^ qq) << 4);
    const uint32_t fb = (uint32_t)(kABytes + (wn * kWaveN + l32) * kRow) + (((uint32_t)h ^ qq) << 4);

    f32x16 acc[4][kBJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kBJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = p.K / BK;
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
        if (k < nk) issue(k);
    for (int kt = 0; kt < nk; ++kt) {
        wait_slice(min(kAhead - 1, nk - 1 - kt));   // this wave's loads of slice kt have landed
        lds_barrier();             // ... every wave's, and slice kt-1's stage is free
        if (kt + kAhead < nk) issue(kt + kAhead);
        const uint32_t st = sbase + (uint32_t)((kt % kStages) * kStageBytes);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const uint32_t xa = (st + fa) ^ (uint32_t)(s << 5);
            const uint32_t xb = (st + fb) ^ (uint32_t)(s << 5);
            bf16x8 af[4], bfr[kBJ];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_read_b128(xa + (uint32_t)(i * 32 * kRow));
#pragma unroll
            for (int j = 0; j < kBJ; ++j) bfr[j] = lds_read_b128(xb + (uint32_t)(j * 32 * kRow));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < kBJ; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    }

    // epilogue: stage the wave's 128 x 64 fp32 tile, kPassRows at a time, in its
    // quarter of the ring (result lane l holds column l % 32, rows 8 (r / 4) +
    // 4 (l / 32) + r % 4 of each block), then finish 8 consecutive columns of
    // a row per lane.  (A wave's LDS accesses complete in order: no barrier
    // between its own writes and reads.)
    lds_sync();
    float* stg = reinterpret_cast<float*>(smem) + wave * kPassRows * kPitch;
    const int c8 = (lane % kColGroups) * 8;
    const int n = n0 + wn * kWaveN + c8;
    float bias[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) bias[k] = 0.0f;
    if (p.bias) {
#pragma unroll
        for (int k = 0; k < 8; ++k) bias[k] = p.bias[n + k];
    }
#pragma unroll
    for (int pass = 0; pass < 128 / kPassRows; ++pass) {
#pragma unroll
    for (int i = 0; i < kPassRows / 32; ++i)
#pragma unroll
        for (int j = 0; j < kBJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                stg[(32 * i + 8 * (r >> 2) + 4 * h + (r & 3)) * kPitch + 32 * j + l32] =
                    acc[pass * (kPassRows / 32) + i][j][r];
#pragma unroll 4
    for (int it = 0; it < kPassRows * kColGroups / 64; ++it) {
        const int rr = (64 / kColGroups) * it + lane / kColGroups;
        const int64_t m = m0 + wm * 128 + kPassRows * pass + rr;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(stg + rr * kPitch + c8);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(stg + rr * kPitch + c8 + 4);
        if (m < p.M) {
            float xv[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                xv[k] = v0[k] + bias[k];
                xv[4 + k] = v1[k] + bias[4 + k];
            }
            if (p.cp) {
                const u32x4 w = {pack2(xv[0], xv[1]), pack2(xv[2], xv[3]), pack2(xv[4], xv[5]),
                                 pack2(xv[6], xv[7])};
                *reinterpret_cast<u32x4*>(p.cp + m * p.ldcp + n) = w;
            }
            if (p.silu) {
#pragma unroll
                for (int k = 0; k < 8; ++k) xv[k] = silu_fast(xv[k]);
            }
            if (p.res) {
                const u32x4 rv = *reinterpret_cast<const u32x4*>(p.res + m * p.ldr + n);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xv[2 * k] += __uint_as_float(rv[k] << 16);
                    xv[2 * k + 1] += __uint_as_float(rv[k] & 0xffff0000u);
                }
            }
            const u32x4 w = {pack2(xv[0], xv[1]), pack2(xv[2], xv[3]), pack2(xv[4], xv[5]),
                             pack2(xv[6], xv[7])};
            *reinterpret_cast<u32x4*>(p.c + m * p.ldc + n) = w;
        }
    }
    }
}

bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
    if (g.M <= 0) return hipSuccess;
    if (g.N % BN || g.K % BK || g.K <= 0 || g.lda % 8 || g.ldb % 8 || g.ldc % 8 ||
        (g.residual && g.ldr % 8) || (g.c_pre && g.ldcp % 8) || !aligned16(g.a) || !aligned16(g.b) ||
        !aligned16(g.c) || (g.residual && !aligned16(g.residual)) || (g.c_pre && !aligned16(g.c_pre)))
        return hipErrorInvalidValue;
    if ((int64_t)BM * g.lda * 2 > 0x7fffffffLL || (int64_t)BN * g.ldb * 2 > 0x7fffffffLL)
        return hipErrorInvalidValue;
    Params p;
    p.M = g.M; p.N = g.N; p.K = g.K;
    p.a = static_cast<const uint16_t*>(g.a); p.lda = g.lda;
    p.b = static_cast<const uint16_t*>(g.b); p.ldb = g.ldb;
    p.bias = g.bias;
    p.res = static_cast<const uint16_t*>(g.residual); p.ldr = g.ldr;
    p.c = static_cast<uint16_t*>(g.c); p.ldc = g.ldc;
    p.silu = g.silu;
    p.cp = static_cast<uint16_t*>(g.c_pre); p.ldcp = g.ldcp;
    p.tiles_n = g.N / BN;
    const int64_t tiles = ((g.M + BM - 1) / BM) * (int64_t)p.tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(kThreads), kSmem, stream, p);
    return hipGetLastError();
}

}  // namespace hstu
