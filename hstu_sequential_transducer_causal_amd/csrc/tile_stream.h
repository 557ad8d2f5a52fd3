// tile_stream.h -- streaming [32][128] bf16 tiles of a row-major matrix into
// an LDS ring with direct-to-LDS buffer loads (the gradient kernels): rows
// past the valid count fall outside the buffer's range and arrive as zeros.
#pragma once

#include "tile_ops.h"

namespace hstu {

constexpr int kTileBytes = 32 * kRowBytes;   // one [32][128] bf16 tile

// Loads of one 32-row tile of a [rows][128] bf16 matrix (one head's columns of
// one sequence) into a ring stage: wave w writes tile rows 8w .. 8w+7 with two
// 1 KiB buffer loads; lane l of load m writes row 8w + 4m + l / 16 at physical
// chunk l % 16, so it fetches the logical chunk the swizzle puts there.
struct TileSrc {
    u32x4 rs;
    uint32_t off[2];       // per-lane byte offsets of the two loads
    uint32_t tile_bytes;   // scalar step per 32-row tile
};

__device__ __forceinline__ TileSrc tile_src(const uint16_t* base, int64_t stride, int L, int lane, int wave,
                                            bool vlayout) {
    TileSrc t;
    t.rs = make_rsrc(base, (uint32_t)(L * stride * 2));
    const int pc = lane & 15;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int r = 8 * wave + 4 * m + (lane >> 4);
        const int c = vlayout ? (pc ^ ((r & 3) << 2)) : (pc ^ (r & 15));
        t.off[m] = (uint32_t)(r * stride * 2 + c * 16);
    }
    t.tile_bytes = (uint32_t)(32 * stride * 2);
    return t;
}

__device__ __forceinline__ void issue_part(const TileSrc& t, const uint8_t* ring, int stage, int tile, int wave) {
    const uint32_t l0 = lds_addr(ring) + (uint32_t)(stage * kTileBytes + 2 * wave * 1024);
    const uint32_t soff = uniu((uint32_t)tile * t.tile_bytes);
#pragma unroll
    for (int m = 0; m < 2; ++m) dma16(t.rs, uniu(l0 + m * 1024), t.off[m], soff);
}

}  // namespace hstu
