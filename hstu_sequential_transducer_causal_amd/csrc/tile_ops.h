// tile_ops.h -- gfx950 building blocks of the attention kernels: 32x32x16
// MFMA, LDS tiles of 32 rows x 128 bf16 columns in two swizzled layouts,
// direct-to-LDS buffer loads with explicit waits, and the transposed LDS
// reads that turn such a tile into MFMA B operands.
//
// v_mfma_f32_32x32x16_bf16: A operand lane l holds row l % 32, k values
// 8 (l / 32) .. +7; B operand lane l holds column l % 32, the same k slots;
// the 16 results of lane l are column l % 32, rows 8 (r / 4) + 4 (l / 32) +
// r % 4.  Any k order consistent between A and B gives the same product.
#pragma once

#include "hstu_device.h"

namespace hstu {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128 * 2;   // one tile row: 128 bf16

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniu(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

typedef __attribute__((address_space(3))) void lds_void;

// 4 bf16 of V^T through the LDS transpose read: within each 16-lane group,
// output lane i, element k comes from input lane 4k + i/4, element i % 4.
__device__ __forceinline__ u32x2 ds_read_tr(const uint8_t* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p);
    return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ int kswz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 15)) << 4); }
__device__ __forceinline__ int vswz(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row & 3) << 2)) << 4); }

// Each block opens with 5 wait states: the compiler does not look inside
// inline assembly for hazards, and a VALU write of an SGPR (a v_readlane
// reloading a spilled descriptor, say) needs 5 before a vector memory
// instruction may read that SGPR (the M0 write needs 1).
//
// The tile loads are issued from inline assembly, so the compiler sees no
// LDS write it has to wait for: it cannot tell the ring stage being filled
// from the one being read, and with the loads visible to it would wait for
// every load in flight before each LDS read.  The waits are explicit
// instead: the vmcnt below before a stage is read, then a bare s_barrier (the
// memory clobber keeps LDS accesses on their side of it).  Loads complete in
// issue order, and loads the compiler issues itself after these only make
// its own vmcnt waits stricter, never looser.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void dma4(const u32x4& rsrc, uint32_t lds, uint32_t voff) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// This wave's LDS accesses (ordinary stores included) are complete.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Barrier after which every wave sees the others' ordinary LDS stores; vector
// memory operations (the output stores of the previous item) stay in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Buffer resource: base, stride 0, num_records bytes (accesses at or past it
// read as zero).
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = uniu((uint32_t)a);
    r[1] = uniu((uint32_t)(a >> 32) & 0xffffu);
    r[2] = uniu(bytes);
    r[3] = 0x00020000u;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// vmcnt(n) with the other counters left alone (n <= 15).
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// Fragment reads by 32-bit LDS address.  Every per-lane address of a tile is
// one base XOR a constant: K fragment kc of lane l (row l % 32, chunk
// 2 kc + l / 32, swizzled by row & 15) sits at base ^ (kc << 5), and the V^T
// fragment for column block nb at base ^ (nb << 6) (the swizzle moves whole
// 64-byte quarters by row & 3), with the chunk and the second row group as
// immediate offsets.  Only the two bases stay live across the tile loop.
__device__ __forceinline__ uint32_t k_lane_offset(int lane) {
    const int l32 = lane & 31, h2 = lane >> 5;
    return (uint32_t)(l32 * kRowBytes + ((h2 ^ (l32 & 15)) << 4));
}
__device__ __forceinline__ uint32_t v_lane_offset(int lane) {
    const int m = lane & 15;
    const int row = 4 * (lane >> 5) + (m >> 2);                  // key row of chunk 0
    const int x = ((lane >> 4) & 1) * 2 + ((m & 3) >> 1);         // 16-byte chunk within the column quarter
    return (uint32_t)(row * kRowBytes + ((((row & 3) << 2) | x) << 4) + 8 * (m & 1));
}
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    return *(lds_bf16x8*)(uintptr_t)addr;
}
__device__ __forceinline__ u32x2 lds_read_tr(uint32_t addr) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr);
    return __builtin_bit_cast(u32x2, r);
}
// B operand fragments of a [32][128] tile stored with vswz, for a product
// whose contraction runs over the tile's rows (O += A V over keys in the
// forward), for both 16-row chunks c: for each 32-column block nb, lane l gets
// column nb*32 + l % 32 at rows 16c + 4 (l / 32) + 0..3 and 16c + 8 +
// 4 (l / 32) + 0..3 -- the row order in which a 32x32 accumulator, packed by
// 4-element groups, holds the A operand (two transposed reads of 4 rows x 4
// columns per 16-lane group).  voff = v_lane_offset(lane).
__device__ __forceinline__ void read_v_tile(uint32_t stage_base, uint32_t voff, u32x4 (&vf)[2][4]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const uint32_t a = stage_base + (voff ^ (uint32_t)(nb << 6));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x2 v0 = lds_read_tr(a + c * 16 * kRowBytes);
            const u32x2 v1 = lds_read_tr(a + c * 16 * kRowBytes + 8 * kRowBytes);
            vf[c][nb] = u32x4{v0[0], v0[1], v1[0], v1[1]};
        }
    }
}

// Turning a 32x32 accumulator over.  Packed to bf16 by 4-element groups, an
// accumulator (lane l = column l % 32, values of rows 8 (r / 4) + 4 (l / 32)
// + r % 4) is the A operand of two 32x32x16 products whose rows are its
// columns and whose contraction runs over its rows: chunk c, slot e of lane
// l standing for row 16 c + 8 (e / 4) + 4 (l / 32) + e % 4.  Against these
// two B operands -- the identity over those rows -- the products give the
// transpose in accumulator form: lane l = row l % 32, values of columns
// 8 (r / 4) + 4 (l / 32) + r % 4.  Each bf16 value passes exactly.
__device__ __forceinline__ void transpose_identity(int lane, bf16x8 (&idf)[2]) {
    const int n = lane & 31, h2 = lane >> 5;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if ((n >> 4) == c && ((n >> 2) & 1) == h2) {
            const int e = 4 * ((n >> 3) & 1) + (n & 3);
            z[e >> 1] = 0x3F80u << (16 * (e & 1));
        }
        idf[c] = __builtin_bit_cast(bf16x8, z);
    }
}

// Bucket index (leading zeros of 2|dt| + 1) of an encoded gap 2|dt|.
__device__ __forceinline__ uint32_t clz_gap(uint32_t gap2) { return __builtin_clz(gap2 + 1u); }

}  // namespace hstu
