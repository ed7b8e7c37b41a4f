// fa_device.h -- small device helpers shared by the gfx950 kernels: vector
// types for the bf16 matrix-core builtins, bf16 <-> fp32 conversion, wave
// reductions, and the workgroup-to-XCD remapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    const bf16x2 v = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order this wave's LDS accesses before and after (another lane's data is read
// back through LDS).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Writes a 32-row x D-column bf16 tile whose fp32 values the wave holds as
// transposed 32x32 matrix-core results: lane l has row l % 32, and register
// 4t + k of block b is column 32b + 8t + 4(l / 32) + k.  Each value is
// multiplied by s and rounded; row r goes to dst + (row0 + r) * D, rows at or
// past nrows are skipped.  A lane holds 4-column pieces of a single row, so
// the tile passes through a 4 KiB LDS stage of this wave, 32 rows x 64
// columns at a time (row r's 16-byte chunk c at chunk c ^ (r % 8) of its 128
// bytes): each store then writes 8 rows x 128 contiguous bytes instead of
// 32 rows x 16 bytes.
template <int D>
__device__ __forceinline__ void store_rows_staged(uint8_t *stg, const f32x16 *acc, float s,
                                                  uint16_t *dst, int64_t row0, int64_t nrows,
                                                  int lane) {
    const int lr = lane & 31, g = lane >> 5;
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x16 &a = acc[2 * h + b2];
                const u32x2 w = {pack_bf16x2(a[4 * t] * s, a[4 * t + 1] * s),
                                 pack_bf16x2(a[4 * t + 2] * s, a[4 * t + 3] * s)};
                *(u32x2 *)(stg + lr * 128 + (((4 * b2 + t) ^ (lr & 7)) << 4) + 8 * g) = w;
            }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + (lane >> 3), ch = lane & 7;
            const u32x4 w = *(const u32x4 *)(stg + r * 128 + ((ch ^ (r & 7)) << 4));
            if (row0 + r < nrows) *(u32x4 *)(dst + (row0 + r) * D + 64 * h + 8 * ch) = w;
        }
        wave_lds_sync();  // the next piece overwrites the stage only after these reads
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---------------------------------------------------------------------------
// LDS tiles streamed with global_load_lds_dwordx4.
//
// A tile is row-major with 16-byte chunks; chunk c of row r is stored at chunk
// c ^ swz<ROWB>(r).  The gfx950 LDS serves a 16-byte read to 16 lanes per
// clock from 64 four-byte banks (one 256-byte bank row), and a transposed
// 8-byte read from 4 rows x 32 bytes per 16 lanes.  The two access patterns
// of the attention kernels are
//   row reads:        16 lanes read the same logical chunk of 16 consecutive
//                     rows (one matrix-core operand per lane);
//   transposed reads: lanes read 32 bytes (two chunks) of 4 consecutive rows
//                     starting at a multiple of 4, with the chunk pair 2-aligned;
// the swizzles below put every lane of such a group on its own banks:
//   128-byte rows (two per bank row): swz = 4*((r>>1)&1) + ((r>>2)&3), which
//     takes 8 distinct values on the even and on the odd rows of any 16;
//   256-byte rows: swz = 4*(r&3) + ((r>>2)&3), 16 distinct values on any 16
//     consecutive rows, and distinct 4-aligned chunk groups on 4 rows.
// Both are unchanged by adding 16 rows, so tiles may be indexed with
// immediates in steps of 16 rows.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int ROWB>
__device__ __forceinline__ int swz(int r) {
    static_assert(ROWB == 128 || ROWB == 256, "row size");
    return ROWB == 128 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// Byte offset of logical chunk c of row r.
template <int ROWB>
__device__ __forceinline__ int chunk_off(int r, int c) {
    return r * ROWB + 16 * (c ^ swz<ROWB>(r));
}

// Transposed-read base of this lane: rows 8h + 4*(lane/32) + (lane%16)/4 and
// columns 32b + 16*((lane/16)%2) + 4*(lane%4); with the read at +16k rows.
template <int ROWB>
__device__ __forceinline__ int tr_off(int lane, int b, int h) {
    const int g = lane >> 5, s = lane & 15, G = lane >> 4;
    const int row = 8 * h + 4 * g + (s >> 2);
    const int chunk = 4 * b + 2 * (G & 1) + ((s >> 1) & 1);
    return chunk_off<ROWB>(row, chunk) + 8 * (s & 1);
}

// Wait until at most N of this wave's vector-memory operations are pending
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8; LDS operations are also drained).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Wait until at most n (0 <= n <= MAX, wave-uniform) groups of PER loads of
// this wave are still in flight.
template <int PER, int MAX>
__device__ __forceinline__ void wait_steps(int n) {
    if constexpr (MAX == 0) {
        wait_vm<0>();
    } else {
        if (n >= MAX)
            wait_vm<MAX * PER>();
        else
            wait_steps<PER, MAX - 1>(n);
    }
}

// Workgroup barrier that orders LDS accesses but does not drain outstanding
// global loads (a ring prefetch stays in flight across it).
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte pieces addressed by lanes i/4 + 4t (t = 0..3); lanes that
// address a 4-row x 16-column bf16 block receive its columns.
__device__ __forceinline__ u32x2 tr_read(const uint8_t *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// DMA of global memory into LDS (global_load_lds): lane i of the wave writes
// `bytes` bytes at dst + bytes*i; dst must be the same in every lane.  The
// loads are issued through inline assembly so that the compiler does not
// track them: every ring here synchronises them itself (wait_vm, then a
// barrier), whereas a DMA the compiler knows about makes it wait for all
// outstanding loads before each transposed LDS read, draining the ring.
// m0 is reserved by the compiler and cannot be named as a clobber; none of
// the kernels uses m0 otherwise (the generated code writes it only here).
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(uint8_t *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_u8 *)p);
}

// The DMA loads below take the LDS destination as a byte address in the LDS
// aperture (lds_addr of a pointer, or lds_addr(smem) plus a wave-uniform byte
// offset, which keeps the address arithmetic on the scalar unit).

// 16-byte DMA of `src` into LDS: lane i of the wave writes lds + 16*i.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma16(const void *src, uint8_t *dst) { dma16(src, lds_addr(dst)); }

// The same with a wave-uniform base address (scalar registers) and a 32-bit
// per-lane byte offset: no vector address arithmetic per load.
// `base` must be the same in every lane; it is read from the first lane.
__device__ __forceinline__ void dma16_s(const void *base, uint32_t off, uint32_t lds) {
    // readfirstlane returns int: widen through uint32_t, never by sign extension
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"((const void *)(uintptr_t)u),
                        "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma16_s(const void *base, uint32_t off, uint8_t *dst) {
    dma16_s(base, off, lds_addr(dst));
}

// A wave-uniform pointer moved to scalar registers (read from the first lane),
// so that values derived from it stay on the scalar unit.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return (T *)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// 4-byte DMA with a wave-uniform base and a 32-bit per-lane byte offset:
// lane i of the wave writes lds + 4*i.
__device__ __forceinline__ void dma4_s(const void *base, uint32_t off, uint32_t lds) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                     :: "v"(off), "s"((const void *)(uintptr_t)u),
                        "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// 4-byte DMA: lane i of the wave writes lds + 4*i.
__device__ __forceinline__ void dma4(const void *src, uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                     :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void *src, uint8_t *dst) { dma4(src, lds_addr(dst)); }

// Workgroups are dealt round-robin over the 8 XCDs (bid % 8).  Workgroup
// `bid` of a grid of heads * tiles -> (head, tile rank), rank 0 = the tile
// with the most work.  When the heads split evenly over the XCDs each XCD
// takes a contiguous range of heads, so that the tiles sharing a head's
// streamed operands share that XCD's L2.  The range is walked in groups of
// `group` heads (tile_group), rank-major inside a group: the heaviest tiles
// of the group's heads start first and the light ones fill the end, while the
// operands of only `group` heads are live in the L2 at a time.  (Head-major
// order, group = 1, leaves one slot of a CU running a head's heavy tiles while
// the other has finished: about a third of a causal dK/dV or dQ launch idled.)
struct TileId {
    uint32_t head, rank;
};
__host__ __device__ __forceinline__ TileId tile_order(uint32_t bid, uint32_t heads,
                                                      uint32_t tiles, uint32_t group) {
    uint32_t x = 0, r = bid, hx = heads;
    if (heads % 8u == 0) {
        x = bid % 8u;
        r = bid / 8u;
        hx = heads / 8u;
    }
    const uint32_t per = group * tiles;
    const uint32_t gi = r / per, w = r % per;
    return {x * hx + gi * group + w % group, w / group};
}

// Heads per group for tile_order: every head an XCD takes (all heads when
// they do not split over the XCDs).  Smaller groups, sized so that a group's
// K and V (or Q and dO) fit in half of an XCD's L2, cut the HBM re-reads of
// the causal d = 128 forward from 3.7x to about 1x the algorithmic bytes but
// measured slower in every pass (forward 562 vs 545 us, backward 297 vs
// 274 us): the balance of the launch matters more than the re-reads, which
// use HBM bandwidth the matrix-core-bound kernels leave idle.
#ifndef FA_TILE_GROUP  // heads per group (0: every head an XCD takes)
#define FA_TILE_GROUP 0
#endif
inline uint32_t tile_group(int64_t heads) {
    const int64_t per_xcd = heads % 8 == 0 ? heads / 8 : heads;
    if (FA_TILE_GROUP > 0 && per_xcd % FA_TILE_GROUP == 0) return (uint32_t)FA_TILE_GROUP;
    return (uint32_t)per_xcd;
}

}  // namespace fa
