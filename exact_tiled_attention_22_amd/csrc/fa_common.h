// fa_common.h — device-side helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const FA_LDS void*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the LDS pipeline.  Unlike __syncthreads() it does not wait for outstanding
// vector-memory loads (the prefetch of the next tile must stay in flight across it); callers wait
// for their own direct-to-LDS loads with wait_vmcnt first.  Pending LDS reads are drained, and the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Value of lane (l ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) {
    return __shfl_xor(x, 32, 64);
}

// max / sum of x over lanes l and l ^ 32 (gfx950 v_permlane32_swap: the upper half of the first
// register trades places with the lower half of the second).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-byte direct HBM->LDS copy per lane: lane l writes LDS bytes [m0 + 16 l, m0 + 16 l + 16).
// Issued as inline assembly so that the compiler does not treat the in-flight copy as a pending
// LDS write (it would otherwise wait for every outstanding copy before each LDS read); the
// caller waits with wait_vmcnt before a barrier.  lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base));
}

// Same copy with a wave-uniform 64-bit base (scalar registers) and a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_base));
}

// The same with the non-temporal hint, for data that is read exactly once (the decode path's key/value
// cache: bf16 B8 H32 Nq8 Nk32768 d128 723.8 -> 624.2 us).  Tiles that other workgroups read again
// from L2 keep the default policy.
__device__ __forceinline__ void dma16s_nt(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_base));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of three floats (one v_max3_f32).
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Round-to-nearest-even packing of 8 floats into the MFMA operand of type T.
template <typename T> struct Vec;
template <> struct Vec<__bf16> {
    typedef bf16x8 x8;
    typedef bf16x4 x4;
    __device__ static __forceinline__ x8 pack(const float* f) {
        x8 r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
        return r;
    }
    __device__ static __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ x4 read_tr(const void* lds) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS x4*)lds);
    }
};
template <> struct Vec<_Float16> {
    typedef f16x8 x8;
    typedef f16x4 x4;
    __device__ static __forceinline__ x8 pack(const float* f) {
        x8 r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (_Float16)f[i];
        return r;
    }
    __device__ static __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ x4 read_tr(const void* lds) {
        typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
        return __builtin_bit_cast(x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((FA_LDS h4*)lds));
    }
};

// ---- LDS tile layouts ----
// A tile holds rows of CPR 16-byte chunks.  The LDS serves 16 groups of 16 bytes per clock; the kernels'
// operand fetches must each hit 16 distinct groups:
//   * a score-style fetch: 16 lanes read one logical chunk of 16 consecutive rows;
//   * a transposing fetch (ds_read_b64_tr_*): 32 lanes read 4 logical chunks of 4 consecutive rows
//     (row % 4 == 0).
//
// Row-major rows with an XOR swizzle: chunk c of row r sits at slot r * CPR + (c ^ xswz<CPR>(r)).  Rows
// of 256 or 512 bytes start in group 0, so the group is the physical chunk mod 16: swapping the two
// 2-bit halves of (row mod 16) serves both fetches.  Rows of 128 bytes alternate between groups 0
// and 8, so the parity of the row already separates pairs and 3 bits suffice.
template <int CPR>
__device__ __forceinline__ int xswz(int row) {
    if constexpr (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int CPR>
struct XorRows {
    static constexpr int ROW_CHUNKS = CPR;
    __device__ static __forceinline__ int slot(int row, int c) { return row * CPR + (c ^ xswz<CPR>(row)); }
    __device__ static __forceinline__ void row_chunk(int slot, int& row, int& c) {
        row = slot / CPR;
        c = (slot % CPR) ^ xswz<CPR>(row);
    }
};

// Direct HBM->LDS copy of rows [r0, r0 + ROWS) of a row-major slice of N rows, `stride` bytes apart, of
// which the first CPR 16-byte chunks are copied into a tile laid out by L, with THREADS threads: copy
// instruction t of wave w fills LDS slots [t * THREADS + 64 w, + 64).  Rows past N - 1 repeat row N - 1
// (their results are masked or never stored).  `src` is the slice's first row, `lds` the tile's base;
// NT marks data read only once (dma16s_nt).
template <class L, int ROWS, int CPR, int THREADS, bool NT = false>
__device__ __forceinline__ void copy_tile(const void* __restrict__ src, int r0, int N, int stride, uint32_t lds,
                                          int tid, int wave) {
    constexpr int NL = ROWS * CPR / THREADS;
    static_assert(ROWS * CPR % THREADS == 0, "the tile splits evenly over the threads");
    const char* base = (const char*)src + (size_t)r0 * stride;
    const int lim = min(ROWS, N - r0) - 1;  // last row of the slice inside this tile (wave-uniform)
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        int row, c;
        L::row_chunk(t * THREADS + tid, row, c);
        const uint32_t off = (uint32_t)(min(row, lim) * stride + c * 16), dst = lds + (uint32_t)((t * THREADS + wave * 64) * 16);
        if constexpr (NT) dma16s_nt(base, off, dst);
        else dma16s(base, off, dst);
    }
}

// The per-thread byte offsets of copy_tile's full-tile copies (the same for every full tile) ...
template <class L, int ROWS, int CPR, int THREADS>
__device__ __forceinline__ void tile_offsets(int stride, int tid, uint32_t (&off)[ROWS * CPR / THREADS]) {
#pragma unroll
    for (int t = 0; t < ROWS * CPR / THREADS; ++t) {
        int row, c;
        L::row_chunk(t * THREADS + tid, row, c);
        off[t] = (uint32_t)(row * stride + c * 16);
    }
}

// ... and a full-tile copy from them: no vector instructions per copy.
template <int NL, int THREADS>
__device__ __forceinline__ void copy_tile_full(const void* __restrict__ src_tile, uint32_t lds, int wave,
                                               const uint32_t (&off)[NL]) {
#pragma unroll
    for (int t = 0; t < NL; ++t) dma16s(src_tile, off[t], lds + (uint32_t)((t * THREADS + wave * 64) * 16));
}

// ---- output staging: a wave's 32 x D output tile of 2-byte elements through LDS ----
// The matrix accumulator leaves a lane with 4-column pieces of one row (32 rows per register), so
// stores straight from registers would touch 32 rows with 8 bytes per lane.  Staged in the wave's own
// LDS region (row r at r * 2D bytes, 16-byte chunk c at physical chunk c ^ xswz(r)), the tile
// leaves as whole rows: one 16-byte-per-lane store covers 64 / (D / 8) rows of contiguous output.
// The swizzle (xswz) spreads the 16 rows of one 8-byte-per-lane write, and the rows of one 16-byte read,
// over distinct 16-byte bank groups of the 64-bank LDS.

// Lane (row n32, half h) writes its 4 elements of columns 8 * chunk + 4 * h + 0..3.
template <int D, typename X4>
__device__ __forceinline__ void ostage_put(char* wl, int n32, int h, int chunk, const X4& val) {
    static_assert(sizeof(X4) == 8, "four 2-byte elements");
    *(X4*)(wl + n32 * (2 * D) + (chunk ^ xswz<D / 8>(n32)) * 16 + h * 8) = val;
}

// After every lane of the wave has put its pieces: rows row0 + r (r < 32, row0 + r < nrows) of dst.
template <typename T, int D>
__device__ __forceinline__ void ostage_flush(T* __restrict__ dst, int row0, int nrows, const char* wl, int lane) {
    constexpr int CPR = D / 8, RPS = 64 / CPR;
    // the wave's own LDS writes land before its lanes read each other's rows back
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 32 / RPS; ++i) {
        const int r = i * RPS + lane / CPR, c = lane % CPR;
        const i32x4 val = *(const i32x4*)(wl + r * (2 * D) + (c ^ xswz<CPR>(r)) * 16);
        if (row0 + r < nrows) *(i32x4*)(dst + (size_t)(row0 + r) * D + c * 8) = val;
    }
}

// Work partition: block id -> (head slice bh, query tile qt).
// Consecutive block ids are dispatched round-robin over the 8 XCDs (each with its own L2), so when
// B*H is a multiple of 8 every XCD is given whole heads: all query tiles of a head then read that
// head's K/V through one L2.  Causal grids run the longest query tiles (most key tiles) first.
__device__ __forceinline__ void map_block(int bid, int BH, int ntq, bool causal, int& bh, int& qt) {
    if ((BH & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
        if (causal) {
            qt = ntq - 1 - slot / hpx;
            bh = xcd * hpx + slot % hpx;
        } else {
            bh = xcd * hpx + slot / ntq;
            qt = slot % ntq;
        }
    } else if (causal) {
        qt = ntq - 1 - bid / BH;
        bh = bid % BH;
    } else {
        bh = bid / ntq;
        qt = bid % ntq;
    }
}

}  // namespace fa
