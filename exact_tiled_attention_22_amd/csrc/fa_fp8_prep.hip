// fa_fp8_prep.hip — block absmax quantisation to OCP e4m3 with an optional Hadamard rotation.
//
// FlashAttention-3 article, "Drei technische Hebel", item 3 "FP8-Blockquantisierung" (operands in
// eight bits, block by block, with a Hadamard transform against quantisation error) and concept card
// "FlashAttention 2 + 3 — speicherbewusste Attention-Kernels", "Kernpunkte" (absmax scaling).
//
// Per (b,h) slice and block of `block` rows:  x' = (x * s) H_d / sqrt(d)  (or x' = x without signs),
// amax = max |x'|, scale = amax / 448, code = e4m3_RNE(x' * (448 / amax)).  The arithmetic is float32
// in a fixed order (butterfly strides 1, 2, ..., d/2, each mapping (a, b) to (a + b, a - b); then a
// multiply by float32(1/sqrt(d)); a division 448/amax; a multiply; the e4m3 conversion), so the codes
// are a deterministic function of the input bits.
//
// HBM-bound.  Each lane owns 32 contiguous columns of one row (d/32 lanes per row), so the butterflies
// with strides 1..16 stay inside the lane and the remaining one to three stages are DPP lane swaps
// inside a quad / half-row.  A 256-thread workgroup covers 256*32/d rows per pass (64 for d = 128,
// i.e. one whole 64-row block), loads it with 16-byte vector loads, keeps it in registers (up to two
// passes), reduces the block maximum, and stores the codes with 16-byte stores.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kEPL = 32;          // elements per lane
constexpr int kCachePasses = 2;   // blocks of up to 2 row-passes stay in registers

// Sign flips of the random +/-1 vector, as XOR masks on the raw input words: for lane position li and
// 32-bit word k (elements 2k, 2k+1 of the lane's 32 columns), bit 15 flips element 2k and bit 31
// flips element 2k+1.  A sign flip is exact, so (x * s) equals x with its sign bit toggled.
struct SignMasks {
    uint32_t w[8][16];
};

// Load the lane's 32 consecutive elements (optionally sign-flipped) as float32.
template <typename Tin, bool ROT>
__device__ __forceinline__ void load32(const Tin* p, const uint32_t* m, float* f);
template <>
__device__ __forceinline__ void load32<float, false>(const float* p, const uint32_t*, float* f) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const f32x4 a = *(const f32x4*)(p + 4 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[4 * v + i] = a[i];
    }
}
template <>
__device__ __forceinline__ void load32<float, true>(const float* p, const uint32_t* m, float* f) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const i32x4 a = *(const i32x4*)(p + 4 * v);
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const uint32_t mk = m[2 * v + i / 2];
            f[4 * v + i] = __uint_as_float((uint32_t)a[i] ^ (mk << 16));
            f[4 * v + i + 1] = __uint_as_float((uint32_t)a[i + 1] ^ (mk & 0x80000000u));
        }
    }
}
template <bool ROT>
__device__ __forceinline__ void load32_bf16(const __bf16* p, const uint32_t* m, float* f) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const i32x4 a = *(const i32x4*)(p + 8 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t wd = ROT ? ((uint32_t)a[i] ^ m[4 * v + i]) : (uint32_t)a[i];
            f[8 * v + 2 * i] = __uint_as_float(wd << 16);
            f[8 * v + 2 * i + 1] = __uint_as_float(wd & 0xffff0000u);
        }
    }
}
template <bool ROT>
__device__ __forceinline__ void load32_f16(const _Float16* p, const uint32_t* m, float* f) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const i32x4 a = *(const i32x4*)(p + 8 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t wd = ROT ? ((uint32_t)a[i] ^ m[4 * v + i]) : (uint32_t)a[i];
            f[8 * v + 2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd & 0xffffu));
            f[8 * v + 2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> 16));
        }
    }
}
template <>
__device__ __forceinline__ void load32<__bf16, false>(const __bf16* p, const uint32_t* m, float* f) {
    load32_bf16<false>(p, m, f);
}
template <>
__device__ __forceinline__ void load32<__bf16, true>(const __bf16* p, const uint32_t* m, float* f) {
    load32_bf16<true>(p, m, f);
}
template <>
__device__ __forceinline__ void load32<_Float16, false>(const _Float16* p, const uint32_t* m, float* f) {
    load32_f16<false>(p, m, f);
}
template <>
__device__ __forceinline__ void load32<_Float16, true>(const _Float16* p, const uint32_t* m, float* f) {
    load32_f16<true>(p, m, f);
}

// value of lane (l ^ M) for M = 1, 2 (quad permutes).  Every source lane lies in the same quad, so
// the zero-fill flag never applies; it lets the compiler fold the move into the add that consumes it.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
    const int v = __float_as_int(x);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
    return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
}

// Walsh-Hadamard transform of a row whose 32-column pieces sit in consecutive lanes (this lane is
// piece li): butterflies of strides 1..16 inside the lane, strides 32, 64, 128 across lanes, then the
// 1/sqrt(d) factor.  Across lanes the lower piece forms other + x and the upper piece other + (-x),
// which is the same IEEE operation as other - x.
template <int D>
__device__ __forceinline__ void hadamard32(float* x, int li, float rs) {
#pragma unroll
    for (int hs = 1; hs < kEPL; hs <<= 1) {
#pragma unroll
        for (int e = 0; e < kEPL; ++e) {
            if ((e & hs) == 0) {
                const float a = x[e], b = x[e + hs];
                x[e] = a + b;
                x[e + hs] = a - b;
            }
        }
    }
    // each pass first forms all 32 operands, then all 32 DPP adds: a DPP read of a register written
    // by the instruction just before it would cost two wait states
    auto cross = [&](auto tag) {
        constexpr int M = decltype(tag)::value;
        const uint32_t neg = (li & M) ? 0x80000000u : 0u;
        float own[kEPL];
#pragma unroll
        for (int e = 0; e < kEPL; ++e) own[e] = __uint_as_float(__float_as_uint(x[e]) ^ neg);
        if constexpr (M == 4) {
            // half-row mirror first (lane i reads 7 - i), the quad reversal is folded into the add
#pragma unroll
            for (int e = 0; e < kEPL; ++e)
                x[e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[e]), 0x141, 0xF, 0xF, true));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < kEPL; ++e)
                x[e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[e]), 0x1B, 0xF, 0xF, true)) + own[e];
        } else {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < kEPL; ++e) x[e] = lane_xor<M>(x[e]) + own[e];
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (D >= 64) cross(std::integral_constant<int, 1>{});
    if constexpr (D >= 128) cross(std::integral_constant<int, 2>{});
    if constexpr (D >= 256) cross(std::integral_constant<int, 4>{});
#pragma unroll
    for (int e = 0; e < kEPL; ++e) x[e] = x[e] * rs;
}

// One block of `block` rows (block bi of slice bh) by one workgroup.
template <typename Tin, int D, bool ROT, bool CACHE>
__device__ __forceinline__ void prep_block(const Tin* __restrict__ X, uint8_t* __restrict__ X8, float* __restrict__ S,
                                           int N, int block, int nblk, float rs, const SignMasks& sm, int bh, int bi,
                                           float* red) {
    constexpr int LPR = D / kEPL;        // lanes per row
    constexpr int RP = kThreads / LPR;   // rows per pass
    const int tid = threadIdx.x;
    const int li = tid % LPR;            // this lane holds columns li*32 .. li*32+31
    uint32_t mask[16];
    if constexpr (ROT) {
#pragma unroll
        for (int k = 0; k < 16; k += 4) {
            const i32x4 t = *(const i32x4*)&sm.w[li][k];
#pragma unroll
            for (int i = 0; i < 4; ++i) mask[k + i] = (uint32_t)t[i];
        }
    }
    const int rsub = tid / LPR;          // row within a pass
    const int r0 = bi * block;
    const int rows = min(block, N - r0);
    const int passes = (rows + RP - 1) / RP;
    const size_t base = ((size_t)bh * N + r0) * D + li * kEPL;

    float cache[CACHE ? kCachePasses : 1][kEPL];
    float amax = 0.0f;
    // rows past the end of the block re-read the block's last row: the block maximum is unchanged
    // and their codes are not stored
    auto load_rot = [&](int p, float* x) {
        const int r = min(p * RP + rsub, rows - 1);
        load32<Tin, ROT>(X + base + (size_t)r * D, mask, x);
        if (ROT) hadamard32<D>(x, li, rs);
    };
    if constexpr (CACHE) {
#pragma unroll
        for (int p = 0; p < kCachePasses; ++p) {
            if (p < passes) {
                load_rot(p, cache[p]);
#pragma unroll
                for (int e = 0; e < kEPL; ++e) amax = fmaxf(amax, fabsf(cache[p][e]));
            }
        }
    } else {
        for (int p = 0; p < passes; ++p) {
            float x[kEPL];
            load_rot(p, x);
#pragma unroll
            for (int e = 0; e < kEPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
        }
    }
    // block-wide max
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) amax = fmaxf(amax, red[w]);

    const bool zero = amax == 0.0f;
    const float safe = zero ? 1.0f : amax;
    const float inv = fminf(448.0f / safe, 3.402823466e38f);
    if (tid == 0) S[(size_t)bh * nblk + bi] = zero ? 1.0f : safe / 448.0f;

    auto store = [&](int p, const float* x) {
        const int r = p * RP + rsub;
        if (r >= rows) return;
        i32x4 q[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
        if (!zero) {
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * w + e] * inv, -448.0f), 448.0f);
                int wd = 0;
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], wd, false);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wd, true);
                q[w >> 2][w & 3] = wd;
            }
        }
        // the codes are written once and read by a later launch: non-temporal stores (e4m3 B4 H16 N4096
        // d128, Q/K/V in one launch: 56.1 -> 50.9 us; non-temporal loads of the input made it slower)
        i32x4* dst = (i32x4*)(X8 + base + (size_t)r * D);
        __builtin_nontemporal_store(q[0], dst);
        __builtin_nontemporal_store(q[1], dst + 1);
    };
    if constexpr (CACHE) {
#pragma unroll
        for (int p = 0; p < kCachePasses; ++p)
            if (p < passes) store(p, cache[p]);
    } else {
        for (int p = 0; p < passes; ++p) {
            float x[kEPL];
            load_rot(p, x);
            store(p, x);
        }
    }
}

template <typename Tin, int D, bool ROT, bool CACHE>
__global__ __launch_bounds__(kThreads) void fp8_prep_kernel(const Tin* __restrict__ X, uint8_t* __restrict__ X8,
                                                            float* __restrict__ S, int N, int block, int nblk,
                                                            float rs, SignMasks sm) {
    __shared__ float red[kThreads / 64];
    prep_block<Tin, D, ROT, CACHE>(X, X8, S, N, block, nblk, rs, sm, blockIdx.x / nblk, blockIdx.x % nblk, red);
}

// Q, K and V of one attention call in one launch: Q and K rotated with the same signs (when ROT), V
// not.  Consecutive workgroups take the same block of Q, K and V, so the butterfly-heavy Q and K blocks
// and the plain V blocks share every CU.
struct Prep3 {
    const void* x[3];
    uint8_t* x8[3];
    float* s[3];
};

template <typename Tin, int D, bool ROT, bool CACHE>
__global__ __launch_bounds__(kThreads) void fp8_prep_qkv_kernel(Prep3 a, int N, int block, int nblk, float rs,
                                                                SignMasks sm) {
    __shared__ float red[kThreads / 64];
    const int t = blockIdx.x % 3, idx = blockIdx.x / 3;
    const int bh = idx / nblk, bi = idx % nblk;
    if (t < 2)
        prep_block<Tin, D, ROT, CACHE>((const Tin*)a.x[t], a.x8[t], a.s[t], N, block, nblk, rs, sm, bh, bi, red);
    else
        prep_block<Tin, D, false, CACHE>((const Tin*)a.x[2], a.x8[2], a.s[2], N, block, nblk, rs, sm, bh, bi, red);
}

template <typename Tin, int D, bool ROT>
hipError_t launch_prep_qkv_t(const Prep3& a, int block, int BH, int N, float rs, const SignMasks& sm,
                             hipStream_t stream) {
    constexpr int RP = kThreads / (D / kEPL);
    const int nblk = (N + block - 1) / block;
    const long long nwg = 3LL * BH * nblk;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    if ((block + RP - 1) / RP <= kCachePasses)
        hipLaunchKernelGGL((fp8_prep_qkv_kernel<Tin, D, ROT, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, a,
                           N, block, nblk, rs, sm);
    else
        hipLaunchKernelGGL((fp8_prep_qkv_kernel<Tin, D, ROT, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                           a, N, block, nblk, rs, sm);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_prep_qkv_dt(const Prep3& a, bool rot, int block, int BH, int N, int d, float rs,
                              const SignMasks& sm, hipStream_t stream) {
    switch (d) {
        case 64: return rot ? launch_prep_qkv_t<Tin, 64, true>(a, block, BH, N, rs, sm, stream)
                            : launch_prep_qkv_t<Tin, 64, false>(a, block, BH, N, rs, sm, stream);
        case 128: return rot ? launch_prep_qkv_t<Tin, 128, true>(a, block, BH, N, rs, sm, stream)
                             : launch_prep_qkv_t<Tin, 128, false>(a, block, BH, N, rs, sm, stream);
        case 256: return rot ? launch_prep_qkv_t<Tin, 256, true>(a, block, BH, N, rs, sm, stream)
                             : launch_prep_qkv_t<Tin, 256, false>(a, block, BH, N, rs, sm, stream);
        default: return hipErrorNotSupported;
    }
}

template <typename Tin, int D, bool ROT>
hipError_t launch_prep_t(const void* x, void* x8, float* scales, int block, int BH, int N, float rs,
                         const SignMasks& sm, hipStream_t stream) {
    constexpr int RP = kThreads / (D / kEPL);
    const int nblk = (N + block - 1) / block;
    const long long nwg = (long long)BH * nblk;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool cache = (block + RP - 1) / RP <= kCachePasses;
    if (cache)
        hipLaunchKernelGGL((fp8_prep_kernel<Tin, D, ROT, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                           (const Tin*)x, (uint8_t*)x8, scales, N, block, nblk, rs, sm);
    else
        hipLaunchKernelGGL((fp8_prep_kernel<Tin, D, ROT, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                           (const Tin*)x, (uint8_t*)x8, scales, N, block, nblk, rs, sm);
    return hipGetLastError();
}

template <typename Tin, int D>
hipError_t launch_prep_d(const void* x, void* x8, float* scales, bool rot, int block, int BH, int N, float rs,
                         const SignMasks& sm, hipStream_t stream) {
    return rot ? launch_prep_t<Tin, D, true>(x, x8, scales, block, BH, N, rs, sm, stream)
               : launch_prep_t<Tin, D, false>(x, x8, scales, block, BH, N, rs, sm, stream);
}

template <typename Tin>
hipError_t launch_prep_dt(const void* x, void* x8, float* scales, bool rot, int block, int BH, int N, int d,
                          float rs, const SignMasks& sm, hipStream_t stream) {
    switch (d) {
        case 64: return launch_prep_d<Tin, 64>(x, x8, scales, rot, block, BH, N, rs, sm, stream);
        case 128: return launch_prep_d<Tin, 128>(x, x8, scales, rot, block, BH, N, rs, sm, stream);
        case 256: return launch_prep_d<Tin, 256>(x, x8, scales, rot, block, BH, N, rs, sm, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

namespace {
SignMasks sign_masks(const uint64_t sign_bits[4]) {
    SignMasks sm{};
    for (int t = 0; t < 256; ++t) {
        if ((sign_bits[t >> 6] >> (t & 63)) & 1) {
            const int li = t / kEPL, e = t % kEPL;
            sm.w[li][e >> 1] |= (e & 1) ? 0x80000000u : 0x00008000u;
        }
    }
    return sm;
}
// float32 value of 1/sqrt(d): the double quotient rounded once to float
float inv_sqrt_d(int d) { return (float)(1.0 / __builtin_sqrt((double)d)); }
}  // namespace

hipError_t launch_fp8_prep_qkv(const void* const x[3], int x_dtype, void* const x8[3], float* const scales[3],
                               bool rotate, const uint64_t sign_bits[4], int block, int BH, int N, int d,
                               hipStream_t stream) {
    const SignMasks sm = sign_masks(sign_bits);
    Prep3 a;
    for (int t = 0; t < 3; ++t) {
        a.x[t] = x[t];
        a.x8[t] = static_cast<uint8_t*>(x8[t]);
        a.s[t] = scales[t];
    }
    const float rs = inv_sqrt_d(d);
    switch (x_dtype) {
        case 0: return launch_prep_qkv_dt<float>(a, rotate, block, BH, N, d, rs, sm, stream);
        case 1: return launch_prep_qkv_dt<_Float16>(a, rotate, block, BH, N, d, rs, sm, stream);
        case 2: return launch_prep_qkv_dt<__bf16>(a, rotate, block, BH, N, d, rs, sm, stream);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_fp8_prep(const void* x, int x_dtype, void* x8, float* scales, bool rotate,
                           const uint64_t sign_bits[4], int block, int BH, int N, int d, hipStream_t stream) {
    const float rs = inv_sqrt_d(d);
    const SignMasks sm = sign_masks(sign_bits);
    switch (x_dtype) {
        case 0: return launch_prep_dt<float>(x, x8, scales, rotate, block, BH, N, d, rs, sm, stream);
        case 1: return launch_prep_dt<_Float16>(x, x8, scales, rotate, block, BH, N, d, rs, sm, stream);
        case 2: return launch_prep_dt<__bf16>(x, x8, scales, rotate, block, BH, N, d, rs, sm, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace fa
