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
// HBM-bound: one workgroup per block reads the block once (each lane 16 or 32 contiguous bytes per
// row), keeps it in registers when it fits (otherwise re-reads it, from L2), and writes the codes
// with 8-byte stores.  Rows past N are not read or written.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kCachePasses = 8;  // blocks of up to 8 row-passes stay in registers

template <typename Tin>
__device__ __forceinline__ void load8(const Tin* p, float* f);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
}
template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float* f) {
    const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)a[i];
}
template <>
__device__ __forceinline__ void load8<_Float16>(const _Float16* p, float* f) {
    const f16x8 a = *(const f16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)a[i];
}

// Rotate 8 consecutive elements of a row held by one lane; the row spans L = D/8 lanes.
template <int D>
__device__ __forceinline__ void rotate8(float* x, uint32_t sign8, int li, float rs) {
    // sign flip (exact); bit e of sign8 = column li*8 + e is negated
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if ((sign8 >> e) & 1) x[e] = -x[e];
    // in-lane butterflies, strides 1, 2, 4
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((e & hs) == 0) {
                const float a = x[e], b = x[e + hs];
                x[e] = a + b;
                x[e + hs] = a - b;
            }
        }
    }
    // cross-lane butterflies, strides 8, 16, ..., D/2 (partner lane li ^ (stride / 8))
#pragma unroll
    for (int ls = 1; ls < D / 8; ls <<= 1) {
        const bool upper = (li & ls) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float other = __shfl_xor(x[e], ls, 64);
            x[e] = upper ? (other - x[e]) : (x[e] + other);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * rs;
}

template <typename Tin, int D, bool ROT, bool CACHE>
__global__ __launch_bounds__(kThreads) void fp8_prep_kernel(const Tin* __restrict__ X, uint8_t* __restrict__ X8,
                                                            float* __restrict__ S, int N, int block, int nblk,
                                                            float rs, uint64_t s0, uint64_t s1, uint64_t s2,
                                                            uint64_t s3) {
    constexpr int L = D / 8;             // lanes per row
    constexpr int RP = kThreads / L;     // rows per pass
    __shared__ float red[kThreads / 64];
    const int tid = threadIdx.x;
    const int li = tid % L;              // position of this lane's 8 columns in the row
    const uint64_t sw = li < 8 ? s0 : li < 16 ? s1 : li < 24 ? s2 : s3;
    const uint32_t sign8 = (uint32_t)(sw >> ((li & 7) * 8)) & 0xFFu;
    const int rsub = tid / L;            // row within a pass
    const int bh = blockIdx.x / nblk, bi = blockIdx.x % nblk;
    const int r0 = bi * block;
    const int rows = min(block, N - r0);
    const int passes = (rows + RP - 1) / RP;
    const size_t base = ((size_t)bh * N + r0) * D + li * 8;

    float cache[CACHE ? kCachePasses : 1][8];
    float amax = 0.0f;
    for (int p = 0; p < (CACHE ? kCachePasses : passes); ++p) {
        if (CACHE && p >= passes) break;
        const int r = p * RP + rsub;
        float x[8];
        if (r < rows) {
            load8<Tin>(X + base + (size_t)r * D, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
        if (ROT) rotate8<D>(x, sign8, li, rs);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
        if (CACHE) {
#pragma unroll
            for (int e = 0; e < 8; ++e) cache[p][e] = x[e];
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

    for (int p = 0; p < (CACHE ? kCachePasses : passes); ++p) {
        if (CACHE && p >= passes) break;
        const int r = p * RP + rsub;
        if (r >= rows) continue;
        float x[8];
        if (CACHE) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = cache[p][e];
        } else {
            load8<Tin>(X + base + (size_t)r * D, x);
            if (ROT) rotate8<D>(x, sign8, li, rs);
        }
        i32x2 packed = {0, 0};
        if (!zero) {
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[e] * inv, -448.0f), 448.0f);
            int w0 = 0, w1 = 0;
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], w1, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
            packed = i32x2{w0, w1};
        }
        *(i32x2*)(X8 + base + (size_t)r * D) = packed;
    }
}

template <typename Tin, int D, bool ROT>
hipError_t launch_prep_t(const void* x, void* x8, float* scales, int block, int BH, int N, float rs,
                         const uint64_t* sb, hipStream_t stream) {
    constexpr int RP = kThreads / (D / 8);
    const int nblk = (N + block - 1) / block;
    const long long nwg = (long long)BH * nblk;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool cache = (block + RP - 1) / RP <= kCachePasses;
    if (cache)
        hipLaunchKernelGGL((fp8_prep_kernel<Tin, D, ROT, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                           (const Tin*)x, (uint8_t*)x8, scales, N, block, nblk, rs, sb[0], sb[1], sb[2], sb[3]);
    else
        hipLaunchKernelGGL((fp8_prep_kernel<Tin, D, ROT, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                           (const Tin*)x, (uint8_t*)x8, scales, N, block, nblk, rs, sb[0], sb[1], sb[2], sb[3]);
    return hipGetLastError();
}

template <typename Tin, int D>
hipError_t launch_prep_d(const void* x, void* x8, float* scales, bool rot, int block, int BH, int N, float rs,
                         const uint64_t* sb, hipStream_t stream) {
    return rot ? launch_prep_t<Tin, D, true>(x, x8, scales, block, BH, N, rs, sb, stream)
               : launch_prep_t<Tin, D, false>(x, x8, scales, block, BH, N, rs, sb, stream);
}

template <typename Tin>
hipError_t launch_prep_dt(const void* x, void* x8, float* scales, bool rot, int block, int BH, int N, int d,
                          float rs, const uint64_t* sb, hipStream_t stream) {
    switch (d) {
        case 64: return launch_prep_d<Tin, 64>(x, x8, scales, rot, block, BH, N, rs, sb, stream);
        case 128: return launch_prep_d<Tin, 128>(x, x8, scales, rot, block, BH, N, rs, sb, stream);
        case 256: return launch_prep_d<Tin, 256>(x, x8, scales, rot, block, BH, N, rs, sb, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_fp8_prep(const void* x, int x_dtype, void* x8, float* scales, bool rotate,
                           const uint64_t sign_bits[4], int block, int BH, int N, int d, hipStream_t stream) {
    // float32 value of 1/sqrt(d): the double quotient rounded once to float
    const float rs = (float)(1.0 / __builtin_sqrt((double)d));
    switch (x_dtype) {
        case 0: return launch_prep_dt<float>(x, x8, scales, rotate, block, BH, N, d, rs, sign_bits, stream);
        case 1: return launch_prep_dt<_Float16>(x, x8, scales, rotate, block, BH, N, d, rs, sign_bits, stream);
        case 2: return launch_prep_dt<__bf16>(x, x8, scales, rotate, block, BH, N, d, rs, sign_bits, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace fa
