// fa_naive.hip — attention the standard, unfused way: the N x N score and probability matrices go
// through HBM.  This is the implementation the pages measure the tiled method against (concept card
// "Worum es geht" and "Kernpunkte": the classic path writes the large score matrix to HBM and reads it
// back, several passes instead of about one; glossary "/02 Technische Vorteile im Überblick": the
// speed-up over it).  It is a measured comparison point, built from three kernels of its own:
//   1. naive_scores_kernel:  S = scale * Q K^T, float32, [B*H, N, ld]   (MFMA GEMM, 128 x 128 tiles,
//      computed as S^T blocks so that a lane stores 4 consecutive keys of a row at once)
//   2. naive_softmax_kernel: P = softmax(S [+ causal mask]) in the input dtype, lse per row (one wave
//      per row, the row held in registers; rows longer than 8192 are read twice)
//   3. naive_pv_kernel:      O = P V                               (MFMA GEMM, 128 rows x d per tile)
// Rows of S and P are ld = N rounded up to 64 elements apart; P is zero on the padding columns, so the
// second GEMM needs no masking.  Every (b, h, row) entry is computed; the causal mask is applied only in
// the softmax, as the standard implementation does.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kLog2eN = 1.4426950408889634f;
constexpr float kLn2N = 0.69314718055994531f;

// Tiles are row-major with the XOR chunk swizzle of the fused kernels (XorRows, fa_common.h).

// ---------------------------------------------------------------- 1. scores S = scale * Q K^T
template <typename T, int D>
struct Scores {
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    static constexpr int BM = 128, KC = 64, NKC = D / KC;
    static constexpr int TILE = BM * KC * 2;                 // 128 rows x 64 elements
    static constexpr int STAGE = 2 * TILE;                   // Q | K
    static constexpr int NSTAGE = NKC > 1 ? 2 : 1;
    static constexpr int LDS_BYTES = NSTAGE * STAGE;

    // rows [r0, r0 + 128), columns [kc*64, kc*64 + 64) of a [N, D] slice -> one tile (rows >= N repeat N - 1)
    static __device__ __forceinline__ void copy(const T* __restrict__ src, int r0, int N, int kc, uint32_t lds,
                                                int wave, int lane) {
        copy_tile<XorRows<8>, BM, 8, 256>(src + kc * KC, r0, N, D * 2, lds, wave * 64 + lane, wave);
    }

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K, float* __restrict__ S,
                                               int BH, int N, int ld, float scale, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const int nt = (N + BM - 1) / BM;
        int bh, tile;
        map_block(blockIdx.x, BH, nt * nt, false, bh, tile);
        const int m0 = (tile / nt) * BM, n0 = (tile % nt) * BM;
        const T* Qh = Q + (size_t)bh * N * D;
        const T* Kh = K + (size_t)bh * N * D;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        const int wm = wave & 1, wn = wave >> 1;   // this wave's 64 x 64 quarter of the 128 x 128 tile

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
        copy(Qh, m0, N, 0, base, wave, lane);
        copy(Kh, n0, N, 0, base + TILE, wave, lane);
        for (int kc = 0; kc < NKC; ++kc) {
            const int st = NSTAGE > 1 ? (kc & 1) : 0;
            wait_vmcnt<0>();
            lds_barrier();  // every wave's copies of chunk kc landed; chunk kc - 1's stage is free
            if (kc + 1 < NKC) {
                copy(Qh, m0, N, kc + 1, base + (st ^ 1) * STAGE, wave, lane);
                copy(Kh, n0, N, kc + 1, base + (st ^ 1) * STAGE + TILE, wave, lane);
            }
            const char* ql = smem + st * STAGE;
            const char* kl = ql + TILE;
#pragma unroll
            for (int ks = 0; ks < KC / 16; ++ks) {
                x8 a[2], b[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wm * 64 + i * 32 + n32;
                    a[i] = *(const x8*)(ql + XorRows<8>::slot(row, 2 * ks + h) * 16);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int row = wn * 64 + j * 32 + n32;
                    b[j] = *(const x8*)(kl + XorRows<8>::slot(row, 2 * ks + h) * 16);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = VT::mfma(b[j], a[i], acc[i][j]);
            }
        }
        // S^T blocks: register r of block (i, j) holds S[query][key] for query wm*64 + i*32 + n32 and
        // key wn*64 + j*32 + (r/4)*8 + h*4 + r%4, so 4 consecutive registers are 4 consecutive keys of a
        // row: one 16-byte store each (keys up to ld - 1 exist in every row; N..ld-1 are padding)
        float* Sh = S + (size_t)bh * N * ld;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int query = m0 + wm * 64 + i * 32 + n32;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int key = n0 + wn * 64 + j * 32 + g * 8 + h * 4;
                    if (query < N && key < N) {
                        f32x4 out;
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = acc[i][j][g * 4 + e] * scale;
                        *(f32x4*)(Sh + (size_t)query * ld + key) = out;
                    }
                }
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void naive_scores_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              float* __restrict__ S, int BH, int N, int ld, float scale) {
    __shared__ __attribute__((aligned(1024))) char smem[Scores<T, D>::LDS_BYTES];
    Scores<T, D>::run(Q, K, S, BH, N, ld, scale, smem);
}

// ---------------------------------------------------------------- 2. row softmax
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 v;
    v[0] = (T)a;
    v[1] = (T)b;
    v[2] = (T)c;
    v[3] = (T)d;
    *(t4*)p = v;
}

// One wave per row; lane l owns elements c*256 + 4l .. c*256 + 4l + 3 for c < NCH (NCH * 256 >= ld).
// Scores are taken to base 2 (x log2 e); key j of row i is visible iff j < N (and j <= i if causal).
template <typename T, int NCH, bool CAUSAL>
__global__ __launch_bounds__(256) void naive_softmax_kernel(const float* __restrict__ S, T* __restrict__ P,
                                                            float* __restrict__ lse, long long rows, int N, int ld) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = (int)(row % N);
    const int limit = CAUSAL ? i + 1 : N;
    const float* s = S + row * ld;
    T* p = P + row * ld;
    float v[NCH][4];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int pos = c * 256 + lane * 4;
        f32x4 x = f32x4{};
        if (pos < limit) x = *(const f32x4*)(s + pos);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[c][e] = pos + e < limit ? x[e] * kLog2eN : -INFINITY;
            m = fmaxf(m, v[c][e]);
        }
    }
    m = wave_max(m);  // finite: every row sees key 0
    float l = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[c][e] = fast_exp2(v[c][e] - m);
            l += v[c][e];
        }
    l = wave_sum(l);
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int pos = c * 256 + lane * 4;
        if (pos < ld) store4(p + pos, v[c][0] * inv, v[c][1] * inv, v[c][2] * inv, v[c][3] * inv);
    }
    if (lane == 0 && lse != nullptr) lse[row] = (m + __log2f(l)) * kLn2N;
}

// Rows too long for registers: a first pass keeps a running (max, sum) per lane, a second pass re-reads
// the row and writes P.
template <typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void naive_softmax_long_kernel(const float* __restrict__ S, T* __restrict__ P,
                                                                 float* __restrict__ lse, long long rows, int N, int ld) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = (int)(row % N);
    const int limit = CAUSAL ? i + 1 : N;
    const float* s = S + row * ld;
    T* p = P + row * ld;
    float m = -INFINITY, l = 0.0f;
    for (int pos = lane * 4; pos < limit; pos += 256) {
        const f32x4 x = *(const f32x4*)(s + pos);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (pos + e < limit) {
                const float y = x[e] * kLog2eN;
                const float mn = fmaxf(m, y);
                l = l * fast_exp2(m - mn) + fast_exp2(y - mn);
                m = mn;
            }
    }
    const float M = wave_max(m);
    const float L = wave_sum(m == -INFINITY ? 0.0f : l * fast_exp2(m - M));
    const float inv = 1.0f / L;
    for (int pos = lane * 4; pos < ld; pos += 256) {
        f32x4 x = f32x4{};
        if (pos < limit) x = *(const f32x4*)(s + pos);
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pos + e < limit ? fast_exp2(x[e] * kLog2eN - M) * inv : 0.0f;
        store4(p + pos, w[0], w[1], w[2], w[3]);
    }
    if (lane == 0 && lse != nullptr) lse[row] = (M + __log2f(L)) * kLn2N;
}

// ---------------------------------------------------------------- 3. O = P V
template <typename T, int D>
struct PV {
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    static constexpr int BM = 128, BN = 64, CPR = D / 8, CB = D / 32;
    static constexpr int PTILE = BM * BN * 2;                // 128 query rows x 64 keys
    static constexpr int VTILE = BN * D * 2;                 // 64 keys x D
    static constexpr int STAGE = PTILE + VTILE;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static constexpr int VLPT = BN * CPR / 256;              // V copies per lane per tile

    static __device__ __forceinline__ void copy(const T* __restrict__ Ph, const T* __restrict__ Vh, int q0, int k0,
                                                int N, int ld, uint32_t lds, int wave, int lane) {
        copy_tile<XorRows<8>, BM, 8, 256>(Ph + k0, q0, N, ld * 2, lds, wave * 64 + lane, wave);
        copy_tile<XorRows<CPR>, BN, CPR, 256>(Vh, k0, N, D * 2, lds + PTILE, wave * 64 + lane, wave);
    }

    static __device__ __forceinline__ void run(const T* __restrict__ P, const T* __restrict__ V, T* __restrict__ O,
                                               int BH, int N, int ld, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const int ntq = (N + BM - 1) / BM;
        int bh, qt;
        map_block(blockIdx.x, BH, ntq, false, bh, qt);
        const int q0 = qt * BM;
        const T* Ph = P + (size_t)bh * N * ld;
        const T* Vh = V + (size_t)bh * N * D;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        const int i16 = lane & 15, G = lane >> 4;
        const int vrow = (G >> 1) * 8 + (i16 >> 2), vcc = (G & 1) * 2 + ((i16 & 3) >> 1), vb = (i16 & 1) * 8;
        const int prow = wave * 32 + n32;

        f32x16 acc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
        const int ntile = ld / BN;
        copy(Ph, Vh, q0, 0, N, ld, base, wave, lane);
        for (int t = 0; t < ntile; ++t) {
            const int st = t & 1;
            wait_vmcnt<0>();
            lds_barrier();  // every wave's copies of tile t landed; tile t - 1's stage is free
            if (t + 1 < ntile) copy(Ph, Vh, q0, (t + 1) * BN, N, ld, base + (st ^ 1) * STAGE, wave, lane);
            const char* pl = smem + st * STAGE;
            const char* vl = pl + PTILE;
            // O^T += V^T P^T per 16 keys: lane (n32, h) supplies P[query n32][keys 16 sp + 8 h .. + 7]
#pragma unroll
            for (int sp = 0; sp < BN / 16; ++sp) {
                const x8 bp = *(const x8*)(pl + XorRows<8>::slot(prow, 2 * sp + h) * 16);
                const int row0 = sp * 16 + vrow, row1 = row0 + 4;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const x4 lo = VT::read_tr(vl + XorRows<CPR>::slot(row0, cb * 4 + vcc) * 16 + vb);
                    const x4 hi = VT::read_tr(vl + XorRows<CPR>::slot(row1, cb * 4 + vcc) * 16 + vb);
                    acc[cb] = VT::mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), bp, acc[cb]);
                }
            }
        }
        // register r of block cb holds O[q0 + wave*32 + n32][cb*32 + (r/4)*8 + h*4 + r%4]
        const int q = q0 + prow;
        if (q < N) {
            T* orow = O + ((size_t)bh * N + q) * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    store4(orow + cb * 32 + g * 8 + h * 4, acc[cb][g * 4], acc[cb][g * 4 + 1], acc[cb][g * 4 + 2],
                           acc[cb][g * 4 + 3]);
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void naive_pv_kernel(const T* __restrict__ P, const T* __restrict__ V,
                                                          T* __restrict__ O, int BH, int N, int ld) {
    __shared__ __attribute__((aligned(1024))) char smem[PV<T, D>::LDS_BYTES];
    PV<T, D>::run(P, V, O, BH, N, ld, smem);
}

// ---------------------------------------------------------------- launchers
template <typename T>
hipError_t scores_t(const void* q, const void* k, float* s, int BH, int N, int d, int ld, float scale,
                    hipStream_t stream) {
    const long long nt = (N + 127) / 128, nwg = (long long)BH * nt * nt;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg), block(256);
    switch (d) {
        case 64:
            hipLaunchKernelGGL((naive_scores_kernel<T, 64>), grid, block, 0, stream, (const T*)q, (const T*)k, s, BH, N, ld, scale);
            break;
        case 128:
            hipLaunchKernelGGL((naive_scores_kernel<T, 128>), grid, block, 0, stream, (const T*)q, (const T*)k, s, BH, N, ld, scale);
            break;
        case 256:
            hipLaunchKernelGGL((naive_scores_kernel<T, 256>), grid, block, 0, stream, (const T*)q, (const T*)k, s, BH, N, ld, scale);
            break;
        default:
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

template <typename T, bool CAUSAL>
hipError_t softmax_t(const float* s, void* p, float* lse, int BH, int N, int ld, hipStream_t stream) {
    const long long rows = (long long)BH * N, nwg = (rows + 3) / 4;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg), block(256);
    const int nch = (ld + 255) / 256;
    T* pp = (T*)p;
#define FA_NAIVE_SM(NC)                                                                                            \
    hipLaunchKernelGGL((naive_softmax_kernel<T, NC, CAUSAL>), grid, block, 0, stream, s, pp, lse, rows, N, ld); \
    break
    switch (nch <= 1 ? 1 : nch <= 2 ? 2 : nch <= 4 ? 4 : nch <= 8 ? 8 : nch <= 16 ? 16 : nch <= 32 ? 32 : 0) {
        case 1: FA_NAIVE_SM(1);
        case 2: FA_NAIVE_SM(2);
        case 4: FA_NAIVE_SM(4);
        case 8: FA_NAIVE_SM(8);
        case 16: FA_NAIVE_SM(16);
        case 32: FA_NAIVE_SM(32);
        default:
            hipLaunchKernelGGL((naive_softmax_long_kernel<T, CAUSAL>), grid, block, 0, stream, s, pp, lse, rows, N, ld);
    }
#undef FA_NAIVE_SM
    return hipGetLastError();
}

template <typename T>
hipError_t pv_t(const void* p, const void* v, void* o, int BH, int N, int d, int ld, hipStream_t stream) {
    const long long nwg = (long long)BH * ((N + 127) / 128);
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg), block(256);
    switch (d) {
        case 64:
            hipLaunchKernelGGL((naive_pv_kernel<T, 64>), grid, block, 0, stream, (const T*)p, (const T*)v, (T*)o, BH, N, ld);
            break;
        case 128:
            hipLaunchKernelGGL((naive_pv_kernel<T, 128>), grid, block, 0, stream, (const T*)p, (const T*)v, (T*)o, BH, N, ld);
            break;
        case 256:
            hipLaunchKernelGGL((naive_pv_kernel<T, 256>), grid, block, 0, stream, (const T*)p, (const T*)v, (T*)o, BH, N, ld);
            break;
        default:
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_naive_scores_16(bool is_bf16, const void* q, const void* k, float* s, int BH, int N, int d, int ld,
                                  float scale, hipStream_t stream) {
    return is_bf16 ? scores_t<__bf16>(q, k, s, BH, N, d, ld, scale, stream)
                   : scores_t<_Float16>(q, k, s, BH, N, d, ld, scale, stream);
}

hipError_t launch_naive_softmax_16(bool is_bf16, const float* s, void* p, float* lse, int BH, int N, int ld, bool causal,
                                   hipStream_t stream) {
    if (is_bf16)
        return causal ? softmax_t<__bf16, true>(s, p, lse, BH, N, ld, stream)
                      : softmax_t<__bf16, false>(s, p, lse, BH, N, ld, stream);
    return causal ? softmax_t<_Float16, true>(s, p, lse, BH, N, ld, stream)
                  : softmax_t<_Float16, false>(s, p, lse, BH, N, ld, stream);
}

hipError_t launch_naive_pv_16(bool is_bf16, const void* p, const void* v, void* o, int BH, int N, int d, int ld,
                              hipStream_t stream) {
    return is_bf16 ? pv_t<__bf16>(p, v, o, BH, N, d, ld, stream) : pv_t<_Float16>(p, v, o, BH, N, d, ld, stream);
}

}  // namespace fa
