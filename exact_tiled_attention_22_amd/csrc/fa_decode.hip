// fa_decode.hip — attention for a few queries against a long cached key/value sequence (decode).
//
// The pages tie the method's memory savings to longer key/value caches at serving time (Flash Attention
// glossary, "/02 Warum ist Flash Attention wichtig?": bigger caches and longer context on the same
// GPU; concept card "Kernpunkte": activation memory at 4k context).  With Nq <= 32 queries per (b, h)
// there is no query tiling to spread over the chip, so the keys are split instead:
//   1. decode_split_kernel: every wave of every workgroup owns one contiguous chunk of the keys of one
//      (b, h) and runs the forward pass's tile loop over it (32-key tiles through the wave's own two
//      LDS stages, scores S^T = K Q^T, online softmax in base 2, O^T += V^T P^T), then stores its
//      partial result: O_c (normalised, float32) and lse_c = m + log2 l (base 2) per query;
//   2. decode_merge_kernel: per (b, h, query), lse = log2 sum_c 2^lse_c and O = sum_c 2^(lse_c - lse) O_c,
//      which is the same softmax over the union of the chunks.
// The waves share nothing, so there is no workgroup barrier; each waits only for its own copies.
// Causal: query i (of Nq) sees keys j <= i + Nk - Nq (the queries are the last Nq positions).
#include <mutex>
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kTauD = 8.0f;  // lazy rescale threshold (log2 units), as in the forward pass

template <typename T, int D, bool CAUSAL>
struct Decode {
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    // waves per workgroup: each wave owns 4 tiles of LDS (64 KiB at d = 256, so two waves there)
    static constexpr int NW = D >= 256 ? 2 : 4, BN = 32, CPR = D / 8, KS = D / 16, CB = D / 32;
    static constexpr int TILE = BN * CPR * 16;           // one K or V tile
    static constexpr int WAVE_LDS = 4 * TILE;             // K0 | V0 | K1 | V1 per wave
    static constexpr int LDS_BYTES = NW * WAVE_LDS;
    static constexpr int LPT = BN * CPR / 64;             // copies per lane per tile

    // copy rows [r0, r0 + BN) of a [Nk, D] slice into this wave's tile (rows >= Nk repeat row Nk - 1),
    // row-major with the XOR swizzle (fa_common.h); the wave copies alone, non-temporal (every key and
    // value row is read once)
    static __device__ __forceinline__ void copy(const T* __restrict__ src, int r0, int Nk, uint32_t lds, int lane) {
        copy_tile<XorRows<CPR>, BN, CPR, 64, true>(src, r0, Nk, D * 2, lds, lane, 0);
    }

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, float* __restrict__ Op,
                                               float* __restrict__ Lp, int Nq, int Nk, int nsplit, int chunk,
                                               float c, uint32_t qflip, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const int bh = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
        const int nc = nsplit * NW, ci = split * NW + wave;      // chunk index of this wave
        const int j0 = ci * chunk, j1 = min(Nk, j0 + chunk);     // its keys
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem)) + wave * WAVE_LDS;
        const char* wl = smem + wave * WAVE_LDS;
        const T* Kh = K + (size_t)bh * Nk * D;
        const T* Vh = V + (size_t)bh * Nk * D;
        const int query = n32, qrow = min(query, Nq - 1);
        const int last_key = CAUSAL ? query + Nk - Nq : Nk - 1;  // last key visible to this lane's query

        const int kperm = ((n32 >> 4) & 1) * 16 + ((n32 >> 2) & 1) * 8 + ((n32 >> 3) & 1) * 4 + (n32 & 3);
        const int i16 = lane & 15, G = lane >> 4;
        const int vrow = (G >> 1) * 8 + (i16 >> 2), vcc = (G & 1) * 2 + ((i16 & 3) >> 1), vb = (i16 & 1) * 8;

        x8 qreg[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            i32x4 raw = *(const i32x4*)(Q + ((size_t)bh * Nq + qrow) * D + ks * 16 + h * 8);
            raw ^= (int)qflip;
            qreg[ks] = __builtin_bit_cast(x8, raw);
        }
        const int ntile = j1 > j0 ? (j1 - j0 + BN - 1) / BN : 0;
        if (ntile > 0) {
            copy(Kh, j0, Nk, lbase, lane);
            copy(Vh, j0, Nk, lbase + TILE, lane);
        }
        f32x16 oacc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
        float m_run = -INFINITY, l_run = 0.0f;

        for (int t = 0; t < ntile; ++t) {
            const int st = t & 1;
            const int kv0 = j0 + t * BN;
            if (t + 1 < ntile) {
                // the stage about to be refilled was last read by this wave's previous tile
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                copy(Kh, kv0 + BN, Nk, lbase + (st ^ 1) * 2 * TILE, lane);
                copy(Vh, kv0 + BN, Nk, lbase + (st ^ 1) * 2 * TILE + TILE, lane);
                wait_vmcnt<2 * LPT>();
            } else {
                wait_vmcnt<0>();
            }
            const char* kl = wl + st * 2 * TILE;
            const char* vl = kl + TILE;
            // S^T = K Q^T for 32 keys: register r holds key kv0 + (r/8)*16 + h*8 + r%8
            f32x16 s = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const x8 kop = *(const x8*)(kl + XorRows<CPR>::slot(kperm, 2 * ks + h) * 16);
                s = VT::mfma(kop, qreg[ks], s);
            }
            if (kv0 + BN > j1 || kv0 + BN - 1 > last_key) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + (r >> 3) * 16 + h * 8 + (r & 7);
                    if (key >= j1 || key > last_key) s[r] = -INFINITY;
                }
            }
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
            const float mt = halves_max(mx) * c;
            if (__ballot(mt > m_run + kTauD)) {
                // a query that has seen no key of the chunk yet keeps m = -inf while another lane of
                // the wave raises its maximum: its factor is 1, not 2^(-inf - -inf)
                const float mn = fmaxf(m_run, mt);
                const float alpha = m_run == mn ? 1.0f : fast_exp2(m_run - mn);
                m_run = mn;
                l_run *= alpha;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
            }
            // while no key of the chunk has been visible to this query, m_run is -inf and every score
            // is -inf: use 0 as the offset so the weights come out 0 (not exp2 of -inf + inf)
            const float negm = m_run == -INFINITY ? 0.0f : -m_run;
            float e[16];
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                e[r] = fast_exp2(__builtin_fmaf(s[r], c, negm));
                sum += e[r];
            }
            l_run += sum;
            const x8 p0 = VT::pack(e), p1 = VT::pack(e + 8);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    const int r0 = sp * 16;
                    const int row0 = r0 + vrow, row1 = r0 + 4 + vrow;
                    const x4 lo = VT::read_tr(vl + XorRows<CPR>::slot(row0, cb * 4 + vcc) * 16 + vb);
                    const x4 hi = VT::read_tr(vl + XorRows<CPR>::slot(row1, cb * 4 + vcc) * 16 + vb);
                    oacc[cb] = VT::mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), sp ? p1 : p0,
                                        oacc[cb]);
                }
            }
        }
        // partial result of this chunk: O_c = O / l, lse_c = m + log2 l (base 2); an empty chunk
        // (no visible key) stores lse_c = -inf and O_c = 0
        const float lt = halves_sum(l_run);
        if (query < Nq) {
            const size_t slot = ((size_t)bh * nc + ci) * Nq + query;
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            float* orow = Op + slot * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = oacc[cb][g * 4 + e] * inv;
                    *(f32x4*)(orow + cb * 32 + g * 8 + h * 4) = out;
                }
            if (h == 0) Lp[slot] = lt > 0.0f ? m_run + __log2f(lt) : -INFINITY;
        }
    }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              const T* __restrict__ V, float* __restrict__ Op,
                                                              float* __restrict__ Lp, int Nq, int Nk, int nsplit,
                                                              int chunk, float c, uint32_t qflip) {
    __shared__ __attribute__((aligned(1024))) char smem[Decode<T, D, CAUSAL>::LDS_BYTES];
    Decode<T, D, CAUSAL>::run(Q, K, V, Op, Lp, Nq, Nk, nsplit, chunk, c, qflip, smem);
}

// ---------------------------------------------------------------------------------------------
// One query per (b, h): S = q K^T and O = P V are dot products, computed on the vector ALU with the
// packed 16-bit dot instruction (v_dot2_f32_{bf16,f16}, float32 accumulation).  K and V rows stream
// straight from HBM into registers with ordinary loads, two iterations deep, so the bytes in flight
// are not bounded by LDS.  Lanes form groups of D/8: lane li of group g holds columns 8 li .. 8 li + 7
// of key j0 + G t + g (G = 64 / (D/8) keys per load instruction, consecutive rows).  Each group runs
// an online softmax over its keys; the groups of a wave are combined at the end and the wave writes
// the same partial (O_c, lse_c) as decode_split_kernel, merged by decode_merge_kernel.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <typename T, int D>
struct DecodeVec {
    static constexpr int NW = 4, LPK = D / 8, G = 64 / LPK, U = 4;
    typedef T t2 __attribute__((ext_vector_type(2)));

    static __device__ __forceinline__ float dot2(t2 a, t2 b, float c) {
        if constexpr (sizeof(T) == 2 && __is_same(T, __bf16)) return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
        else return __builtin_amdgcn_fdot2(a, b, c, false);
    }
    // sum over the LPK lanes of a group, result in every lane of the group
    static __device__ __forceinline__ float group_sum(float x) {
        x += dppf<0xB1>(x);   // lane ^ 1
        x += dppf<0x4E>(x);   // lane ^ 2
        x += dppf<0x141>(x);  // mirror within 8 lanes: the other quad
        if constexpr (LPK >= 16) x += dppf<0x140>(x);  // mirror within 16 lanes: the other 8
        if constexpr (LPK >= 32) x += __shfl_xor(x, 16, 64);
        return x;
    }
    static __device__ __forceinline__ void load(const T* __restrict__ Kh, const T* __restrict__ Vh, int j0, int it,
                                                int g, int last, i32x4 (&kb)[U], i32x4 (&vb)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = min(j0 + (it * U + u) * G + g, last);
            // non-temporal: each key and value row is read once (bf16 B8 H32 Nk32768 d128 728.7 -> 645.8 us)
            kb[u] = __builtin_nontemporal_load((const i32x4*)(Kh + (size_t)key * D));
            vb[u] = __builtin_nontemporal_load((const i32x4*)(Vh + (size_t)key * D));
        }
    }

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, float* __restrict__ Op,
                                               float* __restrict__ Lp, int Nk, int nsplit, int chunk, float c,
                                               uint32_t qflip) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int g = lane / LPK, li = lane % LPK;
        const int bh = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
        const int nc = nsplit * NW, ci = split * NW + wave;
        const int j0 = ci * chunk, j1 = min(Nk, j0 + chunk);
        const T* Kh = K + (size_t)bh * Nk * D + li * 8;
        const T* Vh = V + (size_t)bh * Nk * D + li * 8;
        t2 qv[4];
        {
            i32x4 raw = *(const i32x4*)(Q + (size_t)bh * D + li * 8);
            raw ^= (int)qflip;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // (a bit-cast applied to a vector element directly would read element 0 each time)
                const int w = raw[p];
                qv[p] = __builtin_bit_cast(t2, w);
            }
        }
        float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.0f;
        const int niter = j1 > j0 ? (j1 - j0 + G * U - 1) / (G * U) : 0;
        i32x4 kb[U], vb[U], kn[U], vn[U];
        if (niter > 0) load(Kh, Vh, j0, 0, g, j1 - 1, kb, vb);
        for (int it = 0; it < niter; ++it) {
            if (it + 1 < niter) load(Kh, Vh, j0, it + 1, g, j1 - 1, kn, vn);
            float sv[U];
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc = 0.0f;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int w = kb[u][p];
                    acc = dot2(qv[p], __builtin_bit_cast(t2, w), acc);
                }
                acc = group_sum(acc) * c;
                const int key = j0 + (it * U + u) * G + g;
                sv[u] = key < j1 ? acc : -INFINITY;
                mt = fmaxf(mt, sv[u]);
            }
            const float mn = fmaxf(m, mt);
            // no visible key yet: keep the weights 0 (not exp2 of -inf + inf)
            const float negm = mn == -INFINITY ? 0.0f : -mn;
            const float alpha = m == mn ? 1.0f : fast_exp2(m - mn);
            l *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= alpha;
            m = mn;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = fast_exp2(sv[u] + negm);
                l += p;
                const T pt = (T)p;  // P rounded to the input type, as the matrix path rounds it
                const uint32_t pb = (uint32_t)__builtin_bit_cast(uint16_t, pt);
                const t2 plo = __builtin_bit_cast(t2, pb), phi = __builtin_bit_cast(t2, pb << 16);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int w = vb[u][q];
                    const t2 vv = __builtin_bit_cast(t2, w);
                    o[2 * q] = dot2(vv, plo, o[2 * q]);
                    o[2 * q + 1] = dot2(vv, phi, o[2 * q + 1]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                kb[u] = kn[u];
                vb[u] = vn[u];
            }
        }
        // combine the groups of the wave: (m, l, o) pairs of groups g and g ^ (off / LPK)
#pragma unroll
        for (int off = LPK; off < 64; off *= 2) {
            const float mo = __shfl_xor(m, off, 64), lo = __shfl_xor(l, off, 64);
            const float mn = fmaxf(m, mo);
            const float a = m == mn ? 1.0f : fast_exp2(m - mn), b = mo == mn ? 1.0f : fast_exp2(mo - mn);
            l = l * a + lo * b;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = o[e] * a + __shfl_xor(o[e], off, 64) * b;
            m = mn;
        }
        if (g == 0) {
            const size_t slot = (size_t)bh * nc + ci;  // Nq = 1
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            f32x4 a, b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = o[e] * inv;
                b[e] = o[4 + e] * inv;
            }
            *(f32x4*)(Op + slot * D + li * 8) = a;
            *(f32x4*)(Op + slot * D + li * 8 + 4) = b;
            if (li == 0) Lp[slot] = l > 0.0f ? m + __log2f(l) : -INFINITY;
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_vec_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                         const T* __restrict__ V, float* __restrict__ Op,
                                                         float* __restrict__ Lp, int Nk, int nsplit, int chunk, float c,
                                                         uint32_t qflip) {
    DecodeVec<T, D>::run(Q, K, V, Op, Lp, Nk, nsplit, chunk, c, qflip);
}

// 256 threads per workgroup, D/4 per (b, h, query row): thread t owns output columns 4t .. 4t+3, read as
// one float4 per partial; 1024/D rows per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ Op, const float* __restrict__ Lp,
                                                           T* __restrict__ O, float* __restrict__ LSE, int Nq, int nc,
                                                           long long rows) {
    constexpr int TPR = D / 4, RPB = 256 / TPR;
    const long long r = (long long)blockIdx.x * RPB + threadIdx.x / TPR;  // (b, h, query) row
    if (r >= rows) return;
    const int col = (threadIdx.x % TPR) * 4;
    const long long bh = r / Nq, query = r % Nq;
    const size_t base = (size_t)bh * nc * Nq + query;
    float M = -INFINITY;
    for (int i = 0; i < nc; ++i) M = fmaxf(M, Lp[base + (size_t)i * Nq]);
    float L = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 0; i < nc; ++i) {
        const float lc = Lp[base + (size_t)i * Nq];
        const float w = lc == -INFINITY ? 0.0f : fast_exp2(lc - M);
        L += w;
        const f32x4 o = *(const f32x4*)(Op + (base + (size_t)i * Nq) * D + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, o[e], acc[e]);
    }
    typename Vec<T>::x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (T)(acc[e] / L);
    *(typename Vec<T>::x4*)(O + r * D + col) = out;
    if (LSE != nullptr && col == 0) LSE[r] = (M + __log2f(L)) * 0.69314718055994531f;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, void* o, float* lse, float* work, int BH,
                           int Nq, int Nk, int nsplit, int chunk, float c, uint32_t qflip, hipStream_t stream) {
    // one query: the vector-ALU kernel (its causal mask hides nothing: the query is the last position)
    const bool vec = Nq == 1;
    const int nc = nsplit * (vec ? DecodeVec<T, D>::NW : Decode<T, D, CAUSAL>::NW);
    float* Op = work;
    float* Lp = work + (size_t)BH * nc * Nq * D;
    const long long nwg = (long long)BH * nsplit, nm = (long long)BH * Nq;
    if (nwg > 0x7fffffffLL || nm > 0x7fffffffLL) return hipErrorInvalidValue;
    if (vec) {
        hipLaunchKernelGGL((decode_vec_kernel<T, D>), dim3((unsigned)nwg), dim3(64 * DecodeVec<T, D>::NW), 0, stream,
                           (const T*)q, (const T*)k, (const T*)v, Op, Lp, Nk, nsplit, chunk, c, qflip);
    } else {
        hipLaunchKernelGGL((decode_split_kernel<T, D, CAUSAL>), dim3((unsigned)nwg), dim3(64 * Decode<T, D, CAUSAL>::NW), 0, stream, (const T*)q,
                           (const T*)k, (const T*)v, Op, Lp, Nq, Nk, nsplit, chunk, c, qflip);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int RPB = 1024 / D;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)((nm + RPB - 1) / RPB)), dim3(256), 0, stream,
                       (const float*)Op, (const float*)Lp, (T*)o, lse, Nq, nc, nm);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_dt(const void* q, const void* k, const void* v, void* o, float* lse, float* work, int BH,
                            int Nq, int Nk, int d, bool causal, int nsplit, int chunk, float c, uint32_t qflip,
                            hipStream_t stream) {
    switch (d) {
        case 64:
            return causal ? launch_decode_t<T, 64, true>(q, k, v, o, lse, work, BH, Nq, Nk, nsplit, chunk, c, qflip, stream)
                          : launch_decode_t<T, 64, false>(q, k, v, o, lse, work, BH, Nq, Nk, nsplit, chunk, c, qflip, stream);
        case 128:
            return causal ? launch_decode_t<T, 128, true>(q, k, v, o, lse, work, BH, Nq, Nk, nsplit, chunk, c, qflip, stream)
                          : launch_decode_t<T, 128, false>(q, k, v, o, lse, work, BH, Nq, Nk, nsplit, chunk, c, qflip, stream);
        case 256:
            return causal ? launch_decode_t<T, 256, true>(q, k, v, o, lse, work, BH, Nq, Nk, nsplit, chunk, c, qflip, stream)
                          : launch_decode_t<T, 256, false>(q, k, v, o, lse, work, BH, Nq, Nk, nsplit, chunk, c, qflip, stream);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_merge_partials(bool is_bf16, const float* Op, const float* Lp, void* o, float* lse, int BH, int Nq,
                                 int nc, int d, hipStream_t stream) {
    const long long nm = (long long)BH * Nq;
    if (nm > 0x7fffffffLL) return hipErrorInvalidValue;
    auto go = [&](auto tag, auto dim) -> hipError_t {
        using T = decltype(tag);
        constexpr int D = decltype(dim)::value;
        constexpr int RPB = 1024 / D;
        hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)((nm + RPB - 1) / RPB)), dim3(256), 0, stream,
                           Op, Lp, (T*)o, lse, Nq, nc, nm);
        return hipGetLastError();
    };
    switch (d) {
        case 64: return is_bf16 ? go(__bf16{}, std::integral_constant<int, 64>{}) : go(_Float16{}, std::integral_constant<int, 64>{});
        case 128: return is_bf16 ? go(__bf16{}, std::integral_constant<int, 128>{}) : go(_Float16{}, std::integral_constant<int, 128>{});
        case 256: return is_bf16 ? go(__bf16{}, std::integral_constant<int, 256>{}) : go(_Float16{}, std::integral_constant<int, 256>{});
        default: return hipErrorNotSupported;
    }
}

// ---- library-held workspace of the decode path, for callers that cannot allocate ----
// One array per GPU (the code object's device variable), kept until the process ends; it holds the
// partial results of the last fa_fwd_decode_noalloc call on that GPU.  Every call overwrites each entry
// it reads (an empty key chunk stores O_c = 0, lse_c = -inf), so nothing needs clearing between calls;
// calls that overlap in time on one GPU race on it.  Host code never passes the array's name to a
// kernel: that is a host-side stand-in, not a device address.  decode_scratch_ptr returns the address
// that hipGetSymbolAddress gives for the current device, looked up once per device.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch_ptr(float** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<float*>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode_16(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse, float* work,
                            int BH, int Nq, int Nk, int d, bool causal, int nsplit, int chunk, float c, uint32_t qflip,
                            hipStream_t stream) {
    return is_bf16 ? launch_decode_dt<__bf16>(q, k, v, o, lse, work, BH, Nq, Nk, d, causal, nsplit, chunk, c, qflip, stream)
                   : launch_decode_dt<_Float16>(q, k, v, o, lse, work, BH, Nq, Nk, d, causal, nsplit, chunk, c, qflip,
                                                stream);
}

}  // namespace fa
