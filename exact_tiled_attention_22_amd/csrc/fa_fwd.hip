// fa_fwd.hip — tiled attention forward for 16-bit floats (bf16 / fp16) on gfx950.
//
// The method: "FlashAttention 2 + 3 — speicherbewusste Attention-Kernels", section "Kernpunkte"
// (Q/K/V cut into on-chip blocks of 64-128 rows, online softmax, no N x N matrix in HBM, better work
// partitioning across thread blocks) and "Begriffe auf dieser Seite", entry "Online-Softmax" (running
// maximum plus a correction factor at every tile boundary).  The FlashAttention-3 article's "Drei
// technische Hebel" items 1-2 (copy the next block while computing; keep the matrix units busy) are
// realised here with gfx950 means: direct HBM->LDS loads of the next key/value tile issued before
// the current tile's MFMA work, and MFMA instructions for both products.
//
// Layout of the work (one workgroup = NW waves = BM = NW*32*QB query rows of one (b,h)):
//   * every wave owns QB blocks of 32 query rows; its Q operand lives in registers for the whole
//     kernel;
//   * key/value tiles of BN = 64 rows stream through two LDS stages;
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: lane l then holds the
//     scores of query (l % 32) for 16 keys per 32-key block, so the row maximum and sum are
//     in-lane plus one exchange between the two wave halves;
//   * the K rows feeding the MFMA A-operand are permuted (kperm below) so that the 8 consecutive
//     accumulator registers of a lane correspond to 8 consecutive keys; the probabilities then feed
//     the second MFMA as its B-operand with no data movement: O^T += V^T P^T;
//   * V^T operands come from LDS with the gfx950 transposing read ds_read_b64_tr_b16;
//   * O^T accumulates in registers; lane l holds 16 output columns of query (l % 32) per 32-column
//     block, so the per-row correction factor and the final 1/l are in-lane multiplies.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kTau = 8.0f;  // rescale only when the running maximum grows by more than 2^8

template <int D, int QB, int NW>
struct Tile {
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int QW = 32 * QB;            // query rows per wave
    static constexpr int BM = QW * NW;            // query rows per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int CPR = D / 8;             // 16-byte chunks per row (2-byte elements)
    static constexpr int CHUNKS = BN * CPR;       // chunks per K (or V) tile
    static constexpr int LPT = CHUNKS / THREADS;  // direct-to-LDS loads per thread per tile
    static constexpr int BYTES = CHUNKS * 16;
    static_assert(CHUNKS % THREADS == 0, "tile must split evenly over the workgroup");
};

// XOR swizzle of the 16-byte chunk index inside one LDS row.  Chosen so that (a) the eight rows
// {0,1,2,3,8,9,10,11} (+4) read together by the score MFMA operand fetch, and (b) the four
// consecutive rows read together by a transposing V fetch, land in distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    int f = ((row & 3) << 1) | ((row >> 3) & 1);
    if constexpr (CPR >= 16) f |= ((row >> 2) & 1) << 3;
    return f;
}

// Issue the direct HBM->LDS copy of rows [kv0, kv0+BN) of one head (rows past N are clamped to
// N-1; they are masked out of the softmax).  LDS slot s (16 bytes) holds chunk (s % CPR) ^ swz(row)
// of row s / CPR.
template <int D, int QB, int NW, typename T>
__device__ __forceinline__ void load_tile(const T* __restrict__ src, int kv0, int N, char* lds,
                                          int tid, int wave) {
    using TL = Tile<D, QB, NW>;
#pragma unroll
    for (int t = 0; t < TL::LPT; ++t) {
        const int slot = t * TL::THREADS + tid;
        const int row = slot / TL::CPR;
        const int c = (slot % TL::CPR) ^ swz<TL::CPR>(row);
        const int grow = min(kv0 + row, N - 1);
        const T* g = src + (size_t)grow * D + c * 8;
        char* dst = lds + (t * TL::THREADS + wave * 64) * 16;  // wave-uniform base (M0)
        __builtin_amdgcn_global_load_lds((const void*)g, (FA_LDS void*)dst, 16, 0, 0);
    }
}

template <typename T, int D, int QB, int NW, bool CAUSAL>
struct Fwd {
    using TL = Tile<D, QB, NW>;
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    static constexpr int BN = TL::BN, QW = TL::QW, BM = TL::BM, CPR = TL::CPR;
    static constexpr int KS = D / 16;  // k-steps of the score product
    static constexpr int CB = D / 32;  // 32-column blocks of the output

    // one key/value tile: scores, online softmax, P*V
    static __device__ __forceinline__ void tile(const char* kl, const char* vl, int kv0, int N, int q0w,
                                                int lane, float c, const x8 (&qreg)[QB][KS],
                                                f32x16 (&oacc)[QB][CB], float (&m_run)[QB],
                                                float (&l_run)[QB]) {
        const int n32 = lane & 31;
        const int h = lane >> 5;

        // ---- scores S^T = K Q^T (fp32 accumulate) ----
        const int kperm = ((n32 >> 4) & 1) * 16 + ((n32 >> 2) & 1) * 8 + ((n32 >> 3) & 1) * 4 + (n32 & 3);
        const int ksw = swz<CPR>(kperm);
        f32x16 sacc[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sacc[qb][kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = kb * 32 + kperm;
                const x8 kop = *(const x8*)(kl + (row * CPR + ((2 * ks + h) ^ ksw)) * 16);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = VT::mfma(kop, qreg[qb][ks], sacc[qb][kb]);
            }
        }

        // ---- causal diagonal / ragged tail: hidden keys get -inf ----
        const bool masked = (kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > q0w);
        if (masked) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int query = q0w + qb * 32 + n32;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                        const bool hide = key >= N || (CAUSAL && key > query);
                        if (hide) sacc[qb][kb][r] = -INFINITY;
                    }
            }
        }

        // ---- online softmax: running max (base-2 units), lazy correction ----
        float mt[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = sacc[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
            mx = fmaxf(mx, swap_halves(mx));
            mt[qb] = mx * c;
            grow |= mt[qb] > m_run[qb] + kTau;
        }
        if (__ballot(grow)) {  // wave-uniform: some row's maximum grew by more than 2^tau
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mn = fmaxf(m_run[qb], mt[qb]);
                const float alpha = fast_exp2(m_run[qb] - mn);
                m_run[qb] = mn;
                l_run[qb] *= alpha;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] *= alpha;
            }
        }

        // ---- P = exp2(s*c - m), row sums from fp32 P, P rounded to the operand type ----
        x8 p[QB][4];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float negm = -m_run[qb];
            float ls = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float e[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    e[r] = fast_exp2(__builtin_fmaf(sacc[qb][kb][r], c, negm));
                    ls += e[r];
                }
                p[qb][kb * 2 + 0] = VT::pack(e);
                p[qb][kb * 2 + 1] = VT::pack(e + 8);
            }
            l_run[qb] += ls;
        }

        // ---- O^T += V^T P^T; V^T operand via transposing LDS reads ----
        // lane = 16*G + i; G>>1 selects keys +0..7 / +8..15 of the 16-key step, G&1 the column half
        const int i16 = lane & 15, G = lane >> 4;
        const int vrow = (G >> 1) * 8 + (i16 >> 2);                    // + s*16 + u*4
        const int vcol_chunk = (G & 1) * 2 + ((i16 & 3) >> 1);         // + cb*4
        const int vbyte = (i16 & 1) * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                x4 lo, hi;
                {
                    const int row = s * 16 + vrow;
                    const int ch = cb * 4 + vcol_chunk;
                    lo = VT::read_tr(vl + (row * CPR + (ch ^ swz<CPR>(row))) * 16 + vbyte);
                }
                {
                    const int row = s * 16 + 4 + vrow;
                    const int ch = cb * 4 + vcol_chunk;
                    hi = VT::read_tr(vl + (row * CPR + (ch ^ swz<CPR>(row))) * 16 + vbyte);
                }
                const x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[qb][cb] = VT::mfma(vop, p[qb][s], oacc[qb][cb]);
            }
        }
    }

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, T* __restrict__ O,
                                               float* __restrict__ LSE, int N, int BH, int ntq, float c,
                                               uint32_t qflip, char* k0, char* k1, char* v0, char* v1) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31;
        const int h = lane >> 5;

        int bh, qt;
        map_block(blockIdx.x, BH, ntq, CAUSAL, bh, qt);
        const size_t head = (size_t)bh * N * D;
        const T* Qh = Q + head;
        const T* Kh = K + head;
        const T* Vh = V + head;
        const int q0 = qt * BM;
        const int q0w = q0 + wave * QW;
        const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
        const int nt = (kv_end + BN - 1) / BN;
        const int wave_kv_end = CAUSAL ? min(N, q0w + QW) : N;

        // first K/V tile in flight before the Q loads
        load_tile<D, QB, NW>(Kh, 0, N, k0, tid, wave);
        load_tile<D, QB, NW>(Vh, 0, N, v0, tid, wave);

        // Q operand (B of the score MFMA): lane supplies Q[q0w + qb*32 + n32][ks*16 + h*8 + 0..7]
        x8 qreg[QB][KS];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = min(q0w + qb * 32 + n32, N - 1);
            const T* src = Qh + (size_t)row * D + h * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                i32x4 raw = *(const i32x4*)(src + ks * 16);
                raw ^= (int)qflip;
                qreg[qb][ks] = __builtin_bit_cast(x8, raw);
            }
        }

        f32x16 oacc[QB][CB];
        float m_run[QB], l_run[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] = f32x16{};
        }

        constexpr int LPT2 = 2 * TL::LPT;
        for (int j = 0; j < nt; j += 2) {
            // even tile in stage 0, its successor prefetched into stage 1
            {
                const int kv0 = j * BN;
                if (j + 1 < nt) {
                    load_tile<D, QB, NW>(Kh, kv0 + BN, N, k1, tid, wave);
                    load_tile<D, QB, NW>(Vh, kv0 + BN, N, v1, tid, wave);
                    wait_vmcnt<LPT2>();
                } else {
                    wait_vmcnt<0>();
                }
                lds_barrier();
                if (!CAUSAL || kv0 < wave_kv_end) tile(k0, v0, kv0, N, q0w, lane, c, qreg, oacc, m_run, l_run);
                lds_barrier();
            }
            if (j + 1 < nt) {
                const int kv0 = (j + 1) * BN;
                if (j + 2 < nt) {
                    load_tile<D, QB, NW>(Kh, kv0 + BN, N, k0, tid, wave);
                    load_tile<D, QB, NW>(Vh, kv0 + BN, N, v0, tid, wave);
                    wait_vmcnt<LPT2>();
                } else {
                    wait_vmcnt<0>();
                }
                lds_barrier();
                if (!CAUSAL || kv0 < wave_kv_end) tile(k1, v1, kv0, N, q0w, lane, c, qreg, oacc, m_run, l_run);
                lds_barrier();
            }
        }

        // ---- epilogue: O = acc / l (rounded to T), lse = ln2 * (m + log2 l) ----
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = l_run[qb] + swap_halves(l_run[qb]);
            const float inv = 1.0f / lt;
            const int query = q0w + qb * 32 + n32;
            if (query < N) {
                T* orow = O + head + (size_t)query * D;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        x4 out;
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = (T)(oacc[qb][cb][g * 4 + e] * inv);
                        *(x4*)(orow + cb * 32 + g * 8 + h * 4) = out;
                    }
                if (LSE != nullptr && h == 0)
                    LSE[(size_t)bh * N + query] = (m_run[qb] + __log2f(lt)) * 0.69314718055994531f;
            }
        }
    }
};

template <typename T, int D, int QB, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 1) void fa_fwd16_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              const T* __restrict__ V, T* __restrict__ O,
                                                              float* __restrict__ LSE, int N, int BH, int ntq,
                                                              float c, uint32_t qflip) {
    using TL = Tile<D, QB, NW>;
    __shared__ __attribute__((aligned(16))) char k0[TL::BYTES];
    __shared__ __attribute__((aligned(16))) char k1[TL::BYTES];
    __shared__ __attribute__((aligned(16))) char v0[TL::BYTES];
    __shared__ __attribute__((aligned(16))) char v1[TL::BYTES];
    Fwd<T, D, QB, NW, CAUSAL>::run(Q, K, V, O, LSE, N, BH, ntq, c, qflip, k0, k1, v0, v1);
}

// per head dimension: query blocks per wave and waves per workgroup
template <int D> struct Shape;
template <> struct Shape<64> { static constexpr int QB = 2, NW = 4; };
template <> struct Shape<128> { static constexpr int QB = 2, NW = 4; };
template <> struct Shape<256> { static constexpr int QB = 1, NW = 4; };

template <typename T, int D, bool CAUSAL>
hipError_t launch16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, float c,
                    uint32_t qflip, hipStream_t stream) {
    constexpr int QB = Shape<D>::QB, NW = Shape<D>::NW;
    constexpr int BM = Tile<D, QB, NW>::BM;
    const int ntq = (N + BM - 1) / BM;
    const long long nwg = (long long)BH * ntq;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fa_fwd16_kernel<T, D, QB, NW, CAUSAL>), dim3((unsigned)nwg), dim3(64 * NW), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, N, BH, ntq, c, qflip);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                      bool causal, float c, uint32_t qflip, hipStream_t stream) {
    switch (d) {
        case 64:
            return causal ? launch16<T, 64, true>(q, k, v, o, lse, BH, N, c, qflip, stream)
                          : launch16<T, 64, false>(q, k, v, o, lse, BH, N, c, qflip, stream);
        case 128:
            return causal ? launch16<T, 128, true>(q, k, v, o, lse, BH, N, c, qflip, stream)
                          : launch16<T, 128, false>(q, k, v, o, lse, BH, N, c, qflip, stream);
        case 256:
            return causal ? launch16<T, 256, true>(q, k, v, o, lse, BH, N, c, qflip, stream)
                          : launch16<T, 256, false>(q, k, v, o, lse, BH, N, c, qflip, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_16(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                         int N, int d, bool causal, float c, uint32_t qflip, hipStream_t stream) {
    return is_bf16 ? dispatch16<__bf16>(q, k, v, o, lse, BH, N, d, causal, c, qflip, stream)
                   : dispatch16<_Float16>(q, k, v, o, lse, BH, N, d, causal, c, qflip, stream);
}

}  // namespace fa
