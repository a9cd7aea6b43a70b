// fa_fwd.hip — tiled attention forward for 16-bit floats (bf16 / fp16) on gfx950.
//
// The method: "FlashAttention 2 + 3 — speicherbewusste Attention-Kernels", section "Kernpunkte"
// (Q/K/V cut into on-chip blocks of 64-128 rows, online softmax, no N x N matrix in HBM, better work
// partitioning across thread blocks) and "Begriffe auf dieser Seite", entry "Online-Softmax" (running
// maximum plus a correction factor at every tile boundary).  The FlashAttention-3 article's "Drei
// technische Hebel" items 1-2 (copy the next block while computing; keep the matrix units busy) are
// realised with gfx950 means: direct HBM->LDS copies of the next tiles issued before the current
// tile's work, and the next tile's score MFMAs issued while the current tile's softmax runs on the
// vector ALUs.
//
// Work layout (one workgroup = NW waves = BM = NW * 32 * QB query rows of one (b, h)):
//   * each wave owns QB blocks of 32 query rows; its Q operand is loaded once (HBM -> LDS ->
//     registers) and stays in registers;
//   * key/value tiles of BN = 64 rows stream through two LDS stages each; K runs one tile ahead of V:
//     during iteration j the LDS holds K_{j+1} and V_j while K_{j+2} and V_{j+1} are copied in, so
//     one barrier per tile suffices;
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: lane l holds the scores
//     of query (l % 32) for 16 keys of each 32-key block, so the row maximum and sum are in-lane plus
//     one exchange between the two wave halves;
//   * the K rows feeding the MFMA A-operand are permuted (kperm) so that 8 consecutive accumulator
//     registers of a lane hold 8 consecutive keys; the probabilities then feed O^T += V^T P^T as the
//     B-operand without any data movement;
//   * V^T operands come from LDS through the transposing read ds_read_b64_tr_b16;
//   * O^T accumulates in registers: lane l holds 16 output columns of query (l % 32) per 32-column
//     block, so the correction factor and the final 1/l are in-lane multiplies.
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
    static constexpr int LPT = CHUNKS / THREADS;  // direct-to-LDS copies per thread per tile
    static constexpr int KV_BYTES = CHUNKS * 16;
    static constexpr int Q_CHUNKS = BM * CPR;
    static constexpr int QLPT = Q_CHUNKS / THREADS;
    static constexpr int Q_BYTES = Q_CHUNKS * 16;
    // the Q staging area gets its own LDS region when it fits, otherwise it aliases stage 1 (K1|V1)
    static constexpr bool Q_SEPARATE = Q_BYTES + 4 * KV_BYTES <= 160 * 1024;
    static constexpr int LDS_BYTES = Q_SEPARATE ? Q_BYTES + 4 * KV_BYTES : 4 * KV_BYTES;
    static_assert(CHUNKS % THREADS == 0 && Q_CHUNKS % THREADS == 0, "tiles split evenly over threads");
    static_assert(Q_SEPARATE || Q_BYTES <= 2 * KV_BYTES, "Q staging must fit in stage 1");
    static_assert(LPT <= 16, "vmcnt range");
};

// XOR swizzle of the 16-byte chunk index inside one LDS row: the eight rows {0,1,2,3,8,9,10,11}
// (+4) read together by a score-operand fetch, and the four consecutive rows read together by a
// transposing V fetch, fall into distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    int f = ((row & 3) << 1) | ((row >> 3) & 1);
    if constexpr (CPR >= 16) f |= ((row >> 2) & 1) << 3;
    return f;
}

template <typename T, int D, int QB, int NW, bool CAUSAL>
struct Fwd {
    using TL = Tile<D, QB, NW>;
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    static constexpr int BN = TL::BN, QW = TL::QW, BM = TL::BM, CPR = TL::CPR, LPT = TL::LPT;
    static constexpr int KS = D / 16;  // k-steps of the score product
    static constexpr int CB = D / 32;  // 32-column blocks of the output
    // LDS map (byte offsets)
    static constexpr int OFF_K0 = TL::Q_SEPARATE ? TL::Q_BYTES : 0;
    static constexpr int OFF_V0 = OFF_K0 + TL::KV_BYTES;
    static constexpr int OFF_K1 = OFF_V0 + TL::KV_BYTES;
    static constexpr int OFF_V1 = OFF_K1 + TL::KV_BYTES;
    static constexpr int OFF_Q = TL::Q_SEPARATE ? 0 : OFF_K1;

    // Copy rows [r0, r0 + ROWS) of a [N, D] slice into an LDS tile (rows >= N read row N-1; they are
    // masked or never stored).  Slot s of the tile holds chunk (s % CPR) ^ swz(row) of row s / CPR.
    template <int NLOADS>
    static __device__ __forceinline__ void copy_rows(const T* __restrict__ src, int r0, int N, uint32_t lds,
                                                     int tid, int wave) {
#pragma unroll
        for (int t = 0; t < NLOADS; ++t) {
            const int slot = t * TL::THREADS + tid;
            const int row = slot / CPR;
            const int c = (slot % CPR) ^ swz<CPR>(row);
            const T* g = src + (size_t)min(r0 + row, N - 1) * D + c * 8;
            dma16(g, lds + (uint32_t)((t * TL::THREADS + wave * 64) * 16));
        }
    }

    // S^T = K_tile Q^T for this wave's QB query blocks (fp32 accumulate)
    static __device__ __forceinline__ void scores(const char* kl, const x8 (&qreg)[QB][KS], f32x16 (&s)[QB][2],
                                                  int kbase, int h, int ksw) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int xo = ((2 * ks + h) ^ ksw) * 16;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const x8 kop = *(const x8*)(kl + kbase + kb * 32 * CPR * 16 + xo);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb][kb] = VT::mfma(kop, qreg[qb][ks], s[qb][kb]);
            }
        }
    }

    // Hide keys past N and (causal) keys after the query; true when the tile needs it.
    static __device__ __forceinline__ void mask(f32x16 (&s)[QB][2], int kv0, int N, int q0w, int n32, int h) {
        if ((kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > q0w)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int query = q0w + qb * 32 + n32;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                        if (key >= N || (CAUSAL && key > query)) s[qb][kb][r] = -INFINITY;
                    }
            }
        }
    }

    // Running maximum in base-2 units; the accumulator and sum are rescaled only when some row's
    // maximum grew by more than 2^tau (p = 2^(s*c - m) then stays <= 2^tau, exact either way).
    static __device__ __forceinline__ void update_max(const f32x16 (&s)[QB][2], float c, f32x16 (&oacc)[QB][CB],
                                                      float (&m_run)[QB], float (&l_run)[QB]) {
        float mt[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = fmaxf(s[qb][0][0], s[qb][1][0]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
            mt[qb] = halves_max(mx) * c;
            grow |= mt[qb] > m_run[qb] + kTau;
        }
        if (__ballot(grow)) {
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
    }

    // P = 2^(s*c - m) rounded to T (row sums from the fp32 values)
    static __device__ __forceinline__ void exps(const f32x16 (&s)[QB][2], float c, const float (&m_run)[QB],
                                                float (&l_run)[QB], x8 (&p)[QB][4]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float negm = -m_run[qb];
            float ls = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float e[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    e[r] = fast_exp2(__builtin_fmaf(s[qb][kb][r], c, negm));
                    ls += e[r];
                }
                p[qb][kb * 2 + 0] = VT::pack(e);
                p[qb][kb * 2 + 1] = VT::pack(e + 8);
            }
            l_run[qb] += ls;
        }
    }

    // O^T += V^T P^T for one tile (V^T operands through transposing LDS reads)
    static __device__ __forceinline__ void pv(const char* vl, const x8 (&p)[QB][4], f32x16 (&oacc)[QB][CB],
                                              int vbase_e, int vbase_o) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                x4 half[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    // 64-byte chunk group after the row's swizzle bit 3 (present when CPR >= 16)
                    const int cp = cb ^ (CPR >= 16 ? 2 * u : 0);
                    const int base = (cp & 1) ? vbase_o : vbase_e;
                    half[u] = VT::read_tr(vl + base + (s * 16 + u * 4) * CPR * 16 + cp * 64);
                }
                const x8 vop = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[qb][cb] = VT::mfma(vop, p[qb][s], oacc[qb][cb]);
            }
        }
    }

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, T* __restrict__ O,
                                               float* __restrict__ LSE, int N, int BH, int ntq, float c,
                                               uint32_t qflip, char* smem) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31;
        const int h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

        int bh, qt;
        map_block(blockIdx.x, BH, ntq, CAUSAL, bh, qt);
        const size_t head = (size_t)bh * N * D;
        const T* Qh = Q + head;
        const T* Kh = K + head;
        const T* Vh = V + head;
        const int q0 = qt * BM;
        const int q0w = q0 + wave * QW;
        const int nt = ((CAUSAL ? min(N, q0 + BM) : N) + BN - 1) / BN;   // tiles of the workgroup
        const int ntw = ((CAUSAL ? min(N, q0w + QW) : N) + BN - 1) / BN; // tiles this wave computes

        // per-lane LDS offsets
        const int kperm = ((n32 >> 4) & 1) * 16 + ((n32 >> 2) & 1) * 8 + ((n32 >> 3) & 1) * 4 + (n32 & 3);
        const int kbase = kperm * CPR * 16;
        const int ksw = swz<CPR>(kperm);
        const int i16 = lane & 15, G = lane >> 4;
        const int vrow = (G >> 1) * 8 + (i16 >> 2);
        const int vl_sw = ((i16 >> 2) << 1) | (G >> 1);         // swizzle bits of vrow (bit 2 = u)
        const int vcc = (G & 1) * 2 + ((i16 & 3) >> 1);          // 16-byte chunk within 32 columns
        const int b2 = (vl_sw >> 2) & 1;
        const int vbase = vrow * CPR * 16 + ((vcc ^ vl_sw) & 3) * 16 + (i16 & 1) * 8;
        const int vbase_e = vbase + 64 * b2, vbase_o = vbase - 64 * b2;

        // ---- prologue: Q, K_0, V_0 (and K_1) into LDS ----
        copy_rows<TL::QLPT>(Qh, q0, N, lbase + OFF_Q, tid, wave);
        copy_rows<LPT>(Kh, 0, N, lbase + OFF_K0, tid, wave);
        copy_rows<LPT>(Vh, 0, N, lbase + OFF_V0, tid, wave);
        if constexpr (TL::Q_SEPARATE) {
            if (nt > 1) {
                copy_rows<LPT>(Kh, BN, N, lbase + OFF_K1, tid, wave);
                wait_vmcnt<2 * LPT>();
            } else {
                wait_vmcnt<LPT>();
            }
        } else {
            wait_vmcnt<LPT>();
        }
        lds_barrier();

        x8 qreg[QB][KS];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = wave * QW + qb * 32 + n32;
            const char* qrow = smem + OFF_Q + row * CPR * 16;
            const int qsw = swz<CPR>(row);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                i32x4 raw = *(const i32x4*)(qrow + ((2 * ks + h) ^ qsw) * 16);
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

        f32x16 s0[QB][2], s1[QB][2];
        scores(smem + OFF_K0, qreg, s0, kbase, h, ksw);
        if constexpr (!TL::Q_SEPARATE) {
            lds_barrier();  // every wave has its Q operand: stage 1 may be overwritten
            if (nt > 1) copy_rows<LPT>(Kh, BN, N, lbase + OFF_K1, tid, wave);
        }

        // ---- main loop: iteration j holds K_{j+1} and V_j, copies K_{j+2} and V_{j+1} ----
        auto iteration = [&](int j, f32x16 (&cur)[QB][2], f32x16 (&nxt)[QB][2], int okn, int ov, uint32_t dk,
                             uint32_t dv) {
            wait_vmcnt<0>();
            lds_barrier();
            if (j + 2 < nt) copy_rows<LPT>(Kh, (j + 2) * BN, N, lbase + dk, tid, wave);
            if (j + 1 < nt) copy_rows<LPT>(Vh, (j + 1) * BN, N, lbase + dv, tid, wave);
            if (j < ntw) {
                mask(cur, j * BN, N, q0w, n32, h);
                update_max(cur, c, oacc, m_run, l_run);
                x8 p[QB][4];
                if (j + 1 < ntw) {
                    scores(smem + okn, qreg, nxt, kbase, h, ksw);
                    exps(cur, c, m_run, l_run, p);
                } else {
                    exps(cur, c, m_run, l_run, p);
                }
                pv(smem + ov, p, oacc, vbase_e, vbase_o);
            }
        };
        for (int j = 0; j < nt; j += 2) {
            // even j: K_{j+1} in stage 1, V_j in stage 0; copies K_{j+2} -> stage 0, V_{j+1} -> stage 1
            iteration(j, s0, s1, OFF_K1, OFF_V0, OFF_K0, OFF_V1);
            if (j + 1 < nt) iteration(j + 1, s1, s0, OFF_K0, OFF_V1, OFF_K1, OFF_V0);
        }

        // ---- epilogue: O = acc / l (rounded to T), lse = ln2 * (m + log2 l) ----
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = halves_sum(l_run[qb]);
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
    __shared__ __attribute__((aligned(1024))) char smem[Tile<D, QB, NW>::LDS_BYTES];
    Fwd<T, D, QB, NW, CAUSAL>::run(Q, K, V, O, LSE, N, BH, ntq, c, qflip, smem);
}

// per head dimension: query blocks per wave and waves per workgroup
template <int D> struct Shape;
template <> struct Shape<64> { static constexpr int QB = 1, NW = 8; };
template <> struct Shape<128> { static constexpr int QB = 1, NW = 8; };
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
            return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_fwd_16(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                         int N, int d, bool causal, float c, uint32_t qflip, hipStream_t stream) {
    return is_bf16 ? dispatch16<__bf16>(q, k, v, o, lse, BH, N, d, causal, c, qflip, stream)
                   : dispatch16<_Float16>(q, k, v, o, lse, BH, N, d, causal, c, qflip, stream);
}

}  // namespace fa
