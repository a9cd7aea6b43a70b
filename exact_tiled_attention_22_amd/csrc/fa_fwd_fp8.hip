// fa_fwd_fp8.hip — tiled attention forward with OCP e4m3 operands on gfx950 (bf16 output).
//
// Same method as the 16-bit kernel (concept card "FlashAttention 2 + 3 — speicherbewusste
// Attention-Kernels", "Kernpunkte"; glossary entry "Online-Softmax") with the FP8 ingredients of the
// FlashAttention-3 article ("Drei technische Hebel", item 3 "FP8-Blockquantisierung"): Q, K and V
// arrive as e4m3 codes with one float32 scale per 64 rows (written by the preparation kernel), both
// products run on the gfx950 8-bit matrix instruction v_mfma_f32_32x32x64_f8f6f4 with float32
// accumulation, and the probabilities are rounded to e4m3 for the second product.
//
// How the scales enter (value of element [b,h,n,:] = code * scale[b*H+h][n/64]):
//   * scores: s_ij = (q8_i . k8_j) * sq[i/64] * sk[j/64] * scale.  A wave's 32 query rows share one
//     Q block and a 64-key tile is one K block, so the per-tile softmax constant
//     c_j = |scale| log2(e) sq sk[j] absorbs both scales: p = 2^(s8 * c_j - m);
//   * values: O_i = sum_j p_ij sv[j/64] v8_j / l_i.  The kernel rounds p~ = p * 2^6 to e4m3 (an exact
//     power-of-two boost that lifts most probabilities out of e4m3's subnormal range, below 2^-6; the
//     largest probability of a row, 1 when the running maximum was just set, stays exact), multiplies
//     each 64-key tile's values on the MFMA with a zero accumulator, T = v8^T p~^T, and adds T * sv[j]
//     to the float32 output accumulator.  The V block scale thus never enters the rounded operand:
//     folding it into p~ made the dominant probability of a row a non-power-of-two that e4m3 rounds
//     by up to 2^-4.  The row sum keeps the unrounded p (l += sum(p~) * 2^-6) and the epilogue divides
//     by 2^6 l.  The running maximum is corrected as soon as it grows by more than 2^2, so p <= 4 and
//     p~ <= 256 stays inside e4m3's range (448).  A zero V scale makes its block contribute nothing.
//
// Layouts as in the 16-bit kernel (S^T = K Q^T, O^T += V^T P^T), adapted to 64-wide k-steps: the K
// rows feeding the score MFMA are permuted so that wave half h holds the scores of keys h*32 + 0..31
// of the tile, which is the k-order the P*V MFMA needs; V^T operands come through the transposing
// byte read ds_read_b64_tr_b8 (4 reads give a lane 32 keys of one column).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kTau8 = 2.0f;    // running-maximum slack (base 2)
constexpr float kBoost8 = 6.0f;  // p~ carries an extra 2^6; kTau8 + kBoost8 <= 8 keeps p~ <= 256

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // A and B in e4m3 (format code 0), no block scaling
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D>
struct Tile8 {
    // 4-wave workgroups, two per CU (independent workgroups overlap one's matrix work with the
    // other's softmax better than one 8-wave workgroup does); d = 256 needs 128 KiB: 8 waves, one per CU
    static constexpr int NW = D == 256 ? 8 : 4;
    static constexpr int WPC = D == 256 ? 1 : 2;
    static constexpr int THREADS = 64 * NW;
    static constexpr int BN = 64, QW = 32, BM = QW * NW;
    static constexpr int CPR = D / 16;  // 16-byte chunks per row (1-byte elements)
    static constexpr int CHUNKS = BN * CPR;
    static constexpr int LPT = CHUNKS / THREADS;
    static constexpr int KV_BYTES = CHUNKS * 16;
    static constexpr int Q_CHUNKS = BM * CPR;
    static constexpr int QLPT = Q_CHUNKS / THREADS;
    static constexpr int Q_BYTES = Q_CHUNKS * 16;
    static constexpr int OFF_K0 = 0, OFF_V0 = KV_BYTES, OFF_K1 = 2 * KV_BYTES, OFF_V1 = 3 * KV_BYTES;
    static constexpr int OFF_Q = 4 * KV_BYTES;
    static constexpr int LDS_BYTES = 4 * KV_BYTES + Q_BYTES;
    static_assert(LPT >= 1 && CHUNKS % THREADS == 0 && Q_CHUNKS % THREADS == 0, "tiles split evenly");
    static_assert(LDS_BYTES <= 160 * 1024 / WPC, "LDS budget");
    static_assert(BM * D * 2 <= LDS_BYTES, "bf16 output staging fits the workgroup's LDS");
};

// Tiles of 1-byte elements: row-major rows of CPR 16-byte chunks, chunk c of row r at slot
// r * CPR + (c ^ swz8(r)) (128- or 256-byte rows: 3 bits; 64-byte rows: 2 bits).  Rows read together by
// one operand fetch differ in (row >> 1) & 3 and in bit 5, rows of equal parity then land in distinct
// 16-byte bank groups.  Copied with fa_common.h's copy_tile.
template <int CPR>
__device__ __forceinline__ int swz8(int row) {
    int f = (row >> 1) & 3;
    if constexpr (CPR >= 8) f |= ((row >> 5) & 1) << 2;
    return f;
}

template <int CPR>
struct Rows8 {
    __device__ static __forceinline__ int slot(int row, int c) { return row * CPR + (c ^ swz8<CPR>(row)); }
    __device__ static __forceinline__ void row_chunk(int slot, int& row, int& c) {
        row = slot / CPR;
        c = (slot % CPR) ^ swz8<CPR>(row);
    }
};

template <int D, bool CAUSAL>
struct Fwd8 {
    using TL = Tile8<D>;
    static constexpr int NW = TL::NW, BN = TL::BN, QW = TL::QW, BM = TL::BM, CPR = TL::CPR, LPT = TL::LPT;
    static constexpr int KS = D / 64;  // k-steps of the score product
    static constexpr int CB = D / 32;  // 32-column output blocks

    // Copy rows [r0, r0 + ROWS) into an LDS tile (a ragged last tile reads row N-1 in place of the
    // missing rows), ROWS = NLOADS * THREADS / CPR.
    template <int NLOADS>
    static __device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ src, int r0, int N, uint32_t lds,
                                                     int tid, int wave) {
        copy_tile<Rows8<CPR>, NLOADS * TL::THREADS / CPR, CPR, TL::THREADS>(src, r0, N, D, lds, tid, wave);
    }

    static __device__ __forceinline__ i32x8 read32(const char* base, int row, int c) {
        const i32x4 a = *(const i32x4*)(base + Rows8<CPR>::slot(row, c) * 16);
        const i32x4 b = *(const i32x4*)(base + Rows8<CPR>::slot(row, c + 1) * 16);
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // S^T = K8 Q8^T (raw code products, fp32 accumulate)
    static __device__ __forceinline__ void scores(const char* kl, const i32x8 (&qreg)[KS], f32x16 (&s)[2], int krow0,
                                                  int h) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_fp8(read32(kl, krow0 + kb * 16, ks * 4 + h * 2), qreg[ks], s[kb]);
    }

    static __device__ __forceinline__ void run(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                               const uint8_t* __restrict__ V, __bf16* __restrict__ O,
                                               float* __restrict__ LSE, const float* __restrict__ SQ,
                                               const float* __restrict__ SK, const float* __restrict__ SV, int N,
                                               int BH, int ntq, float c, int qflip, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        int bh, qt;
        map_block(blockIdx.x, BH, ntq, CAUSAL, bh, qt);
        const size_t head = (size_t)bh * N * D;
        const uint8_t* Qh = Q + head;
        const uint8_t* Kh = K + head;
        const uint8_t* Vh = V + head;
        const int q0 = qt * BM, q0w = q0 + wave * QW;
        const int nt = ((CAUSAL ? min(N, q0 + BM) : N) + BN - 1) / BN;
        const int ntw = ((CAUSAL ? min(N, q0w + QW) : N) + BN - 1) / BN;
        const int nblk = (N + 63) / 64;
        const size_t srow = (size_t)bh * nblk;

        // K row of lane n32 = 8a + 4g + b in 32-key block kb: g*32 + kb*16 + 4a + b
        const int krow0 = ((n32 >> 2) & 1) * 32 + (n32 >> 3) * 4 + (n32 & 3);
        // transposing V reads: lane = 16 G + i
        const int i16 = lane & 15, G = lane >> 4;
        const int vkey = (G >> 1) * 32 + (i16 >> 1);  // + u*8
        const int vchunk = G & 1;                      // + cb*2
        const int vbyte = (i16 & 1) * 8;

        copy_rows<TL::QLPT>(Qh, q0, N, lbase + TL::OFF_Q, tid, wave);
        copy_rows<LPT>(Kh, 0, N, lbase + TL::OFF_K0, tid, wave);
        copy_rows<LPT>(Vh, 0, N, lbase + TL::OFF_V0, tid, wave);
        if (nt > 1) {
            copy_rows<LPT>(Kh, BN, N, lbase + TL::OFF_K1, tid, wave);
            wait_vmcnt<2 * LPT>();
        } else {
            wait_vmcnt<LPT>();
        }
        lds_barrier();

        // this wave's Q block scale
        const float sq = SQ != nullptr ? SQ[srow + min(q0w, N - 1) / 64] : 1.0f;
        // this tile's K and V block scales, loaded one tile ahead (scalar loads, so that no tile waits
        // on the scalar cache)
        float sk_j = 1.0f, sv_j = 1.0f;
        if (SQ != nullptr) {
            sk_j = SK[srow];
            sv_j = SV[srow];
        }

        i32x8 qreg[KS];
        {
            const int row = wave * QW + n32;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qreg[ks] = read32(smem + TL::OFF_Q, row, ks * 4 + h * 2) ^ qflip;
        }
        f32x16 oacc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
        // d = 128: a tile's values T (and its V scale) wait in registers until the next iteration adds
        // them to the accumulator, so that the matrix latency is covered (e4m3 B4 H16 N4096: 345 -> 326 us;
        // d = 64 measured slower with it, d = 256 has no registers for it)
        constexpr bool DEFER = D == 128;
        f32x16 tv[DEFER ? CB : 1];
        float wpend = 0.0f;
#pragma unroll
        for (int cb = 0; cb < (DEFER ? CB : 1); ++cb) tv[cb] = f32x16{};
        float m_run = -INFINITY, l_run = 0.0f;

        f32x16 s0[2], s1[2];
        scores(smem + TL::OFF_K0, qreg, s0, krow0, h);

        auto iteration = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], int okn, int ov, uint32_t dk, uint32_t dv) {
            wait_vmcnt<0>();
            lds_barrier();
            if (j + 2 < nt) copy_rows<LPT>(Kh, (j + 2) * BN, N, lbase + dk, tid, wave);
            if (j + 1 < nt) copy_rows<LPT>(Vh, (j + 1) * BN, N, lbase + dv, tid, wave);
            if (j >= ntw) return;
            const int kv0 = j * BN;
            float cj = c * sq;
            const float wv = sv_j;  // this tile's V block scale
            if (SQ != nullptr) {
                cj *= sk_j;
                const int jn = min(j + 1, nblk - 1);
                sk_j = SK[srow + jn];
                sv_j = SV[srow + jn];
            }
            // mask
            if ((kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > q0w)) {
                const int query = q0w + n32;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + h * 32 + kb * 16 + r;
                        if (key >= N || (CAUSAL && key > query)) cur[kb][r] = -INFINITY;
                    }
            }
            if constexpr (DEFER) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[cb][r] = __builtin_fmaf(tv[cb][r], wpend, oacc[cb][r]);
            }
            // running maximum with lazy correction
            {
                // 32 values -> 1 through 3-input maxima only (a value counted twice is harmless; a
                // 2-input maximum of matrix results costs two extra canonicalising instructions)
                float t1[11];
#pragma unroll
                for (int i = 0; i < 10; ++i) {
                    const int a = 3 * i, b = 3 * i + 1, e = 3 * i + 2;
                    t1[i] = max3(cur[a >> 4][a & 15], cur[b >> 4][b & 15], cur[e >> 4][e & 15]);
                }
                t1[10] = max3(cur[1][14], cur[1][15], cur[0][0]);
                const float t2a = max3(t1[0], t1[1], t1[2]), t2b = max3(t1[3], t1[4], t1[5]);
                const float t2c = max3(t1[6], t1[7], t1[8]), t2d = max3(t1[9], t1[10], t1[0]);
                const float mx = max3(max3(t2a, t2b, t2c), t2d, t2a);
                const float mt = halves_max(mx) * cj;
                if (__ballot(mt > m_run + kTau8)) {
                    const float mn = fmaxf(m_run, mt);
                    const float alpha = fast_exp2(m_run - mn);
                    m_run = mn;
                    l_run *= alpha;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
                }
            }
            // d = 128: the next tile's scores are always computed (on a wave's last tile from a stage
            // that holds some earlier tile: in bounds, result unused) so that they sit in one basic
            // block with the exponentials and the value products, which the schedule below interleaves;
            // the wave runs at raised priority meanwhile, as in the 16-bit kernel.  d = 256 has no
            // registers to spare for that, and d = 64 (two score MFMAs per tile) measured slower with
            // it; both keep the branch.
            if constexpr (D == 128) {
                __builtin_amdgcn_s_setprio(1);
                scores(smem + okn, qreg, nxt, krow0, h);
            } else if (j + 1 < ntw) {
                scores(smem + okn, qreg, nxt, krow0, h);
            }
            // p~ = 2^(s*c_j - m + 6), rounded to e4m3, 4 per dword: keys h*32 + kb*16 + r
            i32x8 p;
            float part[8];  // row sum as a shallow tree: 4-term partial sums, then pairs
            const float add = kBoost8 - m_run;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    float e[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) e[t] = fast_exp2(__builtin_fmaf(cur[kb][w4 * 4 + t], cj, add));
                    part[kb * 4 + w4] = (e[0] + e[1]) + (e[2] + e[3]);
                    int wd = 0;
                    wd = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], wd, false);
                    wd = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], wd, true);
                    p[kb * 4 + w4] = wd;
                }
            const float ls = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
            l_run += ls * (1.0f / 64.0f);
            // O^T += V8^T P~^T
            const char* vl = smem + ov;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                i32x8 vop;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int key = vkey + u * 8;
                    const int ch = cb * 2 + vchunk;
                    const i32x2 t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (FA_LDS i32x2*)(vl + Rows8<CPR>::slot(key, ch) * 16 + vbyte));
                    vop[2 * u] = t2[0];
                    vop[2 * u + 1] = t2[1];
                }
                // this tile's values alone, then scaled by its V block scale into the accumulator
                if constexpr (DEFER) {
                    tv[cb] = mfma_fp8(vop, p, f32x16{});
                } else {
                    const f32x16 t = mfma_fp8(vop, p, f32x16{});
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[cb][r] = __builtin_fmaf(t[r], wv, oacc[cb][r]);
                }
            }
            wpend = wv;
            if constexpr (D == 128) {
                // each score MFMA followed by 8 vector instructions of the softmax (its K operands two
                // ahead), then each value MFMA with the next V operand reads and 8 more
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 2 * KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 2 < 2 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < CB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 1 < CB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
                __builtin_amdgcn_s_setprio(0);
            }
        };
        for (int j = 0; j < nt; j += 2) {
            iteration(j, s0, s1, TL::OFF_K1, TL::OFF_V0, TL::OFF_K0, TL::OFF_V1);
            if (j + 1 < nt) iteration(j + 1, s1, s0, TL::OFF_K0, TL::OFF_V1, TL::OFF_K1, TL::OFF_V0);
        }

        if constexpr (DEFER) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] = __builtin_fmaf(tv[cb][r], wpend, oacc[cb][r]);
        }
        // the output leaves through this wave's LDS region as whole rows (every stage is free once
        // all waves are past their last tile)
        lds_barrier();
        char* wl = smem + wave * QW * D * 2;
        const float lt = halves_sum(l_run);
        const float inv = 1.0f / (64.0f * lt);  // undo the 2^kBoost8 carried by p~
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = (__bf16)(oacc[cb][g * 4 + e] * inv);
                ostage_put<D>(wl, n32, h, cb * 4 + g, out);
            }
        const int query = q0w + n32;
        if (LSE != nullptr && h == 0 && query < N)
            LSE[(size_t)bh * N + query] = (m_run + __log2f(lt)) * 0.69314718055994531f;
        ostage_flush<__bf16, D>(O + head, q0w, N, wl, lane);
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(Tile8<D>::THREADS, Tile8<D>::NW * Tile8<D>::WPC / 4) void fa_fwd8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    int N, int BH, int ntq, float c, int qflip) {
    __shared__ __attribute__((aligned(1024))) char smem[Tile8<D>::LDS_BYTES];
    Fwd8<D, CAUSAL>::run(Q, K, V, O, LSE, SQ, SK, SV, N, BH, ntq, c, qflip, smem);
}

template <int D, bool CAUSAL>
hipError_t launch8(const void* q, const void* k, const void* v, void* o, float* lse, const float* sq, const float* sk,
                   const float* sv, int BH, int N, float c, int qflip, hipStream_t stream) {
    constexpr int BM = Tile8<D>::BM;
    const int ntq = (N + BM - 1) / BM;
    const long long nwg = (long long)BH * ntq;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fa_fwd8_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(Tile8<D>::THREADS), 0, stream,
                       (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (__bf16*)o, lse, sq, sk, sv, N, BH,
                       ntq, c, qflip);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, const float* sq,
                          const float* sk, const float* sv, int BH, int N, int d, bool causal, float c, bool qneg,
                          hipStream_t stream) {
    // a negative scale negates Q: flip the sign bit of every e4m3 code (exact)
    const int qflip = qneg ? (int)0x80808080u : 0;
    switch (d) {
        case 64:
            return causal ? launch8<64, true>(q, k, v, o, lse, sq, sk, sv, BH, N, c, qflip, stream)
                          : launch8<64, false>(q, k, v, o, lse, sq, sk, sv, BH, N, c, qflip, stream);
        case 128:
            return causal ? launch8<128, true>(q, k, v, o, lse, sq, sk, sv, BH, N, c, qflip, stream)
                          : launch8<128, false>(q, k, v, o, lse, sq, sk, sv, BH, N, c, qflip, stream);
        case 256:
            return causal ? launch8<256, true>(q, k, v, o, lse, sq, sk, sv, BH, N, c, qflip, stream)
                          : launch8<256, false>(q, k, v, o, lse, sq, sk, sv, BH, N, c, qflip, stream);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace fa
