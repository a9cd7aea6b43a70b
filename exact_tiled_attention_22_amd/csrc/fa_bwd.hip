// fa_bwd.hip — attention backward (dQ, dK, dV) for 16-bit floats on gfx950.
//
// The pages name the backward pass ("FlashAttention 2 + 3 — speicherbewusste Attention-Kernels",
// "Kernpunkte": FlashAttention 2 gains from better parallelism in it) without writing it out.  What
// is computed is the derivative of the attention definition for a given output gradient dO, using
// the row log-sum-exp saved by the forward pass:
//     P = exp(scale Q K^T - lse)   (visible keys),   D_i = sum_t dO[i,t] O[i,t],
//     dS = P o (dO V^T - D),   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
// Like the forward pass it never stores an N x N matrix: P and dS are rebuilt tile by tile from Q,
// K and lse.  Two launches, no atomics (the result is deterministic):
//   1. BwdQ: one workgroup per 128 query rows first forms D = rowsum(dO o O) for its rows (writing it
//      to a caller-provided float32 [B,H,N] buffer), then streams the K/V tiles (as the forward pass
//      does) and accumulates dQ^T = K^T dS^T in registers;
//   2. BwdKV: one workgroup per 128 keys (V rows held in LDS, K rows in registers) streams the Q/dO
//      tiles (with their lse and D) and accumulates dV^T = dO^T P and dK^T = Q^T dS in registers.
// Operand conventions are the forward pass's: v_mfma_f32_32x32x16 with the A-operand rows permuted
// so that 8 consecutive accumulator registers of a lane hold 8 consecutive rows (keys in BwdQ,
// queries in BwdKV), which lets P and dS feed the next MFMA as its B operand in place, and
// transposed operands (K^T, dO^T, Q^T) read from LDS with ds_read_b64_tr_b16.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Per-lane fetch geometry inside an LDS tile (row-major rows, XOR chunk swizzle: XorRows in
// fa_common.h), lane = 32 h + n32.
template <int CPR>
struct Geo {
    using L = XorRows<CPR>;
    int prow, h;        // A operand: permuted row prow (+32 for the second block), chunk 2*ks + h
    int trow, tcc, tb;  // transposing read: row u*4 + trow, chunk cb*4 + tcc, byte tb
    __device__ __forceinline__ Geo(int lane) {
        const int n32 = lane & 31;
        h = lane >> 5;
        prow = ((n32 >> 4) & 1) * 16 + ((n32 >> 2) & 1) * 8 + ((n32 >> 3) & 1) * 4 + (n32 & 3);
        const int i16 = lane & 15, G = lane >> 4;
        trow = (G >> 1) * 8 + (i16 >> 2);
        tcc = (G & 1) * 2 + ((i16 & 3) >> 1);
        tb = (i16 & 1) * 8;
    }
    // A operand for k-step ks of row block rb
    __device__ __forceinline__ int aoff(int rb, int ks) const { return L::slot(rb * 32 + prow, 2 * ks + h) * 16; }
    // transposed operand (rows = d block cb, contraction = 16 tile rows from 16 * st), half u
    __device__ __forceinline__ int toff(int cb, int st, int u) const {
        return L::slot(st * 16 + u * 4 + trow, cb * 4 + tcc) * 16 + tb;
    }
};

// A value the optimiser cannot see through.  The non-causal d = 256 kernels pass their per-wave tile
// bound through it so that the tile step's early exit stays a branch: without it the step becomes
// one scheduling region and 79 (dQ) / 200 (dK/dV) registers spill.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// ---------------------------------------------------------------------------------------------
// D = rowsum(dO o O) in float32 for this lane's query row.  Lane (n32, h) holds the row's 16-byte
// chunks 2 ks + h (ks < KS) of dO in dreg and reads the same chunks of O.  Each chunk is a chain of
// fused multiply-adds; the chunk sums then combine as a butterfly from the widest distance down (chunk
// distance D/16 ... 2 inside the lane, distance 1 across the two wave halves), one fixed order.
template <typename T, int KS>
__device__ __forceinline__ float row_delta(const T* __restrict__ orow, int h, const typename Vec<T>::x8 (&dreg)[KS]) {
    using x8 = typename Vec<T>::x8;
    float p[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const x8 o = *(const x8*)(orow + ks * 16 + h * 8);
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = __builtin_fmaf((float)o[e], (float)dreg[ks][e], a);
        p[ks] = a;
    }
#pragma unroll
    for (int off = KS / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int ks = 0; ks < off; ++ks) p[ks] = p[ks] + p[ks + off];
    return halves_sum(p[0]);
}

// ---------------------------------------------------------------------------------------------
// dQ: one workgroup = 4 waves x 32 query rows; key/value tiles of 64 rows.  d <= 128 (run_pipe) runs
// the scores one tile ahead with three K and two V stages; d = 256 (run) takes each tile in order
// with two stages each (the pipelined form measured slower there).
template <typename T, int D, bool CAUSAL>
struct BwdQ {
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    static constexpr int NW = 4, THREADS = 256, QW = 32, BM = NW * QW, BN = 64;
    static constexpr int CPR = D / 8, KS = D / 16, CB = D / 32;
    static constexpr int TILE = BN * CPR * 16;
    // d <= 128 (run_pipe): K0 | K1 | K2 | V0 | V1; d = 256 (run): K0 | V0 | K1 | V1
    static constexpr bool PIPE = D <= 128;
    static constexpr int LDS_BYTES = (PIPE ? 5 : 4) * TILE;
    static constexpr int OFF_V = 3 * TILE;

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, const T* __restrict__ dO,
                                               const T* __restrict__ O, const float* __restrict__ LSE,
                                               float* __restrict__ Dl, T* __restrict__ dQ, int N, int BH, int ntq,
                                               float c, float scale, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        int bh, qt;
        map_block(blockIdx.x, BH, ntq, CAUSAL, bh, qt);
        const size_t head = (size_t)bh * N * D;
        const int q0 = qt * BM, q0w = q0 + wave * QW, query = q0w + n32, qrow = min(query, N - 1);
        const int nt = ((CAUSAL ? min(N, q0 + BM) : N) + BN - 1) / BN;
        const int ntw = CAUSAL ? (min(N, q0w + QW) + BN - 1) / BN : (D >= 256 ? opaque(nt) : nt);
        const Geo<CPR> g(lane);

        // B operands of S^T = K Q^T and dP^T = V dO^T: this lane's query row, 8 columns per k-step
        x8 qreg[KS], dreg[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks] = *(const x8*)(Q + head + (size_t)qrow * D + ks * 16 + h * 8);
            dreg[ks] = *(const x8*)(dO + head + (size_t)qrow * D + ks * 16 + h * 8);
        }
        const float lse2 = LSE[(size_t)bh * N + qrow] * kLog2e;
        // D for this row, written once (by the lower wave half) for the dK/dV kernel
        const float dd = row_delta<T, KS>(O + head + (size_t)qrow * D, h, dreg);
        if (h == 0 && query < N) Dl[(size_t)bh * N + query] = dd;
        copy_tile<XorRows<CPR>, BN, CPR, THREADS>(K + head, 0, N, D * 2, lbase, tid, wave);
        copy_tile<XorRows<CPR>, BN, CPR, THREADS>(V + head, 0, N, D * 2, lbase + TILE, tid, wave);

        f32x16 acc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};

        auto iteration = [&](int j, int ok, int ov, uint32_t dk, uint32_t dv) {
            wait_vmcnt<0>();
            lds_barrier();
            if (j + 1 < nt) {
                copy_tile<XorRows<CPR>, BN, CPR, THREADS>(K + head, (j + 1) * BN, N, D * 2, lbase + dk, tid, wave);
                copy_tile<XorRows<CPR>, BN, CPR, THREADS>(V + head, (j + 1) * BN, N, D * 2, lbase + dv, tid, wave);
            }
            if (j >= ntw) return;
            const char* kl = smem + ok;
            const char* vl = smem + ov;
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = dp[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    s[kb] = VT::mfma(*(const x8*)(kl + g.aoff(kb, ks)), qreg[ks], s[kb]);
                    dp[kb] = VT::mfma(*(const x8*)(vl + g.aoff(kb, ks)), dreg[ks], dp[kb]);
                }
                if constexpr (D >= 256)
                    if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
            // dS^T = P^T o (dP^T - D): register r of key block kb holds key kb*32 + (r/8)*16 + h*8 + r%8
            x8 ds[4];
            const bool edge = (j * BN + BN > N) || (CAUSAL && j * BN + BN - 1 > q0w);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    float v8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int r = hf * 8 + e;
                        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -lse2));
                        if (edge) {
                            const int key = j * BN + kb * 32 + hf * 16 + h * 8 + e;
                            if (key >= N || (CAUSAL && key > query)) p = 0.0f;
                        }
                        v8[e] = p * (dp[kb][r] - dd);
                    }
                    ds[kb * 2 + hf] = VT::pack(v8);
                }
            }
            // dQ^T += K^T dS^T over the tile's four 16-key steps
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const x4 lo = VT::read_tr(kl + g.toff(cb, st, 0));
                    const x4 hi = VT::read_tr(kl + g.toff(cb, st, 1));
                    acc[cb] = VT::mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), ds[st], acc[cb]);
                    // d = 256: keep the scheduler from hoisting every operand read of the tile (registers)
                    if constexpr (D >= 256)
                        if (cb & 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (D <= 128) {
                // S^T / dP^T MFMAs two at a time behind their operand reads, then dQ MFMAs behind theirs
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 2 * KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    if (i + 2 < 2 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 4 * CB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 2 < 4 * CB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
        };
        for (int j = 0; j < nt; j += 2) {
            iteration(j, 0, TILE, 2 * TILE, 3 * TILE);
            if (j + 1 < nt) iteration(j + 1, 2 * TILE, 3 * TILE, 0, TILE);
        }
        if (query < N) {
            T* row = dQ + head + (size_t)query * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = (T)(acc[cb][gq * 4 + e] * scale);
                    *(x4*)(row + cb * 32 + gq * 8 + h * 4) = out;
                }
        }
    }

    // d <= 128: the scores run one tile ahead.  The iteration of key tile j first computes dP_j while the
    // exponentials of S_j (from the previous iteration) run beside it, then dS_j, the dQ products, and
    // S_{j+1} behind them; K has three LDS stages (K_j for dQ, K_{j+1} for S_{j+1}, K_{j+2} in flight),
    // V two.  80 KiB of LDS at d = 128, two workgroups per CU.
    static __device__ __forceinline__ void run_pipe(const T* __restrict__ Q, const T* __restrict__ K,
                                                    const T* __restrict__ V, const T* __restrict__ dO,
                                                    const T* __restrict__ O, const float* __restrict__ LSE,
                                                    float* __restrict__ Dl, T* __restrict__ dQ, int N, int BH,
                                                    int ntq, float c, float scale, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        int bh, qt;
        map_block(blockIdx.x, BH, ntq, CAUSAL, bh, qt);
        const size_t head = (size_t)bh * N * D;
        const int q0 = qt * BM, q0w = q0 + wave * QW, query = q0w + n32, qrow = min(query, N - 1);
        // key tiles of the workgroup; a wave's tiles past its own last query (at most two, causal) are
        // fully masked and add zero, which costs less than a branch in the loop
        const int nt = ((CAUSAL ? min(N, q0 + BM) : N) + BN - 1) / BN;
        const float hidden = c > 0.0f ? -INFINITY : INFINITY;  // score of a hidden key: 2^(hidden c) = 0
        const Geo<CPR> g(lane);
        int ao[KS], to[CB][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ao[ks] = g.aoff(0, ks);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int u = 0; u < 2; ++u) to[cb][u] = g.toff(cb, 0, u);

        x8 qreg[KS], dreg[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks] = *(const x8*)(Q + head + (size_t)qrow * D + ks * 16 + h * 8);
            dreg[ks] = *(const x8*)(dO + head + (size_t)qrow * D + ks * 16 + h * 8);
        }
        const float lse2 = LSE[(size_t)bh * N + qrow] * kLog2e;
        // D for this row, written once (by the lower wave half) for the dK/dV kernel
        const float dd = row_delta<T, KS>(O + head + (size_t)qrow * D, h, dreg);
        if (h == 0 && query < N) Dl[(size_t)bh * N + query] = dd;
        auto copy_k = [&](int j, int st) {
            copy_tile<XorRows<CPR>, BN, CPR, THREADS>(K + head, j * BN, N, D * 2, lbase + st * TILE, tid, wave);
        };
        auto copy_v = [&](int j, int st) {
            copy_tile<XorRows<CPR>, BN, CPR, THREADS>(V + head, j * BN, N, D * 2, lbase + OFF_V + st * TILE, tid,
                                                      wave);
        };
        // S^T = K_tile Q^T for the tile's two 32-key blocks from K stage st
        auto scores = [&](int st, f32x16 (&s)[2]) {
            const char* kl = smem + st * TILE;
            s[0] = s[1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) s[kb] = VT::mfma(*(const x8*)(kl + kb * 32 * CPR * 16 + ao[ks]), qreg[ks], s[kb]);
        };
        copy_k(0, 0);
        if (nt > 1) copy_k(1, 1);
        copy_v(0, 0);
        wait_vmcnt<0>();
        lds_barrier();
        f32x16 s[2];
        scores(0, s);

        f32x16 acc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};

        // tile j at phase K = j % 6: K_j in stage K % 3, V_j in stage K % 2
        auto iteration = [&](int j, auto phase) {
            constexpr int PH = decltype(phase)::value;
            constexpr int KC = PH % 3, KN = (PH + 1) % 3, KP = (PH + 2) % 3, VC = PH % 2, VP = (PH + 1) % 2;
            wait_vmcnt<0>();
            lds_barrier();  // K_{j+1}, V_j visible; K stage KP and V stage VP are free
            if (j + 2 < nt) copy_k(j + 2, KP);
            if (j + 1 < nt) copy_v(j + 1, VP);
            const char* kl = smem + KC * TILE;
            const char* vl = smem + OFF_V + VC * TILE;
            // register r of key block kb holds key kb*32 + (r/8)*16 + h*8 + r%8
            if ((j * BN + BN > N) || (CAUSAL && j * BN + BN - 1 > q0w)) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = j * BN + kb * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                        if (key >= N || (CAUSAL && key > query)) s[kb][r] = hidden;
                    }
            }
            // dP^T = V dO^T, with P^T = 2^(S^T c - lse) beside it
            f32x16 dp[2];
            dp[0] = dp[1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) dp[kb] = VT::mfma(*(const x8*)(vl + kb * 32 * CPR * 16 + ao[ks]), dreg[ks], dp[kb]);
            float pv[32];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) pv[kb * 16 + r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -lse2));
            // dP MFMAs two at a time behind their operand reads, each pair followed by exponential work
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (i + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // dS^T = P^T o (dP^T - D)
            x8 ds[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    float v8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v8[e] = pv[kb * 16 + hf * 8 + e] * (dp[kb][hf * 8 + e] - dd);
                    ds[kb * 2 + hf] = VT::pack(v8);
                }
            __builtin_amdgcn_sched_barrier(0);
            // dQ^T += K^T dS^T over the tile's four 16-key steps
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    constexpr int SO = 16 * CPR * 16;  // the 16-key step: 16 rows further
                    const x4 lo = VT::read_tr(kl + st * SO + to[cb][0]);
                    const x4 hi = VT::read_tr(kl + st * SO + to[cb][1]);
                    acc[cb] = VT::mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), ds[st], acc[cb]);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 4 * CB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + 2 < 4 * CB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // S_{j+1} right behind them (on the last tile from a stage holding an older tile: unused)
            scores(KN, s);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (i + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        using P3 = std::integral_constant<int, 3>;
        using P4 = std::integral_constant<int, 4>;
        using P5 = std::integral_constant<int, 5>;
        // whole groups of six tiles, then the rest (no exit inside the unrolled body)
        int j = 0;
        for (; j + 6 <= nt; j += 6) {
            iteration(j, P0{});
            iteration(j + 1, P1{});
            iteration(j + 2, P2{});
            iteration(j + 3, P3{});
            iteration(j + 4, P4{});
            iteration(j + 5, P5{});
        }
        if (j < nt) iteration(j, P0{});
        if (j + 1 < nt) iteration(j + 1, P1{});
        if (j + 2 < nt) iteration(j + 2, P2{});
        if (j + 3 < nt) iteration(j + 3, P3{});
        if (j + 4 < nt) iteration(j + 4, P4{});
        if (query < N) {
            T* row = dQ + head + (size_t)query * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = (T)(acc[cb][gq * 4 + e] * scale);
                    *(x4*)(row + cb * 32 + gq * 8 + h * 4) = out;
                }
        }
    }
};

// ---------------------------------------------------------------------------------------------
// dK, dV: one workgroup = 4 waves x 32 keys.  The workgroup's 128 V rows stay in LDS for the whole
// kernel (B operand of dP = dO V^T); the K rows of a wave stay in its registers (B operand of
// S = Q K^T).  Query tiles of 32 rows stream through LDS.  A wave's scores run one tile ahead: the
// iteration of tile t first computes dP_t while the exponentials of S_t (from the previous
// iteration) run beside it, then dS_t, the dV_t and dK_t products, and S_{t+1} right behind them,
// so the exponentials no longer wait for the score MFMAs.  Q therefore has three LDS stages (Q_t for
// dK_t, Q_{t+1} for S_{t+1}, Q_{t+2} in flight), dO and lse/D two.  This keeps a wave under 256
// registers and the workgroup at 72.5 KiB of LDS (d = 128), so two workgroups share a CU.
// LDS: Q stages 0..2 | dO stages 0..1 | (lse * log2(e) [32], D [32]) stages 0..1 | V [128 rows].
template <typename T, int D, bool CAUSAL>
struct BwdKV {
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    static constexpr int NW = 4, THREADS = 256, KW = 32, BK = NW * KW, BQ = 32;
    static constexpr int CPR = D / 8, KS = D / 16, CB = D / 32;
    static constexpr int TILE = BQ * CPR * 16;
    static constexpr int VBYTES = BK * CPR * 16;
    // the stages first, so that their offsets fit a ds_read's 16-bit immediate (d <= 128)
    static constexpr int OFF_Q = 0, OFF_G = 3 * TILE, OFF_L = 5 * TILE;
    static constexpr int LSTAGE = 2 * BQ * 4;
    static constexpr int OFF_V = OFF_L + 2 * LSTAGE;
    static constexpr int LDS_BYTES = OFF_V + VBYTES;

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, const T* __restrict__ dO,
                                               const float* __restrict__ LSE, const float* __restrict__ Dl,
                                               T* __restrict__ dK, T* __restrict__ dV, int N, int BH, int nkt,
                                               float c, float scale, char* smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31, h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        int bh, t;
        map_block(blockIdx.x, BH, nkt, CAUSAL, bh, t);
        const int kt = CAUSAL ? nkt - 1 - t : t;  // causal: the first key tiles see the most queries
        const size_t head = (size_t)bh * N * D;
        const float* lseh = LSE + (size_t)bh * N;
        const float* dlh = Dl + (size_t)bh * N;
        const int k0 = kt * BK, kw0 = k0 + wave * KW, key = kw0 + n32, krow = min(key, N - 1);
        const int ntq = (N + BQ - 1) / BQ;
        // first query tile with a visible key of the workgroup; a wave's tiles before its own first one
        // (at most three) are fully masked and add zero, which costs less than a branch in the loop
        const int t0 = CAUSAL ? k0 / BQ : 0;
        const float hidden = c > 0.0f ? -INFINITY : INFINITY;  // score of a hidden key: 2^(hidden c) = 0
        const Geo<CPR> g(lane);
        const int vrow = wave * KW + n32;           // this lane's V row in LDS
        // Byte offsets of this lane's operand fetches inside a tile (A operand per k-step, transposed
        // operand per 32-column block and half; the 16-query step adds a constant) and of its V row
        int ao[KS], vo[KS], to[CB][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ao[ks] = g.aoff(0, ks);
            vo[ks] = OFF_V + XorRows<CPR>::slot(vrow, 2 * ks + g.h) * 16;
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int u = 0; u < 2; ++u) to[cb][u] = g.toff(cb, 0, u);

        // B operand of S = Q K^T: this lane's key row, 8 columns per k-step
        x8 kreg[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kreg[ks] = *(const x8*)(K + head + (size_t)krow * D + ks * 16 + h * 8);
        // lse and D of a query tile: wave 0 loads lse, wave 1 loads D, one row per lane (clamped)
        auto load_ld = [&](int tq) -> float {
            const int r = min(tq * BQ + (lane & (BQ - 1)), N - 1);
            return wave == 0 ? lseh[r] * kLog2e : dlh[r];
        };
        auto copy_q = [&](int tq, int st) {
            copy_tile<XorRows<CPR>, BQ, CPR, THREADS>(Q + head, tq * BQ, N, D * 2, lbase + OFF_Q + st * TILE, tid,
                                                      wave);
        };
        auto copy_g = [&](int tq, int st) {
            copy_tile<XorRows<CPR>, BQ, CPR, THREADS>(dO + head, tq * BQ, N, D * 2, lbase + OFF_G + st * TILE, tid,
                                                      wave);
        };
        // S = Q_tile K^T for this wave's keys from Q stage st
        auto scores = [&](int st, f32x16& s) {
            const char* ql = smem + OFF_Q + st * TILE;
            s = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s = VT::mfma(*(const x8*)(ql + ao[ks]), kreg[ks], s);
                if constexpr (D >= 256)
                    if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        };

        copy_tile<XorRows<CPR>, BK, CPR, THREADS>(V + head, k0, N, D * 2, lbase + OFF_V, tid, wave);
        float ldv = 0.0f;
        if (t0 < ntq) {
            copy_q(t0, 0);
            if (t0 + 1 < ntq) copy_q(t0 + 1, 1);
            copy_g(t0, 0);
            if (wave < 2) ldv = load_ld(t0);
        }
        wait_vmcnt<0>();
        lds_barrier();
        // S_{t0} (used only when this wave sees tile t0; stage 0 holds valid data either way)
        f32x16 s;
        scores(0, s);

        f32x16 adk[CB], adv[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) adk[cb] = adv[cb] = f32x16{};

        // tile tq at phase K = (tq - t0) % 6: Q_tq in stage K % 3, dO_tq and lse/D in stage K % 2
        auto iteration = [&](int tq, auto phase) {
            constexpr int PH = decltype(phase)::value;
            constexpr int QC = PH % 3, QN = (PH + 1) % 3, QP = (PH + 2) % 3, GC = PH % 2, GP = (PH + 1) % 2;
            wait_vmcnt<0>();
            if (wave < 2 && lane < BQ) *(float*)(smem + OFF_L + GC * LSTAGE + wave * BQ * 4 + lane * 4) = ldv;
            lds_barrier();  // Q_{tq+1}, dO_tq, lse/D_tq visible; Q stage QP and dO stage GP are free
            if (tq + 2 < ntq) copy_q(tq + 2, QP);
            if (tq + 1 < ntq) {
                copy_g(tq + 1, GP);
                if (wave < 2) ldv = load_ld(tq + 1);
            }
            const char* ql = smem + OFF_Q + QC * TILE;
            const char* gl = smem + OFF_G + GC * TILE;
            const float* lsl = (const float*)(smem + OFF_L + GC * LSTAGE);
            const float* dsl = lsl + BQ;
            // register r holds query (r/8)*16 + h*8 + r%8 of the tile, key `key`
            if ((tq * BQ + BQ > N) || (CAUSAL && kw0 + KW - 1 > tq * BQ)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qq = tq * BQ + (r >> 3) * 16 + h * 8 + (r & 7);
                    if (qq >= N || (CAUSAL && key > qq)) s[r] = hidden;
                }
            }
            // dP_t = dO_t V^T, with P_t = 2^(S_t c - lse) beside it
            f32x16 dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const x8 vop = *(const x8*)(smem + vo[ks]);
                dp = VT::mfma(*(const x8*)(gl + ao[ks]), vop, dp);
                if constexpr (D >= 256)
                    if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
            float pv[16];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int qi = st * 16 + h * 8;
                const f32x4 l0 = *(const f32x4*)(lsl + qi), l1 = *(const f32x4*)(lsl + qi + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[st * 8 + e] = fast_exp2(__builtin_fmaf(s[st * 8 + e], c, -(e < 4 ? l0[e] : l1[e - 4])));
            }
            if constexpr (D <= 128) {
                // dP MFMAs two reads (dO, V operands) ahead, each followed by exponential work
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // the phases below keep their own order
            // dS_t = P_t o (dP_t - D)
            x8 pb[2], dsb[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int qi = st * 16 + h * 8;
                const f32x4 d0 = *(const f32x4*)(dsl + qi), d1 = *(const f32x4*)(dsl + qi + 4);
                float dv8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) dv8[e] = pv[st * 8 + e] * (dp[st * 8 + e] - (e < 4 ? d0[e] : d1[e - 4]));
                pb[st] = VT::pack(pv + st * 8);
                dsb[st] = VT::pack(dv8);
            }
            __builtin_amdgcn_sched_barrier(0);
            // dV^T += dO^T P, dK^T += Q^T dS over the tile's two 16-query steps
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    constexpr int SO = 16 * CPR * 16;  // the 16-query step: 16 rows further
                    const x4 glo = VT::read_tr(gl + st * SO + to[cb][0]);
                    const x4 ghi = VT::read_tr(gl + st * SO + to[cb][1]);
                    adv[cb] = VT::mfma(__builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7), pb[st], adv[cb]);
                    const x4 qlo = VT::read_tr(ql + st * SO + to[cb][0]);
                    const x4 qhi = VT::read_tr(ql + st * SO + to[cb][1]);
                    adk[cb] = VT::mfma(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), dsb[st], adk[cb]);
                    // d = 256: keep the scheduler from hoisting every operand read of the tile (registers)
                    if constexpr (D >= 256)
                        if (cb & 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (D <= 128) {
                // dV / dK MFMAs behind their transposed operand reads
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 4 * CB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 2 < 4 * CB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // S_{t+1} right behind them (on the wave's last tile from a stage holding an older tile: in
            // bounds, unused)
            scores(QN, s);
            if constexpr (D <= 128) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        using P3 = std::integral_constant<int, 3>;
        using P4 = std::integral_constant<int, 4>;
        using P5 = std::integral_constant<int, 5>;
        // whole groups of six tiles, then the rest: no exit inside the unrolled body, which otherwise
        // costs the register allocator hundreds of spilled registers
        int tq = t0;
        for (; tq + 6 <= ntq; tq += 6) {
            iteration(tq, P0{});
            iteration(tq + 1, P1{});
            iteration(tq + 2, P2{});
            iteration(tq + 3, P3{});
            iteration(tq + 4, P4{});
            iteration(tq + 5, P5{});
        }
        if (tq < ntq) iteration(tq, P0{});
        if (tq + 1 < ntq) iteration(tq + 1, P1{});
        if (tq + 2 < ntq) iteration(tq + 2, P2{});
        if (tq + 3 < ntq) iteration(tq + 3, P3{});
        if (tq + 4 < ntq) iteration(tq + 4, P4{});
        if (key < N) {
            T* krw = dK + head + (size_t)key * D;
            T* vrw = dV + head + (size_t)key * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    x4 ok, ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ok[e] = (T)(adk[cb][gq * 4 + e] * scale);
                        ov[e] = (T)adv[cb][gq * 4 + e];
                    }
                    *(x4*)(krw + cb * 32 + gq * 8 + h * 4) = ok;
                    *(x4*)(vrw + cb * 32 + gq * 8 + h * 4) = ov;
                }
        }
    }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void bwd_q_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                       const T* __restrict__ V, const T* __restrict__ dO,
                                                       const T* __restrict__ O, const float* __restrict__ LSE,
                                                       float* __restrict__ Dl, T* __restrict__ dQ, int N, int BH,
                                                       int ntq, float c, float scale) {
    __shared__ __attribute__((aligned(1024))) char smem[BwdQ<T, D, CAUSAL>::LDS_BYTES];
    if constexpr (BwdQ<T, D, CAUSAL>::PIPE)
        BwdQ<T, D, CAUSAL>::run_pipe(Q, K, V, dO, O, LSE, Dl, dQ, N, BH, ntq, c, scale, smem);
    else
        BwdQ<T, D, CAUSAL>::run(Q, K, V, dO, O, LSE, Dl, dQ, N, BH, ntq, c, scale, smem);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void bwd_kv_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        const T* __restrict__ V, const T* __restrict__ dO,
                                                        const float* __restrict__ LSE, const float* __restrict__ Dl,
                                                        T* __restrict__ dK, T* __restrict__ dV, int N, int BH,
                                                        int nkt, float c, float scale) {
    __shared__ __attribute__((aligned(1024))) char smem[BwdKV<T, D, CAUSAL>::LDS_BYTES];
    BwdKV<T, D, CAUSAL>::run(Q, K, V, dO, LSE, Dl, dK, dV, N, BH, nkt, c, scale, smem);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int N, float scale,
                        hipStream_t stream) {
    const int ntq = (N + BwdQ<T, D, CAUSAL>::BM - 1) / BwdQ<T, D, CAUSAL>::BM;
    const int nkt = (N + BwdKV<T, D, CAUSAL>::BK - 1) / BwdKV<T, D, CAUSAL>::BK;
    if ((long long)BH * ntq > 0x7fffffffLL || (long long)BH * nkt > 0x7fffffffLL)
        return hipErrorInvalidValue;
    // c keeps its sign and at least 1e-30 of magnitude, so that a masked score (set to -inf, or +inf
    // when c < 0) gives an exponent of -inf; below that magnitude every weight rounds as it does for
    // scale 0 in float32
    float c = scale * kLog2e;
    if (std::signbit(c)) c = fminf(c, -1e-30f);
    else c = fmaxf(c, 1e-30f);
    // the dQ launch writes D, which the dK/dV launch after it on the stream reads
    hipLaunchKernelGGL((bwd_q_kernel<T, D, CAUSAL>), dim3((unsigned)(BH * ntq)), dim3(256), 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)dout, (const T*)o, lse, delta, (T*)dq, N, BH, ntq, c,
                       scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kv_kernel<T, D, CAUSAL>), dim3((unsigned)(BH * nkt)), dim3(256), 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)dout, lse, (const float*)delta, (T*)dk, (T*)dv, N, BH,
                       nkt, c, scale);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dt(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int N, int d,
                         bool causal, float scale, hipStream_t stream) {
    switch (d) {
        case 64:
            return causal ? launch_bwd_t<T, 64, true>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, scale, stream)
                          : launch_bwd_t<T, 64, false>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, scale, stream);
        case 128:
            return causal ? launch_bwd_t<T, 128, true>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, scale, stream)
                          : launch_bwd_t<T, 128, false>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, scale, stream);
        case 256:
            return causal ? launch_bwd_t<T, 256, true>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, scale, stream)
                          : launch_bwd_t<T, 256, false>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, scale, stream);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_bwd_16(bool is_bf16, const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int N, int d,
                         bool causal, float scale, hipStream_t stream) {
    return is_bf16 ? launch_bwd_dt<__bf16>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, d, causal, scale, stream)
                   : launch_bwd_dt<_Float16>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, d, causal, scale,
                                             stream);
}

}  // namespace fa
