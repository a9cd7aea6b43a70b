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
//   * each wave owns QB blocks of 32 query rows; its Q operand is loaded once from HBM straight into
//     registers (together with the first K/V copies, so the prologue pays one memory latency);
//   * key/value tiles of BN = 64 rows (32 for d = 256) stream through two LDS stages each; for
//     d <= 128 K runs one tile ahead of V: during iteration j the LDS holds K_{j+1} and V_j while
//     K_{j+2} and V_{j+1} are copied in, so one barrier per tile suffices;
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: lane l holds the scores
//     of query (l % 32) for 16 keys of each 32-key block, so the row maximum and sum are in-lane plus
//     one exchange between the two wave halves;
//   * the K rows feeding the MFMA A-operand are permuted (kperm) so that 8 consecutive accumulator
//     registers of a lane hold 8 consecutive keys; the probabilities then feed O^T += V^T P^T as the
//     B-operand without any data movement;
//   * V^T operands come from LDS through the transposing read ds_read_b64_tr_b16;
//   * O^T accumulates in registers: lane l holds 16 output columns of query (l % 32) per 32-column
//     block, so the correction factor and the final 1/l are in-lane multiplies.
#include <mutex>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kTau = 8.0f;  // rescale only when the running maximum grows by more than 2^8

template <int D, int QB, int NW, int WPC>
struct Tile {
    // keys per tile: 64, or 32 for d = 256 (16 KiB tiles, 64 KiB of stages per workgroup)
    static constexpr int BN = D >= 256 ? 32 : 64;
    static constexpr int QW = 32 * QB;            // query rows per wave
    static constexpr int BM = QW * NW;            // query rows per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int CPR = D / 8;             // 16-byte chunks per row (2-byte elements)
    static constexpr int CHUNKS = BN * CPR;       // chunks per K (or V) tile
    static constexpr int LPT = CHUNKS / THREADS;  // direct-to-LDS copies per thread per tile
    static constexpr int KV_BYTES = CHUNKS * 16;
    // WPC workgroups share a CU's 160 KiB of LDS: two K stages and two V stages.  Q goes from HBM
    // straight into registers.
    static constexpr int LDS_LIMIT = 160 * 1024 / WPC;
    static constexpr int LDS_BYTES = 4 * KV_BYTES;
    static constexpr int OFF_K0 = 0, OFF_V0 = KV_BYTES, OFF_K1 = 2 * KV_BYTES, OFF_V1 = 3 * KV_BYTES;
    static_assert(CHUNKS % THREADS == 0, "tiles split evenly over threads");
    static_assert(LDS_BYTES <= LDS_LIMIT, "LDS budget");
    static_assert(LPT <= 16, "vmcnt range");
    static_assert(D > 128 || BM * D * 2 <= LDS_BYTES, "output staging fits the K/V stages");
};

// Key split (SPLIT): the workgroups of one query tile each take a contiguous share of its key tiles and
// write a partial result (O normalised over the share, float32, and lse in base 2; an empty share gives
// O = 0 and lse = -inf) that a second launch merges.  n = shares per query tile.
struct SplitOut {
    int n;
    float* Op;  // [BH, n, Nq, D]
    float* Lp;  // [BH, n, Nq]
};

template <typename T, int D, int QB, int NW, int WPC, bool CAUSAL, bool SPLIT>
struct Fwd {
    using TL = Tile<D, QB, NW, WPC>;
    using VT = Vec<T>;
    using x8 = typename VT::x8;
    using x4 = typename VT::x4;
    static constexpr int BN = TL::BN, QW = TL::QW, BM = TL::BM, CPR = TL::CPR, LPT = TL::LPT;
    static constexpr int KS = D / 16;  // k-steps of the score product
    static constexpr int CB = D / 32;  // 32-column blocks of the output
    static constexpr int OFF_K0 = TL::OFF_K0, OFF_V0 = TL::OFF_V0, OFF_K1 = TL::OFF_K1, OFF_V1 = TL::OFF_V1;
    static constexpr int NKB = BN / 32;  // 32-key blocks per tile

    // K/V tiles: BN rows of CPR chunks, row-major with the XOR swizzle (fa_common.h).  A full tile copies
    // from the lane's byte offsets in foff (the same for every full tile, computed once), so it costs no
    // vector instructions for d <= 128; d = 256 has no registers to spare for them and recomputes them;
    // a ragged last tile reads row N-1 in place of the missing rows (masked or never stored).
    using Layout = XorRows<CPR>;
    template <int NLOADS>
    static __device__ __forceinline__ void copy_rows(const T* __restrict__ src, int r0, int N, uint32_t lds,
                                                     int tid, int wave, const uint32_t (&foff)[NLOADS]) {
        static_assert(NLOADS * TL::THREADS == BN * CPR, "one tile");
        if (D <= 128 && r0 + BN <= N)
            copy_tile_full<NLOADS, TL::THREADS>(src + (size_t)r0 * D, lds, wave, foff);
        else
            copy_tile<Layout, BN, CPR, TL::THREADS>(src, r0, N, D * (int)sizeof(T), lds, tid, wave);
    }

    template <int NLOADS>
    static __device__ __forceinline__ void copy_offsets(int tid, uint32_t (&foff)[NLOADS]) {
        tile_offsets<Layout, BN, CPR, TL::THREADS>(D * (int)sizeof(T), tid, foff);
    }

    // Per-lane geometry of the MFMA operand fetches inside one LDS tile.  With 32-chunk rows (d = 256)
    // the swizzle changes only the low four bits of a chunk index, so chunks 16 apart sit 256 bytes
    // apart in every row: the offsets of the upper half are those of the lower half plus an immediate,
    // and eight address registers serve the sixteen score k-steps (four serve the eight value blocks
    // of each row group).  That keeps the non-causal d = 256 kernel within its registers (7 spilled
    // before; fp16 B2 H8 N4096 266.8 -> 254.6 us, bitwise the same); the causal instances measured 2-6 %
    // slower with it (their 4 spilled values sit outside the tile loop) and keep one register per offset.
    struct Lane {
        int kperm, h;     // score A-operand: row kperm (+32 for the second key block), chunk 2*ks + h
        int vrow, vcc, vb;  // value A-operand (transposing read): row u*4 + vrow, chunk cb*4 + vcc, byte vb
        static constexpr bool HALVES = CPR >= 32 && !CAUSAL;
        int ko[HALVES ? 8 : 1], vo[HALVES ? 2 : 1][HALVES ? 4 : 1];
        __device__ __forceinline__ void init() {
            if constexpr (HALVES) {
                static_assert(Layout::ROW_CHUNKS == 32, "the upper 16 chunks of a row keep their order");
#pragma unroll
                for (int i = 0; i < 8; ++i) ko[i] = Layout::slot(kperm, 2 * i + h) * 16;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) vo[u][i] = Layout::slot(u * 4 + vrow, i * 4 + vcc) * 16 + vb;
            }
        }
        __device__ __forceinline__ int koff(int ks) const {
            if constexpr (HALVES) return ko[ks & 7] + (ks >> 3) * 256;
            else return Layout::slot(kperm, 2 * ks + h) * 16;
        }
        __device__ __forceinline__ int voff(int cb, int u) const {
            if constexpr (HALVES) return vo[u][cb & 3] + (cb >> 2) * 256;
            const int row = u * 4 + vrow;
            return Layout::slot(row, cb * 4 + vcc) * 16 + vb;
        }
    };

    // S^T = K_tile Q^T for this wave's QB query blocks (fp32 accumulate).  A second 32-key block
    // sits 32 rows further (a compile-time offset).
    static __device__ __forceinline__ void scores(const char* kl, const x8 (&qreg)[QB][KS], f32x16 (&s)[QB][NKB],
                                                  const Lane& ln) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const x8 kop = *(const x8*)(kl + ln.koff(ks) + kb * 32 * CPR * 16);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb][kb] = VT::mfma(kop, qreg[qb][ks], s[qb][kb]);
            }
        }
    }

    // Hide keys past Nk and (causal) keys after the query's position; qp0 is the position in the key
    // sequence of the wave's first query row.  Only tiles that need it pay for the compares.
    static __device__ __forceinline__ void mask(f32x16 (&s)[QB][NKB], int kv0, int Nk, int qp0, int n32, int h) {
        if ((kv0 + BN > Nk) || (CAUSAL && kv0 + BN - 1 > qp0)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int query = qp0 + qb * 32 + n32;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                        if (key >= Nk || (CAUSAL && key > query)) s[qb][kb][r] = -INFINITY;
                    }
            }
        }
    }

    // Running maximum in base-2 units; the accumulator and sum are rescaled only when some row's
    // maximum grew by more than 2^tau (p = 2^(s*c - m) then stays <= 2^tau, exact either way).
    static __device__ __forceinline__ void update_max(const f32x16 (&s)[QB][NKB], float c, f32x16 (&oacc)[QB][CB],
                                                      float (&m_run)[QB], float (&l_run)[QB]) {
        float mt[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // 16 NKB values -> 1 as a shallow tree of 3-input maxima (short dependency chain).  Every
            // node takes three operands (a value counted twice is harmless for a maximum): a 2-input
            // maximum of matrix results costs two extra canonicalising instructions.
            float mx;
            if constexpr (NKB == 2) {
                float t1[11];
#pragma unroll
                for (int i = 0; i < 10; ++i) {
                    const int a = 3 * i, b = 3 * i + 1, d = 3 * i + 2;
                    t1[i] = max3(s[qb][a >> 4][a & 15], s[qb][b >> 4][b & 15], s[qb][d >> 4][d & 15]);
                }
                t1[10] = max3(s[qb][1][14], s[qb][1][15], s[qb][0][0]);
                const float t2a = max3(t1[0], t1[1], t1[2]), t2b = max3(t1[3], t1[4], t1[5]);
                const float t2c = max3(t1[6], t1[7], t1[8]), t2d = max3(t1[9], t1[10], t1[0]);
                mx = max3(max3(t2a, t2b, t2c), t2d, t2a);
            } else {
                float t1[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) t1[i] = max3(s[qb][0][3 * i], s[qb][0][3 * i + 1], s[qb][0][3 * i + 2]);
                mx = max3(max3(t1[0], t1[1], t1[2]), max3(t1[3], t1[4], s[qb][0][15]), t1[0]);
            }
            mt[qb] = halves_max(mx) * c;
            grow |= mt[qb] > m_run[qb] + kTau;
        }
        if (__ballot(grow)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mn = fmaxf(m_run[qb], mt[qb]);
                // a key share can leave a row without any visible key so far (m = -inf on both sides)
                const float alpha = (SPLIT && m_run[qb] == mn) ? 1.0f : fast_exp2(m_run[qb] - mn);
                m_run[qb] = mn;
                l_run[qb] *= alpha;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] *= alpha;
            }
        }
    }

    // P = 2^(s*c - m) rounded to T (row sums from the fp32 values)
    static __device__ __forceinline__ void exps(const f32x16 (&s)[QB][NKB], float c, const float (&m_run)[QB],
                                                float (&l_run)[QB], x8 (&p)[QB][2 * NKB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // a row with no visible key in its share keeps m = -inf: its probabilities are 0, not NaN
            const float negm = (SPLIT && m_run[qb] == -INFINITY) ? 0.0f : -m_run[qb];
            float part[2 * NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float e[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) e[r] = fast_exp2(__builtin_fmaf(s[qb][kb][r], c, negm));
                p[qb][kb * 2 + 0] = VT::pack(e);
                p[qb][kb * 2 + 1] = VT::pack(e + 8);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float* q = e + 8 * hf;
                    part[kb * 2 + hf] = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
                }
            }
            if constexpr (NKB == 2) l_run[qb] += (part[0] + part[1]) + (part[2] + part[3]);
            else l_run[qb] += part[0] + part[1];
        }
    }

    // O^T += V^T P^T for one tile (V^T operands through transposing LDS reads); 16-key step s sits
    // 16 rows further (a compile-time offset).
    static __device__ __forceinline__ void pv(const char* vl, const x8 (&p)[QB][2 * NKB], f32x16 (&oacc)[QB][CB],
                                              const Lane& ln) {
#pragma unroll
        for (int s = 0; s < 2 * NKB; ++s) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const x4 lo = VT::read_tr(vl + ln.voff(cb, 0) + s * 16 * CPR * 16);
                const x4 hi = VT::read_tr(vl + ln.voff(cb, 1) + s * 16 * CPR * 16);
                const x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[qb][cb] = VT::mfma(vop, p[qb][s], oacc[qb][cb]);
            }
        }
    }

    // Instruction order for the scheduler inside one tile's straight-line body: the K operand reads
    // run a few ahead of the score MFMAs, each score MFMA is followed by softmax VALU work (which does
    // not depend on it), then the V operand reads run ahead of the value MFMAs.
    static __device__ __forceinline__ void interleave() {
        constexpr int NQK = KS * NKB * QB, NKR = KS * NKB, NPV = 2 * NKB * CB * QB;
        constexpr int AHEAD = D >= 256 ? 2 : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // first K reads
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // score MFMA
            if (i + AHEAD < NKR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next K read
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // softmax VALU
        }
        constexpr int VAHEAD = D >= 256 ? 1 : 2;  // value MFMAs whose operands are in flight
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VAHEAD, 0);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // value MFMA
            if (i + VAHEAD < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // V^T operand reads
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
    }

    // O = acc / l rounded to T, and lse = ln2 * (m + log2 l).  The tile goes out through this wave's
    // LDS region as whole rows (ostage_put / ostage_flush); the caller has passed a workgroup barrier
    // after the last tile, so every LDS stage is free.
    static __device__ __forceinline__ void epilogue(T* __restrict__ O, float* __restrict__ LSE, size_t head, int bh,
                                                    int Nq, int q0w, int lane, char* wl,
                                                    const f32x16 (&oacc)[QB][CB], const float (&m_run)[QB],
                                                    const float (&l_run)[QB]) {
        const int n32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = halves_sum(l_run[qb]);
            const float inv = 1.0f / lt;
            char* tile = wl + qb * 32 * D * (int)sizeof(T);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = (T)(oacc[qb][cb][g * 4 + e] * inv);
                    ostage_put<D>(tile, n32, h, cb * 4 + g, out);
                }
            if (LSE != nullptr && h == 0) {
                const int query = q0w + qb * 32 + n32;
                if (query < Nq) LSE[(size_t)bh * Nq + query] = (m_run[qb] + __log2f(lt)) * 0.69314718055994531f;
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            ostage_flush<T, D>(O + head, q0w + qb * 32, Nq, wl + qb * 32 * D * (int)sizeof(T), lane);
    }

    // The same output written straight from registers (8 bytes per lane and store, 32 rows per
    // store); d = 256 keeps it: staging its 512-byte rows measured slower there.
    static __device__ __forceinline__ void epilogue_direct(T* __restrict__ O, float* __restrict__ LSE, size_t head,
                                                           int bh, int Nq, int q0w, int n32, int h,
                                                           const f32x16 (&oacc)[QB][CB], const float (&m_run)[QB],
                                                           const float (&l_run)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = halves_sum(l_run[qb]);
            const float inv = 1.0f / lt;
            const int query = q0w + qb * 32 + n32;
            if (query < Nq) {
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
                    LSE[(size_t)bh * Nq + query] = (m_run[qb] + __log2f(lt)) * 0.69314718055994531f;
            }
        }
    }

    // Partial result of a key share: O_s = acc / l (float32) and lse_s = m + log2 l (base 2), or O_s = 0
    // and lse_s = -inf for a row that saw no key of its share.
    static __device__ __forceinline__ void epilogue_split(const SplitOut& so, int split, int bh, int Nq, int q0w,
                                                          int n32, int h, const f32x16 (&oacc)[QB][CB],
                                                          const float (&m_run)[QB], const float (&l_run)[QB]) {
        const size_t part = (size_t)bh * so.n + split;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = halves_sum(l_run[qb]);
            const bool empty = lt == 0.0f;
            const float inv = empty ? 0.0f : 1.0f / lt;
            const int query = q0w + qb * 32 + n32;
            if (query < Nq) {
                float* orow = so.Op + (part * Nq + query) * D;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        f32x4 out;
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = oacc[qb][cb][g * 4 + e] * inv;
                        *(f32x4*)(orow + cb * 32 + g * 8 + h * 4) = out;
                    }
                if (h == 0) so.Lp[part * Nq + query] = empty ? -INFINITY : m_run[qb] + __log2f(lt);
            }
        }
    }

    // Rows of an empty key share: O_s = 0, lse_s = -inf.
    static __device__ __forceinline__ void empty_split(const SplitOut& so, int split, int bh, int Nq, int q0) {
        const size_t part = (size_t)bh * so.n + split;
        for (int i = threadIdx.x; i < BM * D / 4; i += TL::THREADS) {
            const int row = i / (D / 4), col = (i % (D / 4)) * 4;
            if (q0 + row < Nq) *(f32x4*)(so.Op + (part * Nq + q0 + row) * D + col) = f32x4{};
        }
        for (int row = threadIdx.x; row < BM; row += TL::THREADS)
            if (q0 + row < Nq) so.Lp[part * Nq + q0 + row] = -INFINITY;
    }

    // Key tiles [jb, je) of this workgroup: all of them, or its share when SPLIT.
    static __device__ __forceinline__ void tile_range(int nt, int split, int nsplit, int& jb, int& je) {
        jb = 0;
        je = nt;
        if constexpr (SPLIT) {
            const int per = (nt + nsplit - 1) / nsplit;
            jb = min(nt, split * per);
            je = min(nt, jb + per);
        }
    }

    // Key order of a causal workgroup.  Block ids go round-robin over the 8 XCDs, so an XCD runs its
    // workgroups in the order of (block id / 8), cap of them at once.  Causal grids run the longest query
    // tiles first; when one of the first cap workgroups ends, the next takes its place, so the k-th
    // replacement starts k steps of tile length after the first one, with a range shorter by as much.
    // Walking its keys from its diagonal down to key 0, every workgroup of such a round (an odd one)
    // reaches a given key tile at the same time as the others on its XCD, which then read it through the
    // XCD's L2 once instead of once per workgroup; even rounds start together and walk upward.  (The
    // online softmax is independent of the key order.)  Key shares and non-causal grids walk upward, and
    // so do queries placed at a position qpos that is not a multiple of 32: walking down, a wave's first
    // tile is the one holding its last row's key, and only with 32-aligned rows does every row of the
    // wave see a key of that tile (a row that sees none would keep a running maximum of -inf while
    // others raise theirs, and the correction factor 2^(-inf - -inf) is not a number).
    static __device__ __forceinline__ bool keys_down(int cap, int qpos) {
        if constexpr (!CAUSAL || SPLIT) return false;
        return (qpos & 31) == 0 && (((blockIdx.x >> 3) / cap) & 1);
    }

    // Block id -> (bh, query tile, key share); the shares of a query tile sit nbase ids apart, so with
    // nbase a multiple of 8 they run on the same XCD (L2) as the unsplit tile would.
    // A causal grid with B*H a multiple of 8 takes each XCD's heads G at a time, G = 2 cap / ntq: the
    // G heads' query tiles (longest first, the heads interleaved) fill two rounds of cap workgroups, the
    // first walking its keys upward from a common start, the second downward to a common end (keys_down),
    // so the workgroups resident together read the same few heads' keys at the same time and each
    // group starts in step.  Interleaving all of an XCD's heads in every round re-reads their K/V once per
    // round when they exceed the L2 (bf16 B2 H16 N8192 causal: 1.71x the algorithmic bytes, 1.25x
    // grouped; one head per round reaches 1.0x but runs about 1 % slower than two).
    static __device__ __forceinline__ void locate(int BH, int ntq, int nsplit, int& bh, int& qt, int& split,
                                                  int cap) {
        int bid = blockIdx.x;
        split = 0;
        if constexpr (SPLIT) {
            const int nbase = BH * ntq;
            split = bid / nbase;
            bid -= split * nbase;
        }
        if (CAUSAL && !SPLIT && (BH & 7) == 0) {
            const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
            const int G = max(1, 2 * cap / ntq);             // heads per group (two rounds)
            const int grp = slot / (G * ntq);                // group of G heads
            const int gl = min(G, hpx - grp * G);            // heads in this group (the last may have fewer)
            const int w = slot - grp * G * ntq;
            qt = ntq - 1 - w / gl;
            bh = xcd * hpx + grp * G + w % gl;
            return;
        }
        map_block(bid, BH, ntq, CAUSAL, bh, qt);
    }

    // In-order pipeline for large head dimensions (one score buffer): iteration j holds K_j and V_j
    // in stage j % 2 and copies K_{j+1}, V_{j+1} into the other stage; the scores of tile j come first,
    // then its softmax, whose exponentials interleave with the value MFMAs.
    static __device__ __forceinline__ void run_seq(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const T* __restrict__ V, T* __restrict__ O,
                                                   float* __restrict__ LSE, int Nq, int Nk, int qpos, int BH,
                                                   int ntq, float c, uint32_t qflip, char* smem, SplitOut so,
                                                   int cap) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31;
        const int h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        int bh, qt, split;
        locate(BH, ntq, so.n, bh, qt, split, cap);
        const size_t head = (size_t)bh * Nq * D;  // Q, O
        const size_t headk = (size_t)bh * Nk * D; // K, V
        const T* Qh = Q + head;
        const T* Kh = K + headk;
        const T* Vh = V + headk;
        const int q0 = qt * BM;
        const int q0w = q0 + wave * QW;
        int jb, je;  // key tiles of this workgroup (its share when split)
        tile_range(((CAUSAL ? min(Nk, qpos + q0 + BM) : Nk) + BN - 1) / BN, split, so.n, jb, je);
        if (SPLIT && jb >= je) {
            empty_split(so, split, bh, Nq, q0);
            return;
        }
        // tiles this wave computes: [jb, ntw); iteration j handles key tile kt(j)
        const int ntw = min(je, ((CAUSAL ? min(Nk, qpos + q0w + QW) : Nk) + BN - 1) / BN);
        const bool down = keys_down(cap, qpos);
        auto kt = [&](int j) { return down ? jb + je - 1 - j : j; };
        Lane ln;
        ln.kperm = ((n32 >> 4) & 1) * 16 + ((n32 >> 2) & 1) * 8 + ((n32 >> 3) & 1) * 4 + (n32 & 3);
        ln.h = h;
        {
            const int i16 = lane & 15, G = lane >> 4;
            ln.vrow = (G >> 1) * 8 + (i16 >> 2);
            ln.vcc = (G & 1) * 2 + ((i16 & 3) >> 1);
            ln.vb = (i16 & 1) * 8;
        }
        ln.init();
        uint32_t foff[LPT];
        copy_offsets<LPT>(tid, foff);
        // Q operand straight from HBM (the first iteration's wait covers these loads and the copies)
        x8 qreg[QB][KS];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const T* src = Qh + (size_t)min(q0w + qb * 32 + n32, Nq - 1) * D + h * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                i32x4 raw = *(const i32x4*)(src + ks * 16);
                raw ^= (int)qflip;
                qreg[qb][ks] = __builtin_bit_cast(x8, raw);
            }
        }
        copy_rows<LPT>(Kh, kt(jb) * BN, Nk, lbase + OFF_K0, tid, wave, foff);
        copy_rows<LPT>(Vh, kt(jb) * BN, Nk, lbase + OFF_V0, tid, wave, foff);
        f32x16 oacc[QB][CB];
        float m_run[QB], l_run[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] = f32x16{};
        }
        auto iteration = [&](int j, int ok, int ov, uint32_t dk, uint32_t dv) {
            wait_vmcnt<0>();
            lds_barrier();  // K_j, V_j visible; the other stage is free
            if (j + 1 < je) {
                copy_rows<LPT>(Kh, kt(j + 1) * BN, Nk, lbase + dk, tid, wave, foff);
                copy_rows<LPT>(Vh, kt(j + 1) * BN, Nk, lbase + dv, tid, wave, foff);
            }
            if (kt(j) < ntw) {
                f32x16 sc[QB][NKB];
                scores(smem + ok, qreg, sc, ln);
                // score MFMAs paced by their K operand reads, two reads ahead (fp16 B1 H8 N16384 causal
                // 1025 -> 1001 us, B4 H8 N2048 causal 108 -> 103 us)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < KS * NKB * QB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 2 < KS * NKB * QB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                mask(sc, kt(j) * BN, Nk, qpos + q0w, n32, h);
                update_max(sc, c, oacc, m_run, l_run);
                x8 p[QB][2 * NKB];
                exps(sc, c, m_run, l_run, p);
                pv(smem + ov, p, oacc, ln);
                // value MFMAs paced by their V operand reads, two softmax instructions after each
                // (fp16 B2 H8 N4096 d256 non-causal 280 -> 263 us; the long causal workload unchanged)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < 2 * NKB * CB * QB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + 1 < 2 * NKB * CB * QB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
            }
        };
        for (int j = jb; j < je; j += 2) {
            iteration(j, OFF_K0, OFF_V0, OFF_K1, OFF_V1);
            if (j + 1 < je) iteration(j + 1, OFF_K1, OFF_V1, OFF_K0, OFF_V0);
        }
        if constexpr (SPLIT)
            epilogue_split(so, split, bh, Nq, q0w, n32, h, oacc, m_run, l_run);
        else
            epilogue_direct(O, LSE, head, bh, Nq, q0w, n32, h, oacc, m_run, l_run);
    }

    static __device__ __forceinline__ void run(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V, T* __restrict__ O,
                                               float* __restrict__ LSE, int Nq, int Nk, int qpos, int BH,
                                               int ntq, float c, uint32_t qflip, char* smem, SplitOut so,
                                               int cap) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n32 = lane & 31;
        const int h = lane >> 5;
        const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

        int bh, qt, split;
        locate(BH, ntq, so.n, bh, qt, split, cap);
        const size_t head = (size_t)bh * Nq * D;  // Q, O
        const size_t headk = (size_t)bh * Nk * D; // K, V
        const T* Qh = Q + head;
        const T* Kh = K + headk;
        const T* Vh = V + headk;
        const int q0 = qt * BM;
        const int q0w = q0 + wave * QW;
        int jb, je;  // key tiles of the workgroup (its share when split)
        tile_range(((CAUSAL ? min(Nk, qpos + q0 + BM) : Nk) + BN - 1) / BN, split, so.n, jb, je);
        if (SPLIT && jb >= je) {
            empty_split(so, split, bh, Nq, q0);
            return;
        }
        // tiles this wave computes: [jb, ntw); iteration j handles key tile kt(j)
        const int ntw = min(je, ((CAUSAL ? min(Nk, qpos + q0w + QW) : Nk) + BN - 1) / BN);
        const bool down = keys_down(cap, qpos);
        auto kt = [&](int j) { return down ? jb + je - 1 - j : j; };

        Lane ln;
        ln.kperm = ((n32 >> 4) & 1) * 16 + ((n32 >> 2) & 1) * 8 + ((n32 >> 3) & 1) * 4 + (n32 & 3);
        ln.h = h;
        {
            const int i16 = lane & 15, G = lane >> 4;  // transposing read: lane = 16 G + i
            ln.vrow = (G >> 1) * 8 + (i16 >> 2);
            ln.vcc = (G & 1) * 2 + ((i16 & 3) >> 1);
            ln.vb = (i16 & 1) * 8;
        }
        ln.init();

        uint32_t foff[LPT];
        copy_offsets<LPT>(tid, foff);

        // ---- prologue: Q straight into registers, K_0, V_0, K_1 into LDS, one memory latency ----
        // Q operand (B of the score MFMA): lane supplies Q[q0w + qb*32 + n32][ks*16 + h*8 + 0..7]
        x8 qreg[QB][KS];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const T* src = Qh + (size_t)min(q0w + qb * 32 + n32, Nq - 1) * D + h * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                i32x4 raw = *(const i32x4*)(src + ks * 16);
                raw ^= (int)qflip;
                qreg[qb][ks] = __builtin_bit_cast(x8, raw);
            }
        }
        copy_rows<LPT>(Kh, kt(jb) * BN, Nk, lbase + OFF_K0, tid, wave, foff);
        copy_rows<LPT>(Vh, kt(jb) * BN, Nk, lbase + OFF_V0, tid, wave, foff);
        if (jb + 1 < je) copy_rows<LPT>(Kh, kt(jb + 1) * BN, Nk, lbase + OFF_K1, tid, wave, foff);
        wait_vmcnt<0>();
        lds_barrier();

        f32x16 oacc[QB][CB];
        float m_run[QB], l_run[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] = f32x16{};
        }

        f32x16 s0[QB][NKB], s1[QB][NKB];
        scores(smem + OFF_K0, qreg, s0, ln);

        // ---- main loop: iteration j holds K_{j+1} and V_j, copies K_{j+2} and V_{j+1} ----
        auto iteration = [&](int j, f32x16 (&cur)[QB][NKB], f32x16 (&nxt)[QB][NKB], int okn, int ov, uint32_t dk,
                             uint32_t dv) {
            wait_vmcnt<0>();
            lds_barrier();
            if (j + 2 < je) copy_rows<LPT>(Kh, kt(j + 2) * BN, Nk, lbase + dk, tid, wave, foff);
            if (j + 1 < je) copy_rows<LPT>(Vh, kt(j + 1) * BN, Nk, lbase + dv, tid, wave, foff);
            if (kt(j) < ntw) {
                mask(cur, kt(j) * BN, Nk, qpos + q0w, n32, h);
                update_max(cur, c, oacc, m_run, l_run);
                // next tile's scores (its K stage always holds valid data; on the last tile the result is
                // unused) in the same basic block as this tile's exponentials so the two overlap; with
                // d = 256 the registers only allow the two in sequence
                // raised wave priority while this wave streams MFMAs: the other workgroup's wave on
                // the SIMD (in its softmax-maximum or copy phase) then fills the issue gaps instead
                // of competing with the matrix instructions
                __builtin_amdgcn_s_setprio(1);
                scores(smem + okn, qreg, nxt, ln);
                x8 p[QB][2 * NKB];
                exps(cur, c, m_run, l_run, p);
                pv(smem + ov, p, oacc, ln);
                interleave();
                __builtin_amdgcn_s_setprio(0);
            } else if (down && j + 1 < je && kt(j + 1) < ntw) {
                // walking down, a wave's first tiles can lie past its last query row: the tile before
                // its first computed one still computes that one's scores
                scores(smem + okn, qreg, nxt, ln);
            }
        };
        for (int j = jb; j < je; j += 2) {
            // j - jb even: K_{j+1} in stage 1, V_j in stage 0; copies K_{j+2} -> stage 0, V_{j+1} -> stage 1
            iteration(j, s0, s1, OFF_K1, OFF_V0, OFF_K0, OFF_V1);
            if (j + 1 < je) iteration(j + 1, s1, s0, OFF_K0, OFF_V1, OFF_K1, OFF_V0);
        }

        if constexpr (SPLIT) {
            epilogue_split(so, split, bh, Nq, q0w, n32, h, oacc, m_run, l_run);
        } else {
            lds_barrier();  // every wave is past its last LDS read: the stages become output staging
            epilogue(O, LSE, head, bh, Nq, q0w, lane, smem + wave * QW * D * (int)sizeof(T), oacc, m_run, l_run);
        }
    }
};

// One workgroup per (b, h, query tile) (and key share when SPLIT); WPC of them share a CU, two waves
// per SIMD in total.  With two workgroups per CU one's prologue and epilogue overlap the other's tile
// loop; with one (d = 256) its eight waves share every K/V tile copy.
template <typename T, int D, int QB, int NW, int WPC, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(64 * NW, (NW * WPC) / 4) void fa_fwd16_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, int Nq, int Nk, int qpos, int BH, int ntq, float c, uint32_t qflip, SplitOut so,
    int cap) {
    __shared__ __attribute__((aligned(1024))) char smem[Tile<D, QB, NW, WPC>::LDS_BYTES];
    if constexpr (D <= 128)
        Fwd<T, D, QB, NW, WPC, CAUSAL, SPLIT>::run(Q, K, V, O, LSE, Nq, Nk, qpos, BH, ntq, c, qflip, smem, so, cap);
    else
        Fwd<T, D, QB, NW, WPC, CAUSAL, SPLIT>::run_seq(Q, K, V, O, LSE, Nq, Nk, qpos, BH, ntq, c, qflip, smem, so,
                                                       cap);
}

// Compute units per XCD of the current device (its CU count / 8), queried once per device.
int cus_per_xcd() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 32;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
        cached[dev] = n / 8;
    }
    return cached[dev];
}

// per head dimension: query blocks per wave, waves per workgroup, workgroups per CU
template <int D> struct Shape;
template <> struct Shape<64> { static constexpr int QB = 1, NW = 4, WPC = 2; };
template <> struct Shape<128> { static constexpr int QB = 1, NW = 4, WPC = 2; };
// d = 256: one 8-wave workgroup per CU (256 query rows share each K/V tile copy; measured faster
// than two independent 4-wave workgroups here, unlike d = 128)
template <> struct Shape<256> { static constexpr int QB = 1, NW = 8, WPC = 1; };

template <typename T, int D, bool CAUSAL>
hipError_t launch16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Nq, int Nk,
                    int qpos, float c, uint32_t qflip, SplitOut so, hipStream_t stream) {
    constexpr int QB = Shape<D>::QB, NW = Shape<D>::NW, WPC = Shape<D>::WPC;
    constexpr int BM = Tile<D, QB, NW, WPC>::BM;
    const int ntq = (Nq + BM - 1) / BM;
    const long long nwg = (long long)BH * ntq * (so.n > 0 ? so.n : 1);
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const int cap = cus_per_xcd() * WPC;  // workgroups resident at once on one XCD
    if (so.n > 0)
        hipLaunchKernelGGL((fa_fwd16_kernel<T, D, QB, NW, WPC, CAUSAL, true>), dim3((unsigned)nwg), dim3(64 * NW), 0,
                           stream, (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, Nq, Nk, qpos, BH, ntq, c, qflip,
                           so, cap);
    else
        hipLaunchKernelGGL((fa_fwd16_kernel<T, D, QB, NW, WPC, CAUSAL, false>), dim3((unsigned)nwg), dim3(64 * NW), 0,
                           stream, (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, Nq, Nk, qpos, BH, ntq, c, qflip,
                           so, cap);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Nq, int Nk,
                      int qpos, int d, bool causal, float c, uint32_t qflip, SplitOut so, hipStream_t stream) {
    switch (d) {
        case 64:
            return causal ? launch16<T, 64, true>(q, k, v, o, lse, BH, Nq, Nk, qpos, c, qflip, so, stream)
                          : launch16<T, 64, false>(q, k, v, o, lse, BH, Nq, Nk, qpos, c, qflip, so, stream);
        case 128:
            return causal ? launch16<T, 128, true>(q, k, v, o, lse, BH, Nq, Nk, qpos, c, qflip, so, stream)
                          : launch16<T, 128, false>(q, k, v, o, lse, BH, Nq, Nk, qpos, c, qflip, so, stream);
        case 256:
            return causal ? launch16<T, 256, true>(q, k, v, o, lse, BH, Nq, Nk, qpos, c, qflip, so, stream)
                          : launch16<T, 256, false>(q, k, v, o, lse, BH, Nq, Nk, qpos, c, qflip, so, stream);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_fwd_16(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                         int Nq, int Nk, int qpos, int d, bool causal, float c, uint32_t qflip,
                         hipStream_t stream) {
    const SplitOut none{0, nullptr, nullptr};
    return is_bf16 ? dispatch16<__bf16>(q, k, v, o, lse, BH, Nq, Nk, qpos, d, causal, c, qflip, none, stream)
                   : dispatch16<_Float16>(q, k, v, o, lse, BH, Nq, Nk, qpos, d, causal, c, qflip, none, stream);
}

hipError_t launch_fwd_16_split(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse,
                               float* work, int nsplit, int BH, int Nq, int Nk, int qpos, int d, bool causal, float c,
                               uint32_t qflip, hipStream_t stream) {
    float* Op = work;
    float* Lp = work + (size_t)BH * nsplit * Nq * d;
    const SplitOut so{nsplit, Op, Lp};
    hipError_t e = is_bf16 ? dispatch16<__bf16>(q, k, v, o, lse, BH, Nq, Nk, qpos, d, causal, c, qflip, so, stream)
                           : dispatch16<_Float16>(q, k, v, o, lse, BH, Nq, Nk, qpos, d, causal, c, qflip, so, stream);
    if (e != hipSuccess) return e;
    return launch_merge_partials(is_bf16, Op, Lp, o, lse, BH, Nq, nsplit, d, stream);
}

}  // namespace fa
