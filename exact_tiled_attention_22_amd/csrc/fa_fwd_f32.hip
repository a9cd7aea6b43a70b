// fa_fwd_f32.hip — tiled attention forward for float32 inputs on gfx950.
//
// Same method as the 16-bit kernel (concept card "FlashAttention 2 + 3 — speicherbewusste
// Attention-Kernels", "Kernpunkte" and glossary entry "Online-Softmax"): query rows stay in
// registers, 32-key tiles of K and V pass through LDS, a running maximum and sum are corrected at
// every tile boundary, and both products run on the float32 matrix instruction
// v_mfma_f32_32x32x2_f32.  The probabilities stay float32 for the second product.
//
// Scores are computed transposed (S^T = K Q^T) so lane l holds query (l % 32).  The K rows that
// feed the MFMA A-operand are permuted so that accumulator register r of wave half h holds key
// 2r + h, which is exactly the B-operand layout the P*V product (O^T += V^T P^T) needs.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_fwd32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, float* __restrict__ O,
                                                          float* __restrict__ LSE, int N, int BH, int ntq, float c,
                                                          float qsign) {
    constexpr int NW = 4, BM = 32 * NW, BN = 32, LD = D + 1;  // LDS rows padded by one float
    constexpr int CB = D / 32, KS = D / 2;
    __shared__ float kl[BN * LD];
    __shared__ float vl[BN * LD];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    int bh, qt;
    map_block(blockIdx.x, BH, ntq, CAUSAL, bh, qt);
    const size_t head = (size_t)bh * N * D;
    const int q0 = qt * BM, q0w = q0 + wave * 32;
    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BN - 1) / BN;
    const int wave_kv_end = CAUSAL ? min(N, q0w + 32) : N;

    float qreg[KS];
    {
        const float* src = Q + head + (size_t)min(q0w + n32, N - 1) * D + h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = src[2 * ks] * qsign;
    }
    f32x16 oacc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;

    // A-operand row of lane (n32 = 8a + 4g + b): key 8a + 2b + g
    const int kperm = (n32 >> 3) * 8 + (n32 & 3) * 2 + ((n32 >> 2) & 1);

    for (int j = 0; j < nt; ++j) {
        const int kv0 = j * BN;
        __syncthreads();
        for (int idx = tid; idx < BN * D / 4; idx += 256) {
            const int row = idx / (D / 4), col = (idx % (D / 4)) * 4;
            const size_t g = head + (size_t)min(kv0 + row, N - 1) * D + col;
            const f32x4 kx = *(const f32x4*)(K + g);
            const f32x4 vx = *(const f32x4*)(V + g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kl[row * LD + col + e] = kx[e];
                vl[row * LD + col + e] = vx[e];
            }
        }
        __syncthreads();
        if (CAUSAL && kv0 >= wave_kv_end) continue;

        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[kperm * LD + 2 * ks + h], qreg[ks], s, 0, 0, 0);

        const int query = q0w + n32;
        if ((kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > q0w)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 2 * r + h;
                if (key >= N || (CAUSAL && key > query)) s[r] = -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, swap_halves(mx));
        const float mn = fmaxf(m_run, mx * c);
        const float alpha = fast_exp2(m_run - mn);
        m_run = mn;
        float p[16], ls = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(__builtin_fmaf(s[r], c, -mn));
            ls += p[r];
        }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[(2 * t + h) * LD + cb * 32 + n32], p[t], oacc[cb],
                                                                 0, 0, 0);
    }

    const float lt = l_run + swap_halves(l_run);
    const float inv = 1.0f / lt;
    const int query = q0w + n32;
    if (query < N) {
        float* orow = O + head + (size_t)query * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = oacc[cb][g * 4 + e] * inv;
                *(f32x4*)(orow + cb * 32 + g * 8 + h * 4) = out;
            }
        if (LSE != nullptr && h == 0) LSE[(size_t)bh * N + query] = (m_run + __log2f(lt)) * 0.69314718055994531f;
    }
}

template <int D, bool CAUSAL>
hipError_t launch32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, float c,
                    bool qneg, hipStream_t stream) {
    constexpr int BM = 128;
    const int ntq = (N + BM - 1) / BM;
    const long long nwg = (long long)BH * ntq;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fa_fwd32_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(256), 0, stream, q, k, v, o, lse, N,
                       BH, ntq, c, qneg ? -1.0f : 1.0f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          bool causal, float c, bool qneg, hipStream_t stream) {
    switch (d) {
        case 64:
            return causal ? launch32<64, true>(q, k, v, o, lse, BH, N, c, qneg, stream)
                          : launch32<64, false>(q, k, v, o, lse, BH, N, c, qneg, stream);
        case 128:
            return causal ? launch32<128, true>(q, k, v, o, lse, BH, N, c, qneg, stream)
                          : launch32<128, false>(q, k, v, o, lse, BH, N, c, qneg, stream);
        case 256:
            return causal ? launch32<256, true>(q, k, v, o, lse, BH, N, c, qneg, stream)
                          : launch32<256, false>(q, k, v, o, lse, BH, N, c, qneg, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace fa
