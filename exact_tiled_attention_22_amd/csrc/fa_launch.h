// fa_launch.h — internal launchers between the C ABI (fa_host.cpp) and the HIP kernels.
// Inputs are already validated by the caller; each launcher only picks the kernel instance and
// enqueues it.  Returns hipSuccess, or the launch error reported by the runtime, or
// hipErrorInvalidValue when no instance exists for the request.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// 16-bit float path (bf16 or fp16): v_mfma_f32_32x32x16_{bf16,f16}.  Nq queries per head against Nk
// keys; causal: query i sits at position qpos + i of the key sequence (qpos = 0, Nq = Nk: square).
// c = |scale| * log2(e) (> 0), qflip = 0x80008000 to negate Q (negative scale) else 0.
hipError_t launch_fwd_16(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse,
                         int BH, int Nq, int Nk, int qpos, int d, bool causal, float c, uint32_t qflip,
                         hipStream_t stream);

// Same kernel with each query tile's key tiles split into nsplit contiguous shares (one workgroup per
// share), followed by a merge launch: work = float32 [BH, nsplit, Nq, d] partial outputs, then
// [BH, nsplit, Nq] partial lse (base 2).  For shapes with too few query tiles to fill the GPU.
hipError_t launch_fwd_16_split(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse,
                               float* work, int nsplit, int BH, int Nq, int Nk, int qpos, int d, bool causal, float c,
                               uint32_t qflip, hipStream_t stream);

// Merge of per-share partial results: O = sum_s 2^(lse_s - lse) O_s, lse = log2 sum_s 2^lse_s (written in
// natural-log units when lse != NULL).  Op [BH, nc, Nq, d], Lp [BH, nc, Nq]; an entry with lse_s = -inf
// (a share without a visible key) contributes nothing.
hipError_t launch_merge_partials(bool is_bf16, const float* Op, const float* Lp, void* o, float* lse, int BH, int Nq,
                                 int nc, int d, hipStream_t stream);

// float32 path: v_mfma_f32_32x32x2_f32.  c as above; qneg negates Q.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float c, bool qneg, hipStream_t stream);

// fp8 e4m3 path (bf16 output).  Scales may be NULL (unit scales).  block must be 64.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          const float* sq, const float* sk, const float* sv,
                          int BH, int N, int d, bool causal, float c, bool qneg, hipStream_t stream);

// fp8 prep: x_dtype 0 = f32, 1 = f16, 2 = bf16.  sign_bits: bit t set = sign -1 at column t
// (4 x 64-bit words cover d <= 256).  rotate == false ignores sign_bits.
hipError_t launch_fp8_prep(const void* x, int x_dtype, void* x8, float* scales, bool rotate,
                           const uint64_t sign_bits[4], int block, int BH, int N, int d,
                           hipStream_t stream);

// The same for the Q, K and V of one attention call in one launch: x[0], x[1] (Q, K) rotated when `rotate`,
// x[2] (V) never; all three [BH, N, d] of x_dtype.
hipError_t launch_fp8_prep_qkv(const void* const x[3], int x_dtype, void* const x8[3], float* const scales[3],
                               bool rotate, const uint64_t sign_bits[4], int block, int BH, int N, int d,
                               hipStream_t stream);

// backward (bf16 / fp16, d in {64, 128, 256}): delta <- rowsum(dout o o), then dq, then dk and dv.
hipError_t launch_bwd_16(bool is_bf16, const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int N, int d,
                         bool causal, float scale, hipStream_t stream);

// decode (bf16 / fp16, d in {64, 128, 256}, Nq <= 32): split the keys over nsplit workgroups of NW waves per
// (b, h) (NW = 4, or 2 at d = 256), chunks of `chunk` keys per wave; work = float32 [BH, NW nsplit, Nq, d]
// then [BH, NW nsplit, Nq].
hipError_t launch_decode_16(bool is_bf16, const void* q, const void* k, const void* v, void* o, float* lse, float* work,
                            int BH, int Nq, int Nk, int d, bool causal, int nsplit, int chunk, float c, uint32_t qflip,
                            hipStream_t stream);

// Library-held decode workspace (fa_fwd_decode_noalloc): its size, and its device address on the current
// device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch_ptr(float** ptr);

// unfused attention (bf16 / fp16, d in {64, 128, 256}): S = scale Q K^T as float32 [BH, N, ld]; P = softmax(S)
// in the input dtype [BH, N, ld] (zero on the padding columns) with lse; O = P V.  ld = N rounded up to 64.
hipError_t launch_naive_scores_16(bool is_bf16, const void* q, const void* k, float* s, int BH, int N, int d, int ld,
                                  float scale, hipStream_t stream);
hipError_t launch_naive_softmax_16(bool is_bf16, const float* s, void* p, float* lse, int BH, int N, int ld, bool causal,
                                   hipStream_t stream);
hipError_t launch_naive_pv_16(bool is_bf16, const void* p, const void* v, void* o, int BH, int N, int d, int ld,
                              hipStream_t stream);

}  // namespace fa
