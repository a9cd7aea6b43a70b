/*
 * fa.h — C ABI of the exact tiled attention library for AMD Instinct MI355X (gfx950).
 *
 * Operation.  For every batch b < B and head h < H the forward pass computes
 *     O[b,h] = softmax(scale * Q[b,h] * K[b,h]^T  [+ causal mask]) * V[b,h]
 *     lse[b,h,i] = ln sum_j exp(scale * q_i . k_j)       (over the keys visible to query i)
 * exactly in real arithmetic, without ever storing the N x N score matrix: query tiles stay in
 * registers, key/value tiles stream through on-chip LDS and an online softmax keeps a running row
 * maximum and sum that are corrected at every tile boundary.  Sources: "FlashAttention 2 + 3 —
 * speicherbewusste Attention-Kernels", sections "Kernpunkte" (same output as softmax(QK^T/sqrt d)V,
 * tiles of 64-128 rows, online softmax, no N x N matrix in HBM) and "Begriffe auf dieser Seite"
 * (entry "Online-Softmax": running maximum and a correction factor at each tile boundary).
 * The causal mask (key j visible to query i iff j <= i) and the lse output are not on the pages;
 * they are this library's contract.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the library allocates nothing
 *     and keeps no state between calls except a thread-local error string (and, for
 *     fa_fwd_decode_noalloc only, one device array per GPU).
 *   - Tensors are contiguous row-major [B, H, N, d] (lse: [B, H, N], float32).  N_q = N_k = N for
 *     fa_fwd, fa_fwd_ex and fa_bwd; fa_fwd_rect, fa_fwd_split and fa_fwd_decode take q as
 *     [B, H, Nq, d] and k, v as [B, H, Nk, d].
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream).  No call synchronises the host.  Calls are thread-safe.
 *   - Arguments are validated before anything is enqueued: a non-FA_OK return means no work was
 *     launched.  fa_last_error() then describes the problem.  A launch failure reported by the HIP
 *     runtime returns FA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation.  NaN/Inf tensor contents are not checked.
 *   - Pointers must be 16-byte aligned (FA_ERR_ALIGN); B, H, N >= 0 with B*H*N == 0 a no-op
 *     returning FA_OK; supported head dimensions d are 64, 128 and 256 (FA_ERR_UNSUPPORTED).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 3

typedef enum {
    FA_F32 = 0,      /* float32 in, float32 out */
    FA_F16 = 1,      /* IEEE binary16 in, binary16 out */
    FA_BF16 = 2,     /* bfloat16 in, bfloat16 out */
    FA_FP8_E4M3 = 3  /* OCP e4m3fn bytes in (see fa_fp8_prep), bfloat16 out */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,       /* negative or overflowing sizes */
    FA_ERR_DTYPE = 3,       /* unknown dtype code */
    FA_ERR_UNSUPPORTED = 4, /* valid request the library does not implement (e.g. d not in {64,128,256}) */
    FA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    FA_ERR_ARG = 6,         /* other invalid argument (non-finite scale, causal not 0/1, bad signs) */
    FA_ERR_HIP = 7          /* the HIP runtime rejected a launch */
} fa_status;

/*
 * Per-block dequantisation scales of the FP8 path, as written by fa_fp8_prep: DEVICE pointers to
 * float32 arrays [B*H, ceil(N/block)].  Element t of row bh multiplies rows t*block .. t*block+block-1
 * of that (b,h) slice.  The forward kernel supports block == 64 only.
 */
typedef struct {
    const float* q_scale;
    const float* k_scale;
    const float* v_scale;
    int block;
} fa_fp8_scales;

/*
 * Attention forward.
 *   q, k, v : [B,H,N,d] inputs of type `dtype` (FA_F32, FA_F16 or FA_BF16; FA_FP8_E4M3 means unit
 *             scales, i.e. fa_fwd_ex with s8 == NULL).
 *   o       : [B,H,N,d] output, same type as the inputs (bfloat16 for FA_FP8_E4M3).  Must not alias
 *             q, k or v.
 *   lse     : [B,H,N] float32 natural-log log-sum-exp per query row, or NULL to skip it.
 *   causal  : 0 = every key visible; 1 = key j visible to query i iff j <= i.
 *   scale   : finite float32 multiplier of q.k (callers normally pass 1/sqrt(d)).
 * Returns an fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * Attention forward with FP8 (e4m3) operands and per-block scales (FlashAttention-3 article,
 * "Drei technische Hebel", item 3 "FP8-Blockquantisierung": blockwise 8-bit operands).
 * Identical to fa_fwd for other dtypes (s8 is then ignored).  For FA_FP8_E4M3 the inputs are e4m3
 * codes; the value of element [b,h,n,:] is code * scale[b*H+h][n / block].  s8 == NULL means all
 * scales are 1.  Scores and the P*V product accumulate in float32; P (times an exact 2^6) is rounded
 * to e4m3 for the second product, whose 64-key blocks are each multiplied by their V scale in float32;
 * o is bfloat16.  Scales are read on the device, so they are not validated: they must be finite and
 * non-negative, as fa_fp8_prep writes them (a V scale of 0 makes its block contribute nothing; other
 * values give unspecified output, never a fault).  The three arrays must each hold
 * B*H*ceil(N/block) floats.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, int causal, float scale, int dtype,
              const fa_fp8_scales* s8, void* stream);

/*
 * Attention forward of Nq queries against Nk keys per (b, h): the same definition and the same tiled
 * kernel as fa_fwd, for a query range that is not the whole key sequence.  The concept card
 * ("FlashAttention 2 + 3 — speicherbewusste Attention-Kernels", "Kernpunkte") splits the queries into
 * blocks that are processed independently against the streamed keys; this entry point exposes one
 * contiguous range of those blocks.  Uses: one GPU's share of a sequence-sharded forward (queries
 * q_start .. q_start + Nq - 1 of a sequence whose Nk keys and values are all present), and a prefill
 * chunk appended to a key/value cache (q_start = Nk - Nq).
 *   q, o    : DEVICE [B,H,Nq,d];  k, v : DEVICE [B,H,Nk,d];  lse : DEVICE [B,H,Nq] float32 or NULL.
 *   causal  : 0 = every key visible (q_start must be 0; any Nq, Nk >= 1);
 *             1 = query i sees keys j <= q_start + i; requires 0 <= q_start <= Nk - Nq.
 *   dtype   : FA_F16 or FA_BF16 (FA_ERR_UNSUPPORTED otherwise); d : 64, 128 or 256.
 * o must overlap none of q, k, v; lse must not overlap o.  With Nq = Nk and q_start = 0 the result is
 * fa_fwd's, bit for bit.  The query rows a .. a + Nq - 1 of a sequence of Nk (q_start = a when causal)
 * give fa_fwd's rows of that range bit for bit when a is a multiple of 128 and Nq a multiple of 32 (or
 * the range ends the sequence) and, if causal, both launches walk the keys of those rows in the same
 * order: the kernel then puts the same rows into each wave.  A causal launch with more workgroups than
 * the GPU runs at once walks the keys of alternate dispatch rounds in
 * opposite orders when its rows start at a multiple of 32, so rows that fall in rounds of different
 * parity in the two launches differ by float32 summation order.  Nq = 0 or B*H = 0
 * is a no-op; Nq > 0 with Nk = 0 is FA_ERR_SHAPE.  Returns an fa_status; nothing is enqueued on error.
 */
int fa_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Nq, int Nk, int q_start, int d, int causal, float scale, int dtype,
                void* stream);

/*
 * fa_fwd_rect with each query tile's key range split into `nsplit` contiguous shares handled by
 * separate workgroups, each with its own online softmax (running maximum and sum over its share); a
 * second launch merges the shares' partial results exactly: lse = log sum_s exp(lse_s) and
 * O = sum_s exp(lse_s - lse) O_s (the same merge the decode path uses).  The result is the same
 * attention (FlashAttention 2 + 3 concept card, "Kernpunkte": tiling and online softmax; the running
 * maximum and correction factor of the glossary entry "Online-Softmax" are what makes partial results
 * over key ranges mergeable).  For shapes whose B*H*ceil(Nq/128) workgroups cannot fill the GPU, e.g.
 * one GPU's share of a sequence-sharded long-context forward.
 *   Arguments as fa_fwd_rect, plus:
 *   nsplit    : 1..64 shares per query tile (1 gives fa_fwd_rect's result bit for bit whenever
 *               fa_fwd_rect walks every key range upward: key shares always do, fa_fwd_rect's later
 *               dispatch rounds of a large causal grid may walk downward).
 *   workspace : DEVICE scratch of at least fa_fwd_split_workspace_bytes(B, H, Nq, d, nsplit) bytes,
 *               owned by the caller, 16-byte aligned, overlapping no tensor; contents on return are
 *               unspecified.  Calls that share a workspace must not overlap in time.
 * Returns an fa_status; nothing is enqueued on error.
 */
size_t fa_fwd_split_workspace_bytes(int B, int H, int Nq, int d, int nsplit);
int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int q_start, int d, int causal, float scale, int dtype,
                 int nsplit, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block absmax quantisation to OCP e4m3fn with an optional Hadamard rotation of the head dimension
 * (FlashAttention-3 article, "Drei technische Hebel", item 3 and "Praxischeck"/"Präzision": blockwise
 * eight-bit operands, a Hadamard transform to reduce quantisation error; concept card "Kernpunkte":
 * absmax scaling).
 *   x        : DEVICE [BH, N, d] input of type x_dtype (FA_F32, FA_F16 or FA_BF16).
 *   x8       : DEVICE [BH, N, d] output bytes (e4m3fn codes).
 *   scales   : DEVICE [BH, ceil(N/block)] float32 output, dequantisation scale per block.
 *   hadamard : HOST pointer to d int8 values, each +1 or -1 (the random sign vector s), or NULL for
 *              no rotation.  With signs, each row is replaced by (x * s) H_d / sqrt(d) (H_d the
 *              Sylvester Hadamard matrix) before quantisation; pass the same signs for Q and K so
 *              that Q K^T is preserved.  Requires d to be a power of two.
 *   block    : rows per scale block, 1..1024 (64 for the forward kernel).
 * Per block: amax = max |x'|, scale = amax/448, code = e4m3_RNE(x' * (448/amax)) computed in float32
 * (the rotation as float32 butterflies with strides 1, 2, ..., d/2 followed by a multiply with the
 * float32 value of 1/sqrt(d)); an all-zero block stores scale 1 and zero codes.
 */
int fa_fp8_prep(const void* x, int x_dtype, void* x8, float* scales,
                const int8_t* hadamard, int block, int BH, int N, int d, void* stream);

/*
 * fa_fp8_prep of the Q, K and V of one attention call in one launch (FlashAttention-3 article,
 * "Drei technische Hebel", item 3): q and k are rotated with the same sign vector `hadamard` (or not at
 * all when it is NULL), v is never rotated; each gets its codes and block scales exactly as fa_fp8_prep
 * writes them (bitwise).  All three inputs are DEVICE [BH, N, d] of x_dtype; q8, k8, v8 DEVICE [BH, N, d]
 * bytes; q_scales, k_scales, v_scales DEVICE [BH, ceil(N/block)] float32.  No output may overlap another
 * output or an input (FA_ERR_ARG).  Validation and errors as fa_fp8_prep.
 */
int fa_fp8_prep_qkv(const void* q, const void* k, const void* v, int x_dtype, void* q8, void* k8, void* v8,
                    float* q_scales, float* k_scales, float* v_scales, const int8_t* hadamard, int block,
                    int BH, int N, int d, void* stream);

/*
 * Attention of a few queries against a long cached key/value sequence (decode).  The pages tie the
 * method's memory savings to bigger key/value caches and longer context at serving time (Flash
 * Attention glossary, "/02 Warum ist Flash Attention wichtig?").  Same definition as fa_fwd with
 * Nq queries and Nk >= Nq keys per (b, h):
 *   q, o : DEVICE [B,H,Nq,d];  k, v : DEVICE [B,H,Nk,d];  lse : DEVICE [B,H,Nq] float32 or NULL.
 *   causal : 1 = query i sees keys j <= i + Nk - Nq (the queries are the last Nq positions).
 *   dtype : FA_F16 or FA_BF16; d : 64, 128 or 256; 1 <= Nq <= 32 (FA_ERR_UNSUPPORTED otherwise).
 *   workspace : DEVICE scratch of at least fa_decode_workspace_bytes(B, H, Nq, Nk, d) bytes, owned by
 *               the caller, 16-byte aligned, overlapping no tensor; its contents on return are
 *               unspecified.  Calls that share a workspace must not overlap in time.
 * The keys are split into chunks handled by independent waves (per-chunk online softmax), and a
 * second launch merges the chunks' (O, lse) pairs; float32 accumulation, P rounded to `dtype`.
 * Nq = 1 runs its dot products on the vector ALU, Nq > 1 on the matrix cores.
 * Returns an fa_status.
 */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, int causal, float scale, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_decode without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The partial
 * results go to a library-held array of FA_DECODE_NOALLOC_BYTES bytes per GPU (a device variable of
 * the library, kept until the process ends); the call allocates nothing.  Shapes whose
 * fa_decode_workspace_bytes(B, H, Nq, Nk, d) exceeds FA_DECODE_NOALLOC_BYTES return
 * FA_ERR_UNSUPPORTED before anything is enqueued (use fa_fwd_decode with a caller workspace).  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on the same GPU (other streams,
 * other threads) race and give undefined results; calls ordered on one stream are safe.  Arguments,
 * result and errors are otherwise those of fa_fwd_decode; the output is bitwise the same.
 */
#define FA_DECODE_NOALLOC_BYTES (64u << 20)
int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, int d, int causal, float scale, int dtype, void* stream);

/*
 * Attention backward: the gradients of fa_fwd's output with respect to q, k and v for a given output
 * gradient dout, rebuilt tile by tile from the saved row log-sum-exp (no N x N matrix in memory).
 * The pages name the backward pass without writing it out ("FlashAttention 2 + 3 — speicherbewusste
 * Attention-Kernels", "Kernpunkte": FlashAttention 2 improves its parallelism); what is computed is
 * the derivative of the forward definition:
 *     P = exp(scale q k^T - lse) on the visible keys,  D_i = sum_t dout[i,t] o[i,t],
 *     dS = P o (dout v^T - D),  dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout.
 *   q, k, v, o, dout : DEVICE [B,H,N,d] inputs of type `dtype` (FA_F16 or FA_BF16); o is fa_fwd's
 *                      output for the same q, k, v, causal, scale.
 *   lse              : DEVICE [B,H,N] float32, fa_fwd's lse for the same call (required).
 *   dq, dk, dv       : DEVICE [B,H,N,d] outputs of type `dtype`; must overlap neither each other nor
 *                      any input.
 *   delta            : DEVICE [B,H,N] float32 workspace owned by the caller; on return it holds D.
 *   d                : 64, 128 or 256 (FA_ERR_UNSUPPORTED otherwise; FA_F32 and FA_FP8_E4M3 likewise).
 * Products accumulate in float32; P and dS are rounded to `dtype` as MFMA operands.  Deterministic:
 * no atomics (dq comes from one pass over the key tiles, dk and dv from one over the query tiles).
 * Returns an fa_status.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * Unfused attention: the standard implementation that the tiled method is measured against (concept
 * card "FlashAttention 2 + 3 — speicherbewusste Attention-Kernels", "Worum es geht" and "Kernpunkte":
 * the classic path writes the full score matrix to HBM and reads it back; Flash Attention glossary,
 * "/02 Technische Vorteile im Überblick": the speed-up over that path).  Same definition and outputs
 * as fa_fwd, computed in three launches with the N x N matrices in device memory:
 *   fa_naive_scores  : s = scale q k^T, float32 [B*H, N, ld]; columns >= N of a row are padding
 *                      (unspecified values).
 *   fa_naive_softmax : p = softmax(s [+ causal mask, key j visible to query i iff j <= i]) per row, of
 *                      type `dtype`, [B*H, N, ld], written as 0 on the masked and padding columns;
 *                      lse [B,H,N] float32 (natural log, may be NULL).  float32 arithmetic, p rounded
 *                      to nearest even.
 *   fa_naive_pv      : o = p v, [B,H,N,d] of type `dtype`, float32 accumulation.
 *   fa_fwd_naive     : the three in order, with s and p placed in `workspace`.
 * ld = fa_naive_row_stride(N) = N rounded up to a multiple of 64 (elements).  q, k, v, o are DEVICE
 * [B,H,N,d] of type `dtype` (FA_F16 or FA_BF16); d is 64, 128 or 256.  Every pointer is a caller-owned
 * DEVICE pointer, 16-byte aligned; outputs overlap no input.  The causal mask is applied in the
 * softmax only (every score is computed).  workspace: at least fa_naive_workspace_bytes(B, H, N)
 * bytes (B*H*N*ld*6: s, then p); its contents on return are s and p.  Returns an fa_status.
 */
int fa_naive_row_stride(int N);
size_t fa_naive_workspace_bytes(int B, int H, int N);
int fa_naive_scores(const void* q, const void* k, float* s, int B, int H, int N, int d, float scale, int dtype,
                    void* stream);
int fa_naive_softmax(const float* s, void* p, float* lse, int B, int H, int N, int causal, int dtype, void* stream);
int fa_naive_pv(const void* p, const void* v, void* o, int B, int H, int N, int d, int dtype, void* stream);
int fa_fwd_naive(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* fa_status_str(int status);

/* Detail of the last non-FA_OK return on the calling thread ("" if none).  Valid until the next call
 * on the same thread. */
const char* fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
