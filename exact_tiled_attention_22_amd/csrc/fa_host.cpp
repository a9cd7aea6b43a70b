// fa_host.cpp — the C ABI declared in include/fa.h: argument validation, kernel selection, launch.
//
// Validation runs before any HIP call, so an invalid request returns its status without touching
// the device.  No exception crosses the ABI; errors are reported through the return status and a
// thread-local message (fa_last_error).
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_launch.h"

namespace {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int elem_bytes(int dtype) {
    switch (dtype) {
        case FA_F32: return 4;
        case FA_F16: return 2;
        case FA_BF16: return 2;
        case FA_FP8_E4M3: return 1;
        default: return 0;
    }
}

// B*H*N*d must stay well inside int64 and every index the kernels form from (B*H, N) in int32.
int check_sizes(long long BH, long long N, long long d) {
    if (BH > 0x7fffffffLL) return fail(FA_ERR_SHAPE, "B*H = %lld exceeds 2^31-1", BH);
    if (N > 0x7fffffffLL / 1024) return fail(FA_ERR_SHAPE, "N = %lld too large", N);
    const double total = static_cast<double>(BH) * static_cast<double>(N) * static_cast<double>(d);
    if (total > 4.0e18) return fail(FA_ERR_SHAPE, "B*H*N*d = %.3g exceeds 2^62", total);
    return FA_OK;
}

// Key split of the decode path.  One query (the vector-ALU kernel, 4 waves per workgroup, no LDS):
// about 16 waves per CU, chunks of at least 256 keys.  Several queries (the matrix kernel, 4 waves per
// workgroup or 2 at d = 256, one workgroup per CU by LDS): enough workgroups to cover the 256 CUs,
// chunks of at least 64 keys per wave.  Chunk lengths are multiples of 32 keys.
void decode_plan(long long BH, int Nq, long long Nk, int d, int* nw, int* nsplit, int* chunk) {
    const bool vec = Nq == 1;
    const int w = vec ? 4 : (d >= 256 ? 2 : 4);
    long long ns = vec ? (1024 + BH - 1) / BH : (256 + BH - 1) / BH;
    const long long maxs = Nk / (w * (vec ? 256 : 64));
    if (ns > maxs) ns = maxs;
    if (ns < 1) ns = 1;
    const long long nc = ns * w;
    long long ck = (Nk + nc - 1) / nc;
    ck = (ck + 31) / 32 * 32;
    *nw = w;
    *nsplit = static_cast<int>(ns);
    *chunk = static_cast<int>(ck);
}

size_t decode_bytes(long long BH, int Nq, int Nk, int d) {
    int nw = 4, ns = 1, ck = 32;
    decode_plan(BH, Nq, Nk, d, &nw, &ns, &ck);
    return static_cast<size_t>(BH) * ns * nw * Nq * (d + 1) * sizeof(float);
}

// Row stride (elements) of the unfused path's score and probability matrices.
long long naive_ld(long long N) { return (N + 63) / 64 * 64; }

// Shared checks of the unfused entry points: 16-bit dtype, sizes, and that every launch index fits.
int naive_check(int dtype, int B, int H, int N) {
    if (dtype != FA_F16 && dtype != FA_BF16) {
        if (elem_bytes(dtype) == 0) return fail(FA_ERR_DTYPE, "dtype code %d is not a fa_dtype", dtype);
        return fail(FA_ERR_UNSUPPORTED, "unfused path dtype %d (supported: FA_F16, FA_BF16)", dtype);
    }
    if (B < 0 || H < 0 || N < 0) return fail(FA_ERR_SHAPE, "negative size B=%d H=%d N=%d", B, H, N);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (int st = check_sizes(BH, N, 256)) return st;
    const double elems = static_cast<double>(BH) * static_cast<double>(N) * static_cast<double>(naive_ld(N));
    if (elems * 6.0 > 4.0e18) return fail(FA_ERR_SHAPE, "B*H*N*ld = %.3g: the N x N matrices exceed 2^62 bytes", elems);
    const long long nt = (N + 127) / 128;
    if (BH * nt * nt > 0x7fffffffLL || (BH * N + 3) / 4 > 0x7fffffffLL)
        return fail(FA_ERR_SHAPE, "B*H*N = %lld too large for the unfused path's grids", BH * N);
    return FA_OK;
}

int from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return FA_OK;
    if (e == hipErrorNotSupported) return fail(FA_ERR_UNSUPPORTED, "%s: no kernel instance for this request", what);
    return fail(FA_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_last_error(void) { return g_err; }

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative or overflowing sizes";
        case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid request not implemented by this library";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointer not 16-byte aligned";
        case FA_ERR_ARG: return "FA_ERR_ARG: invalid argument";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a launch";
        default: return "unknown fa_status";
    }
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
              int causal, float scale, int dtype, const fa_fp8_scales* s8, void* stream) {
    g_err[0] = '\0';
    const int eb = elem_bytes(dtype);
    if (eb == 0) return fail(FA_ERR_DTYPE, "dtype code %d is not one of FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3", dtype);
    if (B < 0 || H < 0 || N < 0) return fail(FA_ERR_SHAPE, "negative size B=%d H=%d N=%d", B, H, N);
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (int st = check_sizes(BH, N, d)) return st;
    if (!q || !k || !v || !o) return fail(FA_ERR_NULL, "q, k, v and o must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
        return fail(FA_ERR_ALIGN, "q, k, v, o, lse must be 16-byte aligned");
    const size_t in_bytes = static_cast<size_t>(BH) * N * d * eb;
    const size_t out_bytes = static_cast<size_t>(BH) * N * d * (dtype == FA_FP8_E4M3 ? 2 : eb);
    if (overlaps(o, out_bytes, q, in_bytes) || overlaps(o, out_bytes, k, in_bytes) || overlaps(o, out_bytes, v, in_bytes))
        return fail(FA_ERR_ARG, "o must not overlap q, k or v");
    if (lse && overlaps(lse, static_cast<size_t>(BH) * N * 4, o, out_bytes))
        return fail(FA_ERR_ARG, "lse must not overlap o");

    // softmax in base 2: p = 2^(s*c - m) with c = |scale| * log2(e); a negative scale negates Q.
    // c is kept >= 1e-30 so that masked scores (-inf) times c stay -inf; for |scale| below that the
    // result is the same as for scale 0 in float32 (every weight rounds to 1).
    float c = static_cast<float>(std::fabs(static_cast<double>(scale)) * 1.4426950408889634);
    if (!(c >= 1e-30f)) c = 1e-30f;
    const bool qneg = std::signbit(scale);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int bh = static_cast<int>(BH);

    switch (dtype) {
        case FA_F32:
            return from_hip(fa::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                               static_cast<const float*>(v), static_cast<float*>(o), lse, bh, N, d,
                                               causal != 0, c, qneg, st),
                            "fa_fwd(f32)");
        case FA_F16:
        case FA_BF16:
            return from_hip(fa::launch_fwd_16(dtype == FA_BF16, q, k, v, o, lse, bh, N, N, 0, d, causal != 0, c,
                                              qneg ? 0x80008000u : 0u, st),
                            dtype == FA_BF16 ? "fa_fwd(bf16)" : "fa_fwd(f16)");
        case FA_FP8_E4M3: {
            const float *sq = nullptr, *sk = nullptr, *sv = nullptr;
            if (s8) {
                if (s8->block != 64) return fail(FA_ERR_UNSUPPORTED, "fp8 scale block %d (supported: 64)", s8->block);
                if (!s8->q_scale || !s8->k_scale || !s8->v_scale)
                    return fail(FA_ERR_NULL, "fp8 scales: q_scale, k_scale and v_scale must be non-NULL");
                if (misaligned(s8->q_scale) || misaligned(s8->k_scale) || misaligned(s8->v_scale))
                    return fail(FA_ERR_ALIGN, "fp8 scale arrays must be 16-byte aligned");
                sq = s8->q_scale;
                sk = s8->k_scale;
                sv = s8->v_scale;
            }
            return from_hip(fa::launch_fwd_fp8(q, k, v, o, lse, sq, sk, sv, bh, N, d, causal != 0, c, qneg, st),
                            "fa_fwd(fp8)");
        }
        default:
            return fail(FA_ERR_DTYPE, "dtype code %d", dtype);
    }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
           float scale, int dtype, void* stream) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, nullptr, stream);
}

int fa_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                int q_start, int d, int causal, float scale, int dtype, void* stream) {
    g_err[0] = '\0';
    const int eb = elem_bytes(dtype);
    if (eb == 0) return fail(FA_ERR_DTYPE, "dtype code %d is not one of FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3", dtype);
    if (dtype != FA_F16 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "fa_fwd_rect dtype %d (supported: FA_F16, FA_BF16)", dtype);
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return fail(FA_ERR_SHAPE, "negative size B=%d H=%d Nq=%d Nk=%d", B, H, Nq, Nk);
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (causal ? (q_start < 0 || static_cast<long long>(q_start) + Nq > Nk) : q_start != 0)
        return fail(FA_ERR_ARG, "q_start = %d: causal needs 0 <= q_start <= Nk - Nq (Nq=%d, Nk=%d), non-causal 0",
                    q_start, Nq, Nk);
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || Nq == 0) return FA_OK;
    if (Nk == 0) return fail(FA_ERR_SHAPE, "Nq = %d queries against no keys", Nq);
    if (int st = check_sizes(BH, Nq, d)) return st;
    if (int st = check_sizes(BH, Nk, d)) return st;
    if (!q || !k || !v || !o) return fail(FA_ERR_NULL, "q, k, v and o must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
        return fail(FA_ERR_ALIGN, "q, k, v, o, lse must be 16-byte aligned");
    const size_t qbytes = static_cast<size_t>(BH) * Nq * d * eb, kbytes = static_cast<size_t>(BH) * Nk * d * eb;
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
        return fail(FA_ERR_ARG, "o must not overlap q, k or v");
    if (lse && overlaps(lse, static_cast<size_t>(BH) * Nq * 4, o, qbytes)) return fail(FA_ERR_ARG, "lse must not overlap o");
    float c = static_cast<float>(std::fabs(static_cast<double>(scale)) * 1.4426950408889634);
    if (!(c >= 1e-30f)) c = 1e-30f;
    return from_hip(fa::launch_fwd_16(dtype == FA_BF16, q, k, v, o, lse, static_cast<int>(BH), Nq, Nk, q_start, d,
                                      causal != 0, c, std::signbit(scale) ? 0x80008000u : 0u,
                                      reinterpret_cast<hipStream_t>(stream)),
                    dtype == FA_BF16 ? "fa_fwd_rect(bf16)" : "fa_fwd_rect(f16)");
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int Nq, int d, int nsplit) {
    if (B <= 0 || H <= 0 || Nq <= 0 || d <= 0 || nsplit <= 0) return 0;
    return static_cast<size_t>(B) * H * nsplit * Nq * (d + 1) * sizeof(float);
}

int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                 int q_start, int d, int causal, float scale, int dtype, int nsplit, void* workspace,
                 size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    const int eb = elem_bytes(dtype);
    if (eb == 0) return fail(FA_ERR_DTYPE, "dtype code %d is not one of FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3", dtype);
    if (dtype != FA_F16 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "fa_fwd_split dtype %d (supported: FA_F16, FA_BF16)", dtype);
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return fail(FA_ERR_SHAPE, "negative size B=%d H=%d Nq=%d Nk=%d", B, H, Nq, Nk);
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (causal ? (q_start < 0 || static_cast<long long>(q_start) + Nq > Nk) : q_start != 0)
        return fail(FA_ERR_ARG, "q_start = %d: causal needs 0 <= q_start <= Nk - Nq (Nq=%d, Nk=%d), non-causal 0",
                    q_start, Nq, Nk);
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    if (nsplit < 1 || nsplit > 64) return fail(FA_ERR_ARG, "nsplit must be 1..64, got %d", nsplit);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || Nq == 0) return FA_OK;
    if (Nk == 0) return fail(FA_ERR_SHAPE, "Nq = %d queries against no keys", Nq);
    if (int st = check_sizes(BH, Nq, d)) return st;
    if (int st = check_sizes(BH, Nk, d)) return st;
    if (int st = check_sizes(BH * nsplit, Nq, d + 1)) return st;
    if (!q || !k || !v || !o || !workspace) return fail(FA_ERR_NULL, "q, k, v, o and workspace must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) || misaligned(workspace))
        return fail(FA_ERR_ALIGN, "q, k, v, o, lse and workspace must be 16-byte aligned");
    const size_t need = fa_fwd_split_workspace_bytes(B, H, Nq, d, nsplit);
    if (workspace_bytes < need) return fail(FA_ERR_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const size_t qbytes = static_cast<size_t>(BH) * Nq * d * eb, kbytes = static_cast<size_t>(BH) * Nk * d * eb;
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
        return fail(FA_ERR_ARG, "o must not overlap q, k or v");
    const size_t lbytes = static_cast<size_t>(BH) * Nq * 4;
    if (overlaps(workspace, need, q, qbytes) || overlaps(workspace, need, k, kbytes) ||
        overlaps(workspace, need, v, kbytes) || overlaps(workspace, need, o, qbytes) ||
        (lse && overlaps(workspace, need, lse, lbytes)))
        return fail(FA_ERR_ARG, "workspace must not overlap any tensor");
    if (lse && overlaps(lse, lbytes, o, qbytes)) return fail(FA_ERR_ARG, "lse must not overlap o");
    float c = static_cast<float>(std::fabs(static_cast<double>(scale)) * 1.4426950408889634);
    if (!(c >= 1e-30f)) c = 1e-30f;
    return from_hip(fa::launch_fwd_16_split(dtype == FA_BF16, q, k, v, o, lse, static_cast<float*>(workspace), nsplit,
                                            static_cast<int>(BH), Nq, Nk, q_start, d, causal != 0, c,
                                            std::signbit(scale) ? 0x80008000u : 0u,
                                            reinterpret_cast<hipStream_t>(stream)),
                    dtype == FA_BF16 ? "fa_fwd_split(bf16)" : "fa_fwd_split(f16)");
}

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
    return decode_bytes(static_cast<long long>(B) * H, Nq, Nk, d);
}

}  // extern "C"

namespace {

static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_BYTES, "the header states the library-held size");

// Checks shared by the decode entry points; own_ws: the library-held array replaces the caller workspace.
int decode_check(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                 int d, int causal, float scale, int dtype, const void* ws, size_t ws_bytes, bool own_ws,
                 const char* fn) {
    if (dtype != FA_F16 && dtype != FA_BF16) {
        if (elem_bytes(dtype) == 0) return fail(FA_ERR_DTYPE, "dtype code %d is not a fa_dtype", dtype);
        return fail(FA_ERR_UNSUPPORTED, "%s dtype %d (supported: FA_F16, FA_BF16)", fn, dtype);
    }
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return fail(FA_ERR_SHAPE, "negative size B=%d H=%d Nq=%d Nk=%d", B, H, Nq, Nk);
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (d != 64 && d != 128 && d != 256)
        return fail(FA_ERR_UNSUPPORTED, "%s head dimension d=%d (supported: 64, 128, 256)", fn, d);
    if (Nq > 32) return fail(FA_ERR_UNSUPPORTED, "%s takes at most 32 queries per head, got %d", fn, Nq);
    if (Nq > Nk) return fail(FA_ERR_SHAPE, "fewer keys (%d) than queries (%d)", Nk, Nq);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || Nq == 0) return FA_OK;
    if (int st = check_sizes(BH, Nk, d)) return st;
    if (!q || !k || !v || !o || (!own_ws && !ws))
        return fail(FA_ERR_NULL, own_ws ? "q, k, v and o must be non-NULL" : "q, k, v, o and workspace must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) || misaligned(ws))
        return fail(FA_ERR_ALIGN, "q, k, v, o, lse and workspace must be 16-byte aligned");
    const size_t need = decode_bytes(BH, Nq, Nk, d);
    if (own_ws) {
        if (need > fa::kDecodeScratchBytes)
            return fail(FA_ERR_UNSUPPORTED, "%s: this shape needs %zu bytes of workspace, more than the library-held "
                        "%zu bytes (use fa_fwd_decode with a caller workspace)", fn, need, fa::kDecodeScratchBytes);
    } else if (ws_bytes < need) {
        return fail(FA_ERR_ARG, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    }
    const size_t qb = static_cast<size_t>(BH) * Nq * d * 2, kb = static_cast<size_t>(BH) * Nk * d * 2;
    if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb))
        return fail(FA_ERR_ARG, "o must not overlap q, k or v");
    if (!own_ws && (overlaps(ws, need, q, qb) || overlaps(ws, need, k, kb) || overlaps(ws, need, v, kb) ||
                    overlaps(ws, need, o, qb) || (lse && overlaps(ws, need, lse, static_cast<size_t>(BH) * Nq * 4))))
        return fail(FA_ERR_ARG, "workspace must not overlap any tensor");
    if (lse && overlaps(lse, static_cast<size_t>(BH) * Nq * 4, o, qb)) return fail(FA_ERR_ARG, "lse must not overlap o");
    return FA_OK;
}

int decode_launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, int causal, float scale, int dtype, float* work, void* stream) {
    const long long BH = static_cast<long long>(B) * H;
    float c = static_cast<float>(std::fabs(static_cast<double>(scale)) * 1.4426950408889634);
    if (!(c >= 1e-30f)) c = 1e-30f;
    int nw = 4, ns = 1, ck = 32;
    decode_plan(BH, Nq, Nk, d, &nw, &ns, &ck);
    return from_hip(fa::launch_decode_16(dtype == FA_BF16, q, k, v, o, lse, work, static_cast<int>(BH), Nq, Nk, d,
                                         causal != 0, ns, ck, c, std::signbit(scale) ? 0x80008000u : 0u,
                                         reinterpret_cast<hipStream_t>(stream)),
                    dtype == FA_BF16 ? "fa_fwd_decode(bf16)" : "fa_fwd_decode(f16)");
}

}  // namespace

extern "C" {

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    if (int st = decode_check(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, workspace, workspace_bytes, false,
                              "fa_fwd_decode"))
        return st;
    if (static_cast<long long>(B) * H == 0 || Nq == 0) return FA_OK;
    return decode_launch(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, static_cast<float*>(workspace), stream);
}

int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                          int Nk, int d, int causal, float scale, int dtype, void* stream) {
    g_err[0] = '\0';
    if (int st = decode_check(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, nullptr, 0, true,
                              "fa_fwd_decode_noalloc"))
        return st;
    if (static_cast<long long>(B) * H == 0 || Nq == 0) return FA_OK;
    float* work = nullptr;
    const hipError_t e = fa::decode_scratch_ptr(&work);
    if (e != hipSuccess)
        return fail(FA_ERR_HIP, "fa_fwd_decode_noalloc: device address of the library-held workspace: %s",
                    hipGetErrorString(e));
    return decode_launch(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, work, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* delta, int B, int H, int N, int d, int causal, float scale, int dtype,
           void* stream) {
    g_err[0] = '\0';
    if (dtype != FA_F16 && dtype != FA_BF16) {
        if (elem_bytes(dtype) == 0) return fail(FA_ERR_DTYPE, "dtype code %d is not a fa_dtype", dtype);
        return fail(FA_ERR_UNSUPPORTED, "fa_bwd dtype %d (supported: FA_F16, FA_BF16)", dtype);
    }
    if (B < 0 || H < 0 || N < 0) return fail(FA_ERR_SHAPE, "negative size B=%d H=%d N=%d", B, H, N);
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "fa_bwd head dimension d=%d (supported: 64, 128, 256)", d);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (int st = check_sizes(BH, N, d)) return st;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta)
        return fail(FA_ERR_NULL, "q, k, v, o, lse, dout, dq, dk, dv and delta must be non-NULL");
    const void* all[] = {q, k, v, o, lse, dout, dq, dk, dv, delta};
    for (const void* ptr : all)
        if (misaligned(ptr)) return fail(FA_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const size_t tb = static_cast<size_t>(BH) * N * d * 2, rb = static_cast<size_t>(BH) * N * 4;
    const void* ins[] = {q, k, v, o, dout};
    void* outs[] = {dq, dk, dv};
    for (void* out : outs) {
        for (const void* in : ins)
            if (overlaps(out, tb, in, tb)) return fail(FA_ERR_ARG, "dq, dk, dv must not overlap q, k, v, o or dout");
        if (overlaps(out, tb, lse, rb) || overlaps(out, tb, delta, rb))
            return fail(FA_ERR_ARG, "dq, dk, dv must not overlap lse or delta");
    }
    if (overlaps(dq, tb, dk, tb) || overlaps(dq, tb, dv, tb) || overlaps(dk, tb, dv, tb))
        return fail(FA_ERR_ARG, "dq, dk and dv must not overlap each other");
    for (const void* in : ins)
        if (overlaps(delta, rb, in, tb)) return fail(FA_ERR_ARG, "delta must not overlap the inputs");
    if (overlaps(delta, rb, lse, rb)) return fail(FA_ERR_ARG, "delta must not overlap lse");
    return from_hip(fa::launch_bwd_16(dtype == FA_BF16, q, k, v, o, lse, dout, dq, dk, dv, delta, static_cast<int>(BH),
                                      N, d, causal != 0, scale, reinterpret_cast<hipStream_t>(stream)),
                    dtype == FA_BF16 ? "fa_bwd(bf16)" : "fa_bwd(f16)");
}

int fa_naive_row_stride(int N) { return N <= 0 ? 0 : static_cast<int>(naive_ld(N)); }

size_t fa_naive_workspace_bytes(int B, int H, int N) {
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    return static_cast<size_t>(B) * H * N * naive_ld(N) * 6;
}

int fa_naive_scores(const void* q, const void* k, float* s, int B, int H, int N, int d, float scale, int dtype,
                    void* stream) {
    g_err[0] = '\0';
    if (int st = naive_check(dtype, B, H, N)) return st;
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (!q || !k || !s) return fail(FA_ERR_NULL, "q, k and s must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(s)) return fail(FA_ERR_ALIGN, "q, k and s must be 16-byte aligned");
    const size_t in = static_cast<size_t>(BH) * N * d * 2, sb = static_cast<size_t>(BH) * N * naive_ld(N) * 4;
    if (overlaps(s, sb, q, in) || overlaps(s, sb, k, in)) return fail(FA_ERR_ARG, "s must not overlap q or k");
    return from_hip(fa::launch_naive_scores_16(dtype == FA_BF16, q, k, s, static_cast<int>(BH), N, d,
                                               static_cast<int>(naive_ld(N)), scale, reinterpret_cast<hipStream_t>(stream)),
                    "fa_naive_scores");
}

int fa_naive_softmax(const float* s, void* p, float* lse, int B, int H, int N, int causal, int dtype, void* stream) {
    g_err[0] = '\0';
    if (int st = naive_check(dtype, B, H, N)) return st;
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (!s || !p) return fail(FA_ERR_NULL, "s and p must be non-NULL");
    if (misaligned(s) || misaligned(p) || misaligned(lse)) return fail(FA_ERR_ALIGN, "s, p and lse must be 16-byte aligned");
    const size_t cells = static_cast<size_t>(BH) * N * naive_ld(N);
    if (overlaps(p, cells * 2, s, cells * 4)) return fail(FA_ERR_ARG, "p must not overlap s");
    if (lse && (overlaps(lse, static_cast<size_t>(BH) * N * 4, s, cells * 4) ||
                overlaps(lse, static_cast<size_t>(BH) * N * 4, p, cells * 2)))
        return fail(FA_ERR_ARG, "lse must not overlap s or p");
    return from_hip(fa::launch_naive_softmax_16(dtype == FA_BF16, s, p, lse, static_cast<int>(BH), N,
                                                static_cast<int>(naive_ld(N)), causal != 0,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "fa_naive_softmax");
}

int fa_naive_pv(const void* p, const void* v, void* o, int B, int H, int N, int d, int dtype, void* stream) {
    g_err[0] = '\0';
    if (int st = naive_check(dtype, B, H, N)) return st;
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (!p || !v || !o) return fail(FA_ERR_NULL, "p, v and o must be non-NULL");
    if (misaligned(p) || misaligned(v) || misaligned(o)) return fail(FA_ERR_ALIGN, "p, v and o must be 16-byte aligned");
    const size_t ob = static_cast<size_t>(BH) * N * d * 2, pb = static_cast<size_t>(BH) * N * naive_ld(N) * 2;
    if (overlaps(o, ob, p, pb) || overlaps(o, ob, v, ob)) return fail(FA_ERR_ARG, "o must not overlap p or v");
    return from_hip(fa::launch_naive_pv_16(dtype == FA_BF16, p, v, o, static_cast<int>(BH), N, d,
                                           static_cast<int>(naive_ld(N)), reinterpret_cast<hipStream_t>(stream)),
                    "fa_naive_pv");
}

int fa_fwd_naive(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                 int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    if (int st = naive_check(dtype, B, H, N)) return st;
    if (causal != 0 && causal != 1) return fail(FA_ERR_ARG, "causal must be 0 or 1, got %d", causal);
    if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale must be finite");
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    const long long BH = static_cast<long long>(B) * H;
    if (BH == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !workspace) return fail(FA_ERR_NULL, "q, k, v, o and workspace must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) || misaligned(workspace))
        return fail(FA_ERR_ALIGN, "q, k, v, o, lse and workspace must be 16-byte aligned");
    const size_t need = fa_naive_workspace_bytes(B, H, N);
    if (workspace_bytes < need) return fail(FA_ERR_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const size_t tb = static_cast<size_t>(BH) * N * d * 2;
    if (overlaps(o, tb, q, tb) || overlaps(o, tb, k, tb) || overlaps(o, tb, v, tb))
        return fail(FA_ERR_ARG, "o must not overlap q, k or v");
    if (overlaps(workspace, need, q, tb) || overlaps(workspace, need, k, tb) || overlaps(workspace, need, v, tb) ||
        overlaps(workspace, need, o, tb) || (lse && overlaps(workspace, need, lse, static_cast<size_t>(BH) * N * 4)))
        return fail(FA_ERR_ARG, "workspace must not overlap any tensor");
    if (lse && overlaps(lse, static_cast<size_t>(BH) * N * 4, o, tb)) return fail(FA_ERR_ARG, "lse must not overlap o");
    float* s = static_cast<float*>(workspace);
    char* p = static_cast<char*>(workspace) + static_cast<size_t>(BH) * N * naive_ld(N) * 4;
    if (int st = fa_naive_scores(q, k, s, B, H, N, d, scale, dtype, stream)) return st;
    if (int st = fa_naive_softmax(s, p, lse, B, H, N, causal, dtype, stream)) return st;
    return fa_naive_pv(p, v, o, B, H, N, d, dtype, stream);
}

}  // extern "C"

namespace {

// Checks shared by the preparation entry points; fills the sign bit set.  *empty is set for a no-op.
int prep_check(int x_dtype, const int8_t* hadamard, int block, int BH, int N, int d, uint64_t bits[4], bool* empty,
               const char* fn) {
    *empty = false;
    if (x_dtype != FA_F32 && x_dtype != FA_F16 && x_dtype != FA_BF16)
        return fail(FA_ERR_DTYPE, "%s input dtype %d (supported: FA_F32, FA_F16, FA_BF16)", fn, x_dtype);
    if (BH < 0 || N < 0) return fail(FA_ERR_SHAPE, "negative size BH=%d N=%d", BH, N);
    if (block < 1 || block > 1024) return fail(FA_ERR_ARG, "block must be in 1..1024, got %d", block);
    if (d != 64 && d != 128 && d != 256) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d (supported: 64, 128, 256)", d);
    bits[0] = bits[1] = bits[2] = bits[3] = 0;
    if (hadamard) {
        for (int t = 0; t < d; ++t) {
            if (hadamard[t] == -1)
                bits[t >> 6] |= uint64_t{1} << (t & 63);
            else if (hadamard[t] != 1)
                return fail(FA_ERR_ARG, "hadamard[%d] = %d; signs must be +1 or -1", t, static_cast<int>(hadamard[t]));
        }
    }
    if (BH == 0 || N == 0) {
        *empty = true;
        return FA_OK;
    }
    return check_sizes(BH, N, d);
}

int prep_code(int x_dtype) { return x_dtype == FA_F32 ? 0 : x_dtype == FA_F16 ? 1 : 2; }

}  // namespace

extern "C" {

int fa_fp8_prep(const void* x, int x_dtype, void* x8, float* scales, const int8_t* hadamard, int block, int BH, int N,
                int d, void* stream) {
    g_err[0] = '\0';
    uint64_t bits[4];
    bool empty = false;
    if (int st = prep_check(x_dtype, hadamard, block, BH, N, d, bits, &empty, "fa_fp8_prep")) return st;
    if (empty) return FA_OK;
    if (!x || !x8 || !scales) return fail(FA_ERR_NULL, "x, x8 and scales must be non-NULL");
    if (misaligned(x) || misaligned(x8) || misaligned(scales))
        return fail(FA_ERR_ALIGN, "x, x8 and scales must be 16-byte aligned");
    return from_hip(fa::launch_fp8_prep(x, prep_code(x_dtype), x8, scales, hadamard != nullptr, bits, block, BH, N, d,
                                        reinterpret_cast<hipStream_t>(stream)),
                    "fa_fp8_prep");
}

int fa_fp8_prep_qkv(const void* q, const void* k, const void* v, int x_dtype, void* q8, void* k8, void* v8,
                    float* q_scales, float* k_scales, float* v_scales, const int8_t* hadamard, int block, int BH,
                    int N, int d, void* stream) {
    g_err[0] = '\0';
    uint64_t bits[4];
    bool empty = false;
    if (int st = prep_check(x_dtype, hadamard, block, BH, N, d, bits, &empty, "fa_fp8_prep_qkv")) return st;
    if (empty) return FA_OK;
    const void* xs[3] = {q, k, v};
    void* x8s[3] = {q8, k8, v8};
    float* ss[3] = {q_scales, k_scales, v_scales};
    for (int t = 0; t < 3; ++t) {
        if (!xs[t] || !x8s[t] || !ss[t]) return fail(FA_ERR_NULL, "every input, code and scale pointer must be non-NULL");
        if (misaligned(xs[t]) || misaligned(x8s[t]) || misaligned(ss[t]))
            return fail(FA_ERR_ALIGN, "every pointer must be 16-byte aligned");
    }
    const int eb = elem_bytes(x_dtype);
    const size_t in_b = static_cast<size_t>(BH) * N * d * eb, code_b = static_cast<size_t>(BH) * N * d;
    const size_t sc_b = static_cast<size_t>(BH) * ((N + block - 1) / block) * 4;
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 3; ++b) {
            if (overlaps(x8s[a], code_b, xs[b], in_b) || overlaps(ss[a], sc_b, xs[b], in_b) ||
                overlaps(ss[a], sc_b, x8s[b], code_b) || (a != b && (overlaps(x8s[a], code_b, x8s[b], code_b) ||
                                                                     overlaps(ss[a], sc_b, ss[b], sc_b))))
                return fail(FA_ERR_ARG, "the outputs must not overlap each other or the inputs");
        }
    }
    return from_hip(fa::launch_fp8_prep_qkv(xs, prep_code(x_dtype), x8s, ss, hadamard != nullptr, bits, block, BH, N,
                                            d, reinterpret_cast<hipStream_t>(stream)),
                    "fa_fp8_prep_qkv");
}

}  // extern "C"
