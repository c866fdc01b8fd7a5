// fa_api.hip -- the C ABI of libfa.so (declared in include/fa.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// then enqueues its kernels on the caller's stream and returns.  The library
// allocates, frees and synchronises nothing; fa_bwd_gqa_noalloc keeps its
// scratch in a fixed device array instead of a caller's workspace.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_d(int d) { return d == 64 || d == 128; }

// Element count a*b*c*d, or -1 when it leaves int64 or is non-positive.
int64_t count4(int64_t a, int64_t b, int64_t c, int64_t d) {
    if (a <= 0 || b <= 0 || c <= 0 || d <= 0) return -1;
    const int64_t lim = INT64_MAX / 8;
    int64_t x = a;
    for (int64_t f : {b, c, d}) {
        if (x > lim / f) return -1;
        x *= f;
    }
    return x;
}

fa_status check_common(int B, int H, int Nq, int Nk, int d, float scale, fa_dtype dtype) {
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
    if (count4(B, H, Nq, d) < 0 || count4(B, H, Nk, d) < 0) return FA_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX) return FA_ERR_SHAPE;
    if (!isfinite(scale)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

fa_status check_heads(int H, int H_kv) {
    return (H_kv < 1 || H % H_kv != 0) ? FA_ERR_SHAPE : FA_OK;
}

fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                   int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if ((st = check_heads(H, H_kv)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::FwdParams p{q, k, v, o, lse, B, H, Nq, Nk, d, causal != 0, dtype == FA_BF16, scale, 0};
    p.H_kv = H_kv;
    return from_hip(fa::launch_fwd(p, (hipStream_t)stream));
}

fa_status splitkv_impl(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                       int H, int H_kv, int Nq, int Nk, int d, int causal, float scale, int num_splits,
                       fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_NULL;
    fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if ((st = check_heads(H, H_kv)) != FA_OK) return st;
    if (num_splits < 1 || num_splits > Nk) return FA_ERR_SHAPE;
    if (count4(num_splits, B, H, (int64_t)Nq * d) < 0) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) || ((uintptr_t)lse_part & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::FwdParams p{q, k, v, o_part, lse_part, B, H, Nq, Nk, d, causal != 0, dtype == FA_BF16, scale,
                    num_splits};
    p.H_kv = H_kv;
    // One query row sees every key whatever the causal flag (j <= 0 + Nk - 1):
    // the streaming kernel serves it; longer query blocks use the tiled kernel.
    if (Nq == 1) return from_hip(fa::launch_decode(p, (hipStream_t)stream));
    return from_hip(fa::launch_fwd(p, (hipStream_t)stream));
}

// Scratch of the no-allocation backward: the backward's fp32 D and lse-in-base-2
// of up to FA_BWD_NOALLOC_MAX_ROWS query rows.  Each GPU that loads the library
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device array: the kernels get the device address
// that hipGetSymbolAddress returns on the current device, kept per device.
constexpr size_t kScratchBytes = (size_t)FA_BWD_NOALLOC_MAX_ROWS * 8u;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_lookup;

// Device address of `scratch` on the current device, looked up on the first call
// on each device (with that device current) and kept.
fa_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(scratch_lookup);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int d, int causal, float scale,
                 fa_dtype dtype, void* stream) {
    return fwd_impl(q, k, v, o, lse, B, H, H, Nq, Nk, d, causal, scale, dtype, stream);
}

fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale,
                     fa_dtype dtype, void* stream) {
    return fwd_impl(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, causal, scale, dtype, stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int* cu_seqlens_q, const int* cu_seqlens_k,
                         int B, int H, int H_kv, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int d, int causal, float scale,
                         fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0) return FA_ERR_SHAPE;
    if (total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1) return FA_ERR_SHAPE;
    if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_SHAPE;
    if (count4(total_q, H, d, 1) < 0 || count4(total_k, H_kv, d, 1) < 0) return FA_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX || B == INT32_MAX) return FA_ERR_SHAPE;
    // a K/V tile (64 rows of H_kv * d values) must lie within a 32-bit byte range
    if ((int64_t)H_kv * d * 2 * 64 > INT32_MAX) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u) ||
        ((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::FwdParams p{q, k, v, o, lse, B, H, max_seqlen_q, max_seqlen_k, d, causal != 0, dtype == FA_BF16,
                    scale, 0, true, cu_seqlens_q, cu_seqlens_k, H_kv, total_q, total_k};
    return from_hip(fa::launch_fwd(p, (hipStream_t)stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq) {
    const int64_t n = count4(B, H, Nq, 1);
    if (n < 0 || n > INT64_MAX / 8) return 0;
    return (size_t)n * 8u;   // D and LSE * log2(e), fp32 each
}

namespace {

// Argument checks of the backward except the workspace (host only, no HIP call).
fa_status bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
                    fa_dtype dtype) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if ((st = check_heads(H, H_kv)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 15u))
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int H_kv,
                   int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype, void* stream) {
    if (!workspace) return FA_ERR_NULL;
    fa_status st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq)) return FA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15u) return FA_ERR_UNSUPPORTED;
    fa::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, Nq, Nk, d, causal != 0,
                    dtype == FA_BF16, scale, H_kv};
    return from_hip(fa::launch_bwd(p, (hipStream_t)stream));
}

}  // namespace

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 int B, int H, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype, void* stream) {
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, Nq, Nk, d, causal,
                    scale, dtype, stream);
}

fa_status fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                     int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype,
                     void* stream) {
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H_kv, Nq, Nk, d, causal,
                    scale, dtype, stream);
}

fa_status fa_bwd_gqa_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq,
                             int Nk, int d, int causal, float scale, fa_dtype dtype, void* stream) {
    fa_status st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    const size_t need = fa_bwd_workspace_bytes(B, H, Nq);
    if (need == 0 || need > kScratchBytes) return FA_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != FA_OK) return st;
    fa::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, (float*)ws, B, H, Nq, Nk, d, causal != 0,
                    dtype == FA_BF16, scale, H_kv};
    return from_hip(fa::launch_bwd(p, (hipStream_t)stream));
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, void* workspace, size_t workspace_bytes, int B, int H, int H_kv,
                        int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                        float scale, fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k || !workspace)
        return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || check_heads(H, H_kv) != FA_OK) return FA_ERR_SHAPE;
    if (total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1) return FA_ERR_SHAPE;
    if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_SHAPE;
    if (count4(total_q, H, d, 1) < 0 || count4(total_k, H_kv, d, 1) < 0) return FA_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX || B == INT32_MAX) return FA_ERR_SHAPE;
    // a tile (64 rows of H * d values) must lie within a 32-bit byte range
    if ((int64_t)H * d * 2 * 64 > INT32_MAX) return FA_ERR_SHAPE;
    if (workspace_bytes < fa_bwd_workspace_bytes(1, H, total_q)) return FA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 15u) || ((uintptr_t)workspace & 15u) ||
        ((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, max_seqlen_q, max_seqlen_k, d,
                    causal != 0, dtype == FA_BF16, scale, H_kv};
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.total_q = total_q;
    p.total_k = total_k;
    return from_hip(fa::launch_bwd(p, (hipStream_t)stream));
}

size_t fa_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits) {
    if (!supported_d(d) || num_splits < 1) return 0;
    const int64_t n = count4(num_splits, B, H, Nq);
    if (n < 0 || n > INT64_MAX / 4 / (d + 1)) return 0;
    return (size_t)n * (size_t)(d + 1) * 4u;
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                         int B, int H, int Nq, int Nk, int d, int causal, float scale,
                         int num_splits, fa_dtype dtype, void* stream) {
    return splitkv_impl(q, k, v, o_part, lse_part, B, H, H, Nq, Nk, d, causal, scale, num_splits, dtype, stream);
}

fa_status fa_fwd_splitkv_gqa(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                             int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale,
                             int num_splits, fa_dtype dtype, void* stream) {
    return splitkv_impl(q, k, v, o_part, lse_part, B, H, H_kv, Nq, Nk, d, causal, scale, num_splits, dtype,
                        stream);
}

fa_status fa_fwd_splitkv_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seqlens_k,
                               float* o_part, float* lse_part,
                               int B, int H, int H_kv, int d, int page_size, int max_pages, int num_pages,
                               float scale, int num_splits, fa_dtype dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seqlens_k || !o_part || !lse_part) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || num_splits < 1) return FA_ERR_SHAPE;
    if (page_size < 1 || (page_size & (page_size - 1)) != 0) return FA_ERR_SHAPE;
    if (max_pages < 1 || num_pages < 1 || (int64_t)max_pages * page_size > INT32_MAX) return FA_ERR_SHAPE;
    if (count4(num_pages, page_size, H_kv, d) < 0 || count4(B, H, d, num_splits) < 0 ||
        count4(B, max_pages, 1, 1) < 0)
        return FA_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_part) ||
        ((uintptr_t)lse_part & 3u) || ((uintptr_t)block_table & 3u) || ((uintptr_t)seqlens_k & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::FwdParams p{q, k_cache, v_cache, o_part, lse_part, B, H, 1, max_pages * page_size, d, false,
                    dtype == FA_BF16, scale, num_splits};
    p.H_kv = H_kv;
    p.block_table = block_table;
    p.seqlens_k = seqlens_k;
    p.page_size = page_size;
    p.max_pages = max_pages;
    p.num_pages = num_pages;
    return from_hip(fa::launch_decode(p, (hipStream_t)stream));
}

fa_status fa_fwd_splitkv_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens_k,
                                float* o_part, float* lse_part,
                                int B, int H, int H_kv, int total_k, int max_seqlen_k, int d,
                                float scale, int num_splits, fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !cu_seqlens_k || !o_part || !lse_part) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || num_splits < 1) return FA_ERR_SHAPE;
    if (total_k < 1 || max_seqlen_k < 1 || max_seqlen_k > total_k) return FA_ERR_SHAPE;
    if (count4(total_k, H_kv, d, 1) < 0 || count4(B, H, d, num_splits) < 0) return FA_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX || B == INT32_MAX) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) || ((uintptr_t)lse_part & 3u) ||
        ((uintptr_t)cu_seqlens_k & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::FwdParams p{q, k, v, o_part, lse_part, B, H, 1, max_seqlen_k, d, false, dtype == FA_BF16, scale,
                    num_splits, true, nullptr, cu_seqlens_k, H_kv, B, total_k};
    return from_hip(fa::launch_decode(p, (hipStream_t)stream));
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                     const float* k_descale, const float* v_descale, void* o, float* lse,
                     int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale, void* stream) {
    if (!q || !k || !v || !q_descale || !k_descale || !v_descale || !o || !lse) return FA_ERR_NULL;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
    if (check_heads(H, H_kv) != FA_OK) return FA_ERR_SHAPE;
    if (count4(B, H, Nq, d) < 0 || count4(B, H_kv, Nk, d) < 0 || (int64_t)B * H > INT32_MAX) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u) ||
        ((uintptr_t)q_descale & 3u) || ((uintptr_t)k_descale & 3u) || ((uintptr_t)v_descale & 3u))
        return FA_ERR_UNSUPPORTED;
    fa::Fp8Params p{q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, H_kv, Nq, Nk, causal != 0, scale};
    return from_hip(fa::launch_fwd_fp8(p, (hipStream_t)stream));
}

fa_status fa_quantize_fp8(const void* x, void* x8, float* descale, int G, int N, int d, int block_rows,
                          fa_dtype dtype, void* stream) {
    if (!x || !x8 || !descale) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (d < 8 || d % 8 != 0) return FA_ERR_UNSUPPORTED;
    if (G < 1 || N < 1 || block_rows < 1 || count4(G, N, d, 1) < 0) return FA_ERR_SHAPE;
    if ((int64_t)G * ((N + (int64_t)block_rows - 1) / block_rows) > INT32_MAX) return FA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(x8) || ((uintptr_t)descale & 3u)) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_quant_fp8(x, x8, descale, G, N, d, block_rows, dtype == FA_BF16,
                                         (hipStream_t)stream));
}

fa_status fa_splitkv_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                             int B, int H, int Nq, int d, int num_splits, fa_dtype dtype, void* stream) {
    if (!o_part || !lse_part || !o || !lse) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Nq < 1 || num_splits < 1) return FA_ERR_SHAPE;
    const int64_t rows = count4(B, H, Nq, 1);
    if (rows < 0 || count4(num_splits, rows, d, 1) < 0) return FA_ERR_SHAPE;
    if (((uintptr_t)o_part & 3u) || ((uintptr_t)lse_part & 3u) || ((uintptr_t)o & 1u) || ((uintptr_t)lse & 3u))
        return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_combine(o_part, lse_part, o, lse, rows, d, num_splits, dtype == FA_BF16,
                                       (hipStream_t)stream));
}

const char* fa_status_str(fa_status status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid size: B, H, Nq, Nk must be >= 1, 1 <= num_splits <= Nk, H_kv divides H, no overflow";
        case FA_ERR_UNSUPPORTED: return "unsupported: d must be 64 or 128, dtype f16/bf16, finite scale, 16-byte aligned tensors";
        case FA_ERR_WORKSPACE: return "workspace too small";
        case FA_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

}  // extern "C"
