// fa_launch.h -- host-side launchers behind the C ABI (internal to libfa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Validated arguments of one forward launch.  In split mode `o` is the fp32
// o_part buffer and `lse` is lse_part; otherwise `o` holds dtype values.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Nq, Nk, d;
    bool causal;
    bool bf16;
    float scale;
    int num_splits;   // 0: plain forward; >= 1: split-KV partials
    // packed variable-length sequences with grouped K/V heads (then Nq and Nk
    // are the longest query and key sequences)
    bool varlen;
    const int* cu_q;  // device, B + 1 offsets
    const int* cu_k;
    int H_kv;
    int total_q, total_k;
    // paged K/V cache for the single-row decode (k, v: [num_pages, page_size,
    // H_kv, d]; Nk unused): non-null block_table selects it
    const int* block_table = nullptr;   // device, [B, max_pages]
    const int* seqlens_k = nullptr;     // device, [B]
    int page_size = 0, max_pages = 0, num_pages = 0;
};

// Validated arguments of one backward launch (q, o, dout, dq [B, H, Nq, d]; k, v,
// dk, dv [B, H_kv, Nk, d], H_kv = 0 meaning H; delta is the caller's fp32
// workspace of 2 * B * H * Nq values).
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;
    int B, H, Nq, Nk, d;
    bool causal;
    bool bf16;
    float scale;
    int H_kv = 0;
    // packed sequences (non-null cu_q): q, o, dout, dq [total_q, H, d], k, v, dk,
    // dv [total_k, H_kv, d], lse [H, total_q]; B sequences with offsets cu_q,
    // cu_k [B + 1] on the device; Nq, Nk the longest sequence's lengths
    const int* cu_q = nullptr;
    const int* cu_k = nullptr;
    int total_q = 0, total_k = 0;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
// Validated arguments of one FP8 forward: e4m3 q [B, H, Nq, 128], k and v
// [B, H_kv, Nk, 128]; descales q [B, H, ceil(Nq/128)], k [B, H_kv,
// ceil(Nk/128)], v [B, H_kv]; o bf16 [B, H, Nq, 128], lse [B, H, Nq].
struct Fp8Params {
    const void* q;
    const void* k;
    const void* v;
    const float* q_descale;
    const float* k_descale;
    const float* v_descale;
    void* o;
    float* lse;
    int B, H, H_kv, Nq, Nk;
    bool causal;
    float scale;
};

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream);
// x [G, N, d] 16-bit -> e4m3 codes [G, N, d] and descale [G, ceil(N / rows)]
hipError_t launch_quant_fp8(const void* x, void* x8, float* descale, int64_t G, int N, int d, int rows,
                            bool bf16, hipStream_t stream);
hipError_t launch_decode(const FwdParams& p, hipStream_t stream);
hipError_t launch_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                          int64_t rows, int d, int num_splits, bool bf16, hipStream_t stream);

// Workgroups of 256 query rows (eight wavefronts, one per CU) against 128 rows
// (four, two per CU) for a walk over nk keys, given how many 256-row workgroups
// the launch would make: the wider ones load each tile once for twice the rows
// but leave the grid half as fine.  Timed over B, H and N (256 to 16384) on the
// forward, the FP8 forward and the dQ kernel, the wider ones win from min_keys
// keys on when the grid keeps 256 of them, and from 4096 keys on with 128.
inline bool wide_rows(int64_t wide_blocks, int nk, int min_keys) {
    return (nk >= min_keys && wide_blocks >= 256) || (nk >= 4096 && wide_blocks >= 128);
}

// 256-row workgroups a launch over nq query rows of bh heads makes (causal:
// query tiles t and n-1-t share a workgroup).
inline int64_t wide_blocks(int nq, int64_t bh, bool causal) {
    const int64_t n = (nq + 255) / 256;
    return (causal ? (n + 1) / 2 : n) * bh;
}

// Keys per split chunk: ceil(Nk / num_splits).
inline int split_chunk(int Nk, int num_splits) { return (Nk + num_splits - 1) / num_splits; }

}  // namespace fa
