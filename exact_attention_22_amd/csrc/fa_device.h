// fa_device.h -- gfx950 (CDNA4) building blocks shared by the attention kernels.
//
// Only device code lives here: MFMA wrappers, 16-bit packing, LDS transpose
// reads, the cross-half lane exchange, the LDS swizzle, buffer loads into LDS,
// and the length ranking of packed sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16) * B(16x32) on 16-bit inputs.
// Lane l holds A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32] (8 halves
// each, as 4 dwords); the result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> one dword of two 16-bit values, round to nearest even
// (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <bool BF16>
__device__ __forceinline__ u32 pack2(float lo, float hi) {
    if constexpr (BF16)
        return __builtin_bit_cast(u32, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    else
        return __builtin_bit_cast(u32, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// 16-bit -> fp32 (exact).
template <bool BF16>
__device__ __forceinline__ float widen(uint16_t x) {
    if constexpr (BF16)
        return __uint_as_float((u32)x << 16);
    else
        return (float)__builtin_bit_cast(_Float16, x);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, result lane j receives, as
// element r (0..3), the 16-bit element j%4 of the 8 bytes addressed by lane
// 4*r + j/4 of the group.  Used to read V (row-major [key][d] in LDS) as the
// key-contiguous operand of the P*V product.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
}

// Larger of two floats, NaN if either is NaN (v_maximum3_f32 on gfx950).  Unlike
// fmaxf it needs no canonicalisation of matrix-core results first.
__device__ __forceinline__ float fmax_raw(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Sum / max of a value over lanes l and l^32 (v_permlane32_swap: every lane
// ends with both halves' values).
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS tiles hold rows of D 16-bit values split into 16-byte chunks; chunk c of
// row r is stored at chunk position c ^ swz(r).  The swizzle keeps three access
// patterns free of bank conflicts (64 banks x 4 bytes):
//   * 16-byte writes of whole rows (consecutive lanes -> consecutive chunks);
//   * 16-byte reads of one chunk from 16 rows whose low 4 bits are distinct
//     (the K operand);
//   * transpose reads of 4 consecutive rows x 4 consecutive chunks (the V operand).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128)
        return ((r & 3) << 2) | ((r >> 2) & 3);        // 16 chunks per row
    else
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); // 8 chunks per row, 2 rows per bank line
}

template <int D>
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

// Raw buffer resource (stride 0) over `bytes` bytes at `base`; loads at
// offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, u32 bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// buffer_load_dwordx4 ... lds: every lane fetches the 16 bytes at byte offset
// voff of the buffer, and the wave's 64 results land contiguously in LDS,
// lane i at lds + 16*i (lds must be wave-uniform).  The caller waits for
// completion (s_waitcnt vmcnt(0)) before the barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, void* lds, u32 voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds,
                                             16, voff, 0, 0, 0);
}

// The packed sequence of rank p when the B <= 64 sequences are ordered by
// length cu[b+1] - cu[b], longest first (equal lengths in index order, so the
// ranks are a permutation of 0..B-1).  Every lane of the wavefront must call it;
// lane b takes sequence b and counts the sequences ranked before it.
__device__ __forceinline__ int seq_at_rank(const int* cu, int B, int p) {
    const int lane = threadIdx.x & 63;
    const int len = lane < B ? cu[lane + 1] - cu[lane] : 0;
    int rank = 0;
    for (int j = 0; j < B; ++j) {
        const int lj = __builtin_amdgcn_readlane(len, j);
        rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
    }
    const unsigned long long m = __ballot(lane < B && rank == p);
    return m ? (int)__builtin_ctzll(m) : p;
}

}  // namespace fa
