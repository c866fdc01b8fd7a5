// fa_fp8.hip -- FP8 (e4m3) forward with per-block scales on gfx950, and the
// block quantizer that produces its inputs.
//
// Method (the pages this follows): Q K^T and P V run on FP8 operands and a
// per-block scale factor keeps each block of data inside the narrow e4m3 range
// (Ringi, "Lecture 25", section 5.4); small attention weights underflowing in
// e4m3 are countered by scaling P per block before it is rounded (the FP8
// question of section 8.3).  Everything else is the FlashAttention-2 forward of
// fa_fwd.hip: Q outer, KV inner, online softmax with an unnormalised
// accumulator, causal tiles past the diagonal skipped.
//
// Scales (a dequantized value is code * descale):
//   * Q: one descale per 128 query rows -- one workgroup's rows;
//   * K: one descale per 128 keys -- one key tile;
//   * V: one descale per (batch, K/V head).
// The Q and K descales of a tile fold into the tile's exponent multiplier
// c = |scale| * log2(e) * qd * kd, so they cost nothing.  A V scale per key tile
// would force a rescale of the output accumulator at every tile; per head it
// multiplies the output once.
//
// P: p = 2^(s*c - M + LIFT) with the lazy reference M moved only when a row's
// maximum passes M + TAU.  With TAU = LIFT = 4 every p is at most 2^8 = 256,
// below e4m3's 448, and the largest weight of a row sits in [2^4, 2^8], so
// weights down to 2^-10 of it keep e4m3's full 3-bit precision and only those
// below about 2^-13 of it flush to zero.  The row sum is taken from the fp32 p
// before rounding; the LIFT cancels in O and is removed from the LSE.
//
// gfx950 mapping (not from the pages):
//   * v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales: 32x32 outputs,
//     K = 64, twice the bf16 rate.  Its two operands pair byte j of lane
//     32h + i (A) with byte j of lane 32h + n (B), so any consistent placement
//     of the contraction index works.
//   * S^T = K Q^T: Q in registers (32 bytes of d per lane and 64-wide slice), K
//     rows from LDS in the order with bits 2 and 3 swapped, so that accumulator
//     registers 8p..8p+7 are 8 consecutive keys; converting the two 32-key
//     blocks of a 64-key group to e4m3 in register order gives exactly the
//     B operand of O^T += V^T P^T.
//   * V^T through ds_read_b64_tr_b8 (within 16 lanes, result lane j, byte e
//     is byte j % 8 of the 8 bytes addressed by lane 2e + j / 8): four reads
//     give a lane the 32 keys of its P bytes for one d column.
//   * K/V tiles of 128 rows x 128 bytes in a two-stage LDS ring filled by
//     buffer loads that write LDS directly; rows past the last key read as
//     zeros.  XOR swizzle of the 16-byte chunks: conflict-free for the row
//     writes, the K chunk reads and the transposed V reads.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int F8_D = 128;       // head dimension (bytes per row)
constexpr int F8_QB = 128;      // query rows per Q scale block
constexpr int F8_BC = 128;      // keys per tile = K scale block
constexpr float F8_TAU = 4.0f;  // lazy-rescale threshold, log2 units
constexpr float F8_LIFT = 4.0f; // P lift, log2 units (TAU + LIFT <= log2(448))

struct F8Args {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const float* qd;   // [B, H, n_qblk]
    const float* kd;   // [B, H_kv, n_kblk]
    const float* vd;   // [B, H_kv]
    uint16_t* o;       // bf16 [B, H, Nq, d]
    float* lse;        // [B, H, Nq]
    int B, H, H_kv, group, Nq, Nk, BH, n_qtiles, n_kblk;
    int n_qblk;        // Q scale blocks per head: ceil(Nq / 128)
    float c;           // |scale| * log2(e)
    u32 qsign;         // 0x80808080 flips Q's sign when scale < 0
};

// Key index (within a 32-key block) that accumulator row i stands for: bits 2 and 3 swapped.
__device__ __forceinline__ int f8_perm_row(int i) {
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Tiles hold rows of 128 bytes (8 chunks of 16); chunk c of row r is stored at
// chunk position c ^ f8_swz(r), which depends on row bits 1..3 only.
__device__ __forceinline__ int f8_swz(int r) {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
__device__ __forceinline__ int f8_off(int row, int chunk) {
    return row * F8_D + ((chunk ^ f8_swz(row)) << 4);
}

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
    // scale operands 127: E8M0 exponent of 1.0 for both block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// four fp32 values -> one dword of four e4m3 codes (round to nearest even)
__device__ __forceinline__ int pack4_f8(float x0, float x1, float x2, float x3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// NW wavefronts per workgroup, 32 query rows each: 4 (two workgroups per CU) or 8
// (one per CU; each K/V tile is then loaded once for 256 query rows)
template <bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_fp8_kernel(F8Args a) {
    constexpr int BR = 32 * NW;                 // query rows per workgroup
    constexpr int TILE = F8_BC * F8_D;          // 16 KiB per K or V tile
    constexpr int NPW = TILE / 1024 / NW;       // 1 KiB loads per wave per tensor per tile
    constexpr int ND = F8_D / 32;               // 32-wide d blocks of O^T
    __shared__ __attribute__((aligned(16))) unsigned char stage0[2 * TILE];   // [K | V]
    __shared__ __attribute__((aligned(16))) unsigned char stage1[2 * TILE];

    // work items: XCD-contiguous ranges.  Causal: one workgroup runs query tiles
    // n_qtiles-1-t and t, which together see a fixed number of key tiles (equal
    // work per workgroup for the round-robin dispatcher); otherwise one tile.
    const int total = gridDim.x;
    int L = blockIdx.x;
    if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
    auto run_item = [&](const int qt, const int bh) __attribute__((always_inline)) {
        const int bkv = (bh / a.H) * a.H_kv + (bh % a.H) / a.group;
        const int q0 = qt * BR;
        const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;

        const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l32 = lane & 31, h = lane >> 5;
        const int qw = q0 + 32 * w, qi = qw + l32;

        const uint8_t* qg = a.q + (size_t)bh * Nq * F8_D;
        const uint8_t* kg = a.k + (size_t)bkv * Nk * F8_D;
        const uint8_t* vg = a.v + (size_t)bkv * Nk * F8_D;
        const float cq = a.c * a.qd[(size_t)bh * a.n_qblk + (q0 + 32 * w) / F8_QB];   // this wave's Q block
        const float* kdh = a.kd + (size_t)bkv * a.n_kblk;

        int hi = Nk;
        if (CAUSAL) hi = min(hi, min(Nq, q0 + BR) + off);
        const int n_tiles = hi > 0 ? (hi + F8_BC - 1) / F8_BC : 0;

        // Q: bytes 64ks + 32h .. +31 of this lane's row, for ks = 0, 1.  All four
        // loads go out before any is used (rows past Nq read the last row and are
        // zeroed, and the sign flipped, after the first tile's loads are issued).
        u32x4 qx[4];
        {
            const u32x4* src = (const u32x4*)(qg + (size_t)min(qi, Nq - 1) * F8_D + 32 * h);
    #pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                qx[2 * ks] = src[4 * ks];
                qx[2 * ks + 1] = src[4 * ks + 1];
            }
        }
        i32x8 qf[2];

        // LDS-direct loads: lane i of a 1 KiB load lands at byte 16 i; it fetches the
        // global chunk that the swizzled layout keeps there
        u32 voff[NPW];
    #pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int pos = (w * NPW + u) * 1024 + lane * 16;
            const int row = pos / F8_D, pchunk = (pos % F8_D) >> 4;
            voff[u] = (u32)(row * F8_D + ((pchunk ^ f8_swz(row)) << 4));
        }
        auto load_tile = [&](int tile, unsigned char* stage) {
            const int k0 = tile * F8_BC;
            const u32 nrec = (u32)__builtin_amdgcn_readfirstlane(min(Nk - k0, F8_BC)) * F8_D;
            const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kg + (size_t)k0 * F8_D, nrec);
            const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vg + (size_t)k0 * F8_D, nrec);
    #pragma unroll
            for (int u = 0; u < NPW; ++u) lds_dma16(rk, stage + (w * NPW + u) * 1024, voff[u]);
    #pragma unroll
            for (int u = 0; u < NPW; ++u) lds_dma16(rv, stage + TILE + (w * NPW + u) * 1024, voff[u]);
        };

        // operand offsets: K chunks 4ks + 2h and 4ks + 2h + 1 of row f8_perm_row(l32)
        // (32-key blocks only add constants); V^T reads as in the file comment
        const int krow = f8_perm_row(l32);
        int koff[2][2];
    #pragma unroll
        for (int ks = 0; ks < 2; ++ks)
    #pragma unroll
            for (int j = 0; j < 2; ++j) koff[ks][j] = f8_off(krow, 4 * ks + 2 * h + j);
        const int s16 = lane & 15, g16 = lane >> 4;
        const int vrow = 8 * h + (s16 >> 1);
        int vo[ND];
    #pragma unroll
        for (int db = 0; db < ND; ++db) vo[db] = f8_off(vrow, 2 * db + (g16 & 1)) + 8 * (s16 & 1);

        f32x16 oacc[ND];
    #pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
        float Mu = -INFINITY;   // exponent reference, log2 units of scaled scores
        float lsum = 0.f;       // this lane's half of the lifted row sum, relative to Mu

        // One key tile: S^T = K Q^T (4 blocks of 32 keys), online softmax update,
        // O^T += V^T P^T (2 groups of 64 keys).  MASKED tiles cross the key tail or
        // the causal diagonal.
        auto tile_step = [&](const unsigned char* Kb, const unsigned char* Vb, int tile, auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int k0 = tile * F8_BC;
            const float c = cq * kdh[tile];
            f32x16 sacc[4];
    #pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sacc[kb] = f32x16{};
    #pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const u32x4 x0 = *(const u32x4*)(Kb + 32 * kb * F8_D + koff[ks][0]);
                    const u32x4 x1 = *(const u32x4*)(Kb + 32 * kb * F8_D + koff[ks][1]);
                    const i32x8 kf = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                    sacc[kb] = mfma_f8(kf, qf[ks], sacc[kb]);
                }
            }
            // register r of block kb holds key k0 + 32kb + 16(r/8) + 8h + r%8
            int bound = 0;
            if constexpr (MASKED) {
                bound = Nk - k0 - 8 * h;
                if (CAUSAL) bound = min(bound, qi + off - k0 - 8 * h + 1);
    #pragma unroll
                for (int kb = 0; kb < 4; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * kb + 16 * (r >> 3) + (r & 7) >= bound) sacc[kb][r] = -INFINITY;
            }
            float mx = sacc[0][0];
    #pragma unroll
            for (int kb = 0; kb < 4; ++kb)
    #pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmax_raw(mx, sacc[kb][r]);
            mx = max_halves(mx);
            const float Mc = (mx == -INFINITY) ? -INFINITY : mx * c;
            if (__ballot(Mc > Mu + F8_TAU)) {        // wave-uniform: move the reference
                const float Mn = fmaxf(Mu, Mc);
                const float alpha = (Mn == -INFINITY) ? 1.f : exp2_fast(Mu - Mn);
                lsum *= alpha;
    #pragma unroll
                for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
                Mu = Mn;
            }
            const float bias = F8_LIFT - ((Mu == -INFINITY) ? 0.f : Mu);
    #pragma unroll
            for (int kb = 0; kb < 4; ++kb)
    #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_fast(__builtin_fmaf(sacc[kb][r], c, bias));
                    if constexpr (MASKED)
                        if (32 * kb + 16 * (r >> 3) + (r & 7) >= bound) p = 0.f;
                    sacc[kb][r] = p;
                    lsum += p;
                }
            // O^T += V^T P^T per 64-key group: P bytes in register order, V^T by
            // transposed reads (read t covers keys 16t + 8h + 0..7 of the group)
    #pragma unroll
            for (int kg = 0; kg < 2; ++kg) {
                const f32x16& P0 = sacc[2 * kg];
                const f32x16& P1 = sacc[2 * kg + 1];
                const i32x8 pb = {pack4_f8(P0[0], P0[1], P0[2], P0[3]), pack4_f8(P0[4], P0[5], P0[6], P0[7]),
                                  pack4_f8(P0[8], P0[9], P0[10], P0[11]), pack4_f8(P0[12], P0[13], P0[14], P0[15]),
                                  pack4_f8(P1[0], P1[1], P1[2], P1[3]), pack4_f8(P1[4], P1[5], P1[6], P1[7]),
                                  pack4_f8(P1[8], P1[9], P1[10], P1[11]), pack4_f8(P1[12], P1[13], P1[14], P1[15])};
    #pragma unroll
                for (int db = 0; db < ND; ++db) {
                    i32x8 va;
    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (__attribute__((address_space(3))) i32x2*)(Vb + (64 * kg + 16 * t) * F8_D + vo[db]));
                        va[2 * t] = r2[0];
                        va[2 * t + 1] = r2[1];
                    }
                    oacc[db] = mfma_f8(va, pb, oacc[db]);
                }
            }
        };

        // tiles from the last one down: the ones crossing the key tail or the
        // diagonal come first
        int n_masked = 0;
        while (n_masked < n_tiles) {
            const int k0 = (n_tiles - 1 - n_masked) * F8_BC;
            const bool clean = k0 + F8_BC <= Nk && (!CAUSAL || k0 + F8_BC - 1 <= q0 + off);
            if (clean) break;
            ++n_masked;
        }
        const int qmax_w = min(qw + 31, Nq - 1);
        if (n_tiles > 0) load_tile(n_tiles - 1, stage0);
        {
            const u32 sg = qi < Nq ? a.qsign : 0u;
            const u32 keep = qi < Nq ? ~0u : 0u;
    #pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 x0 = qx[2 * ks], x1 = qx[2 * ks + 1];
                qf[ks] = i32x8{(int)((x0[0] ^ sg) & keep), (int)((x0[1] ^ sg) & keep), (int)((x0[2] ^ sg) & keep),
                               (int)((x0[3] ^ sg) & keep), (int)((x1[0] ^ sg) & keep), (int)((x1[1] ^ sg) & keep),
                               (int)((x1[2] ^ sg) & keep), (int)((x1[3] ^ sg) & keep)};
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // the masked tiles, then the clean ones, each two per trip so that every step
        // reads one fixed LDS stage (one body per loop: nothing meets at a branch join,
        // and the compiler can tell the stage being read from the one being filled)
        int it = 0;
        auto masked_step = [&](unsigned char* cur, unsigned char* nxt) {
            const int tile = n_tiles - 1 - it;
            if (it + 1 < n_tiles) load_tile(tile - 1, nxt);
            const int k0 = tile * F8_BC;
            if (qw < Nq && (!CAUSAL || k0 <= qmax_w + off)) tile_step(cur, cur + TILE, tile, std::true_type{});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ++it;
        };
        auto clean_step = [&](unsigned char* cur, unsigned char* nxt) {
            const int tile = n_tiles - 1 - it;
            if (it + 1 < n_tiles) load_tile(tile - 1, nxt);
            tile_step(cur, cur + TILE, tile, std::false_type{});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ++it;
        };
    #pragma clang loop unroll(disable)
        while (it < n_masked) {
            masked_step(stage0, stage1);
            if (it < n_masked) masked_step(stage1, stage0);
        }
        if ((it & 1) && it < n_tiles) clean_step(stage1, stage0);
    #pragma clang loop unroll(disable)
        while (it < n_tiles) {
            clean_step(stage0, stage1);
            if (it < n_tiles) clean_step(stage1, stage0);
        }

        // epilogue: O = vd * O_acc / l (bf16); LSE = (M + log2 l - LIFT) ln 2
        const float lt = sum_halves(lsum);
        const float inv = (lt == 0.f || lt != lt) ? 1.f : a.vd[bkv] / lt;
        const float lse_v = (lt == 0.f) ? -INFINITY : (Mu + log2f(lt) - F8_LIFT) * kLn2;
        if (qi < Nq) {
            uint16_t* op = a.o + ((size_t)bh * Nq + qi) * F8_D;
    #pragma unroll
            for (int db = 0; db < ND; ++db)
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2 v2 = {pack2<true>(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                                      pack2<true>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                    *(u32x2*)(op + 32 * db + 8 * g + 4 * h) = v2;
                }
            if (h == 0) a.lse[(size_t)bh * Nq + qi] = lse_v;
        }
    };
    if constexpr (CAUSAL) {
        // the two items run through one copy of the item code (a single query tile
        // is the pair t = 0)
        const int npairs = (a.n_qtiles + 1) >> 1;
        const int t = L % npairs, bh = L / npairs;
    #pragma clang loop unroll(disable)
        for (int r = 0; r < 2; ++r) {
            if (r == 1) {
                if (t == a.n_qtiles - 1 - t) break;
                __syncthreads();        // the next item refills stage0
            }
            run_item(r == 0 ? a.n_qtiles - 1 - t : t, bh);
        }
    } else {
        run_item(a.n_qtiles - 1 - (L % a.n_qtiles), (L / a.n_qtiles) % a.BH);
    }
}

// Block quantizer: x [G, N, d] (16-bit) -> codes [G, N, d] (e4m3) and descale
// [G, nb], one workgroup per (g, block of `rows` rows).  Per block: amax = max
// |x|; descale = amax / 448 (1 for an all-zero block); code = nearest e4m3 of
// x * (448 / amax), clamped to +-448 first (ties to even).
template <bool BF16>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                                        float* __restrict__ dsc, int N, int d, int rows, int nb) {
    __shared__ float s_max[4];
    const int g = blockIdx.x / nb, b = blockIdx.x % nb;
    const int r0 = b * rows, r1 = min(N, r0 + rows);
    const size_t base = ((size_t)g * N + r0) * d;
    const int64_t n = (int64_t)(r1 - r0) * d;     // a multiple of 8
    const int tid = threadIdx.x;
    float am = 0.f;
    for (int64_t e = (int64_t)tid * 8; e < n; e += 256 * 8) {
        const u32x4 v = *(const u32x4*)(x + base + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            am = fmaxf(am, fabsf(widen<BF16>((uint16_t)(v[i] & 0xffff))));
            am = fmaxf(am, fabsf(widen<BF16>((uint16_t)(v[i] >> 16))));
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) am = fmaxf(am, __shfl_xor(am, m));
    if ((tid & 63) == 0) s_max[tid >> 6] = am;
    __syncthreads();
    am = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float scl = am > 0.f ? 448.0f / am : 0.f;
    for (int64_t e = (int64_t)tid * 8; e < n; e += 256 * 8) {
        const u32x4 v = *(const u32x4*)(x + base + e);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = fminf(fmaxf(widen<BF16>((uint16_t)(v[i] & 0xffff)) * scl, -448.0f), 448.0f);
            f[2 * i + 1] = fminf(fmaxf(widen<BF16>((uint16_t)(v[i] >> 16)) * scl, -448.0f), 448.0f);
        }
        const u32x2 out = {(u32)pack4_f8(f[0], f[1], f[2], f[3]), (u32)pack4_f8(f[4], f[5], f[6], f[7])};
        *(u32x2*)(x8 + base + e) = out;
    }
    if (tid == 0) dsc[(size_t)g * nb + b] = am > 0.f ? am / 448.0f : 1.0f;
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream) {
    F8Args a;
    a.q = (const uint8_t*)p.q;
    a.k = (const uint8_t*)p.k;
    a.v = (const uint8_t*)p.v;
    a.qd = p.q_descale;
    a.kd = p.k_descale;
    a.vd = p.v_descale;
    a.o = (uint16_t*)p.o;
    a.lse = p.lse;
    a.B = p.B;
    a.H = p.H;
    a.H_kv = p.H_kv;
    a.group = p.H / p.H_kv;
    a.Nq = p.Nq;
    a.Nk = p.Nk;
    a.BH = p.B * p.H;
    // 8 wavefronts (256 query rows per workgroup) where they beat 4 (wide_rows)
    const bool wide = wide_rows(wide_blocks(p.Nq, (int64_t)p.B * p.H, p.causal), p.Nk, 2048);
    const int br = wide ? 256 : 128;
    a.n_qtiles = (p.Nq + br - 1) / br;
    a.n_qblk = (p.Nq + F8_QB - 1) / F8_QB;
    a.n_kblk = (p.Nk + F8_BC - 1) / F8_BC;
    a.c = fabsf(p.scale) * kLog2e;
    a.qsign = p.scale < 0.f ? 0x80808080u : 0u;
    const int64_t blocks = p.causal ? (int64_t)((a.n_qtiles + 1) / 2) * a.BH : (int64_t)a.n_qtiles * a.BH;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (p.causal) {
        if (wide) hipLaunchKernelGGL((fwd_fp8_kernel<true, 8>), dim3((int)blocks), dim3(512), 0, stream, a);
        else hipLaunchKernelGGL((fwd_fp8_kernel<true, 4>), dim3((int)blocks), dim3(256), 0, stream, a);
    } else {
        if (wide) hipLaunchKernelGGL((fwd_fp8_kernel<false, 8>), dim3((int)blocks), dim3(512), 0, stream, a);
        else hipLaunchKernelGGL((fwd_fp8_kernel<false, 4>), dim3((int)blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* x, void* x8, float* descale, int64_t G, int N, int d, int rows,
                            bool bf16, hipStream_t stream) {
    const int nb = (N + rows - 1) / rows;
    const int64_t blocks = G * nb;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL((quant_fp8_kernel<true>), dim3((int)blocks), dim3(256), 0, stream, (const uint16_t*)x,
                           (uint8_t*)x8, descale, N, d, rows, nb);
    else
        hipLaunchKernelGGL((quant_fp8_kernel<false>), dim3((int)blocks), dim3(256), 0, stream, (const uint16_t*)x,
                           (uint8_t*)x8, descale, N, d, rows, nb);
    return hipGetLastError();
}

}  // namespace fa
