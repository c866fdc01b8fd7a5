// fa_decode.hip -- split-KV partials for a single query row per head (decode).
//
// With seqlen_q = 1 a grid over query tiles has only B*H workgroups, so the keys
// are split into num_splits chunks that run in parallel, each producing a
// normalised partial (O, LSE) that a combine kernel merges (LLM Infra Atlas
// "FA2: parallelism", section 2; Ringi "Lecture 25", section 0.3).
//
// gfx950 design (not from the pages): the work is ~1 FLOP per byte, so this is
// a streaming kernel, not a matrix one.  One workgroup (4 wavefronts) owns one
// (b, h, split).  A key row of D 16-bit values is spread over D/8 lanes, 16
// bytes each, so every load instruction of a wavefront reads 1 KiB of
// consecutive memory (4 rows at d = 128, 8 at d = 64).  The dot product is
// finished with DPP row operations (the products as fp32 dot products of 16-bit
// pairs), every lane of the row keeps the online
// softmax state of its row, and each lane accumulates its own 8 output values.
// Eight groups of keys are loaded per step so that enough bytes are in flight
// to cover HBM latency.  At the end the 16 (d = 128) or 32 (d = 64) partial
// states of the workgroup merge through LDS with the online-softmax identity
// (Ringi, Lecture 25, section 2.2).
//
// Grouped K/V heads (KingOfEgg, "Flash Attention (4)", section 5): the GP query
// heads of one workgroup read the same K/V head, so the workgroup streams that
// head's chunk once and scores every loaded key row against all GP queries;
// decode bytes per query head fall by GP.
//
// Paged K/V cache (the pages pose it: a cache scattered over fixed-size pages
// and how the load addressing changes; Ringi, "Lecture 25", section 8.3,
// question on PagedAttention): keys live in pages of page_size rows
// [num_pages, page_size, H_kv, d]; sequence b's logical page j sits in the
// physical page block_table[b][j].  A key row stays 256 contiguous bytes (d =
// 128), so every wavefront load still reads whole rows.  Each sequence has its
// own length and is split into num_splits equal chunks.  With 2 or 4 query heads
// per K/V head and H_kv a multiple of 4, decode_paged_hg_kernel reads one key of
// four adjacent K/V heads per wave load (their rows are contiguous in a page)
// with one scalar page lookup per key; otherwise decode_kernel looks pages up
// per wave load (scalar) or per lane.
//
// At d = 128 with 4 query heads per workgroup, contiguous and packed keys use
// eight wavefronts per workgroup, which stream one split twice as fast.
//
// Packed sequences (the varlen interface with cumulative offsets instead of
// padding, Ringi, "Lecture 25", section 7; split-KV for decode, LLM Infra Atlas,
// section 2): sequence b's keys are rows [cu_k[b], cu_k[b+1]) of k, v [total_k,
// H_kv, d], so a key row of one head is again 256 contiguous bytes (d = 128),
// H_kv * d elements after the previous one; each sequence is split into
// num_splits chunks of its own length, as in the paged mode.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

struct DecArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* o_part;
    float* lse_part;
    int BH, Nk, S;
    int split_chunk;
    float c;   // scale * log2(e), sign included
    int H, H_kv, group;   // query heads, K/V heads, query heads per K/V head
    // paged K/V cache
    const int* block_table;   // [B, max_pages]
    const int* seqlens;       // [B]
    int page_shift;           // log2(page_size)
    int max_pages, num_pages;
    // packed sequences: key offsets [B + 1], total rows of k and v, longest sequence
    const int* cu_k;
    int total_k, max_k;
};

// Where the keys of a decode come from.
enum KvLayout { KV_DENSE = 0, KV_PAGED = 1, KV_PACKED = 2 };

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the CH lanes that hold one key row (CH = 16 or 8, aligned groups).
template <int CH>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_mov<0xB1>(x);          // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);          // quad_perm [2,3,0,1]
    if constexpr (CH == 16) {
        x += dpp_mov<0x124>(x);     // row_ror:4
        x += dpp_mov<0x128>(x);     // row_ror:8
    } else {
        x += dpp_mov<0x141>(x);     // row_half_mirror
    }
    return x;
}

template <bool BF16>
__device__ __forceinline__ void widen8(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = widen<BF16>((uint16_t)(x[i] & 0xffff));
        f[2 * i + 1] = widen<BF16>((uint16_t)(x[i] >> 16));
    }
}

// a.x * b.x + a.y * b.y + acc over two packed 16-bit values, in fp32.
template <bool BF16>
__device__ __forceinline__ float dot2(u32 a, u32 b, float acc) {
    if constexpr (BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

// One step of a decode wave: the scores of U key rows (this lane's 8 values of
// each in kr) against GP queries (qp), the online-softmax update of the GP
// states M, l, acc, and P V accumulation with the U value rows (vr).  A key that
// does not exist (ok false) scores -inf; its K and V values are zeros.  CH lanes
// hold one key row.
template <bool BF16, int CH, int GP, int U>
__device__ __forceinline__ void decode_step(const u32x4 (&qp)[GP], const u32x4* kr, const u32x4* vr, const bool* ok,
                                            float c, float (&M)[GP], float (&l)[GP], float (&acc)[GP][8]) {
    float s[GP][U];
    float mx[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) mx[g] = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) part = dot2<BF16>(qp[g][i], kr[u][i], part);
            s[g][u] = row_sum<CH>(part) * c;
            if (!ok[u]) s[g][u] = -INFINITY;
            mx[g] = fmaxf(mx[g], s[g][u]);
        }
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float Mn = fmaxf(M[g], mx[g]);
        const float alpha = (Mn == -INFINITY) ? 1.f : exp2_fast(M[g] - Mn);
        M[g] = Mn;
        l[g] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float vf[8];
        widen8<BF16>(vr[u], vf);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float p = exp2_fast(s[g][u] - ((M[g] == -INFINITY) ? 0.f : M[g]));
            l[g] += p;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[g][i] = __builtin_fmaf(p, vf[i], acc[g][i]);
        }
    }
}

// GP: query heads per workgroup (a divisor of the group size).  KV: dense
// [B, H_kv, Nk, d] keys, the paged caches, or packed sequences.  NWV wavefronts
// share a (sequence, query heads, split); wave w takes the key groups w, w + NWV,
// ... of the split.
template <bool BF16, int D, int GP, int KV, int NWV = 4>
__global__ __launch_bounds__(64 * NWV) void decode_kernel(DecArgs a) {
    constexpr bool PAGED = KV == KV_PAGED;
    constexpr int CH = D / 8;          // lanes per key row
    constexpr int KPI = 64 / CH;       // key rows per wavefront load
    constexpr int U = GP >= 4 ? 4 : 8; // key groups in flight per step
    constexpr int NP = NWV * KPI;      // partial states per workgroup and query head
    __shared__ float s_m[GP][NP], s_l[GP][NP];
    __shared__ __attribute__((aligned(16))) float s_o[GP][NP * D];

    const int split = blockIdx.x % a.S;
    const int bh0 = (blockIdx.x / a.S) * GP;          // first of GP consecutive query heads
    const int bkv = (bh0 / a.H) * a.H_kv + (bh0 % a.H) / a.group;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane % CH, r = lane / CH;

    int ks, ke;
    const uint16_t* kg;
    const uint16_t* vg;
    const int* bt = nullptr;   // this sequence's row of the block table
    int hk = 0;
    if constexpr (PAGED) {
        const int b = bh0 / a.H;
        hk = (bh0 % a.H) / a.group;
        const int len = a.seqlens[b];
        // a length outside [0, max_pages * page_size] leaves the rows unwritten
        if (len < 0 || len > (a.max_pages << a.page_shift)) return;
        const int chunk = (len + a.S - 1) / a.S;
        ks = min(len, split * chunk);
        ke = min(len, ks + chunk);
        kg = a.k;
        vg = a.v;
        bt = a.block_table + (size_t)b * a.max_pages;
    } else if constexpr (KV == KV_PACKED) {
        const int b = bh0 / a.H;
        hk = (bh0 % a.H) / a.group;
        // offsets outside [0, total_k], decreasing or longer than the declared
        // maximum leave the sequence's rows unwritten
        const int k_lo = a.cu_k[b], k_hi = a.cu_k[b + 1];
        if (k_lo < 0 || k_hi < k_lo || k_hi > a.total_k || k_hi - k_lo > a.max_k) return;
        const int len = k_hi - k_lo;
        const int chunk = (len + a.S - 1) / a.S;
        ks = min(len, split * chunk);
        ke = min(len, ks + chunk);
        kg = a.k + ((size_t)k_lo * a.H_kv + hk) * D;
        vg = a.v + ((size_t)k_lo * a.H_kv + hk) * D;
    } else {
        ks = min(a.Nk, split * a.split_chunk);
        ke = min(a.Nk, ks + a.split_chunk);
        kg = a.k + (size_t)bkv * a.Nk * D;
        vg = a.v + (size_t)bkv * a.Nk * D;
    }
    const int ngroups = (ke - ks + KPI - 1) / KPI;
    // physical page of a key of this split (-1 past the split's end); only keys
    // below the sequence length index the block table
    auto page_of = [&](int key) -> int { return key < ke ? bt[key >> a.page_shift] : -1; };

    // this lane's 8 query values per head, kept packed: the score is c times a
    // dot product of 16-bit pairs accumulated in fp32 (v_dot2_f32_{f16,bf16};
    // the products are exact in fp32)
    u32x4 qp[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) qp[g] = *(const u32x4*)(a.q + (size_t)(bh0 + g) * D + 8 * c);

    float M[GP], l[GP], acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        M[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
    }

    auto consume = [&](const u32x4* kr, const u32x4* vr, const bool* ok) {
        decode_step<BF16, CH, GP, U>(qp, kr, vr, ok, a.c, M, l, acc);
    };

    // Paged keys whose groups never straddle a page (the split starts at a
    // multiple of KPI and a page holds a multiple of KPI rows): the KPI keys of a
    // wave load share one page, so its entry is one scalar load and its row base
    // scalar arithmetic, and the rows come through a buffer resource that ends
    // with the group's last key before the split's end (no records for an
    // invalid page), so a lane's offset is a constant and absent rows read as
    // zeros.  This takes the per-lane page lookup and 64-bit row arithmetic out
    // of the vector work (decode_paged 219.8 -> 214.4 us, same partials).  With
    // one query head per workgroup the extra registers would cost a wavefront
    // per SIMD, so that case keeps the per-lane path.
    const int pmask = (1 << a.page_shift) - 1;
    if (PAGED && GP >= 2 && (ks % KPI) == 0 && ((pmask + 1) % KPI) == 0) {
        const int wu = __builtin_amdgcn_readfirstlane(w);
        const int ksu = __builtin_amdgcn_readfirstlane(ks), keu = __builtin_amdgcn_readfirstlane(ke);
        const u32 lo = (u32)((r * a.H_kv * D + 8 * c) * 2);
        for (int g0 = wu; g0 < ngroups; g0 += NWV * U) {
            u32x4 kr[U], vr[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kf = ksu + (g0 + NWV * u) * KPI;              // the group's first key
                const int pg = kf < keu ? __builtin_amdgcn_readfirstlane(bt[kf >> a.page_shift]) : -1;
                const bool pok = (unsigned)pg < (unsigned)a.num_pages;
                const int nrows = pok ? min(KPI, keu - kf) : 0;
                ok[u] = pok && kf + r < keu;
                const size_t rowb = (((size_t)(pok ? pg : 0) << a.page_shift) + (kf & pmask)) * a.H_kv + hk;
                const u32 nrec = nrows > 0 ? (u32)(((nrows - 1) * a.H_kv * D + D) * 2) : 0u;
                const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kg + rowb * D, nrec);
                const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vg + rowb * D, nrec);
                kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)lo, 0, 0));
                vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lo, 0, 0));
            }
            consume(kr, vr, ok);
        }
    } else {
        // page entries of the first step (paged)
        int pnext[U];
#pragma unroll
        for (int u = 0; u < U; ++u) pnext[u] = PAGED ? page_of(ks + (w + NWV * u) * KPI + r) : 0;

        for (int g0 = w; g0 < ngroups; g0 += NWV * U) {
            u32x4 kr[U], vr[U];
            int key[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                key[u] = ks + (g0 + NWV * u) * KPI + r;
                size_t row;
                if constexpr (PAGED) {
                    // a page entry outside [0, num_pages) drops its keys
                    const int pg = pnext[u];
                    ok[u] = key[u] < ke && (unsigned)pg < (unsigned)a.num_pages;
                    row = (((size_t)pg << a.page_shift) + (key[u] & pmask)) * a.H_kv + hk;
                } else {
                    ok[u] = key[u] < ke;
                    row = KV == KV_PACKED ? (size_t)key[u] * a.H_kv : (size_t)key[u];
                }
                if (ok[u]) {
                    kr[u] = *(const u32x4*)(kg + row * D + 8 * c);
                    vr[u] = *(const u32x4*)(vg + row * D + 8 * c);
                } else {
                    kr[u] = u32x4{0, 0, 0, 0};
                    vr[u] = u32x4{0, 0, 0, 0};
                }
            }
            if constexpr (PAGED) {
#pragma unroll
                for (int u = 0; u < U; ++u) pnext[u] = page_of(key[u] + NWV * U * KPI);   // next step's keys
            }
            consume(kr, vr, ok);
        }
    }

    // merge the workgroup's partial states, per query head
    const int pidx = w * KPI + r;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        if (c == 0) {
            s_m[g][pidx] = M[g];
            s_l[g][pidx] = l[g];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s_o[g][pidx * D + 8 * c + i] = acc[g][i];
    }
    __syncthreads();
    for (int t = tid; t < GP * D; t += 64 * NWV) {
        const int g = t / D, col = t % D;
        float Ms = -INFINITY;
        for (int i = 0; i < NP; ++i) Ms = fmaxf(Ms, s_m[g][i]);
        float den = 0.f, num = 0.f;
        for (int i = 0; i < NP; ++i) {
            const float wgt = (s_m[g][i] == -INFINITY) ? 0.f : exp2_fast(s_m[g][i] - Ms);
            den = __builtin_fmaf(wgt, s_l[g][i], den);
            num = __builtin_fmaf(wgt, s_o[g][i * D + col], num);
        }
        const size_t row = (size_t)split * a.BH + bh0 + g;
        a.o_part[row * D + col] = den > 0.f ? num / den : 0.f;
        if (col == 0) a.lse_part[row] = den > 0.f ? (Ms + log2f(den)) * kLn2 : -INFINITY;
    }
}

// Paged decode with the K/V heads of one key spread over a wave load.  In the
// cache [num_pages, page_size, H_kv, d] the rows of HG adjacent K/V heads of one
// key are HG * 256 contiguous bytes (d = 128), where one head's consecutive keys
// lie H_kv * 256 bytes apart.  A workgroup of 16 wavefronts takes HG = 4 K/V
// heads (and all their query heads, GP = H / H_kv of each) of one (sequence,
// split); a wave load reads one key for all four heads, lane row r holding head
// hk0 + r, so every load instruction covers 1 KiB of consecutive memory.  The
// key's page entry is one scalar load, its row base scalar arithmetic, and the
// rows come through a buffer resource with no records for an invalid page.  Wave
// w takes keys w, w + 16, ... of the split, so its partial state covers the keys
// that partial w of decode_kernel covers, in the same order: the partials are
// decode_kernel's bit for bit.  The 16 partial states per (head, query) merge
// through LDS as there.
template <bool BF16, int GP>
__global__ __launch_bounds__(1024) void decode_paged_hg_kernel(DecArgs a) {
    constexpr int D = 128, CH = 16, HG = 4, NWV = 16, U = 4;
    __shared__ float s_m[HG][GP][NWV], s_l[HG][GP][NWV];
    __shared__ __attribute__((aligned(16))) float s_o[HG][GP][NWV * D];

    const int split = blockIdx.x % a.S;
    const int rest = blockIdx.x / a.S;
    const int nhg = a.H_kv / HG;
    const int b = rest / nhg, hk0 = (rest - b * nhg) * HG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane % CH, r = lane / CH;
    const int len = a.seqlens[b];
    // a length outside [0, max_pages * page_size] leaves the rows unwritten
    if (len < 0 || len > (a.max_pages << a.page_shift)) return;
    const int chunk = (len + a.S - 1) / a.S;
    const int ks = __builtin_amdgcn_readfirstlane(min(len, split * chunk));
    const int ke = __builtin_amdgcn_readfirstlane(min(len, ks + chunk));
    const int* bt = a.block_table + (size_t)b * a.max_pages;
    const int pmask = (1 << a.page_shift) - 1;
    const int qh0 = b * a.H + (hk0 + r) * a.group;    // first query head of this lane's K/V head

    u32x4 qp[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) qp[g] = *(const u32x4*)(a.q + (size_t)(qh0 + g) * D + 8 * c);
    float M[GP], l[GP], acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        M[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
    }

    const u32 lo = (u32)((r * D + 8 * c) * 2);
    for (int k0 = ks + w; k0 < ke; k0 += NWV * U) {
        u32x4 kr[U], vr[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = k0 + NWV * u;
            // a page entry outside [0, num_pages) drops its key
            const int pg = key < ke ? __builtin_amdgcn_readfirstlane(bt[key >> a.page_shift]) : -1;
            ok[u] = (unsigned)pg < (unsigned)a.num_pages;
            const size_t rowb = (((size_t)(ok[u] ? pg : 0) << a.page_shift) + (key & pmask)) * a.H_kv + hk0;
            const u32 nrec = ok[u] ? (u32)(HG * D * 2) : 0u;
            const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(a.k + rowb * D, nrec);
            const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(a.v + rowb * D, nrec);
            kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)lo, 0, 0));
            vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lo, 0, 0));
        }
        decode_step<BF16, CH, GP, U>(qp, kr, vr, ok, a.c, M, l, acc);
    }

#pragma unroll
    for (int g = 0; g < GP; ++g) {
        if (c == 0) {
            s_m[r][g][w] = M[g];
            s_l[r][g][w] = l[g];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s_o[r][g][w * D + 8 * c + i] = acc[g][i];
    }
    __syncthreads();
    for (int t = tid; t < HG * GP * D; t += NWV * 64) {
        const int hh = t / (GP * D), g = (t / D) % GP, col = t % D;
        float Ms = -INFINITY;
        for (int i = 0; i < NWV; ++i) Ms = fmaxf(Ms, s_m[hh][g][i]);
        float den = 0.f, num = 0.f;
        for (int i = 0; i < NWV; ++i) {
            const float wgt = (s_m[hh][g][i] == -INFINITY) ? 0.f : exp2_fast(s_m[hh][g][i] - Ms);
            den = __builtin_fmaf(wgt, s_l[hh][g][i], den);
            num = __builtin_fmaf(wgt, s_o[hh][g][i * D + col], num);
        }
        const size_t row = (size_t)split * a.BH + b * a.H + (hk0 + hh) * a.group + g;
        a.o_part[row * D + col] = den > 0.f ? num / den : 0.f;
        if (col == 0) a.lse_part[row] = den > 0.f ? (Ms + log2f(den)) * kLn2 : -INFINITY;
    }
}

// Max / sum over the 64 lanes of a wavefront (xor butterfly; every lane ends
// with the result, combined in the same fixed order on every run).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// One wavefront per output row.  Lane l reads the LSE of split l (64 splits per
// pass), and the first 16 partial rows are requested in the same round of loads,
// before the row maximum is known, so a decode with up to 16 splits waits for
// memory once; the weighted rows are then summed in split order (16 rows' loads
// in flight per later round).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ op, const float* __restrict__ lp,
                                                      uint16_t* __restrict__ o, float* __restrict__ lse,
                                                      int64_t R, int S) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= R) return;
    constexpr int nd = D / 64;   // values per lane (1 or 2)
    constexpr int SB = 16;       // partial rows per round of loads
    auto load_rows = [&](float (&x)[SB][nd], int j0, int ns) {
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int j = min(j0 + u, ns - 1);     // in bounds; rows past ns get weight 0
            const float* src = op + ((size_t)j * R + row) * D;
#pragma unroll
            for (int c = 0; c < nd; ++c) x[u][c] = src[lane + 64 * c];
        }
    };
    const float ls_first = lane < S ? lp[(size_t)lane * R + row] : -INFINITY;
    float x[SB][nd];
    load_rows(x, 0, S);
    float M = ls_first;
    for (int s0 = 64; s0 < S; s0 += 64)
        if (s0 + lane < S) M = fmaxf(M, lp[(size_t)(s0 + lane) * R + row]);
    M = wave_max(M);
    float num[2] = {0.f, 0.f};
    float den = 0.f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < S; s0 += 64) {
            const float ls = s0 == 0 ? ls_first : ((s0 + lane < S) ? lp[(size_t)(s0 + lane) * R + row] : -INFINITY);
            const float wl = (ls == -INFINITY) ? 0.f : exp2_fast((ls - M) * kLog2e);
            den += wl;
            const int ns = min(64, S - s0);
            for (int j0 = 0; j0 < ns; j0 += SB) {
                if (s0 + j0 > 0) load_rows(x, s0 + j0, s0 + ns);
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const float wj = (j0 + u < ns) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0 + u))
                                                   : 0.f;
#pragma unroll
                    for (int c = 0; c < nd; ++c)   // empty splits add nothing
                        num[c] = (wj != 0.f) ? __builtin_fmaf(wj, x[u][c], num[c]) : num[c];
                }
            }
        }
        den = wave_sum(den);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int j = 0; j < nd; ++j) {
        const float x = num[j] * inv;
        uint16_t bits;
        if constexpr (BF16)
            bits = __builtin_bit_cast(uint16_t, (__bf16)x);
        else
            bits = __builtin_bit_cast(uint16_t, (_Float16)x);
        o[row * D + lane + 64 * j] = bits;
    }
    if (lane == 0) lse[row] = den > 0.f ? M + logf(den) : -INFINITY;
}

template <bool BF16, int D, int KV>
hipError_t launch_dec(const DecArgs& a, int gp, int blocks, hipStream_t stream) {
    switch (gp) {
        case 8: hipLaunchKernelGGL((decode_kernel<BF16, D, 8, KV>), dim3(blocks), dim3(256), 0, stream, a); break;
        case 4:
            // d = 128: eight wavefronts per (sequence, 4 query heads, split), as the
            // packed layout takes (the two then give the same partials bit for bit)
            if constexpr (D == 128 && KV == KV_DENSE) {
                hipLaunchKernelGGL((decode_kernel<BF16, D, 4, KV, 8>), dim3(blocks), dim3(512), 0, stream, a);
                break;
            }
            hipLaunchKernelGGL((decode_kernel<BF16, D, 4, KV>), dim3(blocks), dim3(256), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<BF16, D, 2, KV>), dim3(blocks), dim3(256), 0, stream, a); break;
        default: hipLaunchKernelGGL((decode_kernel<BF16, D, 1, KV>), dim3(blocks), dim3(256), 0, stream, a); break;
    }
    return hipGetLastError();
}

template <int KV>
hipError_t launch_dec_d(const DecArgs& a, int d, bool bf16, int gp, int blocks, hipStream_t stream) {
    if (d == 128) return bf16 ? launch_dec<true, 128, KV>(a, gp, blocks, stream)
                              : launch_dec<false, 128, KV>(a, gp, blocks, stream);
    return bf16 ? launch_dec<true, 64, KV>(a, gp, blocks, stream) : launch_dec<false, 64, KV>(a, gp, blocks, stream);
}

hipError_t launch_paged_hg(const DecArgs& a, bool bf16, int blocks, hipStream_t stream) {
    if (a.group == 4) {
        if (bf16) hipLaunchKernelGGL((decode_paged_hg_kernel<true, 4>), dim3(blocks), dim3(1024), 0, stream, a);
        else hipLaunchKernelGGL((decode_paged_hg_kernel<false, 4>), dim3(blocks), dim3(1024), 0, stream, a);
    } else {
        if (bf16) hipLaunchKernelGGL((decode_paged_hg_kernel<true, 2>), dim3(blocks), dim3(1024), 0, stream, a);
        else hipLaunchKernelGGL((decode_paged_hg_kernel<false, 2>), dim3(blocks), dim3(1024), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FwdParams& p, hipStream_t stream) {
    DecArgs a;
    a.q = (const uint16_t*)p.q;
    a.k = (const uint16_t*)p.k;
    a.v = (const uint16_t*)p.v;
    a.o_part = (float*)p.o;
    a.lse_part = p.lse;
    a.BH = p.B * p.H;
    a.Nk = p.Nk;
    a.S = p.num_splits;
    a.split_chunk = split_chunk(p.Nk, p.num_splits);
    a.c = p.scale * kLog2e;
    a.H = p.H;
    a.H_kv = p.H_kv > 0 ? p.H_kv : p.H;
    a.group = p.H / a.H_kv;
    // query heads per workgroup: the largest of 8, 4, 2, 1 dividing the group
    const int gp = a.group % 8 == 0 ? 8 : a.group % 4 == 0 ? 4 : a.group % 2 == 0 ? 2 : 1;
    const int64_t blocks = (int64_t)a.BH / gp * a.S;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    a.block_table = p.block_table;
    a.seqlens = p.seqlens_k;
    a.max_pages = p.max_pages;
    a.num_pages = p.num_pages;
    a.page_shift = 0;
    while ((1 << a.page_shift) < p.page_size) ++a.page_shift;
    a.cu_k = p.cu_k;
    a.total_k = p.total_k;
    a.max_k = p.Nk;
    // a paged cache with d = 128, H_kv a multiple of 4 and 2 or 4 query heads per
    // K/V head: four K/V heads per workgroup, one key of all four per wave load
    // (decode_paged 213.5 -> 197.4 us, same partials).  Packed keys have the same
    // layout but gain nothing: their time is set by the longest sequences, which
    // workgroups four times larger balance worse (122.5 -> 124.3 us).
    if (p.block_table && p.d == 128 && a.H_kv % 4 == 0 && (a.group == 2 || a.group == 4)) {
        const int64_t hb = (int64_t)p.B * (a.H_kv / 4) * a.S;
        if (hb <= 0 || hb > 0x7fffffff) return hipErrorInvalidValue;
        return launch_paged_hg(a, p.bf16, (int)hb, stream);
    }
    if (p.block_table) return launch_dec_d<KV_PAGED>(a, p.d, p.bf16, gp, (int)blocks, stream);
    if (p.varlen) {
        // packed sequences differ in length and the longest splits set the time:
        // eight wavefronts per workgroup stream a split twice as fast (decode_varlen
        // 124.5 -> 118.5 us, sixteen measured 134 us; the dense grouped decode takes
        // eight too, 192.7 -> 188.7 us)
        if (p.d == 128 && gp == 4) {
            if (p.bf16) hipLaunchKernelGGL((decode_kernel<true, 128, 4, KV_PACKED, 8>), dim3((int)blocks), dim3(512), 0, stream, a);
            else hipLaunchKernelGGL((decode_kernel<false, 128, 4, KV_PACKED, 8>), dim3((int)blocks), dim3(512), 0, stream, a);
            return hipGetLastError();
        }
        return launch_dec_d<KV_PACKED>(a, p.d, p.bf16, gp, (int)blocks, stream);
    }
    return launch_dec_d<KV_DENSE>(a, p.d, p.bf16, gp, (int)blocks, stream);
}

hipError_t launch_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                          int64_t rows, int d, int num_splits, bool bf16, hipStream_t stream) {
    const int64_t blocks = (rows + 3) / 4;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    uint16_t* ob = (uint16_t*)o;
    if (d == 128) {
        if (bf16) hipLaunchKernelGGL((combine_kernel<true, 128>), dim3((int)blocks), dim3(256), 0, stream, o_part,
                                     lse_part, ob, lse, rows, num_splits);
        else hipLaunchKernelGGL((combine_kernel<false, 128>), dim3((int)blocks), dim3(256), 0, stream, o_part,
                                lse_part, ob, lse, rows, num_splits);
    } else {
        if (bf16) hipLaunchKernelGGL((combine_kernel<true, 64>), dim3((int)blocks), dim3(256), 0, stream, o_part,
                                     lse_part, ob, lse, rows, num_splits);
        else hipLaunchKernelGGL((combine_kernel<false, 64>), dim3((int)blocks), dim3(256), 0, stream, o_part,
                                lse_part, ob, lse, rows, num_splits);
    }
    return hipGetLastError();
}

}  // namespace fa
