// fa_bwd.hip -- FlashAttention-2 backward on gfx950 MFMA: dQ, dK, dV from Q, K,
// V, O, dO and the forward's LSE.
//
// Method (the pages this follows):
//   * Recompute instead of storing P: each tile re-forms S = scale * Q K^T and
//     P = exp(S - LSE) from the saved log-sum-exp (Ringi, "Lecture 25", section
//     3.3; AIInfraGuide 6.2, forward pseudocode: the saved statistic is
//     L = m + log l).
//   * Gradients: dV = P^T dO, dP = dO V^T, dS = P o (dP - D) with
//     D = rowsum(dP o P) = rowsum(dO o O), dQ = scale dS K, dK = scale dS^T Q
//     (Ringi, section 3.3; the scale enters through S).
//   * Parallelism: dK and dV of a key block collect every query that sees it, so
//     a workgroup fixes a key block and walks the query tiles; dQ of a query
//     block collects every key block, which the pages do with atomics or a
//     deterministic scheme (LLM Infra Atlas, "FA2: parallelism", section 5).
//     Here a second kernel fixes a query block and walks the key tiles, so no
//     atomics are used and the result is deterministic.
//
// gfx950 mapping (not from the pages):
//   * dQ kernel (the forward's layout): S^T = K Q^T and dP^T = V dO^T on
//     v_mfma_f32_32x32x16 with Q and dO held in registers; K and V rows enter in
//     the order with bits 2 and 3 swapped, so registers 8p..8p+7 of the
//     accumulators are the 8 consecutive keys a lane supplies as the B operand
//     of dQ^T += K^T dS^T, with K^T read through ds_read_b64_tr_b16.  One lane
//     owns one query row: LSE and D are per-lane scalars.
//   * dK/dV kernel (its transpose): each wave owns 32 keys held in registers;
//     S = Q K^T and dP = dO V^T with Q and dO rows in the swapped order, so P and
//     dS feed dV^T += dO^T P and dK^T += Q^T dS directly.  LSE (in base 2) and
//     D of the tile's query rows sit in LDS next to the Q and dO tiles.  At one
//     wave per SIMD no other wave hides a wave's LDS latency, so the instruction
//     order is fixed by scheduling fences (which order memory operations) and
//     empty asm statements on the products' accumulators (which keep the pure
//     arithmetic between them): operand reads (above all the transposed ones)
//     run 8 to 16 reads ahead of their products, the first block's element-wise
//     work runs beside the second block's scores, and the second block's beside
//     the first block's gradient products.
//   * Rows past the end of Q read as zeros (so they add nothing to dK, dV), and
//     keys past the end of K only reach their own, unstored, dK/dV columns; the
//     dK/dV kernel therefore only applies the causal condition, as a select per
//     score in the tiles that cross a wave's diagonal.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int BQ = 128;   // dQ kernel: query rows per workgroup of 4 waves (32 each)
constexpr int BK = 64;    // dQ kernel: keys per tile
constexpr int CK = 128;   // dK/dV kernel: keys per workgroup (4 waves x 32)
constexpr int CQ = 64;    // dK/dV kernel: query rows per tile

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    float* delta;        // D = rowsum(dO o O), laid out as lse
    float* lse2;         // LSE * log2(e), laid out as lse
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int BH, Nq, Nk;
    int H, H_kv, group;  // query heads, K/V heads, query heads per K/V head
    float c;             // scale * log2(e), sign included
    float scale;
    int n_qtiles;        // dQ kernel work items per head
    int n_ktiles;        // dK/dV kernel work items per head
    // packed sequences: q, o, dout, dq [total_q, H, d], k, v, dk, dv [total_k,
    // H_kv, d], lse [H, total_q]; sequence b owns rows cu_q[b]..cu_q[b+1] and
    // cu_k[b]..cu_k[b+1]; Nq and Nk are then the longest sequence's lengths
    const int* cu_q;
    const int* cu_k;
    int total_q, total_k;
};

// Rows of one (sequence, query head, K/V head) item: element offsets of its first
// Q / K row and first LSE entry, row strides in elements, the offset steps to the
// next query head (Q rows, LSE entries), and the item's lengths.  ok is false
// for a packed sequence whose offsets fall outside [0, total], decrease or span
// more than the longest length: its item writes nothing.
struct Seq {
    size_t q, k, l, qh, lh;
    int sq, sk, Nq, Nk;
    bool ok;
};

template <int D, bool VARLEN>
__device__ __forceinline__ Seq seq_of(const BwdArgs& a, int bq, int bkv) {
    Seq s;
    if constexpr (VARLEN) {
        const int b = bq / a.H, h = bq - b * a.H, hk = bkv - b * a.H_kv;
        const int qs = a.cu_q[b], q1 = a.cu_q[b + 1], ks = a.cu_k[b], k1 = a.cu_k[b + 1];
        s.ok = 0 <= qs && qs <= q1 && q1 <= a.total_q && q1 - qs <= a.Nq && 0 <= ks && ks <= k1 &&
               k1 <= a.total_k && k1 - ks <= a.Nk;
        s.Nq = s.ok ? q1 - qs : 0;
        s.Nk = s.ok ? k1 - ks : 0;
        s.q = ((size_t)qs * a.H + h) * D;
        s.k = ((size_t)ks * a.H_kv + hk) * D;
        s.l = (size_t)h * a.total_q + qs;
        s.qh = D;
        s.lh = a.total_q;
        s.sq = a.H * D;
        s.sk = a.H_kv * D;
    } else {
        s.ok = true;
        s.Nq = a.Nq;
        s.Nk = a.Nk;
        s.q = (size_t)bq * a.Nq * D;
        s.k = (size_t)bkv * a.Nk * D;
        s.l = (size_t)bq * a.Nq;
        s.qh = (size_t)a.Nq * D;
        s.lh = a.Nq;
        s.sq = D;
        s.sk = D;
    }
    return s;
}

// Row index (within a 32-row block) that accumulator row i stands for: bits 2 and 3 swapped.
__device__ __forceinline__ int perm_row(int i) {
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// D_i = sum_t dO[i,t] O[i,t] in fp32, and LSE_i * log2(e).  A row's D 16-bit
// values are spread over D/8 lanes, 16 bytes each, so every wave load reads whole
// rows of consecutive memory; the lanes' partial sums are added by a fixed xor
// butterfly.  Each wave handles DELTA_U groups of 64/(D/8) rows, their loads
// issued together.  Packed sequences: row = h * total_q + i reads O row (i, h).
constexpr int DELTA_U = 4;
template <int D>
constexpr int delta_rows_per_block() { return 4 * (64 / (D / 8)) * DELTA_U; }

template <bool BF16, int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a, int64_t rows) {
    constexpr int CH = D / 8, RPW = 64 / CH;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane % CH, r = lane / CH;
    int64_t row[DELTA_U];
    u32x4 ov[DELTA_U], gv[DELTA_U];
#pragma unroll
    for (int u = 0; u < DELTA_U; ++u) {
        row[u] = (int64_t)blockIdx.x * delta_rows_per_block<D>() + (u * 4 + w) * RPW + r;
        size_t orow = (size_t)row[u];
        if constexpr (VARLEN) {
            const int64_t h = row[u] / a.total_q;
            orow = (size_t)(row[u] - h * a.total_q) * a.H + (size_t)h;
        }
        if (row[u] < rows) {
            ov[u] = *(const u32x4*)(a.o + orow * D + 8 * c);
            gv[u] = *(const u32x4*)(a.dout + orow * D + 8 * c);
        } else {
            ov[u] = u32x4{0, 0, 0, 0};
            gv[u] = u32x4{0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int u = 0; u < DELTA_U; ++u) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = __builtin_fmaf(widen<BF16>((uint16_t)(ov[u][i] & 0xffff)), widen<BF16>((uint16_t)(gv[u][i] & 0xffff)),
                                 acc);
            acc = __builtin_fmaf(widen<BF16>((uint16_t)(ov[u][i] >> 16)), widen<BF16>((uint16_t)(gv[u][i] >> 16)), acc);
        }
#pragma unroll
        for (int m = 1; m < CH; m <<= 1) acc += __shfl_xor(acc, m);
        if (c == 0 && row[u] < rows) {
            a.delta[row[u]] = acc;
            a.lse2[row[u]] = a.lse[row[u]] * kLog2e;
        }
    }
}

// Per-lane LDS offsets shared by both kernels (tiles of rows of D 16-bit values,
// XOR-swizzled): row reads of the A operand with rows in the swapped order, and
// transposed reads of 4 rows x 4 chunks.
template <int D>
struct Offsets {
    int row[D / 16];          // A operand: row perm_row(l32), chunk 2s + h
    int tr[2][D / 32];        // transposed A operand: block db, half 0/1
    __device__ __forceinline__ Offsets(int lane) {
        const int l32 = lane & 31, h = lane >> 5;
        const int r0 = perm_row(l32);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) row[s] = lds_off<D>(r0, 2 * s + h);
        const int r4 = (lane & 15) >> 2, c4 = lane & 3, g1 = (lane >> 4) & 1;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                tr[half][db] = lds_off<D>(8 * h + r4 + 4 * half, 4 * db + 2 * g1 + (c4 >> 1)) + (c4 & 1) * 8;
    }
};

// A operand of rows^T (d block db, 16 rows starting at `rows`) via transposed reads.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const unsigned char* rows, const Offsets<D>& of, int db) {
    const u32x2 l2 = __builtin_bit_cast(u32x2, lds_read_tr16(rows + of.tr[0][db]));
    const u32x2 h2 = __builtin_bit_cast(u32x2, lds_read_tr16(rows + of.tr[1][db]));
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Fill `nload` 1 KiB chunks of an LDS tile of rows (the wave's share) from
// global rows through buffer loads that write LDS; rows past the descriptor's
// record count read as zeros.
// Rows lie row_bytes apart; the record count ends at the first missing row, so
// no lane reads past the last present row.
template <int D, int NPW>
__device__ __forceinline__ void load_rows(const uint16_t* base, int rows_left, unsigned char* dst_tile, int w,
                                          const u32 (&voff)[NPW], int row_bytes) {
    // wave-uniform record count (a per-lane value would wrap each load in a
    // readfirstlane loop)
    const u32 nrec = (u32)__builtin_amdgcn_readfirstlane(min(max(rows_left, 0), 64)) * (u32)row_bytes;   // tiles hold 64 rows
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base, nrec);
    unsigned char* dst = dst_tile + w * NPW * 1024;
#pragma unroll
    for (int u = 0; u < NPW; ++u) lds_dma16(r, dst + u * 1024, voff[u]);
}

// Global byte offsets (rows row_bytes apart) of the chunks this lane moves into
// the swizzled LDS tile.
template <int D, int NPW>
__device__ __forceinline__ void dma_offsets(int w, int lane, u32 (&voff)[NPW], int row_bytes) {
    constexpr int ROWB = D * 2;
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
        const int pos = (w * NPW + u) * 1024 + lane * 16;
        const int row = pos / ROWB, pchunk = (pos % ROWB) >> 4;
        voff[u] = (u32)(row * row_bytes + ((pchunk ^ swz<D>(row)) << 4));
    }
}

// Work items of this workgroup: XCD-contiguous ranges (tiles of one head share
// an XCD's L2), `per_head` tiles per head, tile index in the order given (the
// longest causal tile first).  PAIR (causal): the workgroup runs tiles t and
// per_head-1-t, which together carry a fixed amount of work, so the XCD
// round-robin dispatcher never stalls on one XCD's long tile.  XCD = false keeps
// the dispatcher's own round-robin order instead: packed sequences differ in
// work by orders of magnitude, and contiguous ranges would put a long sequence's
// heads on one XCD.
//
// With packed sequences (cu, the B + 1 offsets of the lengths that set the work)
// the heads of the longest sequence come first, then the next longest: the
// longest items start first and the short ones fill the end of the grid.  Every
// wavefront ranks the B <= 64 lengths itself (seq_at_rank); with more sequences
// the index order is kept.
template <bool PAIR, bool XCD = true, class F>
__device__ __forceinline__ void for_items(int per_head, int BH, F&& item, const int* cu = nullptr, int heads = 1) {
    const int total = gridDim.x;
    int L = blockIdx.x;
    if (XCD && (total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
    auto order = [&](int bh) {
        const int B = BH / heads;
        if (cu == nullptr || B > 64) return bh;
        return seq_at_rank(cu, B, bh / heads) * heads + bh % heads;
    };
    if (PAIR && per_head >= 2) {
        const int npairs = (per_head + 1) >> 1;
        const int t = L % npairs, bh = order(L / npairs);
        item(t, bh);
        if (t != per_head - 1 - t) {
            __syncthreads();        // the next item refills the LDS stages
            item(per_head - 1 - t, bh);
        }
    } else {
        item(L % per_head, order((L / per_head) % BH));
    }
}

// Workgroups of a launch over `per_head` tiles per head (see for_items).
inline int64_t item_blocks(bool pair, int per_head, int BH) {
    return (pair && per_head >= 2) ? (int64_t)((per_head + 1) / 2) * BH : (int64_t)per_head * BH;
}

// Two score products over one 32-row block of LDS tiles: S = A1 B1 and
// P' = A2 B2, with A1, A2 the rows 32kb.. of tiles T1, T2 (in the swapped order)
// and B1, B2 the lane's register-resident operands.  dK/dV kernel: S = Q K^T,
// dP = dO V^T; dQ kernel: S^T = K Q^T, dP^T = V dO^T.
template <bool BF16, int D>
__device__ __forceinline__ void scores(const unsigned char* T1, const unsigned char* T2, int kb,
                                       const Offsets<D>& of, const u32x4 (&b1)[D / 16],
                                       const u32x4 (&b2)[D / 16], f32x16& s, f32x16& dp) {
    constexpr int NS = D / 16, ROWB = D * 2;
    u32x4 a1[NS], a2[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        a1[i] = *(const u32x4*)(T1 + 32 * kb * ROWB + of.row[i]);
        a2[i] = *(const u32x4*)(T2 + 32 * kb * ROWB + of.row[i]);
    }
    s = mfma32<BF16>(a1[0], b1[0], f32x16{});
    dp = mfma32<BF16>(a2[0], b2[0], f32x16{});
#pragma unroll
    for (int i = 1; i < NS; ++i) {
        s = mfma32<BF16>(a1[i], b1[i], s);
        dp = mfma32<BF16>(a2[i], b2[i], dp);
    }
}

// Store a wave's 32 x D output tile held in the transposed-accumulator layout
// (acc[db] register 4g + i is column 32 db + 8g + 4h + i of row l32) as 16-bit
// values times `mul`: the tile goes through the wave's own LDS region `reg`
// (32 rows, 16-byte chunks XOR-swizzled by row) and leaves one 16-byte chunk per
// lane, so each store instruction covers whole rows.  Rows r with row0 + r >= n
// are not stored.  The caller guarantees no other wave uses `reg` meanwhile.
template <bool BF16, int D>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[D / 32], float mul, unsigned char* reg,
                                                  uint16_t* dst, int row_stride, int row0, int n, int lane) {
    constexpr int ROWB = D * 2, CH = ROWB / 16, RPI = 1024 / ROWB;
    // the lane's LDS addresses are formed here, after the walk: computed at the
    // kernel's start (the compiler's choice otherwise) they would stay live across
    // the whole walk and spill to scratch
    asm volatile("" : "+v"(lane));
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2 v2 = {pack2<BF16>(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                              pack2<BF16>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
            const int c = 4 * db + g;
            *(u32x2*)(reg + l32 * ROWB + ((c ^ (l32 & (CH - 1))) << 4) + 8 * h) = v2;
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int c = lane % CH;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
        const int r = it * RPI + lane / CH;
        const u32x4 v4 = *(const u32x4*)(reg + r * ROWB + ((c ^ (r & (CH - 1))) << 4));
        if (row0 + r < n) *(u32x4*)(dst + (size_t)(row0 + r) * row_stride + 8 * c) = v4;
    }
}

// ---- dQ ---------------------------------------------------------------------
// dS^T for one 32-key block (register 8p + e stands for key k0 + 32kb + 16p + 8h
// + e), packed as the B operand of dQ^T += K^T dS^T.  MASK zeroes P from key
// 16p + e >= bound on (the key tail, or keys past this row's diagonal).
template <bool BF16, bool MASK>
__device__ __forceinline__ void dq_probs(const f32x16& s, const f32x16& dp, float lse2, float dlt, float c,
                                         int bound, u32x4 (&dsb)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float pr = exp2_fast(__builtin_fmaf(s[8 * p + e], c, -lse2));
            if (MASK) pr = (16 * p + e < bound) ? pr : 0.f;
            ds[e] = pr * (dp[8 * p + e] - dlt);
        }
        dsb[p] = u32x4{pack2<BF16>(ds[0], ds[1]), pack2<BF16>(ds[2], ds[3]), pack2<BF16>(ds[4], ds[5]),
                       pack2<BF16>(ds[6], ds[7])};
    }
}

// dQ^T += K^T dS^T over the keys of that block, K^T through transposed reads.
template <bool BF16, int D>
__device__ __forceinline__ void dq_accum(const unsigned char* Kb, int kb, const Offsets<D>& of,
                                         const u32x4 (&dsb)[2], f32x16 (&dq)[D / 32]) {
    constexpr int ROWB = D * 2;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const unsigned char* kr = Kb + (32 * kb + 16 * p) * ROWB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mfma32<BF16>(tr_operand<D>(kr, of, db), dsb[p], dq[db]);
    }
}

// NW wavefronts of 32 query rows: 4 (two workgroups per CU) or 8 (one per CU;
// each K/V tile is then loaded once for 256 rows)
template <bool BF16, int D, bool CAUSAL, bool VARLEN, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_dq_kernel(BwdArgs a) {
    constexpr int ROWB = D * 2, TILE = BK * ROWB, NS = D / 16, ND = D / 32;
    constexpr int BQW = 32 * NW;                 // query rows per workgroup
    constexpr int NPW = TILE / 1024 / NW;
    __shared__ __attribute__((aligned(16))) unsigned char stage0[2 * TILE];   // [K | V]
    __shared__ __attribute__((aligned(16))) unsigned char stage1[2 * TILE];

    auto run_item = [&](const int t, const int bh) __attribute__((always_inline)) {
        const int bkv = a.group == 1 ? bh : (bh / a.H) * a.H_kv + (bh % a.H) / a.group;   // K/V head read
        const Seq sg = seq_of<D, VARLEN>(a, bh, bkv);
        const int Nq = sg.Nq, Nk = sg.Nk, off = Nk - Nq;
        const int nqt = VARLEN ? (Nq + BQW - 1) / BQW : a.n_qtiles;
        if (VARLEN && (!sg.ok || t >= nqt)) return;      // past this sequence's rows
        const int qt = nqt - 1 - t;                      // longest causal rows first
        const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), l32 = lane & 31, h = lane >> 5;
        const int q0 = qt * BQW, qw = q0 + 32 * w, qi = qw + l32;
        const uint16_t* kg = a.k + sg.k;
        const uint16_t* vg = a.v + sg.k;

        int hi = Nk;
        if (CAUSAL) hi = min(hi, min(Nq, q0 + BQW) + off);
        const int n_tiles = hi > 0 ? (hi + BK - 1) / BK : 0;

        // this lane's query row: Q and dO chunks, LSE (log2 units) and D
        u32x4 qf[NS], gf[NS];
        const bool qok = qi < Nq;
    #pragma unroll
        for (int s = 0; s < NS; ++s) {
            const size_t e = sg.q + (size_t)qi * sg.sq + 16 * s + 8 * h;
            qf[s] = qok ? *(const u32x4*)(a.q + e) : u32x4{0, 0, 0, 0};
            gf[s] = qok ? *(const u32x4*)(a.dout + e) : u32x4{0, 0, 0, 0};
        }
        const float lse2 = qok ? a.lse2[sg.l + qi] : 0.f;
        const float dlt = qok ? a.delta[sg.l + qi] : 0.f;

        u32 voff[NPW];
        dma_offsets<D, NPW>(w, lane, voff, sg.sk * 2);
        auto load_tile = [&](int tile, unsigned char* stage) {
            const int k0 = tile * BK;
            load_rows<D, NPW>(kg + (size_t)k0 * sg.sk, Nk - k0, stage, w, voff, sg.sk * 2);
            load_rows<D, NPW>(vg + (size_t)k0 * sg.sk, Nk - k0, stage + TILE, w, voff, sg.sk * 2);
        };
        const Offsets<D> of(lane);

        f32x16 dqacc[ND];
    #pragma unroll
        for (int db = 0; db < ND; ++db) dqacc[db] = f32x16{};

        // One key tile of two 32-key blocks.  Keys at or past `bound` (relative to
        // k0 + 8h; the key tail or, causal, past this row's diagonal) get P = 0 in
        // masked tiles.  The scores of the second block are issued before the first
        // block's element-wise work.
        auto step = [&](const unsigned char* Kb, const unsigned char* Vb, int bound, auto mask) {
            constexpr bool MASK = decltype(mask)::value;
            f32x16 s0, d0, s1, d1;
            u32x4 ds0[2], ds1[2];
            scores<BF16, D>(Kb, Vb, 0, of, qf, gf, s0, d0);
            scores<BF16, D>(Kb, Vb, 1, of, qf, gf, s1, d1);
            dq_probs<BF16, MASK>(s0, d0, lse2, dlt, a.c, bound, ds0);
            dq_accum<BF16, D>(Kb, 0, of, ds0, dqacc);
            dq_probs<BF16, MASK>(s1, d1, lse2, dlt, a.c, bound - 32, ds1);
            dq_accum<BF16, D>(Kb, 1, of, ds1, dqacc);
        };

        // key tiles from the last one down: the ones crossing the diagonal or the key
        // tail come first
        int n_masked = 0;
        while (n_masked < n_tiles) {
            const int k0 = (n_tiles - 1 - n_masked) * BK;
            const bool clean = k0 + BK <= Nk && (!CAUSAL || k0 + BK - 1 <= q0 + off);
            if (clean) break;
            ++n_masked;
        }
        if (n_tiles > 0) load_tile(n_tiles - 1, stage0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // the masked tiles (per-wave visibility, stage chosen at run time), then the
        // clean ones two per trip so that each step reads one fixed LDS stage: one
        // body per loop, so the accumulators never meet at a branch join
        int it = 0;
    #pragma clang loop unroll(disable)
        for (; it < n_masked; ++it) {
            const int tile = n_tiles - 1 - it;
            unsigned char* cur = (it & 1) ? stage1 : stage0;
            unsigned char* nxt = (it & 1) ? stage0 : stage1;
            if (it + 1 < n_tiles) load_tile(tile - 1, nxt);
            const int k0 = tile * BK;
            if (qw < Nq && (!CAUSAL || k0 <= min(qw + 31, Nq - 1) + off)) {
                int bound = Nk - k0;
                if (CAUSAL) bound = min(bound, qi + off - k0 + 1);
                step(cur, cur + TILE, bound - 8 * h, std::true_type{});
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        auto clean_one = [&](unsigned char* cur, unsigned char* nxt) {
            const int tile = n_tiles - 1 - it;
            if (it + 1 < n_tiles) load_tile(tile - 1, nxt);
            step(cur, cur + TILE, BK, std::false_type{});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ++it;
        };
        if ((it & 1) && it < n_tiles) clean_one(stage1, stage0);
    #pragma clang loop unroll(disable)
        while (it < n_tiles) {
            clean_one(stage0, stage1);
            if (it < n_tiles) clean_one(stage1, stage0);
        }

        // the walk ended with a barrier, so the stages are free: each wave stages
        // its 32 rows in its own quarter of stage 0 (waves 4..7: of stage 1)
        store_rows_staged<BF16, D>(dqacc, a.scale, (w < 4 ? stage0 : stage1) + (w & 3) * (32 * ROWB), a.dq + sg.q,
                                   sg.sq, qw, Nq, lane);
    };
    for_items<CAUSAL, !VARLEN>(a.n_qtiles, a.BH, run_item, VARLEN ? a.cu_q : nullptr, a.H);
}

// ---- dK, dV -------------------------------------------------------------------
// P = exp(S - LSE) and dS = P o (dP - D) for those rows, packed as the B operands
// of the dV and dK products; register 8p + e stands for query row
// 32kb + 16p + 8h + e (`rb` = 32kb + 8h).  Ls holds LSE * log2(e).  MASK zeroes
// P where 16p + e < lim: rows that do not yet see this lane's key.
template <bool BF16, bool MASK>
__device__ __forceinline__ void dkdv_probs(const f32x16& s, const f32x16& dp, const float* Ls, const float* Ds,
                                           int rb, float c, int lim, u32x4 (&pb)[2], u32x4 (&sb)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const f32x4 la = *(const f32x4*)(Ls + rb + 16 * p), lb = *(const f32x4*)(Ls + rb + 16 * p + 4);
        const f32x4 da = *(const f32x4*)(Ds + rb + 16 * p), dbv = *(const f32x4*)(Ds + rb + 16 * p + 4);
        const float lr[8] = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3]};
        const float dr[8] = {da[0], da[1], da[2], da[3], dbv[0], dbv[1], dbv[2], dbv[3]};
        float pr[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pr[e] = exp2_fast(__builtin_fmaf(s[8 * p + e], c, -lr[e]));
            if (MASK) pr[e] = (16 * p + e < lim) ? 0.f : pr[e];
            ds[e] = pr[e] * (dp[8 * p + e] - dr[e]);
        }
        pb[p] = u32x4{pack2<BF16>(pr[0], pr[1]), pack2<BF16>(pr[2], pr[3]), pack2<BF16>(pr[4], pr[5]),
                      pack2<BF16>(pr[6], pr[7])};
        sb[p] = u32x4{pack2<BF16>(ds[0], ds[1]), pack2<BF16>(ds[2], ds[3]), pack2<BF16>(ds[4], ds[5]),
                      pack2<BF16>(ds[6], ds[7])};
    }
}

// Empty asm statements that take a value as an operand: the value's computation
// is then ordered before the statement.  Scheduling fences order memory operations
// only; without these, pure arithmetic (matrix products included) drifts past a
// fence towards its first use.  The matrix accumulators live in the AGPR file.
#define FA_PIN_A(x) asm volatile("" : "+a"(x))
#define FA_PIN_V(x) asm volatile("" : "+v"(x))

// Four of those rows (register 8p + e0 .. 8p + e0 + 3, e0 in {0, 4}): the same
// values as dkdv_probs, written into words e0/2, e0/2 + 1 of pb[p] and sb[p].
template <bool BF16, bool MASK>
__device__ __forceinline__ void dkdv_probs4(const f32x16& s, const f32x16& dp, const f32x4& l4, const f32x4& d4,
                                            float c, int lim, int p, int e0, u32x4& pbp, u32x4& sbp) {
    float pr[4], ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pr[e] = exp2_fast(__builtin_fmaf(s[8 * p + e0 + e], c, -l4[e]));
        if (MASK) pr[e] = (16 * p + e0 + e < lim) ? 0.f : pr[e];
        ds[e] = pr[e] * (dp[8 * p + e0 + e] - d4[e]);
    }
    u32 w0 = pack2<BF16>(pr[0], pr[1]), w1 = pack2<BF16>(pr[2], pr[3]);
    u32 w2 = pack2<BF16>(ds[0], ds[1]), w3 = pack2<BF16>(ds[2], ds[3]);
    FA_PIN_V(w0);
    FA_PIN_V(w1);
    FA_PIN_V(w2);
    FA_PIN_V(w3);
    pbp[e0 / 2] = w0;
    pbp[e0 / 2 + 1] = w1;
    sbp[e0 / 2] = w2;
    sbp[e0 / 2 + 1] = w3;
}

template <bool BF16, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
    constexpr int ROWB = D * 2, QTILE = CQ * ROWB, NS = D / 16, ND = D / 32;
    constexpr int NPW = QTILE / 1024 / 4;
    constexpr int STAGE = 2 * QTILE + 2048;             // [Q | dO | LSE*log2e (1 KiB) | D (1 KiB)]
    __shared__ __attribute__((aligned(16))) unsigned char stage0[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char stage1[STAGE];

    // key tile 0 first: the longest causal columns
    auto run_item = [&](const int kt, const int bh) __attribute__((always_inline)) {
        // bh is the K/V head b*H_kv + hk; its query heads b*H + hk*group + g
        // (g < group) each add their rows' contributions to dK and dV
        const int bq0 = (bh / a.H_kv) * a.H + (bh % a.H_kv) * a.group;
        const Seq sg = seq_of<D, VARLEN>(a, bq0, bh);
        const int Nq = sg.Nq, Nk = sg.Nk, off = Nk - Nq;
        if (VARLEN && (!sg.ok || kt * CK >= Nk)) return;   // past this sequence's keys
        const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), l32 = lane & 31, h = lane >> 5;
        const int k0 = kt * CK, kw = k0 + 32 * w, kj = kw + l32;

        // first query row that sees a key of this block, and the query tiles from it
        const int q_lo = CAUSAL ? max(0, k0 - off) : 0;
        const int t0 = q_lo / CQ;
        const int n_qt = (Nq + CQ - 1) / CQ;
        const int n_tiles = q_lo < Nq ? n_qt - t0 : 0;

        // this lane's key row: K and V chunks (the B operands)
        u32x4 kf[NS], vf[NS];
        const bool kok = kj < Nk;
    #pragma unroll
        for (int s = 0; s < NS; ++s) {
            const size_t e = sg.k + (size_t)kj * sg.sk + 16 * s + 8 * h;
            kf[s] = kok ? *(const u32x4*)(a.k + e) : u32x4{0, 0, 0, 0};
            vf[s] = kok ? *(const u32x4*)(a.v + e) : u32x4{0, 0, 0, 0};
        }

        u32 voff[NPW];
        dma_offsets<D, NPW>(w, lane, voff, sg.sq * 2);
        // the query tile `tile` of query head g of the group
        auto load_tile = [&](int g, int tile, unsigned char* stage) {
            const int i0 = tile * CQ;
            const uint16_t* qg = a.q + sg.q + g * sg.qh;
            const uint16_t* gg = a.dout + sg.q + g * sg.qh;
            const float* lg = a.lse2 + sg.l + g * sg.lh;
            const float* dg = a.delta + sg.l + g * sg.lh;
            load_rows<D, NPW>(qg + (size_t)i0 * sg.sq, Nq - i0, stage, w, voff, sg.sq * 2);
            load_rows<D, NPW>(gg + (size_t)i0 * sg.sq, Nq - i0, stage + QTILE, w, voff, sg.sq * 2);
            // 64 LSE and 64 D values (256 B each) land at lane*16 of a 1 KiB area;
            // lanes past 64 rows read zeros
            const u32 nrec = (u32)__builtin_amdgcn_readfirstlane(min(max(Nq - i0, 0), CQ)) * 4;
            if (w == 0) lds_dma16(buffer_rsrc(lg + i0, nrec), stage + 2 * QTILE, (u32)lane * 16);
            if (w == 1) lds_dma16(buffer_rsrc(dg + i0, nrec), stage + 2 * QTILE + 1024, (u32)lane * 16);
        };
        const Offsets<D> of(lane);

        f32x16 dkacc[ND], dvacc[ND];
    #pragma unroll
        for (int db = 0; db < ND; ++db) {
            dkacc[db] = f32x16{};
            dvacc[db] = f32x16{};
        }

        // One query tile of two 32-row blocks.  The scores of the second block are
        // issued before the first block's element-wise work, which then runs beside
        // those matrix instructions.
        auto step = [&](const unsigned char* st, int i0, auto mask) {
            constexpr bool MASK = decltype(mask)::value;
            const unsigned char* Qb = st;
            const unsigned char* Gb = st + QTILE;
            const float* Ls = (const float*)(st + 2 * QTILE);
            const float* Ds = (const float*)(st + 2 * QTILE + 1024);
            const int lim = kj - i0 - off - 8 * h;
            constexpr int ROWB = D * 2;
            // Operand reads are issued in a fixed order (scheduling fences) well ahead of
            // the products that use them: at one wave per SIMD the LDS latency, above all
            // of the transposed reads, is not hidden by other waves.
            auto rows = [&](const unsigned char* T, int kb, int i) {
                return *(const u32x4*)(T + 32 * kb * ROWB + of.row[i]);
            };
            auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
            u32x4 qa[NS], ga[NS], qb[NS], gb[NS];
    #pragma unroll
            for (int i = 0; i < NS; ++i) {
                qa[i] = rows(Qb, 0, i);
                ga[i] = rows(Gb, 0, i);
            }
            fence();
            // S and dP of rows 0..31, the operands of rows 32..63 read beside them
            f32x16 s0 = f32x16{}, d0 = f32x16{}, s1 = f32x16{}, d1 = f32x16{};
    #pragma unroll
            for (int i = 0; i < NS; ++i) {
                s0 = mfma32<BF16>(qa[i], kf[i], s0);
                FA_PIN_A(s0);
                qb[i] = rows(Qb, 1, i);
                d0 = mfma32<BF16>(ga[i], vf[i], d0);
                FA_PIN_A(d0);
                gb[i] = rows(Gb, 1, i);
                fence();
            }
            // S and dP of rows 32..63 beside the element-wise work of rows 0..31
            // (and the first transposed operands of rows 0..31's gradient products read
            // beside them, so that those products start without waiting)
            u32x4 pb[2], sb[2], pb1[2], sb1[2];
            u32x4 tg0[ND], tq0[ND], tg1[ND], tq1[ND];
            f32x4 l1[4], dd1[4];
            // LSE and D of rows 32..63 (read before the transposed operands that follow
            // them: LDS reads complete in order, so a later read would wait for those)
            auto read_ld1 = [&](int qtr) {
                const int o = 32 + 8 * h + 16 * (qtr >> 1) + 4 * (qtr & 1);
                l1[qtr] = *(const f32x4*)(Ls + o);
                dd1[qtr] = *(const f32x4*)(Ds + o);
            };
            if constexpr (D == 128) {
                // the element-wise work of rows 0..31 in quarters between the score
                // products of rows 32..63 (at d = 64 the extra registers would cost
                // the second wavefront per SIMD)
                f32x4 l0[4], dd0[4];
    #pragma unroll
                for (int qtr = 0; qtr < 4; ++qtr) {
                    const int o = 8 * h + 16 * (qtr >> 1) + 4 * (qtr & 1);
                    l0[qtr] = *(const f32x4*)(Ls + o);
                    dd0[qtr] = *(const f32x4*)(Ds + o);
                }
    #pragma unroll
                for (int i = 0; i < NS; ++i) {
                    s1 = mfma32<BF16>(qb[i], kf[i], s1);
                    FA_PIN_A(s1);
                    d1 = mfma32<BF16>(gb[i], vf[i], d1);
                    FA_PIN_A(d1);
                    if (i < ND) {
                        tg0[i] = tr_operand<D>(Gb, of, i);
                        tq0[i] = tr_operand<D>(Qb, of, i);
                    } else if (i < ND + 4) {
                        read_ld1(i - ND);
                    }
                    if (i % (NS / 4) == NS / 4 - 1) {
                        const int qtr = i / (NS / 4), p = qtr >> 1, e0 = 4 * (qtr & 1);
                        dkdv_probs4<BF16, MASK>(s0, d0, l0[qtr], dd0[qtr], a.c, lim, p, e0, pb[p], sb[p]);
                    }
                    fence();
                }
            } else {
    #pragma unroll
                for (int i = 0; i < NS; ++i) {
                    s1 = mfma32<BF16>(qb[i], kf[i], s1);
                    d1 = mfma32<BF16>(gb[i], vf[i], d1);
                    if (i < ND) {
                        tg0[i] = tr_operand<D>(Gb, of, i);
                        tq0[i] = tr_operand<D>(Qb, of, i);
                    }
                }
                dkdv_probs<BF16, MASK>(s0, d0, Ls, Ds, 8 * h, a.c, lim, pb, sb);
                fence();
            }
            // dV^T += dO^T P and dK^T += Q^T dS over one 32-row block: the transposed
            // operands of its first 16 rows (tg, tq) already read, those of the next 16
            // beside the first products; `before` runs first, the four quarters of
            // `beside` run spread over the products, and `next(db)` reads operands
            // for what follows beside the second half's products
            auto accum = [&](int kb, const u32x4 (&pp)[2], const u32x4 (&ss)[2], const u32x4 (&tg)[ND],
                             const u32x4 (&tq)[ND], auto&& before, auto&& beside, auto&& next) {
                const unsigned char* q0r = Qb + (32 * kb) * ROWB;
                const unsigned char* g0r = Gb + (32 * kb) * ROWB;
                before();
                u32x4 ug[ND], uq[ND];
                // the 2 ND product pairs carry the four quarters of `beside` evenly
                auto quarter = [&](int u) {
                    if (((u + 1) * 4) % (2 * ND) == 0) beside((u + 1) * 4 / (2 * ND) - 1);
                };
                fence();
    #pragma unroll
                for (int db = 0; db < ND; ++db) {
                    dvacc[db] = mfma32<BF16>(tg[db], pp[0], dvacc[db]);
                    FA_PIN_A(dvacc[db]);
                    ug[db] = tr_operand<D>(g0r + 16 * ROWB, of, db);
                    dkacc[db] = mfma32<BF16>(tq[db], ss[0], dkacc[db]);
                    FA_PIN_A(dkacc[db]);
                    uq[db] = tr_operand<D>(q0r + 16 * ROWB, of, db);
                    quarter(db);
                    fence();
                }
    #pragma unroll
                for (int db = 0; db < ND; ++db) {
                    dvacc[db] = mfma32<BF16>(ug[db], pp[1], dvacc[db]);
                    FA_PIN_A(dvacc[db]);
                    dkacc[db] = mfma32<BF16>(uq[db], ss[1], dkacc[db]);
                    FA_PIN_A(dkacc[db]);
                    quarter(ND + db);
                    next(db);
                    fence();
                }
            };
            // the element-wise work of rows 32..63, a quarter beside every four products
            // of rows 0..31 (at d = 128 its LSE and D values were read beside the
            // score products)
            accum(0, pb, sb, tg0, tq0, [&] {
                if constexpr (D != 128)
    #pragma unroll
                    for (int qtr = 0; qtr < 4; ++qtr) read_ld1(qtr);
            }, [&](int qtr) {
                const int p = qtr >> 1, e0 = 4 * (qtr & 1);
                dkdv_probs4<BF16, MASK>(s1, d1, l1[qtr], dd1[qtr], a.c, lim - 32, p, e0, pb1[p], sb1[p]);
            }, [&](int db) {
                tg1[db] = tr_operand<D>(Gb + 32 * ROWB, of, db);
                tq1[db] = tr_operand<D>(Qb + 32 * ROWB, of, db);
            });
            accum(1, pb1, sb1, tg1, tq1, [] {}, [](int) {}, [](int) {});
        };

        // Query tiles upward from the diagonal, for each query head of the group in
        // turn.  Causal: the first n_mt tiles of a head hold rows that do not yet see
        // every key of the block and run the masked body (a wave whose keys no row of
        // the tile sees skips it); all later tiles run the unmasked body.  Separate
        // loops keep one body per loop, so the accumulators never meet at a branch join.
        int n_mt = 0;
        if (CAUSAL && n_tiles > 0) {
            const int last_partial = k0 + CK - 2 - off;   // last row that misses a key of the block
            n_mt = last_partial < 0 ? 0 : min(n_tiles, last_partial / CQ - t0 + 1);
        }
        const int n_steps = n_tiles * a.group;
        if (n_steps > 0) load_tile(0, t0, stage0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int it = 0;                    // steps done (the stage of step it is it & 1)
        // load the tile after (g, tile): the head's next tile, else the next head's first
        auto prefetch = [&](int g, int tile, unsigned char* nxt) {
            if (tile + 1 < t0 + n_tiles) load_tile(g, tile + 1, nxt);
            else if (g + 1 < a.group) load_tile(g + 1, t0, nxt);
        };
        auto clean_one = [&](int g, int& tile, unsigned char* cur, unsigned char* nxt) {
            prefetch(g, tile, nxt);
            step(cur, tile * CQ, std::false_type{});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ++tile;
            ++it;
        };
    #pragma clang loop unroll(disable)
        for (int g = 0; g < a.group && n_tiles > 0; ++g) {
            int tile = t0;
    #pragma clang loop unroll(disable)
            for (; tile < t0 + n_mt; ++tile, ++it) {
                unsigned char* cur = (it & 1) ? stage1 : stage0;
                unsigned char* nxt = (it & 1) ? stage0 : stage1;
                prefetch(g, tile, nxt);
                const int i0 = tile * CQ;
                if (kw <= i0 + CQ - 1 + off) step(cur, i0, std::true_type{});
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            }
            if ((it & 1) && tile < t0 + n_tiles) clean_one(g, tile, stage1, stage0);
    #pragma clang loop unroll(disable)
            while (tile < t0 + n_tiles) {
                clean_one(g, tile, stage0, stage1);
                if (tile < t0 + n_tiles) clean_one(g, tile, stage1, stage0);
            }
        }

        // the walk ended with a barrier, so the stages are free: each wave stages its
        // 32 dK rows in its quarter of stage 0 and its dV rows in stage 1
        store_rows_staged<BF16, D>(dkacc, a.scale, stage0 + w * (32 * ROWB), a.dk + sg.k, sg.sk, kw, Nk, lane);
        store_rows_staged<BF16, D>(dvacc, 1.f, stage1 + w * (32 * ROWB), a.dv + sg.k, sg.sk, kw, Nk, lane);
    };
    // over the K/V heads; packed sequences longest first
    for_items<CAUSAL, !VARLEN>(a.n_ktiles, a.BH / a.group, run_item, VARLEN ? a.cu_k : nullptr, a.H_kv);
}

// 8-wavefront dQ workgroups for dense d = 128 where they beat 4 (wide_rows; the
// dQ walk wins from 1024 keys on)
inline bool dq_wide(bool varlen, int d, int Nq, int Nk, int64_t bh, bool causal) {
    return !varlen && d == 128 && wide_rows(wide_blocks(Nq, bh, causal), Nk, 1024);
}

template <bool BF16, int D, bool VARLEN>
hipError_t launch_bwd_t(const BwdArgs& a, bool causal, int64_t rows, hipStream_t s) {
    const int64_t dblocks = (rows + delta_rows_per_block<D>() - 1) / delta_rows_per_block<D>();
    hipLaunchKernelGGL((bwd_delta_kernel<BF16, D, VARLEN>), dim3((int)dblocks), dim3(256), 0, s, a, rows);
    const int kv_blocks = (int)item_blocks(causal, a.n_ktiles, a.BH / a.group);
    const int q_blocks = (int)item_blocks(causal, a.n_qtiles, a.BH);
    const bool wide = dq_wide(VARLEN, D, a.Nq, a.Nk, a.BH, causal);
    if (causal) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, true, VARLEN>), dim3(kv_blocks), dim3(256), 0, s, a);
        if constexpr (D == 128 && !VARLEN)
            if (wide) {
                hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, true, VARLEN, 8>), dim3(q_blocks), dim3(512), 0, s, a);
                return hipGetLastError();
            }
        hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, true, VARLEN, 4>), dim3(q_blocks), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, false, VARLEN>), dim3(kv_blocks), dim3(256), 0, s, a);
        if constexpr (D == 128 && !VARLEN)
            if (wide) {
                hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, false, VARLEN, 8>), dim3(q_blocks), dim3(512), 0, s, a);
                return hipGetLastError();
            }
        hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, false, VARLEN, 4>), dim3(q_blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <bool VARLEN>
hipError_t launch_bwd_v(const BwdArgs& a, int d, bool bf16, bool causal, int64_t rows, hipStream_t stream) {
    if (d == 128) return bf16 ? launch_bwd_t<true, 128, VARLEN>(a, causal, rows, stream)
                              : launch_bwd_t<false, 128, VARLEN>(a, causal, rows, stream);
    return bf16 ? launch_bwd_t<true, 64, VARLEN>(a, causal, rows, stream)
                : launch_bwd_t<false, 64, VARLEN>(a, causal, rows, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    BwdArgs a;
    a.q = (const uint16_t*)p.q;
    a.k = (const uint16_t*)p.k;
    a.v = (const uint16_t*)p.v;
    a.o = (const uint16_t*)p.o;
    a.dout = (const uint16_t*)p.dout;
    a.lse = p.lse;
    a.delta = p.delta;
    const bool varlen = p.cu_q != nullptr;
    // LSE, D and LSE * log2(e) rows: [B, H, Nq], or [H, total_q] for packed sequences
    const int64_t rows = varlen ? (int64_t)p.H * p.total_q : (int64_t)p.B * p.H * p.Nq;
    a.lse2 = p.delta + rows;
    a.cu_q = p.cu_q;
    a.cu_k = p.cu_k;
    a.total_q = p.total_q;
    a.total_k = p.total_k;
    a.dq = (uint16_t*)p.dq;
    a.dk = (uint16_t*)p.dk;
    a.dv = (uint16_t*)p.dv;
    a.BH = p.B * p.H;
    a.H = p.H;
    a.H_kv = p.H_kv > 0 ? p.H_kv : p.H;
    a.group = p.H / a.H_kv;
    a.Nq = p.Nq;
    a.Nk = p.Nk;
    a.c = p.scale * kLog2e;
    a.scale = p.scale;
    const int bq = dq_wide(varlen, p.d, p.Nq, p.Nk, (int64_t)p.B * p.H, p.causal) ? 2 * BQ : BQ;
    a.n_qtiles = (p.Nq + bq - 1) / bq;
    a.n_ktiles = (p.Nk + CK - 1) / CK;
    if ((int64_t)a.n_qtiles * a.BH > 0x7fffffff || (int64_t)a.n_ktiles * a.BH > 0x7fffffff ||
        (rows + delta_rows_per_block<128>() - 1) / delta_rows_per_block<128>() > 0x7fffffff)
        return hipErrorInvalidValue;
    return varlen ? launch_bwd_v<true>(a, p.d, p.bf16, p.causal, rows, stream)
                  : launch_bwd_v<false>(a, p.d, p.bf16, p.causal, rows, stream);
}

}  // namespace fa
