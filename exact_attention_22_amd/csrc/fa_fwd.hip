// fa_fwd.hip -- FlashAttention-2 forward on gfx950 MFMA (prefill and split-KV
// partials for any Nq).
//
// Method (the pages this follows):
//   * Q outer, KV inner: one workgroup owns one tile of Br = 128 (or 256) query
//     rows of one (b, h) and walks the key tiles; O stays on chip and is written once
//     (AIInfraGuide 6.2 "FlashAttention V2 explained", section 2; LLM Infra
//     Atlas "FA2: parallelism", section 2: grid over query tiles x batch x heads).
//   * split-Q: each wavefront owns 32 query rows and computes their whole
//     softmax, so waves never reduce across each other (LLM Infra Atlas,
//     section 3; AIInfraGuide 6.2, section 4).
//   * online softmax with an unnormalised accumulator: O <- alpha*O + P V and
//     l <- alpha*l + rowsum(P), divided by l once at the end (Ringi, "Lecture 25",
//     sections 2.2-2.3; AIInfraGuide 6.2, section 3.2).  exp is evaluated as
//     exp2 with scale*log2(e) folded into one multiplier (LLM Infra Atlas,
//     section 1; KingOfEgg "Flash Attention (4)", section 3.1).
//   * causal: key tiles past the diagonal are never loaded; only tiles crossing
//     the diagonal or the key tail are masked, and walking the tiles from the
//     last one down puts those first (LLM Infra Atlas, section 4; KingOfEgg,
//     section 3.2).
//   * epilogue: inv = 1 when the row sum is 0 or NaN; LSE = max*scale + ln(sum);
//     O is re-laid through shared memory so that the stores cover whole rows
//     (KingOfEgg, section 3.5).
//
// gfx950 mapping (not from the pages):
//   * S^T = K Q^T on v_mfma_f32_32x32x16: a lane's accumulator holds one query
//     (lane % 32) against 16 of 32 keys, so the row max and row sum are in-lane
//     plus one exchange between lane l and l^32 (v_permlane32_swap).
//   * K rows enter the first product in an order with bits 2 and 3 of the key
//     index swapped; then accumulator registers 8p..8p+7 of a lane are exactly
//     the 8 consecutive keys 16p + 8*(lane/32) + 0..7 that lane must supply as
//     the B operand of O^T = V^T P^T.  P goes from the first product's
//     accumulator to the second product's operand with one v_cvt_pk per pair
//     and no LDS round trip.
//   * O^T accumulates in registers: each lane owns its query's output values,
//     so the rescale by alpha is a per-lane multiply.
//   * V stays row-major in LDS and ds_read_b64_tr_b16 produces the key-major
//     operand.  K and V tiles are double-buffered in LDS through 16-byte
//     coalesced buffer loads that write LDS directly and an XOR swizzle
//     (fa_device.h).
//   * Lazy rescale: the exponent reference only moves (and O, l are only
//     rescaled) when it would let a weight grow too large, decided per
//     wavefront.  Any reference gives the same O = sum 2^(t-M) v / sum 2^(t-M).
//     Each 32-key block is exponentiated against the current reference and kept
//     when every lane's sum of its 16 weights stays <= 2^12; otherwise the
//     reference moves to the block's exact running maximum and the block is
//     exponentiated again (rescaling between blocks is the online-softmax
//     merge), so no row maximum is taken while the reference holds.  Keys past
//     the diagonal or the key tail weigh exactly 0.  The reference is always an
//     observed maximum, so it never exceeds the true one; every P stays <= 2^12,
//     far inside fp16 range.
//   * Within a 64-key tile, block 1's S^T products are issued between block
//     0's softmax instructions, and block 0's P V products between block 1's
//     (scheduling groups), so a wavefront's vector work runs while its own
//     products occupy the matrix core.
//   * A workgroup is 4 wavefronts (128 query rows, two workgroups per CU) or,
//     over long key ranges at d = 128 and over full grids at d = 64 without the
//     mask, 8 (256 rows, one per CU), which loads each K/V tile into LDS once for
//     twice the query rows.
//   * Workgroups are mapped so that consecutive tiles of one head share an XCD
//     (and its L2).  Causal [B, H, N, d]: one workgroup runs query tiles
//     n_qtiles-1-t and t, which together see a fixed number of key tiles, so
//     every workgroup carries the same work and the XCD round-robin dispatcher
//     never stalls on one XCD's long tile; otherwise (and for packed sequences)
//     the heaviest tile goes first.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int BC = 64;      // keys per tile
constexpr float SUM_CAP = 4096.f;  // largest per-lane sum of a block's 16 weights kept without moving the reference

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    void* o;
    float* lse;
    int B, H, Nq, Nk;
    int BH;
    float c;           // |scale| * log2(e)
    u32 qsign;         // 0x80008000 flips Q's sign when scale < 0
    int n_qtiles;
    int split_chunk;   // keys per split (split mode)
    // packed variable-length sequences (varlen mode): q, o [total_q, H, d];
    // k, v [total_k, H_kv, d]; lse [H, total_q]; sequence b spans offsets
    // [cu[b], cu[b+1]) of cu_q / cu_k
    const int* cu_q;
    const int* cu_k;
    int H_kv, group;   // group = H / H_kv query heads per K/V head
    int total_q, total_k, max_q, max_k;
    int paired;        // one workgroup runs query tiles n-1-t and t (causal [B,H,N,d]; packed sequences)
};

// Key index (within a 32-key block) that accumulator row i stands for: bits 2 and 3 swapped.
__device__ __forceinline__ int perm_row(int i) {
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// NW wavefronts per workgroup, 32 query rows each: 4 (two workgroups per CU) or 8
// (one per CU; each K/V tile is then loaded once for 256 query rows)
template <bool BF16, int D, bool CAUSAL, bool SPLIT, bool VARLEN, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_kernel(FwdArgs a) {
    static_assert(!(SPLIT && VARLEN), "split-KV partials take the [B,H,N,d] layout");
    constexpr int BR = 32 * NW;                  // query rows per workgroup
    constexpr int ROWB = D * 2;                  // bytes per K/V row
    constexpr int TILE = BC * ROWB;              // bytes per K (or V) tile
    constexpr int NS = D / 16;                   // 16-wide d slices of Q
    constexpr int ND = D / 32;                   // 32-wide d blocks of O^T
    // two LDS stages, each [K tile | V tile]; separate objects so the compiler
    // can tell a stage being filled from the one being read
    __shared__ __attribute__((aligned(16))) unsigned char stage0[2 * TILE];
    __shared__ __attribute__((aligned(16))) unsigned char stage1[2 * TILE];

    // ---- work items ------------------------------------------------------
    // Workgroup b runs on XCD b % 8 (the hardware dispatches round-robin).
    const int total = gridDim.x;
    int L = blockIdx.x;
    if (!VARLEN && (total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);   // XCD-contiguous ranges
    // One query tile of one (sequence, head[, split]).
    auto run_item = [&](const int qt, const int bh, const int split) __attribute__((always_inline)) {
        const int q0 = qt * BR;

        // ---- this item's sequence: sizes, base pointers, row strides -------------
        int Nq = a.Nq, Nk = a.Nk;
        const uint16_t* qg;                           // row 0 of this (sequence, head)
        const uint16_t* kg;
        const uint16_t* vg;
        int q_rs = D, kv_rs = D;                      // elements between consecutive rows
        size_t o0 = (size_t)bh * a.Nq * D;            // element offset of this item's output row 0
        int o_rs = D;
        float* lse_g = a.lse + (size_t)bh * a.Nq;
        if constexpr (VARLEN) {
            // Offsets come from the caller's device arrays: a sequence whose offsets
            // leave [0, total], decrease or exceed the declared maximum is skipped,
            // so no access ever leaves the tensors.
            const int b = bh / a.H, hq = bh - b * a.H;
            const int qs = a.cu_q[b], qe = a.cu_q[b + 1], ks0 = a.cu_k[b], ke0 = a.cu_k[b + 1];
            if (qs < 0 || qe < qs || qe > a.total_q || qe - qs > a.max_q) return;
            if (ks0 < 0 || ke0 < ks0 || ke0 > a.total_k || ke0 - ks0 > a.max_k) return;
            Nq = qe - qs;
            Nk = ke0 - ks0;
            if (q0 >= Nq) return;
            const int hk = hq / a.group;
            q_rs = a.H * D;
            kv_rs = a.H_kv * D;
            o_rs = a.H * D;
            qg = a.q + (size_t)qs * q_rs + (size_t)hq * D;
            kg = a.k + (size_t)ks0 * kv_rs + (size_t)hk * D;
            vg = a.v + (size_t)ks0 * kv_rs + (size_t)hk * D;
            o0 = (size_t)qs * o_rs + (size_t)hq * D;
            lse_g = a.lse + (size_t)hq * a.total_q + qs;
        } else {
            // [B, H, N, d] queries; keys and values [B, H_kv, N, d], query head h
            // reading K/V head h / group (group = 1 without grouped heads)
            const int bkv = a.group == 1 ? bh : (bh / a.H) * a.H_kv + (bh % a.H) / a.group;
            qg = a.q + (size_t)bh * a.Nq * D;
            kg = a.k + (size_t)bkv * a.Nk * D;
            vg = a.v + (size_t)bkv * a.Nk * D;
        }
        const int kv_rowb = kv_rs * 2;                // bytes between consecutive K/V rows

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
        const int l32 = lane & 31;
        const int h = lane >> 5;
        const int qw = q0 + 32 * w;
        const int qi = qw + l32;
        const int off = Nk - Nq;                      // causal: key j visible iff j <= i + off

        int ks = 0, ke = Nk;
        if (SPLIT) {
            ks = min(Nk, split * a.split_chunk);
            ke = min(Nk, ks + a.split_chunk);
        }
        int hi = ke;
        if (CAUSAL) hi = min(hi, min(Nq, q0 + BR) - 1 + off + 1);
        const int n_tiles = hi > ks ? (hi - ks + BC - 1) / BC : 0;

        // ---- Q fragments, resident for the whole key loop ----------------------
        // Every load is issued before any is used (rows past Nq read the last row
        // and are zeroed afterwards), so the item waits for memory once; a load
        // inside the row check made each one wait for the previous.
        u32x4 qf[NS];
        {
            const uint16_t* qrow = qg + (size_t)min(qi, Nq - 1) * q_rs + 8 * h;
    #pragma unroll
            for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4*)(qrow + 16 * s);
        }

        // ---- K/V tiles: buffer loads straight into LDS ---------------------------
        // One wave instruction fills 1 KiB of LDS, lane i landing at byte 16*i.  Lane
        // i therefore fetches the global chunk that the swizzled layout stores at
        // that position (global rows are kv_rowb bytes apart); these offsets do not
        // change from tile to tile.  Reads past the sequence's last key return zeros
        // (the descriptor's record count ends with that key's row).
        constexpr int NPW = TILE / 1024 / NW;        // 1 KiB loads per wave per tensor per tile
        u32 voff[NPW];
    #pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int pos = (w * NPW + u) * 1024 + lane * 16;
            const int row = pos / ROWB, pchunk = (pos % ROWB) >> 4;
            voff[u] = (u32)(row * kv_rowb + ((pchunk ^ swz<D>(row)) << 4));
        }
        // which = 0 loads the K tile of `tile` into the stage, 1 its V tile
        auto load_half = [&](int tile, unsigned char* stage, int which) {
            const int k0 = ks + tile * BC;
            const u32 nrec = (u32)(min(Nk - k0, BC) - 1) * kv_rowb + ROWB;
            const __amdgpu_buffer_rsrc_t r = buffer_rsrc((which ? vg : kg) + (size_t)k0 * kv_rs, nrec);
            unsigned char* dst = stage + which * TILE + w * NPW * 1024;
    #pragma unroll
            for (int u = 0; u < NPW; ++u) lds_dma16(r, dst + u * 1024, voff[u]);
        };
        auto load_half_if = [&](int tile, unsigned char* stage, int which, bool on) {
            const int k0 = ks + tile * BC;
            const u32 nrec = on ? (u32)(min(Nk - k0, BC) - 1) * kv_rowb + ROWB : 0u;
            const __amdgpu_buffer_rsrc_t r = buffer_rsrc((which ? vg : kg) + (size_t)k0 * kv_rs, nrec);
            unsigned char* dst = stage + which * TILE + w * NPW * 1024;
    #pragma unroll
            for (int u = 0; u < NPW; ++u) lds_dma16(r, dst + u * 1024, voff[u]);
        };
        auto load_tile = [&](int tile, unsigned char* stage) {
            load_half(tile, stage, 0);
            load_half(tile, stage, 1);
        };

        f32x16 oacc[ND];
    #pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
        float Mu = -INFINITY;   // exponent reference (log2 units of scaled scores)
        float lsum = 0.f;       // this lane's half of the row sum, relative to Mu

        // per-lane LDS byte offsets of the operand reads (rows differing in bits
        // 4-5 share a swizzle, so the 32-key block and 16-key group only add constants)
        const int krow0 = perm_row(l32);             // K row fed to S^T within a 32-key block
        int koff[NS];
    #pragma unroll
        for (int s = 0; s < NS; ++s) koff[s] = lds_off<D>(krow0, 2 * s + h);
        const int r4 = (lane & 15) >> 2, c4 = lane & 3, g1 = (lane >> 4) & 1;
        int voffs[2][ND];
    #pragma unroll
        for (int half = 0; half < 2; ++half)
    #pragma unroll
            for (int db = 0; db < ND; ++db)
                voffs[half][db] = lds_off<D>(8 * h + r4 + 4 * half, 4 * db + 2 * g1 + (c4 >> 1)) + (c4 & 1) * 8;

        // One key tile: S^T = K Q^T, online softmax update, O^T += V^T P^T.
        // MASKED tiles cross the chunk end or (causal) the diagonal.  after_s runs
        // once the S^T products are issued.
        // Fully visible tile, exponentiated one 32-key block at a time against the
        // current reference: block kb is kept when every lane's partial sum of its
        // 16 weights stays <= 2^12 (so every weight does) and the reference is set;
        // otherwise the reference moves to the block's exact running maximum (O and
        // l rescaled first) and the block is exponentiated again.  Rescaling between
        // blocks is the online-softmax merge itself, so no row maximum is needed
        // while the reference holds.
        // masked blocks: register r of block kb holds key k0 + 8h + kofs(kb, r) and
        // is visible iff kofs < bound; a hidden key weighs exactly 0 (also when the
        // scale is 0, where its score times the scale is not defined)
        auto kofs = [](int kb, int r) { return 32 * kb + 16 * (r >> 3) + (r & 7); };
        auto expo16 = [&](const f32x16& sc, float* pv, float& t0, float& t1, auto masked_tag, int kb, int bound) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const float Mg = (Mu == -INFINITY) ? 0.f : Mu;
            t0 = 0.f;
            t1 = 0.f;
    #pragma unroll
            for (int r = 0; r < 16; r += 2) {
                pv[r] = exp2_fast(__builtin_fmaf(sc[r], a.c, -Mg));
                pv[r + 1] = exp2_fast(__builtin_fmaf(sc[r + 1], a.c, -Mg));
                if constexpr (MASKED) {
                    if (kofs(kb, r) >= bound) pv[r] = 0.f;
                    if (kofs(kb, r + 1) >= bound) pv[r + 1] = 0.f;
                }
                t0 += pv[r];
                t1 += pv[r + 1];
            }
        };
        auto guard = [&](const f32x16& sc, float* pv, float& t0, float& t1, auto masked_tag, int kb, int bound) {
            if (__ballot(!(t0 + t1 <= SUM_CAP) || Mu == -INFINITY)) {
                float mx = sc[0];
    #pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmax_raw(mx, sc[r]);
                mx = max_halves(mx);
                const float Mn = fmaxf(Mu, (mx == -INFINITY) ? -INFINITY : mx * a.c);
                const float alpha = (Mn == -INFINITY) ? 1.f : exp2_fast(Mu - Mn);
                lsum *= alpha;
    #pragma unroll
                for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
                Mu = Mn;
                expo16(sc, pv, t0, t1, masked_tag, kb, bound);
            }
            lsum += t0 + t1;
        };
        auto pack16 = [&](const float* pv, u32x4* pb) {
    #pragma unroll
            for (int p = 0; p < 2; ++p)
                pb[p] = u32x4{pack2<BF16>(pv[8 * p + 0], pv[8 * p + 1]), pack2<BF16>(pv[8 * p + 2], pv[8 * p + 3]),
                              pack2<BF16>(pv[8 * p + 4], pv[8 * p + 5]), pack2<BF16>(pv[8 * p + 6], pv[8 * p + 7])};
        };
        auto pv_block = [&](const unsigned char* Vb, int kb, const u32x4* pb) {
    #pragma unroll
            for (int p = 0; p < 2; ++p) {
                const unsigned char* vb = Vb + (32 * kb + 16 * p) * ROWB;
    #pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lds_read_tr16(vb + voffs[0][db]));
                    const u32x2 h2 = __builtin_bit_cast(u32x2, lds_read_tr16(vb + voffs[1][db]));
                    oacc[db] = mfma32<BF16>(u32x4{l2[0], l2[1], h2[0], h2[1]}, pb[p], oacc[db]);
                }
            }
        };
        // One fully visible key tile.  Block 1's S^T products are issued between
        // block 0's softmax instructions and block 0's P V products between block
        // 1's, so the wave's own vector work runs while the matrix core is busy.
        // MASKED tiles cross the chunk end or (causal) the diagonal; their hidden
        // scores are set to -inf (so a fallback's row maximum ignores them) and their
        // weights to 0.
        auto key_tile = [&](const unsigned char* Kb, const unsigned char* Vb, int k0, auto masked_tag,
                            auto&& after_s) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            int bound = 0;
            if constexpr (MASKED) {
                bound = ke - k0 - 8 * h;
                if (CAUSAL) bound = min(bound, qi + off - k0 - 8 * h + 1);
            }
            auto hide = [&](f32x16& sc, int kb) {
                if constexpr (MASKED)
    #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kofs(kb, r) >= bound) sc[r] = -INFINITY;
            };
            f32x16 s0 = f32x16{}, s1 = f32x16{};
    #pragma unroll
            for (int s = 0; s < NS; ++s)
                s0 = mfma32<BF16>(*(const u32x4*)(Kb + koff[s]), qf[s], s0);
            after_s();
    #pragma unroll
            for (int s = 0; s < NS; ++s)
                s1 = mfma32<BF16>(*(const u32x4*)(Kb + 32 * ROWB + koff[s]), qf[s], s1);
            hide(s0, 0);
            float p0[16], t0, t1;
            expo16(s0, p0, t0, t1, masked_tag, 0, bound);
    #pragma unroll
            for (int s = 0; s < NS; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA (block 0)
            }
            __builtin_amdgcn_sched_group_barrier(0x010, 4, 0);       // the next tile's V loads
    #pragma unroll
            for (int s = 0; s < NS; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA (block 1)
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // block 0's softmax
            }
            guard(s0, p0, t0, t1, masked_tag, 0, bound);
            u32x4 pb0[2];
            pack16(p0, pb0);
            pv_block(Vb, 0, pb0);
            hide(s1, 1);
            float p1[16], u0, u1;
            expo16(s1, p1, u0, u1, masked_tag, 1, bound);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);       // V reads of the first two products
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);       // block 0's packing
    #pragma unroll
            for (int s = 0; s < 2 * ND; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // one MFMA (block 0's P V)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);   // V reads one product ahead
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);   // block 1's softmax
            }
            guard(s1, p1, u0, u1, masked_tag, 1, bound);
            u32x4 pb1[2];
            pack16(p1, pb1);
            pv_block(Vb, 1, pb1);
        };

        // Tiles are walked from the last one down.  The first n_masked of them may
        // cross the key-chunk end or the causal diagonal for some wave; all later
        // ones are fully visible to every row of the workgroup.
        int n_masked = 0;
        while (n_masked < n_tiles) {
            const int k0 = ks + (n_tiles - 1 - n_masked) * BC;
            const bool clean = k0 + BC <= ke && (!CAUSAL || k0 + BC - 1 <= q0 + off);
            if (clean) break;
            ++n_masked;
        }
        const int qmax_w = min(qw + 31, Nq - 1);
        if (n_tiles > 0) load_tile(n_tiles - 1, stage0);
        // the Q sign flip (and the zero rows) only now, so that the Q loads and the
        // first tile's loads are in flight together
        const bool qin = qi < Nq;
    #pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = qin ? (qf[s] ^ a.qsign) : u32x4{0, 0, 0, 0};
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // masked tiles: per-wave visibility checks, two per trip so that each step
        // reads one fixed stage (with the stage chosen at run time the compiler
        // cannot tell the stage being read from the one being filled, and waits
        // for the next tile's loads in the middle of the step)
        int it = 0;
        auto masked_step = [&](unsigned char* cur, unsigned char* nxt) {
            const int tile = n_tiles - 1 - it;
            if (it + 1 < n_tiles) load_tile(tile - 1, nxt);
            const int k0 = ks + tile * BC;
            const bool active = qw < Nq && (!CAUSAL || k0 <= qmax_w + off);
            if (active) key_tile(cur, cur + TILE, k0, std::true_type{}, [] {});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ++it;
        };
    #pragma clang loop unroll(disable)
        while (it < n_masked) {
            masked_step(stage0, stage1);
            if (it < n_masked) masked_step(stage1, stage0);
        }
        // clean tiles, two per trip so that each half reads one fixed stage.  The
        // next tile's K loads go out at the start of the step and its V loads after
        // the S^T products: one burst of all of a workgroup's loads would queue in
        // the CU's address unit and stall every wave at the step start.
        auto clean_step = [&](unsigned char* cur, unsigned char* nxt) {
            const int tile = n_tiles - 1 - it;
            const bool more = it + 1 < n_tiles;
            if (more) load_half(tile - 1, nxt, 0);
            // the V loads sit inside one scheduling region with the products, so they
            // are issued without a branch (no records: nothing is read past the last tile)
            key_tile(cur, cur + TILE, ks + tile * BC, std::false_type{},
                     [&] { load_half_if(more ? tile - 1 : 0, nxt, 1, more); });
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ++it;
        };
        if ((it & 1) && it < n_tiles) clean_step(stage1, stage0);
    #pragma clang loop unroll(disable)
        while (it < n_tiles) {
            clean_step(stage0, stage1);
            if (it < n_tiles) clean_step(stage1, stage0);
        }

        // ---- epilogue -------------------------------------------------------------
        const float lt = sum_halves(lsum);
        const float inv = (lt == 0.f || lt != lt) ? 1.f : 1.f / lt;
        const float lse_v = (lt == 0.f) ? -INFINITY : (Mu + log2f(lt)) * kLn2;
        if (qi < Nq) {
            if constexpr (SPLIT) {
                float* op = (float*)a.o + (((size_t)split * a.BH + bh) * a.Nq + qi) * D;
    #pragma unroll
                for (int db = 0; db < ND; ++db)
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v4 = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                          oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
                        *(f32x4*)(op + 32 * db + 8 * g + 4 * h) = v4;
                    }
                if (h == 0) a.lse[((size_t)split * a.BH + bh) * a.Nq + qi] = lse_v;
            } else {
                if (h == 0) lse_g[qi] = lse_v;
            }
        }
        if constexpr (!SPLIT) {
            // O leaves through LDS: the wave's 32 x D tile is written in the MFMA
            // layout (8 bytes per lane per block, 16-byte chunks XOR-swizzled by
            // row) into its own 32-row region of the idle stages, then read back
            // one 16-byte chunk per lane so that each store covers whole rows.
            // The last tile ended with a barrier, so no wave still reads the
            // stages; each wave touches only its own region.
            constexpr int CH = ROWB / 16;                // 16-byte chunks per row
            constexpr int RPI = 1024 / ROWB;             // rows per 1 KiB wave access
            unsigned char* reg = (w < 4 ? stage0 : stage1) + (w & 3) * (32 * ROWB);
    #pragma unroll
            for (int db = 0; db < ND; ++db)
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2 v2 = {pack2<BF16>(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                                      pack2<BF16>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                    const int c = 4 * db + g;
                    *(u32x2*)(reg + l32 * ROWB + ((c ^ (l32 & (CH - 1))) << 4) + 8 * h) = v2;
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int c = lane % CH;
    #pragma unroll
            for (int it2 = 0; it2 < 32 / RPI; ++it2) {
                const int r = it2 * RPI + lane / CH;
                const u32x4 v4 = *(const u32x4*)(reg + r * ROWB + ((c ^ (r & (CH - 1))) << 4));
                if (qw + r < Nq) *(u32x4*)((uint16_t*)a.o + o0 + (size_t)(qw + r) * o_rs + 8 * c) = v4;
            }
        }
    };

    if (VARLEN && a.paired) {
        // Packed sequences differ in length, so contiguous ranges would leave one
        // XCD with the longest sequence: instead K/V group (b, hk) goes to XCD
        // (b*H_kv + hk) % 8, where its H/H_kv query heads share the L2.  Within a
        // sequence of nb query tiles a workgroup runs tiles nb-1-t and t (equal
        // work per workgroup of a sequence under the causal mask; half as many
        // workgroups past the end of short sequences).
        const int per_group = a.group * ((a.n_qtiles + 1) >> 1);
        const int j = blockIdx.x >> 3, gi = j / per_group, r = j - gi * per_group;
        const int grp = gi * 8 + (blockIdx.x & 7);
        const int hk = grp % a.H_kv;
        // sequences longest first (B <= 64; otherwise in index order): the longest
        // items start first and short ones fill the end of the grid
        const int b = a.B <= 64 ? seq_at_rank(a.cu_q, a.B, grp / a.H_kv) : grp / a.H_kv;
        const int t = r / a.group, bh = b * a.H + hk * a.group + r % a.group;
        const int len = a.cu_q[b + 1] - a.cu_q[b];     // run_item checks the offsets themselves
        const int nb = (len > 0 && len <= a.max_q) ? (len + BR - 1) / BR : 0;
        if (t < ((nb + 1) >> 1)) {
            // the two items run through one copy of the item code (a loop, not two
            // inlined calls), which keeps the kernel small for the instruction cache
    #pragma clang loop unroll(disable)
            for (int r = 0; r < 2; ++r) {
                if (r == 1) {
                    if (t == nb - 1 - t) break;
                    __syncthreads();    // the next item refills stage0
                }
                run_item(r == 0 ? nb - 1 - t : t, bh, 0);
            }
        }
    } else if constexpr (CAUSAL && !VARLEN && !SPLIT) {
        // Causal query tiles t and n_qtiles-1-t together see a fixed number of key
        // tiles, so pairing them gives every workgroup the same work: the
        // round-robin dispatcher then never waits on one XCD's long tile while
        // another XCD has free slots.  (A single query tile is the pair t = 0.)
        const int npairs = (a.n_qtiles + 1) >> 1;
        const int t = L % npairs, bh = L / npairs;
    #pragma clang loop unroll(disable)
        for (int r = 0; r < 2; ++r) {
            if (r == 1) {
                if (t == a.n_qtiles - 1 - t) break;
                __syncthreads();        // the next item refills stage0
            }
            run_item(r == 0 ? a.n_qtiles - 1 - t : t, bh, 0);
        }
    } else {
        const int rest = L / a.n_qtiles;
        run_item(a.n_qtiles - 1 - (L % a.n_qtiles), rest % a.BH, SPLIT ? rest / a.BH : 0);   // heaviest first
    }
}

template <bool BF16, int D, bool CAUSAL, bool SPLIT, bool VARLEN, int NW>
hipError_t launch_t(const FwdArgs& a, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<BF16, D, CAUSAL, SPLIT, VARLEN, NW>), dim3(blocks), dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

// mode: 0 plain [B,H,N,d], 1 split-KV partials, 2 packed variable-length; wide:
// eight wavefronts per workgroup (plain mode only; with the causal mask, d = 128 only)
template <bool BF16, int D>
hipError_t dispatch_cs(const FwdArgs& a, int blocks, bool causal, int mode, bool wide, hipStream_t s) {
    if (causal) {
        if (mode == 1) return launch_t<BF16, D, true, true, false, 4>(a, blocks, s);
        if (mode == 2) return launch_t<BF16, D, true, false, true, 4>(a, blocks, s);
        if constexpr (D == 128)
            if (wide) return launch_t<BF16, D, true, false, false, 8>(a, blocks, s);
        return launch_t<BF16, D, true, false, false, 4>(a, blocks, s);
    }
    if (mode == 1) return launch_t<BF16, D, false, true, false, 4>(a, blocks, s);
    if (mode == 2) return launch_t<BF16, D, false, false, true, 4>(a, blocks, s);
    if (wide) return launch_t<BF16, D, false, false, false, 8>(a, blocks, s);
    return launch_t<BF16, D, false, false, false, 4>(a, blocks, s);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
    FwdArgs a;
    a.q = (const uint16_t*)p.q;
    a.k = (const uint16_t*)p.k;
    a.v = (const uint16_t*)p.v;
    a.o = p.o;
    a.lse = p.lse;
    a.B = p.B;
    a.H = p.H;
    a.Nq = p.Nq;
    a.Nk = p.Nk;
    a.BH = p.B * p.H;
    a.c = fabsf(p.scale) * kLog2e;
    a.qsign = p.scale < 0.f ? 0x80008000u : 0u;
    const bool split = p.num_splits > 0;
    const int mode = p.varlen ? 2 : (split ? 1 : 0);
    // Each workgroup loads every K/V tile it attends to once for its query rows,
    // so 256 query rows per workgroup (eight wavefronts, one workgroup per CU)
    // halve the K/V traffic into LDS, with half as many workgroups (wide_rows).  At
    // d = 64, where the softmax bounds the kernel, the wider form wins 3-6% without
    // the mask whenever the grid fills the 256 CUs; with the mask it gained at most
    // 3% and lost up to a third on smaller grids, so there it is not used.
    const int64_t wb = wide_blocks(p.Nq, (int64_t)p.B * p.H, p.causal);
    const bool wide = mode == 0 && (p.d == 128 ? wide_rows(wb, p.Nk, 2048) : (!p.causal && wb >= 256));
    const int BR = wide ? 256 : 128;
    a.n_qtiles = (p.Nq + BR - 1) / BR;        // varlen: Nq is the longest query sequence
    const int S = split ? p.num_splits : 1;
    a.split_chunk = split_chunk(p.Nk, S);
    a.cu_q = p.cu_q;
    a.cu_k = p.cu_k;
    a.H_kv = p.H_kv > 0 ? p.H_kv : p.H;
    a.group = p.H / a.H_kv;
    a.total_q = p.total_q;
    a.total_k = p.total_k;
    a.max_q = p.Nq;
    a.max_k = p.Nk;
    // causal [B,H,N,d]: one workgroup per pair of query tiles (two pairs per
    // workgroup, one dispatch round with no rebalancing, measured slower)
    a.paired = (p.causal && mode == 0) || (mode == 2 && (a.B * a.H_kv) % 8 == 0);
    const int64_t blocks = a.paired ? (int64_t)((a.n_qtiles + 1) / 2) * a.BH : (int64_t)a.n_qtiles * a.BH * S;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (p.d == 128)
        return p.bf16 ? dispatch_cs<true, 128>(a, (int)blocks, p.causal, mode, wide, stream)
                      : dispatch_cs<false, 128>(a, (int)blocks, p.causal, mode, wide, stream);
    return p.bf16 ? dispatch_cs<true, 64>(a, (int)blocks, p.causal, mode, wide, stream)
                  : dispatch_cs<false, 64>(a, (int)blocks, p.causal, mode, wide, stream);
}

}  // namespace fa
