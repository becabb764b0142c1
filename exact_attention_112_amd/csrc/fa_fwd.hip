// fa_fwd.hip -- attention forward pass for gfx950 (AMD Instinct MI355X).
//
// Computes O = softmax(scale * Q K^T [causal]) V and the per-row log-sum-exp,
// tile by tile with the online softmax, so the N x N score matrix never
// leaves the compute unit.  Method sources (pages cited by site:
// [nanhubrain] = nanhubrain.csdn.net, FlashAttention in CANN ops-transformer;
// [ascendai] = ascendai.csdn.net, efficient attention in CANN ops-nn;
// [pwwt] = www.pwwt.cn/news/2518640):
//   * [nanhubrain] "tiling skeleton": query tiles outer, key/value tiles inner;
//     scores of one tile pair exist only on chip; after the inner loop the
//     accumulator is normalised by the row sum once and written once.
//   * [nanhubrain] "online softmax mathematics" and [ascendai] 2.2: running row
//     max m and row sum l; when m grows, the previous sum and accumulator are
//     rescaled by exp(m_old - m_new), which is exact.
//   * [ascendai] 3.2 (kernel): causal key blocks that lie entirely after the
//     query block are skipped; [ascendai] 6.1: inside a block straddling the
//     diagonal, key j is visible to query i iff j <= i.
//   * [ascendai] 6.2/7.2 and [pwwt] "key differences" (third difference):
//     accumulate in fp32.
//
// gfx950 design (the pages' Cube/Vector/UB design targets another machine;
// only the method carries over):
//   * one workgroup = NW wavefronts x 32 queries; grid over (batch*head,
//     query tile), remapped so the tiles of one head run on one XCD (L2);
//   * Q fragment held in VGPRs for the whole loop;
//   * K and V tiles of 64 keys go HBM -> LDS directly (global_load_lds, 16
//     bytes a lane), two LDS stages each, rows XOR-swizzled in 16-byte units
//     against bank conflicts;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulate): a lane owns
//     one query column, so the row max / row sum are in-lane plus one swap of
//     the two 32-lane halves (v_permlane32_swap);
//   * software pipeline inside each wave, its instruction order fixed by
//     hand: while the matrix core computes the scores of key tile j+1, the
//     vector ALU turns the scores of tile j into probabilities; while it
//     computes O += P_j V_j, the vector ALU takes the row max of tile j+1;
//     LDS fragments are read three MFMAs ahead.  Two waves per SIMD fill
//     each other's gaps;
//   * P stays in registers: rounded to bf16 (RNE, v_cvt_pk_bf16_f32) and fed as
//     the B operand of O^T = V^T P^T; V^T fragments come straight from the
//     row-major LDS tile through ds_read_b64_tr_b16 (transposing LDS read);
//   * exp2 with scale*log2(e) folded into one FMA; the running max moves
//     only when a tile's max exceeds it by more than 2^4 in p, which makes
//     rescaling the accumulator rare; the normaliser of O carries the bf16
//     rounding error of each tile's largest p, so a row that one key
//     dominates still gets exactly that key's V row;
//   * epilogue: O = acc / l in fp32 (or bf16), LSE = (m2 + log2 l) * ln 2.
// A plain fp32 kernel (v_mfma_f32_32x32x2f32, P kept in fp32) serves fp32
// inputs; there the running max moves only when a tile's max exceeds it by
// more than 2^8 (exact: numerator and denominator share the stale max), which
// makes rescaling the accumulator rare.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <algorithm>
#include <atomic>

#include "fa355.h"
#include "fa_common.h"

namespace fa355 {

// fp32 kernel: the running max moves only when a tile max exceeds it by more
// than this (log2 units); probabilities then stay below 2^8 before the final
// normalisation, which fp32 holds without loss.
constexpr float kLazyRescale = 8.0f;

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    long long q_sb, q_sh, q_sn;   // element strides of Q and O (batch, head, row)
    long long k_sb, k_sh, k_sn;   // element strides of K and V
    int H, Nq, Nk;
    int n_qtiles;                 // ceil(Nq / rows per workgroup)
    int BH;                       // B * H
    float scale_log2;             // scale * log2(e)
    int group;                    // query heads per key/value head (H / Hkv)
    int wl, wr;                   // band: keys i-wl .. i+wr visible (negative: unbounded)
    const unsigned char* block_mask;  // block-sparse: [B*H][n_qb][n_kb], nonzero = computed
    int n_qb, n_kb;               // mask blocks: 256 queries x 64 keys
};

// Variants of the bf16 forward kernel.
enum : int { kPlain = 0, kBand = 1, kSparse = 2 };
constexpr int kMaxSparseTiles = 4096;   // key tiles of 64 a block-sparse launch may list

// ---------------------------------------------------------------------------
// bf16 kernel
//
// D: head dim (64 or 128).  NW: waves per workgroup (32 queries each).
// OUT_BF16: write O as bf16 instead of fp32.
//
// Register layout of one wave (32 queries; lane = (col, hi), col = lane % 32
// is the query, hi = lane / 32 picks half of each 8-key group):
//   S^T tile (two f32x16 per 64 keys): s[kb][r] = score of key
//     kb*32 + (r/4)*8 + hi*4 + r%4 against query col;
//   O^T accumulator: oacc[db][r] = O[col][db*32 + (r/4)*8 + hi*4 + r%4].

template <int D>
struct RowState {
    f32x16 oacc[D / 32];
    float m;          // running max of scale*log2(e)*s (same in both halves), kept
                      // within kLazyMax below the true one
    float l0, l1;     // two partial sums of P over this lane's keys
    float dl;         // sum of bf16(p) - p over the lane's largest score of each tile
    float xl;         // this lane's largest raw score in the tile whose P is next
};

// The running max moves only when a tile's max exceeds it by more than this
// (log2 units), so P lies in [0, 2^kLazyMax] and the accumulator is rescaled
// only a few times per row.  The row's largest key then has p = 2^delta (not
// exactly 1), whose bf16 rounding would leave a relative error of up to 2^-8
// in O for a row that one key dominates; so the normaliser of O adds the
// rounding error of each tile's largest p (dl), which makes that key's weight
// exact again, while the LSE keeps the sum of the unrounded P.
constexpr float kLazyMax = 4.0f;

// S^T = K Q^T for one 64-key tile: 2 x D/16 MFMAs.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const bf16x8 (&qreg)[D / 16],
                                        const u32x4* __restrict__ ks, int col, int hi) {
    constexpr int DCH = D / 8, KK = D / 16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int row = kb * 32 + col;
            const u32x4 kx = ks[row * DCH + k_swz<D>(row, 2 * kk + hi)];
            const f32x16 c = kk == 0 ? f32x16{} : s[kb];
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), qreg[kk], c,
                                                            0, 0, 0);
        }
    }
}

// Keys >= Nk and (causal) keys after the lane's query -> -inf.  The lane's
// key for slot (kb, r) is key0 + hi*4 + [kb*32 + (r/4)*8 + r%4]; it is visible
// iff the bracket is <= lim.
template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int key0, int q, int Nk, int hi) {
    const int lim = (CAUSAL ? min(Nk - 1, q) : Nk - 1) - (key0 + hi * 4);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[kb][r] = (kb * 32 + (r >> 2) * 8 + (r & 3)) <= lim ? s[kb][r] : -INFINITY;
}

// Band mask: key j is visible to this lane's query iff lo <= j <= hi (lane
// constants: lo = i - wl or no bound, hi = min(Nk-1, i + wr, causal ? i)).
__device__ __forceinline__ void mask_tile_band(f32x16 (&s)[2], int key0, int lo, int hi_key, int hi) {
    const int base = key0 + hi * 4;
    const int lo_r = lo - base, hi_r = hi_key - base;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
            s[kb][r] = (off >= lo_r && off <= hi_r) ? s[kb][r] : -INFINITY;
        }
}

// Row max of the tile, scaled to log2 units (the scale is > 0, so the max of
// the scaled scores is the scaled max); -inf if every key of the row is masked.
__device__ __forceinline__ float tile_max_scaled(const f32x16 (&s)[2], float sl2, float& lane_max) {
    // two chains of 3-input maxes (v_max3_f32), 8 each
    float a = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    float b = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
        a = fmaxf(fmaxf(a, s[0][r]), s[0][r + 1]);
        b = fmaxf(fmaxf(b, s[1][r]), s[1][r + 1]);
    }
    lane_max = fmaxf(fmaxf(a, s[0][15]), fmaxf(b, s[1][15]));
    return pair_max(lane_max) * sl2;
}

// P = exp2(s*scale*log2e - m), accumulated into the two row-sum chains and
// packed to bf16 pairs (the B operand of the P V product).  Masked scores are
// -inf and give exactly 0 (the scale is > 0).
__device__ __forceinline__ void tile_exp(const f32x16 (&s)[2], float m, float sl2, unsigned (&pk)[2][8],
                                         float& l0, float& l1) {
    const float nm = -m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * j], sl2, nm));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * j + 1], sl2, nm));
            l0 += e0;
            l1 += e1;
            pk[kb][j] = pack_bf16x2(e0, e1);
        }
}

// The rounding error bf16(p) - p of the lane's largest p in the tile (the p
// that tile_exp computes for the score xl, with the same operations), added
// to the normaliser of O.  -inf (all keys of the lane masked) gives 0.
__device__ __forceinline__ void round_fix(float xl, float m, float sl2, float& dl) {
    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(xl, sl2, -m));
    const float r = __builtin_bit_cast(float, pack_bf16x2(0.0f, e) & 0xffff0000u);
    dl += r - e;
}

// O^T += V^T P^T for one 64-key tile: 4 x D/32 MFMAs.  The lane's P slots
// 0..3 of 16-key group u hold keys 16u + hi*4 + 0..3 and slots 4..7 keys
// 16u + 8 + hi*4 + 0..3; the V^T fragment is read for the same keys.
template <int D>
__device__ __forceinline__ void pv_tile(f32x16 (&oacc)[D / 32], const unsigned (&pk)[2][8],
                                        const lds_char* __restrict__ vs, int tr_row, int tr_dd) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 pb = __builtin_bit_cast(
                bf16x8, (u32x4){pk[kb][4 * u + 0], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]});
            const int r0 = kb * 32 + 16 * u + tr_row;    // keys of P slots 0..3
            const int r1 = r0 + 8;                       // keys of P slots 4..7
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dd = db * 32 + tr_dd;
                const int c = dd >> 3, w = (dd & 7) * 2;
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vs + r0 * (D * 2) + v_swz<D>(r0, c) * 16 + w));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vs + r1 * (D * 2) + v_swz<D>(r1, c) * 16 + w));
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
            }
        }
    }
}

// Take a new tile whose scaled row max is mt2 into the running max.  The
// whole wave moves (every row to its true max, rescaling by alpha =
// exp2(m_old - m_new)) when some row's tile max exceeds its running max by
// more than kLazyMax; otherwise nothing changes.
// SAFE: a row may have seen no visible key yet (m = -inf), so alpha is taken
// as 1 where the max did not move instead of exp2(-inf - -inf).
template <int D, bool SAFE = false>
__device__ __forceinline__ void update_max(RowState<D>& st, float mt2) {
    if (__builtin_amdgcn_ballot_w64(mt2 > st.m + kLazyMax)) {
        // every row of the wave moves to its true max
        const float m_new = fmaxf(mt2, st.m);
        float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
        if constexpr (SAFE) alpha = mt2 > st.m ? alpha : 1.0f;
        st.l0 *= alpha;
        st.l1 *= alpha;
        st.dl *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
        st.m = m_new;
    }
}

// The same step with its instruction order fixed by hand (every group ends
// in a scheduling fence): phase A issues each K fragment read three MFMAs
// ahead of its use and runs one or two exponentials per score MFMA; its last
// three groups already fetch the first V^T fragments; phase B issues each
// V^T fragment three MFMAs ahead, finishes the exponentials and takes the
// row max of tile j+1 in small chunks once its scores have left the matrix
// core.  BOUNDARY: tile j+1 is the first tile of the next query tile (the
// persistent kernel): the running max is left alone and the next tile's
// scaled max is returned.
template <int D, bool BOUNDARY = false>
__device__ __forceinline__ float wave_step_sw(RowState<D>& st, const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                             const bf16x8 (&qreg)[D / 16], const u32x4* __restrict__ ks,
                                             const lds_char* __restrict__ vs, float sl2, int col, int hi,
                                             int tr_row, int tr_dd) {
    constexpr int DCH = D / 8, DB = D / 32;
    constexpr int NA = 2 * (D / 16);      // score MFMAs
    constexpr int NB = 4 * DB;            // P V MFMAs
    // exponentials (32 per lane and tile), element by element: EA of them in
    // phase A (the first EP before its first MFMA, the others spread evenly
    // over its NA groups), the rest over the first GB groups of phase B, each
    // before the P V MFMA that needs it (d = 128: 6 + 16 + 10, about one per
    // score MFMA and one per P V MFMA, so that no group's vector work exceeds
    // what the other wave's MFMA hides)
    constexpr int EA = D == 128 ? 22 : 32;
    constexpr int GB = D == 128 ? 10 : 1;
    constexpr int CPS = NB == 16 ? 1 : 2; // max chunks per P V MFMA
    constexpr int MS = D == 128 ? 4 : 2;   // first group of the max chunks
    auto kread = [&](int i) -> bf16x8 {
        const int kk = i >> 1, kb = i & 1, row = kb * 32 + col;
        return __builtin_bit_cast(bf16x8, ks[row * DCH + k_swz<D>(row, 2 * kk + hi)]);
    };
    auto vread = [&](int i) -> bf16x8 {
        const int kb = i / (2 * DB), u = (i / DB) & 1, db = i % DB;
        const int r0 = kb * 32 + 16 * u + tr_row, r1 = r0 + 8;
        const int dd = db * 32 + tr_dd, c = dd >> 3, w = (dd & 7) * 2;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vs + r0 * (D * 2) + v_swz<D>(r0, c) * 16 + w));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vs + r1 * (D * 2) + v_swz<D>(r1, c) * 16 + w));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    const float nm = -st.m;
    unsigned pk[2][8];
    float ev[32];
    // element e: score s_cur[e / 16][e % 16]; odd elements close a pair
    auto elem = [&](int e) {
        const int b = e >> 4, r = e & 15;
        ev[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[b][r], sl2, nm));
        if (e & 1) {
            st.l1 += ev[e];
            pk[b][r >> 1] = pack_bf16x2(ev[e - 1], ev[e]);
        } else {
            st.l0 += ev[e];
        }
    };
    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int i = 0; i < 3; ++i) kf[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
    // phase A.  The wave raises its issue priority (s_setprio 1) for phase A
    // and the first half of phase B, and drops it after P V MFMA NB/2 - 1:
    // when the two waves of a SIMD are in different phases, the one computing
    // scores and exponentials is served first and the other's P V MFMAs fill
    // in behind it (1.6-2.4 % faster at B4 H32 N8192 d128 than equal
    // priorities; priority only over phase A, or to the end of phase B,
    // gained less, and around each MFMA alone it lost 1 %)
    __builtin_amdgcn_s_setprio(1);
    // EP of phase A's exponentials go before its first MFMA: they need only
    // this tile's scores (in registers), so they fill the wait for the first
    // K fragments after the barrier (0.4-0.65 % faster at B4 H32 N8192 d128
    // than none; 2, 4, 5 or 8 gained as much or less)
    constexpr int EP = 6;
#pragma unroll
    for (int e = 0; e < EP; ++e) elem(e);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        if (i + 3 < NA) kf[(i + 3) & 3] = kread(i + 3);
        else vf[i + 3 - NA] = vread(i + 3 - NA);
        const int kb = i & 1;
        s_nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i & 3], qreg[i >> 1], i < 2 ? f32x16{} : s_nxt[kb],
                                                            0, 0, 0);
#pragma unroll
        for (int e = EP + ((EA - EP) * i) / NA; e < EP + ((EA - EP) * (i + 1)) / NA; ++e) elem(e);
        __builtin_amdgcn_sched_barrier(0);
    }
    // phase B
    float a = 0.f, bm = 0.f, mt2 = 0.f, xl_new = 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (i + 3 < NB) vf[(i + 3) & 3] = vread(i + 3);
        const int kb = i / (2 * DB), u = (i / DB) & 1, db = i % DB;
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, (u32x4){pk[kb][4 * u + 0], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]});
        st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 3], pb, st.oacc[db], 0, 0, 0);
        if (i < GB) {
#pragma unroll
            for (int e = EA + ((32 - EA) * i) / GB; e < EA + ((32 - EA) * (i + 1)) / GB; ++e) elem(e);
        }
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc) {
            const int c = (i - MS) * CPS + cc;   // max chunk 0..7
            if (i >= MS && c == 0) {
                a = fmaxf(fmaxf(s_nxt[0][0], s_nxt[0][1]), s_nxt[0][2]);
                bm = fmaxf(fmaxf(s_nxt[1][0], s_nxt[1][1]), s_nxt[1][2]);
            } else if (i >= MS && c >= 1 && c <= 6) {
                a = fmaxf(fmaxf(a, s_nxt[0][2 * c + 1]), s_nxt[0][2 * c + 2]);
                bm = fmaxf(fmaxf(bm, s_nxt[1][2 * c + 1]), s_nxt[1][2 * c + 2]);
            } else if (i >= MS && c == 7) {
                xl_new = fmaxf(fmaxf(a, s_nxt[0][15]), fmaxf(bm, s_nxt[1][15]));
            }
        }
        if (i == MS + 8 / CPS) mt2 = pair_max(xl_new) * sl2;
        if (i == MS + 1 + 8 / CPS) round_fix(st.xl, st.m, sl2, st.dl);
        if (i == NB / 2 - 1) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    }
    st.xl = xl_new;
    if constexpr (BOUNDARY) return mt2;   // s_nxt starts the next query tile: no rescale
    update_max(st, mt2);
    return 0.f;
}

// The same step without the overlap, for the few masked tiles at the end:
// P_j and O += P_j V_j from the scores in s, then (HAS_NXT) the scores of
// tile j+1, masked, into the same registers, and the max update.  Half the
// score registers of wave_step.
template <int D, bool CAUSAL, bool HAS_NXT>
__device__ __forceinline__ void wave_step_serial(RowState<D>& st, f32x16 (&s)[2], const bf16x8 (&qreg)[D / 16],
                                                 const u32x4* ks_nxt, const lds_char* vs_cur, int key0_nxt, int q,
                                                 int Nk, float sl2, int col, int hi, int tr_row, int tr_dd) {
    unsigned pk[2][8];
    tile_exp(s, st.m, sl2, pk, st.l0, st.l1);
    round_fix(st.xl, st.m, sl2, st.dl);
    pv_tile<D>(st.oacc, pk, vs_cur, tr_row, tr_dd);
    if constexpr (HAS_NXT) {
        qk_tile<D>(s, qreg, ks_nxt, col, hi);
        mask_tile<CAUSAL>(s, key0_nxt, q, Nk, hi);
        update_max(st, tile_max_scaled(s, sl2, st.xl));
    }
}

// The serial step under a band: rows may have no visible key so far (m =
// -inf), so the exponent uses a finite stand-in for m (every score of such a
// row is -inf and still gives 0) and the max update is the safe one.
template <int D, bool HAS_NXT>
__device__ __forceinline__ void wave_step_band(RowState<D>& st, f32x16 (&s)[2], const bf16x8 (&qreg)[D / 16],
                                               const u32x4* ks_nxt, const lds_char* vs_cur, int key0_nxt, int lo,
                                               int hi_key, float sl2, int col, int hi, int tr_row, int tr_dd) {
    unsigned pk[2][8];
    const float m_fin = fmaxf(st.m, -3.0e38f);
    tile_exp(s, m_fin, sl2, pk, st.l0, st.l1);
    round_fix(st.xl, m_fin, sl2, st.dl);
    pv_tile<D>(st.oacc, pk, vs_cur, tr_row, tr_dd);
    if constexpr (HAS_NXT) {
        qk_tile<D>(s, qreg, ks_nxt, col, hi);
        mask_tile_band(s, key0_nxt, lo, hi_key, hi);
        update_max<D, true>(st, tile_max_scaled(s, sl2, st.xl));
    }
}

template <int D, int NW>
struct Bf16Cfg {
    static constexpr int BC = 64;                 // keys per tile
    static constexpr int BR = NW * 32;            // queries per workgroup
    static constexpr int DCH = D / 8;             // 16-byte chunks per row
    static constexpr int TILE_CH = BC * DCH;      // chunks per K (or V) tile
    static constexpr int TILE_BYTES = TILE_CH * 16;
    static constexpr int LPW = TILE_CH / 64 / NW; // direct-to-LDS loads per wave per operand
    static_assert(TILE_CH % (64 * NW) == 0, "tile must split evenly over the waves");
};

// MODE kBand: keys outside the band i-wl .. i+wr are masked and the tiles
// outside the workgroup's band are never loaded.  MODE kSparse: the key
// tiles a block mask marks off for the workgroup's 256 queries are never
// loaded; the workgroup runs over the sorted list of the others.  In both,
// rows may see no key at all (O = 0, LSE = -inf).
template <int D, int NW, bool CAUSAL, bool OUT_BF16, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(FwdParams p) {
    constexpr bool BAND = MODE == kBand, SPARSE = MODE == kSparse, SAFE = MODE != kPlain;
    using C = Bf16Cfg<D, NW>;
    constexpr int BC = C::BC, BR = C::BR, DCH = C::DCH, TILE_CH = C::TILE_CH, TB = C::TILE_BYTES;
    constexpr int LPW = C::LPW, KK = D / 16, DB = D / 32;

    // LDS: K stages 0, 1, V stages 0, 1 ([TILE_CH] 16-byte chunks each) and,
    // block-sparse, the list of key tiles and its length, in one LDS array
    // (with a second LDS variable the compiler makes every read of a tile
    // wait for the loads in flight into the other stage)
    constexpr int LIST_CH = SPARSE ? kMaxSparseTiles * 2 / 16 + 1 : 0;
    __shared__ u32x4 smem[4 * TILE_CH + LIST_CH];
    unsigned short* const tile_list = reinterpret_cast<unsigned short*>(smem + 4 * TILE_CH);
    int* const list_len = reinterpret_cast<int*>(tile_list + kMaxSparseTiles);

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int col = lane & 31;
    const int hi = lane >> 5;

    int bh, qt;
    // long causal sequences: one head at a time per XCD (32 CUs each)
    tile_of_block(__builtin_amdgcn_workgroup_id_x(), p.n_qtiles, p.BH, CAUSAL, bh, qt, p.n_qtiles >= 32);
    const int b = bh / p.H;
    const int h = bh - b * p.H;

    const int q_wg0 = qt * BR;
    const int q_w0 = q_wg0 + wave * 32;   // first query of this wave
    const int q = q_w0 + col;             // this lane's query
    const int Nq = p.Nq, Nk = p.Nk;

    const int hk = h / p.group;           // key/value head of this query head
    const __bf16* qbase = (const __bf16*)p.q + (long long)b * p.q_sb + (long long)h * p.q_sh;
    const char* kbase = (const char*)((const __bf16*)p.k + (long long)b * p.k_sb + (long long)hk * p.k_sh);
    const char* vbase = (const char*)((const __bf16*)p.v + (long long)b * p.k_sb + (long long)hk * p.k_sh);
    const long long row_bytes = p.k_sn * 2;

    // Key tiles this workgroup needs: [t_begin, n_kt).  Tiles [t_full_lo,
    // n_full) need no mask for any wave (every key < Nk and, causal, <= the
    // workgroup's first query; band: inside every row's band); the rest are
    // masked, and a wave skips the tiles past its last visible key (causal,
    // band) or all of them if its rows are all padding.
    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q_wg0 + BR, Nq));
    int n_kt = (kv_end + BC - 1) / BC;
    int n_full = Nk / BC;
    if (CAUSAL) n_full = min(n_full, (q_wg0 + 1) / BC);
    n_full = min(n_full, n_kt);
    // (padding waves, q_w0 >= Nq, run like the others: their Q rows are zero
    // and their results are not stored)
    int n_kt_wave = CAUSAL ? min(n_kt, (q_w0 + 31) / BC + 1) : n_kt;
    int t_begin = 0, t_full_lo = 0;
    // band limits of this lane's query (visible keys lo_key .. hi_key)
    int lo_key = 0, hi_key = 0;
    if constexpr (BAND) {
        const int big = 1 << 30;
        const int q_last = min(q_wg0 + BR, Nq) - 1;
        const int wl = p.wl, wr = p.wr;
        int key_lo = wl >= 0 ? max(0, q_wg0 - wl) : 0;          // first key any row sees
        int key_hi = min(Nk - 1, wr >= 0 ? q_last + wr : big);  // last key any row sees
        if (CAUSAL) key_hi = min(key_hi, q_last);
        // tiles every row of the workgroup sees whole
        int x_hi = min(Nk - 1, wr >= 0 ? q_wg0 + wr : big);
        if (CAUSAL) x_hi = min(x_hi, q_wg0);
        const int full_lo = wl >= 0 ? max(0, (q_last - wl + BC - 1) / BC) : 0;
        if (key_lo > key_hi) {
            t_begin = n_kt = n_full = t_full_lo = 0;           // no row sees any key
        } else {
            t_begin = key_lo / BC;
            n_kt = key_hi / BC + 1;
            t_full_lo = min(n_kt, max(t_begin, full_lo));
            n_full = max(t_full_lo, min(n_kt, (x_hi + 1) / BC));
        }
        int w_hi = min(Nk - 1, wr >= 0 ? q_w0 + 31 + wr : big);
        if (CAUSAL) w_hi = min(w_hi, q_w0 + 31);
        n_kt_wave = min(n_kt, w_hi / BC + 1);
        lo_key = wl >= 0 ? q - wl : -big;
        hi_key = min(Nk - 1, wr >= 0 ? q + wr : big);
        if (CAUSAL) hi_key = min(hi_key, q);
    }
    // ---- Q fragment (B operand of S^T = K Q^T): lane holds Q[q][16kk + 8hi .. +7]
    // (loaded before the block-sparse list is built, so the two latencies overlap)
    bf16x8 qreg[KK];
    {
        const bool ok = q < Nq;
        const __bf16* qrow = qbase + (long long)(ok ? q : 0) * p.q_sn + hi * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 x = ok ? *(const u32x4*)(qrow + kk * 16) : (u32x4){0u, 0u, 0u, 0u};
            qreg[kk] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // Block-sparse: the workgroup walks the sorted list of its unmasked-off
    // tiles; "tile" v below is then list entry v.  The tiles a wave or the
    // whole workgroup sees in full are a prefix of the list (the list is
    // sorted and only the diagonal / last tiles need a mask).
    if constexpr (SPARSE) {
        const unsigned char* mrow = p.block_mask + ((long long)bh * p.n_qb + qt) * p.n_kb;
        if (wave == 0) {
            const int count = build_list(tile_list, n_kt, lane, [&](int t) { return mrow[t] != 0 ? 1u : 0u; });
            if (lane == 0) *list_len = count;
        }
        __syncthreads();
        const int n_list = *list_len;
        int v_full = 0, v_wave = 0;
        for (int base = 0; base < n_list; base += 64) {
            const int v = base + lane;
            const int t = v < n_list ? (int)tile_list[v] : (1 << 30);
            v_full += __builtin_popcountll(__builtin_amdgcn_ballot_w64(t < n_full));
            v_wave += __builtin_popcountll(__builtin_amdgcn_ballot_w64(t < n_kt_wave));
        }
        n_kt = n_list;
        n_full = v_full;
        n_kt_wave = v_wave;
        lo_key = -(1 << 30);
        hi_key = CAUSAL ? min(Nk - 1, q) : Nk - 1;
    }
#define FA_TILE(v) (SPARSE ? (int)tile_list[(v)] : (v))

    // ---- direct HBM -> LDS staging (buffer_load ... lds, 16 bytes a lane).
    // Each wave instruction writes 64 consecutive 16-byte LDS chunks: RPW
    // whole rows of the tile.  Lane i fills physical chunk i % DCH of its row,
    // so it fetches the logical chunk (i % DCH) ^ swz(row) (the swizzles are
    // XORs, their own inverse).  The buffer descriptor is rebased on each
    // tile (scalar), the lane offset is fixed.  A tile that runs past Nk
    // reads row Nk-1 in place of the missing rows: their scores are masked,
    // and the V rows stay finite.
    const unsigned rb = (unsigned)row_bytes;
    unsigned ld_koff, ld_voff;   // byte offsets inside a tile (load round 0)
    {
        const int row = wave * (64 / DCH) + lane / DCH, ch = lane % DCH;
        ld_koff = row * rb + k_swz<D>(row, ch) * 16;
        ld_voff = row * rb + v_swz<D>(row, ch) * 16;
    }
    lds_char* const lds = (lds_char*)smem;
    const unsigned long long kaddr = to_sgpr((unsigned long long)kbase);
    const unsigned long long vaddr = to_sgpr((unsigned long long)vbase);
    const unsigned long long tile_bytes = (unsigned long long)BC * (unsigned long long)row_bytes;
    lds_char* const ldst = lds + wave * 1024;   // this wave's rows of load round 0 in a stage
    // tile t lives in stage (t - t_begin) % 2 (t_begin = 0 without a band)
#define FA_K_STAGE(t) (lds + (((t) - t_begin) & 1) * TB)
#define FA_V_STAGE(t) (lds + (2 + (((t) - t_begin) & 1)) * TB)
#define FA_ISSUE_K(t) issue_tile<LPW, DCH, BC, NW>(kaddr + (unsigned long long)FA_TILE(t) * tile_bytes, rb, \
                                              ld_koff, ldst + (((t) - t_begin) & 1) * TB, Nk - FA_TILE(t) * BC, \
                                              wave, lane)
#define FA_ISSUE_V(t) issue_tile<LPW, DCH, BC, NW>(vaddr + (unsigned long long)FA_TILE(t) * tile_bytes, rb, \
                                              ld_voff, ldst + (2 + (((t) - t_begin) & 1)) * TB,              \
                                              Nk - FA_TILE(t) * BC, wave, lane)

    RowState<D> st;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.f;
    st.m = -INFINITY;
    st.l0 = 0.f;
    st.l1 = 0.f;
    st.dl = 0.f;
    st.xl = -INFINITY;
    const float sl2 = p.scale_log2;

    // V^T fragment addressing for ds_read_b64_tr_b16: within each 16-lane
    // group, lane 4r+c fetches 4 consecutive d values of key row r; lane i
    // then receives column i (one d value) of the 4 rows.
    const int tg = lane >> 4, ti = lane & 15;
    const int tr_row = hi * 4 + (ti >> 2);            // key offset inside an 8-key group
    const int tr_dd = 16 * (tg & 1) + 4 * (ti & 3);   // d offset inside a 32-wide d block

    // Pipeline.  K tile t lives in K stage t%2, V tile t in V stage t%2.
    // Step j (top: K tile j+1 and V tile j have landed for every wave, and
    // every wave is done with step j-1) first refills the stages step j-1
    // read: K tile j+2 and V tile j+1; then computes P_j, O += P_j V_j and
    // the scores of tile j+1.
    f32x16 sa[2], sb[2];   // scores of the current / next tile (roles alternate)
    if (!SAFE || n_kt > 0) {
        FA_ISSUE_K(t_begin);
        FA_ISSUE_V(t_begin);
        if (t_begin + 1 < n_kt) FA_ISSUE_K(t_begin + 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        // Scores of the first tile.  Without a band every row (padding rows
        // included: their Q is zero) sees key 0, so the first max is finite.
        qk_tile<D>(sa, qreg, (const u32x4*)FA_K_STAGE(t_begin), col, hi);
        if constexpr (SAFE) {
            if (t_begin < t_full_lo || t_begin >= n_full)
                mask_tile_band(sa, FA_TILE(t_begin) * BC, lo_key, hi_key, hi);
        } else {
            if (n_full == 0) mask_tile<CAUSAL>(sa, 0, q, Nk, hi);
        }
        st.m = tile_max_scaled(sa, sl2, st.xl);
    }

#define FA_TOP(j)                                      \
    do {                                               \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); \
        __syncthreads();                               \
        if ((j) + 2 < n_kt) FA_ISSUE_K((j) + 2);       \
        if ((j) + 1 < n_kt) FA_ISSUE_V((j) + 1);       \
    } while (0)
#define FA_KS(t) ((const u32x4*)FA_K_STAGE(t))

    int j = t_begin;
    if constexpr (BAND) {
        // Masked first tiles (the band's left edge), serial, until tile j
        // itself is whole for every row, so every row has seen a key (finite
        // running max) before the pipelined step, which has no stand-in for
        // a max of -inf, forms its P; then one more serial step if needed so
        // the pipelined loop starts on stage 0.
        for (; j < t_full_lo && j + 1 < n_kt; ++j) {
            FA_TOP(j);
            wave_step_band<D, true>(st, sa, qreg, FA_KS(j + 1), FA_V_STAGE(j), (j + 1) * BC, lo_key, hi_key, sl2,
                                    col, hi, tr_row, tr_dd);
        }
        if (((j - t_begin) & 1) && j + 1 < n_full) {
            FA_TOP(j);
            wave_step_band<D, true>(st, sa, qreg, FA_KS(j + 1), FA_V_STAGE(j), (j + 1) * BC, lo_key, hi_key, sl2,
                                    col, hi, tr_row, tr_dd);
            ++j;
        }
    }
    // Steps whose tiles j and j+1 are both unmasked, two at a time so the
    // score buffers swap roles without copies.
    for (; j + 2 < n_full; j += 2) {
        FA_TOP(j);
        wave_step_sw<D>(st, sa, sb, qreg, FA_KS(j + 1), FA_V_STAGE(j), sl2, col, hi, tr_row, tr_dd);
        FA_TOP(j + 1);
        wave_step_sw<D>(st, sb, sa, qreg, FA_KS(j + 2), FA_V_STAGE(j + 1), sl2, col, hi, tr_row, tr_dd);
    }
    // The remaining steps (at most a few): masks on, per-wave skips, no
    // overlap (one score buffer).
    for (; j < n_kt; ++j) {
        FA_TOP(j);
        if (j < n_kt_wave) {
            if constexpr (SAFE) {
                if (j + 1 < n_kt_wave)
                    wave_step_band<D, true>(st, sa, qreg, FA_KS(j + 1), FA_V_STAGE(j), FA_TILE(j + 1) * BC, lo_key,
                                            hi_key, sl2, col, hi, tr_row, tr_dd);
                else
                    wave_step_band<D, false>(st, sa, qreg, nullptr, FA_V_STAGE(j), 0, lo_key, hi_key, sl2, col, hi,
                                             tr_row, tr_dd);
            } else {
                if (j + 1 < n_kt_wave)
                    wave_step_serial<D, CAUSAL, true>(st, sa, qreg, FA_KS(j + 1), FA_V_STAGE(j), (j + 1) * BC, q, Nk,
                                                      sl2, col, hi, tr_row, tr_dd);
                else
                    wave_step_serial<D, CAUSAL, false>(st, sa, qreg, nullptr, FA_V_STAGE(j), 0, q, Nk, sl2, col, hi,
                                                       tr_row, tr_dd);
            }
        }
    }

#undef FA_K_STAGE
#undef FA_V_STAGE
#undef FA_ISSUE_K
#undef FA_ISSUE_V
#undef FA_TOP
#undef FA_KS
#undef FA_TILE

    // ---- epilogue
    const float l_tot = pair_sum(st.l0 + st.l1);
    const float dl_tot = pair_sum(st.dl);
    // the lane's half, recomputed (mbcnt) rather than kept live through the loops
    const int hi_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
    {
        // (band: a row that saw no key has l = 0 and gets O = 0, LSE = -inf)
        const float inv = (!SAFE || l_tot > 0.f) ? 1.0f / (l_tot + dl_tot) : 0.f;
        const long long orow0 = (long long)b * p.q_sb + (long long)h * p.q_sh + (long long)q_w0 * p.q_sn;
        store_acc_rows<D, OUT_BF16, 0>(st.oacc, inv, (char*)p.o + orow0 * (OUT_BF16 ? 2 : 4), p.q_sn, Nq - q_w0,
                                  col, hi_e);
    }
    if (q < Nq) {
        if (p.lse && hi_e == 0)
            p.lse[(long long)bh * Nq + q] = (!SAFE || l_tot > 0.f) ? (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2
                                                                   : -INFINITY;
    }
}


// ---------------------------------------------------------------------------
// Persistent form of the plain non-causal kernel, for Nk a multiple of 128
// (every key tile whole, an even number of them).
//
// gridDim.x workgroups (a multiple of 8, about one per CU) each take the
// query tiles bid, bid + G, bid + 2G, ... of the ordinary kernel's
// workgroup order (so an XCD keeps the heads tile_of_block gives it) and run
// their key tiles as one stream: the loads issued at the top of a query
// tile's last two steps already fetch the next query tile's Q (into an LDS
// buffer) and its first K and V tiles, and its last step computes the next
// query tile's first scores while it finishes P V of its own last tile.  A
// query tile thus starts without waiting for its Q or its first tiles, and
// ends without a serial step; O and LSE are stored between the two.
template <int D, int NW, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_persist(FwdParams p, int n_items) {
    using C = Bf16Cfg<D, NW>;
    constexpr int BC = C::BC, BR = C::BR, DCH = C::DCH, TILE_CH = C::TILE_CH, TB = C::TILE_BYTES;
    constexpr int LPW = C::LPW, KK = D / 16, DB = D / 32;
    constexpr int Q_CH = BR * DCH, LPQ = Q_CH / 64 / NW;   // the Q tile in LDS, loads per wave
    static_assert(Q_CH % (64 * NW) == 0, "Q tile must split evenly over the waves");

    // LDS: K stages 0, 1, V stages 0, 1, then the Q tile (one LDS array)
    __shared__ u32x4 smem[4 * TILE_CH + Q_CH];
    lds_char* const lds = (lds_char*)smem;
    lds_char* const qbuf = lds + 4 * TB;

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hi = lane >> 5;
    const int G = __builtin_amdgcn_readfirstlane((int)gridDim.x);
    const int Nq = p.Nq, Nk = p.Nk;
    const int n_kt = Nk / BC;                     // even, >= 2
    const unsigned rb = (unsigned)(p.k_sn * 2);   // K/V row bytes
    const unsigned qrb = (unsigned)(p.q_sn * 2);  // Q/O row bytes (in elements x 2)
    const int my_row = wave * 32 + col;           // this lane's query row in the tile

    // the query tile of work item `it` (a workgroup id of the ordinary kernel):
    // its (batch, head) and first row; addresses are formed when needed
    struct Item {
        int bh, q0;
    };
    auto item_of = [&](int it) {
        Item r;
        int qt;
        tile_of_block(it, p.n_qtiles, p.BH, false, r.bh, qt);
        r.q0 = qt * BR;
        return r;
    };
    const unsigned long long v_minus_k =
        (unsigned long long)((const char*)p.v - (const char*)p.k);   // V's offset from K (same strides)
    auto k_addr = [&](const Item& it) {
        const int b = it.bh / p.H, h = it.bh - b * p.H, hk = h / p.group;
        return to_sgpr((unsigned long long)((const __bf16*)p.k + (long long)b * p.k_sb + (long long)hk * p.k_sh));
    };
    auto q_addr = [&](const Item& it) {
        const int b = it.bh / p.H, h = it.bh - b * p.H;
        return to_sgpr((unsigned long long)((const __bf16*)p.q + (long long)b * p.q_sb + (long long)h * p.q_sh +
                                            (long long)it.q0 * p.q_sn));
    };

    unsigned ld_koff, ld_voff, ld_qoff;   // byte offsets inside a tile (load round 0)
    {
        const int row = wave * (64 / DCH) + lane / DCH, ch = lane % DCH;
        ld_koff = row * rb + k_swz<D>(row, ch) * 16;
        ld_voff = row * rb + v_swz<D>(row, ch) * 16;
        ld_qoff = row * qrb + k_swz<D>(row, ch) * 16;
    }
    const unsigned long long tile_bytes = (unsigned long long)BC * rb;
    lds_char* const ldst = lds + wave * 1024;         // this wave's rows of load round 0 in a stage
    lds_char* const ldq = qbuf + wave * 1024;
#define FA_K_STAGE(t) (lds + ((t) & 1) * TB)
#define FA_V_STAGE(t) (lds + (2 + ((t) & 1)) * TB)
// (kb: the K base of the query tile's head, a scalar; V is at kb + v_minus_k)
#define FA_ISSUE_K(kb, t) issue_tile<LPW, DCH, BC, NW>((kb) + (unsigned long long)(t) * tile_bytes, rb, ld_koff, \
                                                       ldst + ((t) & 1) * TB, BC, wave, lane)
#define FA_ISSUE_V(kb, t) issue_tile<LPW, DCH, BC, NW>((kb) + v_minus_k + (unsigned long long)(t) * tile_bytes, rb, \
                                                       ld_voff, ldst + (2 + ((t) & 1)) * TB, BC, wave, lane)
#define FA_ISSUE_Q(qb, q0) issue_tile<LPQ, DCH, BR, NW>((qb), qrb, ld_qoff, ldq, Nq - (q0), wave, lane)
    const int tg = lane >> 4, ti = lane & 15;
    const int tr_row = hi * 4 + (ti >> 2);
    const int tr_dd = 16 * (tg & 1) + 4 * (ti & 3);
    const float sl2 = p.scale_log2;

    // Q fragment of this lane's row from the LDS Q tile (rows past Nq hold
    // copies of row Nq-1: finite, not stored)
    bf16x8 qreg[KK];
    auto load_q = [&]() {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qreg[kk] = __builtin_bit_cast(
                bf16x8, *(const u32x4*)(qbuf + my_row * (D * 2) + k_swz<D>(my_row, 2 * kk + hi) * 16));
    };
    RowState<D> st;
    auto reset = [&](float m) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.f;
        st.m = m;
        st.l0 = 0.f;
        st.l1 = 0.f;
        st.dl = 0.f;
    };
    // O = acc / (l + dl) and LSE of the finished query tile
    auto store_out = [&](const Item& it) {
        const float l_tot = pair_sum(st.l0 + st.l1);
        const float dl_tot = pair_sum(st.dl);
        const int hi_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
        const int q_w0 = it.q0 + wave * 32;
        const int q = q_w0 + col;
        {
            const float inv = 1.0f / (l_tot + dl_tot);
            const int b = it.bh / p.H, h = it.bh - b * p.H;
            const long long orow0 = (long long)b * p.q_sb + (long long)h * p.q_sh + (long long)q_w0 * p.q_sn;
            store_acc_rows<D, OUT_BF16, 1>(st.oacc, inv, (char*)p.o + orow0 * (OUT_BF16 ? 2 : 4), p.q_sn, Nq - q_w0,
                                      col, hi_e);
        }
        if (q < Nq && p.lse && hi_e == 0)
            p.lse[(long long)it.bh * Nq + q] = (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2;
    };

    int item = __builtin_amdgcn_workgroup_id_x();
    if (item >= n_items) return;                  // (the host launches at most n_items workgroups)
    Item cur = item_of(item);
    unsigned long long k_cur = k_addr(cur);
    f32x16 sa[2], sb[2];
    // the first query tile: Q, K tiles 0 and 1, V tile 0, then its first scores
    FA_ISSUE_Q(q_addr(cur), cur.q0);
    FA_ISSUE_K(k_cur, 0);
    FA_ISSUE_V(k_cur, 0);
    FA_ISSUE_K(k_cur, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    load_q();
    qk_tile<D>(sa, qreg, (const u32x4*)FA_K_STAGE(0), col, hi);
    st.xl = -INFINITY;
    reset(tile_max_scaled(sa, sl2, st.xl));

    // every wave's wait for its own tile loads sits at the end of the step
    // before a top (the first top of a query tile: after the O stores)
#define FA_WAIT_LOADS() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")
    for (;;) {
        const int nxt = item + G;
        const bool has_nxt = nxt < n_items;
        const Item next = item_of(has_nxt ? nxt : item);
        const unsigned long long k_nxt = k_addr(next), q_nxt = q_addr(next);
        // Step j (top: K tile j+1 and V tile j have landed for every wave,
        // and every wave is done with step j-1) refills the stages step j-1
        // read (K tile j+2, V tile j+1, of this query tile or the next);
        // then computes P_j, O += P_j V_j and the scores of tile j+1.
#define FA_TOP(j)                                                                  \
    do {                                                                           \
        __syncthreads();                                                           \
        if ((j) + 2 < n_kt) FA_ISSUE_K(k_cur, (j) + 2);                            \
        else if (has_nxt) FA_ISSUE_K(k_nxt, (j) + 2 - n_kt);                       \
        if ((j) + 1 < n_kt) FA_ISSUE_V(k_cur, (j) + 1);                            \
        else if (has_nxt) FA_ISSUE_V(k_nxt, 0);                                    \
        if ((j) + 2 == n_kt && has_nxt) FA_ISSUE_Q(q_nxt, next.q0);               \
    } while (0)
        // (n_kt is even, so inside the loop every tile to load is this query tile's)
#define FA_TOP_IN(j)                                      \
    do {                                                  \
        __syncthreads();                                  \
        FA_ISSUE_K(k_cur, (j) + 2);                       \
        FA_ISSUE_V(k_cur, (j) + 1);                       \
    } while (0)
        int j = 0;
        for (; j + 2 < n_kt; j += 2) {
            FA_TOP_IN(j);
            wave_step_sw<D>(st, sa, sb, qreg, (const u32x4*)FA_K_STAGE(j + 1), FA_V_STAGE(j), sl2, col, hi,
                            tr_row, tr_dd);
            FA_WAIT_LOADS();
            FA_TOP_IN(j + 1);
            wave_step_sw<D>(st, sb, sa, qreg, (const u32x4*)FA_K_STAGE(j + 2), FA_V_STAGE(j + 1), sl2, col, hi,
                            tr_row, tr_dd);
            FA_WAIT_LOADS();
        }
#undef FA_TOP_IN
        // j = n_kt - 2: P_j and the scores of the last tile (the Q loads
        // into the LDS buffer are safe: every wave read its fragment of this
        // query tile before its first barrier)
        FA_TOP(j);
        wave_step_sw<D>(st, sa, sb, qreg, (const u32x4*)FA_K_STAGE(j + 1), FA_V_STAGE(j), sl2, col, hi, tr_row,
                        tr_dd);
        FA_WAIT_LOADS();
        ++j;
        // j = n_kt - 1: P of the last tile; the next query tile's Q and its
        // K tile 0 landed at this top
        FA_TOP(j);
        float m_next = 0.f;
        if (!has_nxt) {
            wave_step_serial<D, false, false>(st, sb, qreg, nullptr, FA_V_STAGE(j), 0, 0, Nk, sl2, col, hi, tr_row,
                                              tr_dd);
        } else {
            load_q();
            m_next = wave_step_sw<D, true>(st, sb, sa, qreg, (const u32x4*)FA_K_STAGE(0), FA_V_STAGE(j), sl2, col,
                                           hi, tr_row, tr_dd);
        }
        store_out(cur);
        if (!has_nxt) break;
        // the next query tile's first top needs K tile 1 and V tile 0, whose
        // loads were issued before this wave's O stores: vector memory
        // counts return in issue order, so after a full tile (D/8 stores)
        // the wait lets the stores stay in flight
        if (cur.q0 + wave * 32 + 32 <= Nq) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D / 8) : "memory");
        else FA_WAIT_LOADS();
        // the Q fragments again, so that they hold no registers during the
        // stores (the empty asm keeps the compiler from reusing the first read)
        asm volatile("" ::: "memory");
        load_q();
        reset(m_next);
        item = nxt;
        cur = next;
        k_cur = k_nxt;
#undef FA_TOP
    }
#undef FA_K_STAGE
#undef FA_V_STAGE
#undef FA_ISSUE_K
#undef FA_ISSUE_V
#undef FA_ISSUE_Q
#undef FA_WAIT_LOADS
}

// ---------------------------------------------------------------------------
// Short-key kernel (bf16, at most 32*NKB <= 128 keys, no band or block mask).
//
// With this few keys a query row costs little arithmetic and the pass is
// bound by HBM: reading Q and writing O.  All of the head's K and V sit in
// LDS, loaded once per workgroup; the 4 waves of a workgroup then stream
// query tiles of 32 rows (T each, the waves' tiles side by side), and each
// row's softmax is taken over all its keys at once (one max, one sum, no
// rescaling).  A wave's Q tile comes in one tile ahead through direct-to-LDS
// loads that cover whole rows (two stages per wave, no barriers); its O tile
// goes out through the stage it has just read, so every store instruction
// also writes whole rows (whole 128-byte lines).
// two workgroups of the kernel fit a CU's 160 KB of LDS (else one: one wave per SIMD)
template <int D, int NKB>
constexpr int KVB_FITS_TWICE = 2 * (2 * NKB * 32 * D * 2 + 4 * 2 * 32 * D * 2) <= 160 * 1024 ? 1 : 0;

template <int D, int NKB, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1 + KVB_FITS_TWICE<D, NKB>)))
void fa_fwd_short_kernel(FwdParams p, int T, int chunks) {
    constexpr int NWS = 4, DCH = D / 8, KK = D / 16, DB = D / 32, NK = NKB * 32;
    constexpr int QTB = 32 * D * 2;              // one Q tile (bytes) = one pass of the O tile
    constexpr int KVB = NK * D * 2;              // the head's K (or V), rows past Nk zero
    constexpr int RPI = 64 / DCH;                // rows one load instruction covers
    constexpr int ES = OUT_BF16 ? 2 : 4;         // bytes per O element
    constexpr int NPASS = ES / 2;                // O tile passes through one stage
    constexpr int DP = D / NPASS;                // d values per pass
    __shared__ __attribute__((aligned(16))) char smem[2 * KVB + NWS * 2 * QTB];

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hi = lane >> 5;
    const int bid = __builtin_amdgcn_workgroup_id_x();
    const int bh = bid / chunks;
    const int chunk = bid - bh * chunks;
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    const int Nq = p.Nq, Nk = p.Nk;

    lds_char* const ks = (lds_char*)smem;
    lds_char* const vs = ks + KVB;
    lds_char* const qst = vs + KVB + wave * 2 * QTB;    // this wave's two stages

    // K and V of the KV head into LDS (rows past Nk zero): K swizzled for the
    // 32-row ds_read_b128, V for the transposing reads
    {
        const long long kvoff = (long long)b * p.k_sb + (long long)(h / p.group) * p.k_sh;
        const __bf16* kg = (const __bf16*)p.k + kvoff;
        const __bf16* vg = (const __bf16*)p.v + kvoff;
#pragma unroll
        for (int e = tid; e < NK * DCH; e += NWS * 64) {
            const int row = e / DCH, ch = e % DCH;
            u32x4 kx = (u32x4){0u, 0u, 0u, 0u}, vx = kx;
            if (row < Nk) {
                kx = *(const u32x4*)(kg + (long long)row * p.k_sn + ch * 8);
                vx = *(const u32x4*)(vg + (long long)row * p.k_sn + ch * 8);
            }
            *(u32x4*)(ks + (row * DCH + k_swz<D>(row, ch)) * 16) = kx;
            *(u32x4*)(vs + (row * DCH + v_swz<D>(row, ch)) * 16) = vx;
        }
    }

    // this wave's query tiles: rows row0(it) .. +31, it = 0 .. T-1
    const int wg_row0 = chunk * (T * NWS * 32);
    auto tile_row0 = [&](int it) { return wg_row0 + (it * NWS + wave) * 32; };
    const long long qoff = (long long)b * p.q_sb + (long long)h * p.q_sh;
    const unsigned qrb = (unsigned)(p.q_sn * 2);
    // Q tile `it` into stage `st`: instruction j, lane l -> row j*RPI + l/DCH,
    // LDS chunk l%DCH (holding logical chunk (l%DCH) ^ swizzle); rows past Nq
    // are outside the buffer's range and read as zero
    auto issue_q = [&](int it, int st) {
        const int r0 = tile_row0(it);
        const int nvalid = max(0, min(32, Nq - r0));
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)to_sgpr((unsigned long long)((const __bf16*)p.q + qoff + (long long)min(r0, Nq - 1) * p.q_sn)),
            (short)0, (int)(nvalid * qrb), 0x00020000);
#pragma unroll
        for (int j = 0; j < 32 / RPI; ++j) {
            const int row = j * RPI + lane / DCH;
            const int lch = (lane % DCH) ^ (k_swz<D>(row, 0));   // logical chunk landing at LDS chunk lane%DCH
            load_lds16(rsrc, qst + st * QTB + j * 1024, (unsigned)(row * qrb + lch * 16), 0u);
        }
    };
    if (tile_row0(0) < Nq) issue_q(0, 0);
    __syncthreads();    // K and V in LDS

    const float sl2 = p.scale_log2;
    const int tg = lane >> 4, ti = lane & 15;
    const int tr_row = hi * 4 + (ti >> 2);
    const int tr_dd = 16 * (tg & 1) + 4 * (ti & 3);
    const long long o_row_bytes = p.q_sn * ES;

    for (int it = 0; it < T; ++it) {
        const int r0 = tile_row0(it);
        if (r0 >= Nq) break;                                   // whole wave
        const int st = it & 1;
        lds_char* const stg = qst + st * QTB;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // Q tile `it` landed, earlier stores done
        bf16x8 qreg[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qreg[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(stg + (col * DCH + k_swz<D>(col, 2 * kk + hi)) * 16));
        // the other stage was last read by the previous tile's O stores
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (it + 1 < T && tile_row0(it + 1) < Nq) issue_q(it + 1, st ^ 1);

        // S^T = K Q^T over all keys
        f32x16 s[NKB];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int row = kb * 32 + col;
                const u32x4 kx = *(const u32x4*)(ks + (row * DCH + k_swz<D>(row, 2 * kk + hi)) * 16);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), qreg[kk],
                                                                kk == 0 ? f32x16{} : s[kb], 0, 0, 0);
            }
        // keys past Nk and (causal) after the row's query -> -inf; every row
        // sees key 0, so its max is finite
        const int q = r0 + col;
        const int lim = (CAUSAL ? min(Nk - 1, q) : Nk - 1) - hi * 4;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = (kb * 32 + (r >> 2) * 8 + (r & 3)) <= lim ? s[kb][r] : -INFINITY;
                mx = fmaxf(mx, s[kb][r]);
            }
        const float m2 = pair_max(mx) * sl2;
        float l0 = 0.f, l1 = 0.f;
        unsigned pk[NKB][8];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * jj], sl2, -m2));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * jj + 1], sl2, -m2));
                l0 += e0;
                l1 += e1;
                pk[kb][jj] = pack_bf16x2(e0, e1);
            }
        const float l_tot = pair_sum(l0 + l1);
        // O^T = V^T P^T
        f32x16 oacc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8 pb = __builtin_bit_cast(
                    bf16x8, (u32x4){pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]});
                const int ra = kb * 32 + 16 * u + tr_row, rb = ra + 8;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int dd = db * 32 + tr_dd;
                    const int c = dd >> 3, w = (dd & 7) * 2;
                    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(vs + ra * (D * 2) + v_swz<D>(ra, c) * 16 + w));
                    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(vs + rb * (D * 2) + v_swz<D>(rb, c) * 16 + w));
                    const bf16x8 va =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
                }
            }

        // O = acc / l through the stage just read, NPASS passes of DP d values:
        // each lane writes its row's pieces (16-byte chunks XOR-swizzled by
        // row), then each store instruction takes 64/(D/8) whole pass-rows
        const float inv = 1.0f / l_tot;
        char* const obase = (char*)p.o + qoff * ES;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            if (ps > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // previous pass read back
#pragma unroll
            for (int db = ps * (DB / NPASS); db < (ps + 1) * (DB / NPASS); ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int dl = db * 32 + g * 8 + hi * 4 - ps * DP;      // first of 4 d values, in the pass
                    const int byte = dl * ES;
                    const int phys = (byte >> 4) ^ (col % DCH);
                    lds_char* dst = stg + col * (DP * ES) + phys * 16 + (byte & 15);
                    if constexpr (OUT_BF16) {
                        *(u32x2*)dst = (u32x2){pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                                               pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                    } else {
                        *(float4*)dst = make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                                    oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                    }
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int j = 0; j < 32 / RPI; ++j) {
                const int row = j * RPI + lane / DCH, c = lane % DCH;
                const u32x4 x = *(const u32x4*)(stg + row * (DP * ES) + ((c ^ (row % DCH)) * 16));
                if (r0 + row < Nq)
                    *(u32x4*)(obase + (long long)(r0 + row) * o_row_bytes + ps * (DP * ES) + c * 16) = x;
            }
        }
        if (p.lse && hi == 0 && q < Nq)
            p.lse[(long long)bh * Nq + q] = (m2 + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same method, v_mfma_f32_32x32x2f32, P kept in fp32, one
// 32-key tile per iteration, single-buffered padded LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_f32_kernel(FwdParams p) {
    constexpr int NW = 4, BR = NW * 32, BC = 32, NT = NW * 64;
    constexpr int LD = D + 1;            // padded LDS row (floats)
    constexpr int DB = D / 32;
    constexpr int C4 = D / 4;            // float4 chunks per row

    __shared__ float ks[BC * LD];
    __shared__ float vs[BC * LD];

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int hi = lane >> 5;

    int bh, qt;
    tile_of_block(__builtin_amdgcn_workgroup_id_x(), p.n_qtiles, p.BH, CAUSAL, bh, qt);
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    const int q_wg0 = qt * BR;
    const int q_w0 = q_wg0 + wave * 32;
    const int q = q_w0 + col;
    const int Nq = p.Nq, Nk = p.Nk;

    const float* qbase = (const float*)p.q + (long long)b * p.q_sb + (long long)h * p.q_sh;
    const float* kbase = (const float*)p.k + (long long)b * p.k_sb + (long long)h * p.k_sh;
    const float* vbase = (const float*)p.v + (long long)b * p.k_sb + (long long)h * p.k_sh;

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q_wg0 + BR, Nq));
    const int n_kt = (kv_end + BC - 1) / BC;

    // Q fragment: lane holds Q[q][2kk + hi]
    float qreg[D / 2];
    {
        const bool ok = q < Nq;
        const float* qrow = qbase + (long long)(ok ? q : 0) * p.q_sn;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) qreg[kk] = ok ? qrow[2 * kk + hi] : 0.f;
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int key0 = kt * BC;
        __syncthreads();   // previous tile fully consumed
        for (int idx = tid; idx < BC * C4; idx += NT) {
            const int row = idx / C4, c4 = idx - row * C4;
            const int key = key0 + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < Nk) {
                const long long off = (long long)key * p.k_sn + c4 * 4;
                kx = *(const float4*)(kbase + off);
                vx = *(const float4*)(vbase + off);
            }
            float* kd = ks + row * LD + c4 * 4;
            float* vd = vs + row * LD + c4 * 4;
            kd[0] = kx.x; kd[1] = kx.y; kd[2] = kx.z; kd[3] = kx.w;
            vd[0] = vx.x; vd[1] = vx.y; vd[2] = vx.z; vd[3] = vx.w;
        }
        __syncthreads();
        if (q_w0 >= Nq || (CAUSAL && key0 > q_w0 + 31)) continue;

        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[col * LD + 2 * kk + hi], qreg[kk], sacc, 0, 0, 0);

        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = key0 + (r >> 2) * 8 + hi * 4 + (r & 3);
            const bool ok = key < Nk && (!CAUSAL || key <= q);
            sacc[r] = ok ? sacc[r] : -INFINITY;
            mx = fmaxf(mx, sacc[r]);
        }
        mx = pair_max(mx);
        const float mt2 = (mx == -INFINITY) ? -INFINITY : mx * sl2;
        const bool move = mt2 > m_run + kLazyRescale;
        const float m_new = move ? mt2 : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        if (__builtin_amdgcn_ballot_w64(move)) {
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        m_run = m_new;

        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -m_new));
            pv[r] = (sacc[r] == -INFINITY) ? 0.f : e;
            l_run += pv[r];
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = (r >> 2) * 8 + hi * 4 + (r & 3);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * LD + db * 32 + col], pv[r],
                                                                 oacc[db], 0, 0, 0);
            }
    }

    const float l_tot = pair_sum(l_run);
    if (q < Nq) {
        const float inv = 1.0f / l_tot;
        float* obase = (float*)p.o + (long long)b * p.q_sb + (long long)h * p.q_sh + (long long)q * p.q_sn;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dd = db * 32 + g * 8 + hi * 4;
                *(float4*)(obase + dd) = make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                                     oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
            }
        if (p.lse && hi == 0)
            p.lse[(long long)bh * Nq + q] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

}  // namespace fa355

// ---------------------------------------------------------------------------
// C ABI

using namespace fa355;

namespace {

#ifndef FA_PERSIST
#define FA_PERSIST 1
#endif
#ifndef FA_WAVES_BF16
#define FA_WAVES_BF16 8
#endif
constexpr int kWavesBf16 = FA_WAVES_BF16;   // queries per workgroup = 32 * waves
constexpr int kWavesF32 = 4;
// A block-sparse mask row covers one workgroup's queries and a mask column
// one key tile: the public granularity must match the kernel's tiling.
static_assert(32 * kWavesBf16 == FA_SPARSE_BQ, "block-mask rows must be the bf16 kernel's query tiles");
static_assert(Bf16Cfg<128, kWavesBf16>::BC == FA_SPARSE_BK, "block-mask columns must be the bf16 kernel's key tiles");

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_bf16(const FwdParams& p, int grid, int mode, hipStream_t s) {
    if (mode == kBand)
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, kWavesBf16, CAUSAL, OUT_BF16, kBand>), dim3(grid),
                           dim3(kWavesBf16 * 64), 0, s, p);
    else if (mode == kSparse)
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, kWavesBf16, CAUSAL, OUT_BF16, kSparse>), dim3(grid),
                           dim3(kWavesBf16 * 64), 0, s, p);
    else
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, kWavesBf16, CAUSAL, OUT_BF16, kPlain>), dim3(grid),
                           dim3(kWavesBf16 * 64), 0, s, p);
    return hipGetLastError();
}

// Persistent non-causal kernel: `grid` workgroups over n_items query tiles.
template <int D, bool OUT_BF16>
hipError_t launch_persist(const FwdParams& p, int grid, int n_items, hipStream_t s) {
    hipLaunchKernelGGL((fa_fwd_bf16_persist<D, kWavesBf16, OUT_BF16>), dim3(grid), dim3(kWavesBf16 * 64), 0, s, p,
                       n_items);
    return hipGetLastError();
}

// CUs of the current device (cached per device; 0 if unknown).
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Short-key kernel: NKB = ceil(Nk / 32) blocks of 32 keys.
#ifndef FA_SHORT_WG_TARGET
#define FA_SHORT_WG_TARGET 512
#endif
constexpr long long kShortWgTarget = FA_SHORT_WG_TARGET;   // workgroups to aim for: one resident round
template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_short(const FwdParams& p, int nkb, int grid, int T, int chunks, hipStream_t s) {
    switch (nkb) {
    case 1: hipLaunchKernelGGL((fa_fwd_short_kernel<D, 1, CAUSAL, OUT_BF16>), dim3(grid), dim3(256), 0, s, p, T, chunks); break;
    case 2: hipLaunchKernelGGL((fa_fwd_short_kernel<D, 2, CAUSAL, OUT_BF16>), dim3(grid), dim3(256), 0, s, p, T, chunks); break;
    case 3: hipLaunchKernelGGL((fa_fwd_short_kernel<D, 3, CAUSAL, OUT_BF16>), dim3(grid), dim3(256), 0, s, p, T, chunks); break;
    default: hipLaunchKernelGGL((fa_fwd_short_kernel<D, 4, CAUSAL, OUT_BF16>), dim3(grid), dim3(256), 0, s, p, T, chunks); break;
    }
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL>), dim3(grid), dim3(kWavesF32 * 64), 0, s, p);
    return hipGetLastError();
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

}  // namespace

extern "C" int fa_abi_version(void) { return FA355_ABI_VERSION; }

extern "C" const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        default: return "FA_UNKNOWN_STATUS";
    }
}

namespace {

fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, const unsigned char* block_mask,
                   int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window_left,
                   int window_right, int layout, int in_dtype, int o_dtype, void* stream) {
    // ---- validation: no HIP call before it passes
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (layout != FA_BHND && layout != FA_BSND) return FA_ERR_INVALID_ARG;
    if (in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_INVALID_ARG;
    if (o_dtype != FA_BF16 && o_dtype != FA_F32) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
    if (scale != scale || fabsf(scale) == INFINITY) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (in_dtype == FA_F32 && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
    // a band edge beyond every key masks nothing: such an edge is unbounded
    // (the same result; it also keeps every key index the kernels form within
    // int range)
    if (Nq >= (1 << 30) || Nk >= (1 << 30)) return FA_ERR_UNSUPPORTED;
    if (window_left >= Nq) window_left = -1;      // i - wl < 0 for every query i
    if (window_right >= Nk) window_right = -1;    // i + wr >= Nk - 1 for every query
    const bool band = window_left >= 0 || window_right >= 0;
    // the fp32 kernel serves plain attention only
    if (in_dtype == FA_F32 && (band || Hkv != H || block_mask)) return FA_ERR_UNSUPPORTED;
    if (block_mask && (band || (Nk + 63) / 64 > kMaxSparseTiles)) return FA_ERR_UNSUPPORTED;
    const int mode = block_mask ? kSparse : band ? kBand : kPlain;

    const int rows_per_wg = 32 * (in_dtype == FA_BF16 ? kWavesBf16 : kWavesF32);
    const long long n_qtiles = ((long long)Nq + rows_per_wg - 1) / rows_per_wg;
    const long long grid = n_qtiles * B * H;
    if ((long long)B * H > INT32_MAX || grid > INT32_MAX) return FA_ERR_UNSUPPORTED;
    // the bf16 kernel addresses a 64-row key tile with 32-bit byte offsets
    // (and row offsets with 24-bit multiplies)
    const long long kv_row_bytes = (layout == FA_BSND ? (long long)Hkv * d : (long long)d) * 2;
    if (in_dtype == FA_BF16 && 64 * kv_row_bytes >= (1LL << 30)) return FA_ERR_UNSUPPORTED;

    if (scale < 0.f) scale = 1.0f / sqrtf((float)d);

    FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    const long long D = d;
    if (layout == FA_BHND) {
        p.q_sb = (long long)H * Nq * D; p.q_sh = (long long)Nq * D; p.q_sn = D;
        p.k_sb = (long long)Hkv * Nk * D; p.k_sh = (long long)Nk * D; p.k_sn = D;
    } else {
        p.q_sb = (long long)Nq * H * D; p.q_sh = D; p.q_sn = (long long)H * D;
        p.k_sb = (long long)Nk * Hkv * D; p.k_sh = D; p.k_sn = (long long)Hkv * D;
    }
    p.H = H; p.Nq = Nq; p.Nk = Nk;
    p.n_qtiles = (int)n_qtiles;
    p.BH = B * H;
    p.group = H / Hkv;
    p.wl = window_left < 0 ? -1 : window_left;
    p.wr = window_right < 0 ? -1 : window_right;
    p.block_mask = block_mask;
    p.n_qb = (Nq + FA_SPARSE_BQ - 1) / FA_SPARSE_BQ;   // mask rows (= the kernel's query tiles)
    p.n_kb = (Nk + FA_SPARSE_BK - 1) / FA_SPARSE_BK;   // mask columns (= its key tiles)
    // scale 0 (uniform weights) runs as a tiny positive scale: every scaled
    // score is then below 2^-24 in magnitude and every probability rounds to
    // exactly 1, as with scale 0, while masked (-inf) scores still give 0.
    p.scale_log2 = scale > 0.f ? scale * kLog2e : 1e-30f;

    hipStream_t s = (hipStream_t)stream;
    const bool c = causal != 0;
    hipError_t err;
    // At most 128 keys (bf16, no band, no block mask): the short-key kernel.
    // Each workgroup streams T tiles of 128 query rows; T is chosen so that
    // all workgroups are resident at once (two per compute unit, 256 CUs on
    // MI355X), which measured fastest on the cross-attention workload.
    const long long q_row_bytes = (layout == FA_BSND ? (long long)H * d : (long long)d) * 2;
    if (in_dtype == FA_BF16 && mode == kPlain && Nk <= 128 && 32 * q_row_bytes < (1LL << 31)) {
        const long long n128 = ((long long)Nq + 127) / 128;
        const long long total = (long long)B * H * n128;
        const int T = (int)std::max(1LL, std::min(n128, (total + kShortWgTarget - 1) / kShortWgTarget));
        const long long chunks = (n128 + T - 1) / T;
        if ((long long)B * H * chunks > INT32_MAX) return FA_ERR_UNSUPPORTED;
        const int g = (int)((long long)B * H * chunks), nkb = (Nk + 31) / 32, ch = (int)chunks;
        const bool ob = o_dtype == FA_BF16;
        if (d == 128)
            err = c ? (ob ? launch_short<128, true, true>(p, nkb, g, T, ch, s) : launch_short<128, true, false>(p, nkb, g, T, ch, s))
                    : (ob ? launch_short<128, false, true>(p, nkb, g, T, ch, s) : launch_short<128, false, false>(p, nkb, g, T, ch, s));
        else
            err = c ? (ob ? launch_short<64, true, true>(p, nkb, g, T, ch, s) : launch_short<64, true, false>(p, nkb, g, T, ch, s))
                    : (ob ? launch_short<64, false, true>(p, nkb, g, T, ch, s) : launch_short<64, false, false>(p, nkb, g, T, ch, s));
        return err == hipSuccess ? FA_OK : FA_ERR_HIP;
    }
    if (in_dtype == FA_BF16) {
        const bool ob = o_dtype == FA_BF16;
        // Plain non-causal attention over whole key tiles (an even number),
        // with at least two query tiles per CU: the persistent kernel, one
        // workgroup per CU (a multiple of 8, for the XCD map)
        const int ncu = cu_count() & ~7;
        if (FA_PERSIST && mode == kPlain && !c && Nk % 128 == 0 && ncu > 0 && grid >= 2LL * ncu) {
            const int g = ncu, ni = (int)grid;
            if (d == 128) err = ob ? launch_persist<128, true>(p, g, ni, s) : launch_persist<128, false>(p, g, ni, s);
            else err = ob ? launch_persist<64, true>(p, g, ni, s) : launch_persist<64, false>(p, g, ni, s);
            return err == hipSuccess ? FA_OK : FA_ERR_HIP;
        }
        const int g = (int)grid;
        if (d == 128) {
            err = c ? (ob ? launch_bf16<128, true, true>(p, g, mode, s) : launch_bf16<128, true, false>(p, g, mode, s))
                    : (ob ? launch_bf16<128, false, true>(p, g, mode, s) : launch_bf16<128, false, false>(p, g, mode, s));
        } else {
            err = c ? (ob ? launch_bf16<64, true, true>(p, g, mode, s) : launch_bf16<64, true, false>(p, g, mode, s))
                    : (ob ? launch_bf16<64, false, true>(p, g, mode, s) : launch_bf16<64, false, false>(p, g, mode, s));
        }
    } else {
        if (d == 128) err = c ? launch_f32<128, true>(p, (int)grid, s) : launch_f32<128, false>(p, (int)grid, s);
        else err = c ? launch_f32<64, true>(p, (int)grid, s) : launch_f32<64, false>(p, (int)grid, s);
    }
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                               int window_left, int window_right, int layout, int in_dtype, int o_dtype,
                               void* stream) {
    return fwd_impl(q, k, v, o, lse, nullptr, B, H, Hkv, Nq, Nk, d, scale, causal, window_left, window_right,
                    layout, in_dtype, o_dtype, stream);
}

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            int layout, int in_dtype, int o_dtype, void* stream) {
    return fwd_impl(q, k, v, o, lse, nullptr, B, H, H, Nq, Nk, d, scale, causal, -1, -1, layout, in_dtype, o_dtype,
                    stream);
}

extern "C" fa_status fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const unsigned char* block_mask, int B, int H, int Nq, int Nk, int d, float scale,
                                   int causal, int layout, int in_dtype, int o_dtype, void* stream) {
    if (!block_mask) return FA_ERR_INVALID_ARG;
    return fwd_impl(q, k, v, o, lse, block_mask, B, H, H, Nq, Nk, d, scale, causal, -1, -1, layout, in_dtype,
                    o_dtype, stream);
}
