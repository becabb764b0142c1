// fa_bwd.hip -- attention backward pass for gfx950 (AMD Instinct MI355X).
//
// Gradients dQ, dK, dV of O = softmax(scale * Q K^T [causal]) V for an
// upstream gradient dO.  Method ([nanhubrain] = nanhubrain.csdn.net,
// FlashAttention in CANN ops-transformer, section "backward recomputation"):
// the probabilities are not stored by the forward pass but rebuilt tile by
// tile from its per-row statistics, here the log-sum-exp
// (P_ij = exp(scale * q_i.k_j - LSE_i)), and the gradient chain is
//   dV += P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ += dS K,  dK += dS^T Q
// with the score scale entering dQ and dK.  The row term D_i must be summed
// over the whole row, D_i = sum_j P_ij dP_ij, which equals dO_i . O_i; the
// listing's sum over one key block is not the softmax derivative.  D is
// computed once per row from O and dO.
//
// gfx950 design (three kernels on one stream; no atomics, so results are
// deterministic):
//   1. delta:  D = rowsum(dO * O) into a caller-provided float32 workspace.
//   2. dK/dV:  key blocks outer (128 keys per workgroup, 32 per wave), query
//      tiles of 32 inner.  The wave's K^T fragment stays in VGPRs, its dK^T
//      and dV^T accumulators (fp32) too; the workgroup's V block sits in LDS
//      for the whole loop.  Q and dO tiles go HBM -> LDS directly, two
//      stages, and are read both as MFMA rows (ds_read_b128, for S = Q K^T
//      and dP = dO V^T) and transposed (ds_read_b64_tr_b16, for
//      dV^T += dO^T P and dK^T += Q^T dS).  A lane owns one key: S and dP
//      come out with the key as the lane's column, so P and dS, packed to
//      bf16, are directly the B operands of the two accumulations.
//   3. dQ:     query tiles outer, like the forward kernel (32 queries per
//      wave, key tiles of 64 inner, two LDS stages for K and V).  Q and dO
//      fragments stay in VGPRs; S^T = K Q^T and dP^T = V dO^T give a lane
//      one query, so LSE_i and D_i are per-lane scalars, and
//      dQ^T += K^T dS^T reads K^T through transposing LDS reads.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 (RNE) as MFMA operands.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa355.h"
#include "fa_common.h"

namespace fa355 {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    float* dq;
    float* dk;
    float* dv;
    float* delta;
    long long q_sb, q_sh, q_sn;   // element strides of Q, O, dO and dQ (batch, head, row)
    long long k_sb, k_sh, k_sn;   // element strides of K, V, dK and dV
    int H, Nq, Nk;
    int group;                    // query heads per key/value head (H / Hkv)
    int Hkv;
    int wl, wr;                   // band: keys i-wl .. i+wr visible (-1: unbounded)
    const unsigned char* block_mask;  // block-sparse: [B*H][n_qb][n_kb], nonzero = computed
    int n_qb, n_kb;               // mask blocks: 256 queries x 64 keys
    int n_tiles;                  // row tiles of the kernel's outer loop
    int BH;                       // B * H for the delta and dQ kernels, B * Hkv for dK/dV
    float scale;                  // softmax scale (>= 0)
    float scale_log2;             // scale * log2(e); a tiny positive value for scale 0
};

// Most 64-key tiles (dQ) or 256-query blocks (dK/dV) a block-sparse call lists.
constexpr int kMaxSparseList = 4096;

// Swizzle selector for the LDS tiles: 0 = k_swz (rows read only with
// ds_read_b128), 2 = kv_swz (rows read both ways).
template <int D, int SWZ>
__device__ __forceinline__ int swz(int row, int ch) {
    if constexpr (SWZ == 0) return k_swz<D>(row, ch);
    else return kv_swz<D>(row, ch);
}

// acc[kb] = A_kb B for 32 rows of A per kb: A rows from an LDS tile (row
// kb*32 + col, chunks 2kk + hi of 8 bf16), B fragments in registers
// (bfrag[kk] = 8 values along the contraction for this lane's column).
template <int D, int NKB, int SWZ>
__device__ __forceinline__ void rows_times_frag(f32x16 (&acc)[NKB], const bf16x8 (&bfrag)[D / 16],
                                                const u32x4* __restrict__ tile, int col, int hi) {
    constexpr int DCH = D / 8, KK = D / 16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int row = kb * 32 + col;
            const u32x4 a = tile[row * DCH + swz<D, SWZ>(row, 2 * kk + hi)];
            const f32x16 c = kk == 0 ? f32x16{} : acc[kb];
            acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), bfrag[kk], c, 0, 0, 0);
        }
    }
}

// Four consecutive floats from LDS.  (Read through a __restrict__ pointer
// like the tiles: the compiler then adds no wait for tile loads in flight.)
__device__ __forceinline__ float4 lds_f4(const float* __restrict__ p) { return *(const float4*)p; }

// acc[db] += T^T X for a tile T of 32*NKB rows in LDS (read transposed) and X
// the packed bf16 operand of those rows in the 32x32 output layout of a
// previous product (pk[kb][j] = rows (kb*32 + 2j, +1) of the lane's column,
// in the permuted order the MFMA contraction accepts): slots 0..3 of 16-row
// group u are rows 16u + hi*4 + 0..3, slots 4..7 rows 16u + 8 + hi*4 + 0..3.
template <int D, int NKB>
__device__ __forceinline__ void tr_times_packed(f32x16 (&acc)[D / 32], const unsigned (&pk)[NKB][8],
                                                const lds_char* __restrict__ tile, int tr_row, int tr_dd) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 pb = __builtin_bit_cast(
                bf16x8, (u32x4){pk[kb][4 * u + 0], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]});
            const int r0 = kb * 32 + 16 * u + tr_row;
            const int r1 = r0 + 8;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dd = db * 32 + tr_dd;
                const int c = dd >> 3, w = (dd & 7) * 2;
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(tile + r0 * (D * 2) + kv_swz<D>(r0, c) * 16 + w));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(tile + r1 * (D * 2) + kv_swz<D>(r1, c) * 16 + w));
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[db], 0, 0, 0);
            }
        }
    }
}

// Row-major bf16 fragment from global memory: 8 values at column 16kk + 8hi
// of row `row` for every kk (zero when the row is past the sequence).
template <int D>
__device__ __forceinline__ void load_frag(bf16x8 (&f)[D / 16], const __bf16* base, long long row_stride, int row,
                                          int nrows, int hi) {
    const bool ok = row < nrows;
    const __bf16* r = base + (long long)(ok ? row : 0) * row_stride + hi * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 x = ok ? *(const u32x4*)(r + kk * 16) : (u32x4){0u, 0u, 0u, 0u};
        f[kk] = __builtin_bit_cast(bf16x8, x);
    }
}

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . O_i, one row per D/8 threads (8 elements each).
template <int D, bool O_BF16>
__global__ __launch_bounds__(256) void fa_bwd_delta_kernel(BwdParams p) {
    constexpr int TPR = D / 8, RPB = 256 / TPR;
    const int tid = __builtin_amdgcn_workitem_id_x();
    const long long r = (long long)__builtin_amdgcn_workgroup_id_x() * RPB + tid / TPR;
    const int part = tid % TPR;
    const long long total = (long long)p.BH * p.Nq;
    float acc = 0.f;
    if (r < total) {
        const long long bh = r / p.Nq, i = r - bh * p.Nq;
        const long long b = bh / p.H, h = bh - b * p.H;
        const long long off = b * p.q_sb + h * p.q_sh + i * p.q_sn + part * 8;
        const bf16x8 g = __builtin_bit_cast(bf16x8, *(const u32x4*)((const __bf16*)p.dout + off));
        if constexpr (O_BF16) {
            const bf16x8 o = __builtin_bit_cast(bf16x8, *(const u32x4*)((const __bf16*)p.o + off));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)g[e], (float)o[e], acc);
        } else {
            const float4 o0 = *(const float4*)((const float*)p.o + off);
            const float4 o1 = *(const float4*)((const float*)p.o + off + 4);
            const float of[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)g[e], of[e], acc);
        }
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (r < total && part == 0) p.delta[r] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK and dV: key blocks outer.
//
// Register layout of one wave (32 keys; lane = (col, hi), col = lane % 32 is
// the key, hi = lane / 32):
//   S and dP of a 32-query tile: s[r] = query (r/4)*8 + hi*4 + r%4 of the
//   tile against key col;
//   dK^T, dV^T accumulators: acc[db][r] = d index db*32 + (r/4)*8 + hi*4 + r%4
//   of key col.
//
// One step of a wave: the 32 queries of the tile in the Q and dO stages
// against the wave's 32 keys, in four chains of MFMAs with the instruction
// order fixed by hand (each group ends in a scheduling fence), every LDS
// operand read issued two or three MFMAs ahead of its use:
//   A: S = Q K^T (Q rows from LDS, K^T in registers);
//   B: dP = dO V^T (dO rows and V rows from LDS), and under it the
//      probabilities P = exp2(S scale log2e - LSE log2e), element by element;
//   C: dV^T += dO^T P (dO read transposed), and under it dS = P (dP - D);
//   D: dK^T += Q^T dS (Q read transposed).
// MASK: element e (query off(e) = (e/4)*8 + hi*4 + e%4 of the tile) is kept
// only if vlo <= (e/4)*8 + e%4, and with UPPER also <= vhi (the bounds
// already less hi*4).
//   qt, gt: this step's Q and dO stages; vb: the V block; st: this step's
//   statistics (LSE log2e of the 32 queries, then D).
#ifndef DKDV_QA
#define DKDV_QA 3
#endif
#ifndef DKDV_GB
#define DKDV_GB 2
#endif
#ifndef DKDV_TC
#define DKDV_TC 2
#endif
// Per-lane LDS byte offsets of a dK/dV step's reads.  The swizzles only flip
// bits inside a row's chunk field, so one XOR with a constant (and an
// immediate offset) turns each into the address of every read of the step:
//   qa: row col, chunk hi of a Q or dO tile; read kk at qa ^ 32kk
//   va: row vrow, chunk hi of the V block; read kk at va ^ 32kk
//   ta0, ta1: transposed reads of rows tr_row and tr_row + 8, d values from
//        tr_dd; MFMA (u, db) at (ta ^ 64db) + 16u rows
// (valid for tile bases that are multiples of 256 bytes)
struct DkdvOffsets {
    unsigned qa, va, ta0, ta1;
};
template <int D>
__device__ __forceinline__ DkdvOffsets dkdv_offsets(int col, int hi, int vrow, int tr_row, int tr_dd) {
    constexpr int RB = D * 2;
    const int c0 = tr_dd >> 3, w = (tr_dd & 7) * 2;
    DkdvOffsets o;
    o.qa = col * RB + kv_swz<D>(col, hi) * 16;
    o.va = vrow * RB + k_swz<D>(vrow, hi) * 16;
    o.ta0 = tr_row * RB + kv_swz<D>(tr_row, c0) * 16 + w;
    o.ta1 = (tr_row + 8) * RB + kv_swz<D>(tr_row + 8, c0) * 16 + w;
    return o;
}
__device__ __forceinline__ unsigned lds_addr(const lds_char* p) { return (unsigned)(uintptr_t)p; }

template <int D, bool MASK, bool UPPER>
__device__ __forceinline__ void dkdv_step(f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], const bf16x8 (&kreg)[D / 16],
                                          const lds_char* qt, const lds_char* gt, const lds_char* vb,
                                          const float* __restrict__ st, DkdvOffsets o, int hi, float sl2, int vlo,
                                          int vhi, bool masked) {
    constexpr int KK = D / 16, DB = D / 32, NT = 2 * DB, RB = D * 2;
    // the offsets pass through an empty asm statement: the compiler then
    // forms each read's address next to the read, every step, instead of
    // keeping all of them in registers across the loop
    asm volatile("" : "+v"(o.qa), "+v"(o.va), "+v"(o.ta0), "+v"(o.ta1));
    const unsigned qb = lds_addr(qt) + o.qa, gb = lds_addr(gt) + o.qa, vbb = lds_addr(vb) + o.va;
    const unsigned tq0 = lds_addr(qt) + o.ta0, tq1 = lds_addr(qt) + o.ta1;
    const unsigned tg0 = lds_addr(gt) + o.ta0, tg1 = lds_addr(gt) + o.ta1;
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    auto rd = [](unsigned a) { return __builtin_bit_cast(bf16x8, *(lds_u32x4*)(uintptr_t)a); };
    auto qread = [&](int kk) { return rd(qb ^ (32u * kk)); };
    auto gread = [&](int kk) { return rd(gb ^ (32u * kk)); };
    auto vread = [&](int kk) { return rd(vbb ^ (32u * kk)); };
    // A operand of MFMA i = u*DB + db of a transposed product (tile Q or dO)
    auto trread = [&](bool q, int i) -> bf16x8 {
        const int u = i / DB, db = i % DB;
        const unsigned a0 = ((q ? tq0 : tg0) ^ (64u * db)) + 16u * u * RB;
        const unsigned a1 = ((q ? tq1 : tg1) ^ (64u * db)) + 16u * u * RB;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto vis = [&](int e) {
        const int c = (e >> 2) * 8 + (e & 3);
        return !MASK || (c >= vlo && (!UPPER || c <= vhi));
    };

    // read-ahead distances (MFMAs) of the Q rows, of the dO and V rows, and
    // of the transposed reads
    constexpr int QA = DKDV_QA, GB = DKDV_GB, TC = DKDV_TC;
    f32x16 s, dp;      // S, then P in place, then dS in place
    unsigned pkp[8], pks[8];
    bf16x8 qf[QA + 1], gf[GB + 1], vf[GB + 1], tf[TC + 1];
    float4 l4[2], d4[2];

    // The wave raises its issue priority (s_setprio 1) over chains A and B
    // (the scores and the exponentials) and drops it for C and D, so the two
    // waves of a SIMD tend to take turns; measured 0.4 % faster on the
    // B4 H32 N8192 backward, 1.0 % on the causal and 2.5 % on the band one,
    // while priority over the dQ kernel's step made the first slower.
    __builtin_amdgcn_s_setprio(1);
    // A: S chain; Q reads QA MFMAs ahead, then the first dO / V reads for B
#pragma unroll
    for (int i = 0; i < QA; ++i) qf[i] = qread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (kk + QA < KK) qf[(kk + QA) % (QA + 1)] = qread(kk + QA);
        if (kk == KK - 3) l4[0] = lds_f4(st + 0 * 8 + hi * 4);
        if (kk >= KK - GB) {
            const int j = kk - (KK - GB);
            gf[j] = gread(j);
            vf[j] = vread(j);
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[kk % (QA + 1)], kreg[kk], kk == 0 ? f32x16{} : s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // B: dP chain, dO / V reads GB MFMAs ahead; the 16 exponentials over
    // groups 1 .. KK-1 (group 0 would wait for the last S MFMA)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (kk + GB < KK) {
            gf[(kk + GB) % (GB + 1)] = gread(kk + GB);
            vf[(kk + GB) % (GB + 1)] = vread(kk + GB);
        }
        if (kk >= KK - TC) tf[kk - (KK - TC)] = trread(false, kk - (KK - TC));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gf[kk % (GB + 1)], vf[kk % (GB + 1)], kk == 0 ? f32x16{} : dp,
                                                     0, 0, 0);
        if (kk >= 1) {
            const int e0 = 16 * (kk - 1) / (KK - 1), e1 = 16 * kk / (KK - 1);
#pragma unroll
            for (int e = e0; e < e1; ++e) {
                const int g = e >> 2;
                if ((e & 3) == 0 && g + 1 < 4) l4[(g + 1) & 1] = lds_f4(st + (g + 1) * 8 + hi * 4);
                const float4 l = l4[g & 1];
                const float lv = (e & 3) == 0 ? l.x : (e & 3) == 1 ? l.y : (e & 3) == 2 ? l.z : l.w;
                s[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sl2, -lv));
            }
            // the mask only on the tiles that cross an edge (a wave-uniform
            // branch: the other tiles skip its compares and selects)
            if (MASK && masked) {
#pragma unroll
                for (int e = e0; e < e1; ++e)
                    if (!vis(e)) s[e] = 0.f;
            }
#pragma unroll
            for (int e = e0; e < e1; ++e)
                if (e & 1) pkp[e >> 1] = pack_bf16x2(s[e - 1], s[e]);
        }
        if (kk == KK - 1) d4[0] = lds_f4(st + 32 + 0 * 8 + hi * 4);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // C: dV chain, transposed reads TC MFMAs ahead (read n = 0 .. 2NT-1:
    // dO^T for C, then Q^T for D, into tf[n % (TC+1)]); dS over groups
    // 1 .. NT-1
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int n = i + TC;
        if (n < NT) tf[n % (TC + 1)] = trread(false, n);
        else tf[n % (TC + 1)] = trread(true, n - NT);
        const int u = i / DB, db = i % DB;
        const bf16x8 pb =
            __builtin_bit_cast(bf16x8, (u32x4){pkp[4 * u + 0], pkp[4 * u + 1], pkp[4 * u + 2], pkp[4 * u + 3]});
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i % (TC + 1)], pb, dv[db], 0, 0, 0);
        if (i >= 1) {
#pragma unroll
            for (int e = 16 * (i - 1) / (NT - 1); e < 16 * i / (NT - 1); ++e) {
                const int g = e >> 2;
                if ((e & 3) == 0 && g + 1 < 4) d4[(g + 1) & 1] = lds_f4(st + 32 + (g + 1) * 8 + hi * 4);
                const float4 dd = d4[g & 1];
                const float dv_ = (e & 3) == 0 ? dd.x : (e & 3) == 1 ? dd.y : (e & 3) == 2 ? dd.z : dd.w;
                s[e] = s[e] * (dp[e] - dv_);
                if (e & 1) pks[e >> 1] = pack_bf16x2(s[e - 1], s[e]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // D: dK chain, Q^T reads TC MFMAs ahead
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (i + TC < NT) tf[(NT + i + TC) % (TC + 1)] = trread(true, i + TC);
        const int u = i / DB, db = i % DB;
        const bf16x8 sb =
            __builtin_bit_cast(bf16x8, (u32x4){pks[4 * u + 0], pks[4 * u + 1], pks[4 * u + 2], pks[4 * u + 3]});
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[(NT + i) % (TC + 1)], sb, dk[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// dQ step: the 64 keys of the tile in the K and V stages against the wave's
// 32 queries (lane = (col, hi), col = the query), in three MFMA phases with
// the instruction order fixed by hand (each group fenced), every LDS operand
// read ahead of its use:
//   A: S^T = K Q^T, both 32-key halves interleaved (K rows from LDS);
//   B: dP^T = V dO^T, half 0 then half 1 (V rows from LDS), and under it the
//      probabilities P = exp2(S scale log2e - lse2) and, under half 1,
//      dS = P (dP - D) of half 0;
//   C: dQ^T += K^T dS^T (K read transposed), and under its first half dS of
//      key half 1.
// MASK: element (kb, r) (key kb*32 + (r/4)*8 + hi*4 + r%4 of the tile) is
// kept only if kb*32 + (r/4)*8 + r%4 <= vhi (the bound already less hi*4),
// applied behind a wave-uniform branch on the tiles that need it (`masked`:
// the causal diagonal and the ragged last tile).  Offsets as for the dK/dV
// step (qa: row col of a K tile, kv_swz; va: row col of a V tile, k_swz;
// ta0/ta1: the transposed reads).  The same order without the mask branch
// (the compares and selects on every tile) was 0.5 % slower than the
// compiler's; with it 1.4 % faster at B4 H32 N8192, bit for bit the same.
#ifndef DQ_KA
#define DQ_KA 3
#endif
#ifndef DQ_VB
#define DQ_VB 3
#endif
#ifndef DQ_TC
#define DQ_TC 2
#endif
template <int D, bool MASK>
__device__ __forceinline__ void dq_step(f32x16 (&acc)[D / 32], const bf16x8 (&qreg)[D / 16],
                                        const bf16x8 (&greg)[D / 16], const lds_char* kt, const lds_char* vt,
                                        DkdvOffsets o, float lse2, float dlt, float sl2, int vhi, bool masked) {
    constexpr int KK = D / 16, DB = D / 32, NA = 2 * KK, NC = 4 * DB, RB = D * 2;
    constexpr int KA = DQ_KA, VB = DQ_VB, TC = DQ_TC;
    asm volatile("" : "+v"(o.qa), "+v"(o.va), "+v"(o.ta0), "+v"(o.ta1));
    const unsigned kb0 = lds_addr(kt) + o.qa, vb0 = lds_addr(vt) + o.va;
    const unsigned t0 = lds_addr(kt) + o.ta0, t1 = lds_addr(kt) + o.ta1;
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    auto rd = [](unsigned a) { return __builtin_bit_cast(bf16x8, *(lds_u32x4*)(uintptr_t)a); };
    // A operand of S^T MFMA i = 2kk + kb (K row kb*32 + col) and of dP^T MFMA
    // i = kb*KK + kk (V row kb*32 + col)
    auto kread = [&](int i) { return rd((kb0 ^ (32u * (i >> 1))) + (i & 1) * 32 * RB); };
    auto vread = [&](int i) { return rd((vb0 ^ (32u * (i % KK))) + (i / KK) * 32 * RB); };
    // A operand of dQ^T MFMA i = (kb*2 + u)*DB + db: K rows kb*32 + 16u + tr_row (+8)
    auto trread = [&](int i) -> bf16x8 {
        const int ku = i / DB, db = i % DB;
        const unsigned a0 = (t0 ^ (64u * db)) + 16u * ku * RB;
        const unsigned a1 = (t1 ^ (64u * db)) + 16u * ku * RB;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto vis = [&](int kb, int r) {
        const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
        return !MASK || c <= vhi;
    };

    f32x16 s[2], dp[2];    // S^T, then P in place, then dS in place
    unsigned pk[2][8];
    bf16x8 kf[KA + 1], vf[VB + 1], tf[TC + 1];
    auto p_elem = [&](int e) {   // e = kb*16 + r
        const int kb = e >> 4, r = e & 15;
        s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], sl2, -lse2));
    };
    auto ds_elem = [&](int e) {
        const int kb = e >> 4, r = e & 15;
        s[kb][r] = s[kb][r] * (dp[kb][r] - dlt);
        if (r & 1) pk[kb][r >> 1] = pack_bf16x2(s[kb][r - 1], s[kb][r]);
    };

    // A: S^T, K reads KA MFMAs ahead, then the first V reads
#pragma unroll
    for (int i = 0; i < KA; ++i) kf[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        if (i + KA < NA) kf[(i + KA) % (KA + 1)] = kread(i + KA);
        if (i >= NA - VB) vf[i - (NA - VB)] = vread(i - (NA - VB));
        const int kb = i & 1;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % (KA + 1)], qreg[i >> 1], i < 2 ? f32x16{} : s[kb], 0, 0,
                                                        0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // B: dP^T half 0 then half 1, V reads VB ahead; the 32 exponentials
    // over groups 1 .. NA/2 (group 0 would wait for the last S^T MFMAs), dS
    // of half 0 over the groups after the first two of half 1
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        if (i + VB < NA) vf[(i + VB) % (VB + 1)] = vread(i + VB);
        if (i >= NA - TC) tf[i - (NA - TC)] = trread(i - (NA - TC));
        const int kb = i / KK, kk = i % KK;
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (VB + 1)], greg[kk], kk == 0 ? f32x16{} : dp[kb], 0,
                                                         0, 0);
        constexpr int PG = NA / 2;                    // exponential groups 1 .. PG
        if (i >= 1 && i <= PG) {
#pragma unroll
            for (int e = 32 * (i - 1) / PG; e < 32 * i / PG; ++e) p_elem(e);
            if (MASK && masked) {
#pragma unroll
                for (int e = 32 * (i - 1) / PG; e < 32 * i / PG; ++e)
                    if (!vis(e >> 4, e & 15)) s[e >> 4][e & 15] = 0.f;
            }
        }
        constexpr int DG0 = KK + 2, DGN = NA - DG0;   // dS of half 0 over groups DG0 .. NA-1
        if (i >= DG0) {
#pragma unroll
            for (int e = 16 * (i - DG0) / DGN; e < 16 * (i - DG0 + 1) / DGN; ++e) ds_elem(e);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // C: dQ^T, transposed reads TC ahead; dS of half 1 over groups 1 .. NC/2
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        if (i + TC < NC) tf[(i + TC) % (TC + 1)] = trread(i + TC);
        const int kb = i / (2 * DB), u = (i / DB) & 1, db = i % DB;
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, (u32x4){pk[kb][4 * u + 0], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i % (TC + 1)], pb, acc[db], 0, 0, 0);
        constexpr int SG = NC / 2;
        if (i >= 1 && i <= SG) {
#pragma unroll
            for (int e = 16 + 16 * (i - 1) / SG; e < 16 + 16 * i / SG; ++e) ds_elem(e);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, bool CAUSAL, bool BAND, bool GQA, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
    constexpr int NW = 4, BK = NW * 32, BQ = 32, DCH = D / 8, KK = D / 16, DB = D / 32;
    // block-sparse: the 128 keys are two mask columns, and a mask row (256
    // queries) is 8 query tiles
    static_assert(BK == 2 * FA_SPARSE_BK && FA_SPARSE_BQ == 8 * BQ, "mask granularity");
    constexpr int QT_CH = BQ * DCH, QTB = QT_CH * 16;     // one Q (or dO) tile
    constexpr int VB_CH = BK * DCH;                       // the V block
    constexpr int LPWQ = QT_CH / 64 / NW, LPWV = VB_CH / 64 / NW;
    static_assert(QT_CH % (64 * NW) == 0 && VB_CH % (64 * NW) == 0, "tiles must split evenly");

    // LDS: the V block, Q stages 0 and 1, dO stages 0 and 1, the two stages'
    // statistics ([stage][lse*log2e, D][query]) and, block-sparse, the list of
    // query blocks and its length.  One LDS array for all of it: with a second
    // LDS variable in the kernel the compiler makes every read of a tile wait
    // for the tile loads still in flight (those of the next step, into the
    // other stage).
    constexpr int STAT_CH = 2 * 2 * BQ * 4 / 16;
    constexpr int LIST_CH = SPARSE ? kMaxSparseList * 2 / 16 + 1 : 0;
    __shared__ __attribute__((aligned(256))) u32x4 smem[VB_CH + 4 * QT_CH + STAT_CH + LIST_CH];
    float(*const stat)[2][BQ] = reinterpret_cast<float(*)[2][BQ]>(smem + VB_CH + 4 * QT_CH);
    unsigned short* const qb_list = reinterpret_cast<unsigned short*>(smem + VB_CH + 4 * QT_CH + STAT_CH);
    int* const qb_len = reinterpret_cast<int*>(qb_list + kMaxSparseList);

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hi = lane >> 5;

    // workgroup -> (batch, KV head, key block); the query heads of the KV
    // head's group all feed this block's dK and dV
    // causal and block-sparse: the key blocks in ascending order, heads fastest,
    // so the blocks that most queries see (the first keys under the causal
    // mask; global columns at the start of a block-sparse mask) start first
    // and no long block is left for the end of the grid
    int bh, kt;
    tile_of_block(__builtin_amdgcn_workgroup_id_x(), p.n_tiles, p.BH, CAUSAL || SPARSE, bh, kt);
    if (CAUSAL || SPARSE) kt = p.n_tiles - 1 - kt;
    const int b = bh / p.Hkv;
    const int hk = bh - b * p.Hkv;
    const int h0 = hk * p.group;           // first query head of the group
    const int Nq = p.Nq, Nk = p.Nk;
    const int k0 = kt * BK;               // first key of the workgroup
    const int kw0 = k0 + wave * 32;       // first key of this wave
    const int key = kw0 + col;            // this lane's key

    const long long qoff = (long long)b * p.q_sb + (long long)h0 * p.q_sh;
    const long long koff = (long long)b * p.k_sb + (long long)hk * p.k_sh;
    const char* qbase = (const char*)((const __bf16*)p.q + qoff);
    const char* gbase = (const char*)((const __bf16*)p.dout + qoff);
    const char* vbase = (const char*)((const __bf16*)p.v + koff + (long long)k0 * p.k_sn);
    const unsigned qrb = (unsigned)(p.q_sn * 2), krb = (unsigned)(p.k_sn * 2);
    const unsigned long long head_bytes = (unsigned long long)p.q_sh * 2;   // next query head

    // queries that see a key of the block [k0, k1]: causal ones are >= k0;
    // under the band, i + wr >= k0 and i - wl <= k1
    const int k1 = min(k0 + BK, Nk) - 1;
    int q_begin = CAUSAL ? k0 : 0;
    int q_last = Nq - 1;
    // the same for this wave's keys (a wave past Nk sees no query)
    int wq_lo = CAUSAL ? kw0 : 0, wq_hi = kw0 < Nk ? Nq - 1 : -1;
    if constexpr (BAND) {
        if (p.wr >= 0) {
            q_begin = max(q_begin, k0 - p.wr);
            wq_lo = max(wq_lo, kw0 - p.wr);
        }
        if (p.wl >= 0) {
            q_last = min(q_last, k1 + p.wl);
            wq_hi = min(wq_hi, min(kw0 + 31, Nk - 1) + p.wl);
        }
    }
    const int n_qt = q_begin <= q_last ? (q_last - q_begin) / BQ + 1 : 0;
    // K^T fragment (B operand of S = Q K^T): K[key][16kk + 8hi .. +7]
    // (loaded before the block-sparse list is built, so the two latencies overlap)
    bf16x8 kreg[KK];
    load_frag<D>(kreg, (const __bf16*)p.k + koff, p.k_sn, key, Nk, hi);
    // Block-sparse: the block's 128 keys are two mask columns (waves 0-1 and
    // 2-3); the steps run over the 32-row tiles of the sorted list of the
    // 256-query blocks that mark either column (entry: block - first block,
    // bit 14 + c if column c is marked); a wave skips the blocks that leave
    // its own column off and sees the others whole (apart from the causal
    // diagonal and rows past Nq)
    int n_sp = 0;                          // block-sparse steps
    const int qb0 = q_begin / FA_SPARSE_BQ;
    if constexpr (SPARSE) {
        const unsigned char* mk = p.block_mask + (long long)bh * p.n_qb * p.n_kb;
        const int c0 = kt * 2, c1 = kt * 2 + 1;
        if (wave == 0) {
            const int cnt = build_list(qb_list, p.n_qb - qb0, lane, [&](int t) {
                const unsigned char* mr = mk + (long long)(qb0 + t) * p.n_kb;
                return (mr[c0] != 0 ? 0x4000u : 0u) | (c1 < p.n_kb && mr[c1] != 0 ? 0x8000u : 0u);
            });
            if (lane == 0) *qb_len = cnt;
        }
        __syncthreads();
        const int n_list = *qb_len;
        n_sp = 8 * n_list;
        if (n_list > 0 && qb0 + (qb_list[n_list - 1] & 0xFFF) == p.n_qb - 1)   // the last block may be partial
            n_sp -= 8 - (Nq - (p.n_qb - 1) * FA_SPARSE_BQ + BQ - 1) / BQ;
    }
    // first query of block-sparse step v
    auto sp_row = [&](int v) { return (qb0 + (qb_list[v >> 3] & 0xFFF)) * FA_SPARSE_BQ + (v & 7) * BQ; };


    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;

    lds_char* const lds = (lds_char*)smem;
    lds_char* const vblk = lds;
    lds_char* const qst = lds + VB_CH * 16;             // Q stage t at qst + t*QTB
    lds_char* const gst = lds + VB_CH * 16 + 2 * QTB;   // dO stage t

    // staging offsets (one per lane and tensor; see issue_tile)
    unsigned ld_q, ld_v;
    {
        const int row = wave * (64 / DCH) + lane / DCH, ch = lane % DCH;
        ld_q = row * qrb + kv_swz<D>(row, ch) * 16;
        ld_v = row * krb + k_swz<D>(row, ch) * 16;
    }
    const unsigned long long qaddr = to_sgpr((unsigned long long)qbase);
    const unsigned long long gaddr = to_sgpr((unsigned long long)gbase);
    const int wofs = wave * 1024;   // this wave's part of a stage (bytes)
    // step v: Q and dO rows i0 .. of the query head whose rows start at
    // byte offset hoff (the steps run head-major)
#define FA_ISSUE_QG(v, hoff, i0)                                                                                 \
    do {                                                                                                         \
        const unsigned long long o_ = (hoff) + (unsigned long long)(i0) * qrb;                                   \
        issue_tile<LPWQ, DCH, BQ, NW>(qaddr + o_, qrb, ld_q, qst + ((v) & 1) * QTB + wofs, Nq - (i0), wave, lane); \
        issue_tile<LPWQ, DCH, BQ, NW>(gaddr + o_, qrb, ld_q, gst + ((v) & 1) * QTB + wofs, Nq - (i0), wave, lane); \
    } while (0)

    // statistics of a query tile: lse * log2(e) and D (lanes 0..31 of wave 0),
    // rows i0 .. of the query head whose statistics start at stat_row.  Rows
    // past Nq (their Q and dO are copies of row Nq-1, finite) take lse = +inf
    // and D = 0, so their P is exactly 0, and so is their dS: they add nothing
    // and need no mask.
    float st_lse = 0.f, st_dl = 0.f;
    auto load_stat = [&](long long stat_row, int i0) {
        const int i = i0 + lane;
        st_lse = INFINITY;
        st_dl = 0.f;
        if (wave == 0 && lane < BQ && i < Nq) {
            st_lse = p.lse[stat_row + i];
            st_dl = p.delta[stat_row + i];
        }
    };
    // (the loads above are first used here, after the step's wait for all
    // loads: using them earlier would wait for the tile loads issued before)
    auto store_stat = [&](int t) {
        if (wave == 0 && lane < BQ) {
            stat[t & 1][0][lane] = st_lse * kLog2e;
            stat[t & 1][1][lane] = st_dl;
        }
    };

    // V^T fragment addressing (B operand of dP = dO V^T): V block row
    // wave*32 + col, chunk 2kk + hi
    const int vrow = wave * 32 + col;
    // transposing-read addressing (see tr_times_packed)
    const int tg = lane >> 4, ti = lane & 15;
    const int tr_row = hi * 4 + (ti >> 2);
    const int tr_dd = 16 * (tg & 1) + 4 * (ti & 3);
    const float sl2 = p.scale_log2;
    const DkdvOffsets offs = dkdv_offsets<D>(col, hi, vrow, tr_row, tr_dd);

    // steps t = 0 .. n_vt - 1, each issuing the next one's loads; with
    // grouped heads the query heads of the group run one after the other
    // (step t: head h0 + t / n_qt, query tile t % n_qt, tracked by counters)
    const long long stat0 = ((long long)b * p.H + h0) * Nq;
    const int n_vt = SPARSE ? n_sp : GQA ? n_qt * p.group : n_qt;
    unsigned long long hoff_nxt = 0;      // the next step's head: Q/dO byte offset,
    long long stat_nxt = stat0;           // statistics row
    int i_nxt = q_begin;                  // and first query
    if (n_vt > 0) {
        const int r0 = SPARSE ? sp_row(0) : q_begin;
        issue_tile<LPWV, DCH, BK, NW>(to_sgpr((unsigned long long)vbase), krb, ld_v, vblk + wofs, Nk - k0, wave,
                                      lane);
        FA_ISSUE_QG(0, 0ull, r0);
        load_stat(stat0, r0);
    }
    for (int t = 0; t < n_vt; ++t) {
        int i0;
        if constexpr (GQA) {
            i0 = i_nxt;
            i_nxt += BQ;
            if (i_nxt > q_last) {         // the next step starts the next query head
                i_nxt = q_begin;
                hoff_nxt += head_bytes;
                stat_nxt += Nq;
            }
        } else if constexpr (SPARSE) {
            i0 = sp_row(t);
        } else {
            i0 = q_begin + t * BQ;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        store_stat(t);
        __syncthreads();
        if (t + 1 < n_vt) {
            if constexpr (GQA) {
                FA_ISSUE_QG(t + 1, hoff_nxt, i_nxt);
                load_stat(stat_nxt, i_nxt);
            } else if constexpr (SPARSE) {
                const int r1 = sp_row(t + 1);
                FA_ISSUE_QG(t + 1, 0ull, r1);
                load_stat(stat0, r1);
            } else {
                FA_ISSUE_QG(t + 1, 0ull, i0 + BQ);
                load_stat(stat0, i0 + BQ);
            }
        }
        // a wave none of whose keys this tile's queries see has nothing to add
        if constexpr (BAND) {
            if (i0 + BQ - 1 < wq_lo || i0 > wq_hi) continue;
        } else if constexpr (SPARSE) {
            if (((qb_list[t >> 3] >> (14 + (wave >> 1))) & 1) == 0 || (CAUSAL && i0 + BQ - 1 < kw0)) continue;
        } else {
            if (CAUSAL && i0 + BQ - 1 < kw0) continue;
        }

        // P = exp2(s*scale*log2e - lse2), dS = P (dP - D); pairs outside the
        // causal mask or the band get 0, on the tiles that cross an edge (rows
        // past Nq have P = 0 from their statistics)
        const lds_char* const qt = qst + (t & 1) * QTB;
        const lds_char* const gt = gst + (t & 1) * QTB;
        const float* const st = &stat[t & 1][0][0];
        bool masked = CAUSAL && i0 < kw0 + 31;
        if constexpr (BAND)
            masked = masked || (p.wl >= 0 && i0 + BQ - 1 - p.wl > kw0) || (p.wr >= 0 && i0 + p.wr < kw0 + 31);
        if constexpr (CAUSAL || BAND) {
            // element bounds of dkdv_step (the lane's query offset less hi*4),
            // used only on the tiles that cross an edge
            const int base = key - i0 - hi * 4;
            int vlo = CAUSAL ? base : -(1 << 30), vhi = 1 << 30;
            if (BAND && p.wr >= 0) vlo = max(vlo, (int)max((long long)base - p.wr, -(1LL << 30)));
            if (BAND && p.wl >= 0) vhi = (int)min((long long)base + p.wl, 1LL << 30);
            dkdv_step<D, true, BAND>(dk, dv, kreg, qt, gt, vblk, st, offs, hi, sl2, vlo, vhi, masked);
        } else {
            dkdv_step<D, false, false>(dk, dv, kreg, qt, gt, vblk, st, offs, hi, sl2, 0, 0, false);
        }
    }
#undef FA_ISSUE_QG

    store_acc_rows<D, false, 0>(dk, p.scale, (char*)(p.dk + koff + (long long)kw0 * p.k_sn), p.k_sn, Nk - kw0, col,
                                hi);
    store_acc_rows<D, false, 1>(dv, 1.0f, (char*)(p.dv + koff + (long long)kw0 * p.k_sn), p.k_sn, Nk - kw0, col, hi);
}

// ---------------------------------------------------------------------------
// 3. dQ: query tiles outer.
//
// Register layout of one wave (32 queries; lane = (col, hi), col = the query):
//   S^T, dP^T of a 64-key tile: s[kb][r] = key kb*32 + (r/4)*8 + hi*4 + r%4
//   against query col;  dQ^T accumulator: acc[db][r] = d index
//   db*32 + (r/4)*8 + hi*4 + r%4 of query col.
template <int D, bool CAUSAL, bool BAND, bool SPARSE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdParams p) {
    constexpr int NW = 8, BC = 64, BR = NW * 32, DCH = D / 8, KK = D / 16, DB = D / 32;
    // block-sparse: a mask row is this kernel's query tile, a column its key tile
    static_assert(BR == FA_SPARSE_BQ && BC == FA_SPARSE_BK, "mask granularity");
    constexpr int TILE_CH = BC * DCH, TB = TILE_CH * 16, LPW = TILE_CH / 64 / NW;
    static_assert(TILE_CH % (64 * NW) == 0, "tile must split evenly over the waves");

    // LDS: K stages 0, 1, V stages 0, 1 and, block-sparse, the list of key
    // tiles and its length, in one LDS array (with a second LDS variable the
    // compiler makes every read of a tile wait for the loads in flight into
    // the other stage)
    constexpr int LIST_CH = SPARSE ? kMaxSparseList * 2 / 16 + 1 : 0;
    __shared__ u32x4 smem[4 * TILE_CH + LIST_CH];
    unsigned short* const tile_list = reinterpret_cast<unsigned short*>(smem + 4 * TILE_CH);
    int* const list_len = reinterpret_cast<int*>(tile_list + kMaxSparseList);

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hi = lane >> 5;

    int bh, qt;
    tile_of_block(__builtin_amdgcn_workgroup_id_x(), p.n_tiles, p.BH, CAUSAL, bh, qt);
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    const int Nq = p.Nq, Nk = p.Nk;
    const int q_wg0 = qt * BR;
    const int q_w0 = q_wg0 + wave * 32;
    const int q = q_w0 + col;

    const long long qoff = (long long)b * p.q_sb + (long long)h * p.q_sh;
    const long long koff = (long long)b * p.k_sb + (long long)(h / p.group) * p.k_sh;
    const unsigned krb = (unsigned)(p.k_sn * 2);

    // key tiles t_lo .. t_lo + n_kt - 1 (this wave's: tw_lo .. tw_hi): causal
    // queries see keys <= query only; under the band, keys i - wl .. i + wr
    int t_lo = 0, n_kt, tw_lo = 0, tw_hi;
    // band limits of this lane's query: visible keys lo_key .. hi_key
    int lo_key = 0, hi_key = 0;
    const int q_wl = min(q_w0 + 31, Nq - 1);
    if constexpr (BAND) {
        const int q_last = min(q_wg0 + BR, Nq) - 1;
        int key_lo = 0, key_hi = CAUSAL ? min(Nk - 1, q_last) : Nk - 1;
        // a wave past Nq sees no key
        int wk_lo = 0, wk_hi = q_w0 < Nq ? (CAUSAL ? min(Nk - 1, q_wl) : Nk - 1) : -1;
        hi_key = CAUSAL ? min(Nk - 1, q) : Nk - 1;
        if (p.wl >= 0) {
            key_lo = max(0, q_wg0 - p.wl);
            wk_lo = max(0, q_w0 - p.wl);
            lo_key = q - p.wl;
        }
        if (p.wr >= 0) {
            key_hi = min(key_hi, q_last + p.wr);
            wk_hi = min(wk_hi, q_wl + p.wr);
            hi_key = min(hi_key, q + p.wr);
        }
        t_lo = key_lo / BC;
        n_kt = key_lo <= key_hi ? key_hi / BC + 1 - t_lo : 0;
        tw_lo = wk_lo / BC;
        tw_hi = wk_lo <= wk_hi ? wk_hi / BC : -1;
    } else {
        int kv_end = Nk;
        if (CAUSAL) kv_end = min(Nk, min(q_wg0 + BR, Nq));
        n_kt = (kv_end + BC - 1) / BC;
        tw_hi = (CAUSAL ? min(n_kt, (q_w0 + 31) / BC + 1) : n_kt) - 1;
    }
    const int n_kt_wave = tw_hi + 1;      // no band: the wave's tiles are 0 .. n_kt_wave - 1
    // (loaded before the block-sparse list is built, so the two latencies overlap)
    bf16x8 qreg[KK], greg[KK];
    load_frag<D>(qreg, (const __bf16*)p.q + qoff, p.q_sn, q, Nq, hi);
    load_frag<D>(greg, (const __bf16*)p.dout + qoff, p.q_sn, q, Nq, hi);
    float lse2 = 0.f, dlt = 0.f;
    if (q < Nq) {
        lse2 = p.lse[(long long)bh * Nq + q] * kLog2e;
        dlt = p.delta[(long long)bh * Nq + q];
    }
    // Block-sparse: the workgroup's 256 queries are one mask row; the steps
    // run over the sorted list of the key tiles it marks (a marked tile is
    // seen whole, apart from the causal diagonal and the ragged last tile)
    if constexpr (SPARSE) {
        const unsigned char* mrow = p.block_mask + ((long long)bh * p.n_qb + qt) * p.n_kb;
        if (wave == 0) {
            const int cnt = build_list(tile_list, n_kt, lane, [&](int t) { return mrow[t] != 0 ? 1u : 0u; });
            if (lane == 0) *list_len = cnt;
        }
        __syncthreads();
        n_kt = *list_len;
    }


    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    unsigned ld_k, ld_v;
    {
        const int row = wave * (64 / DCH) + lane / DCH, ch = lane % DCH;
        ld_k = row * krb + kv_swz<D>(row, ch) * 16;
        ld_v = row * krb + k_swz<D>(row, ch) * 16;
    }
    lds_char* const lds = (lds_char*)smem;
    const unsigned long long kaddr = to_sgpr((unsigned long long)((const __bf16*)p.k + koff));
    const unsigned long long vaddr = to_sgpr((unsigned long long)((const __bf16*)p.v + koff));
    const unsigned long long tile_bytes = (unsigned long long)BC * krb;
    lds_char* const ldst = lds + wave * 1024;
    // step j: key tile t_lo + j (no band: tile j; block-sparse: list entry j),
    // LDS stage j & 1
#define FA_STEP_TILE(j) (SPARSE ? (int)tile_list[(j)] : BAND ? t_lo + (j) : (j))
#define FA_ISSUE_KV(j)                                                                                           \
    do {                                                                                                         \
        const int t_ = FA_STEP_TILE(j);                                                                          \
        issue_tile<LPW, DCH, BC, NW>(kaddr + (unsigned long long)t_ * tile_bytes, krb, ld_k, ldst + ((j) & 1) * TB, \
                                     Nk - t_ * BC, wave, lane);                                                  \
        issue_tile<LPW, DCH, BC, NW>(vaddr + (unsigned long long)t_ * tile_bytes, krb, ld_v,                     \
                                     ldst + (2 + ((j) & 1)) * TB, Nk - t_ * BC, wave, lane);                     \
    } while (0)

    const int tg = lane >> 4, ti = lane & 15;
    const int tr_row = hi * 4 + (ti >> 2);
    const int tr_dd = 16 * (tg & 1) + 4 * (ti & 3);
    const float sl2 = p.scale_log2;
    const DkdvOffsets offs = dkdv_offsets<D>(col, hi, col, tr_row, tr_dd);

    if ((!BAND && !SPARSE) || n_kt > 0) FA_ISSUE_KV(0);
    for (int j = 0; j < n_kt; ++j) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (j + 1 < n_kt) FA_ISSUE_KV(j + 1);
        const int tile = FA_STEP_TILE(j);
        if constexpr (BAND) {
            if (tile < tw_lo || tile > tw_hi) continue;
        } else if constexpr (SPARSE) {
            if (tile > tw_hi) continue;
        } else {
            if (j >= n_kt_wave) continue;
        }

        const lds_char* ks = lds + (j & 1) * TB;
        const lds_char* vs = lds + (2 + (j & 1)) * TB;
        // P = exp2(S*scale*log2e - lse2), dS = P (dP - D), dQ += dS K; keys
        // past Nk, and pairs outside the causal mask or the band, get 0 on the
        // tiles that cross an edge
        const int key0 = tile * BC;
        bool masked = key0 + BC > Nk || (CAUSAL && key0 + BC - 1 > q_w0);
        if constexpr (BAND)
            masked = masked || (p.wl >= 0 && key0 < q_wl - p.wl) || (p.wr >= 0 && key0 + BC - 1 > q_w0 + p.wr);
        const int lim = (BAND ? hi_key : CAUSAL ? min(Nk - 1, q) : Nk - 1) - (key0 + hi * 4);
        if constexpr (!BAND) {
            dq_step<D, true>(acc, qreg, greg, ks, vs, offs, lse2, dlt, sl2, lim, masked);
        } else {
            // (the band keeps the compiler's order: the hand-ordered step needs
            // more registers than the band's bookkeeping leaves)
            f32x16 s[2], dp[2];
            rows_times_frag<D, 2, 2>(s, qreg, (const u32x4*)ks, col, hi);
            rows_times_frag<D, 2, 0>(dp, greg, (const u32x4*)vs, col, hi);
            const int lo_lim = lo_key - (key0 + hi * 4);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], sl2, -lse2));
            // the per-element mask only on tiles that need it (a uniform branch)
            if (masked) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                        s[kb][r] = off <= lim && (!BAND || off >= lo_lim) ? s[kb][r] : 0.f;
                    }
            }
            unsigned pk[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    pk[kb][jj] = pack_bf16x2(s[kb][2 * jj] * (dp[kb][2 * jj] - dlt),
                                             s[kb][2 * jj + 1] * (dp[kb][2 * jj + 1] - dlt));
            tr_times_packed<D, 2>(acc, pk, ks, tr_row, tr_dd);
        }
    }
#undef FA_ISSUE_KV
#undef FA_STEP_TILE

    store_acc_rows<D, false, 2>(acc, p.scale, (char*)(p.dq + qoff + (long long)q_w0 * p.q_sn), p.q_sn, Nq - q_w0, col,
                                hi);
}

}  // namespace fa355

using namespace fa355;

namespace {

bool aligned_b(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

template <int D, bool CAUSAL, bool BAND, bool SPARSE>
hipError_t launch_bwd(BwdParams p, int B, bool o_bf16, long long n_rows, hipStream_t s) {
    // 1. D = rowsum(dO * O)
    const long long rpb = 256 / (D / 8);
    const long long g1 = (n_rows + rpb - 1) / rpb;
    if (o_bf16)
        hipLaunchKernelGGL((fa_bwd_delta_kernel<D, true>), dim3((unsigned)g1), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((fa_bwd_delta_kernel<D, false>), dim3((unsigned)g1), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 2. dK, dV (128 keys of one KV head per workgroup)
    BwdParams p2 = p;
    p2.n_tiles = (p.Nk + 127) / 128;
    p2.BH = B * p.Hkv;
    if (!SPARSE && p.group > 1)
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, BAND, true, false>),
                           dim3((unsigned)((long long)p2.n_tiles * p2.BH)), dim3(256), 0, s, p2);
    else
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, BAND, false, SPARSE>),
                           dim3((unsigned)((long long)p2.n_tiles * p2.BH)), dim3(256), 0, s, p2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 3. dQ (256 queries of one query head per workgroup)
    BwdParams p3 = p;
    p3.n_tiles = (p.Nq + 255) / 256;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, BAND, SPARSE>), dim3((unsigned)((long long)p3.n_tiles * p.BH)),
                       dim3(512), 0, s, p3);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(BwdParams p, int B, bool causal, bool band, bool sparse, bool o_bf16, long long n_rows,
                        hipStream_t s) {
    if (sparse) return causal ? launch_bwd<D, true, false, true>(p, B, o_bf16, n_rows, s)
                              : launch_bwd<D, false, false, true>(p, B, o_bf16, n_rows, s);
    if (band) return causal ? launch_bwd<D, true, true, false>(p, B, o_bf16, n_rows, s)
                            : launch_bwd<D, false, true, false>(p, B, o_bf16, n_rows, s);
    return causal ? launch_bwd<D, true, false, false>(p, B, o_bf16, n_rows, s)
                  : launch_bwd<D, false, false, false>(p, B, o_bf16, n_rows, s);
}

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, const unsigned char* block_mask, float* dq, float* dk, float* dv, float* delta,
                   int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int window_left, int window_right, int layout, int in_dtype, int o_dtype, void* stream) {
    // ---- validation: no HIP call before it passes
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (layout != FA_BHND && layout != FA_BSND) return FA_ERR_INVALID_ARG;
    if (in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_INVALID_ARG;
    if (o_dtype != FA_BF16 && o_dtype != FA_F32) return FA_ERR_INVALID_ARG;
    if (!aligned_b(q, 16) || !aligned_b(k, 16) || !aligned_b(v, 16) || !aligned_b(o, 16) || !aligned_b(dout, 16) ||
        !aligned_b(dq, 16) || !aligned_b(dk, 16) || !aligned_b(dv, 16))
        return FA_ERR_INVALID_ARG;
    if (!aligned_b(lse, 4) || !aligned_b(delta, 4)) return FA_ERR_INVALID_ARG;
    if (scale != scale || fabsf(scale) == INFINITY) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (Nq >= (1 << 30) || Nk >= (1 << 30)) return FA_ERR_UNSUPPORTED;
    const long long BH = (long long)B * H;
    const long long n_rows = BH * Nq;
    if (BH > INT32_MAX || n_rows / 16 > INT32_MAX || (long long)B * Hkv * ((Nk + 127) / 128) > INT32_MAX ||
        BH * ((Nq + 255) / 256) > INT32_MAX)
        return FA_ERR_UNSUPPORTED;
    // tiles of up to 128 rows are addressed with 32-bit byte offsets
    const long long q_row_bytes = (layout == FA_BSND ? (long long)H * d : (long long)d) * 2;
    const long long k_row_bytes = (layout == FA_BSND ? (long long)Hkv * d : (long long)d) * 2;
    if (128 * q_row_bytes >= (1LL << 31) || 128 * k_row_bytes >= (1LL << 31)) return FA_ERR_UNSUPPORTED;

    if (scale < 0.f) scale = 1.0f / sqrtf((float)d);
    // a band edge beyond every key changes nothing: such edges are unbounded
    // (which also keeps every key index the kernels form within int range)
    int wl = window_left < 0 ? -1 : window_left;
    int wr = window_right < 0 ? -1 : window_right;
    if (wl >= Nq) wl = -1;     // i - wl < 0 <= every key for every query i < Nq
    if (wr >= Nk) wr = -1;     // i + wr >= Nk - 1 for every query
    const bool band = wl >= 0 || wr >= 0;
    // block-sparse: no band, no grouped heads, mask lists within kMaxSparseList
    const bool sparse = block_mask != nullptr;
    if (sparse && (band || Hkv != H || (Nk + 63) / 64 > kMaxSparseList || (Nq + 255) / 256 > kMaxSparseList))
        return FA_ERR_UNSUPPORTED;

    BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv; p.delta = delta;
    const long long D = d;
    if (layout == FA_BHND) {
        p.q_sb = (long long)H * Nq * D; p.q_sh = (long long)Nq * D; p.q_sn = D;
        p.k_sb = (long long)Hkv * Nk * D; p.k_sh = (long long)Nk * D; p.k_sn = D;
    } else {
        p.q_sb = (long long)Nq * H * D; p.q_sh = D; p.q_sn = (long long)H * D;
        p.k_sb = (long long)Nk * Hkv * D; p.k_sh = D; p.k_sn = (long long)Hkv * D;
    }
    p.H = H; p.Nq = Nq; p.Nk = Nk;
    p.Hkv = Hkv;
    p.group = H / Hkv;
    p.wl = wl;
    p.wr = wr;
    p.block_mask = block_mask;
    p.n_qb = (Nq + FA_SPARSE_BQ - 1) / FA_SPARSE_BQ;   // mask rows: 256 queries
    p.n_kb = (Nk + FA_SPARSE_BK - 1) / FA_SPARSE_BK;   // mask columns: 64 keys
    p.n_tiles = 0;
    p.BH = (int)BH;
    p.scale = scale;
    // scale 0 runs the exponentials with a tiny positive factor (every scaled
    // score rounds away against the log-sum-exp, as with scale 0) and the
    // gradients of Q and K are multiplied by the exact 0
    p.scale_log2 = scale > 0.f ? scale * kLog2e : 1e-30f;

    hipStream_t s = (hipStream_t)stream;
    const bool c = causal != 0, ob = o_dtype == FA_BF16;
    const hipError_t err = d == 128 ? launch_bwd_d<128>(p, B, c, band, sparse, ob, n_rows, s)
                                    : launch_bwd_d<64>(p, B, c, band, sparse, ob, n_rows, s);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, float* dq, float* dk, float* dv, float* delta,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            int layout, int in_dtype, int o_dtype, void* stream) {
    return bwd_impl(q, k, v, o, dout, lse, nullptr, dq, dk, dv, delta, B, H, H, Nq, Nk, d, scale, causal, -1, -1,
                    layout, in_dtype, o_dtype, stream);
}

extern "C" fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, float* dq, float* dk, float* dv, float* delta,
                               int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                               int window_left, int window_right, int layout, int in_dtype, int o_dtype,
                               void* stream) {
    return bwd_impl(q, k, v, o, dout, lse, nullptr, dq, dk, dv, delta, B, H, Hkv, Nq, Nk, d, scale, causal,
                    window_left, window_right, layout, in_dtype, o_dtype, stream);
}

extern "C" fa_status fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, const unsigned char* block_mask, float* dq, float* dk,
                                   float* dv, float* delta, int B, int H, int Nq, int Nk, int d, float scale,
                                   int causal, int layout, int in_dtype, int o_dtype, void* stream) {
    if (!block_mask) return FA_ERR_INVALID_ARG;
    return bwd_impl(q, k, v, o, dout, lse, block_mask, dq, dk, dv, delta, B, H, H, Nq, Nk, d, scale, causal, -1,
                    -1, layout, in_dtype, o_dtype, stream);
}
