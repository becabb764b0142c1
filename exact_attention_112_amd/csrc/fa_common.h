// fa_common.h -- device primitives shared by the attention kernels of
// libfa355 for gfx950 (AMD Instinct MI355X): vector types, LDS address
// spaces, the workgroup -> (head, tile) map, the LDS swizzles, bf16 packing,
// the cross-half reductions of a wave, the direct HBM -> LDS load and the
// list of a block-sparse mask row or column.
#ifndef FA355_COMMON_H
#define FA355_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Workgroup id -> (batch*head, tile of rows).  Workgroups are dispatched round
// robin over the 8 XCDs; when B*H is a multiple of 8, each XCD gets a
// contiguous block of whole heads so one head's K/V stays in one XCD's L2.
// Causal: heaviest (last) query tiles first -- across the XCD's heads, or,
// with head_major (long sequences, at least as many tiles per head as an XCD
// has CUs), one head after another, so the tiles an XCD runs at once belong
// to one head and walk its keys together through L2.  A bijection in all
// cases.
__device__ __forceinline__ void tile_of_block(int bid, int n_tiles, int BH, bool causal,
                                              int& bh, int& qt, bool head_major = false) {
    if ((BH & 7) == 0) {
        const int hpx = BH >> 3;
        const int xcd = bid & 7;
        const int s = bid >> 3;
        if (causal && head_major) {
            bh = xcd * hpx + s / n_tiles;
            qt = n_tiles - 1 - s % n_tiles;
        } else if (causal) {
            qt = n_tiles - 1 - s / hpx;
            bh = xcd * hpx + s % hpx;
        } else {
            bh = xcd * hpx + s / n_tiles;
            qt = s % n_tiles;
        }
    } else if (causal) {
        qt = n_tiles - 1 - bid / BH;
        bh = bid % BH;
    } else {
        bh = bid / n_tiles;
        qt = bid % n_tiles;
    }
}

// 16-byte-chunk swizzles of the LDS tiles (row = key within the tile, ch =
// logical chunk of 8 bf16 along d).  K is read with ds_read_b128 by 32 lanes
// on 32 consecutive rows at one chunk; V is read with ds_read_b64_tr_b16 on
// 8 consecutive rows at 4 consecutive chunks.
template <int D>
__device__ __forceinline__ int k_swz(int row, int ch) {
    if constexpr (D == 128) return ch ^ (row & 15);
    else return ch ^ ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row, int ch) {
    if constexpr (D == 128) return ch ^ ((row & 3) << 2);
    else return ch ^ (((row >> 1) & 1) << 2);
}

// The swizzle of a tile read both ways (32-row ds_read_b128 and 8-row
// ds_read_b64_tr_b16): the 16-row phase of k_swz, with bit 2-3 of it further
// XORed by the row's position in its group of 4 (d = 128), or the 8-row-pair
// phase with bit 2 XORed by the pair's parity (d = 64).  Both maps are
// bijections on a row's chunks; 16 consecutive rows at one logical chunk hit
// 16 different chunks, and the 4 rows of a transposing read hit 4 different
// groups of 4 chunks.
template <int D>
__device__ __forceinline__ int kv_swz(int row, int ch) {
    if constexpr (D == 128) return ch ^ ((row & 15) ^ ((row & 3) << 2));
    else return ch ^ (((row >> 1) & 7) ^ (((row >> 1) & 1) << 2));
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    bf16x2 r = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(unsigned, r);
}

// x of this lane and x of the lane 32 apart, combined (every lane gets the
// result for its pair).  v_permlane32_swap(a, b) exchanges lanes 32..63 of a
// with lanes 0..31 of b; with a = b = x the two registers then hold x's low
// half and x's high half, each in both halves.  Written as inline assembly:
// the compiler's builtin for it returns the first register twice.  The
// s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
    unsigned u = __builtin_bit_cast(unsigned, x), w = u;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(w));
    a = __builtin_bit_cast(float, u);
    b = __builtin_bit_cast(float, w);
}
__device__ __forceinline__ float pair_max(float x) {
    float a, b;
    swap_halves(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
    float a, b;
    swap_halves(x, a, b);
    return a + b;
}

// One 16-byte-per-lane buffer load into LDS: lane i of the wave writes the
// 16 bytes at rsrc + soff + voff (soff wave-uniform) to lds_dst + 16*i.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, lds_char* lds_dst, unsigned voff,
                                           unsigned soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 16, voff, (int)soff, 0, 0);
}

// A wave-uniform value moved to scalar registers (the compiler cannot always
// prove uniformity on its own; a buffer descriptor must be scalar).
__device__ __forceinline__ unsigned long long to_sgpr(unsigned long long a) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

// Issue the loads of one tile of rows (K, V, Q or dO) into an LDS stage.  Load j of wave w
// fills tile rows j*RPL + w*RPW .. +RPW-1 (RPW = 64/DCH rows per wave load,
// RPL = NW*RPW rows per round of loads), all DCH chunks of each.
//   tile: address of the tile's first row (wave-uniform)
//   off: this lane's byte offset inside the tile for load 0; load j adds the
//        uniform j*RPL*rb (the swizzles repeat every 16 rows and RPL is a
//        multiple of 16 whenever LPW > 1, so the chunk part is the same)
//   dst: this wave's LDS chunks of load 0; load j adds j*RPL rows
//   nvalid: rows of the tile inside the sequence (rows past it re-read the
//        last valid row)
template <int LPW, int DCH, int BC, int NW>
__device__ __forceinline__ void issue_tile(unsigned long long tile, unsigned rb, unsigned off, lds_char* dst,
                                           int nvalid, int wave, int lane) {
    constexpr int RPW = 64 / DCH, RPL = NW * RPW;
    static_assert(LPW == 1 || RPL % 16 == 0, "load rounds must keep the swizzle phase");
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)to_sgpr(tile), (short)0, (int)(BC * rb), 0x00020000);
    if (nvalid >= BC) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) load_lds16(rsrc, dst + j * RPL * DCH * 16, off, j * RPL * rb);
    } else {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int row = j * RPL + wave * RPW + lane / DCH;
            const unsigned o = off - (unsigned)(row - min(row, nvalid - 1)) * rb;
            load_lds16(rsrc, dst + j * RPL * DCH * 16, o, j * RPL * rb);
        }
    }
}

// Sorted list of the indices t < n whose entry(t) is nonzero (a block-sparse
// mask row or column), built by one wave into LDS; returns the count.  Bits
// 12-15 of entry(t) are kept in the stored entry (t < 4096).  A round covers
// 256 indices: lane i tests 4i .. 4i+3, so the mask reads of a round are in
// flight together and a list of up to 256 entries costs one memory latency.
// An entry's position is the number of marked indices in the lower lanes
// (ballot + mbcnt per slot) plus those before it in its own lane.
template <typename F>
__device__ __forceinline__ int build_list(unsigned short* list, int n, int lane, F entry) {
    int count = 0;
    for (int base = 0; base < n; base += 256) {
        const int t0 = base + 4 * lane;
        unsigned e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = t0 + i < n ? entry(t0 + i) : 0u;
        int pos = count;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned long long bal = __builtin_amdgcn_ballot_w64(e[i] != 0u);
            pos += (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
            count += __builtin_popcountll(bal);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (e[i] != 0u) list[pos++] = (unsigned short)((unsigned)(t0 + i) | (e[i] & 0xF000u));
    }
    return count;
}

// A d x 32 accumulator of one wave (lane column = the output row, registers
// = d: acc[db][r] is row col, element db*32 + (r/4)*8 + hi*4 + r%4) times
// `mul`, written as rows of the output.  As accumulated, the lanes of row c
// (col c, hi 0 and 1) hold its 16-byte pieces 2m + hi (m = 4 db + g, g =
// r/4): one store per register set would write 32 bytes into each of 32
// rows.  v_permlane16_swap trades the pieces of two adjacent m, 2m' and
// 2m' + 1, between the lanes of rows c and c + 16 (c < 16): afterwards the
// first register set of the four lanes of cols c and c + 16 holds pieces
// 4m' .. 4m' + 3 of row c, the second those of row c + 16, so every store
// writes 64 contiguous, aligned bytes into each of 16 rows (half the write
// requests).  Every lane must be active; rows at or past n_rows are not
// stored.  The accumulator is scaled and swapped in place (it is dead
// afterwards).  row0 points at element 0 of the wave's first row; rows are
// row_elems elements apart; OUT_BF16 rounds to bf16 (else fp32).
// SITE: each call site instantiates its own copy (one copy inlined into two
// kernels changed how the compiler allocated the other kernel's registers).
__device__ __forceinline__ void swap_rows16(unsigned& a, unsigned& b) {
    // lanes 16..31 and 48..63 of a trade with lanes 0..15 and 32..47 of b
    // (the s_nop covers the VALU-write -> permlane-read hazard)
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

template <int D, bool OUT_BF16, int SITE>
__device__ __forceinline__ void store_acc_rows(f32x16 (&acc)[D / 32], float mul, char* row0, long long row_elems,
                                               int n_rows, int col, int hi) {
    constexpr int DB = D / 32, ES = OUT_BF16 ? 2 : 4;
    const int sel = col >> 4;
    const int r = col & 15;
    const bool ok0 = r < n_rows, ok1 = r + 16 < n_rows;
    char* const p0 = row0 + (long long)r * row_elems * ES;   // row r
    char* const p1 = p0 + 16LL * row_elems * ES;              // row r + 16
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        acc[db] *= mul;
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            // elements 8 gp .. 8 gp + 3: piece 2m' + hi (g = 2 gp) of this
            // lane's row; 8 gp + 4 .. + 7: piece 2m' + 2 + hi (g = 2 gp + 1).
            // Swapped, elements e0.. hold row r and e0 + 4.. row r + 16, piece
            // 8 db + 4 gp + 2 sel + hi of that row.
            const int e0 = 8 * gp;
            const int dd = db * 32 + gp * 16 + sel * 8 + hi * 4;
            if constexpr (OUT_BF16) {
                unsigned x0 = pack_bf16x2(acc[db][e0], acc[db][e0 + 1]);
                unsigned x1 = pack_bf16x2(acc[db][e0 + 2], acc[db][e0 + 3]);
                unsigned y0 = pack_bf16x2(acc[db][e0 + 4], acc[db][e0 + 5]);
                unsigned y1 = pack_bf16x2(acc[db][e0 + 6], acc[db][e0 + 7]);
                swap_rows16(x0, y0);
                swap_rows16(x1, y1);
                if (ok0) *(u32x2*)(p0 + dd * 2) = (u32x2){x0, x1};
                if (ok1) *(u32x2*)(p1 + dd * 2) = (u32x2){y0, y1};
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // (through a float: a bit cast of a vector element itself
                    // reads element 0)
                    const float fx = acc[db][e0 + w], fy = acc[db][e0 + 4 + w];
                    unsigned x = __builtin_bit_cast(unsigned, fx);
                    unsigned y = __builtin_bit_cast(unsigned, fy);
                    swap_rows16(x, y);
                    acc[db][e0 + w] = __builtin_bit_cast(float, x);
                    acc[db][e0 + 4 + w] = __builtin_bit_cast(float, y);
                }
                if (ok0)
                    *(float4*)(p0 + dd * 4) =
                        make_float4(acc[db][e0], acc[db][e0 + 1], acc[db][e0 + 2], acc[db][e0 + 3]);
                if (ok1)
                    *(float4*)(p1 + dd * 4) =
                        make_float4(acc[db][e0 + 4], acc[db][e0 + 5], acc[db][e0 + 6], acc[db][e0 + 7]);
            }
        }
    }
}

}  // namespace fa355

#endif  // FA355_COMMON_H
