// fa_decode.hip -- decode attention over a paged KV cache, gfx950.
//
// Nq new tokens per sequence (token t of sequence b at position
// L_b - Nq + t) attend to the sequence's L_b cached keys, which live in a
// paged cache: [num_blocks, block_size, Hkv, d] for K and for V, with
// logical block i of sequence b in physical block block_tables[b][i]
// ([nanhubrain] "GatherPAKVCache": block tables, and only the KV heads the
// grouped query heads need).  The page gathers the blocks into a contiguous
// copy first; here the attention kernel reads the blocks in place, so the
// cache is read from HBM exactly once and nothing is copied.
//
// The keys of a sequence are split into S chunks (split-KV); each (sequence,
// KV head, row tile, chunk) is one wavefront that runs the online softmax
// over its chunk and writes a partial (O_s normalised, LSE_s); a second
// kernel merges the chunks with the online-softmax merge of [nanhubrain]
// "online softmax mathematics" applied once per chunk:
//   LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
//
// gfx950 design:
//   * rows of a wave = the grouped query heads of one KV head times the new
//     tokens (32 per row tile), the MFMA B operand, held in VGPRs;
//   * a 32-key tile is read one tile ahead into registers, each load
//     instruction covering whole key rows (whole 128-byte lines: a lane
//     owning one key row, as the MFMA operand layout would have it, makes
//     an instruction touch 32 lines and runs at about half the bandwidth);
//     a tile starts at a multiple of 32 keys and blocks hold >= 16 keys, so
//     it spans at most two blocks, whose numbers are read one tile earlier
//     still, off the path of the tile's own loads;
//   * at the top of its step the tile goes from registers into LDS, K
//     swizzled for the 32-row ds_read_b128 of S^T = K Q^T
//     (v_mfma_f32_32x32x16_bf16), V for the transposing reads
//     (ds_read_b64_tr_b16) of O^T += V^T P^T;
//   * the four waves of a workgroup are independent (no barriers), 16 KB of
//     LDS each at d = 128 (one K and one V tile).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <atomic>

#include "fa355.h"
#include "fa_common.h"

namespace fa355 {

struct DecodeParams {
    const void* q;            // [B, Nq, H, d] bf16
    const void* k_cache;      // [num_blocks, block_size, Hkv, d] bf16
    const void* v_cache;
    const int* block_tables;  // [B, max_blocks]
    const int* seq_lens;      // [B]
    float* part_o;            // [B, H, Nq, S, d] fp32 partial outputs (normalised)
    float* part_lse;          // [B, H, Nq, S] fp32 partial log-sum-exps
    void* o;                  // [B, Nq, H, d]
    float* lse;               // [B, H, Nq] or NULL
    int B, H, Hkv, Nq;
    int group;                // H / Hkv
    int G;                    // rows per KV head: group * Nq
    int n_rt;                 // row tiles of 32: ceil(G / 32)
    int S;                    // key chunks per sequence
    int chunk;                // keys per chunk (multiple of 32)
    int bs_log2;              // log2(block_size)
    int max_blocks;
    float scale_log2;         // scale * log2(e) (tiny positive for scale 0)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_decode_split_kernel(DecodeParams p) {
    constexpr int NWV = 4, TK = 32, DCH = D / 8, KK = D / 16, DB = D / 32;
    constexpr int STAGE = TK * DCH;          // 16-byte slots of one K or V tile
    constexpr int RPI = 64 / DCH;            // key rows one load instruction covers
    constexpr int NLD = TK / RPI;            // load instructions per tile and operand
    __shared__ u32x4 smem[NWV * 2 * STAGE];

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int hi = lane >> 5;

    const int total = p.B * p.Hkv * p.n_rt * p.S;
    const int item = __builtin_amdgcn_workgroup_id_x() * NWV + wave;
    if (item >= total) return;                       // whole wave; no barriers below
    // KV head fastest: the waves of a workgroup read the same tokens of
    // neighbouring heads (one token's heads are contiguous in the cache)
    int rest = item;
    const int hk = rest % p.Hkv; rest /= p.Hkv;
    const int rt = rest % p.n_rt; rest /= p.n_rt;
    const int s = rest % p.S;
    const int b = rest / p.S;

    const int cap = p.max_blocks << p.bs_log2;
    const int L = min(max(p.seq_lens[b], 0), cap);
    const int k_begin = s * p.chunk;
    const int k_end = min(L, k_begin + p.chunk);

    // this lane's row (for the B operand and the outputs): row r of the
    // KV head's rows, token t = r / group, query head hk*group + r % group
    const int r = rt * 32 + col;
    const bool row_ok = r < p.G;
    const int t = row_ok ? r / p.group : 0;
    const int h = hk * p.group + (row_ok ? r % p.group : 0);
    // last key this row sees
    const int hi_key = CAUSAL ? min(L - 1, L - p.Nq + t) : L - 1;

    const long long q_row = (((long long)b * p.Nq + t) * p.H + h) * D;
    bf16x8 qreg[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const u32x4 x = row_ok ? *(const u32x4*)((const __bf16*)p.q + q_row + kk * 16 + hi * 8)
                               : (u32x4){0u, 0u, 0u, 0u};
        qreg[kk] = __builtin_bit_cast(bf16x8, x);
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m = -INFINITY, l0 = 0.f, l1 = 0.f;
    const float sl2 = p.scale_log2;

    // this wave's LDS: the K tile (row-major, chunks swizzled for the 32-row
    // ds_read_b128) and the V tile (swizzled for the transposing reads)
    u32x4* const kst = smem + wave * 2 * STAGE;
    lds_char* const vst = (lds_char*)(kst + STAGE);
    const int* table = p.block_tables + (long long)b * p.max_blocks;
    const long long head_off = (long long)hk * D;             // elements
    const long long row_stride = (long long)p.Hkv * D;        // elements per token of a block

    // Loads: instruction j of a tile reads key rows j*RPI .. j*RPI+RPI-1 whole
    // (lane: row j*RPI + lrow, chunk lch), so each instruction covers whole
    // 128-byte lines of the cache; the registers are then written to LDS in
    // the layouts the MFMA operands are read in.
    const int lrow = lane / DCH, lch = lane % DCH;
    // physical blocks of tile i's first and last key: a tile starts at a
    // multiple of 32 keys and blocks hold >= 16, so it spans at most these two
    auto tile_blocks = [&](int i, int& ba, int& bb) {
        const int k0 = k_begin + i * TK;
        ba = table[k0 >> p.bs_log2];
        bb = table[min(k0 + TK - 1, k_end - 1) >> p.bs_log2];
    };
    auto load_tile = [&](int i, int ba, int bb, u32x4 (&kr)[NLD], u32x4 (&vr)[NLD]) {
        const int k0 = k_begin + i * TK;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int key = min(k0 + j * RPI + lrow, k_end - 1);   // past the chunk: its last key (masked)
            const int blk = (key >> p.bs_log2) == (k0 >> p.bs_log2) ? ba : bb;
            const long long tok = ((long long)blk << p.bs_log2) + (key & ((1 << p.bs_log2) - 1));
            const long long off = (tok * row_stride + head_off) * 2 + lch * 16;   // bytes
            // each cached row is read once: nontemporal loads (the nt bit),
            // which stream past the caches (12 % faster than plain loads)
            kr[j] = __builtin_nontemporal_load((const u32x4*)((const char*)p.k_cache + off));
            vr[j] = __builtin_nontemporal_load((const u32x4*)((const char*)p.v_cache + off));
        }
    };

    const int n_tiles = k_end > k_begin ? (k_end - k_begin + TK - 1) / TK : 0;
    u32x4 kn[NLD], vn[NLD];
    int ba = 0, bb = 0;
    if (n_tiles > 0) {
        tile_blocks(0, ba, bb);
        load_tile(0, ba, bb, kn, vn);
        if (n_tiles > 1) tile_blocks(1, ba, bb);
    }

    const int tg = lane >> 4, ti = lane & 15;
    const int tr_row = hi * 4 + (ti >> 2);
    const int tr_dd = 16 * (tg & 1) + 4 * (ti & 3);

    for (int i = 0; i < n_tiles; ++i) {
        // tile i's rows are in kn/vn and tile i+1's block numbers in ba/bb
        // once every load is back
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // into LDS (the wave's reads of tile i-1 have all returned: their
        // data went into tile i-1's MFMAs)
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int r = j * RPI + lrow;
            kst[r * DCH + k_swz<D>(r, lch)] = kn[j];
            *(u32x4*)(vst + (r * DCH + v_swz<D>(r, lch)) * 16) = vn[j];
        }
        if (i + 1 < n_tiles) {
            load_tile(i + 1, ba, bb, kn, vn);
            if (i + 2 < n_tiles) tile_blocks(i + 2, ba, bb);
        }
        const int key0 = k_begin + i * TK;
        f32x16 sc;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const u32x4 kx = kst[col * DCH + k_swz<D>(col, 2 * kk + hi)];
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), qreg[kk],
                                                         kk == 0 ? f32x16{} : sc, 0, 0, 0);
        }
        // keys past the chunk or (causal) after the row's token -> -inf
        const int lim = min(k_end - 1, hi_key) - (key0 + hi * 4);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            sc[e] = ((e >> 2) * 8 + (e & 3)) <= lim ? sc[e] : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, sc[e]), sc[e + 1]);
        const float mt = pair_max(fmaxf(mx, sc[15])) * sl2;
        if (mt > m) {                                   // per lane; alpha = 0 when m was -inf
            const float alpha = __builtin_amdgcn_exp2f(m - mt);
            l0 *= alpha;
            l1 *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            m = mt;
        }
        const float nm = -fmaxf(m, -3.0e38f);           // finite for rows with no key yet
        unsigned pk[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * jj], sl2, nm));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * jj + 1], sl2, nm));
            l0 += e0;
            l1 += e1;
            pk[jj] = pack_bf16x2(e0, e1);
        }
        // O^T += V^T P^T: slots 0..3 of 16-key group u are keys 16u + hi*4 + 0..3,
        // slots 4..7 keys 16u + 8 + hi*4 + 0..3
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]});
            const int r0 = 16 * u + tr_row, r1 = r0 + 8;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dd = db * 32 + tr_dd;
                const int c = dd >> 3, w = (dd & 7) * 2;
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vst + r0 * (D * 2) + v_swz<D>(r0, c) * 16 + w));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vst + r1 * (D * 2) + v_swz<D>(r1, c) * 16 + w));
                const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
            }
        }
    }

    // partial result of this chunk: O_s = acc / l (0 if the row saw no key),
    // LSE_s = m + log2(l) in natural-log units (-inf if no key)
    const float l_tot = pair_sum(l0 + l1);
    if (row_ok) {
        const long long prow = (((long long)b * p.H + h) * p.Nq + t) * p.S + s;
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        float* po = p.part_o + prow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dd = db * 32 + g * 8 + hi * 4;
                *(float4*)(po + dd) = make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                                  oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
            }
        if (hi == 0) p.part_lse[prow] = l_tot > 0.f ? (m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
}

// Merge the S partial results of each (b, h, token) row: one wave per row.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void fa_decode_merge_kernel(DecodeParams p) {
    constexpr int EPL = D / 64;   // elements per lane
    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const long long row = (long long)__builtin_amdgcn_workgroup_id_x() * 4 + (tid >> 6);
    const long long n_rows = (long long)p.B * p.H * p.Nq;
    if (row >= n_rows) return;
    const int t = (int)(row % p.Nq);
    const long long bh = row / p.Nq;
    const int h = (int)(bh % p.H);
    const int b = (int)(bh / p.H);
    const float* pl = p.part_lse + row * p.S;
    float mx = -INFINITY;
    for (int s = 0; s < p.S; ++s) mx = fmaxf(mx, pl[s]);
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float z = 0.f;
    if (mx > -INFINITY) {
        for (int s = 0; s < p.S; ++s) {
            const float w = __expf(pl[s] - mx);        // 0 for an empty chunk (-inf)
            z += w;
            const float* po = p.part_o + (row * p.S + s) * D + lane * EPL;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, po[e], acc[e]);
        }
    }
    const float inv = z > 0.f ? 1.0f / z : 0.f;
    const long long orow = (((long long)b * p.Nq + t) * p.H + h) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float v = acc[e] * inv;
        if constexpr (OUT_BF16) ((__bf16*)p.o)[orow + e] = (__bf16)v;
        else ((float*)p.o)[orow + e] = v;
    }
    if (p.lse && lane == 0) p.lse[bh * p.Nq + t] = z > 0.f ? mx + __logf(z) : -INFINITY;
}

}  // namespace fa355

using namespace fa355;

namespace {

bool aligned_d(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// Key chunks per sequence: enough work items to give every CU's eight waves
// one item (2048 on MI355X), no chunk shorter than 256 keys.
int decode_splits(int B, int H, int Hkv, int Nq, int max_len) {
    const long long G = (long long)(H / Hkv) * Nq;
    const long long base = (long long)B * Hkv * ((G + 31) / 32);
    long long S = (2048 + base - 1) / base;
    const long long cap = (max_len + 255) / 256;
    if (S > cap) S = cap;
    if (S < 1) S = 1;
    return (int)S;
}

}  // namespace

extern "C" size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nq, int d, int max_seq_len) {
    if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Nq < 1 || d < 1 || max_seq_len < 1) return 0;
    const long long S = decode_splits(B, H, Hkv, Nq, max_seq_len);
    return (size_t)((long long)B * H * Nq * S * (d + 1) * 4);
}

namespace {

// The decode call behind fa_decode and fa_decode_noalloc.  With workspace ==
// nullptr the chunk partials go to this device's fixed scratch array (looked
// up only after every argument has been validated).
fa_status decode_impl(const void* q, const void* k_cache, const void* v_cache, const int* block_tables,
                      const int* seq_lens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                      int B, int H, int Hkv, int Nq, int d, int block_size, int max_blocks, float scale,
                      int causal, int in_dtype, int o_dtype, void* stream);

}  // namespace

extern "C" fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* block_tables,
                               const int* seq_lens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                               int B, int H, int Hkv, int Nq, int d, int block_size, int max_blocks, float scale,
                               int causal, int in_dtype, int o_dtype, void* stream) {
    if (!workspace) return FA_ERR_INVALID_ARG;
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, o, lse, workspace, workspace_bytes, B, H, Hkv,
                       Nq, d, block_size, max_blocks, scale, causal, in_dtype, o_dtype, stream);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace: the chunk partials live in a file-scope
// device array of fixed size.  Each GPU the library runs on holds its own
// copy until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (kept per device after
// the first call there), never through the array's name.

namespace {

constexpr size_t kScratchBytes = (size_t)FA_DECODE_NOALLOC_MAX_WORKSPACE;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// This device's address of `scratch` (nullptr on a HIP error).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace

extern "C" fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int* block_tables, const int* seq_lens, void* o, float* lse, int B, int H,
                                       int Hkv, int Nq, int d, int block_size, int max_blocks, float scale, int causal,
                                       int in_dtype, int o_dtype, void* stream) {
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, o, lse, nullptr, 0, B, H, Hkv, Nq, d,
                       block_size, max_blocks, scale, causal, in_dtype, o_dtype, stream);
}

namespace {

fa_status decode_impl(const void* q, const void* k_cache, const void* v_cache, const int* block_tables,
                      const int* seq_lens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                      int B, int H, int Hkv, int Nq, int d, int block_size, int max_blocks, float scale,
                      int causal, int in_dtype, int o_dtype, void* stream) {
    // ---- validation: no HIP call before it passes
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !o) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || d < 1 || max_blocks < 1) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (block_size < 16 || block_size > (1 << 20) || (block_size & (block_size - 1)) != 0) return FA_ERR_INVALID_ARG;
    if (in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_INVALID_ARG;
    if (o_dtype != FA_BF16 && o_dtype != FA_F32) return FA_ERR_INVALID_ARG;
    if (!aligned_d(q, 16) || !aligned_d(k_cache, 16) || !aligned_d(v_cache, 16) || !aligned_d(o, 16) ||
        (workspace && !aligned_d(workspace, 16)) || !aligned_d(block_tables, 4) || !aligned_d(seq_lens, 4))
        return FA_ERR_INVALID_ARG;
    if (lse && !aligned_d(lse, 4)) return FA_ERR_INVALID_ARG;
    if (scale != scale || fabsf(scale) == INFINITY) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    const long long max_len = (long long)max_blocks * block_size;
    if (max_len > INT32_MAX / 2) return FA_ERR_UNSUPPORTED;
    const size_t need = fa_decode_workspace_bytes(B, H, Hkv, Nq, d, (int)max_len);
    if (workspace) {
        if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
    } else {
        // the fixed scratch array: sizes whose partials do not fit are refused
        if (need > kScratchBytes) return FA_ERR_UNSUPPORTED;
    }
    const int S = decode_splits(B, H, Hkv, Nq, (int)max_len);
    const long long G = (long long)(H / Hkv) * Nq;
    const long long n_rt = (G + 31) / 32;
    const long long items = (long long)B * Hkv * n_rt * S;
    const long long rows = (long long)B * H * Nq;
    if (items > INT32_MAX || (items + 3) / 4 > INT32_MAX || (rows + 3) / 4 > INT32_MAX) return FA_ERR_UNSUPPORTED;

    if (!workspace) {
        workspace = scratch_for_current_device();
        if (!workspace) return FA_ERR_HIP;
    }
    if (scale < 0.f) scale = 1.0f / sqrtf((float)d);
    DecodeParams p;
    p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.block_tables = block_tables; p.seq_lens = seq_lens;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)workspace + rows * S * d;
    p.o = o; p.lse = lse;
    p.B = B; p.H = H; p.Hkv = Hkv; p.Nq = Nq;
    p.group = H / Hkv; p.G = (int)G; p.n_rt = (int)n_rt; p.S = S;
    const long long per = (max_len + S - 1) / S;
    p.chunk = (int)((per + 31) / 32 * 32);
    int lg = 0;
    while ((1 << lg) < block_size) ++lg;
    p.bs_log2 = lg;
    p.max_blocks = max_blocks;
    p.scale_log2 = scale > 0.f ? scale * kLog2e : 1e-30f;

    hipStream_t s = (hipStream_t)stream;
    const unsigned g1 = (unsigned)((items + 3) / 4), g2 = (unsigned)((rows + 3) / 4);
    const bool c = causal != 0, ob = o_dtype == FA_BF16;
    if (d == 128) {
        if (c) hipLaunchKernelGGL((fa_decode_split_kernel<128, true>), dim3(g1), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((fa_decode_split_kernel<128, false>), dim3(g1), dim3(256), 0, s, p);
    } else {
        if (c) hipLaunchKernelGGL((fa_decode_split_kernel<64, true>), dim3(g1), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((fa_decode_split_kernel<64, false>), dim3(g1), dim3(256), 0, s, p);
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    if (d == 128) {
        if (ob) hipLaunchKernelGGL((fa_decode_merge_kernel<128, true>), dim3(g2), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((fa_decode_merge_kernel<128, false>), dim3(g2), dim3(256), 0, s, p);
    } else {
        if (ob) hipLaunchKernelGGL((fa_decode_merge_kernel<64, true>), dim3(g2), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((fa_decode_merge_kernel<64, false>), dim3(g2), dim3(256), 0, s, p);
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace
