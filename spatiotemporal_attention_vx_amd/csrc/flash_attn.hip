// Full non-causal attention forward for gfx950 (flash style).
//
// What it computes: o = softmax(scale * Q K^T) V per (batch, head), over
// every token of the sequence, with an optional 3D RoPE applied to Q as it
// is loaded.  Source: the vidax paper (arXiv 2609.18077), §1 (full
// self-attention over all patch tokens of a multi-frame latent) and §2 "3D
// RoPE, 3D VAEs, and flash attention" (unmasked attention runs as flash
// attention, Dao et al. 2022: an online softmax over key tiles, so the
// N x N score matrix never exists).
//
// bf16 path (the hot one).  A workgroup of 8 waves owns 256 query rows of
// one (batch, head); each wave owns 32 rows.
//   * Scores are formed transposed, S^T (32 keys x 32 queries) = K_tile Q^T,
//     with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand,
//     the wave's Q^T fragment stays in VGPRs as the B operand.  In the
//     accumulator, lane l holds query l % 32 and 16 of the 32 keys, so the
//     row statistics are per lane plus one exchange with lane l ^ 32.
//   * The running row maximum m enters each score through the MFMA's C
//     operand (a register block holding -m), so the MFMA hands out s - m
//     with no per-score subtraction.  Without an LSE output, Q is also
//     multiplied by scale * log2(e) as it is loaded (rounded to bf16 once),
//     so s is already a base-2 score and the softmax weight is a bare
//     v_exp_f32.  That rounding moves every score of a row by a little and
//     the LSE with it (O does not feel it: softmax ignores a common shift),
//     so when the caller asks for the LSE the kernel keeps Q exactly as
//     stored, s is the raw dot product, and the weight is
//     v_exp_f32(c * (s - m)) with c = scale * log2(e) applied in fp32: one
//     more multiply per score, and an LSE exact up to fp32 and the bf16
//     rounding of the weights.
//   * m is raised lazily: only when some row's maximum exceeds it by more
//     than 2^8 in weight are the accumulator, the row sums and -m updated.
//     Weights are therefore <= 2^8, and the final division uses the m that
//     was actually subtracted, so the result is exact up to rounding.
//   * P^T is rounded to bf16 in registers and is directly the B operand of
//     O^T (d x 32 queries) += V^T P^T; the k index of that product runs
//     over keys in the order the S^T accumulator hands them out, and the
//     V^T fragments are read in that key order, so P never touches LDS.  The
//     row sum is taken over the same rounded weights with v_dot2_f32_bf16.
//   * K and V tiles go from global memory straight into LDS
//     (buffer_load_dwordx4 ... lds), row-major with a per-row 16-byte chunk
//     permutation, three buffers each; V^T fragments come from the
//     transposing LDS read ds_read_b64_tr_b16.  A tile is 16 KiB: 64 keys at
//     head_dim 128, 128 keys at head_dim 64, 32 MFMAs either way.
//   * Software pipeline, one key tile t per iteration:
//       X: S(t+1) = K(t+1) Q^T (MFMA)  interleaved with  exp/convert of S(t)
//       Y: O += V(t)^T P(t)   (MFMA)  interleaved with  row sum of P(t),
//          row max of S(t+1)
//     with the tile loads for later iterations spread over both phases and
//     one barrier per tile, halfway through Y: the waves pass it with the
//     rest of Y's MFMAs still to issue, which covers the LDS reads of the
//     next tile's first K fragments.  Each MFMA and the work meant to run under it
//     form a group that sched_barrier(0) keeps in order.
//   * Tiles past the sequence end are read through a buffer resource that
//     ends at the sequence end, so they load as zeros with no per-lane test;
//     scores of keys past the end are set to -inf in the last real tile.
//   * Key padding (a per-batch key range that takes no weight, e.g. the
//     padded tail of a joint sequence's text prefix): the tiles that hold
//     padded keys get -inf there, in the same rare branch as the last tile;
//     the key loop starts at a tile with a valid key (FaTiles), so the
//     running maximum is finite from the first tile on.
//   * Workgroups are remapped so each XCD works through a contiguous range
//     of (batch, head, query tile), keeping that head's K/V hot in its L2.
//
// f32 path: fp32 MFMA (v_mfma_f32_32x32x2_f32) for both products with the
// same transposed-score layout, K/V tiles staged through LDS, fp32 online
// softmax (described with the kernel below).
#include <type_traits>

#include "vx_device.h"



namespace vx {

constexpr int FA_MAX_PAD_BATCH = 64;   // batch entries a key-padding call may have

struct FaArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int64_t nq;               // query tokens
    int64_t nk;               // key/value tokens
    int64_t row_stride;       // elements between consecutive tokens (heads * D)
    int64_t batch_stride;     // elements between batch entries of q and o (nq * heads * D)
    int64_t kv_batch_stride;  // elements between batch entries of k and v (nk * heads * D)
    int heads;
    int dma_row_bytes;        // bytes per K/V token row (bf16), below 2^31
    int dma_max_rows;         // rows whose bytes fit a buffer resource (2^31 - 1); >= 128
    int n_qtiles;
    int64_t total_tiles;
    float scale;           // softmax scale (natural units)
    float scale_log2;      // scale * log2(e)
    float lazy_raw;        // FA_LAZY_LOG2 / scale_log2: the lazy threshold in raw dot units
    int use_rope;
    RopeArgs rope;
    // Key padding: keys pad_lo[b] <= j < pad_hi[b] of batch entry b take no
    // weight (lo == hi: none); at least one key of every entry is valid.
    int has_pad;
    int32_t pad_lo[FA_MAX_PAD_BATCH], pad_hi[FA_MAX_PAD_BATCH];
};

// ---------------------------------------------------------------- bf16 MFMA


// Key-tile order of one (batch, head).  Without key padding (PAD false)
// tiles run 0 .. nt - 1 and only the last can hold dead keys (past the
// end).  With padding, tiles run t0, t0 + 1, .., nt - 1, 0, .., t0 - 1: t0
// is 0 unless the padded range starts at key 0, in which case it is the
// tile holding key pad_hi, so the first tile always has a valid key and the
// running maximum starts finite.  Step indices at or past nt (prefetches
// beyond the last step) map to themselves and load as zeros.
template <bool PAD, int BC>
struct FaTiles {
    int nt, t0;
    int nk, lo, hi;   // the host keeps token counts below 2^31
    bool tail;
    __device__ FaTiles(const FaArgs& a, int64_t b) {
        nk = (int)a.nk;
        nt = (int)((nk + BC - 1) / BC);
        lo = PAD ? a.pad_lo[b] : 0;
        hi = PAD ? a.pad_hi[b] : 0;
        t0 = (PAD && lo == 0 && hi > 0) ? hi / BC : 0;
        tail = (nk % BC) != 0;
    }
    __device__ int at(int i) const {
        if constexpr (!PAD) return i;
        const int t = i + t0;
        return i >= nt ? i : (t >= nt ? t - nt : t);
    }
    // does tile tt hold a key past the end or a padded key
    __device__ bool masked(int tt) const {
        if constexpr (!PAD) return tail && tt == nt - 1;
        const int kv0 = tt * BC;
        return (tail && tt == nt - 1) || (kv0 < hi && kv0 + BC > lo);
    }
    __device__ bool dead(int key) const {
        if constexpr (!PAD) return key >= nk;
        return (key >= nk) | ((key >= lo) & (key < hi));
    }
};
// {x[l % 32], x[l % 32 + 32]} in some order, for every lane l, through
// v_permlane32_swap (no LDS round trip); max and sum are symmetric in them.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x with the bare v_exp_f32 (results below 2^-126 may flush to zero,
// which only drops weights already negligible against the row maximum).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// The running maximum may trail a row's true maximum by up to this many
// powers of two before the accumulator is rescaled (weights <= 2^8).
constexpr float FA_LAZY_LOG2 = 8.0f;

// Q fragment of one query row as the B operand of S^T = K Q^T: element
// (ks, e) is column ks * 16 + g * 8 + e.  The row is optionally rotated by
// the 3D RoPE (rounded to bf16, exactly as vx_rope3d_apply stores it), then
// (unless EXACT) multiplied by scale * log2(e) and rounded to bf16.  The lane holds
// columns g * 8 .. g * 8 + 7 of every 16: with adjacent pairs, or with the
// head split in halves (column c pairs with c + D/2, which is k-step
// ks + D/32, same e), both elements of each pair are in the lane; with
// band halves the partner is read from memory.
template <int D, bool EXACT>
__device__ __forceinline__ void load_q_fragment(const FaArgs& a, const uint16_t* qb, int64_t qi,
                                                int g, bf16x8_t* qf) {
    constexpr int NKS = D / 16;
    uint32_t u[NKS][4];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        uint4 w = {0u, 0u, 0u, 0u};
        if (qi < a.nq) w = *(const uint4*)(qb + qi * a.row_stride + ks * 16 + g * 8);
        u[ks][0] = w.x; u[ks][1] = w.y; u[ks][2] = w.z; u[ks][3] = w.w;
    }
    int tp = 0, hp = 0, wp = 0;
    const bool rot = a.use_rope && qi < a.nq && rope_token_pos(a.rope, qi, &tp, &hp, &wp);
    if (rot && a.rope.pairing == 0) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int pair = (ks * 16 + g * 8) / 2 + m;
                float c, s;
                rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &c, &s);
                float x0 = bf16_lo(u[ks][m]), x1 = bf16_hi(u[ks][m]);
                rope_rotate(x0, x1, c, s);
                u[ks][m] = pack_bf16x2(x0, x1);
            }
    } else if (rot && a.rope.pairing == 1) {
#pragma unroll
        for (int ks = 0; ks < NKS / 2; ++ks) {
            float f0[8], f1[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f0[2 * m] = bf16_lo(u[ks][m]);
                f0[2 * m + 1] = bf16_hi(u[ks][m]);
                f1[2 * m] = bf16_lo(u[ks + NKS / 2][m]);
                f1[2 * m + 1] = bf16_hi(u[ks + NKS / 2][m]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pair = ks * 16 + g * 8 + e;
                float c, s;
                rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &c, &s);
                rope_rotate(f0[e], f1[e], c, s);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                u[ks][m] = pack_bf16x2(f0[2 * m], f0[2 * m + 1]);
                u[ks + NKS / 2][m] = pack_bf16x2(f1[2 * m], f1[2 * m + 1]);
            }
        }
    } else if (rot) {
        const uint16_t* qrow = qb + qi * a.row_stride;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xe = (e & 1) ? bf16_hi(u[ks][e >> 1]) : bf16_lo(u[ks][e >> 1]);
                int pair, partner;
                bool second;
                rope_elem_pair(a.rope, ks * 16 + g * 8 + e, &pair, &partner, &second);
                float c, s;
                rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &c, &s);
                const float xp = __uint_as_float((uint32_t)qrow[partner] << 16);
                out[e] = rope_rotate_elem(xe, xp, second, c, s);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) u[ks][m] = pack_bf16x2(out[2 * m], out[2 * m + 1]);
        }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (!EXACT) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                u[ks][m] = pack_bf16x2(bf16_lo(u[ks][m]) * a.scale_log2,
                                       bf16_hi(u[ks][m]) * a.scale_log2);
        }
        qf[ks] = __builtin_bit_cast(bf16x8_t, uint4{u[ks][0], u[ks][1], u[ks][2], u[ks][3]});
    }
}

// ---------------------------------------------------------------- bf16 MFMA, DMA staging
//
// 8 waves and 256 query rows per workgroup.  The K and V tiles go from
// global memory straight into LDS (buffer_load_dwordx4 ... lds: one wave
// instruction moves 1 KiB), so no VGPR staging, no LDS store instructions
// and no register transpose.  A tile is 16 KiB whatever the head dim: 64
// keys at head_dim 128, 128 keys at head_dim 64, so both shapes issue 32
// MFMAs per tile and pay the per-tile costs (barrier, DMA issue) equally;
// head_dim 64 has twice the exponentials per MFMA.  Both tiles are kept
// row-major in LDS, three buffers each, with the 16-byte chunks of row r
// permuted by c -> c ^ swz(r) (chosen by which global chunk each lane
// fetches).  K fragments are plain 16-byte reads; V^T fragments for the P V
// product come from ds_read_b64_tr_b16, which transposes 4 keys x 16
// head-dim columns across each 16-lane group: source lane s reads 4
// consecutive columns of key s / 4, and lane i receives column i of the 4
// keys.

// chunk permutation of a 256-byte row (head_dim 128): a bijection on 0..15
// (16 consecutive rows hit 16 distinct chunks), and 4 consecutive rows
// differ in bits 2-3 (4 rows x 4 aligned chunks hit 16 distinct chunks)
__device__ __forceinline__ int dswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
// chunk permutation of a 128-byte row (head_dim 64), where a row's parity
// picks the half of the 256-byte bank window: among 16 consecutive rows the
// 8 of each parity get distinct values (16 lanes on 16 rows hit 16 distinct
// bank groups), and rows 4m and 4m + 2 differ in bit 2 (4 rows x 4 aligned
// chunks hit 16 distinct bank groups)
__device__ __forceinline__ int dswz64(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
template <int D>
__device__ __forceinline__ int dswz_d(int row) { return D == 128 ? dswz(row) : dswz64(row); }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ bf16x4_t lds_read_tr(const lds_u8* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
}

constexpr int FAD_WAVES = 8;

// EXACT (the caller wants the LSE): Q is kept as stored and scores are raw
// dot products, scaled by c = scale * log2(e) in fp32 before each
// exponential; every m and threshold below is in the MFMA's output units.
template <int D, bool PAD, bool EXACT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * FAD_WAVES, 64 * FAD_WAVES),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_dma_kernel(FaArgs a) {
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int BC = 8192 / D;                      // keys per tile (a tile is 16 KiB)
    constexpr int KB = BC / 32;                       // 32-key blocks of S^T per tile
    constexpr int KS = BC / 16;                       // 16-key steps of P V per tile
    constexpr int NSB = 3 * KB / 2;                   // S^T register blocks in rotation
    constexpr int BR = 32 * FAD_WAVES;                // query rows per workgroup
    constexpr int ROWB = 2 * D;                       // bytes per K or V row
    constexpr int CPR = ROWB / 16;                    // 16-byte chunks per row
    constexpr int RPI = 1024 / ROWB;                  // rows per DMA instruction
    constexpr int TILEB = BC * ROWB;                  // bytes per tile (16 KiB)
    constexpr int NI = TILEB / 1024 / FAD_WAVES;      // DMA instructions per wave per tensor (2)
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[6 * TILEB];
    lds_u8* const lds = (lds_u8*)lds_raw;             // K buffers 0-2, V buffers 3-5

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;

    const int64_t tile = xcd_remap(blockIdx.x, a.total_tiles);
    const int qt = (int)(tile % a.n_qtiles);
    const int64_t bh = tile / a.n_qtiles;
    const int h = (int)(bh % a.heads);
    const int64_t b = bh / a.heads;
    const int64_t off = b * a.batch_stride + (int64_t)h * D;
    const int64_t kv_off = b * a.kv_batch_stride + (int64_t)h * D;
    const uint16_t* kb = a.k + kv_off;
    const uint16_t* vb = a.v + kv_off;
    const int64_t nq = a.nq, nk = a.nk;
    const FaTiles<PAD, BC> tl(a, b);
    const int nt = tl.nt;

    const int64_t qi = (int64_t)qt * BR + wave * 32 + l32;
    bf16x8_t qf[NKK];
    load_q_fragment<D, EXACT>(a, a.q + off, qi, g, qf);
    // base-2 exponent of a score in the MFMA's output units
    const float cw = a.scale_log2;
    auto weight = [&](float s) { return fast_exp2(EXACT ? s * cw : s); };
    const float lazy = EXACT ? a.lazy_raw : FA_LAZY_LOG2;

    // ---- DMA: instruction m of this wave fills rows RPI I .. RPI I + RPI - 1
    // of the tile, I = wave * NI + m; lane L writes LDS bytes 16 L .. of that
    // KiB, i.e. row RPI I + L / CPR, chunk slot L % CPR, which holds global
    // chunk (L % CPR) ^ swz(row).
    const int64_t row_bytes = a.row_stride * 2;
    uint32_t goff[NI];
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        const int row = (wave * NI + m) * RPI + lane / CPR;
        goff[m] = (uint32_t)(row * row_bytes + (((lane % CPR) ^ dswz_d<D>(row)) << 4));
    }
    const int swave = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform, for M0
    // The DMA is written as inline assembly: with the builtin, the compiler
    // cannot tell the destination from the buffers being read and waits for
    // every DMA in flight (vmcnt(0)) before each V read.  Ordering is kept by
    // hand instead: an explicit vmcnt wait and the barrier publish a tile,
    // and no buffer is a DMA target while any wave may still read it.
    // The resource's size is clamped in 32-bit scalar arithmetic, branch-free
    // (token counts are below 2^30, so kv0 fits; int64 compares would go to
    // the VALU).  dma_max_rows >= 128 >= BC, so a clamped size still covers
    // the whole tile.
    // M0 is a reserved register, so the compiler warns that listing it as
    // clobbered does not make it save or restore it.  That is safe here only
    // because nothing the compiler generates in these kernels reads or
    // writes M0 (no LDS-direct, GWS, movrel or message instructions); the
    // host test suite compiles this file and checks exactly that.
    auto dma_one = [&](const uint16_t* base, int t, lds_u8* buf, int m) {
        const int kv0 = t * BC;
        const int rows_left = __builtin_elementwise_min(__builtin_elementwise_max(tl.nk - kv0, 0), a.dma_max_rows);
        const int bytes = rows_left * a.dma_row_bytes;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base + (int64_t)kv0 * a.row_stride), (short)0, bytes, 0x00020000);
        const uint32_t dst = (uint32_t)(uintptr_t)(buf + (swave * NI + m) * 1024);
        __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :
                         : "s"(dst), "v"(goff[m]), "s"(r)
                         : "m0");
    };
    auto dma = [&](const uint16_t* base, int t, lds_u8* buf) {
#pragma unroll
        for (int m = 0; m < NI; ++m) dma_one(base, t, buf, m);
    };
    auto kbuf = [&](int j) { return lds + j * TILEB; };
    auto vbuf = [&](int j) { return lds + (3 + j) * TILEB; };
    // Fragment reads use a per-lane register offset plus a compile-time
    // immediate (buffer and fragment), kept below the 64 KiB immediate
    // range: the V region's base is folded into the per-lane V offsets.

    // K fragment (kb2, kk): row kb2 * 32 + l32, chunk 2 kk + g
    uint32_t koff[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) koff[kk] = l32 * ROWB + (((2 * kk + g) ^ dswz_d<D>(l32)) << 4);
    auto kfrag = [&](int jk, int i) {   // K buffer jk (compile-time), fragment i
        return *(const bf16x8_t*)(lds + koff[i % NKK] + (jk * TILEB + (i / NKK) * 32 * ROWB));
    };
    // V^T fragment (db, kk), half r: keys kk*16 + 4 (2r + g) + s / 4 (the
    // S^T accumulator's key order), columns db*32 + 16 hh + 4 (s & 3)..+3,
    // with s = lane & 15, hh = (lane >> 4) & 1.  Fragments are numbered in
    // the order the P V product takes them: 16-key step kk outer, 32-column
    // block db inner, so consecutive MFMAs go to different accumulators.
    uint32_t voff[2][NDB];
    {
        const int s_ = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int row = 4 * (2 * r + g) + (s_ >> 2);
                const int chunk = 4 * db + 2 * hh + ((s_ & 3) >> 1);
                voff[r][db] = 3 * TILEB + row * ROWB + ((chunk ^ dswz_d<D>(row)) << 4) + (s_ & 1) * 8;
            }
    }
    auto vfrag = [&](int jv, int i) {   // V buffer jv (compile-time), fragment i
        const int db = i % NDB, kk = i / NDB;
        const bf16x4_t lo = lds_read_tr(lds + voff[0][db] + (jv * TILEB + kk * 16 * ROWB));
        const bf16x4_t hi = lds_read_tr(lds + voff[1][db] + (jv * TILEB + kk * 16 * ROWB));
        return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    // S^T of one tile is KB register blocks of 16 (32 keys each).  They
    // rotate through NSB = 3 KB / 2 blocks: step J (= t % 3) reads S(t) from
    // blocks (J KB + k) % NSB and writes S(t+1) to (J KB + KB + k) % NSB, so
    // S(t+1)'s upper half takes the place of S(t)'s lower half, which the
    // exponentials have consumed by then.
    f32x16_t sb[NSB];
    auto mask_tile = [&](auto jm, int t) {   // S(t) held in step jm's "next" blocks
        constexpr int J = decltype(jm)::value;
        const int kv0 = t * BC;
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kv0 + k * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (tl.dead(key)) sb[(J * KB + KB + k) % NSB][i] = -__builtin_inff();
            }
    };
    auto row_max = [&](auto jm) {
        constexpr int J = decltype(jm)::value;
        float mx = sb[(J * KB + KB) % NSB][0];
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sb[(J * KB + KB + k) % NSB][i]);
        return half_max(mx);
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16_t{};
    f32x16_t negm = f32x16_t{};   // -m in every slot: the C operand of the first k-step
    float m_ref, l_run = 0.f, mx_next = 0.f;

    // ---- prologue: K(0..2), V(0..1) into LDS; S(0) into blocks 0 .. KB-1
    // (the "next" blocks of step J = 2); m from tile 0 (step indices; tl.at
    // maps them to key tiles)
    dma(kb, tl.at(0), kbuf(0));
    dma(kb, tl.at(1), kbuf(1));
    dma(kb, tl.at(2), kbuf(2));
    dma(vb, tl.at(0), vbuf(0));
    dma(vb, tl.at(1), vbuf(1));
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's tiles have landed
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            sb[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(0, k * NKK + kk), qf[kk],
                                                            kk == 0 ? negm : sb[k], 0, 0, 0);
    __syncthreads();              // K buffer 0 is refilled in the first iteration
    if (tl.masked(tl.at(0))) mask_tile(std::integral_constant<int, 2>{}, tl.at(0));
    {
        const float mx = row_max(std::integral_constant<int, 2>{});
        m_ref = mx;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -mx;
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
            for (int i = 0; i < 16; ++i) sb[k][i] -= mx;
    }
    bf16x8_t kf[3];
    kf[0] = kfrag(1, 0);
    kf[1] = kfrag(1, 1);

    // Step t uses K buffers (t+1) % 3 (read), (t+2) % 3 (next tile's first
    // fragments), t % 3 (DMA target) and V buffers t % 3 (read), (t+2) % 3
    // (DMA target, refilled after the step's barrier); the loop is unrolled
    // three times so all are compile-time.
    auto step = [&](auto tm, int t) {
        constexpr int J = decltype(tm)::value;   // t % 3
        constexpr int NX = KB * NKK;          // K fragments (MFMAs) of S(t+1)
        constexpr int WPM = 8 * KB / NX;      // P words (2 weights) per MFMA
        constexpr int NY = NDB * KS;          // V^T fragments (MFMAs) of P V
        constexpr int MPM = 16 * KB / (NY / 2);   // scores per MFMA in the row max
        constexpr int SPM = 8 * KB / (NY / 2);    // P words per MFMA in the row sum
        constexpr int j0 = J, j1 = (J + 1) % 3, j2 = (J + 2) % 3;
        auto cur = [](int k) { return (J * KB + k) % NSB; };        // S(t) block k
        auto nxt = [](int k) { return (J * KB + KB + k) % NSB; };   // S(t+1) block k
        // ---- X: S(t+1) = K(t+1) Q^T - m  ||  P(t) = 2^(S(t) - m)
        bf16x8_t vf[3];
        uint32_t pw[8 * KB];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            if (i + 2 < NX) kf[(i + 2) % 3] = kfrag(j1, i + 2);
            const int kb2 = i / NKK, kk = i % NKK;
            f32x16_t& d = sb[nxt(kb2)];
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % 3], qf[kk], kk == 0 ? negm : d, 0, 0, 0);
            // nothing after the MFMA moves above it: otherwise the first
            // group of a step may start with its exponentials and leave the
            // MFMA unit idle at the step boundary (+0.2% at head_dim 128,
            // +0.9% at 64, bit-identical)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < WPM; ++e) {
                const int w = i * WPM + e;   // weights 2w, 2w+1: block (2w) / 16 of S(t)
                const f32x16_t& src = sb[cur((2 * w) / 16)];
                const float p0 = weight(src[(2 * w) & 15]);
                const float p1 = weight(src[(2 * w + 1) & 15]);
                pw[w] = pack_bf16x2(p0, p1);
            }
            // K(t+3) where K(t) was, one request every NX / NI groups
            if (i % (NX / NI) == 0) dma_one(kb, tl.at(t + 3), kbuf(j0), i / (NX / NI));
            if (i + 2 == NX) vf[0] = vfrag(j0, 0);
            if (i + 1 == NX) vf[1] = vfrag(j0, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // P(t) words 4 kk .. 4 kk + 3 as the B operand of 16-key step kk
        auto pb = [&](int kk) {
            return __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]});
        };
        // ---- Y: O += V(t)^T P(t)  ||  row sum of P(t); row max of S(t+1);
        // first K(t+2) fragments
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        float mx = -__builtin_inff(), psum = l_run;
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            if (i == NY / 2) {
                // Mid-step barrier.  Before it each wave waits for its own
                // share of K(t+2) and V(t+1) (the K(t+3) requests issued in
                // X may stay in flight; vmcnt counts only the tile DMAs);
                // after it those tiles are whole in LDS, and every wave is
                // done with K(t+1) and V(t-1), whose buffers may be refilled.
                // The first K(t+2) fragments are read here, so the next
                // step's first MFMA does not wait on LDS.  No fence: only the
                // DMAs need ordering, and the explicit wait covers them.
                __builtin_amdgcn_s_waitcnt(0x0F70 | NI);
                __asm__ volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                __asm__ volatile("" ::: "memory");
                kf[0] = kfrag(j2, 0);
                kf[1] = kfrag(j2, 1);
            }
            if (i + 2 < NY) vf[(i + 2) % 3] = vfrag(j0, i + 2);
            acc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % 3], pb(i / NDB), acc[i % NDB], 0, 0, 0);
            // V(t+2) where V(t-1) was, after the barrier, one request every
            // NY / 2 / NI groups
            if (i >= NY / 2 && (i - NY / 2) % (NY / 2 / NI) == 0)
                dma_one(vb, tl.at(t + 2), vbuf(j2), (i - NY / 2) / (NY / 2 / NI));
            if (i < NY / 2) {
#pragma unroll
                for (int e = 0; e < SPM; ++e)
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i * SPM + e]),
                                                           one, psum, false);
                __asm__ volatile("" ::"v"(psum));   // keep the row sum in this group
            } else {
#pragma unroll
                for (int e = 0; e < MPM; ++e) {
                    const int j = (i - NY / 2) * MPM + e;
                    mx = fmaxf(mx, sb[nxt(j / 16)][j & 15]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run = psum;
        mx_next = half_max(mx);
        // ---- keys past the end or padded take no weight
        if (t + 1 < nt && tl.masked(tl.at(t + 1))) {
            mask_tile(tm, tl.at(t + 1));
            mx_next = row_max(tm);
        }
        // ---- lazy rescale for S(t+1) (rare after the first tiles; laid out
        // off the straight-line path, so a step that skips it does not jump)
        if (__builtin_expect(t + 1 < nt && __builtin_amdgcn_ballot_w64(mx_next > lazy) != 0, 0)) {
            const float delta = fmaxf(mx_next, 0.f);
            const float alpha = weight(-delta);
            m_ref += delta;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) acc[i] *= alpha;
            // -m is rewritten in place: a plain assignment here makes the
            // register allocator copy the block on every tile.
            const float nm = -m_ref;
#pragma unroll
            for (int i = 0; i < 16; ++i) __asm__ volatile("v_mov_b32 %0, %1" : "+v"(negm[i]) : "v"(nm));
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int i = 0; i < 16; ++i) sb[nxt(k)][i] -= delta;
        }
    };

    // S(0) sits in blocks 0 .. KB-1, the "current" blocks of step 0.
    for (int t = 0; t < nt; t += 3) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 >= nt) break;
        step(std::integral_constant<int, 1>{}, t + 1);
        if (t + 2 >= nt) break;
        step(std::integral_constant<int, 2>{}, t + 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // no DMA may land after the workgroup's LDS is released

    const float l_tot = half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (qi < nq) {
        uint16_t* ob = a.o + off + qi * a.row_stride;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x16_t& c = acc[db];
                uint2 w;
                w.x = pack_bf16x2(c[4 * r + 0] * inv, c[4 * r + 1] * inv);
                w.y = pack_bf16x2(c[4 * r + 2] * inv, c[4 * r + 3] * inv);
                *(uint2*)(ob + db * 32 + 8 * r + 4 * g) = w;
            }
        if (a.lse != nullptr && g == 0)
            a.lse[bh * nq + qi] =
                ((EXACT ? m_ref * cw : m_ref) + __builtin_log2f(l_tot)) * 0.69314718055994531f;
    }
}

// ---------------------------------------------------------------- f32 MFMA
//
// fp32 inputs and outputs (a DiT kept in fp32 end to end), fp32 products
// and sums throughout: v_mfma_f32_32x32x2_f32 for both products.  A
// workgroup of 4 waves owns 128 query rows of one (batch, head); each wave
// owns 32.  Lane l = (c, h) with c = l % 32, h = l / 32.
//   * S^T (32 keys x 32 queries) = K_tile Q^T over D / 2 k-steps; k-step s
//     takes head-dim column h * D/2 + s in lane half h, so a lane's Q^T
//     fragment is one contiguous half of its query row (in registers) and
//     its K operand for four k-steps is one 16-byte LDS read.  The
//     accumulator holds query c and keys 8 (i / 4) + 4 h + i % 4 (i < 16).
//   * Online softmax in fp32 on raw dot products: row max over the lane's 16
//     keys and its partner lane (l ^ 32); weights exp2((s - m) * scale *
//     log2 e); a row with no valid key yet keeps zero weight.
//   * O^T (D x 32 queries) += V^T P^T: P^T is the score accumulator itself,
//     register i being the B operand of the k-step over keys 8 (i / 4) + i % 4
//     (half 0) and 8 (i / 4) + 4 + i % 4 (half 1); the A operand is V at
//     those keys read from LDS, so P never moves.
//   * K and V tiles of 32 keys are staged in LDS (rows padded by 16 bytes),
//     double-buffered: the next tile's global loads are issued into
//     registers before the current tile's products and stored to the other
//     buffer after them, one barrier per tile.  Keys past the end load as
//     zeros and, like padded keys, get -inf scores.
constexpr int FA32_WAVES = 4;
constexpr int FA32_BC = 32;    // keys per tile

template <int D, bool PAD>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * FA32_WAVES, 64 * FA32_WAVES),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_f32_mfma_kernel(FaArgs a) {
    constexpr int HALF = D / 2;                     // head-dim columns of a lane half
    constexpr int NDB = D / 32;                     // 32-row blocks of O^T
    constexpr int LROW = D + 4;                     // LDS row stride, floats
    constexpr int TILE = FA32_BC * LROW;            // floats per staged tile
    constexpr int F4ROW = D / 4;                    // float4 per tile row
    constexpr int NF4 = FA32_BC * F4ROW / (64 * FA32_WAVES);   // float4 per thread per tensor
    static_assert(NF4 * 64 * FA32_WAVES == FA32_BC * F4ROW, "tile rows split evenly");
    __shared__ __attribute__((aligned(16))) float lds[2 * 2 * TILE];   // [buffer][K, V]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
    const int64_t tile = xcd_remap(blockIdx.x, a.total_tiles);
    const int qt = (int)(tile % a.n_qtiles);
    const int64_t bh = tile / a.n_qtiles;
    const int hd = (int)(bh % a.heads);
    const int64_t b = bh / a.heads;
    const float* qb = (const float*)a.q + b * a.batch_stride + (int64_t)hd * D;
    const float* kb = (const float*)a.k + b * a.kv_batch_stride + (int64_t)hd * D;
    const float* vb = (const float*)a.v + b * a.kv_batch_stride + (int64_t)hd * D;
    const int64_t nq = a.nq;
    const int nk = (int)a.nk;
    const FaTiles<PAD, FA32_BC> tl(a, b);
    const int nt = tl.nt;

    // ---- Q^T fragment: columns h * HALF .. h * HALF + HALF - 1 of query qi,
    // rotated by the 3D RoPE if asked (the same expressions as
    // vx_rope3d_apply, so fused and separate rotation agree bit for bit)
    const int64_t qi = (int64_t)qt * (32 * FA32_WAVES) + wave * 32 + c;
    float qf[HALF];
    {
        const float* qrow = qb + qi * a.row_stride + h * HALF;
#pragma unroll
        for (int u = 0; u < HALF; u += 4) {
            float4 w = {0.f, 0.f, 0.f, 0.f};
            if (qi < nq) w = *(const float4*)(qrow + u);
            qf[u] = w.x; qf[u + 1] = w.y; qf[u + 2] = w.z; qf[u + 3] = w.w;
        }
        int tp = 0, hp = 0, wp = 0;
        const bool rot = a.use_rope && qi < nq && rope_token_pos(a.rope, qi, &tp, &hp, &wp);
        if (rot && a.rope.pairing == 0) {
#pragma unroll
            for (int m = 0; m < HALF / 2; ++m) {
                const int pair = h * (HALF / 2) + m;
                float cv, sv;
                rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &cv, &sv);
                rope_rotate(qf[2 * m], qf[2 * m + 1], cv, sv);
            }
        } else if (rot) {
            // half-split pairings: partners are read from the row in memory
            const float* full = qb + qi * a.row_stride;
            float out[HALF];
#pragma unroll
            for (int e = 0; e < HALF; ++e) {
                int pair, partner;
                bool second;
                rope_elem_pair(a.rope, h * HALF + e, &pair, &partner, &second);
                float cv, sv;
                rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &cv, &sv);
                out[e] = rope_rotate_elem(qf[e], full[partner], second, cv, sv);
            }
#pragma unroll
            for (int e = 0; e < HALF; ++e) qf[e] = out[e];
        }
    }

    // ---- tile staging: float4 f = tid + 256 j of a tile is row f / F4ROW,
    // columns 4 (f % F4ROW) ..; rows past the key count load as zeros
    float4 rk[NF4], rv[NF4];
    auto stage_load = [&](int t) {
        const int kv0 = t * FA32_BC;
#pragma unroll
        for (int j = 0; j < NF4; ++j) {
            const int f = tid + 64 * FA32_WAVES * j, row = f / F4ROW, col = f % F4ROW;
            const int key = kv0 + row;
            rk[j] = rv[j] = float4{0.f, 0.f, 0.f, 0.f};
            if (key < nk) {
                rk[j] = *(const float4*)(kb + (int64_t)key * a.row_stride + col * 4);
                rv[j] = *(const float4*)(vb + (int64_t)key * a.row_stride + col * 4);
            }
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NF4; ++j) {
            const int f = tid + 64 * FA32_WAVES * j, row = f / F4ROW, col = f % F4ROW;
            *(float4*)(lds + (2 * buf) * TILE + row * LROW + col * 4) = rk[j];
            *(float4*)(lds + (2 * buf + 1) * TILE + row * LROW + col * 4) = rv[j];
        }
    };
    stage_load(0);
    stage_store(0);
    __syncthreads();

    const float cl = a.scale_log2;      // scale * log2(e)
    f32x16_t o[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[j] = f32x16_t{};
    float m_run = -__builtin_inff(), l_run = 0.f;

    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        const float* kt = lds + (2 * buf) * TILE;
        const float* vt = lds + (2 * buf + 1) * TILE;

        // S^T = K Q^T
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int u = 0; u < HALF; u += 4) {
            const float4 k4 = *(const float4*)(kt + c * LROW + h * HALF + u);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.x, qf[u], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.y, qf[u + 1], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.z, qf[u + 2], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.w, qf[u + 3], s, 0, 0, 0);
            if ((u & 15) == 12) __builtin_amdgcn_sched_barrier(0);
        }
        // the next tile's loads, in flight under the softmax and P V
        if (t + 1 < nt) stage_load(t + 1);
        if (tl.masked(t)) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (tl.dead(t * FA32_BC + 8 * (i >> 2) + 4 * h + (i & 3))) s[i] = -__builtin_inff();
        }

        // online softmax (raw dot units; -inf stands for "no valid key yet")
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float m_new = fmaxf(m_run, half_max(mx));
        const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * cl);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = __builtin_amdgcn_exp2f((s[i] - m_use) * cl);
            ps += s[i];
        }
        l_run = __builtin_fmaf(l_run, alpha, ps);
#pragma unroll
        for (int j = 0; j < NDB; ++j) o[j] *= alpha;
        m_run = m_new;

        // O^T += V^T P^T
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
            for (int j = 0; j < NDB; ++j)
                o[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[key * LROW + 32 * j + c], s[i], o[j],
                                                             0, 0, 0);
            // V reads stay within a few k-steps of their MFMAs (hoisting
            // them all would not fit the register file)
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        // every wave is done with the other buffer (read in the previous
        // tile, before the barrier that ended it)
        if (t + 1 < nt) stage_store(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane (c, h) holds O^T rows 32 j + 8 r + 4 h .. + 3 of query c
    const float l_tot = half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (qi < nq) {
        float* orow = (float*)a.o + b * a.batch_stride + (int64_t)hd * D + qi * a.row_stride;
#pragma unroll
        for (int j = 0; j < NDB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *(float4*)(orow + 32 * j + 8 * r + 4 * h) =
                    float4{o[j][4 * r] * inv, o[j][4 * r + 1] * inv, o[j][4 * r + 2] * inv,
                           o[j][4 * r + 3] * inv};
        if (a.lse != nullptr && h == 0) a.lse[bh * nq + qi] = m_run * a.scale + logf(l_tot);
    }
}


// ---------------------------------------------------------------- launch

// Query rows one workgroup covers (the host sizes the grid with it).
int flash_attn_rows_per_workgroup(bool bf16, int64_t head_dim) {
    (void)head_dim;
    return bf16 ? 32 * FAD_WAVES : 32 * FA32_WAVES;
}

hipError_t launch_flash_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t batch, int64_t nq, int64_t nk, int64_t heads,
                             int64_t head_dim, float scale, const RopeArgs* rope,
                             const int32_t* key_pad, bool bf16, hipStream_t st) {
    FaArgs a;
    a.has_pad = key_pad != nullptr;
    for (int i = 0; i < FA_MAX_PAD_BATCH; ++i) {
        const bool in = key_pad != nullptr && i < batch;
        a.pad_lo[i] = in ? key_pad[2 * i] : 0;
        a.pad_hi[i] = in ? key_pad[2 * i + 1] : 0;
    }
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
    a.lse = lse;
    a.nq = nq;
    a.nk = nk;
    a.row_stride = heads * head_dim;
    a.batch_stride = nq * heads * head_dim;
    a.kv_batch_stride = nk * heads * head_dim;
    a.heads = (int)heads;
    a.dma_row_bytes = (int)(heads * head_dim * 2);
    a.dma_max_rows = 0x7fffffff / a.dma_row_bytes;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.lazy_raw = FA_LAZY_LOG2 / a.scale_log2;
    a.use_rope = rope != nullptr;
    if (rope) a.rope = *rope;
    else a.rope = RopeArgs{};

    const int rows_per_wg = flash_attn_rows_per_workgroup(bf16, head_dim);
    a.n_qtiles = (int)((nq + rows_per_wg - 1) / rows_per_wg);
    a.total_tiles = batch * heads * a.n_qtiles;
    const dim3 grid((unsigned)a.total_tiles);
    if (bf16) {
        // the exact-scale instruction stream only when the LSE is wanted
        const int code = (head_dim == 128 ? 4 : 0) | (a.has_pad ? 2 : 0) | (lse != nullptr ? 1 : 0);
        const dim3 block(64 * FAD_WAVES);
#define VX_FA(C, D, P, E) \
    case C: hipLaunchKernelGGL((fa_fwd_bf16_dma_kernel<D, P, E>), grid, block, 0, st, a); break;
        switch (code) {
            VX_FA(0, 64, false, false)
            VX_FA(1, 64, false, true)
            VX_FA(2, 64, true, false)
            VX_FA(3, 64, true, true)
            VX_FA(4, 128, false, false)
            VX_FA(5, 128, false, true)
            VX_FA(6, 128, true, false)
            VX_FA(7, 128, true, true)
        }
#undef VX_FA
    } else {
        const dim3 block(64 * FA32_WAVES);
        if (head_dim == 128 && a.has_pad)
            hipLaunchKernelGGL((fa_fwd_f32_mfma_kernel<128, true>), grid, block, 0, st, a);
        else if (head_dim == 128)
            hipLaunchKernelGGL((fa_fwd_f32_mfma_kernel<128, false>), grid, block, 0, st, a);
        else if (a.has_pad)
            hipLaunchKernelGGL((fa_fwd_f32_mfma_kernel<64, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((fa_fwd_f32_mfma_kernel<64, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}


}  // namespace vx
