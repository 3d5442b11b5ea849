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
//   * Everything is in base-2 units: Q is multiplied by scale * log2(e) as
//     it is loaded, and the running row maximum m enters each score through
//     the MFMA's C operand (a register block holding -m), so the MFMA hands
//     out u - m directly and the softmax weight is a bare v_exp_f32.
//   * m is raised lazily: only when some row's maximum exceeds it by more
//     than 2^8 in weight are the accumulator, the row sums and -m updated.
//     Weights are therefore <= 2^8, and the final division uses the m that
//     was actually subtracted, so the result is exact up to rounding.
//   * P^T is rounded to bf16 in registers and is directly the B operand of
//     O^T (d x 32 queries) += V^T P^T; the k index of that product runs
//     over keys in the order the S^T accumulator hands them out, and the
//     V^T fragments are read in that key order, so P never touches LDS.  The
//     row sum is taken over the same rounded weights with v_dot2_f32_bf16.
//   * Software pipeline, one key tile t per iteration:
//       X: S(t+1) = K(t+1) Q^T (MFMA)  interleaved with  exp/convert of S(t)
//       Y: O += V(t)^T P(t)   (MFMA)  interleaved with  row sum of P(t),
//          row max of S(t+1)
//     with the tile loads for later iterations spread over both phases and
//     one barrier per tile.  Each MFMA and the work meant to run under it
//     form a group that sched_barrier(0) keeps in order.
//   * head_dim 128 (fa_fwd_bf16_dma_kernel): K and V tiles go from global
//     memory straight into LDS (buffer_load_dwordx4 ... lds), row-major with
//     a per-row 16-byte chunk permutation, three buffers each; V^T fragments
//     come from the transposing LDS read ds_read_b64_tr_b16.
//     head_dim 64 (fa_fwd_bf16_kernel): K and V tiles are staged through
//     VGPRs; V is transposed in registers and stored as V^T with an XOR
//     chunk permutation, K with padded rows.
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
// f32 path (small problems and parity): a plain VALU kernel, a few lanes per
// query, K/V tiles staged through LDS, exact expf online softmax.
#include <type_traits>

#include "vx_device.h"

#ifndef VX_FA_WAVES
#define VX_FA_WAVES 8
#endif
#ifndef VX_FA_QG
#define VX_FA_QG 1
#endif


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
    int n_qtiles;
    int64_t total_tiles;
    float scale;           // softmax scale (natural units)
    float scale_log2;      // scale * log2(e)
    int use_rope;
    RopeArgs rope;
    // Key padding: keys pad_lo[b] <= j < pad_hi[b] of batch entry b take no
    // weight (lo == hi: none); at least one key of every entry is valid.
    int has_pad;
    int32_t pad_lo[FA_MAX_PAD_BATCH], pad_hi[FA_MAX_PAD_BATCH];
};

// ---------------------------------------------------------------- bf16 MFMA

constexpr int FA_BC = 64;    // keys per tile

// Key-tile order of one (batch, head).  Without key padding (PAD false)
// tiles run 0 .. nt - 1 and only the last can hold dead keys (past the
// end).  With padding, tiles run t0, t0 + 1, .., nt - 1, 0, .., t0 - 1: t0
// is 0 unless the padded range starts at key 0, in which case it is the
// tile holding key pad_hi, so the first tile always has a valid key and the
// running maximum starts finite.  Step indices at or past nt (prefetches
// beyond the last step) map to themselves and load as zeros.
template <bool PAD>
struct FaTiles {
    int nt, t0;
    int64_t nk, lo, hi;
    bool tail;
    __device__ FaTiles(const FaArgs& a, int64_t b) {
        nk = a.nk;
        nt = (int)((nk + FA_BC - 1) / FA_BC);
        lo = PAD ? a.pad_lo[b] : 0;
        hi = PAD ? a.pad_hi[b] : 0;
        t0 = (PAD && lo == 0 && hi > 0) ? (int)(hi / FA_BC) : 0;
        tail = (nk % FA_BC) != 0;
    }
    __device__ int at(int i) const {
        if constexpr (!PAD) return i;
        const int t = i + t0;
        return i >= nt ? i : (t >= nt ? t - nt : t);
    }
    // does tile tt hold a key past the end or a padded key
    __device__ bool masked(int tt) const {
        if constexpr (!PAD) return tail && tt == nt - 1;
        const int64_t kv0 = (int64_t)tt * FA_BC;
        return (tail && tt == nt - 1) || (kv0 < hi && kv0 + FA_BC > lo);
    }
    __device__ bool dead(int64_t key) const {
        if constexpr (!PAD) return key >= nk;
        return (key >= nk) | ((key >= lo) & (key < hi));
    }
};
constexpr int FA_PAD = 8;    // LDS row padding of K and V^T (elements)
constexpr int FA_WAVES = VX_FA_WAVES;   // waves per workgroup
constexpr int FA_QG = VX_FA_QG;         // 32-row query groups per wave

typedef float f32x8_t __attribute__((ext_vector_type(8)));

template <int D, int WAVES, int QG>
struct FaShape {
    static constexpr int NT = 64 * WAVES;            // threads per workgroup
    static constexpr int BR = 32 * QG * WAVES;       // query rows per workgroup
    static constexpr int KROW = D + FA_PAD;          // K row pitch in LDS
    static constexpr int VROW = FA_BC + FA_PAD;      // V^T row pitch in LDS
    static constexpr int KS = FA_BC * KROW;          // K tile elements
    static constexpr int VS = D * VROW;              // V^T tile elements
    static constexpr int KCH = FA_BC * D / 8 / NT;   // 16-byte K chunks per thread
    static constexpr int DQ = D / 4;                 // V: 4-wide d groups
    static constexpr int KPT = FA_BC * D / 4 / NT;   // V: keys per thread
    static_assert(KCH >= 1 && KPT >= 2 && KPT % 2 == 0 && KPT <= 8, "tile does not divide");
};

// Key order inside each group of 16 keys as the S^T accumulator hands them
// to the P^T operand: lanes 0-31 carry keys {0-3, 8-11}, lanes 32-63 carry
// {4-7, 12-15}.  LDS position p of V^T holds key swap_bits23(p) (an
// involution), so lane half g reads 8 contiguous elements at 8g.
__device__ __forceinline__ int swap_bits23(int p) {
    return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

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

// V^T rows are stored with their 16-byte chunks permuted: chunk c of row r
// sits at chunk c ^ vswz(r).  The transposing stores then write rows 4 apart
// to 16 distinct bank groups, and a fragment read (16 consecutive rows, one
// chunk) still covers every bank group once.
__device__ __forceinline__ int vswz(int row) { return (row >> 4) & 3; }

// Bytes {lo halves} or {hi halves} of two words, as one word: v_perm_b32.
__device__ __forceinline__ uint32_t pick_lo16(uint32_t a0, uint32_t a1) {
    return __builtin_amdgcn_perm(a1, a0, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi16(uint32_t a0, uint32_t a1) {
    return __builtin_amdgcn_perm(a1, a0, 0x07060302u);
}

// Sum of the 8 bf16 values of v, added to acc (v_dot2_f32_bf16 against 1.0).
__device__ __forceinline__ float sum_bf16x8(bf16x8_t v, float acc) {
    const u32x4_t w = __builtin_bit_cast(u32x4_t, v);
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), one, acc, false);
    return acc;
}

// Q fragment of one query row as the B operand of S^T = K Q^T: element
// (ks, e) is column ks * 16 + g * 8 + e.  The row is optionally rotated by
// the 3D RoPE (rounded to bf16, exactly as vx_rope3d_apply stores it), then
// multiplied by scale * log2(e) and rounded to bf16.  The lane holds
// columns g * 8 .. g * 8 + 7 of every 16: with adjacent pairs, or with the
// head split in halves (column c pairs with c + D/2, which is k-step
// ks + D/32, same e), both elements of each pair are in the lane; with
// band halves the partner is read from memory.
template <int D>
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
#pragma unroll
        for (int m = 0; m < 4; ++m)
            u[ks][m] = pack_bf16x2(bf16_lo(u[ks][m]) * a.scale_log2, bf16_hi(u[ks][m]) * a.scale_log2);
        qf[ks] = __builtin_bit_cast(bf16x8_t, uint4{u[ks][0], u[ks][1], u[ks][2], u[ks][3]});
    }
}

template <int D, int WAVES, int QG, bool PAD>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(3 - QG, 3 - QG)))
void fa_fwd_bf16_kernel(FaArgs a) {
    using S = FaShape<D, WAVES, QG>;
    constexpr int NKK = D / 16;      // MFMA k-steps of one S^T block
    constexpr int NDB = D / 32;      // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t lds[3 * S::KS + 2 * S::VS];
    uint16_t* const kbuf[3] = {lds, lds + S::KS, lds + 2 * S::KS};
    uint16_t* const vbuf[2] = {lds + 3 * S::KS, lds + 3 * S::KS + S::VS};

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
    const FaTiles<PAD> tl(a, b);
    const int nt = tl.nt;

    // query group qg of this wave: rows (wave * QG + qg) * 32 + l32 of the tile
    int64_t qi[QG];
    bf16x8_t qf[QG][NKK];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        qi[qg] = (int64_t)qt * S::BR + (wave * QG + qg) * 32 + l32;
        load_q_fragment<D>(a, a.q + off, qi[qg], g, qf[qg]);
    }

    // ---- tile staging: global -> registers -> LDS.  Each thread's byte
    // offsets inside a tile are fixed; the tile start and the sequence end
    // live in a per-tile scalar buffer resource.
    u32x4_t kreg[S::KCH];
    uint2 vreg[S::KPT];
    const int vdq = tid % S::DQ, vkg = tid / S::DQ;
    const int64_t row_bytes = a.row_stride * 2;
    uint32_t koff[S::KCH], voff[S::KPT];
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + S::NT * i;
        koff[i] = (uint32_t)((c / (D / 8)) * row_bytes + (c % (D / 8)) * 16);
    }
#pragma unroll
    for (int s = 0; s < S::KPT; ++s)
        voff[s] = (uint32_t)(swap_bits23(vkg * S::KPT + s) * row_bytes + vdq * 8);

    auto load_k = [&](int t) {
        const int64_t kv0 = (int64_t)t * FA_BC;
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(kb + kv0 * a.row_stride, (nk - kv0) * row_bytes);
#pragma unroll
        for (int i = 0; i < S::KCH; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, koff[i], 0, 0);
    };
    auto load_v = [&](int t) {
        const int64_t kv0 = (int64_t)t * FA_BC;
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(vb + kv0 * a.row_stride, (nk - kv0) * row_bytes);
#pragma unroll
        for (int s = 0; s < S::KPT; ++s) {
            const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, voff[s], 0, 0);
            vreg[s] = uint2{w[0], w[1]};
        }
    };
    auto store_k_chunk = [&](uint16_t* ks, int i) {
        const int c = tid + S::NT * i;
        *(u32x4_t*)(ks + (c / (D / 8)) * S::KROW + (c % (D / 8)) * 8) = kreg[i];
    };
    auto store_k = [&](uint16_t* ks) {
#pragma unroll
        for (int i = 0; i < S::KCH; ++i) store_k_chunk(ks, i);
    };
    // transpose: element j of each of the KPT keys -> one V^T row segment
    auto store_v_row = [&](uint16_t* vt, int j) {
        uint32_t w[S::KPT / 2];
#pragma unroll
        for (int s = 0; s < S::KPT; s += 2) {
            const uint32_t a0 = (j < 2) ? vreg[s].x : vreg[s].y;
            const uint32_t a1 = (j < 2) ? vreg[s + 1].x : vreg[s + 1].y;
            w[s / 2] = (j & 1) ? pick_hi16(a0, a1) : pick_lo16(a0, a1);
        }
        const int row = vdq * 4 + j, pos = vkg * S::KPT;
        uint16_t* dst = vt + row * S::VROW + (((pos >> 3) ^ vswz(row)) << 3) + (pos & 7);
        if constexpr (S::KPT == 8) *(uint4*)dst = uint4{w[0], w[1], w[2], w[3]};
        else if constexpr (S::KPT == 4) *(uint2*)dst = uint2{w[0], w[1]};
        else *(uint32_t*)dst = w[0];
    };
    auto store_v = [&](uint16_t* vt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) store_v_row(vt, j);
    };

    // S^T - m of one query group for both 32-key blocks of the tile at ks
    auto scores = [&](f32x16_t* s, const uint16_t* ks, const bf16x8_t* q, const f32x16_t& negm) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8_t av = *(const bf16x8_t*)(ks + (kb2 * 32 + l32) * S::KROW + kk * 16 + g * 8);
                s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, q[kk], kk == 0 ? negm : s[kb2], 0, 0, 0);
            }
        }
    };
    auto mask_tail = [&](f32x16_t* s, int t) {
        const int64_t kv0 = (int64_t)t * FA_BC;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t key = kv0 + kb2 * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (tl.dead(key)) s[kb2][i] = -__builtin_inff();
            }
    };
    auto row_max = [&](const f32x16_t* s) {
        float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
        return half_max(mx);
    };

    f32x16_t acc[QG][NDB];
    f32x16_t negm[QG];           // -m in every slot: the C operand of the first k-step
    float m_ref[QG], l_run[QG], mx_next[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
        for (int i = 0; i < NDB; ++i) acc[qg][i] = f32x16_t{};
        negm[qg] = f32x16_t{};
        l_run[qg] = 0.f;
        mx_next[qg] = 0.f;
    }
    // ---- prologue: K(0), K(1), K(2) and V(0) into LDS; S(0); m from tile 0
    // (step indices; tl.at maps them to key tiles)
    f32x16_t sA[QG][2], sB[QG][2];
    load_k(tl.at(0));
    load_v(tl.at(0));
    store_k(kbuf[0]);
    store_v(vbuf[0]);
    load_k(tl.at(1));
    store_k(kbuf[1]);
    load_k(tl.at(2));
    store_k(kbuf[2]);
    __syncthreads();
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) scores(sA[qg], kbuf[0], qf[qg], negm[qg]);
    __syncthreads();              // kbuf[0] is refilled in the first iteration
    load_k(tl.at(3));
    load_v(tl.at(1));
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        if (tl.masked(tl.at(0))) mask_tail(sA[qg], tl.at(0));
        const float mx = row_max(sA[qg]);
        m_ref[qg] = mx;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            negm[qg][i] = -mx;
            sA[qg][0][i] -= mx;
            sA[qg][1][i] -= mx;
        }
    }

    // Lane parts of the LDS fragment addresses.  K^T fragment i of a tile:
    // rows (i / NKK) * 32 + l32, columns (i % NKK) * 16 + g * 8.  V^T
    // fragment i: row (i / 4) * 32 + l32, 16-byte chunk 2 (i % 4) + g stored
    // at chunk (2 (i % 4) + g) ^ vswz(row) = (2 (i % 4) ^ (2 (i / 4) & 3)) + (g ^ (l32 >> 4)).
    const int klane = l32 * S::KROW + g * 8;
    const int vlane = l32 * S::VROW + ((g ^ (l32 >> 4)) << 3);
    auto kfrag = [&](const uint16_t* kt, int i) {
        return *(const bf16x8_t*)(kt + klane + (i / NKK) * 32 * S::KROW + (i % NKK) * 16);
    };
    auto vfrag = [&](const uint16_t* vt, int i) {
        const int db = i / 4, kk = i % 4;
        return *(const bf16x8_t*)(vt + vlane + db * 32 * S::VROW + (((2 * kk) ^ ((2 * db) & 3)) << 3));
    };
    // K tiles rotate through three buffers (K(t+1) and K(t+2) are resident
    // while K(t+3) is written), so the first K fragments of the next tile
    // can be read before the barrier; V tiles use two.
    bf16x8_t kf[3];
    kf[0] = kfrag(kbuf[1], 0);
    kf[1] = kfrag(kbuf[1], 1);

    // One key tile.  sc holds S(t) - m (already rescaled), sn receives
    // S(t+1).  The two halves are written out in issue order: every group
    // below pairs one MFMA with the VALU, LDS and global-memory work that
    // is to run under it, and sched_barrier(0) keeps the groups in order.
    auto step = [&](f32x16_t (*sc)[2], f32x16_t (*sn)[2], int t) {
        constexpr int NX = 2 * NKK;          // K fragments of S(t+1), each used by QG MFMAs
        constexpr int WPM = 16 / NX;         // P words (2 weights) per group per fragment
        constexpr int NY = NDB * FA_BC / 16; // V^T fragments of P V, each used by QG MFMAs
        constexpr int MPM = 32 / (NY / 2);   // scores per group per fragment in the row max
        constexpr int SPM = 16 / (NY / 2);   // P words per group per fragment in the row sum
        const int k1 = (t + 1) % 3;
        const uint16_t* kt = lds + k1 * S::KS;                          // K(t+1)
        const uint16_t* kn = lds + (k1 == 2 ? 0 : k1 + 1) * S::KS;      // K(t+2)
        uint16_t* kw = lds + (k1 == 0 ? 2 : k1 - 1) * S::KS;            // K(t+3), where K(t) was
        const uint16_t* vt = lds + 3 * S::KS + (t & 1) * S::VS;         // V(t)
        uint16_t* vw = lds + 3 * S::KS + ((t + 1) & 1) * S::VS;         // V(t+1)
        // ---- X: S(t+1) = K(t+1) Q^T - m  ||  P(t) = 2^(S(t) - m)
        bf16x8_t vf[3];
        uint32_t pw[QG][16];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            if (i + 2 < NX) kf[(i + 2) % 3] = kfrag(kt, i + 2);
            const int kb2 = i / NKK, kk = i % NKK;
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                sn[qg][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    kf[i % 3], qf[qg][kk], kk == 0 ? negm[qg] : sn[qg][kb2], 0, 0, 0);
#pragma unroll
                for (int e = 0; e < WPM; ++e) {
                    const int w = i * WPM + e;   // weights 2w, 2w+1 of the group's 32 scores
                    const float p0 = fast_exp2(sc[qg][(2 * w) >> 4][(2 * w) & 15]);
                    const float p1 = fast_exp2(sc[qg][(2 * w + 1) >> 4][(2 * w + 1) & 15]);
                    pw[qg][w] = pack_bf16x2(p0, p1);
                }
                if (qg == QG - 1 && i + 2 == NX) vf[0] = vfrag(vt, 0);
                if (qg == QG - 1 && i + 1 == NX) vf[1] = vfrag(vt, 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        bf16x8_t pb[QG][FA_BC / 16];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int kk = 0; kk < FA_BC / 16; ++kk)
                pb[qg][kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[qg][4 * kk], pw[qg][4 * kk + 1],
                                                                  pw[qg][4 * kk + 2], pw[qg][4 * kk + 3]});
        // ---- Y: O += V(t)^T P(t)  ||  row sum of P(t); K(t+3), V(t+1) into
        // LDS; loads of K(t+4), V(t+2); row max of S(t+1); first K(t+2) fragments
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        float mx[QG], psum[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            mx[qg] = -__builtin_inff();
            psum[qg] = l_run[qg];
        }
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            if (i + 2 < NY) vf[(i + 2) % 3] = vfrag(vt, i + 2);
            if (i + 2 == NY) kf[0] = kfrag(kn, 0);
            if (i + 1 == NY) kf[1] = kfrag(kn, 1);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                acc[qg][i / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % 3], pb[qg][i % 4],
                                                                         acc[qg][i / 4], 0, 0, 0);
                if (qg == 0) {
                    if (i < S::KCH) store_k_chunk(kw, i);
                    else if (i < S::KCH + 4) store_v_row(vw, i - S::KCH);
                    else if (i == S::KCH + 4) load_k(tl.at(t + 4));
                    else if (i == S::KCH + 5) load_v(tl.at(t + 2));
                }
                if (i < NY / 2) {
#pragma unroll
                    for (int e = 0; e < SPM; ++e) {
                        const int w = i * SPM + e;
                        psum[qg] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2_t, pw[qg][w]), one, psum[qg], false);
                    }
                    __asm__ volatile("" ::"v"(psum[qg]));   // keep the row sum in this group
                } else {
#pragma unroll
                    for (int e = 0; e < MPM; ++e) {
                        const int j = (i - NY / 2) * MPM + e;
                        mx[qg] = fmaxf(mx[qg], sn[qg][j >> 4][j & 15]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        bool need = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            l_run[qg] = psum[qg];
            mx_next[qg] = half_max(mx[qg]);
            need = need || mx_next[qg] > FA_LAZY_LOG2;
        }
        __syncthreads();
        // ---- keys past the end or padded take no weight
        if (t + 1 < nt && tl.masked(tl.at(t + 1))) {
            need = false;
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                mask_tail(sn[qg], tl.at(t + 1));
                mx_next[qg] = row_max(sn[qg]);
                need = need || mx_next[qg] > FA_LAZY_LOG2;
            }
        }
        // ---- lazy rescale for S(t+1) (rare after the first tiles)
        if (t + 1 < nt && __builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                const float delta = fmaxf(mx_next[qg], 0.f);
                const float alpha = fast_exp2(-delta);
                m_ref[qg] += delta;
                l_run[qg] *= alpha;
#pragma unroll
                for (int i = 0; i < NDB; ++i) acc[qg][i] *= alpha;
                // -m is rewritten in place: a plain assignment here makes
                // the register allocator copy the block on every tile.
                const float nm = -m_ref[qg];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __asm__ volatile("v_mov_b32 %0, %1" : "+v"(negm[qg][i]) : "v"(nm));
                    sn[qg][0][i] -= delta;
                    sn[qg][1][i] -= delta;
                }
            }
        }
    };

    for (int t = 0; t < nt; t += 2) {
        step(sA, sB, t);
        if (t + 1 >= nt) break;
        step(sB, sA, t + 1);
    }

    // epilogue: combine the two halves' row sums, normalise, store
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const float l_tot = half_sum(l_run[qg]);
        const float inv = 1.0f / l_tot;
        if (qi[qg] < nq) {
            uint16_t* ob = a.o + off + qi[qg] * a.row_stride;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const f32x16_t& c = acc[qg][db];
                    uint2 w;
                    w.x = pack_bf16x2(c[4 * r + 0] * inv, c[4 * r + 1] * inv);
                    w.y = pack_bf16x2(c[4 * r + 2] * inv, c[4 * r + 3] * inv);
                    *(uint2*)(ob + db * 32 + 8 * r + 4 * g) = w;
                }
            if (a.lse != nullptr && g == 0)
                a.lse[bh * nq + qi[qg]] = (m_ref[qg] + __builtin_log2f(l_tot)) * 0.69314718055994531f;
        }
    }
}

// ---------------------------------------------------------------- bf16 MFMA, DMA staging
//
// Same computation and software pipeline as fa_fwd_bf16_kernel, for
// head_dim 128, 8 waves and 256 query rows per workgroup, but the K and V
// tiles go from global memory straight into LDS (buffer_load_dwordx4 ...
// lds: one wave instruction moves 1 KiB, four 256-byte rows), so no VGPR
// staging, no LDS store instructions and no register transpose.  Both tiles
// are kept row-major in LDS, three buffers each, with the 16-byte chunks of
// row r permuted by c -> c ^ dswz(r) (chosen by which global chunk each lane
// fetches).  K fragments are plain 16-byte reads; V^T fragments for the
// P V product come from ds_read_b64_tr_b16, which transposes 4 keys x 16
// head-dim columns across each 16-lane group: source lane s reads 4
// consecutive columns of key s / 4, and lane i receives column i of the 4
// keys.

// chunk permutation of a 256-byte row: a bijection on 0..15 (16 consecutive
// rows hit 16 distinct chunks), and 4 consecutive rows differ in bits 2-3
// (4 rows x 4 aligned chunks hit 16 distinct chunks)
__device__ __forceinline__ int dswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ bf16x4_t lds_read_tr(const lds_u8* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
}

constexpr int FAD_WAVES = 8;

template <bool PAD>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * FAD_WAVES, 64 * FAD_WAVES),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_dma_kernel(FaArgs a) {
    constexpr int D = 128, NKK = D / 16, NDB = D / 32;
    constexpr int BR = 32 * FAD_WAVES;                // query rows per workgroup
    constexpr int ROWB = 2 * D;                       // bytes per K or V row (256)
    constexpr int TILEB = FA_BC * ROWB;               // bytes per tile (16 KiB)
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
    const FaTiles<PAD> tl(a, b);
    const int nt = tl.nt;

    const int64_t qi = (int64_t)qt * BR + wave * 32 + l32;
    bf16x8_t qf[NKK];
    load_q_fragment<D>(a, a.q + off, qi, g, qf);

    // ---- DMA: instruction m of this wave fills rows 4 I .. 4 I + 3 of the
    // tile, I = wave * NI + m; lane L writes LDS bytes 16 L .. of that KiB,
    // i.e. row 4 I + L / 16, chunk slot L % 16, which holds global chunk
    // (L % 16) ^ dswz(row).
    const int64_t row_bytes = a.row_stride * 2;
    uint32_t goff[NI];
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        const int row = (wave * NI + m) * 4 + (lane >> 4);
        goff[m] = (uint32_t)(row * row_bytes + (((lane & 15) ^ dswz(row)) << 4));
    }
    const int swave = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform, for M0
    // The DMA is written as inline assembly: with the builtin, the compiler
    // cannot tell the destination from the buffers being read and waits for
    // every DMA in flight (vmcnt(0)) before each V read.  Ordering is kept by
    // hand instead: an explicit vmcnt wait and the barrier publish a tile,
    // and no buffer is a DMA target while any wave may still read it.
    auto dma_one = [&](const uint16_t* base, int t, lds_u8* buf, int m) {
        const int64_t kv0 = (int64_t)t * FA_BC;
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base + kv0 * a.row_stride, (nk - kv0) * row_bytes);
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
    for (int kk = 0; kk < NKK; ++kk) koff[kk] = l32 * ROWB + (((2 * kk + g) ^ dswz(l32)) << 4);
    auto kfrag = [&](int jk, int i) {   // K buffer jk (compile-time), fragment i
        return *(const bf16x8_t*)(lds + koff[i % NKK] + (jk * TILEB + (i / NKK) * 32 * ROWB));
    };
    // V^T fragment (db, kk), half r: keys kk*16 + 4 (2r + g) + s / 4 (the
    // S^T accumulator's key order), columns db*32 + 16 hh + 4 (s & 3)..+3,
    // with s = lane & 15, hh = (lane >> 4) & 1
    uint32_t voff[2][NDB];
    {
        const int s_ = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int row = 4 * (2 * r + g) + (s_ >> 2);
                const int chunk = 4 * db + 2 * hh + ((s_ & 3) >> 1);
                voff[r][db] = 3 * TILEB + row * ROWB + ((chunk ^ dswz(row)) << 4) + (s_ & 1) * 8;
            }
    }
    auto vfrag = [&](int jv, int i) {   // V buffer jv (compile-time), fragment i
        const int db = i / 4, kk = i % 4;
        const bf16x4_t lo = lds_read_tr(lds + voff[0][db] + (jv * TILEB + kk * 16 * ROWB));
        const bf16x4_t hi = lds_read_tr(lds + voff[1][db] + (jv * TILEB + kk * 16 * ROWB));
        return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    auto mask_tail = [&](f32x16_t& s0, f32x16_t& s1, int t) {
        const int64_t kv0 = (int64_t)t * FA_BC;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t key = kv0 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (tl.dead(key)) s0[i] = -__builtin_inff();
            if (tl.dead(key + 32)) s1[i] = -__builtin_inff();
        }
    };
    auto row_max = [&](const f32x16_t& s0, const f32x16_t& s1) {
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
        return half_max(mx);
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16_t{};
    f32x16_t negm = f32x16_t{};   // -m in every slot: the C operand of the first k-step
    float m_ref, l_run = 0.f, mx_next = 0.f;

    // ---- prologue: K(0..2), V(0..1) into LDS; S(0); m from tile 0 (step
    // indices; tl.at maps them to key tiles)
    // S tiles rotate through three register blocks: step t reads S(t) from
    // (x, y) and writes S(t+1) to (z, x), since the first half of S(t) is
    // consumed before the second half of S(t+1) is started.
    f32x16_t s0, s1, s2;
    dma(kb, tl.at(0), kbuf(0));
    dma(kb, tl.at(1), kbuf(1));
    dma(kb, tl.at(2), kbuf(2));
    dma(vb, tl.at(0), vbuf(0));
    dma(vb, tl.at(1), vbuf(1));
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's tiles have landed
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(0, kk), qf[kk], kk == 0 ? negm : s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(0, NKK + kk), qf[kk], kk == 0 ? negm : s1, 0, 0, 0);
    }
    __syncthreads();              // K buffer 0 is refilled in the first iteration
    if (tl.masked(tl.at(0))) mask_tail(s0, s1, tl.at(0));
    {
        const float mx = row_max(s0, s1);
        m_ref = mx;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            negm[i] = -mx;
            s0[i] -= mx;
            s1[i] -= mx;
        }
    }
    bf16x8_t kf[3];
    kf[0] = kfrag(1, 0);
    kf[1] = kfrag(1, 1);

    // Step t uses K buffers (t+1) % 3 (read), (t+2) % 3 (next tile's first
    // fragments), t % 3 (DMA target) and V buffers t % 3 (read), (t+2) % 3
    // (DMA target); the loop is unrolled three times so all are compile-time.
    auto step = [&](auto tm, f32x16_t& sc0, f32x16_t& sc1, f32x16_t& sn0, f32x16_t& sn1, int t) {
        constexpr int T3 = decltype(tm)::value;   // t % 3
        constexpr int NX = 2 * NKK;          // K fragments (MFMAs) of S(t+1)
        constexpr int WPM = 16 / NX;         // P words (2 weights) per MFMA
        constexpr int NY = NDB * FA_BC / 16; // V^T fragments (MFMAs) of P V
        constexpr int MPM = 32 / (NY / 2);   // scores per MFMA in the row max
        constexpr int SPM = 16 / (NY / 2);   // P words per MFMA in the row sum
        constexpr int j0 = T3, j1 = (T3 + 1) % 3, j2 = (T3 + 2) % 3;
        // ---- X: S(t+1) = K(t+1) Q^T - m  ||  P(t) = 2^(S(t) - m)
        bf16x8_t vf[3];
        uint32_t pw[16];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            if (i + 2 < NX) kf[(i + 2) % 3] = kfrag(j1, i + 2);
            const int kb2 = i / NKK, kk = i % NKK;
            f32x16_t& d = kb2 ? sn1 : sn0;
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % 3], qf[kk], kk == 0 ? negm : d, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < WPM; ++e) {
                const int w = i * WPM + e;   // weights 2w, 2w+1: block (2w) / 16 of S(t)
                const f32x16_t& src = (2 * w) < 16 ? sc0 : sc1;
                const float p0 = fast_exp2(src[(2 * w) & 15]);
                const float p1 = fast_exp2(src[(2 * w + 1) & 15]);
                pw[w] = pack_bf16x2(p0, p1);
            }
            // K(t+3) where K(t) was, one request every NX / NI groups
            if (i % (NX / NI) == 0) dma_one(kb, tl.at(t + 3), kbuf(j0), i / (NX / NI));
            if (i + 2 == NX) vf[0] = vfrag(j0, 0);
            if (i + 1 == NX) vf[1] = vfrag(j0, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8_t pb[FA_BC / 16];
#pragma unroll
        for (int kk = 0; kk < FA_BC / 16; ++kk)
            pb[kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]});
        // ---- Y: O += V(t)^T P(t)  ||  row sum of P(t); row max of S(t+1);
        // first K(t+2) fragments
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        float mx = -__builtin_inff(), psum = l_run;
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            if (i + 2 < NY) vf[(i + 2) % 3] = vfrag(j0, i + 2);
            acc[i / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % 3], pb[i % 4], acc[i / 4], 0, 0, 0);
            // V(t+2) where V(t-1) was, one request every NY / NI groups
            if (i % (NY / NI) == 0) dma_one(vb, tl.at(t + 2), vbuf(j2), i / (NY / NI));
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
                    mx = fmaxf(mx, (j < 16 ? sn0 : sn1)[j & 15]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run = psum;
        mx_next = half_max(mx);
        // The tiles DMA'd in the previous iteration (K(t+2), V(t+1)) are
        // read after this barrier; this iteration's 2 NI requests may stay
        // in flight.  vmcnt counts only these DMAs in the loop.
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NI));
        __syncthreads();
        kf[0] = kfrag(j2, 0);
        kf[1] = kfrag(j2, 1);
        // ---- keys past the end or padded take no weight
        if (t + 1 < nt && tl.masked(tl.at(t + 1))) {
            mask_tail(sn0, sn1, tl.at(t + 1));
            mx_next = row_max(sn0, sn1);
        }
        // ---- lazy rescale for S(t+1) (rare after the first tiles)
        if (t + 1 < nt && __builtin_amdgcn_ballot_w64(mx_next > FA_LAZY_LOG2) != 0) {
            const float delta = fmaxf(mx_next, 0.f);
            const float alpha = fast_exp2(-delta);
            m_ref += delta;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) acc[i] *= alpha;
            // -m is rewritten in place: a plain assignment here makes the
            // register allocator copy the block on every tile.
            const float nm = -m_ref;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __asm__ volatile("v_mov_b32 %0, %1" : "+v"(negm[i]) : "v"(nm));
                sn0[i] -= delta;
                sn1[i] -= delta;
            }
        }
    };

    for (int t = 0; t < nt; t += 3) {
        step(std::integral_constant<int, 0>{}, s0, s1, s2, s0, t);
        if (t + 1 >= nt) break;
        step(std::integral_constant<int, 1>{}, s2, s0, s1, s2, t + 1);
        if (t + 2 >= nt) break;
        step(std::integral_constant<int, 2>{}, s1, s2, s0, s1, t + 2);
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
            a.lse[bh * nq + qi] = (m_ref + __builtin_log2f(l_tot)) * 0.69314718055994531f;
    }
}

// ---------------------------------------------------------------- f32 VALU

constexpr int FA32_BC = 32;

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_fwd_f32_kernel(FaArgs a) {
    // Every fused multiply-add below is spelled out; implicit contraction is
    // off so each score is rounded once and the same value feeds the running
    // max and the exponent (a lone key then weighs exactly 1).
#pragma clang fp contract(off)
    constexpr int TPQ = D / 32;        // lanes per query, 32 elements each
    constexpr int QPB = 256 / TPQ;     // queries per workgroup
    __shared__ __attribute__((aligned(16))) float ks[FA32_BC * D];
    __shared__ __attribute__((aligned(16))) float vs[FA32_BC * D];

    const int tid = threadIdx.x;
    const int64_t tile = xcd_remap(blockIdx.x, a.total_tiles);
    const int qt = (int)(tile % a.n_qtiles);
    const int64_t bh = tile / a.n_qtiles;
    const int h = (int)(bh % a.heads);
    const int64_t b = bh / a.heads;
    const int64_t off = b * a.batch_stride + (int64_t)h * D;
    const int64_t kv_off = b * a.kv_batch_stride + (int64_t)h * D;
    const float* qb = (const float*)a.q + off;
    const float* kbp = (const float*)a.k + kv_off;
    const float* vbp = (const float*)a.v + kv_off;
    const int64_t nq = a.nq, nk = a.nk;
    const int64_t plo = a.has_pad ? a.pad_lo[b] : 0, phi = a.has_pad ? a.pad_hi[b] : 0;

    const int part = tid % TPQ;
    const int64_t qi = (int64_t)qt * QPB + tid / TPQ;
    float qv[32], acc[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        qv[e] = qi < nq ? qb[qi * a.row_stride + part * 32 + e] : 0.f;
        acc[e] = 0.f;
    }
    int tp = 0, hp = 0, wp = 0;
    const bool rot = a.use_rope && qi < nq && rope_token_pos(a.rope, qi, &tp, &hp, &wp);
    if (rot && a.rope.pairing == 0) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int pair = part * 16 + m;
            float c, s;
            rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &c, &s);
            rope_rotate(qv[2 * m], qv[2 * m + 1], c, s);
        }
    } else if (rot) {
        // half-split pairings: partners are read from the row in memory
        const float* qrow = qb + qi * a.row_stride;
        float out[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            int pair, partner;
            bool second;
            rope_elem_pair(a.rope, part * 32 + e, &pair, &partner, &second);
            float c, s;
            rope_cos_sin(a.rope, rope_pair_pos(a.rope, pair, tp, hp, wp), pair, &c, &s);
            out[e] = rope_rotate_elem(qv[e], qrow[partner], second, c, s);
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) qv[e] = out[e];
    }

    float m_run = -__builtin_inff(), l_run = 0.f;
    for (int64_t kv0 = 0; kv0 < nk; kv0 += FA32_BC) {
        __syncthreads();
        for (int i = tid; i < FA32_BC * D / 4; i += 256) {
            const int key = i / (D / 4), col = i % (D / 4);
            const int64_t kk = kv0 + key;
            float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (kk < nk) {
                kv = *(const float4*)(kbp + kk * a.row_stride + col * 4);
                vv = *(const float4*)(vbp + kk * a.row_stride + col * 4);
            }
            *(float4*)(ks + key * D + col * 4) = kv;
            *(float4*)(vs + key * D + col * 4) = vv;
        }
        __syncthreads();
        const int cnt = (int)((nk - kv0) < FA32_BC ? (nk - kv0) : FA32_BC);
        for (int j = 0; j < cnt; ++j) {
            if (kv0 + j >= plo && kv0 + j < phi) continue;   // padded key
            const float* kr = ks + j * D + part * 32;
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) s = __builtin_fmaf(qv[e], kr[e], s);
#pragma unroll
            for (int x = 1; x < TPQ; x <<= 1) s += __shfl_xor(s, x, 64);
            s *= a.scale;
            const float m_new = fmaxf(m_run, s);
            const float corr = expf(m_run - m_new);
            const float p = expf(s - m_new);
            l_run = __builtin_fmaf(l_run, corr, p);
            const float* vr = vs + j * D + part * 32;
#pragma unroll
            for (int e = 0; e < 32; ++e) acc[e] = __builtin_fmaf(acc[e], corr, p * vr[e]);
            m_run = m_new;
        }
    }
    if (qi < nq) {
        float* ob = (float*)a.o + off + qi * a.row_stride + part * 32;
        const float inv = 1.0f / l_run;
#pragma unroll
        for (int e = 0; e < 32; ++e) ob[e] = acc[e] * inv;
        if (a.lse != nullptr && part == 0) a.lse[bh * nq + qi] = m_run + logf(l_run);
    }
}


// ---------------------------------------------------------------- launch

// Query rows one workgroup covers (the host sizes the grid with it).
int flash_attn_rows_per_workgroup(bool bf16, int64_t head_dim) {
    if (bf16 && head_dim == 128) return 32 * FAD_WAVES;
    return bf16 ? 32 * FA_QG * FA_WAVES : 256 / (int)(head_dim / 32);
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
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.use_rope = rope != nullptr;
    if (rope) a.rope = *rope;
    else a.rope = RopeArgs{};

    const int rows_per_wg = flash_attn_rows_per_workgroup(bf16, head_dim);
    a.n_qtiles = (int)((nq + rows_per_wg - 1) / rows_per_wg);
    a.total_tiles = batch * heads * a.n_qtiles;
    const dim3 grid((unsigned)a.total_tiles);
    if (bf16) {
        const dim3 block(64 * FA_WAVES);
        const dim3 dblock(64 * FAD_WAVES);
        if (head_dim == 128 && a.has_pad)
            hipLaunchKernelGGL(fa_fwd_bf16_dma_kernel<true>, grid, dblock, 0, st, a);
        else if (head_dim == 128)
            hipLaunchKernelGGL(fa_fwd_bf16_dma_kernel<false>, grid, dblock, 0, st, a);
        else if (a.has_pad)
            hipLaunchKernelGGL((fa_fwd_bf16_kernel<64, FA_WAVES, FA_QG, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((fa_fwd_bf16_kernel<64, FA_WAVES, FA_QG, false>), grid, block, 0, st, a);
    } else {
        const dim3 block(256);
        if (head_dim == 128) hipLaunchKernelGGL(fa_fwd_f32_kernel<128>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(fa_fwd_f32_kernel<64>, grid, block, 0, st, a);
    }
    return hipGetLastError();
}


}  // namespace vx
