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
// bf16 path (the hot one), per workgroup of 4 waves and 128 query rows:
//   * Each wave owns 32 query rows.  Scores are formed transposed,
//     S^T (32 keys x 32 queries) = K_tile . Q^T, with
//     v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand, the
//     wave's Q^T fragment stays in VGPRs as the B operand.  In the
//     accumulator, lane l holds query l % 32 and 16 of the 32 keys, so the
//     softmax row statistics are per lane, plus one exchange with lane l^32.
//   * P^T is rounded to bf16 in registers and is directly the B operand of
//     O^T (d x 32 queries) += V^T . P^T.  The k index of that product runs
//     over keys in the order the S^T accumulator hands them out; V^T is
//     stored in LDS with the same key order, so no shuffle is needed.
//   * K (row-major) and V^T (transposed while it is written to LDS) are
//     double-buffered: tile t+1 is fetched into registers while tile t is
//     computed, and written to the other LDS buffer before the barrier.
//   * Key tiles past the sequence end are zero-filled and their scores set
//     to -inf; query rows past the end are computed on zeros and not stored.
//   * Workgroups are remapped so each XCD works through a contiguous range
//     of (batch, head, query tile), keeping that head's K/V hot in its L2.
//
// f32 path (small problems and parity): a plain VALU kernel, a few lanes per
// query, K/V tiles staged through LDS, exact expf online softmax.
#include "vx_device.h"

namespace vx {

struct FaArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int64_t n;             // tokens
    int64_t row_stride;    // elements between consecutive tokens (heads * D)
    int64_t batch_stride;  // elements between batch entries (n * heads * D)
    int heads;
    int n_qtiles;
    int64_t total_tiles;
    float scale;           // softmax scale (natural units)
    float scale_log2;      // scale * log2(e)
    int use_rope;
    RopeArgs rope;
};

// ---------------------------------------------------------------- bf16 MFMA

constexpr int FA_BR = 128;   // query rows per workgroup
constexpr int FA_BC = 64;    // keys per tile
constexpr int FA_PADK = 8;   // LDS row padding of K (elements)
constexpr int FA_PADV = 8;   // LDS row padding of V^T (elements)

template <int D>
struct FaShape {
    static constexpr int KROW = D + FA_PADK;            // K row pitch in LDS
    static constexpr int VROW = FA_BC + FA_PADV;        // V^T row pitch in LDS
    static constexpr int KS = FA_BC * KROW;             // K tile elements
    static constexpr int VS = D * VROW;                 // V^T tile elements
    static constexpr int STAGE = KS + VS;
    static constexpr int KCH = FA_BC * D / 8 / 256;     // 16-byte K chunks per thread
    static constexpr int DQ = D / 4;                    // V: 4-wide d groups
    static constexpr int KPT = FA_BC * D / 4 / 256;     // V: keys per thread
};

typedef float f32x8_t __attribute__((ext_vector_type(8)));

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

// A lazily rescaled running maximum may trail the true one by up to this
// many powers of two before the accumulator is rescaled (weights <= 2^8).
constexpr float FA_LAZY_LOG2 = 8.0f;

template <int D>
__device__ __forceinline__ void load_q_fragment(const FaArgs& a, const uint16_t* qb, int64_t qi,
                                                int g, bf16x8_t* qf) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 w = {0u, 0u, 0u, 0u};
        if (qi < a.n) w = *(const uint4*)(qb + qi * a.row_stride + ks * 16 + g * 8);
        if (a.use_rope && qi < a.n) {
            uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int pair = (ks * 16 + g * 8) / 2 + m;
                int pos, j, width;
                if (rope_pair_geometry(a.rope, qi, pair, &pos, &j, &width)) {
                    float c, s;
                    rope_cos_sin(a.rope, pos, j, width, &c, &s);
                    float x0 = bf16_lo(u[m]), x1 = bf16_hi(u[m]);
                    rope_rotate(x0, x1, c, s);
                    u[m] = pack_bf16x2(x0, x1);
                }
            }
            w = uint4{u[0], u[1], u[2], u[3]};
        }
        qf[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(FaArgs a) {
    using S = FaShape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * S::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;

    const int64_t tile = xcd_remap(blockIdx.x, a.total_tiles);
    const int qt = (int)(tile % a.n_qtiles);
    const int64_t bh = tile / a.n_qtiles;
    const int h = (int)(bh % a.heads);
    const int64_t b = bh / a.heads;
    const int64_t off = b * a.batch_stride + (int64_t)h * D;
    const uint16_t* qb = a.q + off;
    const uint16_t* kb = a.k + off;
    const uint16_t* vb = a.v + off;
    const int64_t n = a.n;

    const int64_t qi = (int64_t)qt * FA_BR + wave * 32 + l32;
    bf16x8_t qf[D / 16];
    load_q_fragment<D>(a, qb, qi, g, qf);

    // ---- tile staging: global -> registers -> LDS
    // Each thread's byte offsets inside a tile are fixed; the tile start
    // and the sequence end live in a per-tile scalar buffer resource, so
    // keys past the end read as zero without any per-lane bounds test.
    u32x4_t kreg[S::KCH];
    uint2 vreg[S::KPT];
    const int vdq = tid % S::DQ, vkg = tid / S::DQ;
    const int64_t row_bytes = a.row_stride * 2;
    uint32_t koff[S::KCH], voff[S::KPT];
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + 256 * i;
        koff[i] = (uint32_t)((c / (D / 8)) * row_bytes + (c % (D / 8)) * 16);
    }
#pragma unroll
    for (int s = 0; s < S::KPT; ++s)
        voff[s] = (uint32_t)(swap_bits23(vkg * S::KPT + s) * row_bytes + vdq * 8);

    auto load_tile = [&](int64_t kv0) {
        const int64_t left = (n - kv0) * row_bytes;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kb + kv0 * a.row_stride, left);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vb + kv0 * a.row_stride, left);
#pragma unroll
        for (int i = 0; i < S::KCH; ++i)
            kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, 0);
#pragma unroll
        for (int s = 0; s < S::KPT; ++s) {
            const auto w = __builtin_amdgcn_raw_buffer_load_b64(rv, voff[s], 0, 0);
            vreg[s] = uint2{w[0], w[1]};
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* ks = lds + buf * S::STAGE;
        uint16_t* vt = ks + S::KS;
#pragma unroll
        for (int i = 0; i < S::KCH; ++i) {
            const int c = tid + 256 * i;
            const int key = c / (D / 8), col = c % (D / 8);
            *(u32x4_t*)(ks + key * S::KROW + col * 8) = kreg[i];
        }
        // transpose: element j of each of the KPT keys -> one V^T row segment
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w[S::KPT / 2];
#pragma unroll
            for (int s = 0; s < S::KPT; s += 2) {
                const uint32_t a0 = (j < 2) ? vreg[s].x : vreg[s].y;
                const uint32_t a1 = (j < 2) ? vreg[s + 1].x : vreg[s + 1].y;
                w[s / 2] = (j & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u))
                                   : ((a0 & 0xffffu) | (a1 << 16));
            }
            uint16_t* dst = vt + (vdq * 4 + j) * S::VROW + vkg * S::KPT;
            if constexpr (S::KPT == 8) *(uint4*)dst = uint4{w[0], w[1], w[2], w[3]};
            else *(uint2*)dst = uint2{w[0], w[1]};
        }
    };

    f32x16_t acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16_t{};
    float m_run = -__builtin_inff();   // running row max, raw score units
    float l_run = 0.f;                 // this lane's share of the row sum

    const int nt = (int)((n + FA_BC - 1) / FA_BC);
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        const uint16_t* ks = lds + buf * S::STAGE;
        const uint16_t* vt = ks + S::KS;
        if (t + 1 < nt) load_tile((int64_t)(t + 1) * FA_BC);

        // S^T = K . Q^T for two blocks of 32 keys
        f32x16_t st[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            st[kb2] = f32x16_t{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const bf16x8_t av = *(const bf16x8_t*)(ks + (kb2 * 32 + l32) * S::KROW + kk * 16 + g * 8);
                st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[kk], st[kb2], 0, 0, 0);
            }
        }

        // keys past the end of the sequence take no weight
        const int64_t kv0 = (int64_t)t * FA_BC;
        if (kv0 + FA_BC > n) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int64_t key = kv0 + kb2 * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key >= n) st[kb2][i] = -__builtin_inff();
                }
        }

        float mx = st[0][0];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb2][i]);
        mx = half_max(mx);
        // Rescale only when some row's maximum outgrew the reference by more
        // than 2^FA_LAZY_LOG2 (always on the first tile, where m_run = -inf).
        if (__builtin_amdgcn_ballot_w64((mx - m_run) * a.scale_log2 > FA_LAZY_LOG2) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2((m_run - m_new) * a.scale_log2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        }
        const float mb = m_run * a.scale_log2;

        float psum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(__builtin_fmaf(st[kb2][i], a.scale_log2, -mb));
                st[kb2][i] = p;
                psum += p;
            }
        l_run += psum;

        // P^T operand: 16 keys per MFMA, taken from accumulator slots 0-7 / 8-15
        bf16x8_t pb[FA_BC / 16];
#pragma unroll
        for (int kk = 0; kk < FA_BC / 16; ++kk) {
            const f32x16_t& src = st[kk >> 1];
            const int o8 = (kk & 1) * 8;
            f32x8_t f = {src[o8 + 0], src[o8 + 1], src[o8 + 2], src[o8 + 3],
                         src[o8 + 4], src[o8 + 5], src[o8 + 6], src[o8 + 7]};
            pb[kk] = __builtin_convertvector(f, bf16x8_t);
        }

        // O^T += V^T . P^T
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int kk = 0; kk < FA_BC / 16; ++kk) {
                const bf16x8_t av = *(const bf16x8_t*)(vt + (db * 32 + l32) * S::VROW + kk * 16 + g * 8);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kk], acc[db], 0, 0, 0);
            }

        if (t + 1 < nt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue: combine the two halves' row sums, normalise, store
    const float l_tot = half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (qi < n) {
        uint16_t* ob = a.o + off + qi * a.row_stride;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x16_t& c = acc[db];
                uint2 w;
                w.x = pack_bf16x2(c[4 * r + 0] * inv, c[4 * r + 1] * inv);
                w.y = pack_bf16x2(c[4 * r + 2] * inv, c[4 * r + 3] * inv);
                *(uint2*)(ob + db * 32 + 8 * r + 4 * g) = w;
            }
        if (a.lse != nullptr && g == 0)
            a.lse[bh * n + qi] = m_run * a.scale + logf(l_tot);
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
    const float* qb = (const float*)a.q + off;
    const float* kbp = (const float*)a.k + off;
    const float* vbp = (const float*)a.v + off;
    const int64_t n = a.n;

    const int part = tid % TPQ;
    const int64_t qi = (int64_t)qt * QPB + tid / TPQ;
    float qv[32], acc[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        qv[e] = qi < n ? qb[qi * a.row_stride + part * 32 + e] : 0.f;
        acc[e] = 0.f;
    }
    if (a.use_rope && qi < n) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            int pos, j, width;
            if (rope_pair_geometry(a.rope, qi, part * 16 + m, &pos, &j, &width)) {
                float c, s;
                rope_cos_sin(a.rope, pos, j, width, &c, &s);
                rope_rotate(qv[2 * m], qv[2 * m + 1], c, s);
            }
        }
    }

    float m_run = -__builtin_inff(), l_run = 0.f;
    for (int64_t kv0 = 0; kv0 < n; kv0 += FA32_BC) {
        __syncthreads();
        for (int i = tid; i < FA32_BC * D / 4; i += 256) {
            const int key = i / (D / 4), col = i % (D / 4);
            const int64_t kk = kv0 + key;
            float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (kk < n) {
                kv = *(const float4*)(kbp + kk * a.row_stride + col * 4);
                vv = *(const float4*)(vbp + kk * a.row_stride + col * 4);
            }
            *(float4*)(ks + key * D + col * 4) = kv;
            *(float4*)(vs + key * D + col * 4) = vv;
        }
        __syncthreads();
        const int cnt = (int)((n - kv0) < FA32_BC ? (n - kv0) : FA32_BC);
        for (int j = 0; j < cnt; ++j) {
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
    if (qi < n) {
        float* ob = (float*)a.o + off + qi * a.row_stride + part * 32;
        const float inv = 1.0f / l_run;
#pragma unroll
        for (int e = 0; e < 32; ++e) ob[e] = acc[e] * inv;
        if (a.lse != nullptr && part == 0) a.lse[bh * n + qi] = m_run + logf(l_run);
    }
}

// ---------------------------------------------------------------- launch

hipError_t launch_flash_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t batch, int64_t n, int64_t heads, int64_t head_dim,
                             float scale, const RopeArgs* rope, bool bf16, hipStream_t st) {
    FaArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
    a.lse = lse;
    a.n = n;
    a.row_stride = heads * head_dim;
    a.batch_stride = n * heads * head_dim;
    a.heads = (int)heads;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.use_rope = rope != nullptr;
    if (rope) a.rope = *rope;
    else a.rope = RopeArgs{1, 1, 1, 0, 0, 0, 0, 1.f};

    const int rows_per_wg = bf16 ? FA_BR : 256 / (int)(head_dim / 32);
    a.n_qtiles = (int)((n + rows_per_wg - 1) / rows_per_wg);
    a.total_tiles = batch * heads * a.n_qtiles;
    const dim3 grid((unsigned)a.total_tiles), block(256);
    if (bf16) {
        if (head_dim == 128) hipLaunchKernelGGL(fa_fwd_bf16_kernel<128>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(fa_fwd_bf16_kernel<64>, grid, block, 0, st, a);
    } else {
        if (head_dim == 128) hipLaunchKernelGGL(fa_fwd_f32_kernel<128>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(fa_fwd_f32_kernel<64>, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace vx
