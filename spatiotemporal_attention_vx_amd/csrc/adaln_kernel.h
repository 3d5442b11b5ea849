// AdaLN modulation kernel for gfx950 (shared by the per-token and the
// per-sample instantiations).
//
// y[n,:] = (x[n,:] - mean_n) / sqrt(var_n + eps) * (1 + scale[m,:]) + shift[m,:]
// with m = n (per-token modulation, Wan2.2: vidax paper, arXiv 2609.18077,
// §2 "Spatiotemporal tensor and sequence sharding", §3.1 and Table 1) or m =
// the sample that token n belongs to (one modulation row per sample,
// broadcast over its tokens, as Wan2.1 does: same paper, §3.1 and Table 1).
// x, the tables and y each are bf16 or f32: the paper keeps Wan2.1's
// residual stream and LTX-2.5's AdaLN tables in fp32, since bf16 there
// degrades the video (§3.2 "Weight import, precision, and verification").
//
// HBM-bound: every byte of x and of per-token tables is read once and y
// written once.  One 64-lane wave owns one row.  A row is cut into groups of
// G consecutive elements, G = 8 if any of x, the tables and y is bf16 (one
// 16-byte chunk in bf16, two in f32), else G = 4 (one f32 chunk); group g
// belongs to lane g % 64, so every load instruction of a wave covers a
// contiguous span.  Each lane issues all its loads up front (the row stays
// in registers; when x and both tables together would take more than ~200
// registers per lane, e.g. f32 tables at width 8192, only x is held and the
// table loads wait for the output pass), then forms exact (count, mean, M2) statistics for each of
// its groups and merges them with Chan's pairwise update (the parallel
// form of Welford's algorithm): first across its groups, then across the
// wave with DPP quad/mirror exchanges and two lane swaps.  When every lane
// holds the same number of groups (the row width is a multiple of 64 G) all
// counts are compile-time constants: no division and no per-group branch.
// Per-token tables are streamed with non-temporal loads; per-sample rows
// are shared by all tokens of a sample and are read through the caches.
#pragma once

#include "vx_device.h"

namespace vx {

// Group size: 8 elements when any tensor is bf16, 4 when all are f32.
template <bool XB, bool MB, bool YB>
constexpr int ada_group() { return (XB || MB || YB) ? 8 : 4; }

// One group of G elements in storage form: 16-byte chunks, G / 8 of them in
// bf16 (G is then 8), G / 4 in f32.
template <bool BF16, int G>
struct Grp {
    static constexpr int C = BF16 ? G / 8 : G / 4;
    u32x4_t c[C];
};

template <bool BF16, int G, bool NT>
__device__ __forceinline__ Grp<BF16, G> load_grp(const u32x4_t* row, int g) {
    Grp<BF16, G> r;
#pragma unroll
    for (int i = 0; i < Grp<BF16, G>::C; ++i) {
        const u32x4_t* p = row + g * Grp<BF16, G>::C + i;
        if constexpr (NT) r.c[i] = __builtin_nontemporal_load(p);
        else r.c[i] = *p;
    }
    return r;
}

template <bool BF16, int G>
__device__ __forceinline__ void unpack_grp(const Grp<BF16, G>& o, float* f) {
#pragma unroll
    for (int i = 0; i < Grp<BF16, G>::C; ++i) unpack_chunk<BF16>(o.c[i], f + i * (BF16 ? 8 : 4));
}

template <bool BF16, int G>
__device__ __forceinline__ void store_grp(u32x4_t* row, int g, const float* f) {
    constexpr int C = Grp<BF16, G>::C;
#pragma unroll
    for (int i = 0; i < C; ++i)
        __builtin_nontemporal_store(pack_chunk<BF16>(f + i * (BF16 ? 8 : 4)), row + g * C + i);
}

// Chan et al. merge of two (count, mean, M2) summaries.
__device__ __forceinline__ void chan_merge(float& n, float& mean, float& m2,
                                           float nb, float meanb, float m2b) {
    const float nt = n + nb;
    if (nt > 0.f) {
        const float delta = meanb - mean;
        const float fb = nb / nt;
        mean = __builtin_fmaf(delta, fb, mean);
        m2 = m2 + m2b + delta * delta * n * fb;
    }
    n = nt;
}

// Exact (mean, M2) of EPC values: pairwise sum, then squared deviations.
template <int EPC>
__device__ __forceinline__ void chunk_stats(const float* f, float& mean, float& m2) {
    float s[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) s[e] = f[e];
#pragma unroll
    for (int w = EPC / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; ++e) s[e] += s[e + w];
    mean = s[0] * (1.0f / EPC);
    float q[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        const float d = f[e] - mean;
        q[e] = d * d;
    }
#pragma unroll
    for (int w = EPC / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; ++e) q[e] += q[e + w];
    m2 = q[0];
}

// Chan's merge of two summaries of equal count n (per side): symmetric in
// its arguments, so both lanes of an exchange compute the same bits.
__device__ __forceinline__ void chan_merge_equal(float& mean, float& m2, float mb, float m2b,
                                                 float n) {
    const float delta = mb - mean;
    mean = (mean + mb) * 0.5f;
    m2 = (m2 + m2b) + delta * delta * (0.5f * n);
}

// x from the lane paired with this one by a DPP control (within 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Lane-swap merges: v_permlane16_swap / v_permlane32_swap of a value with
// itself return {x[l], x[l ^ 16]} (resp. {x[l], x[l ^ 32]}) in some order;
// chan_merge_equal is symmetric, so the order does not matter.
template <int SPAN>
__device__ __forceinline__ void swap_merge(float& mean, float& m2, float n) {
    const uint32_t um = __float_as_uint(mean), uq = __float_as_uint(m2);
    const auto rm = SPAN == 16 ? __builtin_amdgcn_permlane16_swap(um, um, false, false)
                               : __builtin_amdgcn_permlane32_swap(um, um, false, false);
    const auto rq = SPAN == 16 ? __builtin_amdgcn_permlane16_swap(uq, uq, false, false)
                               : __builtin_amdgcn_permlane32_swap(uq, uq, false, false);
    mean = __uint_as_float(rm[0]);
    m2 = __uint_as_float(rq[0]);
    chan_merge_equal(mean, m2, __uint_as_float(rm[1]), __uint_as_float(rq[1]), n);
}

// Wave-wide merge of equal-count summaries (n values each): quad xor 1 and
// 2 (DPP quad_perm), 8-lane and 16-lane mirrors (DPP row_half_mirror,
// row_mirror), then lanes l ^ 16 and l ^ 32.  Every lane ends with the
// summary of all 64, bit-identical across lanes.
__device__ __forceinline__ void wave_merge_equal(float& mean, float& m2, float n) {
    chan_merge_equal(mean, m2, dpp<0xB1>(mean), dpp<0xB1>(m2), n);          // lane ^ 1
    chan_merge_equal(mean, m2, dpp<0x4E>(mean), dpp<0x4E>(m2), 2.f * n);    // lane ^ 2
    chan_merge_equal(mean, m2, dpp<0x141>(mean), dpp<0x141>(m2), 4.f * n);  // 7 - lane (of 8)
    chan_merge_equal(mean, m2, dpp<0x140>(mean), dpp<0x140>(m2), 8.f * n);  // 15 - lane (of 16)
    swap_merge<16>(mean, m2, 16.f * n);
    swap_merge<32>(mean, m2, 32.f * n);
}

// Waves per row: 2 for f32 tables on a row of 8 or more groups per lane
// (an even number, every lane full), else 1.  Such a row held by one wave
// takes 128-256 registers of data per lane, which either costs occupancy or
// makes the compiler sink the table loads into the output pass; split over
// two waves, each holds half the row with every load issued up front, and
// the two half-row summaries are merged through LDS.
template <bool MB, int K, bool FULL>
constexpr int ada_split() { return (!MB && FULL && K >= 8 && K % 2 == 0) ? 2 : 1; }

// XB, MB, YB: x, the tables (shift and scale) and y are bf16 (else f32).
// PER_SAMPLE: the table row of row r is r / n_tokens (else r).  K = groups
// per lane (row width <= 64 G K).  FULL: every lane holds exactly K groups.
// A workgroup of four waves takes 4 / S rows (S = ada_split); with S = 2
// wave w holds groups lane + 64 j, j in [(w & 1) K / 2, (w & 1) K / 2 + K / 2).
template <bool XB, bool MB, bool YB, bool PER_SAMPLE, int K, bool FULL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void adaln_kernel(const u32x4_t* x, const u32x4_t* __restrict__ shift,
                  const u32x4_t* __restrict__ scale, u32x4_t* y, int64_t rows, int64_t n_tokens,
                  int groups, int hidden, float eps) {
    constexpr int G = ada_group<XB, MB, YB>();
    constexpr int XC = Grp<XB, G>::C, MC = Grp<MB, G>::C, YC = Grp<YB, G>::C;   // chunks per group
    constexpr int S = ada_split<MB, K, FULL>();
    constexpr int KW = K / S;                      // groups per lane of this wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * (4 / S) + wave / S;
    const int j0 = (wave % S) * KW;                // this wave's first group index j
    // With two waves per row both take part in the LDS exchange below, so a
    // wave past the last row stays (it loads and stores nothing); a lone wave
    // past the last row leaves.
    const bool live = row < rows;
    if (S == 1 && !live) return;
    const int64_t mrow = PER_SAMPLE ? row / n_tokens : row;
    const u32x4_t* xr = x + row * groups * XC;
    const u32x4_t* shr = shift + mrow * groups * MC;
    const u32x4_t* scr = scale + mrow * groups * MC;
    u32x4_t* yr = y + row * groups * YC;
    auto valid = [&](int j) { return live && (FULL || lane + 64 * (j0 + j) < groups); };

    // Tables are loaded with x unless that would not fit in registers.
    constexpr bool DEFER = KW * 4 * (XC + 2 * MC) > 200;
    Grp<XB, G> xv[KW];
    Grp<MB, G> sh[DEFER ? 1 : KW], sc[DEFER ? 1 : KW];
#pragma unroll
    for (int j = 0; j < KW; ++j) {
        const int g = lane + 64 * (j0 + j);
        if (valid(j)) {
            xv[j] = load_grp<XB, G, true>(xr, g);
            if constexpr (!DEFER) {
                sh[j] = load_grp<MB, G, !PER_SAMPLE>(shr, g);
                sc[j] = load_grp<MB, G, !PER_SAMPLE>(scr, g);
            }
        }
    }

    // Per-lane statistics: exact per group, then Chan's update group by
    // group.  A lane's valid groups are a prefix of j, so after group j the
    // count is G (j + 1): the merge weights are compile-time constants.
    float mean = 0.f, m2 = 0.f, n = 0.f;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
        if (valid(j)) {
            float f[G], mj, qj;
            unpack_grp<XB, G>(xv[j], f);
            chunk_stats<G>(f, mj, qj);
            if (j == 0) {
                mean = mj;
                m2 = qj;
            } else {
                const float wb = 1.0f / (float)(j + 1);               // G / (G (j + 1))
                const float cross = (float)(j * G) * wb;               // n_a n_b / (n_a + n_b)
                const float delta = mj - mean;
                mean = __builtin_fmaf(delta, wb, mean);
                m2 = (m2 + qj) + delta * delta * cross;
            }
            n = (float)((j + 1) * G);
        }
    }

    // Wave merge: every lane ends with the row summary (with two waves per
    // row, that of the wave's half; the halves are then merged through LDS
    // with the symmetric equal-count form, so both waves get the same bits).
    if constexpr (FULL) {
        wave_merge_equal(mean, m2, (float)(KW * G));
        if constexpr (S == 2) {
            __shared__ float half_stats[4][2];
            if (lane == 0) {
                half_stats[wave][0] = mean;
                half_stats[wave][1] = m2;
            }
            __syncthreads();
            chan_merge_equal(mean, m2, half_stats[wave ^ 1][0], half_stats[wave ^ 1][1],
                             (float)(64 * KW * G));
        }
    } else {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float nb = __shfl_xor(n, off, 64);
            const float mb = __shfl_xor(mean, off, 64);
            const float m2b = __shfl_xor(m2, off, 64);
            chan_merge(n, mean, m2, nb, mb, m2b);
        }
    }
    const float var = fmaxf(m2 / (float)hidden, 0.f);
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);

#pragma unroll
    for (int j = 0; j < KW; ++j) {
        if (valid(j)) {
            float fx[G], fs[G], fc[G], out[G];
            unpack_grp<XB, G>(xv[j], fx);
            if constexpr (DEFER) {
                unpack_grp<MB, G>(load_grp<MB, G, !PER_SAMPLE>(shr, lane + 64 * (j0 + j)), fs);
                unpack_grp<MB, G>(load_grp<MB, G, !PER_SAMPLE>(scr, lane + 64 * (j0 + j)), fc);
            } else {
                unpack_grp<MB, G>(sh[j], fs);
                unpack_grp<MB, G>(sc[j], fc);
            }
#pragma unroll
            for (int e = 0; e < G; ++e) {
                const float nrm = (fx[e] - mean) * rstd;
                out[e] = __builtin_fmaf(nrm, 1.0f + fc[e], fs[e]);
            }
            store_grp<YB, G>(yr, lane + 64 * (j0 + j), out);
        }
    }
}

// Groups per lane the launch picks for a row of `groups` groups: the exact
// count when the row fills the wave evenly and that count has a kernel,
// else the next size up of a smaller set (partial lanes).
template <bool XB, bool MB, bool YB, bool PER_SAMPLE, int K, bool FULL>
static void adaln_go(const void* x, const void* shift, const void* scale, void* y, int64_t rows,
                     int64_t n_tokens, int groups, int hidden, float eps, hipStream_t st) {
    constexpr int rows_per_block = 4 / ada_split<MB, K, FULL>();
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((adaln_kernel<XB, MB, YB, PER_SAMPLE, K, FULL>), dim3((unsigned)blocks),
                       dim3(256), 0, st, (const u32x4_t*)x, (const u32x4_t*)shift,
                       (const u32x4_t*)scale, (u32x4_t*)y, rows, n_tokens, groups, hidden, eps);
}

template <bool XB, bool MB, bool YB, bool PER_SAMPLE>
static hipError_t adaln_dispatch_k(const void* x, const void* shift, const void* scale, void* y,
                                   int64_t rows, int64_t n_tokens, int64_t hidden, float eps,
                                   hipStream_t st) {
    // Rows are held in registers: hidden <= 8192, i.e. up to 16 groups of 8
    // per lane, or 32 groups of 4 when all tensors are f32 (then only x is
    // held past 16 groups; the tables are read in the output pass).
    constexpr int G = ada_group<XB, MB, YB>();
    constexpr int KMAX = 8192 / 64 / G;
    const int groups = (int)(hidden / G);
    const int k = (groups + 63) / 64;
    const bool full = groups == 64 * k;
#define VX_ADA(KK, F)                                                                           \
    do {                                                                                        \
        if constexpr (KK <= KMAX)                                                               \
            adaln_go<XB, MB, YB, PER_SAMPLE, KK, F>(x, shift, scale, y, rows, n_tokens, groups, \
                                                    (int)hidden, eps, st);                      \
    } while (0)
    if (full) {
        switch (k) {
            case 1: VX_ADA(1, true); return hipGetLastError();
            case 2: VX_ADA(2, true); return hipGetLastError();
            case 3: VX_ADA(3, true); return hipGetLastError();
            case 4: VX_ADA(4, true); return hipGetLastError();
            case 6: VX_ADA(6, true); return hipGetLastError();
            case 8: VX_ADA(8, true); return hipGetLastError();
            case 10: VX_ADA(10, true); return hipGetLastError();
            case 12: VX_ADA(12, true); return hipGetLastError();
            case 16: VX_ADA(16, true); return hipGetLastError();
            case 20: VX_ADA(20, true); return hipGetLastError();
            case 24: VX_ADA(24, true); return hipGetLastError();
            case 32: VX_ADA(32, true); return hipGetLastError();
            default: break;
        }
    }
    if (k <= 1) VX_ADA(1, false);
    else if (k <= 2) VX_ADA(2, false);
    else if (k <= 4) VX_ADA(4, false);
    else if (k <= 8) VX_ADA(8, false);
    else if (k <= 16) VX_ADA(16, false);
    else VX_ADA(32, false);
#undef VX_ADA
    return hipGetLastError();
}

// Every dtype combination of one modulation mode.
template <bool PER_SAMPLE>
static hipError_t adaln_dispatch(const void* x, const void* shift, const void* scale, void* y,
                                 int64_t rows, int64_t n_tokens, int64_t hidden, float eps,
                                 bool xb, bool mb, bool yb, hipStream_t st) {
    const int code = (xb ? 4 : 0) | (mb ? 2 : 0) | (yb ? 1 : 0);
#define VX_ADA_DT(C, X, M, Y) \
    case C: return adaln_dispatch_k<X, M, Y, PER_SAMPLE>(x, shift, scale, y, rows, n_tokens, hidden, eps, st);
    switch (code) {
        VX_ADA_DT(0, false, false, false)
        VX_ADA_DT(1, false, false, true)
        VX_ADA_DT(2, false, true, false)
        VX_ADA_DT(3, false, true, true)
        VX_ADA_DT(4, true, false, false)
        VX_ADA_DT(5, true, false, true)
        VX_ADA_DT(6, true, true, false)
        VX_ADA_DT(7, true, true, true)
    }
#undef VX_ADA_DT
    return hipErrorInvalidValue;
}

}  // namespace vx
