// Per-token AdaLN modulation for gfx950.
//
// y[n,:] = (x[n,:] - mean_n) / sqrt(var_n + eps) * (1 + scale[n,:]) + shift[n,:]
// (Wan2.2's per-token modulation: vidax paper, arXiv 2609.18077, §2
// "Spatiotemporal tensor and sequence sharding" and §3.1 Table 1.)
//
// HBM-bound: every byte of x, shift and scale is read once and y written
// once.  One 64-lane wave owns one row.  Each lane issues all its 16-byte
// loads of x, shift and scale up front (the row stays in registers), then
// forms exact (count, mean, M2) statistics for each of its 16-byte chunks
// and merges them with Chan's pairwise update (the parallel form of
// Welford's algorithm): first across its chunks, then across the wave with
// DPP quad/mirror exchanges and two lane swaps.  When every lane holds the
// same number of chunks (the row width is a multiple of 64 chunks) all
// counts are compile-time constants: no division and no per-chunk branch.
// Chunk c of a row (16 bytes) belongs to lane c % 64, so every load
// instruction of a wave covers 1 KiB of contiguous memory.
#include "vx_device.h"

namespace vx {

template <bool BF16> struct AdaTraits;
template <> struct AdaTraits<true> { static constexpr int EPC = 8; };   // bf16 per 16 B
template <> struct AdaTraits<false> { static constexpr int EPC = 4; };  // f32 per 16 B

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

// K = 16-byte chunks per lane (row width <= 64 * K * EPC).  FULL: every lane
// holds exactly K chunks (row width == 64 * K * EPC).
template <bool BF16, int K, bool FULL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void adaln_kernel(const u32x4_t* x, const u32x4_t* __restrict__ shift,
                  const u32x4_t* __restrict__ scale, u32x4_t* y, int64_t rows, int chunks,
                  int hidden, float eps) {
    constexpr int EPC = AdaTraits<BF16>::EPC;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t base = row * chunks;
    auto valid = [&](int j) { return FULL || lane + 64 * j < chunks; };

    u32x4_t xv[K], sh[K], sc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int c = lane + 64 * j;
        if (valid(j)) {
            xv[j] = __builtin_nontemporal_load(x + base + c);
            sh[j] = __builtin_nontemporal_load(shift + base + c);
            sc[j] = __builtin_nontemporal_load(scale + base + c);
        }
    }

    // Per-lane statistics: exact per chunk, then Chan's update chunk by
    // chunk.  A lane's valid chunks are a prefix of j, so after chunk j the
    // count is (j + 1) * EPC: the merge weights are compile-time constants.
    float mean = 0.f, m2 = 0.f, n = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (valid(j)) {
            float f[EPC], mj, qj;
            unpack_chunk<BF16>(xv[j], f);
            chunk_stats<EPC>(f, mj, qj);
            if (j == 0) {
                mean = mj;
                m2 = qj;
            } else {
                const float wb = 1.0f / (float)(j + 1);               // EPC / ((j + 1) EPC)
                const float cross = (float)(j * EPC) * wb;             // n_a n_b / (n_a + n_b)
                const float delta = mj - mean;
                mean = __builtin_fmaf(delta, wb, mean);
                m2 = (m2 + qj) + delta * delta * cross;
            }
            n = (float)((j + 1) * EPC);
        }
    }

    // Wave merge: every lane ends with the row summary.
    if constexpr (FULL) {
        wave_merge_equal(mean, m2, (float)(K * EPC));
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
    for (int j = 0; j < K; ++j) {
        const int c = lane + 64 * j;
        if (valid(j)) {
            float fx[EPC], fs[EPC], fc[EPC], out[EPC];
            unpack_chunk<BF16>(xv[j], fx);
            unpack_chunk<BF16>(sh[j], fs);
            unpack_chunk<BF16>(sc[j], fc);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float nrm = (fx[e] - mean) * rstd;
                out[e] = __builtin_fmaf(nrm, 1.0f + fc[e], fs[e]);
            }
            __builtin_nontemporal_store(pack_chunk<BF16>(out), y + base + c);
        }
    }
}

template <bool BF16, int K>
static hipError_t launch_adaln_k(const void* x, const void* shift, const void* scale, void* y,
                                 int64_t rows, int64_t hidden, float eps, hipStream_t st) {
    constexpr int EPC = AdaTraits<BF16>::EPC;
    const int chunks = (int)(hidden / EPC);
    const int64_t blocks = (rows + 3) / 4;
    if (chunks == 64 * K)
        hipLaunchKernelGGL((adaln_kernel<BF16, K, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                           (const u32x4_t*)x, (const u32x4_t*)shift, (const u32x4_t*)scale,
                           (u32x4_t*)y, rows, chunks, (int)hidden, eps);
    else
        hipLaunchKernelGGL((adaln_kernel<BF16, K, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                           (const u32x4_t*)x, (const u32x4_t*)shift, (const u32x4_t*)scale,
                           (u32x4_t*)y, rows, chunks, (int)hidden, eps);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_adaln_t(const void* x, const void* shift, const void* scale, void* y,
                                 int64_t rows, int64_t hidden, float eps, hipStream_t st) {
    constexpr int EPC = AdaTraits<BF16>::EPC;
    const int64_t chunks = hidden / EPC;
    const int64_t k = (chunks + 63) / 64;  // chunks per lane
#define VX_ADA_CASE(KK) \
    if (k <= KK) return launch_adaln_k<BF16, KK>(x, shift, scale, y, rows, hidden, eps, st);
    VX_ADA_CASE(1) VX_ADA_CASE(2) VX_ADA_CASE(3) VX_ADA_CASE(4) VX_ADA_CASE(6)
    VX_ADA_CASE(8) VX_ADA_CASE(10) VX_ADA_CASE(12) VX_ADA_CASE(16)
#undef VX_ADA_CASE
    return hipErrorInvalidValue;  // excluded by host-side validation
}

hipError_t launch_adaln(const void* x, const void* shift, const void* scale, void* y,
                        int64_t rows, int64_t hidden, float eps, bool bf16, hipStream_t st) {
    return bf16 ? launch_adaln_t<true>(x, shift, scale, y, rows, hidden, eps, st)
                : launch_adaln_t<false>(x, shift, scale, y, rows, hidden, eps, st);
}

}  // namespace vx
