// Per-token AdaLN modulation for gfx950.
//
// y[n,:] = (x[n,:] - mean_n) / sqrt(var_n + eps) * (1 + scale[n,:]) + shift[n,:]
// (Wan2.2's per-token modulation: vidax paper, arXiv 2609.18077, §2
// "Spatiotemporal tensor and sequence sharding" and §3.1 Table 1.)
//
// HBM-bound: every byte of x, shift and scale is read once and y written
// once.  One 64-lane wave owns one row.  Each lane issues all its 16-byte
// loads of x, shift and scale up front (the row stays in registers), folds
// its share of x into a Welford (count, mean, M2) triple, then the wave
// merges the 64 triples with Chan's pairwise formula over xor shuffles.
// Chunk c of a row (16 bytes) belongs to lane c % 64, so every load
// instruction of a wave covers 1 KiB of contiguous memory.
#include "vx_device.h"

namespace vx {

template <bool BF16> struct AdaTraits;
template <> struct AdaTraits<true> { static constexpr int EPC = 8; };   // bf16 per 16 B
template <> struct AdaTraits<false> { static constexpr int EPC = 4; };  // f32 per 16 B

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4_t& v, float* f) {
    if constexpr (BF16) {
        const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
    } else {
        f[0] = __uint_as_float(v[0]); f[1] = __uint_as_float(v[1]);
        f[2] = __uint_as_float(v[2]); f[3] = __uint_as_float(v[3]);
    }
}

template <bool BF16>
__device__ __forceinline__ u32x4_t pack(const float* f) {
    u32x4_t r;
    if constexpr (BF16) {
        r[0] = pack_bf16x2(f[0], f[1]); r[1] = pack_bf16x2(f[2], f[3]);
        r[2] = pack_bf16x2(f[4], f[5]); r[3] = pack_bf16x2(f[6], f[7]);
    } else {
        r[0] = __float_as_uint(f[0]); r[1] = __float_as_uint(f[1]);
        r[2] = __float_as_uint(f[2]); r[3] = __float_as_uint(f[3]);
    }
    return r;
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

// K = 16-byte chunks per lane (row width <= 64 * K * EPC).
template <bool BF16, int K>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void adaln_kernel(const u32x4_t* x, const u32x4_t* __restrict__ shift,
                  const u32x4_t* __restrict__ scale, u32x4_t* y, int64_t rows, int chunks,
                  int hidden, float eps) {
    constexpr int EPC = AdaTraits<BF16>::EPC;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t base = row * chunks;

    u32x4_t xv[K], sh[K], sc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int c = lane + 64 * j;
        if (c < chunks) {
            xv[j] = __builtin_nontemporal_load(x + base + c);
            sh[j] = __builtin_nontemporal_load(shift + base + c);
            sc[j] = __builtin_nontemporal_load(scale + base + c);
        }
    }

    // Per-lane Welford.  A lane's valid chunks are a prefix of j, so the
    // running count at element e of chunk j is the constant j*EPC + e + 1.
    float n = 0.f, mean = 0.f, m2 = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (lane + 64 * j < chunks) {
            float f[EPC];
            unpack<BF16>(xv[j], f);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float inv = 1.0f / (float)(j * EPC + e + 1);
                const float d = f[e] - mean;
                mean = __builtin_fmaf(d, inv, mean);
                m2 = __builtin_fmaf(d, f[e] - mean, m2);
            }
            n = (float)((j + 1) * EPC);
        }
    }

    // Wave merge: after the xor butterfly every lane holds the row summary.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float nb = __shfl_xor(n, off, 64);
        const float mb = __shfl_xor(mean, off, 64);
        const float m2b = __shfl_xor(m2, off, 64);
        chan_merge(n, mean, m2, nb, mb, m2b);
    }
    const float var = fmaxf(m2 / (float)hidden, 0.f);
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);

#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int c = lane + 64 * j;
        if (c < chunks) {
            float fx[EPC], fs[EPC], fc[EPC], out[EPC];
            unpack<BF16>(xv[j], fx);
            unpack<BF16>(sh[j], fs);
            unpack<BF16>(sc[j], fc);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float nrm = (fx[e] - mean) * rstd;
                out[e] = __builtin_fmaf(nrm, 1.0f + fc[e], fs[e]);
            }
            __builtin_nontemporal_store(pack<BF16>(out), y + base + c);
        }
    }
}

template <bool BF16, int K>
static hipError_t launch_adaln_k(const void* x, const void* shift, const void* scale, void* y,
                                 int64_t rows, int64_t hidden, float eps, hipStream_t st) {
    constexpr int EPC = AdaTraits<BF16>::EPC;
    const int chunks = (int)(hidden / EPC);
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL((adaln_kernel<BF16, K>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const u32x4_t*)x, (const u32x4_t*)shift, (const u32x4_t*)scale, (u32x4_t*)y,
                       rows, chunks, (int)hidden, eps);
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
