// Device-side helpers shared by the gfx950 kernels of the hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vx {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Widen the low / high bf16 of a 32-bit word (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats to two bf16 in one word, round to nearest even (gfx950
// v_cvt_pk_bf16_f32 under the default rounding mode).  a -> low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t f = {a, b};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// A 16-byte chunk as floats: 8 bf16 (exact widening) or 4 f32.
template <bool BF16>
__device__ __forceinline__ void unpack_chunk(const u32x4_t& v, float* f) {
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
}

// Floats back to one 16-byte chunk (bf16: round to nearest even).
template <bool BF16>
__device__ __forceinline__ u32x4_t pack_chunk(const float* f) {
    u32x4_t r;
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    }
    return r;
}

// RoPE geometry of one call, in kernel-argument form.
struct RopeArgs {
    int32_t T, H, W;
    int32_t n_prefix;
    int32_t d_t, d_h, d_w;
    float theta;
    int32_t pairing;   // 0 adjacent pairs, 1 halves of the head, 2 halves of each band
};

// Position along the band that pair `pair` of the head dimension belongs
// to, and that pair's index and width inside its band.  Returns false for
// text-prefix tokens (no rotation).
__device__ __forceinline__ bool rope_pair_geometry(const RopeArgs& r, int64_t token, int pair,
                                                    int* pos, int* j, int* width) {
    if (token < r.n_prefix) return false;
    const int64_t v = token - r.n_prefix;
    const int64_t hw = (int64_t)r.H * r.W;
    const int t = (int)(v / hw);
    const int h = (int)((v / r.W) % r.H);
    const int w = (int)(v % r.W);
    const int pt = r.d_t >> 1, ph = r.d_h >> 1;
    if (pair < pt) { *pos = t; *j = pair; *width = r.d_t; }
    else if (pair < pt + ph) { *pos = h; *j = pair - pt; *width = r.d_h; }
    else { *pos = w; *j = pair - pt - ph; *width = r.d_w; }
    return true;
}

// Pair of element e of the head dimension under the call's pairing: the
// pair's index in angle order ([t | h | w] bands, as rope_pair_geometry
// numbers them), the other element of the pair, and whether e is the
// pair's second element (the imaginary part of a + i b).
__device__ __forceinline__ void rope_elem_pair(const RopeArgs& r, int e, int* pair, int* partner,
                                               bool* second) {
    if (r.pairing == 0) {            // (2j, 2j + 1)
        *pair = e >> 1;
        *second = (e & 1) != 0;
        *partner = e ^ 1;
    } else if (r.pairing == 1) {     // (k, k + d/2), k-th angle of the whole list
        const int half = (r.d_t + r.d_h + r.d_w) >> 1;
        *second = e >= half;
        *pair = *second ? e - half : e;
        *partner = *second ? e - half : e + half;
    } else {                         // (s_a + j, s_a + j + d_a/2) inside band a
        int start, width, first_pair;
        if (e < r.d_t) { start = 0; width = r.d_t; first_pair = 0; }
        else if (e < r.d_t + r.d_h) { start = r.d_t; width = r.d_h; first_pair = r.d_t >> 1; }
        else { start = r.d_t + r.d_h; width = r.d_w; first_pair = (r.d_t + r.d_h) >> 1; }
        const int l = e - start, hw = width >> 1;
        *second = l >= hw;
        *pair = first_pair + (*second ? l - hw : l);
        *partner = *second ? e - hw : e + hw;
    }
}

// Element e of a rotated pair from its own value xe and its partner's xp,
// the same expressions as rope_rotate.
__device__ __forceinline__ float rope_rotate_elem(float xe, float xp, bool second, float c, float s) {
    return second ? __builtin_fmaf(xp, s, xe * c) : __builtin_fmaf(xe, c, -xp * s);
}

// cos and sin of the RoPE angle pos * theta^(-2j/width), evaluated in double
// precision and rounded to float once.  Called once per (token, pair), never
// per head, so its cost is spread over all heads and over Q and K.
__device__ __forceinline__ void rope_cos_sin(const RopeArgs& r, int pos, int j, int width,
                                             float* c, float* s) {
    const double freq = exp2(-(2.0 * j / (double)width) * log2((double)r.theta));
    double sd, cd;
    sincos((double)pos * freq, &sd, &cd);
    *c = (float)cd;
    *s = (float)sd;
}

// Rotate the pair (x0, x1) by (c, s).
__device__ __forceinline__ void rope_rotate(float& x0, float& x1, float c, float s) {
    const float a = x0, b = x1;
    x0 = __builtin_fmaf(a, c, -b * s);
    x1 = __builtin_fmaf(a, s, b * c);
}

// Workgroup-to-tile remap for a chip whose workgroups are dealt round-robin
// to 8 XCDs (each with its own L2): XCD x receives a contiguous range of
// logical tiles, so neighbouring tiles (same head, same K/V) share one L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t G) {
    const int64_t xcd = b & 7, local = b >> 3;
    const int64_t per = G >> 3, rem = G & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace vx
