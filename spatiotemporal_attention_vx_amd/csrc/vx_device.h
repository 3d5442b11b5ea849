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
constexpr int ROPE_MAX_PAIRS = 128;   // head_dim <= 256
struct RopeArgs {
    int32_t T, H, W;
    int32_t n_prefix;
    int32_t d_t, d_h, d_w;
    int32_t pairing;   // 0 adjacent pairs, 1 halves of the head, 2 halves of each band
    // theta^(-2j / d_a) of every pair in angle order ([t | h | w] bands),
    // evaluated once per call on the host in double precision
    double freq[ROPE_MAX_PAIRS];
};

// Grid position (t, h, w) of a token; false for text-prefix tokens (no
// rotation).  Evaluated once per token row, never per pair.
__device__ __forceinline__ bool rope_token_pos(const RopeArgs& r, int64_t token, int* t, int* h,
                                               int* w) {
    if (token < r.n_prefix) return false;
    const int64_t v = token - r.n_prefix;
    const int64_t hw = (int64_t)r.H * r.W;
    *t = (int)(v / hw);
    const int rem = (int)(v - (int64_t)(*t) * hw);    // < H * W
    *h = rem / r.W;
    *w = rem - *h * r.W;
    return true;
}

// Position along the band that pair `pair` (angle order) belongs to.
__device__ __forceinline__ int rope_pair_pos(const RopeArgs& r, int pair, int t, int h, int w) {
    const int pt = r.d_t >> 1, ph = r.d_h >> 1;
    return pair < pt ? t : (pair < pt + ph ? h : w);
}

// Pair of element e of the head dimension under the call's pairing: the
// pair's index in angle order ([t | h | w] bands, as rope_pair_pos
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

// cos and sin of pair `pair`'s RoPE angle at grid position pos.  The angle
// pos * freq is formed in double precision and reduced by multiples of
// pi/2 there (exact to ~1e-15 rad for any grid index); sin and cos of the
// remainder r (|r| <= pi/4) come from their Taylor series in float, to r^9
// and r^10 (truncation below 2e-9), and the quadrant picks signs and order.
// Branch-free; absolute error a few 1e-7.
__device__ __forceinline__ void rope_cos_sin(const RopeArgs& r, int pos, int pair, float* c,
                                             float* s) {
    const double ang = (double)pos * r.freq[pair];
    const double qd = __builtin_rint(ang * 0.63661977236758134308);        // 2 / pi
    double red = __builtin_fma(-qd, 1.57079632679489655800, ang);          // pi/2, high part
    red = __builtin_fma(-qd, 6.12323399573676588613e-17, red);             // pi/2, low part
    const float x = (float)red, x2 = x * x;
    float sn = __builtin_fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f);
    sn = __builtin_fmaf(x2, sn, 1.0f / 120.0f);
    sn = __builtin_fmaf(x2, sn, -1.0f / 6.0f);
    sn = __builtin_fmaf(x2 * x, sn, x);
    float cn = __builtin_fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f);
    cn = __builtin_fmaf(x2, cn, -1.0f / 720.0f);
    cn = __builtin_fmaf(x2, cn, 1.0f / 24.0f);
    cn = __builtin_fmaf(x2, cn, -0.5f);
    cn = __builtin_fmaf(x2, cn, 1.0f);
    const int quad = (int)((int64_t)qd & 3);
    const float s_ = (quad & 1) ? cn : sn, c_ = (quad & 1) ? sn : cn;
    *s = (quad & 2) ? -s_ : s_;
    *c = ((quad + 1) & 2) ? -c_ : c_;
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
