// C ABI of the hot path: host-side argument checks, error reporting and
// dispatch to the gfx950 kernels.  Nothing here allocates device memory or
// synchronises; every check runs before any HIP call.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include <hip/hip_runtime.h>

#include "../../include/vx.h"
#include "vx_device.h"

namespace vx {
hipError_t launch_adaln_per_token(const void* x, const void* shift, const void* scale, void* y,
                                  int64_t rows, int64_t hidden, float eps, bool xb, bool mb,
                                  bool yb, hipStream_t st);
hipError_t launch_adaln_per_sample(const void* x, const void* shift, const void* scale, void* y,
                                   int64_t rows, int64_t n_tokens, int64_t hidden, float eps,
                                   bool xb, bool mb, bool yb, hipStream_t st);
hipError_t launch_rope3d(void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
                         int64_t head_dim, const RopeArgs& r, bool bf16, hipStream_t st);
hipError_t launch_flash_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t batch, int64_t nq, int64_t nk, int64_t heads,
                             int64_t head_dim, float scale, const RopeArgs* rope,
                             const int32_t* key_pad, bool bf16, hipStream_t st);
constexpr int FA_MAX_PAD_BATCH = 64;
hipError_t launch_attn_merge(const void* oa, const float* lsea, const void* ob, const float* lseb,
                             void* o, float* lse, int64_t batch, int64_t n, int64_t heads,
                             int64_t head_dim, bool bf16, hipStream_t st);
int flash_attn_rows_per_workgroup(bool bf16, int64_t head_dim);
}  // namespace vx

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int ok() {
    g_error.clear();
    return VX_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

// a * b * ... without int64 overflow; false on overflow or a negative factor
bool mul_ok(int64_t& out, std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x < 0) return false;
        if (x != 0 && r > INT64_MAX / x) return false;
        r *= x;
    }
    out = r;
    return true;
}

int check_dtype(const char* fn, int dt) {
    if (dt != VX_F32 && dt != VX_BF16)
        return fail(VX_ERR_INVALID, "%s: dtype %d is not VX_F32 or VX_BF16", fn, dt);
    return VX_OK;
}

int check_rope(const char* fn, const vx_rope3d_desc* r, int64_t n_tokens, int64_t head_dim,
               vx::RopeArgs* out) {
    if (r->T < 0 || r->H < 0 || r->W < 0 || r->n_prefix < 0)
        return fail(VX_ERR_INVALID, "%s: rope grid (%d,%d,%d) and prefix %d must be non-negative",
                    fn, r->T, r->H, r->W, r->n_prefix);
    int64_t nv;
    if (!mul_ok(nv, {r->T, r->H, r->W}) || nv > INT64_MAX - r->n_prefix)
        return fail(VX_ERR_INVALID, "%s: rope grid %dx%dx%d + prefix %d overflows", fn, r->T, r->H,
                    r->W, r->n_prefix);
    if (nv + r->n_prefix != n_tokens)
        return fail(VX_ERR_INVALID, "%s: rope grid %dx%dx%d + prefix %d = %lld tokens, but n_tokens = %lld",
                    fn, r->T, r->H, r->W, r->n_prefix, (long long)(nv + r->n_prefix), (long long)n_tokens);
    if (r->d_t < 0 || r->d_h < 0 || r->d_w < 0 || (r->d_t | r->d_h | r->d_w) & 1)
        return fail(VX_ERR_INVALID, "%s: rope bands (%d,%d,%d) must be even and non-negative",
                    fn, r->d_t, r->d_h, r->d_w);
    if ((int64_t)r->d_t + r->d_h + r->d_w != head_dim)
        return fail(VX_ERR_INVALID, "%s: rope bands (%d,%d,%d) do not sum to head_dim %lld",
                    fn, r->d_t, r->d_h, r->d_w, (long long)head_dim);
    if (!std::isfinite(r->theta) || r->theta <= 0.f)
        return fail(VX_ERR_INVALID, "%s: rope theta %g must be finite and positive", fn,
                    (double)r->theta);
    if (r->pairing < 0 || r->pairing > 2)
        return fail(VX_ERR_INVALID, "%s: rope pairing %d is not 0 (adjacent), 1 (head halves) "
                    "or 2 (band halves)", fn, r->pairing);
    if (head_dim / 2 > vx::ROPE_MAX_PAIRS)
        return fail(VX_ERR_UNSUPPORTED, "%s: rope head_dim %lld above %d", fn, (long long)head_dim,
                    2 * vx::ROPE_MAX_PAIRS);
    vx::RopeArgs a{};
    a.T = r->T; a.H = r->H; a.W = r->W; a.n_prefix = r->n_prefix;
    a.d_t = r->d_t; a.d_h = r->d_h; a.d_w = r->d_w; a.pairing = r->pairing;
    // pair j of band a turns at theta^(-2j / d_a); bands listed t, h, w
    int pair = 0;
    for (int width : {r->d_t, r->d_h, r->d_w})
        for (int j = 0; j < width / 2; ++j)
            a.freq[pair++] = std::pow((double)r->theta, -2.0 * j / (double)width);
    *out = a;
    return VX_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(VX_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// Checks shared by the two AdaLN entry points.  Rows are batch * n_tokens;
// the tables hold mod_tokens rows per batch entry (n_tokens: per token; 1:
// per sample).
int adaln(const char* fn, const void* x, const void* shift, const void* scale, void* y,
          int64_t batch, int64_t n_tokens, int64_t hidden, int64_t mod_tokens, float eps,
          int x_dt, int mod_dt, int y_dt, void* hip_stream) {
    if (!x || !shift || !scale || !y) return fail(VX_ERR_NULL, "%s: NULL tensor", fn);
    for (int dt : {x_dt, mod_dt, y_dt})
        if (int e = check_dtype(fn, dt)) return e;
    if (batch < 0 || n_tokens < 0 || hidden <= 0)
        return fail(VX_ERR_INVALID, "%s: batch %lld, n_tokens %lld, hidden %lld", fn,
                    (long long)batch, (long long)n_tokens, (long long)hidden);
    if (mod_tokens != n_tokens && mod_tokens != 1)
        return fail(VX_ERR_INVALID, "%s: mod_tokens %lld must be n_tokens (%lld) or 1", fn,
                    (long long)mod_tokens, (long long)n_tokens);
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(VX_ERR_INVALID, "%s: eps %g must be finite and >= 0", fn, (double)eps);
    const bool xb = x_dt == VX_BF16, mb = mod_dt == VX_BF16, yb = y_dt == VX_BF16;
    // A row lives in registers, at most 16 groups of 8 elements per lane (32
    // of 4 when every tensor is f32): 8192 wide either way.
    const int64_t group = (xb || mb || yb) ? 8 : 4, max_hidden = 8192;
    if (hidden % group != 0 || hidden > max_hidden)
        return fail(VX_ERR_UNSUPPORTED, "%s: hidden %lld must be a multiple of %lld and <= %lld",
                    fn, (long long)hidden, (long long)group, (long long)max_hidden);
    if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(y))
        return fail(VX_ERR_ALIGN, "%s: tensors must be 16-byte aligned", fn);
    int64_t rows, xbytes, mbytes, ybytes;
    if (!mul_ok(rows, {batch, n_tokens}) || !mul_ok(xbytes, {rows, hidden, xb ? 2 : 4}) ||
        !mul_ok(mbytes, {batch, mod_tokens, hidden, mb ? 2 : 4}) ||
        !mul_ok(ybytes, {rows, hidden, yb ? 2 : 4}) || (rows + 3) / 4 > INT32_MAX)
        return fail(VX_ERR_INVALID, "%s: size overflow", fn);
    if (y == x) {
        if (x_dt != y_dt)
            return fail(VX_ERR_INVALID, "%s: y == x needs the same dtype for both", fn);
        if (overlaps(y, ybytes, shift, mbytes) || overlaps(y, ybytes, scale, mbytes))
            return fail(VX_ERR_INVALID, "%s: y overlaps shift or scale", fn);
    } else if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, shift, mbytes) ||
               overlaps(y, ybytes, scale, mbytes)) {
        return fail(VX_ERR_INVALID, "%s: y overlaps an input (only y == x is allowed)", fn);
    }
    if (rows == 0) return ok();
    const hipStream_t st = (hipStream_t)hip_stream;
    const hipError_t e = (mod_tokens == n_tokens)
        ? vx::launch_adaln_per_token(x, shift, scale, y, rows, hidden, eps, xb, mb, yb, st)
        : vx::launch_adaln_per_sample(x, shift, scale, y, rows, n_tokens, hidden, eps, xb, mb,
                                      yb, st);
    return launched(e, fn);
}

// Checks shared by the two attention entry points; nq == nk for the
// self-attention one.
int flash_attn(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse,
               int64_t batch, int64_t nq, int64_t nk, int64_t heads, int64_t head_dim,
               float softmax_scale, const vx_rope3d_desc* rope_q, const int32_t* key_pad, int dt,
               void* hip_stream) {
    if (!q || !k || !v || !o) return fail(VX_ERR_NULL, "%s: NULL tensor", fn);
    if (int e = check_dtype(fn, dt)) return e;
    if (batch <= 0 || nq <= 0 || nk <= 0 || heads <= 0 || head_dim <= 0)
        return fail(VX_ERR_INVALID, "%s: sizes must be positive", fn);
    if (!std::isfinite(softmax_scale))
        return fail(VX_ERR_INVALID, "%s: softmax_scale must be finite", fn);
    if (head_dim != 64 && head_dim != 128)
        return fail(VX_ERR_UNSUPPORTED, "%s: head_dim %lld (64 or 128 only)", fn, (long long)head_dim);
    if (nq > (int64_t(1) << 30) || nk > (int64_t(1) << 30))
        return fail(VX_ERR_UNSUPPORTED, "%s: token counts above 2^30", fn);
    // a tile of up to 128 token rows must fit one 2^31-byte buffer resource
    // (compared by division: heads * head_dim itself may not fit in int64)
    if (heads > (int64_t(1) << 22) / head_dim)
        return fail(VX_ERR_UNSUPPORTED, "%s: heads %lld * head_dim %lld above 2^22", fn,
                    (long long)heads, (long long)head_dim);
    vx::RopeArgs r;
    if (rope_q)
        if (int e = check_rope(fn, rope_q, nq, head_dim, &r)) return e;
    if (key_pad) {
        if (batch > vx::FA_MAX_PAD_BATCH)
            return fail(VX_ERR_UNSUPPORTED, "%s: key padding serves batch <= %d, not %lld", fn,
                        vx::FA_MAX_PAD_BATCH, (long long)batch);
        for (int64_t i = 0; i < batch; ++i) {
            const int64_t lo = key_pad[2 * i], hi = key_pad[2 * i + 1];
            if (lo < 0 || hi < lo || hi > nk || hi - lo >= nk)
                return fail(VX_ERR_INVALID, "%s: key_pad[%lld] = [%lld, %lld) must satisfy "
                            "0 <= lo <= hi <= n_kv and leave a valid key (n_kv = %lld)", fn,
                            (long long)i, (long long)lo, (long long)hi, (long long)nk);
        }
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fail(VX_ERR_ALIGN, "%s: q, k, v, o must be 16-byte aligned, lse 4-byte", fn);
    const bool bf16 = dt == VX_BF16;
    const int64_t esz = bf16 ? 2 : 4;
    int64_t qbytes, kbytes, lse_bytes, rows;
    const int64_t per_wg = vx::flash_attn_rows_per_workgroup(bf16, head_dim);
    if (!mul_ok(qbytes, {batch, nq, heads, head_dim, esz}) ||
        !mul_ok(kbytes, {batch, nk, heads, head_dim, esz}) ||
        !mul_ok(lse_bytes, {batch, heads, nq, 4}) ||
        !mul_ok(rows, {batch, heads, (nq + per_wg - 1) / per_wg}) || rows > INT32_MAX)
        return fail(VX_ERR_INVALID, "%s: size overflow", fn);
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
        return fail(VX_ERR_INVALID, "%s: o overlaps q, k or v", fn);
    if (lse && (overlaps(lse, lse_bytes, q, qbytes) || overlaps(lse, lse_bytes, k, kbytes) ||
                overlaps(lse, lse_bytes, v, kbytes) || overlaps(lse, lse_bytes, o, qbytes)))
        return fail(VX_ERR_INVALID, "%s: lse overlaps a tensor", fn);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    return launched(vx::launch_flash_attn(q, k, v, o, lse, batch, nq, nk, heads, head_dim, scale,
                                          rope_q ? &r : nullptr, key_pad, bf16,
                                          (hipStream_t)hip_stream),
                    fn);
}

int rope3d(const char* fn, void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
           int64_t head_dim, const vx_rope3d_desc* rope, int dt, void* hip_stream) {
    if ((!q && !k) || !rope) return fail(VX_ERR_NULL, "%s: q and k both NULL, or rope NULL", fn);
    if (int e = check_dtype(fn, dt)) return e;
    if (batch <= 0 || n_tokens <= 0 || heads <= 0 || head_dim <= 0)
        return fail(VX_ERR_INVALID, "%s: sizes must be positive", fn);
    if (q == k) return fail(VX_ERR_INVALID, "%s: q and k must differ", fn);
    if (head_dim % 8 != 0 || head_dim > 256)
        return fail(VX_ERR_UNSUPPORTED, "%s: head_dim %lld must be a multiple of 8 and <= 256", fn,
                    (long long)head_dim);
    vx::RopeArgs r;
    if (int e = check_rope(fn, rope, n_tokens, head_dim, &r)) return e;
    if ((q && !aligned16(q)) || (k && !aligned16(k)))
        return fail(VX_ERR_ALIGN, "%s: tensors must be 16-byte aligned", fn);
    const int64_t esz = dt == VX_BF16 ? 2 : 4;
    int64_t bytes, rows;
    if (!mul_ok(bytes, {batch, n_tokens, heads, head_dim, esz}) || !mul_ok(rows, {batch, n_tokens}) ||
        heads * head_dim / (esz == 2 ? 8 : 4) > INT32_MAX / 4 || (rows + 3) / 4 > INT32_MAX)
        return fail(VX_ERR_INVALID, "%s: size overflow", fn);
    if (q && k && overlaps(q, bytes, k, bytes))
        return fail(VX_ERR_INVALID, "%s: q and k overlap", fn);
    return launched(vx::launch_rope3d(q, k, batch, n_tokens, heads, head_dim, r, dt == VX_BF16,
                                      (hipStream_t)hip_stream),
                    fn);
}

int attn_merge2(const char* fn, const void* o_a, const float* lse_a, const void* o_b,
                const float* lse_b, void* o, float* lse, int64_t batch, int64_t n_tokens,
                int64_t heads, int64_t head_dim, int dt, void* hip_stream) {
    if (!o_a || !lse_a || !o_b || !lse_b || !o) return fail(VX_ERR_NULL, "%s: NULL tensor", fn);
    if (int e = check_dtype(fn, dt)) return e;
    if (batch <= 0 || n_tokens <= 0 || heads <= 0 || head_dim <= 0)
        return fail(VX_ERR_INVALID, "%s: sizes must be positive", fn);
    if (head_dim != 64 && head_dim != 128)
        return fail(VX_ERR_UNSUPPORTED, "%s: head_dim %lld (64 or 128 only)", fn, (long long)head_dim);
    const uintptr_t lmask = 3u;
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(lse_a) & lmask) || (reinterpret_cast<uintptr_t>(lse_b) & lmask) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & lmask)))
        return fail(VX_ERR_ALIGN, "%s: o tensors must be 16-byte aligned, lse 4-byte", fn);
    const bool bf16 = dt == VX_BF16;
    int64_t bytes, lse_bytes, chunks;
    if (!mul_ok(bytes, {batch, n_tokens, heads, head_dim, bf16 ? 2 : 4}) ||
        !mul_ok(lse_bytes, {batch, heads, n_tokens, 4}) || !mul_ok(chunks, {bytes / 16}) ||
        (chunks + 255) / 256 > INT32_MAX)
        return fail(VX_ERR_INVALID, "%s: size overflow", fn);
    // o may be o_a or o_b exactly (in place); any other overlap is invalid.
    // The same holds for lse against lse_a / lse_b.
    if ((o != o_a && overlaps(o, bytes, o_a, bytes)) || (o != o_b && overlaps(o, bytes, o_b, bytes)))
        return fail(VX_ERR_INVALID, "%s: o overlaps o_a or o_b other than exactly", fn);
    if (lse && ((lse != lse_a && overlaps(lse, lse_bytes, lse_a, lse_bytes)) ||
                (lse != lse_b && overlaps(lse, lse_bytes, lse_b, lse_bytes))))
        return fail(VX_ERR_INVALID, "%s: lse overlaps lse_a or lse_b other than exactly", fn);
    if (overlaps(o, bytes, lse_a, lse_bytes) || overlaps(o, bytes, lse_b, lse_bytes) ||
        (lse && (overlaps(lse, lse_bytes, o_a, bytes) || overlaps(lse, lse_bytes, o_b, bytes) ||
                 overlaps(lse, lse_bytes, o, bytes))))
        return fail(VX_ERR_INVALID, "%s: an output overlaps a tensor of the other kind", fn);
    return launched(vx::launch_attn_merge(o_a, lse_a, o_b, lse_b, o, lse, batch, n_tokens, heads,
                                          head_dim, bf16, (hipStream_t)hip_stream),
                    fn);
}

// Every entry point returns one of the vx_status codes.
vx_status st(int code) { return static_cast<vx_status>(code); }

}  // namespace

extern "C" {

vx_status vx_adaln_modulate(const void* x, const void* shift, const void* scale, void* y,
                            int64_t n_tokens, int64_t hidden, float eps, vx_dtype dt,
                            void* hip_stream) {
    return st(adaln("vx_adaln_modulate", x, shift, scale, y, 1, n_tokens, hidden, n_tokens, eps,
                    dt, dt, dt, hip_stream));
}

vx_status vx_adaln_modulate_ex(const void* x, const void* shift, const void* scale, void* y,
                               int64_t batch, int64_t n_tokens, int64_t hidden,
                               int64_t mod_tokens, float eps, vx_dtype x_dt, vx_dtype mod_dt,
                               vx_dtype y_dt, void* hip_stream) {
    return st(adaln("vx_adaln_modulate_ex", x, shift, scale, y, batch, n_tokens, hidden,
                    mod_tokens, eps, x_dt, mod_dt, y_dt, hip_stream));
}

vx_status vx_rope3d_apply(void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
                          int64_t head_dim, const vx_rope3d_desc* rope, vx_dtype dt,
                          void* hip_stream) {
    return st(rope3d("vx_rope3d_apply", q, k, batch, n_tokens, heads, head_dim, rope, dt,
                     hip_stream));
}

vx_status vx_flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t batch, int64_t n_tokens, int64_t heads, int64_t head_dim,
                            float softmax_scale, const vx_rope3d_desc* rope_q, vx_dtype dt,
                            void* hip_stream) {
    return st(flash_attn("vx_flash_attn_fwd", q, k, v, o, lse, batch, n_tokens, n_tokens, heads,
                         head_dim, softmax_scale, rope_q, nullptr, dt, hip_stream));
}

vx_status vx_flash_attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t batch, int64_t n_q, int64_t n_kv, int64_t heads,
                               int64_t head_dim, float softmax_scale,
                               const vx_rope3d_desc* rope_q, vx_dtype dt, void* hip_stream) {
    return st(flash_attn("vx_flash_attn_fwd_kv", q, k, v, o, lse, batch, n_q, n_kv, heads,
                         head_dim, softmax_scale, rope_q, nullptr, dt, hip_stream));
}

vx_status vx_flash_attn_fwd_masked(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int64_t batch, int64_t n_q, int64_t n_kv,
                                   int64_t heads, int64_t head_dim, float softmax_scale,
                                   const vx_rope3d_desc* rope_q, const int32_t* key_pad,
                                   vx_dtype dt, void* hip_stream) {
    if (!key_pad) return st(fail(VX_ERR_NULL, "vx_flash_attn_fwd_masked: key_pad NULL"));
    return st(flash_attn("vx_flash_attn_fwd_masked", q, k, v, o, lse, batch, n_q, n_kv, heads,
                         head_dim, softmax_scale, rope_q, key_pad, dt, hip_stream));
}

vx_status vx_attn_merge2(const void* o_a, const float* lse_a, const void* o_b,
                         const float* lse_b, void* o, float* lse, int64_t batch,
                         int64_t n_tokens, int64_t heads, int64_t head_dim, vx_dtype dt,
                         void* hip_stream) {
    return st(attn_merge2("vx_attn_merge2", o_a, lse_a, o_b, lse_b, o, lse, batch, n_tokens,
                          heads, head_dim, dt, hip_stream));
}

const char* vx_last_error(void) { return g_error.c_str(); }

int vx_version(void) { return 201; }

}  // extern "C"
