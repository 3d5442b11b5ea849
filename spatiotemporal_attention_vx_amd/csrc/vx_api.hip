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
hipError_t launch_adaln(const void* x, const void* shift, const void* scale, void* y,
                        int64_t rows, int64_t hidden, float eps, bool bf16, hipStream_t st);
hipError_t launch_rope3d(void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
                         int64_t head_dim, const RopeArgs& r, bool bf16, hipStream_t st);
hipError_t launch_flash_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t batch, int64_t n, int64_t heads, int64_t head_dim,
                             float scale, const RopeArgs* rope, bool bf16, hipStream_t st);
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
    const int64_t nv = (int64_t)r->T * r->H * r->W;
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
    if (r->pairing != 0)
        return fail(VX_ERR_INVALID, "%s: rope pairing %d is reserved (only 0, adjacent pairs)", fn,
                    r->pairing);
    *out = vx::RopeArgs{r->T, r->H, r->W, r->n_prefix, r->d_t, r->d_h, r->d_w, r->theta};
    return VX_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(VX_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int vx_adaln_modulate(const void* x, const void* shift, const void* scale, void* y,
                      int64_t n_rows, int64_t hidden, float eps, int dt, void* hip_stream) {
    if (!x || !shift || !scale || !y) return fail(VX_ERR_NULL, "vx_adaln_modulate: NULL tensor");
    if (int e = check_dtype("vx_adaln_modulate", dt)) return e;
    if (n_rows < 0 || hidden <= 0)
        return fail(VX_ERR_INVALID, "vx_adaln_modulate: n_rows %lld, hidden %lld", (long long)n_rows,
                    (long long)hidden);
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(VX_ERR_INVALID, "vx_adaln_modulate: eps %g must be finite and >= 0", (double)eps);
    const bool bf16 = dt == VX_BF16;
    const int64_t epc = bf16 ? 8 : 4, max_hidden = bf16 ? 8192 : 4096, esz = bf16 ? 2 : 4;
    if (hidden % epc != 0 || hidden > max_hidden)
        return fail(VX_ERR_UNSUPPORTED, "vx_adaln_modulate: hidden %lld must be a multiple of %lld and <= %lld",
                    (long long)hidden, (long long)epc, (long long)max_hidden);
    if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(y))
        return fail(VX_ERR_ALIGN, "vx_adaln_modulate: tensors must be 16-byte aligned");
    int64_t bytes;
    if (!mul_ok(bytes, {n_rows, hidden, esz}) || (n_rows + 3) / 4 > INT32_MAX)
        return fail(VX_ERR_INVALID, "vx_adaln_modulate: size overflow");
    if (y != x && (overlaps(y, bytes, x, bytes) || overlaps(y, bytes, shift, bytes) ||
                   overlaps(y, bytes, scale, bytes)))
        return fail(VX_ERR_INVALID, "vx_adaln_modulate: y overlaps an input (only y == x is allowed)");
    if (y == x && (overlaps(y, bytes, shift, bytes) || overlaps(y, bytes, scale, bytes)))
        return fail(VX_ERR_INVALID, "vx_adaln_modulate: y overlaps shift or scale");
    if (n_rows == 0) return ok();
    return launched(vx::launch_adaln(x, shift, scale, y, n_rows, hidden, eps, bf16,
                                     (hipStream_t)hip_stream),
                    "vx_adaln_modulate");
}

int vx_rope3d_apply(void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
                    int64_t head_dim, const vx_rope3d_desc* rope, int dt, void* hip_stream) {
    if ((!q && !k) || !rope) return fail(VX_ERR_NULL, "vx_rope3d_apply: q and k both NULL, or rope NULL");
    if (int e = check_dtype("vx_rope3d_apply", dt)) return e;
    if (batch <= 0 || n_tokens <= 0 || heads <= 0 || head_dim <= 0)
        return fail(VX_ERR_INVALID, "vx_rope3d_apply: sizes must be positive");
    if (q == k) return fail(VX_ERR_INVALID, "vx_rope3d_apply: q and k must differ");
    if (head_dim % 8 != 0 || head_dim > 256)
        return fail(VX_ERR_UNSUPPORTED, "vx_rope3d_apply: head_dim %lld must be a multiple of 8 and <= 256",
                    (long long)head_dim);
    vx::RopeArgs r;
    if (int e = check_rope("vx_rope3d_apply", rope, n_tokens, head_dim, &r)) return e;
    if ((q && !aligned16(q)) || (k && !aligned16(k)))
        return fail(VX_ERR_ALIGN, "vx_rope3d_apply: tensors must be 16-byte aligned");
    const int64_t esz = dt == VX_BF16 ? 2 : 4;
    int64_t bytes, rows;
    if (!mul_ok(bytes, {batch, n_tokens, heads, head_dim, esz}) || !mul_ok(rows, {batch, n_tokens}) ||
        heads * head_dim / (esz == 2 ? 8 : 4) > INT32_MAX / 4 || (rows + 3) / 4 > INT32_MAX)
        return fail(VX_ERR_INVALID, "vx_rope3d_apply: size overflow");
    if (q && k && overlaps(q, bytes, k, bytes))
        return fail(VX_ERR_INVALID, "vx_rope3d_apply: q and k overlap");
    return launched(vx::launch_rope3d(q, k, batch, n_tokens, heads, head_dim, r, dt == VX_BF16,
                                      (hipStream_t)hip_stream),
                    "vx_rope3d_apply");
}

int vx_flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t batch, int64_t n_tokens, int64_t heads, int64_t head_dim,
                      float softmax_scale, const vx_rope3d_desc* rope_q, int dt,
                      void* hip_stream) {
    if (!q || !k || !v || !o) return fail(VX_ERR_NULL, "vx_flash_attn_fwd: NULL tensor");
    if (int e = check_dtype("vx_flash_attn_fwd", dt)) return e;
    if (batch <= 0 || n_tokens <= 0 || heads <= 0 || head_dim <= 0)
        return fail(VX_ERR_INVALID, "vx_flash_attn_fwd: sizes must be positive");
    if (!std::isfinite(softmax_scale))
        return fail(VX_ERR_INVALID, "vx_flash_attn_fwd: softmax_scale must be finite");
    if (head_dim != 64 && head_dim != 128)
        return fail(VX_ERR_UNSUPPORTED, "vx_flash_attn_fwd: head_dim %lld (64 or 128 only)",
                    (long long)head_dim);
    vx::RopeArgs r;
    if (rope_q)
        if (int e = check_rope("vx_flash_attn_fwd", rope_q, n_tokens, head_dim, &r)) return e;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fail(VX_ERR_ALIGN, "vx_flash_attn_fwd: q, k, v, o must be 16-byte aligned, lse 4-byte");
    const bool bf16 = dt == VX_BF16;
    const int64_t esz = bf16 ? 2 : 4;
    int64_t bytes, lse_bytes, rows;
    const int64_t per_wg = vx::flash_attn_rows_per_workgroup(bf16, head_dim);
    if (!mul_ok(bytes, {batch, n_tokens, heads, head_dim, esz}) ||
        !mul_ok(lse_bytes, {batch, heads, n_tokens, 4}) ||
        !mul_ok(rows, {batch, heads, (n_tokens + per_wg - 1) / per_wg}) || rows > INT32_MAX)
        return fail(VX_ERR_INVALID, "vx_flash_attn_fwd: size overflow");
    if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
        return fail(VX_ERR_INVALID, "vx_flash_attn_fwd: o overlaps q, k or v");
    if (lse && (overlaps(lse, lse_bytes, q, bytes) || overlaps(lse, lse_bytes, k, bytes) ||
                overlaps(lse, lse_bytes, v, bytes) || overlaps(lse, lse_bytes, o, bytes)))
        return fail(VX_ERR_INVALID, "vx_flash_attn_fwd: lse overlaps a tensor");
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    return launched(vx::launch_flash_attn(q, k, v, o, lse, batch, n_tokens, heads, head_dim, scale,
                                          rope_q ? &r : nullptr, bf16, (hipStream_t)hip_stream),
                    "vx_flash_attn_fwd");
}

const char* vx_last_error(void) { return g_error.c_str(); }

int vx_version(void) { return 100; }

}  // extern "C"
