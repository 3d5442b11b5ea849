/*
 * vx.h - C ABI of the MI355X (gfx950) video-DiT block hot path.
 *
 * Three operations, one per step of a video diffusion-transformer block as
 * the vidax pages describe it:
 *   vx_adaln_modulate   per-token AdaLN modulation
 *                       (vx_adaln_modulate_ex: per-sample tables, mixed dtypes)
 *   vx_rope3d_apply     3D rotary position embedding on Q and K
 *   vx_flash_attn_fwd   full non-causal attention, flash style
 * and, for attention whose keys are split into parts (sharded or in
 * passes):
 *   vx_flash_attn_fwd_kv  attention of one token set over another
 *   vx_flash_attn_fwd_masked  the same with a padded key range per sample
 *   vx_attn_merge2        two partial results combined through their LSEs
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are caller-owned DEVICE pointers (hipMalloc or a framework
 *   allocator), contiguous, row-major, 16-byte aligned.  The library never
 *   allocates, frees or keeps a pointer after it returns.
 * - Element type is given by a vx_dtype: VX_F32 (IEEE float32) or VX_BF16
 *   (bfloat16 bits, uint16 storage).  All arithmetic is float32 inside the
 *   kernels; bf16 results are rounded to nearest-even.
 * - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *   stream) on the calling thread's current device.  No call synchronises.
 * - Arguments are checked on the host before any launch.  On failure the
 *   call returns a non-zero vx_status, launches nothing, and
 *   vx_last_error() describes the problem.  A failed launch returns
 *   VX_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *   synchronisation, as for any asynchronous HIP work.
 * - Calls are re-entrant; the only global state is the per-thread error
 *   string.
 */
#ifndef VX_H
#define VX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { VX_F32 = 0, VX_BF16 = 1 } vx_dtype;

typedef enum {
    VX_OK = 0,
    VX_ERR_NULL = 1,        /* a required pointer is NULL                     */
    VX_ERR_INVALID = 2,     /* sizes or parameters inconsistent or out of range */
    VX_ERR_UNSUPPORTED = 3, /* valid, but not a shape/dtype this library serves */
    VX_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
    VX_ERR_HIP = 5          /* the HIP runtime reported an error at launch     */
} vx_status;

/*
 * Position layout of a 3D RoPE (vidax paper, arXiv 2609.18077, §2 "3D RoPE,
 * 3D VAEs, and flash attention": separate time, height and width frequency
 * bands, one convention per model family; §3.1 "CogVideoX": joint
 * text+video sequences whose text tokens carry no 3D position).
 *
 * Token order: n_prefix text tokens, then the T x H x W video grid with t
 * outermost and w innermost; video positions are the integer grid indices
 * (t, h, w), restarting at 0 after the prefix.  The head dimension is split
 * into contiguous bands [t | h | w] of widths d_t, d_h, d_w (each even,
 * d_t + d_h + d_w == head_dim).  Pair j of band a turns by angle
 * pos_a * theta^(-2j / d_a): (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos);
 * the angles of all bands, listed t then h then w, are the head's d/2
 * angles.  Which elements form a pair is the family's convention (the
 * pages stress that conventions differ per family), given by pairing:
 *   0  adjacent: elements 2j, 2j+1 of the band;
 *   1  halves of the head: the k-th angle turns elements k and k + d/2;
 *   2  halves of each band: elements j and j + d_a/2 of the band.
 * Text tokens are left unchanged.
 */
typedef struct {
    int32_t T, H, W;       /* latent token grid                              */
    int32_t n_prefix;      /* leading unrotated tokens; 0 if none            */
    int32_t d_t, d_h, d_w; /* band widths                                    */
    float theta;           /* frequency base, finite and > 0 (10000 here)    */
    int32_t pairing;       /* 0 adjacent, 1 head halves, 2 band halves        */
} vx_rope3d_desc;

/*
 * Per-token AdaLN modulation (vidax paper §2 "Spatiotemporal tensor and
 * sequence sharding" and §3.1 Table 1: Wan2.2 modulates every token with its
 * own scale and shift after a LayerNorm; the blog post "Weight offloading:
 * trading bandwidth for memory", section "A14B (Wan2.2)": that modulation
 * tensor alone reaches several GB).
 *
 *   y[n, :] = (x[n, :] - mean_n) / sqrt(var_n + eps) * (1 + scale[n, :]) + shift[n, :]
 *
 * mean_n and the biased variance var_n are taken over the `hidden` values of
 * row n; there is no learnable affine.  x, shift, scale, y: [n_tokens,
 * hidden] of type dt (one row per token).  y == x (in place) is allowed; no
 * other overlap is.
 * Errors: VX_ERR_NULL (x, shift, scale or y NULL); VX_ERR_INVALID
 * (n_tokens < 0, hidden <= 0, eps < 0 or not finite, bad dt);
 * VX_ERR_UNSUPPORTED (hidden not a multiple of 8 for bf16 or 4 for f32, or
 * above 8192: a row is held in registers);
 * VX_ERR_ALIGN.  n_rows == 0 launches nothing.
 */
vx_status vx_adaln_modulate(const void* x, const void* shift, const void* scale, void* y,
                            int64_t n_tokens, int64_t hidden, float eps, vx_dtype dt,
                            void* hip_stream);

/*
 * AdaLN modulation with per-sample or per-token tables and mixed dtypes
 * (vidax paper §3.1 and Table 1: Wan2.1 modulates all tokens of a sample
 * with one scale and shift, Wan2.2 every token with its own; §3.2 "Weight
 * import, precision, and verification": Wan2.1's residual stream and
 * LTX-2.5's AdaLN tables stay in fp32, since bf16 there degrades the
 * video).
 *
 *   y[b, n, :] = LN(x[b, n, :]) * (1 + scale[b, m, :]) + shift[b, m, :]
 *
 * with m = n when mod_tokens == n_tokens (per token) and m = 0 when
 * mod_tokens == 1 (per sample, the row broadcast over the sample's tokens).
 * LN as for vx_adaln_modulate.  x: [batch, n_tokens, hidden] of x_dt;
 * shift, scale: [batch, mod_tokens, hidden] of mod_dt; y: [batch, n_tokens,
 * hidden] of y_dt.  Each dtype is VX_F32 or VX_BF16 independently; the
 * arithmetic is float32.  vx_adaln_modulate(x, .., n_tokens, ..) is this
 * call with batch 1, mod_tokens = n_tokens and one dtype throughout.
 * y == x is allowed when x_dt == y_dt; no other overlap with y is.
 * Errors: VX_ERR_NULL; VX_ERR_INVALID (batch or n_tokens < 0, hidden <= 0,
 * mod_tokens neither n_tokens nor 1, eps < 0 or not finite, a bad dtype,
 * overlaps, y == x with different dtypes); VX_ERR_UNSUPPORTED (hidden above
 * 8192, or not a multiple of 8, of 4 when all three dtypes are f32: a row is
 * held in registers); VX_ERR_ALIGN.
 * batch * n_tokens == 0 launches nothing.
 */
vx_status vx_adaln_modulate_ex(const void* x, const void* shift, const void* scale, void* y,
                               int64_t batch, int64_t n_tokens, int64_t hidden,
                               int64_t mod_tokens, float eps, vx_dtype x_dt, vx_dtype mod_dt,
                               vx_dtype y_dt, void* hip_stream);

/*
 * 3D RoPE on Q and K, in place (vidax paper §2 "3D RoPE, 3D VAEs, and flash
 * attention").  q, k: [batch, n_tokens, heads, head_dim] of type dt; either
 * may be NULL (that tensor is skipped) but not both; q != k.  The same
 * angles apply to every head and batch entry.  V is never rotated.
 * Errors: VX_ERR_NULL (q and k NULL, or rope NULL); VX_ERR_INVALID (sizes
 * <= 0, T*H*W + n_prefix != n_tokens, grid or prefix negative, odd or
 * mis-summed bands, theta <= 0 or not finite, pairing not 0, 1 or 2, q == k);
 * VX_ERR_UNSUPPORTED (head_dim not a multiple of 8, or > 256); VX_ERR_ALIGN.
 */
vx_status vx_rope3d_apply(void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
                          int64_t head_dim, const vx_rope3d_desc* rope, vx_dtype dt,
                          void* hip_stream);

/*
 * Full non-causal attention forward (vidax paper §1: full self-attention
 * over every patch token of a multi-frame latent; §2 "3D RoPE, 3D VAEs, and
 * flash attention": unmasked attention runs as flash attention, Dao et al.
 * 2022, so the N x N score matrix is never stored).
 *
 *   o[b, i, h, :] = sum_j softmax_j(scale * q[b, i, h, :] . k[b, j, h, :]) v[b, j, h, :]
 *   lse[b, h, i]  = log sum_j exp(scale * q[b, i, h, :] . k[b, j, h, :])   (natural log)
 *
 * q, k, v, o: [batch, n_tokens, heads, head_dim] of type dt; lse: float32
 * [batch, heads, n_tokens] or NULL (not written).  softmax_scale <= 0 means
 * 1/sqrt(head_dim).  If rope_q is non-NULL, Q is rotated by that 3D RoPE in
 * registers as it is loaded (its buffer is not modified; the result equals
 * vx_rope3d_apply on Q first); K must already be rotated.  o must not
 * overlap q, k or v.
 * Precision (bf16): scores, row sums and the accumulator are fp32, and the
 * softmax weights are rounded to bf16 for the P V product.  When lse is
 * NULL, q * scale * log2(e) is also rounded to bf16 once as Q is loaded
 * (one multiply fewer per score); softmax ignores the common shift this
 * gives a row's scores, so o stays within its bf16 tolerance.  When lse is
 * given, Q is used exactly as stored and the scale is applied in fp32 before
 * each exponential, so the LSE carries only fp32 rounding and that of the
 * bf16 weights (at most 2^-9 relative in the sum).  The two forms may differ
 * in the last bits of o.
 * Errors: VX_ERR_NULL (q, k, v or o NULL); VX_ERR_INVALID (sizes <= 0,
 * softmax_scale not finite, bad rope_q as for vx_rope3d_apply, o aliasing an
 * input); VX_ERR_UNSUPPORTED (head_dim not 64 or 128, more than 2^30 tokens, or
 * heads * head_dim above 2^22); VX_ERR_ALIGN.
 */
vx_status vx_flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t batch, int64_t n_tokens, int64_t heads, int64_t head_dim,
                            float softmax_scale, const vx_rope3d_desc* rope_q, vx_dtype dt,
                            void* hip_stream);

/*
 * Attention of n_q queries over a separate set of n_kv keys (and values):
 * the same definition as vx_flash_attn_fwd with the sum over j running over
 * the n_kv keys.  This is the building block of attention whose keys are
 * split into parts, by a key-sharded sequence (vidax paper §2
 * "Spatiotemporal tensor and sequence sharding": the token axis is cut
 * across devices) or by passes over a long sequence; the parts are then
 * combined with vx_attn_merge2 through their LSEs.
 *
 * q, o: [batch, n_q, heads, head_dim]; k, v: [batch, n_kv, heads, head_dim],
 * all of type dt; lse: float32 [batch, heads, n_q] or NULL.  rope_q, if
 * non-NULL, describes the n_q query tokens (T*H*W + n_prefix == n_q).
 * vx_flash_attn_fwd(..., n_tokens, ...) is this call with n_q = n_kv =
 * n_tokens.  Errors: as vx_flash_attn_fwd, with n_q <= 0 or n_kv <= 0
 * reported as VX_ERR_INVALID.
 */
vx_status vx_flash_attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t batch, int64_t n_q, int64_t n_kv, int64_t heads,
                               int64_t head_dim, float softmax_scale,
                               const vx_rope3d_desc* rope_q, vx_dtype dt, void* hip_stream);

/*
 * Attention with key padding: as vx_flash_attn_fwd_kv, with keys
 * key_pad[2 b] <= j < key_pad[2 b + 1] of batch entry b taking no weight
 * (excluded from the softmax sum).  The vidax pages run CogVideoX's joint
 * text+video attention over a fixed-length text prefix (paper §3.1
 * "CogVideoX"), and report that padding left unmasked drifts CogVideoX's
 * T5 text embeddings in bf16 (agihunt.info summary); a padded range of keys
 * is what such a mask removes: the padded tail of a text prefix, or
 * [len_b, n_kv) for a padded key tail.
 *
 * key_pad: HOST array of 2 * batch int32 (lo, hi) pairs, read during the
 * call (not kept); lo == hi masks nothing for that entry.  batch <= 64.
 * Other arguments as vx_flash_attn_fwd_kv; lse of a row is the log-sum-exp
 * over its unmasked keys.
 * Errors: as vx_flash_attn_fwd_kv; VX_ERR_NULL (key_pad NULL);
 * VX_ERR_INVALID (a range outside 0 <= lo <= hi <= n_kv, or one that
 * leaves no valid key); VX_ERR_UNSUPPORTED (batch > 64).
 */
vx_status vx_flash_attn_fwd_masked(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int64_t batch, int64_t n_q, int64_t n_kv,
                                   int64_t heads, int64_t head_dim, float softmax_scale,
                                   const vx_rope3d_desc* rope_q, const int32_t* key_pad,
                                   vx_dtype dt, void* hip_stream);

/*
 * Merge of two partial attention results over disjoint key sets A and B
 * into the result over A u B (the consumer of the LSE output; same source
 * as vx_flash_attn_fwd_kv):
 *
 *   lse = log(exp(lse_a) + exp(lse_b))
 *   o   = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b
 *
 * per (batch, token, head).  o_a, o_b, o: [batch, n_tokens, heads, head_dim]
 * of type dt; lse_a, lse_b: float32 [batch, heads, n_tokens]; lse: the same,
 * or NULL (not written).  Both LSEs -inf (two empty parts) gives o = 0 and
 * lse = -inf.  In place is allowed: o may be exactly o_a or o_b, lse exactly
 * lse_a or lse_b; any other overlap is invalid.  P parts merge pairwise (the
 * operation is associative up to rounding).
 * Errors: VX_ERR_NULL (o_a, lse_a, o_b, lse_b or o NULL); VX_ERR_INVALID
 * (sizes <= 0, bad dt, overlaps); VX_ERR_UNSUPPORTED (head_dim not 64 or
 * 128); VX_ERR_ALIGN (o tensors not 16-byte, LSEs not 4-byte aligned).
 */
vx_status vx_attn_merge2(const void* o_a, const float* lse_a, const void* o_b,
                         const float* lse_b, void* o, float* lse, int64_t batch,
                         int64_t n_tokens, int64_t heads, int64_t head_dim, vx_dtype dt,
                         void* hip_stream);

/* Message of the last failed vx_* call on this thread ("" if none). */
const char* vx_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int vx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VX_H */
