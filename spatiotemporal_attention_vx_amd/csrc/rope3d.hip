// 3D RoPE on Q and K, in place, for gfx950.
//
// Separate time/height/width frequency bands of the head dimension, one
// convention per model family (vidax paper, arXiv 2609.18077, §2 "3D RoPE,
// 3D VAEs, and flash attention"); text-prefix tokens of a joint text+video
// sequence are not rotated (§3.1, "CogVideoX").  The position layout is the
// one documented on vx_rope3d_desc.
//
// HBM-bound: each rotated row of Q and K is read and written once.  A
// workgroup owns TPB consecutive tokens.  It evaluates cos/sin of the
// head_dim/2 angles of each token into LDS (angles are shared by every head
// and by Q and K, so they cost one evaluation per token and pair) after
// issuing the first loads of the tokens' rows, then streams the 16-byte
// chunks of the Q and K rows, consecutive lanes on consecutive chunks, each
// thread with several loads in flight; rows far larger than the memory-side
// cache are read and written with non-temporal accesses.  With adjacent pairs (pairing 0) both elements of
// a pair sit in one chunk.  With halves of the head (pairing 1) the two
// elements sit in chunks c and c + (chunks per row) / 2 whenever head_dim / 2
// is a whole number of chunks, and one thread rotates that chunk pair.
// Otherwise (halves of each band, pairing 2, or an odd split) a pair spans
// chunks irregularly, so each head row is staged through LDS first and every
// lane reads its elements' partners there.
#include "vx_device.h"

namespace vx {

constexpr int ROPE_TPB = 4;          // tokens per workgroup
constexpr int ROPE_MAX_HALF = ROPE_MAX_PAIRS;

// Q and K rows are read once and written once.  When the rotated tensors
// are much larger than the 256 MiB memory-side cache (NT), non-temporal
// accesses keep them from displacing what is cached and from leaving dirty
// lines behind: the large workload's K (774 MB) then rotates at 76% of HBM
// in the hot path instead of 74%, and 72% instead of 66% back to back.
// Smaller tensors gain from staying partly cached between launches (K of
// 277-528 MB: 77-82% in the hot path with plain accesses, 75-78% with
// non-temporal ones), so the host picks NT by size.
constexpr int64_t ROPE_NT_BYTES = int64_t(640) << 20;   // 2.5 x the memory-side cache

template <bool NT>
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
        return uint4{v[0], v[1], v[2], v[3]};
    } else {
        return *p;
    }
}
template <bool NT>
__device__ __forceinline__ void stream_store(uint4* p, const uint4& v) {
    if constexpr (NT) __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (u32x4_t*)p);
    else *p = v;
}

// Adjacent pairs.  Every thread owns the (token, tensor, chunk) items
// threadIdx.x + 256 j of its workgroup, chunk index fastest, and handles
// them BATCH at a time: all loads of a batch are issued before any chunk is
// rotated and stored, so each thread keeps BATCH 16-byte loads in flight (a
// load issued after a store to another chunk could not be moved above it).
// The first batch is loaded before the angles are evaluated.  Each angle's
// pair frequency is itself a load issued after that batch, so the
// evaluation starts once the batch has landed (loads complete in issue
// order); fetching the frequencies first, so the evaluation runs under the
// batch, measured no faster.  Text-prefix rows are read but never written.
// BATCH is 8 when every thread has at least 8 chunks (wide token rows), else
// 4: eight loads in flight need 87 VGPRs (5 waves per SIMD) against 56 (8
// waves), and rows of a few heads gain more from occupancy than from depth.
constexpr int ROPE_BATCH = 4;        // head-half kernel: loads in flight per thread

template <bool BF16, int BATCH, bool NT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope3d_kernel(uint4* q, uint4* k, int64_t rows, int64_t n_tokens, int heads,
                   int head_dim, RopeArgs r) {
    constexpr int EPC = BF16 ? 8 : 4;    // elements per 16-byte chunk
    __shared__ f32x2_t cs[ROPE_TPB * ROPE_MAX_HALF];
    __shared__ int rotate[ROPE_TPB];     // token exists and is not text
    const int half = head_dim >> 1;
    const int64_t row0 = (int64_t)blockIdx.x * ROPE_TPB;
    const int ntok = (int)(rows - row0 < ROPE_TPB ? rows - row0 : ROPE_TPB);   // >= 1
    const int dpr = head_dim / EPC;      // chunks per head row
    const int cpr = heads * dpr;         // chunks per token row
    // the tensors present (the host passes at least one), q first
    uint4* const ten0 = q != nullptr ? q : k;
    uint4* const ten1 = q != nullptr ? k : nullptr;
    const int nten = ten1 != nullptr ? 2 : 1;

    int c = threadIdx.x, which = 0, tk = 0;
    auto advance = [&]() {
        c += 256;
        while (c >= cpr) { c -= cpr; if (++which == nten) { which = 0; ++tk; } }
    };
    while (c >= cpr) { c -= cpr; if (++which == nten) { which = 0; ++tk; } }

    uint4 v[BATCH];
    uint4* ptr[BATCH];
    int slot[BATCH];                     // tk * half + first pair of the chunk; -1: none
    auto load_batch = [&]() {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) slot[u] = -1;
        // stop at the workgroup's last item: with few heads a thread has only
        // one or two, and walking past them would cost more than the loads
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (tk >= ntok) break;
            ptr[u] = (which ? ten1 : ten0) + (row0 + tk) * cpr + c;
            v[u] = stream_load<NT>(ptr[u]);
            slot[u] = tk * half + (c % dpr) * (EPC / 2);
            advance();
        }
    };
    auto rotate_store_batch = [&]() {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (slot[u] < 0 || !rotate[slot[u] / half]) continue;
            const f32x2_t* t = cs + slot[u];
            uint4 w4 = v[u];
            if constexpr (BF16) {
                uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float a = bf16_lo(w[m]), b = bf16_hi(w[m]);
                    const f32x2_t e = t[m];
                    rope_rotate(a, b, e.x, e.y);
                    w[m] = pack_bf16x2(a, b);
                }
                w4 = uint4{w[0], w[1], w[2], w[3]};
            } else {
                float f[4] = {__uint_as_float(w4.x), __uint_as_float(w4.y),
                              __uint_as_float(w4.z), __uint_as_float(w4.w)};
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const f32x2_t e = t[m];
                    rope_rotate(f[2 * m], f[2 * m + 1], e.x, e.y);
                }
                w4 = uint4{__float_as_uint(f[0]), __float_as_uint(f[1]),
                           __float_as_uint(f[2]), __float_as_uint(f[3])};
            }
            stream_store<NT>(ptr[u], w4);
        }
    };

    load_batch();
    for (int i = threadIdx.x; i < ROPE_TPB * half; i += 256) {
        const int t = i / half, pair = i - t * half;
        float cv = 1.f, sv = 0.f;
        int tp, hp, wp;
        if (t < ntok && rope_token_pos(r, (row0 + t) % n_tokens, &tp, &hp, &wp))
            rope_cos_sin(r, rope_pair_pos(r, pair, tp, hp, wp), pair, &cv, &sv);
        cs[i] = f32x2_t{cv, sv};
    }
    if (threadIdx.x < ROPE_TPB)
        rotate[threadIdx.x] = (int)threadIdx.x < ntok && ((row0 + threadIdx.x) % n_tokens) >= r.n_prefix;
    __syncthreads();
    rotate_store_batch();
    while (tk < ntok) {
        load_batch();
        rotate_store_batch();
    }
}

// Half-split pairings (halves of each band, or halves of the head when a
// half is not a whole number of chunks).  One wave owns one token: every
// (tensor, head) row of it in Q and K.  The wave first evaluates its token's
// cos/sin for all head_dim/2 pairs into its own LDS area, and each lane keeps
// those of its chunk's elements in registers for every row.  Rows then go
// 64 / (head_dim / EPC) per pass and ROPE_SPLIT_U passes at once: every lane
// loads one 16-byte chunk of each of its U rows (U loads in flight), stages
// the raw chunk in the wave's LDS area, and after a wave-level barrier
// rotates each element with its partner read back from there and stores the
// chunk.  A staged row is padded by one 32-bit word, so the rows of a pass
// start on different banks: the partner reads of a wave then hit each bank
// at most twice for the band splits in use, and the chunk writes never
// conflict.  Only lanes of one wave share an LDS area, so waves never wait
// for each other.  Two passes per batch keep the workgroup's LDS at 14 KiB,
// so eight workgroups (32 waves) fit a CU: more passes per batch cost
// occupancy and measured slower.
constexpr int ROPE_SPLIT_U = 2;
// staging words per pass and wave: rows x (row + 1 padding word) <= 256 + 64
constexpr int ROPE_SPLIT_WORDS = 320;

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool BF16, bool NT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope3d_split_kernel(uint4* q, uint4* k, int64_t rows, int64_t n_tokens, int heads,
                         int head_dim, RopeArgs r) {
    static_assert(ROPE_TPB == 4, "one wave per token of the workgroup");
    constexpr int EPC = BF16 ? 8 : 4;
    constexpr int U = ROPE_SPLIT_U;
    __shared__ f32x2_t cs_all[4][ROPE_MAX_HALF];
    __shared__ uint32_t stage_all[4][U * ROPE_SPLIT_WORDS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * ROPE_TPB + wave;   // this wave's token row
    if (row >= rows) return;
    int tp, hp, wp;
    if (!rope_token_pos(r, row % n_tokens, &tp, &hp, &wp)) return;   // text: not rotated
    const int half = head_dim >> 1;
    f32x2_t* const cs = cs_all[wave];
    for (int j = lane; j < half; j += 64) {
        float c, s;
        rope_cos_sin(r, rope_pair_pos(r, j, tp, hp, wp), j, &c, &s);
        cs[j] = f32x2_t{c, s};
    }
    const int dpr = head_dim / EPC;            // chunks per head row (<= 32)
    const int rpp = 64 / dpr;                  // head rows per pass
    const int slot = lane / dpr, c = lane - slot * dpr;
    // staged row stride in 32-bit words: the row plus one word of padding
    const int rs = (BF16 ? head_dim / 2 : head_dim) + 1;
    int partner[EPC];
    float cr[EPC], sr[EPC];
    uint32_t second = 0;
    wave_sync_lds();
#pragma unroll
    for (int m = 0; m < EPC; ++m) {
        int pair;
        bool sec;
        rope_elem_pair(r, c * EPC + m, &pair, &partner[m], &sec);
        second |= (uint32_t)sec << m;
        const f32x2_t e = cs[pair];
        cr[m] = e.x;
        sr[m] = e.y;
    }
    uint32_t* const stage = stage_all[wave];
    // rows of this token: Q heads 0..H-1, then K heads 0..H-1 (absent tensors skipped)
    const int u_begin = q != nullptr ? 0 : heads, u_end = k != nullptr ? 2 * heads : heads;
    const int64_t dpt = (int64_t)heads * dpr;   // chunks per token row
    for (int u0 = u_begin; u0 < u_end; u0 += U * rpp) {
        uint4 raw[U];
        uint4* ptr[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int u = u0 + i * rpp + slot;
            const bool live = slot < rpp && u < u_end;
            uint4* base = u < heads ? q : k;
            const int h = u < heads ? u : u - heads;
            ptr[i] = live ? base + row * dpt + (int64_t)h * dpr + c : nullptr;
            if (live) raw[i] = stream_load<NT>(ptr[i]);
        }
#pragma unroll
        for (int i = 0; i < U; ++i)
            if (ptr[i] != nullptr) {
                uint32_t* dst = stage + (i * rpp + slot) * rs + c * 4;
                dst[0] = raw[i].x; dst[1] = raw[i].y; dst[2] = raw[i].z; dst[3] = raw[i].w;
            }
        wave_sync_lds();
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (ptr[i] == nullptr) continue;
            const uint32_t* srow = stage + (i * rpp + slot) * rs;
            float f[EPC], out[EPC];
            unpack_chunk<BF16>(u32x4_t{raw[i].x, raw[i].y, raw[i].z, raw[i].w}, f);
#pragma unroll
            for (int m = 0; m < EPC; ++m) {
                float xp;
                if constexpr (BF16)
                    xp = __uint_as_float((uint32_t)((const uint16_t*)srow)[partner[m]] << 16);
                else
                    xp = __uint_as_float(srow[partner[m]]);
                out[m] = rope_rotate_elem(f[m], xp, (second >> m) & 1, cr[m], sr[m]);
            }
            const u32x4_t w = pack_chunk<BF16>(out);
            stream_store<NT>(ptr[i], uint4{w[0], w[1], w[2], w[3]});
        }
        wave_sync_lds();   // this pass's reads are done before the next pass writes
    }
}

// Halves of the head (pairing 1) when head_dim / 2 is a whole number of
// 16-byte chunks: element m of chunk c (c < half the row's chunks) pairs with
// element m of chunk c + dpr / 2, so a thread loads both chunks and rotates
// in registers, with the angle of pair c * EPC + m.  As in the adjacent
// kernel, a thread handles its chunk pairs ROPE_BATCH / 2 at a time with all
// loads of a batch issued first, the first batch before the angles.
template <bool BF16, bool NT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope3d_halves_kernel(uint4* q, uint4* k, int64_t rows, int64_t n_tokens, int heads,
                          int head_dim, RopeArgs r) {
    constexpr int EPC = BF16 ? 8 : 4;
    constexpr int U = ROPE_BATCH / 2;    // chunk pairs per batch: ROPE_BATCH loads in flight
    __shared__ f32x2_t cs[ROPE_TPB * ROPE_MAX_HALF];
    __shared__ int rotate[ROPE_TPB];
    const int half = head_dim >> 1;
    const int64_t row0 = (int64_t)blockIdx.x * ROPE_TPB;
    const int ntok = (int)(rows - row0 < ROPE_TPB ? rows - row0 : ROPE_TPB);   // >= 1
    const int dpr = head_dim / EPC, hc = dpr / 2;   // chunks per head row, and per half
    const int per_token = heads * hc;                // chunk pairs per token row and tensor
    uint4* const ten0 = q != nullptr ? q : k;
    uint4* const ten1 = q != nullptr ? k : nullptr;
    const int nten = ten1 != nullptr ? 2 : 1;
    const int items = ntok * nten * per_token;
    // items (token, tensor, head, chunk pair) with the chunk pair fastest;
    // this thread's are threadIdx.x + 256 j, handled U at a time, loads first
    int u = threadIdx.x;
    uint4 v0[U], v1[U];
    uint4* ptr[U];
    int slot[U];                          // tk * half + first pair of the chunk; -1: none
    auto load_batch = [&]() {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            slot[j] = -1;
            if (u < items) {
                const int tw = u / per_token, rem = u - tw * per_token;
                const int tk = tw / nten, which = tw - tk * nten;
                const int h = rem / hc, c = rem - h * hc;
                ptr[j] = (which ? ten1 : ten0) + ((row0 + tk) * heads + h) * dpr + c;
                v0[j] = stream_load<NT>(ptr[j]);
                v1[j] = stream_load<NT>(ptr[j] + hc);
                slot[j] = tk * half + c * EPC;
            }
            u += 256;
        }
    };
    auto rotate_store_batch = [&]() {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if (slot[j] < 0 || !rotate[slot[j] / half]) continue;
            float f0[EPC], f1[EPC];
            unpack_chunk<BF16>(u32x4_t{v0[j].x, v0[j].y, v0[j].z, v0[j].w}, f0);
            unpack_chunk<BF16>(u32x4_t{v1[j].x, v1[j].y, v1[j].z, v1[j].w}, f1);
            const f32x2_t* t = cs + slot[j];
#pragma unroll
            for (int m = 0; m < EPC; ++m) {
                const f32x2_t e = t[m];
                rope_rotate(f0[m], f1[m], e.x, e.y);
            }
            const u32x4_t w0 = pack_chunk<BF16>(f0), w1 = pack_chunk<BF16>(f1);
            stream_store<NT>(ptr[j], uint4{w0[0], w0[1], w0[2], w0[3]});
            stream_store<NT>(ptr[j] + hc, uint4{w1[0], w1[1], w1[2], w1[3]});
        }
    };

    load_batch();
    for (int i = threadIdx.x; i < ROPE_TPB * half; i += 256) {
        const int t = i / half, pair = i - t * half;
        float cv = 1.f, sv = 0.f;
        int tp, hp, wp;
        if (t < ntok && rope_token_pos(r, (row0 + t) % n_tokens, &tp, &hp, &wp))
            rope_cos_sin(r, rope_pair_pos(r, pair, tp, hp, wp), pair, &cv, &sv);
        cs[i] = f32x2_t{cv, sv};
    }
    if (threadIdx.x < ROPE_TPB)
        rotate[threadIdx.x] = (int)threadIdx.x < ntok && ((row0 + threadIdx.x) % n_tokens) >= r.n_prefix;
    __syncthreads();
    rotate_store_batch();
    while (u < items) {
        load_batch();
        rotate_store_batch();
    }
}

// One launch of the kernel `kind` selects: 1 head halves, 2 band halves,
// 8 or 4 adjacent pairs with that many loads in flight per thread.
template <bool BF16, bool NT>
hipError_t launch_rope_kind(int kind, dim3 grid, hipStream_t st, uint4* q, uint4* k, int64_t rows,
                            int64_t n_tokens, int heads, int head_dim, const RopeArgs& r) {
    const dim3 block(256);
    if (kind == 1)
        hipLaunchKernelGGL((rope3d_halves_kernel<BF16, NT>), grid, block, 0, st, q, k, rows,
                           n_tokens, heads, head_dim, r);
    else if (kind == 2)
        hipLaunchKernelGGL((rope3d_split_kernel<BF16, NT>), grid, block, 0, st, q, k, rows,
                           n_tokens, heads, head_dim, r);
    else if (kind == 8)
        hipLaunchKernelGGL((rope3d_kernel<BF16, 8, NT>), grid, block, 0, st, q, k, rows, n_tokens,
                           heads, head_dim, r);
    else
        hipLaunchKernelGGL((rope3d_kernel<BF16, 4, NT>), grid, block, 0, st, q, k, rows, n_tokens,
                           heads, head_dim, r);
    return hipGetLastError();
}

hipError_t launch_rope3d(void* q, void* k, int64_t batch, int64_t n_tokens, int64_t heads,
                         int64_t head_dim, const RopeArgs& r, bool bf16, hipStream_t st) {
    const int64_t rows = batch * n_tokens;
    const dim3 grid((unsigned)((rows + ROPE_TPB - 1) / ROPE_TPB));
    const int epc = bf16 ? 8 : 4;
    const int ntens = (q != nullptr) + (k != nullptr);
    int kind;
    if (r.pairing == 1 && (head_dim / 2) % epc == 0) {
        kind = 1;
    } else if (r.pairing != 0) {
        kind = 2;
    } else {
        // chunks per thread in a full workgroup: ROPE_TPB tokens x tensors x chunks per row
        kind = ROPE_TPB * ntens * heads * (head_dim / epc) / 256 >= 8 ? 8 : 4;
    }
    // bytes of the rotated tensors; one tensor's count fits int64 (checked by
    // the host), so compare per tensor rather than multiply by ntens
    const bool nt = rows * heads * head_dim * (bf16 ? 2 : 4) > ROPE_NT_BYTES / ntens;
    uint4 *qq = (uint4*)q, *kk = (uint4*)k;
    const int h = (int)heads, d = (int)head_dim;
    if (bf16)
        return nt ? launch_rope_kind<true, true>(kind, grid, st, qq, kk, rows, n_tokens, h, d, r)
                  : launch_rope_kind<true, false>(kind, grid, st, qq, kk, rows, n_tokens, h, d, r);
    return nt ? launch_rope_kind<false, true>(kind, grid, st, qq, kk, rows, n_tokens, h, d, r)
              : launch_rope_kind<false, false>(kind, grid, st, qq, kk, rows, n_tokens, h, d, r);
}

}  // namespace vx
