// Merge of two partial attention results by their log-sum-exp.
//
// If the keys of one attention are split into two disjoint sets A and B and
// attention is taken over each, (o_A, lse_A) and (o_B, lse_B), the
// attention over A u B follows from them alone:
//
//   lse = log(exp(lse_A) + exp(lse_B))
//   o   = exp(lse_A - lse) o_A + exp(lse_B - lse) o_B
//
// since each o is its softmax-weighted mean and exp(lse) its softmax
// denominator.  This is how attention over a sequence whose keys live on
// several GPUs (or in several passes) is put back together; the vidax
// paper (arXiv 2609.18077) §2 "Spatiotemporal tensor and sequence
// sharding" shards the token axis across devices, which makes such a merge
// the step after any key-sharded attention.  The operation is associative,
// so P parts merge pairwise.
//
// HBM-bound: o_A and o_B are read once and o written once; the LSE vectors
// are small (one float per (token, head)).  One thread per 16-byte chunk of
// o; the head_dim / EPC threads of one (token, head) are consecutive and lie
// in one wave, so every lane reads both LSEs before any lane writes the
// merged one, which keeps lse == lse_A (or lse_B) in place safe.
#include "vx_device.h"

namespace vx {

template <bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_merge_kernel(const u32x4_t* oa, const float* lsea, const u32x4_t* ob, const float* lseb,
                       u32x4_t* o, float* lse, int64_t chunks, int64_t n, int heads,
                       int chunks_per_head) {
    constexpr int EPC = BF16 ? 8 : 4;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int part = (int)(c % chunks_per_head);
    const int64_t th = c / chunks_per_head;          // (b * n + token) * heads + h
    const int h = (int)(th % heads);
    const int64_t bt = th / heads;                   // b * n + token
    const int64_t b = bt / n, tok = bt % n;
    const int64_t li = (b * heads + h) * n + tok;    // lse is [batch, heads, n]
    const float la = lsea[li], lb = lseb[li];
    const float m = fmaxf(la, lb);
    float wa, wb, l;
    if (m == -__builtin_inff()) {   // both parts empty: no weight anywhere
        wa = wb = 0.f;
        l = m;
    } else {
        const float ea = expf(la - m), eb = expf(lb - m);
        const float inv = 1.0f / (ea + eb);
        wa = ea * inv;
        wb = eb * inv;
        l = m + logf(ea + eb);
    }
    float fa[EPC], fb[EPC], out[EPC];
    const u32x4_t va = oa[c], vb = ob[c];
    unpack_chunk<BF16>(va, fa);
    unpack_chunk<BF16>(vb, fb);
#pragma unroll
    for (int e = 0; e < EPC; ++e) out[e] = __builtin_fmaf(wa, fa[e], wb * fb[e]);
    o[c] = pack_chunk<BF16>(out);
    if (lse != nullptr && part == 0) lse[li] = l;
}

hipError_t launch_attn_merge(const void* oa, const float* lsea, const void* ob, const float* lseb,
                             void* o, float* lse, int64_t batch, int64_t n, int64_t heads,
                             int64_t head_dim, bool bf16, hipStream_t st) {
    const int epc = bf16 ? 8 : 4;
    const int cph = (int)(head_dim / epc);
    const int64_t chunks = batch * n * heads * cph;
    const int64_t blocks = (chunks + 255) / 256;
    if (bf16)
        hipLaunchKernelGGL(attn_merge_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const u32x4_t*)oa, lsea, (const u32x4_t*)ob, lseb, (u32x4_t*)o, lse,
                           chunks, n, (int)heads, cph);
    else
        hipLaunchKernelGGL(attn_merge_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const u32x4_t*)oa, lsea, (const u32x4_t*)ob, lseb, (u32x4_t*)o, lse,
                           chunks, n, (int)heads, cph);
    return hipGetLastError();
}

}  // namespace vx
