// Measurement aid, not part of the hot path: the bf16 MFMA rate this chip
// sustains on given operand data.
//
// MI355X's 2.5 PFLOP/s bf16 figure is its full clock times 4096 flops per
// CU per cycle.  Under a dense MFMA load the chip lowers its clock to stay
// within its power limit, and the power depends on the data multiplied:
// bits that toggle cost energy.  This kernel issues nothing but
// v_mfma_f32_32x32x16_bf16, on operand fragments loaded once into
// registers, so that timing it on the attention workload's own kind of data
// (N(0,1) bf16) gives the MFMA ceiling that data allows.
//
// Layout: workgroup g, wave w (8 waves, two per SIMD) reads 16 fragments of
// 64 lanes x 16 bytes from operands + ((g * 8 + w) * 16) * 1024 bytes:
// fragments 0-7 are A operands, 8-15 B operands.  Each of `iters`
// iterations issues 8 MFMAs, MFMA i taking A fragment i and B fragment
// (3i + 1) mod 8 into accumulator i mod 4, so both operands change from one
// instruction to the next, as the attention kernel's do.  Lane l of the
// wave writes the sum of its 64 accumulator values to out[g * 512 + w * 64 + l].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int WAVES = 8;

__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(2, 2)))
void mfma_bf16_loop(const uint4* __restrict__ operands, float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint4* src = operands + ((size_t)blockIdx.x * WAVES + wave) * 16 * 64;
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_bit_cast(bf16x8_t, src[i * 64 + lane]);
        b[i] = __builtin_bit_cast(bf16x8_t, src[(8 + i) * 64 + lane]);
    }
    f32x16_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(3 * i + 1) & 7],
                                                                 acc[i & 3], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * 64 * WAVES + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Enqueue one launch of `workgroups` x 8 waves, each issuing 8 * iters MFMAs
// (32,768 flops each).  operands: device, 16-byte aligned, workgroups * 128
// KiB of bf16 (see the layout above); out: device, workgroups * 512 floats.
// Returns 0, 1 for a NULL or misaligned pointer, 2 for sizes out of range,
// 5 when the launch fails.  Nothing is allocated or synchronised.
int vx_diag_mfma_bf16_loop(const void* operands, float* out, int workgroups, int iters,
                           void* hip_stream) {
    if (!operands || !out || (reinterpret_cast<uintptr_t>(operands) & 15u) ||
        (reinterpret_cast<uintptr_t>(out) & 3u))
        return 1;
    if (workgroups <= 0 || workgroups > (1 << 20) || iters < 0) return 2;
    hipLaunchKernelGGL(mfma_bf16_loop, dim3(workgroups), dim3(64 * WAVES), 0,
                       (hipStream_t)hip_stream, (const uint4*)operands, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

// flops of one launch
double vx_diag_mfma_bf16_loop_flops(int workgroups, int iters) {
    return (double)workgroups * WAVES * 8.0 * iters * 32.0 * 32.0 * 16.0 * 2.0;
}

}  // extern "C"
