// Machine probes for the benchmark's reference peaks on this GPU (not part of
// the operator): a bf16 matrix-core loop for the achievable dense MFMA rate,
// and a streaming copy for the achievable HBM rate. Both are enqueued on the
// caller's stream; the caller times them.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Each wave runs CHAINS independent accumulators through `iters` rounds of
// v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 x 2 = 16,384 flops each), then writes
// one sum per wave so nothing is dead code.
constexpr int CHAINS = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_bf16_loop(int iters, float* __restrict__ sink) {
    const uint32_t l = threadIdx.x;
    u32x4_t ra, rb;
    for (int j = 0; j < 4; ++j) {
        ra[j] = 0x3F803F80u ^ ((l * 2654435761u + j) & 0x007F007Fu);  // values near 1, lane-dependent
        rb[j] = 0x3F803F80u ^ ((l * 40503u + 7u * j) & 0x007F007Fu);
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ra), b = __builtin_bit_cast(bf16x8_t, rb);
    // (eight named accumulators: an array of them is reshuffled between iterations)
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
        c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
        c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
        c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
    }
    const f32x4_t t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    const float s = (t[0] + t[1]) + (t[2] + t[3]);
    if ((l & 63) == 0) sink[blockIdx.x * (blockDim.x / 64) + (l >> 6)] = s;
}

// 16-byte nontemporal loads and stores: each workgroup pass moves 16 KiB (four
// 4 KiB pieces, every load issued before the first store)
__global__ __launch_bounds__(256) void copy16(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                              size_t n16) {
    const size_t stride = (size_t)gridDim.x * 1024;
    for (size_t base = (size_t)blockIdx.x * 1024 + threadIdx.x; base < n16; base += stride) {
        u32x4_t x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (base + 256 * j < n16) x[j] = __builtin_nontemporal_load(src + base + 256 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (base + 256 * j < n16) __builtin_nontemporal_store(x[j], dst + base + 256 * j);
    }
}

extern "C" {

// flops the probe performs: n_wg workgroups x 4 waves x iters x CHAINS x 16,384
double kda_probe_mfma_bf16_flops(int32_t n_wg, int32_t iters) {
    return (double)n_wg * 4.0 * (double)iters * CHAINS * 16384.0;
}

// sink: device buffer of at least n_wg * 4 floats. Returns 0, or 1 on bad sizes, 2 on a launch error.
int32_t kda_probe_mfma_bf16(int32_t n_wg, int32_t iters, float* sink, void* stream) {
    if (n_wg <= 0 || iters <= 0 || !sink) return 1;
    hipLaunchKernelGGL(mfma_bf16_loop, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// dst <- src, bytes a multiple of 16, both 16-byte aligned and not overlapping.
// Returns 0, or 1 on bad arguments, 2 on a launch error.
int32_t kda_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
    if (!src || !dst || (bytes & 15u) || (((uintptr_t)src | (uintptr_t)dst) & 15u)) return 1;
    const size_t n16 = bytes / 16;
    const size_t wg = (n16 + 1023) / 1024;
    const unsigned grid = (unsigned)(wg < 65536 ? (wg ? wg : 1) : 65536);
    hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
