// Helpers shared by the per-chunk preparation kernels (KDA and the general
// DPLR transition): block-local gate scans, split-order positions, row loads.
#pragma once

#include "kda_common.h"

namespace kda {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LOG2E_LO = 1.925963033500011e-08f;  // log2(e) - LOG2E

// Error-free transformations (Knuth's TwoSum; the product residual by FMA),
// written with explicitly rounded operations so that no step is contracted.
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
    s = __fadd_rn(a, b);
    const float bb = __fsub_rn(s, a);
    e = __fadd_rn(__fsub_rn(a, __fsub_rn(s, bb)), __fsub_rn(b, bb));
}
// x log2(e) as hi + lo with hi = fl(x LOG2E), to about 2^-48 relative
__device__ __forceinline__ void log2_units(float x, float& hi, float& lo) {
    hi = __fmul_rn(x, LOG2E);
    lo = __fadd_rn(__builtin_fmaf(x, LOG2E, -hi), __fmul_rn(x, LOG2E_LO));
}
constexpr float GUARD = 100.0f;  // max gate range inside a 16-row sub-chunk, log2 units

__device__ __forceinline__ float dpp_shr(float x, int d) {
    const int xi = __float_as_int(x);
    int r;
    switch (d) {
        case 1: r = __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xF, 0xF, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xF, 0xF, false); break;
        case 4: r = __builtin_amdgcn_update_dpp(0, xi, 0x114, 0xF, 0xF, false); break;
        default: r = __builtin_amdgcn_update_dpp(0, xi, 0x118, 0xF, 0xF, false); break;
    }
    return __int_as_float(r);
}

// position of chunk row r inside its 32-row slice, in the split k order
__device__ __forceinline__ int split_pos(int r) {
    const int rr = r & 31;
    return 8 * ((rr & 15) >> 2) + 4 * (rr >> 4) + (rr & 3);
}

__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32

// One lane's share of an input row (channels 32 s + split(g, j), j < 8, of each
// 32-channel slice s), held raw (unconverted) so that the loads of every
// input can be issued before the first one is waited for.
template <typename T, int NS>
struct RowRaw {
    static constexpr int W = sizeof(T) == 2 ? 2 : 4;  // dwords per 4 elements
    uint32_t d[NS][2][W];
    __device__ __forceinline__ void load(const T* p, int64_t off, int g) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const T* src = p + off + 32 * s + 16 * hf + 4 * g;
                if constexpr (W == 2) {
                    const u32x2_t u = *reinterpret_cast<const u32x2_t*>(src);
                    d[s][hf][0] = u[0];
                    d[s][hf][1] = u[1];
                } else {
                    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
                    for (int j = 0; j < 4; ++j) d[s][hf][j] = u[j];
                }
            }
    }
    __device__ __forceinline__ void get(float (&x)[NS][8], bool valid, float scale) const {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float f;
                    if constexpr (W == 2)
                        f = __uint_as_float((j & 1) ? (d[s][hf][j >> 1] & 0xffff0000u) : (d[s][hf][j >> 1] << 16));
                    else
                        f = __uint_as_float(d[s][hf][j]);
                    x[s][4 * hf + j] = valid ? f * scale : 0.f;
                }
    }
    // element jj (= 4 hf + j, the order get() uses) of slice s, zero when !valid
    __device__ __forceinline__ float at(int s, int jj, bool valid) const {
        float f;
        if constexpr (W == 2) {
            const uint32_t u = d[s][jj >> 2][(jj & 3) >> 1];
            f = __uint_as_float((jj & 1) ? (u & 0xffff0000u) : (u << 16));
        } else {
            f = __uint_as_float(d[s][jj >> 2][jj & 3]);
        }
        return valid ? f : 0.f;
    }
};

}  // namespace kda
