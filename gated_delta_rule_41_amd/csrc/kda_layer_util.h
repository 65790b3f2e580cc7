// The layer prologue's arithmetic, shared by its own kernel and by the chunk
// preparation kernel's fused variant (which runs it into LDS): short causal
// depthwise convolution (width 4) and Swish on q, k, v, L2 normalisation of q
// and k, the decay gate and beta, as in the GeekNews "Kimi Linear" summary,
// section "Configuração do modelo Kimi Linear". One wave computes G
// consecutive tokens of one head; lane j holds the channel pair 2j, 2j + 1
// (d = 128; channel j for d = 64).
#pragma once
#include "kda_common.h"

namespace kda {

constexpr int CONV_W = 4;
constexpr float LAYER_EPS = 1e-6f;

// Sum over the 64 lanes, the same in every lane: DPP swaps within each row of
// 16 lanes (xor 1, xor 2, then the half-row and row mirrors, which pair every
// lane with one holding the other partial sum), then the four row sums read out
// in a fixed order. No LDS traffic; deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float x) {
    x = dpp_add<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x = dpp_add<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x = dpp_add<0x141>(x);  // row_half_mirror
    x = dpp_add<0x140>(x);  // row_mirror
    const int u = __float_as_int(x);
    return (__int_as_float(__builtin_amdgcn_readlane(u, 0)) + __int_as_float(__builtin_amdgcn_readlane(u, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(u, 32)) + __int_as_float(__builtin_amdgcn_readlane(u, 48)));
}
// Transcendentals on the hardware units (v_exp_f32, v_log_f32, v_rcp_f32, each
// within about an ulp): the library's range-reduced exp, IEEE division and
// log1p would cost several times the instructions of the whole kernel's loads.
constexpr float L_LOG2E = 1.4426950408889634f, L_LN2 = 0.6931471805599453f;
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// 1 / (1 + e^-x); saturates to 0 and 1 (e^-x overflows to inf or underflows to 0)
__device__ __forceinline__ float sigm(float x) { return rcp(1.f + __builtin_amdgcn_exp2f(-x * L_LOG2E)); }
// log(1 + e^x) = max(x, 0) + log1p(e^-|x|). log1p(e) for e in (0, 1] by the
// identity log1p(e) = log(u) e / (u - 1), u = 1 + e rounded (exact when u = 1),
// which cancels the rounding of u to a few ulps (Goldberg, "What every computer
// scientist should know about floating-point arithmetic", theorem 4).
__device__ __forceinline__ float softplus_f(float x) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * L_LOG2E), u = 1.f + e;
    const float lp = u == 1.f ? e : __builtin_amdgcn_logf(u) * L_LN2 * e * rcp(u - 1.f);
    return fmaxf(x, 0.f) + lp;
}

template <typename T>
__device__ __forceinline__ void st_out(T* p, int64_t i, float x);
template <> __device__ __forceinline__ void st_out<float>(float* p, int64_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void st_out<uint16_t>(uint16_t* p, int64_t i, float x) { p[i] = f2bf(x); }

template <typename TE, int PER>
struct Pair;  // PER consecutive channels of one row, loaded and stored together
template <>
struct Pair<uint16_t, 2> {
    static __device__ __forceinline__ void ld(const uint16_t* p, float (&x)[2]) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xffff0000u);
    }
    static __device__ __forceinline__ void st(uint16_t* p, const float (&x)[2]) {
        *reinterpret_cast<uint32_t*>(p) = pack2bf(x[0], x[1]);
    }
};
template <>
struct Pair<float, 2> {
    static __device__ __forceinline__ void ld(const float* p, float (&x)[2]) {
        const float2 u = *reinterpret_cast<const float2*>(p);
        x[0] = u.x;
        x[1] = u.y;
    }
    static __device__ __forceinline__ void st(float* p, const float (&x)[2]) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    }
};
template <typename TE>
struct Pair<TE, 1> {
    static __device__ __forceinline__ void ld(const TE* p, float (&x)[1]) { x[0] = ld_in(p, 0); }
    static __device__ __forceinline__ void st(TE* p, const float (&x)[1]) { st_out(p, 0, x[0]); }
};

// The epilogue of one (token, head) row, held as lane j holding channels
// PER j .. PER j + PER - 1 (PER = D / 64): y = x / sqrt(mean x^2 + eps) * w *
// sigmoid(xg). Every lane of the wave takes part (the mean is a wave sum).
template <int D, typename TE>
__device__ __forceinline__ void epilogue_row(const float (&x)[D / 64], const float (&xg)[D / 64],
                                             const float (&wc)[D / 64], TE* y) {
    constexpr int PER = D / 64;
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p) s += x[p] * x[p];
    const float r = rsqrtf(wave_sum(s) * (1.f / D) + LAYER_EPS);
    float out[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) out[p] = x[p] * r * wc[p] * sigm(xg[p]);
    Pair<TE, PER>::st(y, out);
}

template <int D>
struct ConvFilters {
    static constexpr int PER = D / 64;
    float fw[3][PER][CONV_W], db[PER], scale;
    __device__ __forceinline__ void load(const float* wq, const float* wk, const float* wv, const float* A_log,
                                         const float* dt_bias, int h, int c0) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
#pragma unroll
            for (int i = 0; i < CONV_W; ++i) {
                const int64_t wi = ((int64_t)h * D + c0 + p) * CONV_W + i;
                fw[0][p][i] = wq[wi];
                fw[1][p][i] = wk[wi];
                fw[2][p][i] = wv[wi];
            }
            db[p] = dt_bias[h * D + c0 + p];
        }
        scale = __expf(A_log[h]);
    }
};

template <typename TE>
struct PrologueIn {
    const TE *xq, *xk, *xv, *xa, *xb;
};

// The loads of G tokens t0 .. t0 + G - 1 of head h: the convolution window
// (rows t0 - 3 .. t0 + G - 1 of xq, xk, xv), the gate rows and, in lane j < G,
// token t0 + j's beta input. Row indices are clamped into [0, T), so no load
// sits behind a branch; the caller masks what it must not use.
template <int D, int G, typename TE>
struct PrologueWindow {
    static constexpr int PER = D / 64, W = CONV_W - 1 + G;
    float win[3][W][PER], xg[G][PER], xbl;
    __device__ __forceinline__ void load(const PrologueIn<TE>& in, int h, int t0, int T, int H, int c0, int l) {
        using PR = Pair<TE, PER>;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int s = min(max(t0 - (CONV_W - 1) + i, 0), T - 1);
            const int64_t ro = ((int64_t)s * H + h) * D + c0;
            PR::ld(in.xq + ro, win[0][i]);
            PR::ld(in.xk + ro, win[1][i]);
            PR::ld(in.xv + ro, win[2][i]);
        }
#pragma unroll
        for (int j = 0; j < G; ++j) PR::ld(in.xa + ((int64_t)min(t0 + j, T - 1) * H + h) * D + c0, xg[j]);
        xbl = ld_in(in.xb, (int64_t)min(t0 + (l & (G - 1)), T - 1) * H + h);
    }
    // Token t0 + j (its sequence starting at token fst): the four outputs'
    // PER channels.
    __device__ __forceinline__ void token(const ConvFilters<D>& f, int j, int t, int fst, float (&oq)[PER],
                                          float (&ok)[PER], float (&ov)[PER], float (&og)[PER]) const {
        float y[3][PER];
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < CONV_W; ++i)
                    if (t - (CONV_W - 1) + i >= fst) acc += f.fw[m][p][i] * win[m][j + i][p];
                y[m][p] = acc * sigm(acc);  // swish
            }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            sq += y[0][p] * y[0][p];
            sk += y[1][p] * y[1][p];
        }
        const float nq = rsqrtf(wave_sum(sq) + LAYER_EPS), nk = rsqrtf(wave_sum(sk) + LAYER_EPS);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            oq[p] = y[0][p] * nq;
            ok[p] = y[1][p] * nk;
            ov[p] = y[2][p];
            og[p] = -f.scale * softplus_f(xg[j][p] + f.db[p]);
        }
    }
    // Tokens t0 + j < tend, in order: first(t) is the first token of t's
    // sequence (taps before it read zeros); sink(j, q, k, v, log_alpha) takes
    // each token's PER channels. Returns beta of token t0 + (lane & (G - 1)).
    template <typename First, typename Sink>
    __device__ __forceinline__ float compute(const ConvFilters<D>& f, int t0, int tend, First&& first,
                                             Sink&& sink) const {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int t = t0 + j;
            if (t >= tend) break;
            float oq[PER], ok[PER], ov[PER], og[PER];
            token(f, j, t, first(t), oq, ok, ov, og);
            sink(j, oq, ok, ov, og);
        }
        return sigm(xbl);
    }
    // The same for all G tokens with no branch between them, so that their
    // dependency chains interleave: fst[j] is token t0 + j's first token, every
    // token is computed (rows past the end were clamped on load) and the sink
    // decides what to store.
    template <typename Sink>
    __device__ __forceinline__ float compute_all(const ConvFilters<D>& f, int t0, const int (&fst)[G],
                                                 Sink&& sink) const {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float oq[PER], ok[PER], ov[PER], og[PER];
            token(f, j, t0 + j, fst[j], oq, ok, ov, og);
            sink(j, oq, ok, ov, og);
        }
        return sigm(xbl);
    }
};

}  // namespace kda
