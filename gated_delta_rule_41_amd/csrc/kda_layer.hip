// The KDA layer's prologue and epilogue around the operator.
//
// The GeekNews "Kimi Linear" summary, section "Configuração do modelo Kimi
// Linear", places the operator between a short convolution with Swish on the
// query, key and value (then L2 normalisation of the query and key, and a
// per-channel decay gate through a GDN/Mamba-like decay function) and, before
// the output projection, a per-head RMSNorm and a data-dependent output gate.
// Starting from the projections' outputs (pre-activations):
//
//   prologue:  q = L2(swish(conv(xq))), k = L2(swish(conv(xk))), v = swish(conv(xv)),
//              log_alpha = -exp(A_log[h]) softplus(xa + dt_bias[h, c]), beta = sigmoid(xb)
//   epilogue:  y = o / sqrt(mean(o^2) + eps) * w * sigmoid(xg)
//
// conv is causal and depthwise, width 4, with zero history before each
// sequence's first token; L2(x) = x / sqrt(sum x^2 + eps); eps = 1e-6.
//
// The L2 and RMS sums over a head's channels are wave reductions (a fixed
// butterfly: the results are deterministic). Both kernels stream their bytes
// once and are bound by HBM.
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_layer_util.h"

namespace kda {

// Prologue: a block of four waves covers 32 consecutive tokens of one head,
// each wave eight of them (G), with every load issued before the first wait.
// Eight rather than four: more bytes in flight per wave (91 VGPRs at d = 128
// with bf16, five waves per SIMD) and fewer halo rows per token.
constexpr int G = 8;       // tokens per wave
constexpr int PT = 4 * G;  // tokens per block

template <int D, typename TE>
__global__ __launch_bounds__(256) void layer_prologue_kernel(PrologueIn<TE> in, const float* __restrict__ wq,
                                                             const float* __restrict__ wk, const float* __restrict__ wv,
                                                             const float* __restrict__ A_log,
                                                             const float* __restrict__ dt_bias,
                                                             const int32_t* __restrict__ cu, int N, int T, int H,
                                                             TE* __restrict__ q, TE* __restrict__ k,
                                                             TE* __restrict__ v, TE* __restrict__ la,
                                                             TE* __restrict__ beta) {
    constexpr int PER = D / 64;
    using PR = Pair<TE, PER>;
    const int h = blockIdx.x % H;
    // this wave's first token, stated uniform so that the sequence search below
    // runs on scalar loads (beside the window's vector loads, not behind them)
    const int t0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / H) * PT + (int)(threadIdx.x >> 6) * G);
    if (t0 >= T) return;
    const int l = threadIdx.x & 63, c0 = PER * l;
    PrologueWindow<D, G, TE> win;
    win.load(in, h, t0, T, H, c0, l);
    ConvFilters<D> f;
    f.load(wq, wk, wv, A_log, dt_bias, h, c0);
    // the sequence holding t0 (cu_seqlens sorted; NULL = one sequence), then
    // walk forward across boundaries
    int n = 0, first = 0, next = INT_MAX;
    if (cu != nullptr) {
        int hi = N;
        while (hi - n > 1) {
            const int mid = (n + hi) >> 1;
            if (cu[mid] <= t0) n = mid; else hi = mid;
        }
        first = cu[n];
        next = cu[n + 1];
    }
    auto seq_first = [&](int t) {
        while (n + 1 < N && t >= next) {  // empty sequences end where they start
            first = next;
            ++n;
            next = cu[n + 1];
        }
        return first;
    };
    int fst[G];
#pragma unroll
    for (int j = 0; j < G; ++j) fst[j] = seq_first(t0 + j);
    const float bl = win.compute_all(f, t0, fst, [&](int j, const float (&oq)[PER], const float (&ok)[PER],
                                                    const float (&ov)[PER], const float (&og)[PER]) {
        if (t0 + j >= T) return;
        const int64_t ro = ((int64_t)(t0 + j) * H + h) * D + c0;
        PR::st(q + ro, oq);
        PR::st(k + ro, ok);
        PR::st(v + ro, ov);
        PR::st(la + ro, og);
    });
    if (l < G && t0 + l < T) st_out(beta, (int64_t)(t0 + l) * H + h, bl);
}

// Epilogue: each wave takes G consecutive (token, head) rows and issues all of
// their loads at once (rows clamped into range); lane j holds the channel pair
// 2j, 2j + 1 (d = 128; channel j for d = 64).
template <int D, typename TE>
__global__ __launch_bounds__(256) void layer_epilogue_kernel(const float* __restrict__ o, const TE* __restrict__ g,
                                                             const float* __restrict__ w, int TH,
                                                             TE* __restrict__ y) {
    constexpr int PER = D / 64;
    const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * G;
    if (r0 >= TH) return;  // uniform over the wave
    const int c0 = PER * (threadIdx.x & 63);
    float x[G][PER], xg[G][PER], wc[PER];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int64_t ro = (int64_t)min(r0 + j, TH - 1) * D + c0;
        Pair<float, PER>::ld(o + ro, x[j]);
        Pair<TE, PER>::ld(g + ro, xg[j]);
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) wc[p] = w[c0 + p];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (r0 + j >= TH) break;
        epilogue_row<D, TE>(x[j], xg[j], wc, y + (int64_t)(r0 + j) * D + c0);
    }
}

// The convolution's history after each sequence, for one-token decoding: the
// last three rows of xq, xk, xv (oldest first, zero where the sequence is
// shorter), [N][H][q, k, v][3][D]. One wave per (sequence, head).
template <int D, typename TE>
__global__ __launch_bounds__(256) void layer_conv_state_kernel(PrologueIn<TE> in, const int32_t* __restrict__ cu,
                                                               int N, int T, int H, TE* __restrict__ cs) {
    constexpr int PER = D / 64;
    using PR = Pair<TE, PER>;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= N * H) return;  // uniform over the wave
    const int n = item / H, h = item - n * H, c0 = PER * (threadIdx.x & 63);
    // (offsets clamped into [0, T]: a malformed cu_seqlens reads no row outside the inputs)
    int start = cu != nullptr ? cu[n] : 0, end = cu != nullptr ? cu[n + 1] : T;
    start = min(max(start, 0), T);
    end = min(max(end, start), T);
    const TE* xs[3] = {in.xq, in.xk, in.xv};
    TE* dst = cs + (int64_t)item * 3 * (CONV_W - 1) * D + c0;
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int i = 0; i < CONV_W - 1; ++i) {
            const int t = end - (CONV_W - 1) + i;
            float x[PER] = {};
            if (t >= start) PR::ld(xs[m] + ((int64_t)t * H + h) * D + c0, x);
            PR::st(dst + (m * (CONV_W - 1) + i) * D, x);
        }
}

// One token per sequence after the history cs: the same prologue arithmetic,
// the window being the history's three rows and the new one; the history is
// then shifted by the new row in place. One wave per (sequence, head).
template <int D, typename TE>
__global__ __launch_bounds__(256) void layer_decode_prologue_kernel(
    PrologueIn<TE> in, TE* __restrict__ cs, const float* __restrict__ wq, const float* __restrict__ wk,
    const float* __restrict__ wv, const float* __restrict__ A_log, const float* __restrict__ dt_bias, int NH, int H,
    TE* __restrict__ q, TE* __restrict__ k, TE* __restrict__ v, TE* __restrict__ la, TE* __restrict__ beta) {
    constexpr int PER = D / 64;
    using PR = Pair<TE, PER>;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= NH) return;  // uniform over the wave
    const int h = item % H, l = threadIdx.x & 63, c0 = PER * l;
    TE* hist = cs + (int64_t)item * 3 * (CONV_W - 1) * D + c0;
    const int64_t ro = (int64_t)item * D + c0;
    PrologueWindow<D, 1, TE> pw;
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int i = 0; i < CONV_W - 1; ++i) PR::ld(hist + (m * (CONV_W - 1) + i) * D, pw.win[m][i]);
    PR::ld(in.xq + ro, pw.win[0][CONV_W - 1]);
    PR::ld(in.xk + ro, pw.win[1][CONV_W - 1]);
    PR::ld(in.xv + ro, pw.win[2][CONV_W - 1]);
    PR::ld(in.xa + ro, pw.xg[0]);
    pw.xbl = ld_in(in.xb, item);
    ConvFilters<D> f;
    f.load(wq, wk, wv, A_log, dt_bias, h, c0);
    const float bl = pw.compute(f, 0, 1, [](int) { return INT_MIN; },  // every tap reads the window
                                [&](int, const float (&oq)[PER], const float (&ok)[PER], const float (&ov)[PER],
                                    const float (&og)[PER]) {
                                    PR::st(q + ro, oq);
                                    PR::st(k + ro, ok);
                                    PR::st(v + ro, ov);
                                    PR::st(la + ro, og);
                                });
    if (l == 0) st_out(beta, item, bl);
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int i = 0; i < CONV_W - 1; ++i) PR::st(hist + (m * (CONV_W - 1) + i) * D, pw.win[m][i + 1]);
}

template <int D, typename TE>
static hipError_t launch_conv_state_t(const LayerArgs& a, hipStream_t st) {
    const int64_t items = (int64_t)a.N * a.H;
    const PrologueIn<TE> in{(const TE*)a.xq, (const TE*)a.xk, (const TE*)a.xv, nullptr, nullptr};
    hipLaunchKernelGGL((layer_conv_state_kernel<D, TE>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, in,
                       a.cu, a.N, a.T, a.H, (TE*)a.cs);
    return hipGetLastError();
}

hipError_t launch_layer_conv_state(const LayerArgs& a, hipStream_t st) {
    if (a.D == 128) return a.f32 ? launch_conv_state_t<128, float>(a, st) : launch_conv_state_t<128, uint16_t>(a, st);
    return a.f32 ? launch_conv_state_t<64, float>(a, st) : launch_conv_state_t<64, uint16_t>(a, st);
}

template <int D, typename TE>
static hipError_t launch_decode_prologue_t(const LayerArgs& a, hipStream_t st) {
    const int64_t items = (int64_t)a.N * a.H;
    const PrologueIn<TE> in{(const TE*)a.xq, (const TE*)a.xk, (const TE*)a.xv, (const TE*)a.xa, (const TE*)a.xb};
    hipLaunchKernelGGL((layer_decode_prologue_kernel<D, TE>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st,
                       in, (TE*)a.cs, a.wq, a.wk, a.wv, a.A_log, a.dt_bias, (int)items, a.H, (TE*)a.q, (TE*)a.k,
                       (TE*)a.v, (TE*)a.la, (TE*)a.beta);
    return hipGetLastError();
}

hipError_t launch_layer_decode_prologue(const LayerArgs& a, hipStream_t st) {
    if (a.D == 128)
        return a.f32 ? launch_decode_prologue_t<128, float>(a, st) : launch_decode_prologue_t<128, uint16_t>(a, st);
    return a.f32 ? launch_decode_prologue_t<64, float>(a, st) : launch_decode_prologue_t<64, uint16_t>(a, st);
}

template <int D, typename TE>
static hipError_t launch_prologue_t(const LayerArgs& a, hipStream_t st) {
    const int64_t blocks = (int64_t)((a.T + PT - 1) / PT) * a.H;  // (tile, head), head fastest
    const PrologueIn<TE> in{(const TE*)a.xq, (const TE*)a.xk, (const TE*)a.xv, (const TE*)a.xa, (const TE*)a.xb};
    hipLaunchKernelGGL((layer_prologue_kernel<D, TE>), dim3((unsigned)blocks), dim3(256), 0, st, in, a.wq, a.wk,
                       a.wv, a.A_log, a.dt_bias, a.cu, a.N, a.T, a.H, (TE*)a.q, (TE*)a.k, (TE*)a.v, (TE*)a.la,
                       (TE*)a.beta);
    return hipGetLastError();
}

hipError_t launch_layer_prologue(const LayerArgs& a, hipStream_t st) {
    if (a.D == 128) return a.f32 ? launch_prologue_t<128, float>(a, st) : launch_prologue_t<128, uint16_t>(a, st);
    return a.f32 ? launch_prologue_t<64, float>(a, st) : launch_prologue_t<64, uint16_t>(a, st);
}

template <int D, typename TE>
static hipError_t launch_epilogue_t(const LayerArgs& a, hipStream_t st) {
    const int64_t items = (int64_t)a.T * a.H;  // rows; G per wave, four waves per block
    hipLaunchKernelGGL((layer_epilogue_kernel<D, TE>), dim3((unsigned)((items + 4 * G - 1) / (4 * G))), dim3(256),
                       0, st, a.o, (const TE*)a.g, a.rms_w, (int)items, (TE*)a.y);
    return hipGetLastError();
}

hipError_t launch_layer_epilogue(const LayerArgs& a, hipStream_t st) {
    if (a.D == 128) return a.f32 ? launch_epilogue_t<128, float>(a, st) : launch_epilogue_t<128, uint16_t>(a, st);
    return a.f32 ? launch_epilogue_t<64, float>(a, st) : launch_epilogue_t<64, uint16_t>(a, st);
}

}  // namespace kda
