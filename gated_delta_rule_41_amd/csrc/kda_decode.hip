// K4: one recurrent KDA decode step, in place on the fp32 state.
//
// For each (sequence, head), with a = exp(log_alpha), state S (dk x dv):
//   u = beta * (v - S^T (a * k))       residual against the decayed state
//   S <- Diag(a) S + k u^T             decay, then delta-rule write
//   o = S^T q                          read with the updated state
// (the recurrence for one token; GeekNews "Kimi Linear" summary, sections
// "Da atenção linear ao Gated DeltaNet" and "Controle fino de memória no Kimi
// Delta Attention"; the fixed-size state that decode streams is the point of
// remio.ai "Kimi Linear Acabou de Superar ...", section "Por Que a
// Decodificação de Contexto Longo Coloca a Atenção Completa sob Pressão").
//
// Memory-bound: 2 * dk * dv * 4 bytes of state per head-step. One workgroup of
// NT threads per (sequence, head), streaming that head's contiguous state;
// thread t owns four adjacent value columns (one 16-byte vector per row) of
// dk / R rows, R = 4 NT / dv row groups, so a wave reads whole rows and every
// state byte is read and written once with 16-byte coalesced accesses. The two
// column sums (S^T (a*k) and S^T q) are reduced across row groups through LDS.
// NT = 1024 for d = 128 (measured: 6.04 TB/s at 1024 threads, 5.87 at 256,
// 5.56 at 512 on 256 x 32 heads); 256 for d = 64.
//
// EPI: the layer's epilogue (per-head RMSNorm, output gate; GeekNews "Kimi
// Linear" summary, section "Configuração do modelo Kimi Linear") on the row o
// before it leaves: the workgroup holds the whole row, so wave 0 takes its
// channels as the epilogue kernel's lanes do (lane j: channels PER j ..) and
// runs the same per-row code, and y is bitwise that of this kernel's fp32 o
// followed by the epilogue kernel.
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"
#include "kda_layer_util.h"

namespace kda {

template <int D> constexpr int decode_threads() { return D == 128 ? 1024 : 256; }

template <int D, typename TIn, typename TG, bool OUT_F32, bool EPI = false>
__global__ __launch_bounds__(decode_threads<D>()) void decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                     const TIn* __restrict__ v, const TG* __restrict__ la,
                                                     const TG* __restrict__ beta, float* __restrict__ state,
                                                     void* __restrict__ o, int NH, const TIn* __restrict__ xg,
                                                     const float* __restrict__ rms_w, TIn* __restrict__ y) {
    static_assert(!EPI || OUT_F32, "the epilogue reads o in fp32");
    constexpr int CQ = D / 4;        // column quads
    constexpr int R = decode_threads<D>() / CQ;  // row groups
    constexpr int RPT = D / R;       // rows per thread
    __shared__ f32x4_t red[R][CQ];

    const int unit = blockIdx.x;     // sequence * H + head
    if (unit >= NH) return;
    const int tid = threadIdx.x;
    const int cq = tid % CQ;
    const int rg = tid / CQ;
    const int64_t vec = (int64_t)unit * D;
    f32x4_t* S = reinterpret_cast<f32x4_t*>(state + (int64_t)unit * D * D);

    f32x4_t s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&S[(rg + R * i) * CQ + cq]);

    float a[RPT], kk[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + R * i;
        a[i] = __expf(ld_in(la, vec + r));
        kk[i] = ld_in(k, vec + r);
    }
    // partial S^T (a * k) over this thread's rows
    f32x4_t p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float w = a[i] * kk[i];
        p += w * s[i];
    }
    red[rg][cq] = p;
    __syncthreads();
    f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < R; ++i) tot += red[i][cq];
    const float b = ld_in(beta, (int64_t)unit);
    float vv[4];
    ld_in4(v, vec + 4 * cq, vv);
    f32x4_t u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = b * (vv[j] - tot[j]);

    // decay + write, stream the new state out, and accumulate S^T q
    f32x4_t po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + R * i;
        const f32x4_t ns = a[i] * s[i] + kk[i] * u;
        __builtin_nontemporal_store(ns, &S[r * CQ + cq]);
        po += ld_in(q, vec + r) * ns;
    }
    __syncthreads();  // everyone has read red[] for the first sum
    red[rg][cq] = po;
    __syncthreads();
    if constexpr (EPI) {
        if (tid < 64) {  // wave 0; its lanes cq < CQ hold the row's column quads
            f32x4_t ot = {0.f, 0.f, 0.f, 0.f};
            if (tid < CQ) {
#pragma unroll
                for (int i = 0; i < R; ++i) ot += red[i][cq];
            }
            // lane j takes channels PER j .. PER j + PER - 1 from the quad holding them
            constexpr int PER = D / 64;
            const int c0 = PER * tid;
            float e[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) e[m] = __shfl(ot[m], c0 >> 2);
            float x[PER], xgv[PER], wc[PER];
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int m = (c0 + p) & 3;
                x[p] = m == 0 ? e[0] : m == 1 ? e[1] : m == 2 ? e[2] : e[3];
                wc[p] = rms_w[c0 + p];
            }
            Pair<TIn, PER>::ld(xg + vec + c0, xgv);
            epilogue_row<D, TIn>(x, xgv, wc, y + vec + c0);
        }
        return;
    }
    if (rg == 0) {
        f32x4_t ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < R; ++i) ot += red[i][cq];
        if (OUT_F32) {
            reinterpret_cast<f32x4_t*>(static_cast<float*>(o) + vec)[cq] = ot;
        } else {
            u32x2_t w;
            w[0] = pack2bf(ot[0], ot[1]);
            w[1] = pack2bf(ot[2], ot[3]);
            reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o) + vec)[cq] = w;
        }
    }
}

template <int D, typename TIn, typename TG>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    const int NH = a.N * a.H;
    dim3 grid(NH), block(decode_threads<D>());
    const TIn* xg = static_cast<const TIn*>(a.xg);
    TIn* y = static_cast<TIn*>(a.y);
    if (a.epi) {
        if constexpr (std::is_same<TIn, TG>::value)  // the layer's one dtype (checked by the caller)
            hipLaunchKernelGGL((decode_kernel<D, TIn, TG, true, true>), grid, block, 0, st, (const TIn*)a.q,
                               (const TIn*)a.k, (const TIn*)a.v, (const TG*)a.la, (const TG*)a.beta, a.state,
                               nullptr, NH, xg, a.rms_w, y);
        else
            return hipErrorInvalidValue;
    } else if (a.out_f32)
        hipLaunchKernelGGL((decode_kernel<D, TIn, TG, true>), grid, block, 0, st, (const TIn*)a.q,
                           (const TIn*)a.k, (const TIn*)a.v, (const TG*)a.la, (const TG*)a.beta, a.state,
                           a.o, NH, nullptr, nullptr, nullptr);
    else
        hipLaunchKernelGGL((decode_kernel<D, TIn, TG, false>), grid, block, 0, st, (const TIn*)a.q,
                           (const TIn*)a.k, (const TIn*)a.v, (const TG*)a.la, (const TG*)a.beta, a.state,
                           a.o, NH, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
    if (a.in_f32) {
        if (a.gate_f32) return launch_decode_t<D, float, float>(a, st);
        return launch_decode_t<D, float, uint16_t>(a, st);
    }
    if (a.gate_f32) return launch_decode_t<D, uint16_t, float>(a, st);
    return launch_decode_t<D, uint16_t, uint16_t>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.N == 0) return hipSuccess;
    return a.D == 128 ? launch_decode_d<128>(a, st) : launch_decode_d<64>(a, st);
}

}  // namespace kda
