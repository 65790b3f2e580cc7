// K3: fused chunk output of the chunkwise KDA algorithm.
//
//     O = Q+ h_n + A_qk V_new
//
// the inter-chunk (recurrent) part through the chunk-entry state plus the
// intra-chunk (parallel) part through the gated query-key matrix (GeekNews
// "Kimi Linear" summary, section "Algoritmo paralelo por chunks": the output
// step combines recurrent processing between chunks with parallel processing
// inside the chunk, organised around matrix products).
//
// One 256-thread workgroup per (chunk, head): wave w computes value-column
// tiles {w, w + 4, ...} for all 64 rows. Both products accumulate into the
// same tiles, so the sum never leaves registers; rows past the end of the
// sequence are not stored.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <int D, bool F32, bool OUT_F32>
__global__ __launch_bounds__(256) void output_kernel(const SeqMeta* __restrict__ tab, int N, int T, int H,
                                                     Ws<typename Pol<F32>::E> ws, void* __restrict__ o) {
    using P = Pol<F32>;
    using E = typename P::E;
    using Frag = typename P::Frag;
    constexpr int NS = D / 32;
    constexpr int NT = D / 16;
    constexpr int CPW = NT / 4;  // column tiles per wave

    const int gc = blockIdx.x;
    const int h = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(tab, N, T, gc, loc)) return;
    const int t0 = loc.t0, L = loc.L;
    const int64_t chh = (int64_t)gc * H + h;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;

    const E* qp = ws.qp + chh * 64 * D;
    const E* ap = ws.aqk + chh * 64 * 64;
    const E* hp = ws.h + chh * D * D;
    const E* vp = ws.vn + chh * 64 * D;

    f32x4_t acc[4][CPW];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) acc[I][cc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // inter-chunk part: Q+ h_n (k = key channel)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        Frag bh[CPW];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int ct = w + 4 * cc;
            bh[cc] = P::load(hp + ((int64_t)(ct * NS + s) * 64 + l) * 8);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const Frag a = P::load(qp + ((16 * I + n) * NS + s) * 32 + g * 8);
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) P::mma(acc[I][cc], a, bh[cc]);
        }
    }
    // intra-chunk part: A_qk V_new (k = chunk row)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        Frag bv[CPW];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int ct = w + 4 * cc;
            bv[cc] = P::load(vp + ((ct * 2 + s) * 64 + l) * 8);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (16 * I + 15 < 32 * s) continue;  // A_qk block row I is zero for k-slices above the diagonal
            const Frag a = P::load(ap + ((16 * I + n) * 2 + s) * 32 + g * 8);
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) P::mma(acc[I][cc], a, bv[cc]);
        }
    }
    // store rows 16I + 4g + i, column 16 ct + n
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 16 * I + 4 * g + i;
            if (rr >= L) continue;
            const int64_t ob = ((int64_t)(t0 + rr) * H + h) * D;
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) {
                const int col = 16 * (w + 4 * cc) + n;
                if (OUT_F32)
                    static_cast<float*>(o)[ob + col] = acc[I][cc][i];
                else
                    static_cast<uint16_t*>(o)[ob + col] = f2bf(acc[I][cc][i]);
            }
        }
}

template <int D, bool F32>
static hipError_t launch_output_t(const ChunkArgs& a, hipStream_t st) {
    using E = typename Pol<F32>::E;
    Ws<E> ws{(E*)a.qp, (E*)a.km, (E*)a.wn, (E*)a.u, (E*)a.aqk, a.gam, (E*)a.h, (E*)a.vn};
    dim3 grid(a.NC, a.H), block(256);
    if (a.out_f32)
        hipLaunchKernelGGL((output_kernel<D, F32, true>), grid, block, 0, st, a.tab, a.N, a.T, a.H, ws, a.o);
    else
        hipLaunchKernelGGL((output_kernel<D, F32, false>), grid, block, 0, st, a.tab, a.N, a.T, a.H, ws, a.o);
    return hipGetLastError();
}

hipError_t launch_output(const ChunkArgs& a, hipStream_t st) {
    if (a.D == 128) return a.in_f32 ? launch_output_t<128, true>(a, st) : launch_output_t<128, false>(a, st);
    return a.in_f32 ? launch_output_t<64, true>(a, st) : launch_output_t<64, false>(a, st);
}

}  // namespace kda
