// K2: sequential inter-chunk state recursion of the chunkwise KDA algorithm.
//
// For each chunk n of a sequence, in order (GeekNews "Kimi Linear" summary,
// section "Algoritmo paralelo por chunks": each chunk starts from the previous
// chunk's final state, and the state update is done in matrix form per chunk):
//     h_n   = S                                 (chunk-entry state, kept for the output)
//     V_new = U - W S                            (values corrected by the WY keys)
//     S    <- Diag(gamma) S + K-^T V_new         (gamma = exp(g_last) per key channel)
//
// Columns of S are independent (each product above touches value column j
// only through column j), so one wave owns a 16-wide value-column slab of one
// (sequence, head) and keeps its dk x 16 fp32 slab of S in accumulator
// registers for the whole sequence: nothing but the per-chunk factors moves.
// Thanks to the split k order (kda_common.h) the accumulator tiles of S and of
// V_new are directly the B operands of the next product: no LDS round trip and
// no cross-lane shuffle on the dependency chain. The per-chunk factors for
// chunk n+1 are loaded while chunk n computes.
//
// Workgroup -> work mapping is XCD-aware: workgroups are dispatched round-robin
// over the 8 XCDs, so the dv/16 slabs of one (sequence, head) are given ids that
// are congruent mod 8 and land on the same XCD, where they share the L2 copy of
// that head's W and K- factors.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <int D, bool F32>
struct ChunkFactors {
    using P = Pol<F32>;
    using E = typename P::E;
    using Frag = typename P::Frag;
    static constexpr int NS = D / 32;
    static constexpr int NT = D / 16;
    Frag wn[4][NS];     // -W rows 16I + n, slice s
    Frag km[NT][2];     // K-^T rows 16t + n, chunk-row slice s
    E u[4][4];          // U rows 16I + 4g + i, this slab's column n
    f32x4_t gam[NT];    // gamma for rows 16t + 4g + i

    __device__ __forceinline__ void load(const Ws<E>& ws, int64_t chh, int ct, int l) {
        const int n = l & 15, g = l >> 4;
        const E* wp = ws.wn + chh * 64 * D;
        const E* kp = ws.km + chh * D * 64;
        const E* up = ws.u + chh * 64 * D + (int64_t)ct * 4 * 64 * 4;
        const float* gp = ws.gam + chh * D;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int s = 0; s < NS; ++s) wn[I][s] = P::load(wp + ((16 * I + n) * NS + s) * 32 + g * 8);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) km[t][s] = P::load(kp + ((16 * t + n) * 2 + s) * 32 + g * 8);
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) u[I][i] = up[(I * 64 + l) * 4 + i];
#pragma unroll
        for (int t = 0; t < NT; ++t) gam[t] = *reinterpret_cast<const f32x4_t*>(gp + 16 * t + 4 * g);
    }
};

template <int D, bool F32>
__global__ __launch_bounds__(64) void recur_kernel(const float* __restrict__ s0, float* __restrict__ s_final,
                                                   const int32_t* __restrict__ cu, int N, int T, int H,
                                                   Ws<typename Pol<F32>::E> ws) {
    using P = Pol<F32>;
    using E = typename P::E;
    using Frag = typename P::Frag;
    constexpr int NS = D / 32;
    constexpr int NT = D / 16;  // row tiles over dk == column slabs over dv

    // XCD-aware decode of the workgroup id
    const int b = blockIdx.x;
    const int NU = N * H;
    int unit, ct;
    if ((NU & 7) == 0) {
        ct = (b >> 3) % NT;
        unit = (b & 7) + 8 * (b / (8 * NT));
    } else {
        unit = b / NT;
        ct = b % NT;
    }
    if (unit >= NU) return;
    const int seq = unit / H, h = unit % H;
    const int l = threadIdx.x, n = l & 15, g = l >> 4;

    int co, nch;
    seq_chunks(cu, T, seq, co, nch);

    // state slab: rows 16t + 4g + i, column 16 ct + n
    f32x4_t S[NT];
    const int64_t sbase = (int64_t)unit * D * D + 16 * ct + n;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] = s0 ? s0[sbase + (int64_t)(16 * t + 4 * g + i) * D] : 0.f;

    ChunkFactors<D, F32> cur, nxt;
    if (nch > 0) cur.load(ws, (int64_t)co * H + h, ct, l);
    for (int c = 0; c < nch; ++c) {
        const int64_t chh = (int64_t)(co + c) * H + h;
        if (c + 1 < nch) nxt.load(ws, chh + H, ct, l);

        // h_n = S as B-operand fragments (also the operand of W S below)
        Frag sb[NS];
        E* hp = ws.h + chh * D * D + (int64_t)ct * NS * 64 * 8;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            sb[s] = frag_from_acc<F32>(S[2 * s], S[2 * s + 1]);
            P::store(hp + (s * 64 + l) * 8, sb[s]);
        }
        // V_new = U + (-W) S
        f32x4_t V[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int i = 0; i < 4; ++i) V[I][i] = P::to_f(cur.u[I][i]);
#pragma unroll
            for (int s = 0; s < NS; ++s) P::mma(V[I], cur.wn[I][s], sb[s]);
        }
        Frag vb[2];
        E* vp = ws.vn + chh * 64 * D + (int64_t)ct * 2 * 64 * 8;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            vb[s] = frag_from_acc<F32>(V[2 * s], V[2 * s + 1]);
            P::store(vp + (s * 64 + l) * 8, vb[s]);
        }
        // S <- Diag(gamma) S + K-^T V_new
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            S[t] = cur.gam[t] * S[t];
#pragma unroll
            for (int s = 0; s < 2; ++s) P::mma(S[t], cur.km[t][s], vb[s]);
        }
        if (c + 1 < nch) cur = nxt;
    }
    if (s_final) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_final[sbase + (int64_t)(16 * t + 4 * g + i) * D] = S[t][i];
    }
}

template <int D, bool F32>
static hipError_t launch_recur_t(const ChunkArgs& a, hipStream_t st) {
    using E = typename Pol<F32>::E;
    Ws<E> ws{(E*)a.qp, (E*)a.km, (E*)a.wn, (E*)a.u, (E*)a.aqk, a.gam, (E*)a.h, (E*)a.vn};
    constexpr int NT = D / 16;
    const int NU = a.N * a.H;
    dim3 grid(NU * NT), block(64);
    hipLaunchKernelGGL((recur_kernel<D, F32>), grid, block, 0, st, a.s0, a.s_final, a.cu, a.N, a.T, a.H, ws);
    return hipGetLastError();
}

hipError_t launch_recur(const ChunkArgs& a, hipStream_t st) {
    if (a.D == 128) return a.in_f32 ? launch_recur_t<128, true>(a, st) : launch_recur_t<128, false>(a, st);
    return a.in_f32 ? launch_recur_t<64, true>(a, st) : launch_recur_t<64, false>(a, st);
}

}  // namespace kda
