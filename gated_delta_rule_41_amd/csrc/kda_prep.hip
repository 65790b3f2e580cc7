// K1: per-chunk preparation of the chunkwise KDA algorithm.
//
// One 256-thread workgroup (4 waves) per (chunk, head). Wave w owns chunk rows
// 16w..16w+15 (one secondary chunk). The steps follow the chunkwise algorithm
// of the GeekNews "Kimi Linear" summary, sections "Algoritmo paralelo por
// chunks" and "Menos computação que o DPLR geral":
//
//  1. cumulative log-gate inside the chunk, g_r = sum_{s<=r} log alpha_s, per
//     key channel, kept in the log2 domain (G = g * log2 e) so v_exp_f32 is
//     used directly;
//  2. gated scalings Q+ = 2^G q, K- = 2^(G_last - G) k, K+ = 2^G k; every
//     factor is <= 1 so nothing overflows;
//  3. the two gated intra-chunk matrices the KDA transition needs (its DPLR
//     vectors are both tied to the key): A_kk[r,i] = beta_r sum_c k_rc k_ic
//     2^(G_rc - G_ic) (i < r) and A_qk[r,i] = sum_c q_rc k_ic 2^(G_rc - G_ic)
//     (i <= r), with secondary chunking: block (I, J) of 16 x 16 is one
//     matrix-core product (split bf16 with bf16 inputs) of
//     (x_r 2^(G_r - G_aI)) 2^(G_aI - G_aJ) by k_i 2^(G_aJ - G_i), a_I = first
//     row of block I. Left factors are <= 1, right factors lie in [1, 2^R_J]
//     with R_J the sub-chunk's gate range; a range above GUARD (log2 units)
//     switches the chunk to an exact elementwise path, so the result never
//     depends on overflow. Every exponent is formed from block-local sums
//     (16-row scans and whole-block totals), never as the difference of two
//     large cumulative gates, so fp32 keeps its relative precision;
//  4. the UT transform: T = (I + A_kk)^-1 is never formed; its four 16 x 16
//     diagonal blocks are inverted row by row by forward substitution in LDS,
//     and the WY factors W = T diag(beta) K+ and U = T diag(beta) V come from a
//     blocked forward substitution on the right-hand sides,
//     X_I = T_II (B_I - sum_{K<I} A_IK X_K), on the matrix cores. One inverse
//     serves both factors (nothing downstream inverts again).
//
// Outputs (workspace, layouts in kda_common.h): Q+, K-^T, -W, U, A_qk and
// gamma = 2^G_last for the chunk. Rows past the end of a sequence are
// zero-padded (k = q = v = 0, beta = 0, log alpha = 0), which is exactly
// neutral for every factor.
#include "kda_common.h"
#include "kda_launch.h"

#include <type_traits>

namespace kda {

constexpr float LOG2E = 1.4426950408889634f;
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

template <int D, bool F32>
struct PrepSmem {
    using E = typename Pol<F32>::E;
    using AE = typename APol<F32>::E;
    static constexpr int KT_PLANE = 64 * D;                              // elements per Kt plane
    static constexpr int R1 = APol<F32>::PLANES * 64 * D * (int)sizeof(AE);  // Kt, later -W / slow-path scan
    static constexpr int R4a = D * 64 * (int)sizeof(E);                 // K-^T staging
    static constexpr int R4b = 64 * 64 * 4 + 64 * 64 * (int)sizeof(E) + 4 * 256 * 4;  // Akk, Aqk, T_II
    static constexpr int R4 = R4a > R4b ? R4a : R4b;
    static constexpr int R3 = 64 * D * (int)sizeof(E);                   // beta K+
    static_assert(64 * D * 4 <= R1, "slow-path scan must fit in R1");
    static_assert(64 * D * (int)sizeof(E) <= R1, "-W staging must fit in R1");
    static constexpr int CONST = 22 * D * 4 + 64 * 4;  // tot xf eA eL cIJ, beta
    static constexpr int BYTES = R1 + R4 + R3 + CONST;
};

template <int D, typename TIn, typename TG, bool F32>
__global__ __launch_bounds__(256) void prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                   const TIn* __restrict__ v, const TG* __restrict__ la,
                                                   const TG* __restrict__ beta, const int32_t* __restrict__ cu,
                                                   int N, int T, int H, Ws<typename Pol<F32>::E> ws) {
    using P = Pol<F32>;
    using E = typename P::E;
    using Frag = typename P::Frag;
    using AP = APol<F32>;
    using AE = typename AP::E;
    using AFrag = typename AP::Frag;
    using SM = PrepSmem<D, F32>;
    constexpr int NS = D / 32;    // 32-deep slices over a head dimension
    constexpr int NCT = D / 16;   // 16-wide column tiles over a head dimension
    constexpr int PL = SM::KT_PLANE;

    extern __shared__ __align__(16) char smem[];
    AE* Kt_s = reinterpret_cast<AE*>(smem);                     // [planes][64][NS][4][8]
    E* Ws_s = reinterpret_cast<E*>(smem);                       // [64][NS][4][8] (-W), after Kt is dead
    float* xl_slow = reinterpret_cast<float*>(smem);            // [64][D] slow path: local scans
    char* r4 = smem + SM::R1;
    E* Km_s = reinterpret_cast<E*>(r4);                         // [D][2][4][8]
    float* Akk_s = reinterpret_cast<float*>(r4);                // [64][64]
    E* Aqk_s = reinterpret_cast<E*>(r4 + 64 * 64 * 4);          // [64][64]
    float* Td_s = reinterpret_cast<float*>(r4 + 64 * 64 * 4 + 64 * 64 * sizeof(E));  // [4][16][16]
    E* Bk_s = reinterpret_cast<E*>(smem + SM::R1 + SM::R4);     // [64][D]
    float* cst = reinterpret_cast<float*>(smem + SM::R1 + SM::R4 + SM::R3);
    float* tot = cst;                 // [4][D]  sum of the block's log2 gates
    float* xf = tot + 4 * D;          // [4][D]  log2 gate of the block's first row
    float* eA = xf + 4 * D;           // [4][D]  2^G(first row of I)
    float* eL = eA + 4 * D;           // [4][D]  2^(G_last - G(first row of I))
    float* cIJ = eL + 4 * D;          // [6][D]  2^(G(first row of I) - G(first row of J)), I > J
    float* beta_s = cIJ + 6 * D;      // [64]

    const int gc = blockIdx.x;
    const int h = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(cu, N, T, gc, loc)) return;
    const int t0 = loc.t0, L = loc.L;
    const int64_t chh = (int64_t)gc * H + h;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
    const int r = 16 * w + n;  // this lane's chunk row
    const bool valid = r < L;
    const int64_t rowoff = ((int64_t)(t0 + r) * H + h) * D;

    // ---- 1. log2 gate, scanned inside each 16-row block (per key channel)
    float xl[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
        if (valid) {
            ld_in4(la, rowoff + 32 * s + 4 * g, a4);
            ld_in4(la, rowoff + 32 * s + 16 + 4 * g, b4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xl[s][j] = a4[j] * LOG2E;
            xl[s][4 + j] = b4[j] * LOG2E;
        }
    }
    // inclusive scan across the 16 rows of this wave (lanes n of one DPP row)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) xl[s][j] += dpp_shr(xl[s][j], d);
    }
    if (n == 0 || n == 15) {
        float* dst = (n == 0 ? xf : tot) + w * D;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[32 * s + kslot(g, j)] = xl[s][j];
    }
    if (g == 0) beta_s[r] = valid ? ld_in(beta, (int64_t)(t0 + r) * H + h) : 0.f;
    __syncthreads();

    // ---- 2. per-block channel constants from block sums, and the overflow guard
    for (int idx = tid; idx < 15 * D; idx += 256) {
        const int ty = idx / D, c = idx % D;
        float tt[4], ff[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            tt[I] = tot[I * D + c];
            ff[I] = xf[I * D + c];
        }
        if (ty < 4) {  // 2^G(a_I) = 2^(sum_{J<I} tot_J + xf_I)
            float e = ff[ty];
            for (int J = 0; J < ty; ++J) e += tt[J];
            eA[ty * D + c] = exp2f(e);
        } else if (ty < 8) {  // 2^(G_last - G(a_I)) = 2^((tot_I - xf_I) + sum_{J>I} tot_J)
            const int I = ty - 4;
            float e = tt[I] - ff[I];
            for (int J = I + 1; J < 4; ++J) e += tt[J];
            eL[I * D + c] = exp2f(e);
        } else if (ty < 14) {  // 2^((tot_J - xf_J) + sum_{J<K<I} tot_K + xf_I)
            const int p = ty - 8;
            const int I = p < 1 ? 1 : (p < 3 ? 2 : 3);
            const int J = p - pair_index(I, 0);
            float e = tt[J] - ff[J] + ff[I];
            for (int K = J + 1; K < I; ++K) e += tt[K];
            cIJ[p * D + c] = exp2f(e);
        } else {
            ws.gam[chh * D + c] = exp2f(tt[0] + tt[1] + tt[2] + tt[3]);
        }
    }
    int bad = 0;
    if (tid < D) {
#pragma unroll
        for (int I = 0; I < 4; ++I) bad |= !(xf[I * D + tid] - tot[I * D + tid] <= GUARD);
    }
    const bool slow = __syncthreads_or(bad) != 0;

    // ---- 3. gated scalings
    const float br = beta_s[r];
    float qs[NS][8], ks[NS][8];  // q 2^(G - G_aw), k 2^(G - G_aw)  (fast path)
    E* qp_out = ws.qp + chh * 64 * D;
    E* km_out = ws.km + chh * D * 64;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        float q8[8], k8[8];
        {
            float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
            float c4[4] = {0.f, 0.f, 0.f, 0.f}, d4[4] = {0.f, 0.f, 0.f, 0.f};
            if (valid) {
                ld_in4(q, rowoff + 32 * s + 4 * g, a4);
                ld_in4(q, rowoff + 32 * s + 16 + 4 * g, b4);
                ld_in4(k, rowoff + 32 * s + 4 * g, c4);
                ld_in4(k, rowoff + 32 * s + 16 + 4 * g, d4);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                q8[j] = a4[j];
                q8[4 + j] = b4[j];
                k8[j] = c4[j];
                k8[4 + j] = d4[j];
            }
        }
        float qpv[8], ktv[8];
        if (!slow) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * s + kslot(g, j);
                const float dA = xl[s][j] - xf[w * D + c];  // G_r - G_aw, local sums only
                const float e = exp2f(dA);
                const float ei = exp2f(-dA);
                const float ea = eA[w * D + c];
                qs[s][j] = q8[j] * e;
                ks[s][j] = k8[j] * e;
                ktv[j] = k8[j] * ei;
                qpv[j] = qs[s][j] * ea;
                Km_s[c * 64 + 32 * (r >> 5) + split_pos(r)] = P::from_f(ktv[j] * eL[w * D + c]);
                Bk_s[r * D + c] = P::from_f(ks[s][j] * ea * br);
            }
            AP::store(Kt_s + (r * NS + s) * 32 + g * 8, PL, AP::make(ktv));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * s + kslot(g, j);
                float pre = 0.f, post = tot[w * D + c] - xl[s][j];
                for (int J = 0; J < w; ++J) pre += tot[J * D + c];
                for (int J = w + 1; J < 4; ++J) post += tot[J * D + c];
                const float eg = exp2f(pre + xl[s][j]);  // 2^G_r
                qpv[j] = q8[j] * eg;
                km_out[c * 64 + 32 * (r >> 5) + split_pos(r)] = P::from_f(k8[j] * exp2f(post));
                Bk_s[r * D + c] = P::from_f(k8[j] * eg * br);
                xl_slow[r * D + c] = xl[s][j];
                qs[s][j] = 0.f;
                ks[s][j] = 0.f;
            }
        }
        P::store(qp_out + (r * NS + s) * 32 + g * 8, P::make(qpv));
    }
    __syncthreads();

    // ---- 3b. K-^T to the workspace (fast path) / exact gated products (slow path)
    float akk_sl[16], aqk_sl[16];
    if (!slow) {
        constexpr int VEC = 16 / sizeof(E);
        for (int idx = tid; idx < D * 64 / VEC; idx += 256)
            reinterpret_cast<u32x4_t*>(km_out)[idx] = reinterpret_cast<const u32x4_t*>(Km_s)[idx];
    } else {
        // pair (rr, ii) = (p >> 6, p & 63), p = tid + 256 m; exponent
        // G_rr - G_ii = xl_rr - xl_ii + sum of the whole-block totals between them
#pragma unroll 1
        for (int m = 0; m < 16; ++m) {
            const int p = tid + 256 * m;
            const int rr = p >> 6, ii = p & 63;
            float sq = 0.f, sk = 0.f;
            if (ii <= rr && rr < L) {
                const int I = rr >> 4, J = ii >> 4;
                const int64_t ro = ((int64_t)(t0 + rr) * H + h) * D;
                const int64_t io = ((int64_t)(t0 + ii) * H + h) * D;
                for (int c = 0; c < D; ++c) {
                    float ex = xl_slow[rr * D + c] - xl_slow[ii * D + c];
                    for (int K = J; K < I; ++K) ex += tot[K * D + c];
                    const float kv = ld_in(k, io + c) * exp2f(ex);
                    sq += ld_in(q, ro + c) * kv;
                    sk += ld_in(k, ro + c) * kv;
                }
            }
            aqk_sl[m] = sq;
            akk_sl[m] = ii < rr ? sk * beta_s[rr] : 0.f;
        }
    }
    __syncthreads();

    // ---- 3c. A_qk and A_kk
    if (!slow) {
        const int I = w;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J > I) {
                // upper blocks are zero
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * I + 4 * g + i, cc = 16 * J + n;
                    Akk_s[rr * 64 + cc] = 0.f;
                    Aqk_s[rr * 64 + cc] = P::from_f(0.f);
                }
                continue;
            }
            f32x4_t aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float xq[8], xk[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float cf = (J < I) ? cIJ[pair_index(I, J) * D + 32 * s + kslot(g, j)] : 1.f;
                    xq[j] = qs[s][j] * cf;
                    xk[j] = ks[s][j] * cf;
                }
                const AFrag b = AP::load(Kt_s + ((16 * J + n) * NS + s) * 32 + g * 8, PL);
                AP::mma(aq, AP::make(xq), b);
                AP::mma(ak, AP::make(xk), b);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * I + 4 * g + i, cc = 16 * J + n;
                const bool lo_incl = (J < I) || (n <= 4 * g + i);
                const bool lo_strict = (J < I) || (n < 4 * g + i);
                Aqk_s[rr * 64 + cc] = P::from_f(lo_incl ? aq[i] : 0.f);
                Akk_s[rr * 64 + cc] = lo_strict ? ak[i] * beta_s[rr] : 0.f;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int p = tid + 256 * m;
            Akk_s[p] = akk_sl[m];
            Aqk_s[p] = P::from_f(aqk_sl[m]);
        }
    }
    __syncthreads();
    // ---- 4a. diagonal-block inverses T_II = (I + A_II)^-1 (wave 0); A_qk out (waves 1-3)
    if (w == 0) {
        const int b = l >> 4, j = l & 15;
        float acc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[rr] = (rr == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ti = acc[i];
#pragma unroll
            for (int rr = i + 1; rr < 16; ++rr) acc[rr] -= Akk_s[(16 * b + rr) * 64 + 16 * b + i] * ti;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Td_s[(b * 16 + rr) * 16 + j] = acc[rr];
    } else {
        E* aqk_out = ws.aqk + chh * 64 * 64;
        for (int idx = tid - 64; idx < 64 * 2 * 4; idx += 192) {
            const int rr = idx >> 3, s = (idx >> 2) & 1, gg = idx & 3;
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = P::to_f(Aqk_s[rr * 64 + 32 * s + kslot(gg, j)]);
            P::store(aqk_out + ((rr * 2 + s) * 4 + gg) * 8, P::make(x));
        }
    }
    __syncthreads();

    // ---- 4b. WY factors by blocked forward substitution: X = (I + A_kk)^-1 [beta K+ | beta V]
    {
        constexpr int TPW = NCT / 2;  // column tiles per wave (2 NCT tiles over 4 waves)
        E* u_out = ws.u + chh * 64 * D;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int ctg = w * TPW + tt;           // 0 .. 2 NCT - 1
            const bool isW = ctg < NCT;
            const int ct = isW ? ctg : ctg - NCT;   // column tile inside W or U
            f32x4_t X[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4_t Y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * I + 4 * g + i;
                    if (isW) {
                        Y[i] = P::to_f(Bk_s[rr * D + 16 * ct + n]);
                    } else {
                        Y[i] = rr < L ? beta_s[rr] * ld_in(v, ((int64_t)(t0 + rr) * H + h) * D + 16 * ct + n)
                                      : 0.f;
                    }
                }
                if (I > 0) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (2 * s >= I) break;
                        float xa[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int col = 32 * s + kslot(g, j);
                            xa[j] = (col < 16 * I) ? -Akk_s[(16 * I + n) * 64 + col] : 0.f;
                        }
                        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
                        const Frag bx = frag_from_acc<F32>(X[2 * s], (2 * s + 1 < I) ? X[2 * s + 1] : zero);
                        P::mma(Y, P::make(xa), bx);
                    }
                }
                float ta[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) ta[j] = (j < 4) ? Td_s[(I * 16 + n) * 16 + 4 * g + j] : 0.f;
                const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
                X[I] = zero;
                P::mma(X[I], P::make(ta), frag_from_acc<F32>(Y, zero));
            }
            if (isW) {
                // -W into LDS in the split k order over key channels
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 16 * I + 4 * g + i;
                        const int s = ct >> 1, gg = n >> 2, jj = 4 * (ct & 1) + (n & 3);
                        Ws_s[(rr * NS + s) * 32 + gg * 8 + jj] = P::from_f(-X[I][i]);
                    }
            } else {
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    E* dst = u_out + ((ct * 4 + I) * 64 + l) * 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[i] = P::from_f(X[I][i]);
                }
            }
        }
    }
    __syncthreads();
    {
        constexpr int VEC = 16 / sizeof(E);
        E* wn_out = ws.wn + chh * 64 * D;
        for (int idx = tid; idx < 64 * D / VEC; idx += 256)
            reinterpret_cast<u32x4_t*>(wn_out)[idx] = reinterpret_cast<const u32x4_t*>(Ws_s)[idx];
    }
}

template <int D, typename TIn, typename TG, bool F32>
static hipError_t launch_prep_t(const ChunkArgs& a, hipStream_t st) {
    using E = typename Pol<F32>::E;
    using SM = PrepSmem<D, F32>;
    Ws<E> ws{(E*)a.qp, (E*)a.km, (E*)a.wn, (E*)a.u, (E*)a.aqk, a.gam, (E*)a.h, (E*)a.vn};
    auto kern = prep_kernel<D, TIn, TG, F32>;
    const hipError_t e = allow_dynamic_lds((const void*)kern, SM::BYTES);
    if (e != hipSuccess) return e;
    dim3 grid(a.NC, a.H), block(256);
    hipLaunchKernelGGL(kern, grid, block, SM::BYTES, st, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                       (const TG*)a.la, (const TG*)a.beta, a.cu, a.N, a.T, a.H, ws);
    return hipGetLastError();
}

template <int D, bool F32>
static hipError_t launch_prep_d(const ChunkArgs& a, hipStream_t st) {
    using TIn = typename std::conditional<F32, float, uint16_t>::type;
    if (a.gate_f32) return launch_prep_t<D, TIn, float, F32>(a, st);
    return launch_prep_t<D, TIn, uint16_t, F32>(a, st);
}

hipError_t launch_prep(const ChunkArgs& a, hipStream_t st) {
    if (a.D == 128) return a.in_f32 ? launch_prep_d<128, true>(a, st) : launch_prep_d<128, false>(a, st);
    return a.in_f32 ? launch_prep_d<64, true>(a, st) : launch_prep_d<64, false>(a, st);
}

}  // namespace kda
