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
//     matrix-core product (with bf16 inputs: split bf16 for A_qk, plain bf16
//     for A_kk, which only feeds the UT transform) of
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
// gamma = 2^G_last for the chunk; with fp32 factors and a destination given,
// also the gated key products A_kk / beta, which the backward differentiates.
// Rows past the end of a sequence are zero-padded (k = q = v = 0, beta = 0,
// log alpha = 0), which is exactly neutral for every factor.
//
// The fused-prologue variant (PRO, bf16 only) starts from the layer's
// pre-activations instead of q, k, v, log alpha, beta: each wave first runs the
// layer prologue (kda_layer_util.h) for its 16 rows into LDS, rounded to bf16
// exactly as the prologue kernel stores them, and phase 0 reads that stage.
// A chunk that takes the exact slow path copies its q, k rows to a workspace
// scratch, which that path reads instead of the inputs.
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_layer_util.h"
#include "kda_prep_util.h"

#include <type_traits>

namespace kda {

// LDS plan (bytes). Row strides are padded so that the matrix-core operand
// reads (one 16-byte vector per lane, lanes = 16 rows x 4 k-groups) and the
// transposing writes spread over the banks.
//
// With 16-bit operands (MT) the row -> channel transposes that K-^T, beta K+
// and beta V need are done on the matrix cores: a product with a 0/1 selector
// (exact) turns a lane-per-row operand into a lane-per-channel accumulator
// tile, which is stored with one 8-byte access per lane. K-^T then goes
// straight to the workspace, and beta K+ / beta V are kept as accumulator
// tiles [column tile][row block][lane], the form the WY solve consumes.
template <int D, bool F32>
struct PrepSmem {
    using E = typename Pol<F32>::E;
    using AE = typename APol<F32>::E;
    static constexpr bool MT = !F32;
    static constexpr int KT_STRIDE = D + 8;                  // Kt row (elements)
    static constexpr int KT_PLANE = 64 * KT_STRIDE;          // elements per hi / lo plane
    static constexpr int KM_STRIDE = 64 + 4;                 // K-^T staging row (elements)
    static constexpr int BK_STRIDE = 64 + 4;                 // beta K+ / beta V transposed row (elements)
    static constexpr int AK_STRIDE = 20;                     // A_kk / T_II block row (floats)
    static constexpr int AK_BLOCK = 16 * AK_STRIDE;          // floats per 16 x 16 block
    static constexpr int R1 = APol<F32>::PLANES * KT_PLANE * (int)sizeof(AE);  // Kt; later -W, slow-path scans
    static constexpr int R4a = D * KM_STRIDE * (int)sizeof(E);                // K-^T staging
    static constexpr int R4b = 10 * AK_BLOCK * 4;                             // A_kk lower blocks
    static constexpr int R4 = MT ? R4b : (R4a > R4b ? R4a : R4b);
    static constexpr int R3 = MT ? 64 * D * (int)sizeof(E) : D * BK_STRIDE * (int)sizeof(E);  // beta K+, transposed
    // tot xf eA eL cIJ (fp32 operands: + the low parts of tot and xf); later T_II
    static constexpr int NCONST = F32 ? 30 : 22;
    static constexpr int CONST = NCONST * D * 4;
    static constexpr int BETA = 64 * 4 + 16;  // beta per row, then one overflow flag per wave
    // beta V: with 16-bit operands fp32 accumulator tiles (exact, the WY solve
    // carries it as two fp16 terms) in R1 once Kt is dead, and -W goes from the
    // solve's registers straight to the workspace; with fp32 operands beta V
    // (transposed rows) gets a region of its own and the -W staging takes R1
    static constexpr int RBV = MT ? 64 * D * 4 : D * BK_STRIDE * (int)sizeof(E);
    static constexpr bool BV_IN_R1 = MT;
    static constexpr int R5 = BV_IN_R1 ? 0 : RBV;
    static constexpr int BYTES = R1 + R4 + R3 + CONST + BETA + R5;
    static constexpr int BV_AT = BV_IN_R1 ? 0 : R1 + R4 + R3 + CONST + BETA;
    static constexpr int WS_AT = 0;  // -W staging (fp32 operands only)
    static_assert(64 * D * 4 <= R1, "slow-path scans must fit in R1");
    static_assert(!F32 || 64 * D * 4 <= R4, "slow-path low parts must fit in R4");
    static_assert(!MT || RBV <= R1, "beta V tiles must fit in R1");
    static_assert(64 * D * (int)sizeof(E) <= (MT ? R3 : R1), "-W staging must fit its region");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(4 * AK_BLOCK * 4 <= CONST, "T_II must fit in the constants area");
    // fused prologue: q, k, v, log alpha [64][SS] bf16 and beta [64] fp32, over
    // everything else (all of it is written only after phase 0)
    static constexpr int SS = D + 16;
    static constexpr int STAGE = 4 * 64 * SS * 2 + 64 * 4;
    static_assert(F32 || STAGE <= BYTES, "the prologue stage must fit in the 16-bit plan");
};

// The fused prologue's inputs (unused by the other instantiations).
struct ProArgs {
    PrologueIn<uint16_t> in;
    const float *wq, *wk, *wv, *A_log, *dt_bias;
    uint16_t* qk_scr;  // [chunk-head][q, k][64][D] bf16, written by slow chunks only
    float* epi_part;   // the fused epilogue's per-row partial sums ([chunk-head][D/16][64]), set to -1 here (or null)
};

template <int D, typename TIn, typename TG, bool F32, bool PRO = false>
// (fp32 operands at d = 128 need more than 80 KiB of LDS, so one workgroup per
// CU; the register budget follows)
__global__ __launch_bounds__(256, (F32 && D == 128) ? 1 : 2) void prep_kernel(const TIn* q, const TIn* k, const TIn* v,
                                                      const TG* la, const TG* beta,
                                                      const SeqMeta* __restrict__ tab, int N, int T, int H,
                                                      int g0, Ws<typename Pol<F32>::E> ws, ProArgs pa) {
    static_assert(!PRO || (!F32 && std::is_same<TIn, uint16_t>::value && std::is_same<TG, uint16_t>::value),
                  "the fused prologue is bf16 only");
    using P = Pol<F32>;
    using E = typename P::E;
    using Frag = typename P::Frag;
    using AP = APol<F32>;
    using AE = typename AP::E;
    using AFrag = typename AP::Frag;
    using SM = PrepSmem<D, F32>;
    constexpr int NS = D / 32;    // 32-deep slices over a head dimension
    constexpr int NCT = D / 16;   // 16-wide column tiles over a head dimension
    constexpr int TPW = NCT / 2;  // WY column tiles per wave (W tiles on waves 0-1, U tiles on 2-3)
    constexpr int KTS = SM::KT_STRIDE, KMS = SM::KM_STRIDE, BKS = SM::BK_STRIDE, AKS = SM::AK_STRIDE;
    constexpr int AKB = SM::AK_BLOCK;

    extern __shared__ __align__(16) char smem[];
    AE* Kt_s = reinterpret_cast<AE*>(smem);                     // [planes][64][KTS] keys 2^(G_aJ - G)
    E* Bv_t = reinterpret_cast<E*>(smem + SM::BV_AT);           // beta V transposed ([D][BKS]; fp32 operands)
    float* Bv_f = reinterpret_cast<float*>(smem + SM::BV_AT);   // beta V fp32 tiles (16-bit operands)
    E* Ws_s = reinterpret_cast<E*>(smem + SM::WS_AT);           // [64][NS][4][8] -W staging (fp32 operands)
    float* xl_slow = reinterpret_cast<float*>(smem);            // [64][D] slow path: local scans
    float* xl_slow_lo = reinterpret_cast<float*>(smem + SM::R1); // [64][D] their low parts (fp32 operands)
    char* r4 = smem + SM::R1;
    E* Km_s = reinterpret_cast<E*>(r4);                         // [D][KMS] K-^T in split row order
    float* Akk_s = reinterpret_cast<float*>(r4);                // 10 blocks [16][AKS]: diag I at I, (I,J) at 4+pair
    E* Bk_t = reinterpret_cast<E*>(smem + SM::R1 + SM::R4);     // beta K+ transposed ([D][BKS] or tiles)
    float* cst = reinterpret_cast<float*>(smem + SM::R1 + SM::R4 + SM::R3);
    float* tot = cst;                 // [4][D]  sum of the block's log2 gates
    float* xf = tot + 4 * D;          // [4][D]  log2 gate of the block's first row
    float* eA = xf + 4 * D;           // [4][D]  2^G(first row of I)
    float* eL = eA + 4 * D;           // [4][D]  2^(G_last - G(first row of I))
    float* cIJ = eL + 4 * D;          // [6][D]  2^(G(first row of I) - G(first row of J)), I > J
    float* Td_s = cst;                // [4][16][AKS] T_II, after the constants are dead
    float* tot_lo = cst + 22 * D;     // [4][D]  (fp32 operands) low parts of tot and xf, whose
    float* xf_lo = tot_lo + 4 * D;    // [4][D]  scans are carried as hi + lo pairs
    float* beta_s = cst + SM::NCONST * D;  // [64]
    int* slow_s = reinterpret_cast<int*>(beta_s + 64);  // [4] per-wave overflow flags

    // head fastest: the workgroups dispatched together read whole token rows of
    // the inputs and write consecutive workspace blocks, in the chunk order the
    // state recursion consumes them (slots from g0, the workspace from 0)
    const int lc = blockIdx.x / H;
    const int h = blockIdx.x - lc * H;
    ChunkLoc loc;
    if (!locate_chunk(tab, N, T, g0 + lc, loc)) return;
    const int t0 = loc.t0, L = loc.L;
    const int64_t chh = (int64_t)lc * H + h;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
    const int r = 16 * w + n;  // this lane's chunk row
    if constexpr (PRO) {
        // the recursion's fused epilogue reads a slot's sign bit as "not written
        // yet" (this kernel ends before that one starts)
        if (pa.epi_part)
            for (int i = tid; i < (D / 16) * 64; i += 256) pa.epi_part[chh * (D / 16) * 64 + i] = -1.f;
    }
    const bool valid = r < L;
    const int64_t rowoff = ((int64_t)(t0 + r) * H + h) * D;

    // ---- 0. all row inputs of this lane (channels 32 s + split(g, j)). Rows past
    // the end of the sequence load row t0 (always valid) and are zeroed
    // afterwards, so the loads carry no branch and all of them are in flight at
    // once.
    const int64_t ldoff = valid ? rowoff : ((int64_t)t0 * H + h) * D;
    // (The input pointers are deliberately not __restrict__: loads through
    // restrict-qualified read-only pointers may be moved freely, and the
    // compiler would sink these towards their first uses, serialising them
    // behind the gate scans. The empty asm statement below pins them.)
    RowRaw<TG, NS> rla;
    RowRaw<TIn, NS> rq, rk, rv;
    float bval;
    bool maybe_slow = false;  // fused prologue: this chunk may take the exact path
    if constexpr (PRO) {
        // the layer prologue for rows 16 w .. 16 w + 15 into the stage
        constexpr int SS = SM::SS, PER = D / 64;
        uint16_t* st_q = reinterpret_cast<uint16_t*>(smem);
        uint16_t* st_k = st_q + 64 * SS;
        uint16_t* st_v = st_k + 64 * SS;
        uint16_t* st_la = st_v + 64 * SS;
        float* st_b = reinterpret_cast<float*>(st_la + 64 * SS);
        {
            constexpr int PG = 8;  // tokens per load group
            const int c0 = PER * l;
            const int sstart = loc.start;  // the chunk lies in one sequence
            ConvFilters<D> f;
            using PR = Pair<uint16_t, PER>;
            float gs[PER] = {};  // log2 gate summed over rows 1..15 of this wave's block
#pragma unroll 1
            for (int gi = 0; gi < 16 / PG; ++gi) {
                const int rw = 16 * w + PG * gi, tw = t0 + rw;
                PrologueWindow<D, PG, uint16_t> pw;
                pw.load(pa.in, h, tw, T, H, c0, l);
                if (gi == 0) f.load(pa.wq, pa.wk, pa.wv, pa.A_log, pa.dt_bias, h, c0);
                const float bl = pw.compute(f, tw, t0 + L, [&](int) { return sstart; },
                                            [&](int j, const float (&oq)[PER], const float (&ok)[PER],
                                                const float (&ov)[PER], const float (&og)[PER]) {
                                                const int so = (rw + j) * SS + c0;
                                                PR::st(st_q + so, oq);
                                                PR::st(st_k + so, ok);
                                                PR::st(st_v + so, ov);
                                                PR::st(st_la + so, og);
                                                if (rw + j > 16 * w) {
#pragma unroll
                                                    for (int p = 0; p < PER; ++p)
                                                        gs[p] += bf2f(f2bf(og[p])) * LOG2E;
                                                }
                                            });
                if (l < PG) st_b[rw + l] = bf2f(f2bf(bl));  // as a bf16 beta input reads
            }
            // Phase 2 sends the chunk to the exact path when some block's gate
            // range, minus the sum of its rows 1..15, exceeds GUARD. These sums
            // of the same fp32 terms in another order differ by ~1e-4 near the
            // guard, so a margin of 1 flags every chunk that phase 2 will send
            // (and NaN or infinite gates too).
            bool flag = false;
#pragma unroll
            for (int p = 0; p < PER; ++p) flag |= !(-gs[p] <= GUARD - 1.f);
            maybe_slow = __syncthreads_or(flag);  // also publishes the stage
        }
        const int so = (valid ? r : 0) * SS;
        rla.load(reinterpret_cast<const TG*>(st_la), so, g);
        rq.load(reinterpret_cast<const TIn*>(st_q), so, g);
        rk.load(reinterpret_cast<const TIn*>(st_k), so, g);
        rv.load(reinterpret_cast<const TIn*>(st_v), so, g);
        bval = st_b[valid ? r : 0];
    } else {
        rla.load(la, ldoff, g);  // first: the scans wait only for it
        rq.load(q, ldoff, g);
        rk.load(k, ldoff, g);
        rv.load(v, ldoff, g);
        bval = ld_in(beta, (int64_t)(valid ? t0 + r : t0) * H + h);
        asm volatile("" ::: "memory");
    }
    float xl[NS][8], q8[NS][8], k8[NS][8], v8[NS][8];
    // With fp32 operands the gate is carried as a pair, x = xl + xlo: the exact
    // log2-unit value of each gate, then block scans in double-float. The
    // exponents that matter are differences of two partial sums of the same
    // block (magnitudes up to ~280 under extreme decay); plain fp32 scans leave
    // independent roundings of ~1e-5 in neighbouring rows, which decide the
    // fp32 path's accuracy. With 16-bit operands the plain scan suffices.
    float xlo[F32 ? NS : 1][8];
    if constexpr (F32) {
        rla.get(xl, valid, 1.f);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) log2_units(xl[s][j], xl[s][j], xlo[s][j]);
    } else {
        rla.get(xl, valid, LOG2E);
    }
    rq.get(q8, valid, 1.f);
    rk.get(k8, valid, 1.f);
    rv.get(v8, valid, 1.f);
    if constexpr (PRO) {
        __syncthreads();  // the stage is read; later phases reuse its LDS
        // the exact path re-reads q and k rows: a chunk that may take it keeps
        // its rows in the scratch (published by the barriers of phases 1-3)
        if (maybe_slow && valid) {
            uint16_t* sq = pa.qk_scr + chh * 2 * 64 * D + r * D;
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int c = 32 * s + 16 * hf + 4 * g;
                    u32x2_t pq, pk;
                    pq[0] = pack2bf(q8[s][4 * hf], q8[s][4 * hf + 1]);
                    pq[1] = pack2bf(q8[s][4 * hf + 2], q8[s][4 * hf + 3]);
                    pk[0] = pack2bf(k8[s][4 * hf], k8[s][4 * hf + 1]);
                    pk[1] = pack2bf(k8[s][4 * hf + 2], k8[s][4 * hf + 3]);
                    *reinterpret_cast<u32x2_t*>(sq + c) = pq;
                    *reinterpret_cast<u32x2_t*>(sq + 64 * D + c) = pk;
                }
        }
    }

    // ---- 1. log2 gate scanned inside each 16-row block (lanes n of one DPP row)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if constexpr (F32) {
                    const float yh = dpp_shr(xl[s][j], d), yl = dpp_shr(xlo[s][j], d);
                    float sh, er;
                    two_sum(xl[s][j], yh, sh, er);
                    xl[s][j] = sh;
                    xlo[s][j] = __fadd_rn(__fadd_rn(xlo[s][j], yl), er);
                } else {
                    xl[s][j] += dpp_shr(xl[s][j], d);
                }
            }
    }
    if (n == 0 || n == 15) {
        float* dst = (n == 0 ? xf : tot) + w * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            *reinterpret_cast<f32x4_t*>(dst + 32 * s + 4 * g) = f32x4_t{xl[s][0], xl[s][1], xl[s][2], xl[s][3]};
            *reinterpret_cast<f32x4_t*>(dst + 32 * s + 16 + 4 * g) =
                f32x4_t{xl[s][4], xl[s][5], xl[s][6], xl[s][7]};
            if constexpr (F32) {
                float* dl = (n == 0 ? xf_lo : tot_lo) + w * D;
                *reinterpret_cast<f32x4_t*>(dl + 32 * s + 4 * g) =
                    f32x4_t{xlo[s][0], xlo[s][1], xlo[s][2], xlo[s][3]};
                *reinterpret_cast<f32x4_t*>(dl + 32 * s + 16 + 4 * g) =
                    f32x4_t{xlo[s][4], xlo[s][5], xlo[s][6], xlo[s][7]};
            }
        }
    }
    if (g == 0) beta_s[r] = valid ? bval : 0.f;
    __syncthreads();

    // ---- 2. per-block channel constants from block sums, and the overflow guard.
    // Thread t serves channel t % D and every P-th of the 15 constants, P = 256 / D
    // (the part t / D is uniform over a wave).
    int bad = 0;
    {
        constexpr int P = 256 / D;
        const int c = tid % D, part = tid / D;
        // (every constant below is a sum of same-sign gate terms, or a block
        // total minus its own first row, so the pairs can be folded here)
        float tt[4], ff[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            tt[I] = tot[I * D + c];
            ff[I] = xf[I * D + c];
            if constexpr (F32) {
                tt[I] += tot_lo[I * D + c];
                ff[I] += xf_lo[I * D + c];
            }
        }
#pragma unroll
        for (int ty = 0; ty < 15; ++ty) {
            if (ty % P != part) continue;
            if (ty < 4) {  // 2^G(a_I) = 2^(sum_{J<I} tot_J + xf_I)
                float e = ff[ty];
                for (int J = 0; J < ty; ++J) e += tt[J];
                eA[ty * D + c] = ex2(e);
            } else if (ty < 8) {  // 2^(G_last - G(a_I)) = 2^((tot_I - xf_I) + sum_{J>I} tot_J)
                const int I = ty - 4;
                float e = tt[I] - ff[I];
                for (int J = I + 1; J < 4; ++J) e += tt[J];
                eL[I * D + c] = ex2(e);
            } else if (ty < 14) {  // 2^((tot_J - xf_J) + sum_{J<K<I} tot_K + xf_I)
                const int p = ty - 8;
                const int I = p < 1 ? 1 : (p < 3 ? 2 : 3);
                const int J = p - pair_index(I, 0);
                float e = tt[J] - ff[J] + ff[I];
                for (int K = J + 1; K < I; ++K) e += tt[K];
                cIJ[p * D + c] = ex2(e);
            } else {
                ws.gam[chh * D + c] = ex2(tt[0] + tt[1] + tt[2] + tt[3]);
            }
        }
        if (part == 0) {
#pragma unroll
            for (int I = 0; I < 4; ++I) bad |= !(ff[I] - tt[I] <= GUARD);
        }
    }
    // one flag per wave (a ballot), so the barrier that publishes the
    // constants also publishes the guard
    const bool wave_bad = __ballot(bad) != 0;
    if (l == 0) slow_s[w] = wave_bad;
    __syncthreads();
    const bool slow = (slow_s[0] | slow_s[1] | slow_s[2] | slow_s[3]) != 0;
    // 0/1 selectors for the matrix-core transposes (16-bit operands): with A a
    // lane-per-row operand over a 32-channel slice, A sel[hf] is the 16 x 16
    // block of channels 16 hf .. 16 hf + 15 in accumulator layout (lane n holds
    // channel 16 hf + n, rows 4 g .. 4 g + 3), exactly
    Frag sel[2];
    if constexpr (SM::MT) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float x[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) x[jj] = (g == (n >> 2) && jj == 4 * hf + (n & 3)) ? 1.f : 0.f;
            sel[hf] = P::make(x);
        }
    }
    // transposes one slice s of a lane-per-row vector: K-^T blocks to the
    // workspace (8 bytes per lane at rows 16 w + 4 g + (0..3) of channel
    // 32 s + 16 hf + n, in the split row order), or beta-scaled blocks to
    // accumulator tiles [column tile][row block][lane] in LDS (the destination
    // kind is a compile-time choice, so the phase stays one basic block)
    auto tr_slice = [&](const float (&x)[8], int s, auto to_km, E* dst) {
        const Frag a = P::make(x);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            f32x4_t t = {0.f, 0.f, 0.f, 0.f};
            P::mma(t, a, sel[hf]);
            u32x2_t pk;
            pk[0] = pack2h(t[0], t[1]);
            pk[1] = pack2h(t[2], t[3]);
            if constexpr (decltype(to_km)::value)
                *reinterpret_cast<u32x2_t*>(dst + (32 * s + 16 * hf + n) * 64 + 32 * (w >> 1) + 8 * g + 4 * (w & 1)) = pk;
            else
                *reinterpret_cast<u32x2_t*>(dst + (((2 * s + hf) * 4 + w) * 64 + l) * 4) = pk;
        }
    };

    // ---- 3. gated scalings
    const float br = beta_s[r];
    float qs[NS][8], ks[NS][8];  // q 2^(G - G_aw), k 2^(G - G_aw)  (fast path)
    E* qp_out = ws.qp + chh * 64 * D;
    // Q+: with 16-bit operands in fragment order, [row block][slice][64 lanes][8]
    // (each matrix-core operand fragment of the output product one contiguous
    // 1 KiB); with fp32 operands row-major, [64][slices][32] (split order)
    auto qp_at = [&](int s) -> int64_t {
        if constexpr (SM::MT) return ((int64_t)(w * NS + s) * 64 + l) * 8;
        return (int64_t)(r * NS + s) * 32 + g * 8;
    };
    E* km_out = ws.km + chh * D * 64;
    const int kmpos = 32 * (r >> 5) + split_pos(r);
    // fast and slow paths each cover every slice inside one branch
    if (!slow) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float xf8[8], ea8[8], el8[8], ktv[8], kmv[8], bkv[8], qpv[8];
            float xfl8[F32 ? 8 : 1];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int c0 = 32 * s + 16 * hf + 4 * g;
                const f32x4_t a = *reinterpret_cast<const f32x4_t*>(xf + w * D + c0);
                const f32x4_t b = *reinterpret_cast<const f32x4_t*>(eA + w * D + c0);
                const f32x4_t c = *reinterpret_cast<const f32x4_t*>(eL + w * D + c0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xf8[4 * hf + j] = a[j];
                    ea8[4 * hf + j] = b[j];
                    el8[4 * hf + j] = c[j];
                }
                if constexpr (F32) {
                    const f32x4_t al = *reinterpret_cast<const f32x4_t*>(xf_lo + w * D + c0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) xfl8[4 * hf + j] = al[j];
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * s + kslot(g, j);
                float dA = xl[s][j] - xf8[j];  // G_r - G_aw, local sums only
                if constexpr (F32) dA += xlo[s][j] - xfl8[j];
                const float e = ex2(dA);
                const float ei = ex2(-dA);
                qs[s][j] = q8[s][j] * e;
                ks[s][j] = k8[s][j] * e;
                ktv[j] = k8[s][j] * ei;
                qpv[j] = qs[s][j] * ea8[j];
                kmv[j] = ktv[j] * el8[j];
                bkv[j] = ks[s][j] * ea8[j] * br;
                if constexpr (!SM::MT) {
                    Km_s[c * KMS + kmpos] = P::from_f(kmv[j]);
                    Bk_t[c * BKS + r] = P::from_f(bkv[j]);
                }
            }
            if constexpr (SM::MT) {
                tr_slice(kmv, s, std::true_type{}, km_out);
                tr_slice(bkv, s, std::false_type{}, Bk_t);
            }
            AP::store(Kt_s + r * KTS + s * 32 + g * 8, SM::KT_PLANE, AP::make(ktv));
            P::store(qp_out + qp_at(s), P::make(qpv));
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float kmv[8], bkv[8], qpv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * s + kslot(g, j);
                // pre: totals of the blocks before this one; post: G_last - G_r
                // (the difference of two partial sums of this block comes first,
                // with the low parts on the fp32 path)
                float pre = 0.f, post = tot[w * D + c] - xl[s][j], xr = xl[s][j];
                if constexpr (F32) {
                    post += tot_lo[w * D + c] - xlo[s][j];
                    xr += xlo[s][j];
                }
                for (int J = 0; J < w; ++J) pre += tot[J * D + c] + (F32 ? tot_lo[J * D + c] : 0.f);
                for (int J = w + 1; J < 4; ++J) post += tot[J * D + c] + (F32 ? tot_lo[J * D + c] : 0.f);
                const float eg = exp2f(pre + xr);  // 2^G_r
                qpv[j] = q8[s][j] * eg;
                kmv[j] = k8[s][j] * exp2f(post);
                bkv[j] = k8[s][j] * eg * br;
                if constexpr (!SM::MT) {
                    km_out[c * 64 + kmpos] = P::from_f(kmv[j]);
                    Bk_t[c * BKS + r] = P::from_f(bkv[j]);
                }
                xl_slow[r * D + c] = xl[s][j];
                if constexpr (F32) xl_slow_lo[r * D + c] = xlo[s][j];
                qs[s][j] = 0.f;
                ks[s][j] = 0.f;
            }
            if constexpr (SM::MT) {
                tr_slice(kmv, s, std::true_type{}, km_out);
                tr_slice(bkv, s, std::false_type{}, Bk_t);
            }
            P::store(qp_out + qp_at(s), P::make(qpv));
        }
    }
    __syncthreads();

    // ---- 3b. K-^T to the workspace (fast path, fp32 operands) / exact gated products (slow path)
    float akk_sl[16], aqk_sl[16];
    if (!slow && !SM::MT) {
        for (int idx = tid; idx < D * 16; idx += 256) {  // 4 elements per item
            const int c = idx >> 4, qd = idx & 15;
            const E* src = Km_s + c * KMS + 4 * qd;
            E* dst = km_out + c * 64 + 4 * qd;
            if constexpr (F32)
                *reinterpret_cast<f32x4_t*>(dst) = *reinterpret_cast<const f32x4_t*>(src);
            else
                *reinterpret_cast<u32x2_t*>(dst) = *reinterpret_cast<const u32x2_t*>(src);
        }
    } else if (slow) {
        // pair (rr, ii) = (p >> 6, p & 63), p = tid + 256 m; exponent
        // G_rr - G_ii = xl_rr - xl_ii + sum of the whole-block totals between them
#pragma unroll 1
        for (int m = 0; m < 16; ++m) {
            const int p = tid + 256 * m;
            const int rr = p >> 6, ii = p & 63;
            float sq = 0.f, sk = 0.f;
            if (ii <= rr && rr < L) {
                const int I = rr >> 4, J = ii >> 4;
                const TIn* qsrc = q;
                const TIn* ksrc = k;
                int64_t ro = ((int64_t)(t0 + rr) * H + h) * D;
                int64_t io = ((int64_t)(t0 + ii) * H + h) * D;
                if constexpr (PRO) {
                    qsrc = reinterpret_cast<const TIn*>(pa.qk_scr + chh * 2 * 64 * D);
                    ksrc = qsrc + 64 * D;
                    ro = (int64_t)rr * D;
                    io = (int64_t)ii * D;
                }
                for (int c = 0; c < D; ++c) {
                    // G_rr - G_ii: with the low parts (fp32 operands), each
                    // difference of two partial sums of one block is formed first
                    float ex;
                    if constexpr (F32) {
                        if (J == I) {
                            ex = (xl_slow[rr * D + c] - xl_slow[ii * D + c]) +
                                 (xl_slow_lo[rr * D + c] - xl_slow_lo[ii * D + c]);
                        } else {
                            ex = (tot[J * D + c] - xl_slow[ii * D + c]) + (tot_lo[J * D + c] - xl_slow_lo[ii * D + c]);
                            for (int K = J + 1; K < I; ++K) ex += tot[K * D + c] + tot_lo[K * D + c];
                            ex += xl_slow[rr * D + c] + xl_slow_lo[rr * D + c];
                        }
                    } else {
                        ex = xl_slow[rr * D + c] - xl_slow[ii * D + c];
                        for (int K = J; K < I; ++K) ex += tot[K * D + c];
                    }
                    const float kv = ld_in(ksrc, io + c) * exp2f(ex);
                    sq += ld_in(qsrc, ro + c) * kv;
                    sk += ld_in(ksrc, ro + c) * kv;
                }
            }
            aqk_sl[m] = sq;
            akk_sl[m] = ii < rr ? sk : 0.f;  // beta is applied where A_kk is stored
        }
    }
    if (slow || !SM::MT) __syncthreads();  // (block-uniform condition)

    // ---- 3c. A_qk (straight to the workspace) and A_kk (LDS, lower blocks only)
    // (16-bit operands: two fp16 planes, hi then lo, so the output's A_qk V_new
    // product sees about 22 significant bits of A_qk)
    E* aqk_out = ws.aqk + chh * 64 * 64 * (SM::MT ? 2 : 1);
    // (16-bit operands: fragment order, [row block][slice][64 lanes][8] per plane,
    // as Q+; fp32 operands: row-major [64][2][32], split order)
    auto aqk_put = [&](int rr, int cc, float x) {
        const int s2 = cc >> 5, c2 = cc & 31;
        const int g2 = (c2 & 15) >> 2, j2 = 4 * (c2 >> 4) + (c2 & 3);
        const int at = SM::MT ? ((((rr >> 4) * 2 + s2) * 64 + (rr & 15) + 16 * g2) * 8 + j2)
                              : (rr * 2 + s2) * 32 + 8 * g2 + j2;
        const E hi = P::from_f(x);
        aqk_out[at] = hi;
        if constexpr (SM::MT) aqk_out[64 * 64 + at] = P::from_f(x - P::to_f(hi));
    };
    // the backward's forward recompute (fp32 factors) also keeps the gated key
    // products P_kk = A_kk / beta, row-major [64][64], zero on and above the diagonal
    float* pkk_out = nullptr;
    if constexpr (F32) pkk_out = ws.am ? ws.am + chh * 64 * 64 : nullptr;
    // Wave I computes the blocks (I, J <= I) of both matrices, slice by slice
    // over the channels so that the operands of every block of a slice are
    // read together (I is made a compile-time constant per wave).
    auto products = [&](auto Ic) {
        constexpr int I = decltype(Ic)::value;
        f32x4_t aq[I + 1], ak[I + 1];
#pragma unroll
        for (int J = 0; J <= I; ++J) {
            aq[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ak[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            AFrag bkt[I + 1];
#pragma unroll
            for (int J = 0; J <= I; ++J)
                bkt[J] = AP::load(Kt_s + (16 * J + n) * KTS + s * 32 + g * 8, SM::KT_PLANE);
            f32x4_t c0[I + 1], c1[I + 1];
#pragma unroll
            for (int J = 0; J < I; ++J) {
                const float* cp = cIJ + pair_index(I, J) * D + 32 * s + 4 * g;
                c0[J] = *reinterpret_cast<const f32x4_t*>(cp);
                c1[J] = *reinterpret_cast<const f32x4_t*>(cp + 16);
            }
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                float xq[8], xk[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = J < I ? c0[J][j] : 1.f, b = J < I ? c1[J][j] : 1.f;
                    xq[j] = qs[s][j] * a;
                    xk[j] = ks[s][j] * a;
                    xq[4 + j] = qs[s][4 + j] * b;
                    xk[4 + j] = ks[s][4 + j] * b;
                }
                if constexpr (SM::MT)
                    AP::mma_qk_t(aq[J], xq, ak[J], xk, bkt[J]);  // aq transposed: operand fragments
                else
                    AP::mma_qk(aq[J], xq, ak[J], xk, bkt[J]);
            }
        }
        if constexpr (SM::MT) {
            // A_qk in fragment order: lane n + 16 g holds row 16 I + n at columns
            // 16 J + 4 g + i of each block J (transposed tiles); fragment (I, s)
            // joins blocks 2 s and 2 s + 1. Causal mask on the diagonal block:
            // column 4 g + i <= row n. Two fp16 planes, hi then lo.
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float x[8];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    constexpr int NJ = I + 1;
                    const int J = 2 * s2 + hb;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = 0.f;
                        if (J < I) v = aq[J < NJ ? J : 0][i];
                        else if (J == I) v = (4 * g + i <= n) ? aq[J < NJ ? J : 0][i] : 0.f;
                        x[4 * hb + i] = v;
                    }
                }
                const Frag2 fx = split_frag(x);
                E* dst = aqk_out + ((I * 2 + s2) * 64 + l) * 8;
                P::store(dst, fx.hi);
                P::store(dst + 64 * 64, fx.lo);
            }
        }
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J > I) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (!SM::MT) aqk_put(16 * I + 4 * g + i, 16 * J + n, 0.f);
                    if (pkk_out) pkk_out[(16 * I + 4 * g + i) * 64 + 16 * J + n] = 0.f;
                }
                continue;
            }
            const int blk = (J == I) ? I : 4 + pair_index(I, J);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * g + i;  // row inside the block
                const bool lo_incl = (J < I) || (n <= rl);
                const bool lo_strict = (J < I) || (n < rl);
                if constexpr (!SM::MT) aqk_put(16 * I + rl, 16 * J + n, lo_incl ? aq[J][i] : 0.f);
                Akk_s[blk * AKB + rl * AKS + n] = lo_strict ? ak[J][i] * beta_s[16 * I + rl] : 0.f;
                if (pkk_out) pkk_out[(16 * I + rl) * 64 + 16 * J + n] = lo_strict ? ak[J][i] : 0.f;
            }
        }
    };
    if (!slow) {
        switch (w) {
            case 0: products(std::integral_constant<int, 0>{}); break;
            case 1: products(std::integral_constant<int, 1>{}); break;
            case 2: products(std::integral_constant<int, 2>{}); break;
            default: products(std::integral_constant<int, 3>{}); break;
        }
    } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int p = tid + 256 * m;
            const int rr = p >> 6, ii = p & 63, I = rr >> 4, J = ii >> 4;
            aqk_put(rr, ii, aqk_sl[m]);
            if (pkk_out) pkk_out[rr * 64 + ii] = akk_sl[m];
            if (J <= I) {
                const int blk = (J == I) ? I : 4 + pair_index(I, J);
                Akk_s[blk * AKB + (rr & 15) * AKS + (ii & 15)] = akk_sl[m] * beta_s[rr];
            }
        }
    }
    __syncthreads();

    // beta V, transposed like beta K+, into the now free Kt region. With 16-bit
    // operands each 32-channel slice is split into fp16 hi and lo parts, both
    // transposed on the matrix cores (exact: a selector product), and summed
    // into fp32 accumulator tiles [column tile][row block][lane][4], so beta V
    // reaches the solve unrounded (beta v of bf16 inputs has 16 significant bits)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if constexpr (SM::MT) {
            float bvv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) bvv[j] = v8[s][j] * br;
            const Frag2 bx = split_frag(bvv);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4_t t = {0.f, 0.f, 0.f, 0.f};
                P::mma(t, bx.lo, sel[hf]);
                P::mma(t, bx.hi, sel[hf]);
                *reinterpret_cast<f32x4_t*>(Bv_f + (((2 * s + hf) * 4 + w) * 64 + l) * 4) = t;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) Bv_t[(32 * s + kslot(g, j)) * BKS + r] = P::from_f(v8[s][j] * br);
        }
    }

    // ---- 4a. diagonal-block inverses T_II = (I + A_II)^-1 by row forward substitution (wave 0)
    if (w == 0) {
        const int b = l >> 4, j = l & 15;
        float acc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[rr] = (rr == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ti = acc[i];
#pragma unroll
            for (int rr = i + 1; rr < 16; ++rr) acc[rr] -= Akk_s[b * AKB + rr * AKS + i] * ti;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Td_s[b * AKB + rr * AKS + j] = acc[rr];
    }
    __syncthreads();

    // ---- 4b. WY factors by blocked forward substitution: X = (I + A_kk)^-1 [beta K+ | beta V].
    // With 16-bit operands the B operands of every product here (the blocks X_K
    // and the right-hand side Y) are two-term fp16 (hi + lo): U carries the
    // values themselves, whose single fp16 rounding would already cost a
    // sizeable part of the error budget on heavy-tailed values. The W waves run
    // the same code (their time is hidden behind the U waves' anyway).
    {
        const bool isW = w < 2;
        float* u_out = (F32 ? reinterpret_cast<float*>(ws.u) : ws.uf) + chh * 64 * D;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        f32x4_t X[TPW][4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            // operands shared by every column tile of this wave
            Frag aoff[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (2 * s >= I) break;
                float xa[8];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int K = 2 * s + hf;
                    if (K < I) {
                        const f32x4_t a =
                            *reinterpret_cast<const f32x4_t*>(Akk_s + (4 + pair_index(I, K)) * AKB + n * AKS + 4 * g);
#pragma unroll
                        for (int j = 0; j < 4; ++j) xa[4 * hf + j] = -a[j];
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) xa[4 * hf + j] = 0.f;
                    }
                }
                aoff[s] = P::make(xa);
            }
            Frag at;
            {
                const f32x4_t a = *reinterpret_cast<const f32x4_t*>(Td_s + I * AKB + n * AKS + 4 * g);
                float ta[8] = {a[0], a[1], a[2], a[3], 0.f, 0.f, 0.f, 0.f};
                at = P::make(ta);
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int ct = (w & 1) * TPW + tt;  // column tile inside W (waves 0-1) or U (waves 2-3)
                f32x4_t Y;
                if constexpr (SM::MT) {
                    if (isW) {
                        const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(Bk_t + ((ct * 4 + I) * 64 + l) * 4);
                        Y = f32x4_t{h2f(bb[0] & 0xffffu), h2f(bb[0] >> 16), h2f(bb[1] & 0xffffu), h2f(bb[1] >> 16)};
                    } else {
                        Y = *reinterpret_cast<const f32x4_t*>(Bv_f + ((ct * 4 + I) * 64 + l) * 4);
                    }
                } else {
                    const E* bsrc = (isW ? Bk_t : Bv_t) + (16 * ct + n) * BKS + 16 * I + 4 * g;
                    if constexpr (F32) {
                        Y = *reinterpret_cast<const f32x4_t*>(bsrc);
                    } else {
                        const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(bsrc);
                        Y = f32x4_t{h2f(bb[0] & 0xffffu), h2f(bb[0] >> 16), h2f(bb[1] & 0xffffu), h2f(bb[1] >> 16)};
                    }
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (2 * s >= I) break;
                    const f32x4_t& x1 = (2 * s + 1 < I) ? X[tt][2 * s + 1] : zero;
                    if constexpr (SM::MT)
                        mma2(Y, aoff[s], split_from_acc(X[tt][2 * s], x1));
                    else
                        P::mma(Y, aoff[s], frag_from_acc<F32>(X[tt][2 * s], x1));
                }
                X[tt][I] = zero;
                if constexpr (SM::MT)
                    mma2(X[tt][I], at, split_from_acc(Y, zero));
                else
                    P::mma(X[tt][I], at, frag_from_acc<F32>(Y, zero));
            }
        }
        if constexpr (SM::MT) {
            if (isW) {
                // -W straight to the workspace, 16 bytes per lane. A pair of row
                // blocks (2q, 2q + 1) of column tile ct, rounded to fp16, is the A
                // operand of its transpose (rows in the split k order); a product
                // with a 0/-1 selector takes each 16-row half, leaving lane n + 16 G
                // with row 16 I + n at channels 16 ct + 4 G .. + 3 (exact: fp16
                // values times -1), and the wave's even and odd column tiles of one
                // slice fill the split-order positions 8 G .. 8 G + 7 of that row.
                E* wn_out = ws.wn + chh * 64 * D;
                Frag wsel[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        wsel[hh].v[j] = ((j >> 2) == hh && 4 * g + (j & 3) == n) ? (_Float16)-1.f : (_Float16)0.f;
#pragma unroll
                for (int sp = 0; sp < TPW / 2; ++sp) {
                    const int s = (w & 1) * (TPW / 2) + sp;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float xe[8] = {X[2 * sp][2 * q][0], X[2 * sp][2 * q][1], X[2 * sp][2 * q][2],
                                             X[2 * sp][2 * q][3], X[2 * sp][2 * q + 1][0], X[2 * sp][2 * q + 1][1],
                                             X[2 * sp][2 * q + 1][2], X[2 * sp][2 * q + 1][3]};
                        const float xo[8] = {X[2 * sp + 1][2 * q][0], X[2 * sp + 1][2 * q][1],
                                             X[2 * sp + 1][2 * q][2], X[2 * sp + 1][2 * q][3],
                                             X[2 * sp + 1][2 * q + 1][0], X[2 * sp + 1][2 * q + 1][1],
                                             X[2 * sp + 1][2 * q + 1][2], X[2 * sp + 1][2 * q + 1][3]};
                        const Frag ae = P::make(xe), ao = P::make(xo);
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            f32x4_t ce = zero, co = zero;
                            P::mma(ce, ae, wsel[hh]);
                            P::mma(co, ao, wsel[hh]);
                            const u32x4_t pk = {pack2h(ce[0], ce[1]), pack2h(ce[2], ce[3]), pack2h(co[0], co[1]),
                                                pack2h(co[2], co[3])};
                            *reinterpret_cast<u32x4_t*>(wn_out + (16 * (2 * q + hh) + n) * D + 32 * s + 8 * g) = pk;
                        }
                    }
                }
            } else {
                // U in fp32 accumulator-tile order
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    const int ct = (w & 1) * TPW + tt;
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        *reinterpret_cast<f32x4_t*>(u_out + ((ct * 4 + I) * 64 + l) * 4) = X[tt][I];
                }
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int ct = (w & 1) * TPW + tt;
                if (isW) {
                    // -W into LDS in the split k order over key channels
#pragma unroll
                    for (int I = 0; I < 4; ++I)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rr = 16 * I + 4 * g + i;
                            const int s = ct >> 1, gg = n >> 2, jj = 4 * (ct & 1) + (n & 3);
                            Ws_s[(rr * NS + s) * 32 + gg * 8 + jj] = P::from_f(-X[tt][I][i]);
                        }
                } else {
                    // U in fp32 accumulator-tile order
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        *reinterpret_cast<f32x4_t*>(u_out + ((ct * 4 + I) * 64 + l) * 4) = X[tt][I];
                }
            }
        }
    }
    if constexpr (!SM::MT) {
        __syncthreads();
        constexpr int VEC = 16 / sizeof(E);
        E* wn_out = ws.wn + chh * 64 * D;
        for (int idx = tid; idx < 64 * D / VEC; idx += 256)
            reinterpret_cast<u32x4_t*>(wn_out)[idx] = reinterpret_cast<const u32x4_t*>(Ws_s)[idx];
    }
}

template <int D, typename TIn, typename TG, bool F32, bool PRO = false>
static hipError_t launch_prep_t(const ChunkArgs& a, hipStream_t st) {
    using E = typename Pol<F32>::E;
    using SM = PrepSmem<D, F32>;
    Ws<E> ws{(E*)a.qp, (E*)a.km, (E*)a.wn, (E*)a.u, (E*)a.aqk, a.gam, (E*)a.h, (E*)a.vn, (E*)a.am};
    ws.uf = static_cast<float*>(a.u);  // U is fp32 on every path
    ProArgs pa{};
    if constexpr (PRO)
        pa = ProArgs{{(const uint16_t*)a.xq, (const uint16_t*)a.xk, (const uint16_t*)a.xv, (const uint16_t*)a.xa,
                      (const uint16_t*)a.xb},
                     a.wq, a.wk, a.wv, a.A_log, a.dt_bias, (uint16_t*)a.qk_scr, a.epi ? a.epi_part : nullptr};
    auto kern = prep_kernel<D, TIn, TG, F32, PRO>;
    const hipError_t e = allow_dynamic_lds((const void*)kern, SM::BYTES);
    if (e != hipSuccess) return e;
    dim3 grid(a.slots() * a.H), block(256);  // NC * H < 2^31 (checked by the caller)
    hipLaunchKernelGGL(kern, grid, block, SM::BYTES, st, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                       (const TG*)a.la, (const TG*)a.beta, a.tab, a.N, a.T, a.H, a.piece.g0, ws, pa);
    return hipGetLastError();
}

template <int D, bool F32>
static hipError_t launch_prep_d(const ChunkArgs& a, hipStream_t st) {
    if constexpr (F32) {
        if (a.in_f32)
            return a.gate_f32 ? launch_prep_t<D, float, float, true>(a, st) : launch_prep_t<D, float, uint16_t, true>(a, st);
    }
    // bf16 inputs: fp16 factors, or fp32 factors for the backward's recompute
    return a.gate_f32 ? launch_prep_t<D, uint16_t, float, F32>(a, st) : launch_prep_t<D, uint16_t, uint16_t, F32>(a, st);
}

hipError_t launch_prep(const ChunkArgs& a, hipStream_t st) {
    if (a.pro)  // bf16 pre-activations, fp16 factors (checked by the caller)
        return a.D == 128 ? launch_prep_t<128, uint16_t, uint16_t, false, true>(a, st)
                          : launch_prep_t<64, uint16_t, uint16_t, false, true>(a, st);
    const bool f32 = a.in_f32 || a.f32_factors;
    if (a.D == 128) return f32 ? launch_prep_d<128, true>(a, st) : launch_prep_d<128, false>(a, st);
    return f32 ? launch_prep_d<64, true>(a, st) : launch_prep_d<64, false>(a, st);
}

}  // namespace kda
