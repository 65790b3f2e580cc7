// K1 for the general DPLR transition (the comparison operator):
//
//     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t
//
// KDA ties both low-rank vectors to the key; with free a and b a chunk needs
// four gated intra-chunk matrices instead of two and three more chunk products
// (GeekNews "Kimi Linear" summary, section "Menos computação que o DPLR
// geral"). Per chunk, with inclusive cumulative log2 gate G_r and exclusive one
// E_r = G_r - x_r (the low-rank read of row r sees the state before row r's
// decay):
//   A_ba[r,s] = sum_c b_rc a_sc 2^(E_rc - G_sc), A_bk the same with k   (s < r)
//   A_qk[r,s] = sum_c q_rc k_sc 2^(G_rc - G_sc), A_qa the same with a   (s <= r)
//   T = (I + A_ba)^-1,  W' = T B~ (B~_r = 2^E_r b_r),  U' = T A_bk V
// so that the chunk's low-rank reads are u = W' h + U', its state update
// S' = Diag(2^G_last) h + K-^T V - A-^T u and its output
// O = Q+ h + A_qk V - A_qa u.
//
// One 256-thread workgroup (4 waves) per (chunk, head); wave w owns rows
// 16w..16w+15 (one secondary chunk). The design follows the KDA kernel
// (kda_prep.hip): block-local log2 scans, anchored factors, split-bf16 gated
// products on the matrix cores, diagonal-block inverses by row substitution,
// blocked WY solve in fp16. The anchors here are exclusive: block I's anchor
// is the gate total before the block, so every left factor (q 2^(G_r - E_aI),
// b 2^(E_r - E_aI)) and every cross factor 2^(E_aI - E_aJ) is <= 1 and every
// right factor (k or a times 2^(E_aJ - G_s)) lies in [1, 2^R_J], R_J the
// block's whole gate range (first row included). A range above GUARD switches
// the chunk to an exact elementwise path.
//
// Outputs (workspace, layouts in kda_common.h): Q+ (qp), K-^T V (km), A-^T (am),
// -W' (wn), -U' (u), A_qa (aqk), A_qk V (oh) and gamma = 2^G_last. The state
// recursion then runs the KDA chain with -u in place of V_new (see
// kda_recur.hip). Rows past the end of a sequence are zero (q = k = v = a =
// b = 0, log alpha = 0), which is exactly neutral for every factor.
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_prep_util.h"

#include <type_traits>

namespace kda {

// LDS plan (bytes).
//   R1: the right plane of k (split bf16, hi then lo); after the products the
//       lower blocks of A_ba (fp32), A_bk and A_qk (fp16); after the WY solve
//       the -W' staging. Slow path: the local scans [64][D] fp32.
//   R2: the right plane of a; after the products the B~ and V tiles
//       [D/16][4][64 lanes][4] fp16.
template <int D>
struct DplrSmem {
    static constexpr int KT_STRIDE = D + 8;                 // plane row (elements)
    static constexpr int KT_PLANE = 64 * KT_STRIDE;         // elements per hi / lo plane
    static constexpr int PLANE = 2 * KT_PLANE * 2;          // bytes of one split plane
    static constexpr int AKS = 20, AKB = 16 * AKS;          // fp32 block: row stride, floats per block
    static constexpr int AHS = 24, AHB = 16 * AHS;          // fp16 block: row stride, halfs per block
    static constexpr int ABA = 10 * AKB * 4;                // A_ba blocks (bytes)
    static constexpr int AH = 10 * AHB * 2;                 // A_bk or A_qk blocks (bytes)
    static constexpr int TILES = 64 * D * 2;                // one tile set (bytes)
    static constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
    static constexpr int R1 = max3(PLANE, ABA + 2 * AH, 64 * D * 4);
    static constexpr int R2 = PLANE > 2 * TILES ? PLANE : 2 * TILES;
    static constexpr int CONST = 18 * D * 4 > 4 * AKB * 4 ? 18 * D * 4 : 4 * AKB * 4;  // tot eA eL cIJ; later T_II
    static constexpr int BYTES = R1 + R2 + CONST + 16;      // + one overflow flag per wave
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
};

// The four gated products of one 16 x 16 block and one 32-deep slice. q and b
// (left, <= 1) are split by truncation (hi = top 16 bits exactly, lo = rest
// rounded); the right planes are split bf16 (hi, lo). A_qk, A_qa and A_bk,
// which reach the outputs through the value path, take three products each;
// A_ba, which only feeds the unit-lower inverse, takes the two with a_hi.
__device__ __forceinline__ void mma_dplr(f32x4_t& cqk, f32x4_t& cqa, f32x4_t& cbk, f32x4_t& cba,
                                         const float (&xq)[8], const float (&xb)[8],
                                         const APol<false>::Frag& fk, const APol<false>::Frag& fa) {
    u32x4_t qh, ql, bh, bl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t q0 = __float_as_uint(xq[2 * j]) & 0xffff0000u, q1 = __float_as_uint(xq[2 * j + 1]) & 0xffff0000u;
        const uint32_t b0 = __float_as_uint(xb[2 * j]) & 0xffff0000u, b1 = __float_as_uint(xb[2 * j + 1]) & 0xffff0000u;
        qh[j] = (q0 >> 16) | q1;
        bh[j] = (b0 >> 16) | b1;
        ql[j] = pack2bf(xq[2 * j] - __uint_as_float(q0), xq[2 * j + 1] - __uint_as_float(q1));
        bl[j] = pack2bf(xb[2 * j] - __uint_as_float(b0), xb[2 * j + 1] - __uint_as_float(b1));
    }
    const bf16x8_t qhi = __builtin_bit_cast(bf16x8_t, qh), qlo = __builtin_bit_cast(bf16x8_t, ql);
    const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, bh), blo = __builtin_bit_cast(bf16x8_t, bl);
    cqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo, fk.hi, cqk, 0, 0, 0);
    cqa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo, fa.hi, cqa, 0, 0, 0);
    cbk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(blo, fk.hi, cbk, 0, 0, 0);
    cba = __builtin_amdgcn_mfma_f32_16x16x32_bf16(blo, fa.hi, cba, 0, 0, 0);
    cqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, fk.lo, cqk, 0, 0, 0);
    cqa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, fa.lo, cqa, 0, 0, 0);
    cbk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bhi, fk.lo, cbk, 0, 0, 0);
    cba = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bhi, fa.hi, cba, 0, 0, 0);
    cqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, fk.hi, cqk, 0, 0, 0);
    cqa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, fa.hi, cqa, 0, 0, 0);
    cbk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bhi, fk.hi, cbk, 0, 0, 0);
}

// fp16 A operand over the 32-deep slice s of row block I from 16 x 16 fp16
// blocks (blocks above the diagonal are zero)
template <int AHS, int AHB>
__device__ __forceinline__ Pol<false>::Frag half_blocks_frag(const uint16_t* base, int I, int s, int n, int g) {
    u32x4_t x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int K = 2 * s + hf;
        if (K <= I) {
            const int blk = (K == I) ? I : 4 + pair_index(I, K);
            const u32x2_t u = *reinterpret_cast<const u32x2_t*>(base + blk * AHB + n * AHS + 4 * g);
            x[2 * hf] = u[0];
            x[2 * hf + 1] = u[1];
        }
    }
    Pol<false>::Frag f;
    f.v = __builtin_bit_cast(f16x8_t, x);
    return f;
}

// B operand over chunk rows 32 s .. 32 s + 31 of column tile ct from the
// accumulator-order tiles [ct][I][64 lanes][4] fp16
__device__ __forceinline__ Pol<false>::Frag tiles_frag(const uint16_t* tiles, int ct, int s, int l) {
    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(tiles + ((ct * 4 + 2 * s) * 64 + l) * 4);
    const u32x2_t b = *reinterpret_cast<const u32x2_t*>(tiles + ((ct * 4 + 2 * s + 1) * 64 + l) * 4);
    Pol<false>::Frag f;
    f.v = __builtin_bit_cast(f16x8_t, u32x4_t{a[0], a[1], b[0], b[1]});
    return f;
}

__device__ __forceinline__ u32x2_t pack4h(const f32x4_t& x, float sign) {
    u32x2_t pk;
    pk[0] = pack2h(sign * x[0], sign * x[1]);
    pk[1] = pack2h(sign * x[2], sign * x[3]);
    return pk;
}

template <int D, typename TG>
__global__ __launch_bounds__(256, 2) void dplr_prep_kernel(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                           const uint16_t* av, const uint16_t* bv, const TG* la,
                                                           const SeqMeta* __restrict__ tab, int N, int T, int H,
                                                           Ws<uint16_t> ws) {
    using P = Pol<false>;
    using E = uint16_t;
    using Frag = P::Frag;
    using AP = APol<false>;
    using AFrag = AP::Frag;
    using SM = DplrSmem<D>;
    constexpr int NS = D / 32, NCT = D / 16, TPW = NCT / 2;
    constexpr int KTS = SM::KT_STRIDE, AKS = SM::AKS, AKB = SM::AKB, AHS = SM::AHS, AHB = SM::AHB;

    extern __shared__ __align__(16) char smem[];
    E* Kt_s = reinterpret_cast<E*>(smem);                          // [2][64][KTS] k 2^(E_aJ - G)
    E* At_s = reinterpret_cast<E*>(smem + SM::R1);                 // [2][64][KTS] a 2^(E_aJ - G)
    float* xl_slow = reinterpret_cast<float*>(smem);               // slow path: [64][D] local scans
    float* Aba_s = reinterpret_cast<float*>(smem);                 // 10 fp32 blocks: diag I at I, (I,J) at 4+pair
    E* Abk_s = reinterpret_cast<E*>(smem + SM::ABA);               // 10 fp16 blocks, same numbering
    E* Aqk_s = Abk_s + 10 * AHB;                                   // 10 fp16 blocks
    E* Ws_s = reinterpret_cast<E*>(smem);                          // [64][NS][32] -W' staging
    E* Bt_t = reinterpret_cast<E*>(smem + SM::R1);                 // B~ tiles
    E* Vt_t = Bt_t + 64 * D;                                       // V tiles
    float* cst = reinterpret_cast<float*>(smem + SM::R1 + SM::R2);
    float* tot = cst;          // [4][D] block totals of the log2 gate
    float* eA = tot + 4 * D;   // [4][D] 2^E_aI (gate before block I)
    float* eL = eA + 4 * D;    // [4][D] 2^(G_last - E_aI)
    float* cIJ = eL + 4 * D;   // [6][D] 2^(E_aI - E_aJ), I > J
    float* Td_s = cst;         // [4][16][AKS] T_II, once the constants are dead
    int* slow_s = reinterpret_cast<int*>(smem + SM::R1 + SM::R2 + SM::CONST);

    const int gc = blockIdx.x / H;
    const int h = blockIdx.x - gc * H;
    ChunkLoc loc;
    if (!locate_chunk(tab, N, T, gc, loc)) return;
    const int t0 = loc.t0, L = loc.L;
    const int64_t chh = (int64_t)gc * H + h;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
    const int r = 16 * w + n;
    const bool valid = r < L;
    const int64_t rowoff = ((int64_t)(t0 + r) * H + h) * D;
    const int64_t ldoff = valid ? rowoff : ((int64_t)t0 * H + h) * D;

    // ---- 0. row inputs (raw; converted where used). v is loaded later.
    RowRaw<TG, NS> rla;
    RowRaw<uint16_t, NS> rq, rk, ra, rb;
    rla.load(la, ldoff, g);
    rq.load(q, ldoff, g);
    rk.load(k, ldoff, g);
    ra.load(av, ldoff, g);
    rb.load(bv, ldoff, g);
    asm volatile("" ::: "memory");
    float xl[NS][8];
    rla.get(xl, valid, LOG2E);

    // ---- 1. log2 gate scanned inside each 16-row block
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) xl[s][j] += dpp_shr(xl[s][j], d);
    }
    if (n == 15) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            *reinterpret_cast<f32x4_t*>(tot + w * D + 32 * s + 4 * g) = f32x4_t{xl[s][0], xl[s][1], xl[s][2], xl[s][3]};
            *reinterpret_cast<f32x4_t*>(tot + w * D + 32 * s + 16 + 4 * g) =
                f32x4_t{xl[s][4], xl[s][5], xl[s][6], xl[s][7]};
        }
    }
    __syncthreads();

    // ---- 2. per-block channel constants from block totals, and the overflow guard
    int bad = 0;
    {
        constexpr int PP = 256 / D;
        const int c = tid % D, part = tid / D;
        float tt[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) tt[I] = tot[I * D + c];
#pragma unroll
        for (int ty = 0; ty < 15; ++ty) {
            if (ty % PP != part) continue;
            if (ty < 4) {  // 2^(sum_{K<I} tot_K)
                float e = 0.f;
                for (int K = 0; K < ty; ++K) e += tt[K];
                eA[ty * D + c] = ex2(e);
            } else if (ty < 8) {  // 2^(sum_{K>=I} tot_K)
                const int I = ty - 4;
                float e = 0.f;
                for (int K = I; K < 4; ++K) e += tt[K];
                eL[I * D + c] = ex2(e);
            } else if (ty < 14) {  // 2^(sum_{J<=K<I} tot_K)
                const int p = ty - 8;
                const int I = p < 1 ? 1 : (p < 3 ? 2 : 3);
                const int J = p - pair_index(I, 0);
                float e = 0.f;
                for (int K = J; K < I; ++K) e += tt[K];
                cIJ[p * D + c] = ex2(e);
            } else {
                ws.gam[chh * D + c] = ex2(tt[0] + tt[1] + tt[2] + tt[3]);
            }
        }
        if (part == 0) {
#pragma unroll
            for (int I = 0; I < 4; ++I) bad |= !(-tt[I] <= GUARD);
        }
    }
    const bool wave_bad = __ballot(bad) != 0;
    if (l == 0) slow_s[w] = wave_bad;
    __syncthreads();
    const bool slow = (slow_s[0] | slow_s[1] | slow_s[2] | slow_s[3]) != 0;

    // 0/1 selectors for the matrix-core transposes (see kda_prep.hip)
    Frag sel[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = (g == (n >> 2) && jj == 4 * hf + (n & 3)) ? 1.f : 0.f;
        sel[hf] = P::make(x);
    }
    // one slice s of a lane-per-row vector, transposed: to a [D][64] workspace
    // array in the split row order (to_km) or to accumulator tiles in LDS
    auto tr_slice = [&](const float (&x)[8], int s, auto to_km, E* dst) {
        const Frag a = P::make(x);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            f32x4_t t = {0.f, 0.f, 0.f, 0.f};
            P::mma(t, a, sel[hf]);
            const u32x2_t pk = pack4h(t, 1.f);
            if constexpr (decltype(to_km)::value)
                *reinterpret_cast<u32x2_t*>(dst + (32 * s + 16 * hf + n) * 64 + 32 * (w >> 1) + 8 * g + 4 * (w & 1)) = pk;
            else
                *reinterpret_cast<u32x2_t*>(dst + (((2 * s + hf) * 4 + w) * 64 + l) * 4) = pk;
        }
    };

    // ---- 3. gated scalings
    float qs[NS][8], bs[NS][8];  // left factors q 2^(G - E_aw), b 2^(E - E_aw) (fast path); b 2^E (slow)
    E* qp_out = ws.qp + chh * 64 * D;
    // K-^T goes to the start of this chunk-head's K-^T V array, as scratch: it is
    // read back (by other waves) once every wave is past the barriers below,
    // and the product overwrites it
    E* km_out = ws.km + chh * D * D;
    E* am_out = ws.am + chh * D * 64;
    if (!slow) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float ea8[8], el8[8], ktv[8], atv[8], kmv[8], amv[8], qpv[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int c0 = 32 * s + 16 * hf + 4 * g;
                const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(eA + w * D + c0);
                const f32x4_t c4 = *reinterpret_cast<const f32x4_t*>(eL + w * D + c0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ea8[4 * hf + j] = b4[j];
                    el8[4 * hf + j] = c4[j];
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = rla.at(s, j, valid) * LOG2E;  // the value the scan started from
                const float e = ex2(xl[s][j]);                 // 2^(G_r - E_aw) <= 1
                const float ee = ex2(xl[s][j] - x);            // 2^(E_r - E_aw) <= 1
                const float ei = ex2(-xl[s][j]);               // 2^(E_aw - G_r) >= 1
                qs[s][j] = rq.at(s, j, valid) * e;
                bs[s][j] = rb.at(s, j, valid) * ee;
                ktv[j] = rk.at(s, j, valid) * ei;
                atv[j] = ra.at(s, j, valid) * ei;
                qpv[j] = qs[s][j] * ea8[j];
                kmv[j] = ktv[j] * el8[j];
                amv[j] = atv[j] * el8[j];
            }
            tr_slice(kmv, s, std::true_type{}, km_out);
            tr_slice(amv, s, std::true_type{}, am_out);
            AP::store(Kt_s + r * KTS + s * 32 + g * 8, SM::KT_PLANE, AP::make(ktv));
            AP::store(At_s + r * KTS + s * 32 + g * 8, SM::KT_PLANE, AP::make(atv));
            P::store(qp_out + (r * NS + s) * 32 + g * 8, P::make(qpv));
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float kmv[8], amv[8], qpv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 32 * s + kslot(g, j);
                float pre = 0.f, post = tot[w * D + c] - xl[s][j];
                for (int J = 0; J < w; ++J) pre += tot[J * D + c];
                for (int J = w + 1; J < 4; ++J) post += tot[J * D + c];
                const float x = rla.at(s, j, valid) * LOG2E;
                const float dec = exp2f(post);  // 2^(G_last - G_r)
                qpv[j] = rq.at(s, j, valid) * exp2f(pre + xl[s][j]);
                bs[s][j] = rb.at(s, j, valid) * exp2f(pre + xl[s][j] - x);
                kmv[j] = rk.at(s, j, valid) * dec;
                amv[j] = ra.at(s, j, valid) * dec;
                qs[s][j] = 0.f;
                xl_slow[r * D + c] = xl[s][j];
            }
            tr_slice(kmv, s, std::true_type{}, km_out);
            tr_slice(amv, s, std::true_type{}, am_out);
            P::store(qp_out + (r * NS + s) * 32 + g * 8, P::make(qpv));
        }
    }
    RowRaw<uint16_t, NS> rv;  // values: needed only after the products
    rv.load(v, ldoff, g);
    asm volatile("" ::: "memory");
    __syncthreads();

    // ---- 4. the four gated matrices. Wave I computes blocks (I, J <= I).
    // A_qa goes straight to the workspace; A_qk, A_bk, A_ba stay in registers
    // until the planes are dead.
    E* aqa_out = ws.aqk + chh * 64 * 64;
    auto aqa_put = [&](int rr, int cc, float x) {
        const int s2 = cc >> 5, c2 = cc & 31;
        aqa_out[(rr * 2 + s2) * 32 + 8 * ((c2 & 15) >> 2) + 4 * (c2 >> 4) + (c2 & 3)] = f2h(x);
    };
    f32x4_t cqk[4], cbk[4], cba[4];
    auto products = [&](auto Ic) {
        constexpr int I = decltype(Ic)::value;
        f32x4_t cqa[I + 1];
#pragma unroll
        for (int J = 0; J <= I; ++J) {
            cqk[J] = cbk[J] = cba[J] = cqa[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const AFrag fk = AP::load(Kt_s + (16 * J + n) * KTS + s * 32 + g * 8, SM::KT_PLANE);
                const AFrag fa = AP::load(At_s + (16 * J + n) * KTS + s * 32 + g * 8, SM::KT_PLANE);
                f32x4_t c0 = {1.f, 1.f, 1.f, 1.f}, c1 = {1.f, 1.f, 1.f, 1.f};
                if (J < I) {
                    const float* cp = cIJ + pair_index(I, J) * D + 32 * s + 4 * g;
                    c0 = *reinterpret_cast<const f32x4_t*>(cp);
                    c1 = *reinterpret_cast<const f32x4_t*>(cp + 16);
                }
                float xq[8], xb[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xq[j] = qs[s][j] * c0[j];
                    xb[j] = bs[s][j] * c0[j];
                    xq[4 + j] = qs[s][4 + j] * c1[j];
                    xb[4 + j] = bs[s][4 + j] * c1[j];
                }
                mma_dplr(cqk[J], cqa[J], cbk[J], cba[J], xq, xb, fk, fa);
            }
        }
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * g + i;
                const bool incl = (J < I) || (J == I && n <= rl);
                aqa_put(16 * I + rl, 16 * J + n, (J <= I && incl) ? cqa[J <= I ? J : 0][i] : 0.f);
            }
    };
    if (!slow) {
        switch (w) {
            case 0: products(std::integral_constant<int, 0>{}); break;
            case 1: products(std::integral_constant<int, 1>{}); break;
            case 2: products(std::integral_constant<int, 2>{}); break;
            default: products(std::integral_constant<int, 3>{}); break;
        }
    }
    // slow path: every product exactly, pair (rr, ii) = (p >> 6, p & 63), p = tid + 256 m
    float sl_qk[16], sl_bk[16], sl_ba[16];
    if (slow) {
#pragma unroll 1
        for (int m = 0; m < 16; ++m) {
            const int p = tid + 256 * m;
            const int rr = p >> 6, ii = p & 63;
            float sqk = 0.f, sqa = 0.f, sbk = 0.f, sba = 0.f;
            if (ii <= rr && rr < L) {
                const int I = rr >> 4, J = ii >> 4;
                const int64_t ro = ((int64_t)(t0 + rr) * H + h) * D;
                const int64_t io = ((int64_t)(t0 + ii) * H + h) * D;
                for (int c = 0; c < D; ++c) {
                    float ex = xl_slow[rr * D + c] - xl_slow[ii * D + c];  // G_rr - G_ii
                    for (int K = J; K < I; ++K) ex += tot[K * D + c];
                    const float fq = exp2f(ex);
                    const float kv = ld_in(k, io + c), avv = ld_in(av, io + c);
                    const float qv = ld_in(q, ro + c);
                    sqk += qv * kv * fq;
                    sqa += qv * avv * fq;
                    if (ii < rr) {
                        const float fb = exp2f(ex - ld_in(la, ro + c) * LOG2E);  // 2^(E_rr - G_ii) <= 1
                        const float bvv = ld_in(bv, ro + c);
                        sbk += bvv * kv * fb;
                        sba += bvv * avv * fb;
                    }
                }
            }
            aqa_put(rr, ii, sqa);
            sl_qk[m] = sqk;
            sl_bk[m] = sbk;
            sl_ba[m] = sba;
        }
    }
    __syncthreads();

    // ---- 5. blocks to R1, B~ and V tiles to R2 (both planes are dead now)
    if (!slow) {
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J > w) continue;
            const int blk = (J == w) ? w : 4 + pair_index(w, J);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * g + i;
                const bool incl = (J < w) || (n <= rl), strict = (J < w) || (n < rl);
                Aba_s[blk * AKB + rl * AKS + n] = strict ? cba[J][i] : 0.f;
                Abk_s[blk * AHB + rl * AHS + n] = f2h(strict ? cbk[J][i] : 0.f);
                Aqk_s[blk * AHB + rl * AHS + n] = f2h(incl ? cqk[J][i] : 0.f);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int p = tid + 256 * m;
            const int rr = p >> 6, ii = p & 63, I = rr >> 4, J = ii >> 4;
            if (J <= I) {
                const int blk = (J == I) ? I : 4 + pair_index(I, J);
                const int o32 = blk * AKB + (rr & 15) * AKS + (ii & 15);
                const int o16 = blk * AHB + (rr & 15) * AHS + (ii & 15);
                Aba_s[o32] = sl_ba[m];
                Abk_s[o16] = f2h(sl_bk[m]);
                Aqk_s[o16] = f2h(sl_qk[m]);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        float btv[8], vv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 32 * s + kslot(g, j);
            btv[j] = slow ? bs[s][j] : bs[s][j] * eA[w * D + c];
            vv[j] = rv.at(s, j, valid);
        }
        tr_slice(btv, s, std::false_type{}, Bt_t);
        tr_slice(vv, s, std::false_type{}, Vt_t);
    }
    __syncthreads();

    // ---- 6. diagonal-block inverses T_II = (I + A_ba,II)^-1 by row substitution (wave 0)
    if (w == 0) {
        const int b = l >> 4, j = l & 15;
        float acc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[rr] = (rr == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ti = acc[i];
#pragma unroll
            for (int rr = i + 1; rr < 16; ++rr) acc[rr] -= Aba_s[b * AKB + rr * AKS + i] * ti;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Td_s[b * AKB + rr * AKS + j] = acc[rr];
    }
    __syncthreads();

    // ---- 7. blocked substitution on the matrix cores. Waves 0-1: W' = T B~ and
    // A_qk V; waves 2-3: U' = T (A_bk V). Four column tiles per wave.
    const bool isW = w < 2;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    E* u_out = ws.u + chh * 64 * D;
    E* oh_out = ws.oh + chh * 64 * D;
    f32x4_t X[TPW][4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        Frag aoff[2];  // -A_ba[I, K], K < I
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (2 * s >= I) break;
            float xa[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int K = 2 * s + hf;
                if (K < I) {
                    const f32x4_t a4 =
                        *reinterpret_cast<const f32x4_t*>(Aba_s + (4 + pair_index(I, K)) * AKB + n * AKS + 4 * g);
#pragma unroll
                    for (int j = 0; j < 4; ++j) xa[4 * hf + j] = -a4[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) xa[4 * hf + j] = 0.f;
                }
            }
            aoff[s] = P::make(xa);
        }
        Frag at;
        {
            const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(Td_s + I * AKB + n * AKS + 4 * g);
            float ta[8] = {a4[0], a4[1], a4[2], a4[3], 0.f, 0.f, 0.f, 0.f};
            at = P::make(ta);
        }
        Frag av2[2];  // A_qk[I, K] (waves 0-1) or A_bk[I, K] (waves 2-3), K <= I
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (2 * s > I) break;
            av2[s] = half_blocks_frag<AHS, AHB>(isW ? Aqk_s : Abk_s, I, s, n, g);
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int ct = (w & 1) * TPW + tt;
            f32x4_t Y, Z = zero;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (2 * s > I) break;
                P::mma(Z, av2[s], tiles_frag(Vt_t, ct, s, l));
            }
            if (isW) {
                const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(Bt_t + ((ct * 4 + I) * 64 + l) * 4);
                Y = f32x4_t{h2f(bb[0] & 0xffffu), h2f(bb[0] >> 16), h2f(bb[1] & 0xffffu), h2f(bb[1] >> 16)};
                *reinterpret_cast<u32x2_t*>(oh_out + ((ct * 4 + I) * 64 + l) * 4) = pack4h(Z, 1.f);
            } else {
                Y = Z;
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (2 * s >= I) break;
                P::mma(Y, aoff[s], frag_from_acc<false>(X[tt][2 * s], (2 * s + 1 < I) ? X[tt][2 * s + 1] : zero));
            }
            X[tt][I] = zero;
            P::mma(X[tt][I], at, frag_from_acc<false>(Y, zero));
            if (!isW) *reinterpret_cast<u32x2_t*>(u_out + ((ct * 4 + I) * 64 + l) * 4) = pack4h(X[tt][I], -1.f);
        }
    }
    // ---- 8. the state update's state-independent part K-^T V, dk x dv: wave w
    // takes row tiles t = w * NT/4 .. and every column tile; K-^T (scratch,
    // written before several barriers) as A operands, the V tiles as B
    constexpr int TW = NCT / 4;  // row tiles per wave
    f32x4_t kvt[TW][NCT];
    {
        Frag ka[TW][2];
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s) ka[i][s] = P::load(km_out + ((16 * (w * TW + i) + n) * 2 + s) * 32 + g * 8);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const Frag b0 = tiles_frag(Vt_t, ct, 0, l), b1 = tiles_frag(Vt_t, ct, 1, l);
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                kvt[i][ct] = zero;
                P::mma(kvt[i][ct], ka[i][0], b0);
                P::mma(kvt[i][ct], ka[i][1], b1);
            }
        }
    }
    __syncthreads();  // every block and tile read, the K-^T scratch too: R1 takes the -W' staging
    {
        // K-^T V in [column tile][row tile][64 lanes][4]: one slab's share is 4 D bytes, contiguous
        E* kv_out = ws.km + chh * D * D;
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                *reinterpret_cast<u32x2_t*>(kv_out + ((ct * NCT + w * TW + i) * 64 + l) * 4) = pack4h(kvt[i][ct], 1.f);
    }
    if (isW) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int ct = (w & 1) * TPW + tt;
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * I + 4 * g + i;
                    const int s = ct >> 1, gg = n >> 2, jj = 4 * (ct & 1) + (n & 3);
                    Ws_s[(rr * NS + s) * 32 + gg * 8 + jj] = f2h(-X[tt][I][i]);
                }
        }
    }
    __syncthreads();
    {
        E* wn_out = ws.wn + chh * 64 * D;
        for (int idx = tid; idx < 64 * D / 8; idx += 256)
            reinterpret_cast<u32x4_t*>(wn_out)[idx] = reinterpret_cast<const u32x4_t*>(Ws_s)[idx];
    }
}

template <int D, typename TG>
static hipError_t launch_dplr_prep_t(const ChunkArgs& a, hipStream_t st) {
    using E = uint16_t;
    using SM = DplrSmem<D>;
    Ws<E> ws{(E*)a.qp, (E*)a.km, (E*)a.wn, (E*)a.u, (E*)a.aqk, a.gam, nullptr, nullptr, (E*)a.am, (E*)a.oh};
    auto kern = dplr_prep_kernel<D, TG>;
    const hipError_t e = allow_dynamic_lds((const void*)kern, SM::BYTES);
    if (e != hipSuccess) return e;
    dim3 grid(a.NC * a.H), block(256);  // NC * H < 2^31 (checked by the caller)
    hipLaunchKernelGGL(kern, grid, block, SM::BYTES, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.lr_a, (const uint16_t*)a.lr_b, (const TG*)a.la,
                       a.tab, a.N, a.T, a.H, ws);
    return hipGetLastError();
}

hipError_t launch_dplr_prep(const ChunkArgs& a, hipStream_t st) {
    if (a.D == 128)
        return a.gate_f32 ? launch_dplr_prep_t<128, float>(a, st) : launch_dplr_prep_t<128, uint16_t>(a, st);
    return a.gate_f32 ? launch_dplr_prep_t<64, float>(a, st) : launch_dplr_prep_t<64, uint16_t>(a, st);
}

}  // namespace kda
