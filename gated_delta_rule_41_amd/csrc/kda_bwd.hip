// Backward of the chunkwise KDA prefill: dq, dk, dv, dlog_alpha, dbeta and the
// initial states' gradient, given the gradients of o and of the final states.
//
// The pages present the chunkwise form as a training algorithm (GeekNews "Kimi
// Linear" summary, section "Algoritmo paralelo por chunks"); its backward
// follows from the chunk equations by reverse-mode differentiation:
//
//   forward, per chunk:  V = U - W h,  O = Q+ h + A_qk V,  h' = Diag(gamma) h + K-^T V
//   backward:            dV = A_qk^T dO + K- dh',  dh = Diag(gamma) dh' + Q+^T dO - W^T dV
//
// The state gradient runs backwards over the chunks with the forward chain's
// shape (two dependent products per chunk), so it reuses the state-recursion
// kernel, walking each sequence's chunks in reverse, with K- in place of -W
// and (-W)^T in place of K-^T (read transposed from the forward's own arrays),
// A_qk^T dO in place of U and the state-independent term Q+^T dO added each
// chunk (bwd_prep_kernel computes these two). What stays is
// chunk-local and parallel over chunks (bwd_local_kernel):
//   * the adjoints of the output and the state update: dQ+ = dO h^T,
//     dA_qk = tril(dO V^T), dK- = V dh'^T, dgamma = rowsum(h * dh'),
//     dW = -dV h^T;
//   * the UT transform X = [W | U] = T B with T = (I + A_kk)^-1 and
//     B = [beta K+ | beta V]: dB = T^T dX and, since dT = dX B^T,
//     dA_kk = -T^T dX B^T T^T = -dB X^T on the strictly lower part;
//   * the gated products P[r,i] = sum_c x_rc y_ic e^(g_rc - g_ic): for 16-row
//     blocks below the diagonal the exponential splits at a row between the
//     two blocks (every factor e^(.) <= 1 for decaying gates, so nothing
//     overflows, and an underflowing factor only drops a term smaller than
//     itself) and the adjoints are matrix-core products; the four diagonal
//     blocks are summed pair by pair with the exact exponential;
//   * the gated scalings, then a reverse cumulative sum over the chunk turns the
//     gate gradient into dlog_alpha.
//
// Everything runs in fp32, the products on the matrix cores (16 x 16 x 4 fp32):
// the forward is recomputed with fp32 factors (the prep and recursion kernels'
// fp32 path, which keeps h_n, V_new and the gated key products).
//
// Product convention (v_mfma_f32_16x16x4f32): lane l = 16 G + n supplies A[n][k]
// and B[k][n] for the k of its lane group G; the accumulator holds C[4 G + i][n],
// i < 4. Over four consecutive products lane group G takes k = 4 G + t at step t
// (A and B agree on it), so one 16-byte read per lane feeds four products, and
// an accumulator tile feeds a later product as its B operand unchanged.
//
// Every cross-lane or cross-wave sum runs in a fixed order: the results are
// bitwise repeatable.
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_prep_util.h"

namespace kda {

// row (of a 32-row slice) of element jj held by B-operand fragment lane group g,
// in the fp32 recursion's fragment arrays: h [D/16][D/32][64 lanes][8] and
// V_new [D/16][2][64 lanes][8]
__device__ __forceinline__ int frag_row(int g, int jj) { return 16 * (jj >> 2) + 4 * g + (jj & 3); }
// row-major [rows][ncol] array with columns in the split order per 32
__device__ __forceinline__ int split_index(int row, int col, int ncol) {
    return row * ncol + 32 * (col >> 5) + split_pos(col);
}
// channel stored at position p of a split-ordered row (inverse of split_pos)
__device__ __forceinline__ int split_chan(int p) {
    const int q = p & 31;
    return (p & ~31) + 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
}

__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// acc += sum over 16 k of A[.][k] B[.][k], both read as 4 consecutive k per lane
__device__ __forceinline__ void mma16(f32x4_t& acc, const float* a, const float* b) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(a);
    const f32x4_t y = *reinterpret_cast<const f32x4_t*>(b);
    acc = mfma4(x[0], y[0], acc);
    acc = mfma4(x[1], y[1], acc);
    acc = mfma4(x[2], y[2], acc);
    acc = mfma4(x[3], y[3], acc);
}
// the same with the B operand's four k values in registers
__device__ __forceinline__ void mma16b(f32x4_t& acc, const float* a, const f32x4_t& y) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(a);
    acc = mfma4(x[0], y[0], acc);
    acc = mfma4(x[1], y[1], acc);
    acc = mfma4(x[2], y[2], acc);
    acc = mfma4(x[3], y[3], acc);
}
// Transpose of a 16 x 16 fp32 tile held in accumulator layout (lane n + 16 G:
// rows 4 G + i of column n) into the same layout of its transpose, on the
// matrix cores (a product with the identity: exact up to NaN/infinity
// spreading, as above)
__device__ __forceinline__ f32x4_t tr16(const f32x4_t& x, int l) {
    const int G = l >> 4, n = l & 15;
    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) a = mfma4(x[t], 4 * G + t == n ? 1.f : 0.f, a);
    return a;
}
// e^x for x formed as a difference of cumulative gates (natural log units): the
// sums of 16-bit gates are exact in fp32, so is their difference, and the one
// rounding left is that of x * log2 e
__device__ __forceinline__ float ee(float x) { return ex2(x * LOG2E); }
__device__ __forceinline__ float sum16(float x) {  // over the 16 lanes n of a lane group
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// ---------------------------------------------------------------------------
// Rows of a [T, H, D] array <-> the own-element layout (lane n + 16 G of wave w:
// channel 16 w + n of rows 16 R + 4 G + i, as one f32x4 per row block R),
// through the matrix cores: each lane moves 16 bytes of one row, and a product
// with a 0/1 selector puts every element where the other layout wants it
// (exact: one input times 1 plus zeros; a NaN or infinity among a tile's 16
// channels spreads through the zero products to the rest of its row). Rows at
// or past L read as zeros and are not stored.
template <typename T> struct OwnRows;
template <> struct OwnRows<uint16_t> {  // bf16: lane loads 8 channels of its 32-channel slice
    using Raw = u32x4_t;
    static __device__ __forceinline__ int64_t col(int w, int G) { return 32 * (w >> 1) + 8 * G; }
    static __device__ __forceinline__ void to_own(const Raw (&raw)[4], int w, int l, f32x4_t (&out)[4]) {
        const int G = l >> 4, n = l & 15, own = 16 * (w & 1) + n;
        u32x4_t sv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            sv[jj] = (8 * G + 2 * jj == own ? 0x3F80u : 0u) | (8 * G + 2 * jj + 1 == own ? 0x3F800000u : 0u);
        const bf16x8_t sb = __builtin_bit_cast(bf16x8_t, sv);
#pragma unroll
        for (int R = 0; R < 4; ++R)
            out[R] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, raw[R]), sb,
                                                             f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
};
template <> struct OwnRows<float> {  // fp32: lane loads 4 channels of its wave's 16
    using Raw = f32x4_t;
    static __device__ __forceinline__ int64_t col(int w, int G) { return 16 * w + 4 * G; }
    static __device__ __forceinline__ void to_own(const Raw (&raw)[4], int w, int l, f32x4_t (&out)[4]) {
        const int G = l >> 4, n = l & 15;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) a = mfma4(raw[R][t], 4 * G + t == n ? 1.f : 0.f, a);
            out[R] = a;
        }
    }
};
// issue the loads of rows 16 R + n (the lane's row of each block) of head h
template <typename T>
__device__ __forceinline__ void own_load(const T* p, int t0, int L, int H, int h, int D, int w, int l,
                                         typename OwnRows<T>::Raw (&raw)[4]) {
    using Raw = typename OwnRows<T>::Raw;
    const int n = l & 15;
    const int64_t cc = OwnRows<T>::col(w, l >> 4);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const int r = 16 * R + n;
        raw[R] = *reinterpret_cast<const Raw*>(p + ((int64_t)(t0 + (r < L ? r : 0)) * H + h) * D + cc);
    }
#pragma unroll
    for (int R = 0; R < 4; ++R)
        if (16 * R + n >= L) raw[R] = Raw{};
}
// own tiles -> 16-byte row stores (fp32 outputs)
__device__ __forceinline__ void own_store(float* p, int t0, int L, int H, int h, int D, int w, int l,
                                          const f32x4_t (&x)[4]) {
    const int G = l >> 4, n = l & 15;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) a = mfma4(x[R][t], 4 * G + t == n ? 1.f : 0.f, a);
        // lane n + 16 G: row 16 R + n, channels 16 w + 4 G .. + 3
        if (16 * R + n < L)
            *reinterpret_cast<f32x4_t*>(p + ((int64_t)(t0 + 16 * R + n) * H + h) * D + 16 * w + 4 * G) = a;
    }
}

// ---------------------------------------------------------------------------
// The state-gradient recursion's per-chunk operands for chunk slot gc:
// U := A_qk^T dO (accumulator tiles [dv/16][4][64 lanes][4]) and the added term
// P = Q+^T dO ([dv/16][dk/16][64 lanes][4]). Wave w owns value columns
// 16 w .. 16 w + 15. The chunk's rows pass through LDS in two halves of 32
// (the second half's loads in flight during the first half's products), so a
// workgroup holds 42.5 KiB and three fit on a CU; the products still run over
// the rows in order, so the result is that of one 64-row pass.
template <int D>
struct BwdPrepSmem {
    static constexpr int RS = D + 4, SQS = 68, RH = 32;  // row strides; rows per half
    static constexpr int BYTES = (2 * RH * RS + RH * SQS) * 4;
};

template <int D>
__global__ __launch_bounds__(4 * D) void bwd_prep_kernel(const SeqMeta* __restrict__ tab, int N, int T, int H,
                                                         int g0, Ws<float> f, Ws<float> b,
                                                         const float* __restrict__ d_o) {
    constexpr int NT = D / 16, NTH = 4 * D, RS = BwdPrepSmem<D>::RS, SQS = BwdPrepSmem<D>::SQS;
    constexpr int RH = BwdPrepSmem<D>::RH;
    constexpr int NQ = RH * D / 4 / NTH;      // float4 per thread of a [32][D] half (= 2)
    constexpr int NA = RH * 64 / 4 / NTH;     // ... of a [32][64] half (1 or 2)
    extern __shared__ __align__(16) float sm[];
    float* dO = sm;                // [32][RS]
    float* Qp = dO + RH * RS;      // [32][RS], channels in natural order
    float* Aq = Qp + RH * RS;      // [32][SQS] rows of A_qk
    const int lc = blockIdx.x / H, h = blockIdx.x - lc * H;  // slot g0 + lc, workspace slot lc
    ChunkLoc loc;
    if (!locate_chunk(tab, N, T, g0 + lc, loc)) return;
    const int64_t src = (int64_t)lc * H + h;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, G = l >> 4, n = l & 15;
    f32x4_t xo[NQ], xq[NQ], xa[NA];
    auto load_half = [&](int hf) {  // every load of the half, into registers
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int e = tid + NTH * m, r = RH * hf + e / (D / 4), c4 = 4 * (e - (e / (D / 4)) * (D / 4));
            xo[m] = r < loc.L ? *reinterpret_cast<const f32x4_t*>(d_o + ((int64_t)(loc.t0 + r) * H + h) * D + c4)
                              : f32x4_t{0.f, 0.f, 0.f, 0.f};
            xq[m] = *reinterpret_cast<const f32x4_t*>(f.qp + src * 64 * D + (int64_t)RH * D * hf + 4 * e);
        }
#pragma unroll
        for (int m = 0; m < NA; ++m)
            xa[m] = *reinterpret_cast<const f32x4_t*>(f.aqk + src * 64 * 64 + RH * 64 * hf + 4 * (tid + NTH * m));
    };
    auto store_half = [&]() {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int e = tid + NTH * m, r = e / (D / 4), c4 = 4 * (e - r * (D / 4));
            *reinterpret_cast<f32x4_t*>(dO + r * RS + c4) = xo[m];
#pragma unroll
            for (int j = 0; j < 4; ++j) Qp[r * RS + split_chan(c4 + j)] = xq[m][j];
        }
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            const int e = tid + NTH * m, r = e >> 4, p = 4 * (e & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) Aq[r * SQS + split_chan(p + j)] = xa[m][j];
        }
    };
    const int j0 = 16 * w;
    // P[c][j] = sum_r Q+[r][c] dO[r][j]; U[r][j] = sum_{i >= r} A_qk[i][r] dO[i][j]
    f32x4_t accP[NT], accU[4];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) accP[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int R = 0; R < 4; ++R) accU[R] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // rows 4 kk + G of the chunk, kk in [8 hf, 8 hf + 8), from the half in LDS
    auto products = [&](int hf) {
#pragma unroll 4
        for (int k8 = 0; k8 < 8; ++k8) {
            const int kk = 8 * hf + k8, r = 4 * k8 + G;  // r: the row inside the half
            const float bo = dO[r * RS + j0 + n];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) accP[ct] = mfma4(Qp[r * RS + 16 * ct + n], bo, accP[ct]);
#pragma unroll
            for (int R = 0; R < 4; ++R)
                if (R <= (kk >> 2)) accU[R] = mfma4(Aq[r * SQS + 16 * R + n], bo, accU[R]);
        }
    };
    load_half(0);
    store_half();
    __syncthreads();
    load_half(1);
    products(0);
    __syncthreads();  // the first half is read
    store_half();
    __syncthreads();
    products(1);
    float* pb = const_cast<float*>(b.pb) + src * D * D;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) *reinterpret_cast<f32x4_t*>(pb + ((w * NT + ct) * 64 + l) * 4) = accP[ct];
#pragma unroll
    for (int R = 0; R < 4; ++R)
        *reinterpret_cast<f32x4_t*>(b.u + src * 64 * D + ((w * 4 + R) * 64 + l) * 4) = accU[R];
}

// ---------------------------------------------------------------------------
// Chunk-local adjoints, one workgroup of D/16 waves per (chunk, head). Wave w
// owns key/value channels c = 16 w + n (lane n of each lane group); lane group
// G owns rows 16 R + 4 G + i (R, i < 4) of them: the "own" elements, which is
// the accumulator layout of a 64-row product tile, so every per-channel sum
// over rows stays inside a wave.
template <int D>
struct BwdSmem {
    static constexpr int NW = D / 16;
    static constexpr int RS = D + 4;          // [rows][D] matrices
    static constexpr int RX = 2 * D + 4;      // dB = [dB_k | dB_v]
    static constexpr int SQS = 68;            // [64][64] matrices
    // phase 0: dV then V [64][RS] at 0, dO [64][RS] (h and dh' stay in registers);
    // later: T^T (stride SQS), -W, -U [64][RS] at 0, dB [64][RX], P_kk then dP_kk [64][SQS]
    static constexpr int R_VV = 0, R_DO = R_VV + 64 * RS;
    static constexpr int R_DB = 64 * RS, R_PK = R_DB + 64 * RX;
    static constexpr int PH0_END = R_DO + 64 * RS, LATER_END = R_PK + 64 * SQS;
    static constexpr int R_DPQ = PH0_END > LATER_END ? PH0_END : LATER_END;  // dA_qk, kept to the end
    static constexpr int R_SMALL = R_DPQ + 64 * SQS;
    // small: beta [64], dbeta partials [NW][64] and [4][64]
    static constexpr int FLOATS = R_SMALL + 64 + NW * 64 + 4 * 64;
    static constexpr int BYTES = FLOATS * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(64 * SQS <= R_DB, "T^T below dB");
};

template <int D, typename TIn, typename TG>
__global__ __launch_bounds__(4 * D) void bwd_local_kernel(const TIn* q, const TIn* k, const TIn* v, const TG* la,
                                                          const TG* beta, const SeqMeta* __restrict__ tab, int N,
                                                          int T, int H, int g0, Ws<float> f, Ws<float> b,
                                                          const float* __restrict__ d_o, float* __restrict__ scr,
                                                          float* __restrict__ dq, float* __restrict__ dk,
                                                          float* __restrict__ dv, float* __restrict__ dla,
                                                          float* __restrict__ dbeta) {
    using SM = BwdSmem<D>;
    constexpr int NW = SM::NW, NTH = 64 * NW, NS = D / 32, RS = SM::RS, RX = SM::RX, SQS = SM::SQS;
    extern __shared__ __align__(16) float sm[];
    float* VV = sm + SM::R_VV;         // dV, then V
    float* DO = sm + SM::R_DO;         // dO
    float* TT = sm;                    // T^T (stride SQS), then -W, then -U (stride RS)
    float* DB = sm + SM::R_DB;         // [64][RX]
    float* PK = sm + SM::R_PK;         // P_kk, then dP_kk
    float* DPQ = sm + SM::R_DPQ;       // dA_qk
    float* bet = sm + SM::R_SMALL;     // [64]
    float* dbp = bet + 64;             // [NW][64] dbeta: K+ dB_k + v dB_v, per wave
    float* dap = dbp + NW * 64;        // [4][64] dbeta: dA_kk P_kk, per column block

    const int lc = blockIdx.x / H, h = blockIdx.x - lc * H;  // slot g0 + lc, workspace slot lc
    ChunkLoc loc;
    if (!locate_chunk(tab, N, T, g0 + lc, loc)) return;
    const int t0 = loc.t0, L = loc.L;
    const int64_t fs = (int64_t)lc * H + h;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, G = l >> 4, n = l & 15;
    const int c = 16 * w + n;  // own channel
    const float* Pkk = f.am + fs * 64 * 64;     // [64][64] from the forward recompute
    float* SQ = scr + fs * bwd_scr_floats(D);   // dQ+, own-element tiles [NW][4][64][4]
    float* SK = SQ + 64 * D;                    // dK-, same layout
    const float* hF = f.h + fs * D * D;
    const float* vF = f.vn + fs * 64 * D;
    const float* dhB = b.h + fs * D * D;        // gradient of the chunk's exit state
    const float* dVB = b.vn + fs * 64 * D;      // dV
    auto rowoff = [&](int r) { return ((int64_t)(t0 + r) * H + h) * D; };
    auto own_row = [&](int R, int i) { return 16 * R + 4 * G + i; };

    if (tid < 64) bet[tid] = tid < L ? ld_in(beta, (int64_t)(t0 + tid) * H + h) : 0.f;

    // ---- 0a. dV, dO to LDS; dQ+ = dO h^T and dW = -dV h^T (own tiles), with
    // h^T of this wave's key rows in registers: the recursion stores h (and dh')
    // as [dv/16 value tiles][dk/32 key slices][64 lanes][8], lane n + 16 g
    // holding key rows 32 s + 16 (jj >> 2) + 4 g + (jj & 3) of value column
    // 16 ct + n; the half jj >> 2 = w & 1 of slice s = w >> 1 is the 16 x 16
    // tile (key rows 16 w .., value columns 16 ct ..) in accumulator layout,
    // whose transpose is the B operand of a product over value columns.
    // Every stage issues all of its global loads before it stores any of them, and
    // the next stage's loads are issued before this stage's products.
    constexpr int NVQ = 64 * D / 8 / NTH, NOQ = 64 * D / 4 / NTH, NT = D / 16;
    const int g = l >> 4;
    auto hfrag = [&](const float* base, int ct) {
        return *reinterpret_cast<const f32x4_t*>(base + ((int64_t)(ct * NS + (w >> 1)) * 64 + l) * 8 + 4 * (w & 1));
    };
    f32x4_t hT[NT], xv[NVQ][2], xo[NOQ];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) hT[ct] = hfrag(hF, ct);
#pragma unroll
    for (int m = 0; m < NVQ; ++m) {
        xv[m][0] = *reinterpret_cast<const f32x4_t*>(dVB + (tid + NTH * m) * 8);
        xv[m][1] = *reinterpret_cast<const f32x4_t*>(dVB + (tid + NTH * m) * 8 + 4);
    }
#pragma unroll
    for (int m = 0; m < NOQ; ++m) {
        const int e = tid + NTH * m, r = e / (D / 4), c4 = 4 * (e - r * (D / 4));
        xo[m] = r < L ? *reinterpret_cast<const f32x4_t*>(d_o + rowoff(r) + c4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    auto v_put = [&](float* dst, const f32x4_t (&x)[NVQ][2]) {
#pragma unroll
        for (int m = 0; m < NVQ; ++m) {
            const int q2 = tid + NTH * m, blk = q2 >> 6, ct = blk >> 1, sv = blk & 1, j = 16 * ct + (l & 15);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                dst[(32 * sv + frag_row(g, jj)) * RS + j] = jj < 4 ? x[m][0][jj] : x[m][1][jj - 4];
        }
    };
    v_put(VV, xv);
#pragma unroll
    for (int m = 0; m < NOQ; ++m) {
        const int e = tid + NTH * m, r = e / (D / 4), c4 = 4 * (e - r * (D / 4));
        *reinterpret_cast<f32x4_t*>(DO + r * RS + c4) = xo[m];
    }
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) hT[ct] = tr16(hT[ct], l);  // lane n + 16 G: key row c, values 16 ct + 4 G ..
    __syncthreads();
    // dh' and V in flight during the products
    f32x4_t dhT[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) dhT[ct] = hfrag(dhB, ct);
#pragma unroll
    for (int m = 0; m < NVQ; ++m) {
        xv[m][0] = *reinterpret_cast<const f32x4_t*>(vF + (tid + NTH * m) * 8);
        xv[m][1] = *reinterpret_cast<const f32x4_t*>(vF + (tid + NTH * m) * 8 + 4);
    }
    float dWo[4][4], dVo[4][4];  // own dW and dV
    {
        f32x4_t aq[4], aw[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) aq[R] = aw[R] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s16 = 0; s16 < NT; ++s16) {
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                mma16b(aq[R], DO + (16 * R + n) * RS + 16 * s16 + 4 * G, hT[s16]);
                mma16b(aw[R], VV + (16 * R + n) * RS + 16 * s16 + 4 * G, hT[s16]);
            }
        }
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            *reinterpret_cast<f32x4_t*>(SQ + ((w * 4 + R) * 64 + l) * 4) = aq[R];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dWo[R][i] = -aw[R][i];
                dVo[R][i] = VV[own_row(R, i) * RS + c];
            }
        }
    }
    // ---- 0b. dgamma = rowsum(h * dh') over the value columns of this lane's
    // key row (the four lane groups hold a quarter each), then V over dV
    float dgam;
    {
        float pg = 0.f;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            dhT[ct] = tr16(dhT[ct], l);
#pragma unroll
            for (int i = 0; i < 4; ++i) pg += hT[ct][i] * dhT[ct][i];
        }
        pg += __shfl_xor(pg, 16);
        dgam = pg + __shfl_xor(pg, 32);
    }
    __syncthreads();
    v_put(VV, xv);
    __syncthreads();
    // P_kk in flight during the products
    constexpr int NPK = 64 * 64 / 4 / NTH;
    f32x4_t xp[NPK];
#pragma unroll
    for (int m = 0; m < NPK; ++m) xp[m] = *reinterpret_cast<const f32x4_t*>(Pkk + 4 * (tid + NTH * m));
    // dK- = V dh'^T (own tiles); dA_qk = tril(dO V^T) (tiles spread over the waves)
    {
        f32x4_t ak[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) ak[R] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s16 = 0; s16 < NT; ++s16) {
#pragma unroll
            for (int R = 0; R < 4; ++R) mma16b(ak[R], VV + (16 * R + n) * RS + 16 * s16 + 4 * G, dhT[s16]);
        }
#pragma unroll
        for (int R = 0; R < 4; ++R) *reinterpret_cast<f32x4_t*>(SK + ((w * 4 + R) * 64 + l) * 4) = ak[R];
    }
    for (int tile = w; tile < 16; tile += NW) {
        const int R = tile >> 2, I = tile & 3;
        if (I > R) {  // above the diagonal: zero
#pragma unroll
            for (int i = 0; i < 4; ++i) DPQ[own_row(R, i) * SQS + 16 * I + n] = 0.f;
            continue;
        }
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
        for (int s16 = 0; s16 < D / 16; ++s16)
            mma16(a, DO + (16 * R + n) * RS + 16 * s16 + 4 * G, VV + (16 * I + n) * RS + 16 * s16 + 4 * G);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            DPQ[own_row(R, i) * SQS + 16 * I + n] = (I < R || n <= 4 * G + i) ? a[i] : 0.f;
    }
    // own inputs and the cumulative gate (natural log units)
    float qo[4][4], ko[4][4], g2[4][4];
    {
        typename OwnRows<TIn>::Raw rq[4], rk[4];
        typename OwnRows<TG>::Raw rg[4];
        own_load(q, t0, L, H, h, D, w, l, rq);
        own_load(k, t0, L, H, h, D, w, l, rk);
        own_load(la, t0, L, H, h, D, w, l, rg);
        f32x4_t tq[4], tk[4], tg[4];
        OwnRows<TIn>::to_own(rq, w, l, tq);
        OwnRows<TIn>::to_own(rk, w, l, tk);
        OwnRows<TG>::to_own(rg, w, l, tg);
        float part[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qo[R][i] = tq[R][i];
                ko[R][i] = tk[R][i];
                x += tg[R][i];
                g2[R][i] = x;  // prefix over the lane's 4 rows
            }
            part[R] = x;
        }
        // plus the lane groups before this one in the block and the blocks before
        float off = 0.f;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            float before = 0.f, total = 0.f;
#pragma unroll
            for (int G2 = 0; G2 < 4; ++G2) {
                const float t = __shfl(part[R], 16 * G2 + n);
                if (G2 < G) before += t;
                total += t;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) g2[R][i] += off + before;
            off += total;
        }
    }
    __syncthreads();  // phase-0 arrays dead

    // ---- 1. T = (I + diag(beta) P_kk)^-1, stored transposed: TT[r][m] = T[m][r]
#pragma unroll
    for (int m = 0; m < NPK; ++m) {
        const int e = tid + NTH * m;
        *reinterpret_cast<f32x4_t*>(PK + (e >> 4) * SQS + 4 * (e & 15)) = xp[m];
    }
    __syncthreads();
    if (w == 0) {  // diagonal blocks by forward substitution: lane = (block, column)
        const int bb = l >> 4, j = l & 15;
        float acc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[rr] = (rr == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ti = acc[i];
#pragma unroll
            for (int rr = i + 1; rr < 16; ++rr)
                acc[rr] -= bet[16 * bb + rr] * PK[(16 * bb + rr) * SQS + 16 * bb + i] * ti;
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4_t*>(TT + (16 * bb + j) * SQS + 16 * bb + 4 * r4) =
                f32x4_t{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
    }
    __syncthreads();
    // blocks below the diagonal: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, block row by block row
    for (int I = 1; I < 4; ++I) {
        if (w < I) {
            const int J = w;
            f32x4_t y = {0.f, 0.f, 0.f, 0.f};
            const float bi = bet[16 * I + n];
            for (int K = J; K < I; ++K) {
                const f32x4_t a = *reinterpret_cast<const f32x4_t*>(PK + (16 * I + n) * SQS + 16 * K + 4 * G);
                const f32x4_t t = *reinterpret_cast<const f32x4_t*>(TT + (16 * J + n) * SQS + 16 * K + 4 * G);
#pragma unroll
                for (int s = 0; s < 4; ++s) y = mfma4(bi * a[s], t[s], y);
            }
            f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) x = mfma4(TT[(16 * I + 4 * G + s) * SQS + 16 * I + n], y[s], x);
            *reinterpret_cast<f32x4_t*>(TT + (16 * J + n) * SQS + 16 * I + 4 * G) = -x;
        }
        __syncthreads();
    }

    // ---- 2. dB = T^T [dW | dV] (own tiles); dv = beta dB_v; dbeta's first terms
    f32x4_t xw[NOQ], xu[NOQ];  // -W and U in flight
#pragma unroll
    for (int m = 0; m < NOQ; ++m) {
        xw[m] = *reinterpret_cast<const f32x4_t*>(f.wn + fs * 64 * D + 4 * (tid + NTH * m));
        xu[m] = *reinterpret_cast<const f32x4_t*>(f.u + fs * 64 * D + 4 * (tid + NTH * m));
    }
    typename OwnRows<TIn>::Raw rv[4];
    own_load(v, t0, L, H, h, D, w, l, rv);
    float dBk[4][4];
    {
        f32x4_t vo[4], dvo[4];
        OwnRows<TIn>::to_own(rv, w, l, vo);
        float rowp[4][4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4_t ak = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int R2 = R; R2 < 4; ++R2) {
                const f32x4_t t = *reinterpret_cast<const f32x4_t*>(TT + (16 * R + n) * SQS + 16 * R2 + 4 * G);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    ak = mfma4(t[s], dWo[R2][s], ak);
                    av = mfma4(t[s], dVo[R2][s], av);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = own_row(R, i);
                dBk[R][i] = ak[i];
                dvo[R][i] = bet[r] * av[i];
                rowp[R][i] = ee(g2[R][i]) * ko[R][i] * ak[i] + vo[R][i] * av[i];
                DB[r * RX + c] = ak[i];
                DB[r * RX + D + c] = av[i];
            }
        }
        own_store(dv, t0, L, H, h, D, w, l, dvo);
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = sum16(rowp[R][i]);
                if (n == 0) dbp[w * 64 + own_row(R, i)] = t;
            }
    }
    __syncthreads();  // T dead, dB complete
    // ---- 3. dA_kk = -dB X^T = dB_k (-W)^T + dB_v (-U)^T on the lower tiles
#pragma unroll
    for (int m = 0; m < NOQ; ++m) {  // -W, stored in the split order
        const int e = tid + NTH * m, r = e / (D / 4), p = 4 * (e - r * (D / 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) TT[r * RS + split_chan(p + j)] = xw[m][j];
    }
    __syncthreads();
    constexpr int MT = (10 + NW - 1) / NW;  // lower tiles per wave
    f32x4_t da[MT];
    auto tile_of = [](int t, int& R, int& I) {  // t < 10 -> (R, I), I <= R
        R = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        I = t - R * (R + 1) / 2;
    };
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        da[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int t = w + NW * m;
        if (t < 10) {
            int R, I;
            tile_of(t, R, I);
            for (int s16 = 0; s16 < D / 16; ++s16)
                mma16(da[m], DB + (16 * R + n) * RX + 16 * s16 + 4 * G, TT + (16 * I + n) * RS + 16 * s16 + 4 * G);
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NOQ; ++m) {  // -U, stored as accumulator tiles
        const int e = tid + NTH * m, qd = e >> 6, ll = e & 63, ct = qd >> 2, R = qd & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) TT[(16 * R + 4 * (ll >> 4) + i) * RS + 16 * ct + (ll & 15)] = -xu[m][i];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int t = w + NW * m;
        if (t < 10) {
            int R, I;
            tile_of(t, R, I);
            for (int s16 = 0; s16 < D / 16; ++s16)
                mma16(da[m], DB + (16 * R + n) * RX + D + 16 * s16 + 4 * G,
                      TT + (16 * I + n) * RS + 16 * s16 + 4 * G);
            // dbeta's last term (sum_i dA_kk P_kk per row), then dP_kk = beta dA_kk over P_kk
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = own_row(R, i);
                float* pk = PK + r * SQS + 16 * I + n;
                const float x = (I < R || n < 4 * G + i) ? da[m][i] : 0.f;
                const float t2 = sum16(x * *pk);
                if (n == 0) dap[I * 64 + r] = t2;
                *pk = bet[r] * x;
            }
        }
    }
    __syncthreads();

    // dQ+ and dK- (own tiles, from phase 0) come back from the scratch during phase 4
    f32x4_t dqp4[4], dkm4[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        dqp4[R] = *reinterpret_cast<const f32x4_t*>(SQ + ((w * 4 + R) * 64 + l) * 4);
        dkm4[R] = *reinterpret_cast<const f32x4_t*>(SK + ((w * 4 + R) * 64 + l) * 4);
    }
    // ---- 4. adjoints of the gated products. Lq, Lk: row r as the left factor of
    // A_qk / A_kk; Rr: row i as their right factor (both take the key there)
    float Lq[4][4], Lk[4][4], Rr[4][4];
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) Lq[R][i] = Lk[R][i] = Rr[R][i] = 0.f;
    // blocks below the diagonal, split at the first row of the left factor's block ...
#pragma unroll
    for (int R = 1; R < 4; ++R) {
        const float bR = __shfl(g2[R][0], n);
        f32x4_t aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int R2 = 0; R2 < R; ++R2) {
            const f32x4_t pq = *reinterpret_cast<const f32x4_t*>(DPQ + (16 * R + n) * SQS + 16 * R2 + 4 * G);
            const f32x4_t pk = *reinterpret_cast<const f32x4_t*>(PK + (16 * R + n) * SQS + 16 * R2 + 4 * G);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float y = ko[R2][s] * ee(bR - g2[R2][s]);
                aq = mfma4(pq[s], y, aq);
                ak = mfma4(pk[s], y, ak);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = ee(g2[R][i] - bR);
            Lq[R][i] = aq[i] * e;
            Lk[R][i] = ak[i] * e;
        }
    }
    // ... and at the last row of the right factor's block
#pragma unroll
    for (int I = 0; I < 3; ++I) {
        const float aI = __shfl(g2[I][3], 48 + n);
        f32x4_t ar = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int R2 = I + 1; R2 < 4; ++R2)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = 16 * R2 + 4 * G + s;
                const float e = ee(g2[R2][s] - aI);
                ar = mfma4(DPQ[r * SQS + 16 * I + n], qo[R2][s] * e, ar);
                ar = mfma4(PK[r * SQS + 16 * I + n], ko[R2][s] * e, ar);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) Rr[I][i] = ar[i] * ee(aI - g2[I][i]);
    }
    // diagonal blocks. When no gate falls by more than DIAG_RANGE across a block,
    // the exponential splits at the block's row 8 with every factor at most
    // e^DIAG_RANGE (only the products' true size survives the rescale), and the
    // blocks go to the matrix cores like the others; otherwise pair by pair with
    // the exact exponential.
    constexpr float DIAG_RANGE = 60.f;
    int wide = 0;
#pragma unroll
    for (int B = 0; B < 4; ++B) wide |= __shfl(g2[B][0], n) - __shfl(g2[B][3], 48 + n) > DIAG_RANGE;
    if (!__syncthreads_or(wide)) {
#pragma unroll
        for (int B = 0; B < 4; ++B) {
            const float a = __shfl(g2[B][0], 32 + n);  // the gate at row 16 B + 8
            float up[4], dn[4];                        // e^(g - a), e^(a - g) of the own rows
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                up[i] = ee(g2[B][i] - a);
                dn[i] = ee(a - g2[B][i]);
            }
            f32x4_t aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f}, ar = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t pq = *reinterpret_cast<const f32x4_t*>(DPQ + (16 * B + n) * SQS + 16 * B + 4 * G);
            const f32x4_t pk = *reinterpret_cast<const f32x4_t*>(PK + (16 * B + n) * SQS + 16 * B + 4 * G);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * B + 4 * G + t;
                aq = mfma4(pq[t], ko[B][t] * dn[t], aq);
                ak = mfma4(pk[t], ko[B][t] * dn[t], ak);
                ar = mfma4(DPQ[r * SQS + 16 * B + n], qo[B][t] * up[t], ar);
                ar = mfma4(PK[r * SQS + 16 * B + n], ko[B][t] * up[t], ar);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Lq[B][i] += aq[i] * up[i];
                Lk[B][i] += ak[i] * up[i];
                Rr[B][i] += ar[i] * dn[i];
            }
        }
    } else {
#pragma unroll
    for (int B = 0; B < 4; ++B) {
#pragma unroll 1
        for (int G2 = 0; G2 < 4; ++G2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = 16 * B + 4 * G2 + j;
                const float kp = __shfl(ko[B][j], 16 * G2 + n);
                const float qp = __shfl(qo[B][j], 16 * G2 + n);
                const float gp = __shfl(g2[B][j], 16 * G2 + n);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int x = 16 * B + 4 * G + i;
                    const bool left = p <= x, right = p >= x;
                    const int at = left ? x * SQS + p : p * SQS + x;
                    const float e = ee(left ? g2[B][i] - gp : gp - g2[B][i]);
                    const float pq = DPQ[at], pk = PK[at];
                    if (left) {
                        Lq[B][i] += pq * kp * e;
                        Lk[B][i] += pk * kp * e;
                    }
                    if (right) Rr[B][i] += (pq * qp + pk * kp) * e;
                }
            }
    }
    }

    // ---- 5. gated scalings, the last row's terms, the reverse cumulative sum
    const float gl = __shfl(g2[3][3], 48 + n);  // cumulative gate of the chunk's last row
    float dg[4][4], lsum = 0.f;
    f32x4_t dqo[4], dko[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const f32x4_t dqp = dqp4[R];
        const f32x4_t dkm = dkm4[R];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = own_row(R, i);
            const float E = ee(g2[R][i]), Em = ee(gl - g2[R][i]);
            const float dkp = bet[r] * dBk[R][i];
            const float qv = qo[R][i], kv = ko[R][i];
            const float dqv = Lq[R][i] + E * dqp[i];
            const float dkv = Lk[R][i] + Rr[R][i] + E * dkp + Em * dkm[i];
            dg[R][i] = qv * Lq[R][i] + kv * Lk[R][i] - kv * Rr[R][i] + dqp[i] * E * qv + dkp * E * kv -
                       dkm[i] * Em * kv;
            lsum += dkm[i] * Em * kv;
            dqo[R][i] = dqv;
            dko[R][i] = dkv;
        }
    }
    own_store(dq, t0, L, H, h, D, w, l, dqo);
    own_store(dk, t0, L, H, h, D, w, l, dko);
    {
        float tot = 0.f;
#pragma unroll
        for (int G2 = 0; G2 < 4; ++G2) tot += __shfl(lsum, 16 * G2 + n);
        if (G == 3) dg[3][3] += tot + dgam * ee(gl);  // row 63 (padding rows add nothing)
    }
    {
        float S[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            float s = 0.f;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                s += dg[R][i];
                dg[R][i] = s;
            }
            S[R] = s;
        }
        float later = 0.f;  // whole blocks after R
        f32x4_t dlo[4];
#pragma unroll
        for (int R = 3; R >= 0; --R) {
            float after = 0.f, total = 0.f;
#pragma unroll
            for (int G2 = 3; G2 >= 0; --G2) {
                const float t = __shfl(S[R], 16 * G2 + n);
                if (G2 > G) after += t;
                total += t;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) dlo[R][i] = dg[R][i] + after + later;
            later += total;
        }
        own_store(dla, t0, L, H, h, D, w, l, dlo);
    }
    __syncthreads();
    if (tid < L) {
        float s = 0.f;
        for (int ww = 0; ww < NW; ++ww) s += dbp[ww * 64 + tid];
        for (int I = 0; I <= (tid >> 4); ++I) s += dap[I * 64 + tid];
        dbeta[(int64_t)(t0 + tid) * H + h] = s;
    }
}

template <int D>
static hipError_t launch_bwd_prep_d(const BwdArgs& a, hipStream_t st) {
    auto kern = bwd_prep_kernel<D>;
    const int bytes = BwdPrepSmem<D>::BYTES;
    const hipError_t e = allow_dynamic_lds((const void*)kern, bytes);
    if (e != hipSuccess) return e;
    const ChunkArgs& F = a.fwd;
    const ChunkArgs& B = a.rec;
    Ws<float> f{(float*)F.qp, (float*)F.km, (float*)F.wn, (float*)F.u, (float*)F.aqk, F.gam, (float*)F.h,
                (float*)F.vn};
    Ws<float> b{(float*)B.qp, (float*)B.km, (float*)B.wn, (float*)B.u, (float*)B.aqk, B.gam, (float*)B.h,
                (float*)B.vn, nullptr, nullptr, B.pb};
    hipLaunchKernelGGL(kern, dim3(F.slots() * F.H), dim3(4 * D), bytes, st, F.tab, F.N, F.T, F.H, F.piece.g0, f, b,
                       a.d_o);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t st) {
    return a.fwd.D == 128 ? launch_bwd_prep_d<128>(a, st) : launch_bwd_prep_d<64>(a, st);
}

template <int D, typename TIn, typename TG>
static hipError_t launch_bwd_local_t(const BwdArgs& a, hipStream_t st) {
    using SM = BwdSmem<D>;
    auto kern = bwd_local_kernel<D, TIn, TG>;
    const hipError_t e = allow_dynamic_lds((const void*)kern, SM::BYTES);
    if (e != hipSuccess) return e;
    const ChunkArgs& F = a.fwd;
    const ChunkArgs& B = a.rec;
    Ws<float> f{(float*)F.qp, (float*)F.km, (float*)F.wn, (float*)F.u, (float*)F.aqk, F.gam, (float*)F.h,
                (float*)F.vn, (float*)F.am};
    Ws<float> b{(float*)B.qp, (float*)B.km, (float*)B.wn, (float*)B.u, (float*)B.aqk, B.gam, (float*)B.h,
                (float*)B.vn, nullptr, nullptr, B.pb};
    hipLaunchKernelGGL(kern, dim3(F.slots() * F.H), dim3(4 * D), SM::BYTES, st, (const TIn*)F.q, (const TIn*)F.k,
                       (const TIn*)F.v, (const TG*)F.la, (const TG*)F.beta, F.tab, F.N, F.T, F.H, F.piece.g0, f, b,
                       a.d_o,
                       a.scr, a.dq, a.dk, a.dv, a.dla, a.dbeta);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_local_d(const BwdArgs& a, hipStream_t st) {
    const ChunkArgs& F = a.fwd;
    if (F.in_f32)
        return F.gate_f32 ? launch_bwd_local_t<D, float, float>(a, st) : launch_bwd_local_t<D, float, uint16_t>(a, st);
    return F.gate_f32 ? launch_bwd_local_t<D, uint16_t, float>(a, st) : launch_bwd_local_t<D, uint16_t, uint16_t>(a, st);
}

hipError_t launch_bwd_local(const BwdArgs& a, hipStream_t st) {
    return a.fwd.D == 128 ? launch_bwd_local_d<128>(a, st) : launch_bwd_local_d<64>(a, st);
}

}  // namespace kda
