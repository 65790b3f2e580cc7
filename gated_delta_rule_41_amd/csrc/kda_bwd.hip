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
// kernel on reversed chunk slots, with K- in place of -W, (-W)^T in place of
// K-^T, A_qk^T dO in place of U and the state-independent term Q+^T dO added
// each chunk (bwd_prep_kernel lays these out). What stays is chunk-local and
// parallel over chunks (bwd_local_kernel): the adjoints of the output and the
// state update (dQ+ = dO h^T, dA_qk = tril(dO V^T), dK- = V dh'^T,
// dgamma = rowsum(h * dh'), dW = -dV h^T), of the UT transform X = T B with
// T = (I + A_kk)^-1 (dB = T^T dX, dA_kk = -T^T (dX B^T) T^T on the strictly
// lower part), of the gated products (pairwise exponentials of gate
// differences <= 0, as in the forward's exact path) and of the gated scalings,
// then a reverse cumulative sum turns the gate gradient into dlog_alpha.
//
// Everything runs in fp32: the forward is recomputed with fp32 factors (the
// prep and recursion kernels' fp32 path, which keeps h_n and V_new).
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_prep_util.h"

namespace kda {

// element (kk, j) of a chunk-entry state stored as B-operand fragments
// [D/16 col tile][D/32 slice][64 lanes][8] (the fp32 recursion's h array)
template <int D>
__device__ __forceinline__ int hfrag_index(int kk, int j) {
    const int ct = j >> 4, n = j & 15, s = kk >> 5, k = kk & 31;
    const int g = (k & 15) >> 2, jj = 4 * (k >> 4) + (k & 3);
    return ((ct * (D / 32) + s) * 64 + 16 * g + n) * 8 + jj;
}
// element (r, j) of a chunk's corrected values stored as B-operand fragments
// [D/16 col tile][2 slices][64 lanes][8]
__device__ __forceinline__ int vfrag_index(int r, int j) {
    const int ct = j >> 4, n = j & 15, s = r >> 5, k = r & 31;
    const int g = (k & 15) >> 2, jj = 4 * (k >> 4) + (k & 3);
    return ((ct * 2 + s) * 64 + 16 * g + n) * 8 + jj;
}
// row-major [rows][ncol] array with columns in the split order per 32
__device__ __forceinline__ int split_index(int row, int col, int ncol) {
    return row * ncol + 32 * (col >> 5) + split_pos(col);
}
// element (r, j) of [D/16][4][64 lanes][4] accumulator tiles (64 rows)
__device__ __forceinline__ int tile_index(int r, int j) {
    return (((j >> 4) * 4 + (r >> 4)) * 64 + 16 * ((r & 15) >> 2) + (j & 15)) * 4 + (r & 3);
}

// Chunk slot gc of a sequence -> the slot the reversed recursion uses for it.
__device__ __forceinline__ int reversed_slot(const int32_t* cu, int T, int seq, int gc) {
    int co, nch;
    seq_chunks(cu, T, seq, co, nch);
    return co + nch - 1 - (gc - co);
}

// ---------------------------------------------------------------------------
// Operands of the state-gradient recursion for chunk slot gc, written to its
// reversed slot: -W := K-, K-^T := (-W)^T, U := A_qk^T dO, gamma, and the added
// term Q+^T dO in [dv/16][dk/16][64 lanes][4].
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const int32_t* __restrict__ cu, int N, int T, int H,
                                                       Ws<float> f, Ws<float> b, const float* __restrict__ d_o) {
    constexpr int NS = D / 32, NT = D / 16, RS = D + 4;
    extern __shared__ __align__(16) float sm[];
    float* dO = sm;                // [64][RS]
    float* Qp = dO + 64 * RS;      // [64][RS]
    float* Aq = Qp + 64 * RS;      // [64][65]
    const int gc = blockIdx.x / H, h = blockIdx.x - gc * H;
    ChunkLoc loc;
    if (!locate_chunk(cu, N, T, gc, loc)) return;
    const int rev = reversed_slot(cu, T, loc.seq, gc);
    const int64_t src = (int64_t)gc * H + h, dst = (int64_t)rev * H + h;
    const int tid = threadIdx.x;
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, c = e - r * D;
        dO[r * RS + c] = r < loc.L ? d_o[((int64_t)(loc.t0 + r) * H + h) * D + c] : 0.f;
        Qp[r * RS + c] = f.qp[src * 64 * D + split_index(r, c, D)];
        // K- to the -W layout; (-W)^T to the K-^T layout
        b.wn[dst * 64 * D + split_index(r, c, D)] = f.km[src * D * 64 + split_index(c, r, 64)];
        b.km[dst * D * 64 + split_index(c, r, 64)] = f.wn[src * 64 * D + split_index(r, c, D)];
    }
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        Aq[r * 65 + i] = f.aqk[src * 64 * 64 + split_index(r, i, 64)];
    }
    for (int c = tid; c < D; c += 256) b.gam[dst * D + c] = f.gam[src * D + c];
    __syncthreads();
    // U := A_qk^T dO (A_qk is lower triangular: rows i >= r)
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, j = e - r * D;
        float acc = 0.f;
        for (int i = r; i < 64; ++i) acc += Aq[i * 65 + r] * dO[i * RS + j];
        b.u[dst * 64 * D + tile_index(r, j)] = acc;
    }
    // P := Q+^T dO
    float* pb = const_cast<float*>(b.pb) + dst * D * D;
    for (int e = tid; e < D * D; e += 256) {
        const int c = e / D, j = e - c * D;
        float acc = 0.f;
        for (int r = 0; r < 64; ++r) acc += Qp[r * RS + c] * dO[r * RS + j];
        const int lane = 16 * ((c & 15) >> 2) + (j & 15);
        pb[(((j >> 4) * NT + (c >> 4)) * 64 + lane) * 4 + (c & 3)] = acc;
    }
    (void)NS;
}

// ---------------------------------------------------------------------------
// Chunk-local adjoints, one 256-thread workgroup per (chunk, head). Thread t
// owns channel c = t % D of rows r0 .. r0 + RPT - 1 for every elementwise
// quantity, so per-(row, channel) partial gradients stay in its registers.
template <int D>
struct BwdSmem {
    static constexpr int RS = D + 4;                 // row stride of [rows][D] matrices
    static constexpr int BIGR = D > 128 ? D : 128;   // rows of BIG: h or dh' (D), or q and G (2 x 64)
    static constexpr int BIG = BIGR * RS;
    static constexpr int MAT = 64 * RS;              // [64][RS]
    static constexpr int SQ = 64 * 65;               // [64][65]
    static constexpr int SQX = 2 * SQ <= MAT ? 0 : 2 * SQ;  // two 64 x 64 matrices: in M2 if they fit
    static constexpr int NG = 64 / (64 * D / 256);   // row groups of the thread layout
    static constexpr int FLOATS = BIG + 2 * MAT + SQX + 2 * 64 + 3 * D + NG * D;
    static constexpr int BYTES = FLOATS * 4;
    static_assert(2 * SQ <= BIG, "A and T fit in BIG");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int D, typename TIn, typename TG>
__global__ __launch_bounds__(256) void bwd_local_kernel(const TIn* q, const TIn* k, const TIn* v, const TG* la,
                                                        const TG* beta, const int32_t* __restrict__ cu, int N,
                                                        int T, int H, Ws<float> f, Ws<float> b,
                                                        const float* __restrict__ d_o, float* __restrict__ scr,
                                                        float* __restrict__ dq, float* __restrict__ dk,
                                                        float* __restrict__ dv, float* __restrict__ dla,
                                                        float* __restrict__ dbeta) {
    using SM = BwdSmem<D>;
    constexpr int RS = SM::RS, RPT = 64 * D / 256, NG = 64 / RPT;  // rows per thread, row groups
    extern __shared__ __align__(16) float sm[];
    float* BIGm = sm;                  // [D][RS]
    float* M1 = BIGm + SM::BIG;        // [64][RS]
    float* M2 = M1 + SM::MAT;          // [64][RS]
    float* S1 = SM::SQX ? M2 + SM::MAT : M2;  // [64][65], in M2 (once M2 is free) when it fits
    float* S2 = S1 + SM::SQ;                  // [64][65]
    float* bet = M2 + SM::MAT + SM::SQX;      // [64] beta
    float* dbs = bet + 64;             // [64] dbeta: the dA_kk term (one thread per row)
    float* dgam = dbs + 64;            // [D]
    float* gl = dgam + D;              // [D] cumulative gate at the chunk's last row
    float* gtot = gl + D;              // [NG][D] row-group totals of dg, then of the last-row terms
    // (every cross-thread sum below runs in a fixed order: the results are deterministic)

    const int gc = blockIdx.x / H, h = blockIdx.x - gc * H;
    ChunkLoc loc;
    if (!locate_chunk(cu, N, T, gc, loc)) return;
    const int t0 = loc.t0, L = loc.L;
    const int rev = reversed_slot(cu, T, loc.seq, gc);
    const int64_t fs = (int64_t)gc * H + h, bs = (int64_t)rev * H + h;
    const int tid = threadIdx.x;
    const int c = tid % D, r0 = (tid / D) * RPT, grp = tid / D;
    float* G = scr + fs * bwd_scr_floats(D);   // [64][D] cumulative gate (natural log)
    float* SQp = G + 64 * D;                   // [64][D] dQ+
    float* SW = SQp + 64 * D;                  // [64][D] dW
    float* SKm = SW + 64 * D;                  // [64][D] dK-
    float* SPq = SKm + 64 * D;                 // [64][64] dA_qk
    float* SPk = SPq + 64 * 64;                // [64][64] P_kk (ungated by beta)
    float* SdPk = SPk + 64 * 64;               // [64][64] dP_kk
    const float* hF = f.h + fs * D * D;        // forward chunk-entry state
    const float* vF = f.vn + fs * 64 * D;      // forward corrected values
    const float* dhB = b.h + bs * D * D;       // gradient of the chunk's exit state
    const float* dVB = b.vn + bs * 64 * D;     // dV
    auto rowoff = [&](int r) { return ((int64_t)(t0 + r) * H + h) * D; };
    auto in_q = [&](int r, int cc) { return r < L ? ld_in(q, rowoff(r) + cc) : 0.f; };
    auto in_k = [&](int r, int cc) { return r < L ? ld_in(k, rowoff(r) + cc) : 0.f; };
    auto in_v = [&](int r, int cc) { return r < L ? ld_in(v, rowoff(r) + cc) : 0.f; };

    // ---- 0. beta, cumulative gate, dgamma = rowsum(h * dh')
    if (tid < 64) {
        bet[tid] = tid < L ? ld_in(beta, (int64_t)(t0 + tid) * H + h) : 0.f;
        dbs[tid] = 0.f;
    }
    for (int cc = tid; cc < D; cc += 256) {
        float x = 0.f;
        for (int r = 0; r < 64; ++r) {
            if (r < L) x += ld_in(la, rowoff(r) + cc);
            G[r * D + cc] = x;
        }
        gl[cc] = x;
        float s = 0.f;
        for (int j = 0; j < D; ++j) s += hF[hfrag_index<D>(cc, j)] * dhB[hfrag_index<D>(cc, j)];
        dgam[cc] = s;
    }
    // ---- 1. dQ+ = dO h^T and dW = -dV h^T (h in BIG, dO in M1, dV in M2)
    for (int e = tid; e < D * D; e += 256) {
        const int kk = e / D, j = e - kk * D;
        BIGm[kk * RS + j] = hF[hfrag_index<D>(kk, j)];
    }
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, j = e - r * D;
        M1[r * RS + j] = r < L ? d_o[rowoff(r) + j] : 0.f;
        M2[r * RS + j] = dVB[vfrag_index(r, j)];
    }
    __syncthreads();
    {
        float aq[RPT], aw[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) aq[i] = aw[i] = 0.f;
        for (int j = 0; j < D; j += 4) {
            const f32x4_t hv = *reinterpret_cast<const f32x4_t*>(BIGm + c * RS + j);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(M1 + (r0 + i) * RS + j);
                const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(M2 + (r0 + i) * RS + j);
                aq[i] += o4[0] * hv[0] + o4[1] * hv[1] + o4[2] * hv[2] + o4[3] * hv[3];
                aw[i] -= v4[0] * hv[0] + v4[1] * hv[1] + v4[2] * hv[2] + v4[3] * hv[3];
            }
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            SQp[(r0 + i) * D + c] = aq[i];
            SW[(r0 + i) * D + c] = aw[i];
        }
    }
    __syncthreads();
    // ---- 2. dA_qk = tril(dO V^T) (V in BIG's first 64 rows, dO still in M1)
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, j = e - r * D;
        BIGm[r * RS + j] = vF[vfrag_index(r, j)];
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float acc = 0.f;
        if (i <= r)
            for (int j = 0; j < D; j += 4) {
                const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(M1 + r * RS + j);
                const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(BIGm + i * RS + j);
                acc += a4[0] * b4[0] + a4[1] * b4[1] + a4[2] * b4[2] + a4[3] * b4[3];
            }
        SPq[r * 64 + i] = acc;
    }
    __syncthreads();
    // ---- 3. dK- = V dh'^T (V to M1, dh' in BIG)
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, j = e - r * D;
        M1[r * RS + j] = BIGm[r * RS + j];
    }
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) {
        const int kk = e / D, j = e - kk * D;
        BIGm[kk * RS + j] = dhB[hfrag_index<D>(kk, j)];
    }
    __syncthreads();
    {
        float ak[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) ak[i] = 0.f;
        for (int j = 0; j < D; j += 4) {
            const f32x4_t hv = *reinterpret_cast<const f32x4_t*>(BIGm + c * RS + j);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(M1 + (r0 + i) * RS + j);
                ak[i] += v4[0] * hv[0] + v4[1] * hv[1] + v4[2] * hv[2] + v4[3] * hv[3];
            }
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) SKm[(r0 + i) * D + c] = ak[i];
    }
    __syncthreads();
    // ---- 4. UT transform. k -> M1, G -> M2; P_kk[r][i] = sum_c k_rc k_ic exp(G_rc - G_ic), i < r
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, cc = e - r * D;
        M1[r * RS + cc] = in_k(r, cc);
        M2[r * RS + cc] = G[r * D + cc];
    }
    __syncthreads();
    float* A = BIGm;            // [64][65]: beta_r P_kk, then dT, then Y
    float* Tm = BIGm + 64 * 65; // [64][65]: T = (I + A_kk)^-1
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float acc = 0.f;
        if (i < r)
            for (int cc = 0; cc < D; ++cc)
                acc += M1[r * RS + cc] * M1[i * RS + cc] * __expf(M2[r * RS + cc] - M2[i * RS + cc]);
        SPk[r * 64 + i] = acc;
        A[r * 65 + i] = bet[r] * acc;
    }
    __syncthreads();
    // forward substitution, row by row: T[r][i] = [r == i] - sum_{m=i}^{r-1} A[r][m] T[m][i]
    for (int r = 0; r < 64; ++r) {
        if (tid < 64) {
            const int i = tid;
            float x = (i == r) ? 1.f : 0.f;
            if (i < r)
                for (int m = i; m < r; ++m) x -= A[r * 65 + m] * Tm[m * 65 + i];
            Tm[r * 65 + i] = x;
        }
        __syncthreads();
    }
    // K+ = exp(G) k into M1 (G still in M2), dW into M2's place after: stage dW to S? -> use BIG's tail
    float* dT = A;  // reuse: A is dead after T
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, cc = e - r * D;
        M1[r * RS + cc] = __expf(M2[r * RS + cc]) * M1[r * RS + cc];  // K+
    }
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, cc = e - r * D;
        M2[r * RS + cc] = SW[r * D + cc];  // dW
    }
    for (int e = tid; e < 64 * 64; e += 256) dT[(e >> 6) * 65 + (e & 63)] = 0.f;
    __syncthreads();
    // part K: dT[r][i] += sum_c dW[r][c] beta_i K+[i][c];  dB_k = T^T dW
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float acc = 0.f;
        for (int cc = 0; cc < D; cc += 4) {
            const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(M2 + r * RS + cc);
            const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(M1 + i * RS + cc);
            acc += a4[0] * b4[0] + a4[1] * b4[1] + a4[2] * b4[2] + a4[3] * b4[3];
        }
        dT[r * 65 + i] += bet[i] * acc;
    }
    float dKp[RPT], dbr[RPT];  // dbr: this thread's (row, channel) terms of dbeta
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + i;
        float acc = 0.f;
        for (int m = r; m < 64; ++m) acc += Tm[m * 65 + r] * M2[m * RS + c];
        dKp[i] = bet[r] * acc;
        dbr[i] = M1[r * RS + c] * acc;  // K+[r][c] dB_k[r][c]
    }
    __syncthreads();
    // part V: v -> M1, dV -> M2; dT[r][i] += sum_j dV[r][j] beta_i v[i][j]; dv = beta T^T dV
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, j = e - r * D;
        M1[r * RS + j] = in_v(r, j);
        M2[r * RS + j] = dVB[vfrag_index(r, j)];
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float acc = 0.f;
        for (int j = 0; j < D; j += 4) {
            const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(M2 + r * RS + j);
            const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(M1 + i * RS + j);
            acc += a4[0] * b4[0] + a4[1] * b4[1] + a4[2] * b4[2] + a4[3] * b4[3];
        }
        dT[r * 65 + i] += bet[i] * acc;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + i;
        float acc = 0.f;
        for (int m = r; m < 64; ++m) acc += Tm[m * 65 + r] * M2[m * RS + c];
        if (r < L) dv[rowoff(r) + c] = bet[r] * acc;
        dbr[i] += M1[r * RS + c] * acc;  // v[r][c] dB_v[r][c]
    }
    __syncthreads();
    // dA_kk = -T^T (dT T^T), strictly lower: Y = dT T^T into S1, then dA into S2
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float acc = 0.f;
        for (int m = 0; m <= i; ++m) acc += dT[r * 65 + m] * Tm[i * 65 + m];  // T[i][m] = 0 for m > i
        S1[r * 65 + i] = acc;
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        float acc = 0.f;
        if (i < r)
            for (int m = r; m < 64; ++m) acc += Tm[m * 65 + r] * S1[m * 65 + i];  // T[m][r] = 0 for m < r
        const float dA = -acc;
        SdPk[r * 64 + i] = bet[r] * dA;
        S2[r * 65 + i] = dA * SPk[r * 64 + i];
    }
    __syncthreads();
    if (tid < 64) {
        float s = 0.f;
        for (int i = 0; i < tid; ++i) s += S2[tid * 65 + i];
        dbs[tid] = s;
    }
    __syncthreads();
    // ---- 5. gated products' adjoints. q -> BIG[0:64], G -> BIG[64:128] (D = 128) or
    // M-matrices; k -> M1; dA_qk -> S1, dP_kk -> S2
    float* Qm = BIGm;
    float* Gm = BIGm + 64 * RS;  // BIG has at least 128 rows
    for (int e = tid; e < 64 * D; e += 256) {
        const int r = e / D, cc = e - r * D;
        Qm[r * RS + cc] = in_q(r, cc);
        Gm[r * RS + cc] = G[r * D + cc];
        M1[r * RS + cc] = in_k(r, cc);
    }
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, i = e & 63;
        S1[r * 65 + i] = SPq[r * 64 + i];
        S2[r * 65 + i] = SdPk[r * 64 + i];
    }
    __syncthreads();
    float dqv[RPT], dkv[RPT], dgv[RPT];
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) {
        const int r = r0 + ii;
        const float gr = Gm[r * RS + c], qr = Qm[r * RS + c], kr = M1[r * RS + c];
        float sq = 0.f, skb = 0.f, ska = 0.f, skc = 0.f;
        for (int i = 0; i <= r; ++i) {  // row r as the left factor: i <= r
            const float e = __expf(gr - Gm[i * RS + c]);  // G_r - G_i <= 0
            const float ki = M1[i * RS + c];
            sq += S1[r * 65 + i] * ki * e;
            if (i < r) skb += S2[r * 65 + i] * ki * e;
        }
        for (int rr = r; rr < 64; ++rr) {  // row r as the right factor: rr >= r
            const float e = __expf(Gm[rr * RS + c] - gr);
            ska += S1[rr * 65 + r] * Qm[rr * RS + c] * e;
            if (rr > r) skc += S2[rr * 65 + r] * M1[rr * RS + c] * e;
        }
        dqv[ii] = sq;
        dkv[ii] = ska + skb + skc;
        dgv[ii] = qr * sq - kr * ska + kr * skb - kr * skc;
    }
    // ---- 6. gated scalings, the last row's terms, and the reverse cumulative sum
    {
        float ls = 0.f;
#pragma unroll
        for (int ii = 0; ii < RPT; ++ii) {
            const int r = r0 + ii;
            const float gr = Gm[r * RS + c], qr = Qm[r * RS + c], kr = M1[r * RS + c];
            const float E = __expf(gr), Em = __expf(gl[c] - gr);
            const float dQp = SQp[r * D + c], dKm = SKm[r * D + c];
            dqv[ii] += E * dQp;
            dkv[ii] += E * dKp[ii] + Em * dKm;
            const float km = Em * kr;
            dgv[ii] += dQp * E * qr + dKp[ii] * E * kr - dKm * km;
            ls += dKm * km;
        }
        gtot[grp * D + c] = ls;
    }
    __syncthreads();
    // the chunk's last cumulative gate is G at row 63 (padding rows add 0): its
    // terms go to row 63, which the reverse sum spreads over every row
    if (r0 + RPT == 64) {
        float ls = 0.f;
        for (int gg = 0; gg < NG; ++gg) ls += gtot[gg * D + c];
        dgv[RPT - 1] += ls + dgam[c] * __expf(gl[c]);
    }
    __syncthreads();  // gtot is reused below
    {
        float s = 0.f;
#pragma unroll
        for (int ii = RPT - 1; ii >= 0; --ii) {
            s += dgv[ii];
            dgv[ii] = s;
        }
        gtot[grp * D + c] = s;
    }
    __syncthreads();
    {
        float later = 0.f;
        for (int gg = grp + 1; gg < NG; ++gg) later += gtot[gg * D + c];
#pragma unroll
        for (int ii = 0; ii < RPT; ++ii) {
            const int r = r0 + ii;
            if (r < L) {
                dq[rowoff(r) + c] = dqv[ii];
                dk[rowoff(r) + c] = dkv[ii];
                dla[rowoff(r) + c] = dgv[ii] + later;
            }
        }
    }
    // dbeta: this thread's terms to M2 (free by now), then one thread per row
    // sums them over the channels in order
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) M2[(r0 + ii) * RS + c] = dbr[ii];
    __syncthreads();
    if (tid < L) {
        float s = dbs[tid];
        for (int cc = 0; cc < D; ++cc) s += M2[tid * RS + cc];
        dbeta[(int64_t)(t0 + tid) * H + h] = s;
    }
}

template <int D>
static hipError_t launch_bwd_prep_d(const BwdArgs& a, hipStream_t st) {
    constexpr int RS = D + 4;
    const int bytes = (2 * 64 * RS + 64 * 65) * 4;
    auto kern = bwd_prep_kernel<D>;
    const hipError_t e = allow_dynamic_lds((const void*)kern, bytes);
    if (e != hipSuccess) return e;
    const ChunkArgs& F = a.fwd;
    const ChunkArgs& B = a.rec;
    Ws<float> f{(float*)F.qp, (float*)F.km, (float*)F.wn, (float*)F.u, (float*)F.aqk, F.gam, (float*)F.h,
                (float*)F.vn};
    Ws<float> b{(float*)B.qp, (float*)B.km, (float*)B.wn, (float*)B.u, (float*)B.aqk, B.gam, (float*)B.h,
                (float*)B.vn, nullptr, nullptr, B.pb};
    hipLaunchKernelGGL(kern, dim3(F.NC * F.H), dim3(256), bytes, st, F.cu, F.N, F.T, F.H, f, b, a.d_o);
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
                (float*)F.vn};
    Ws<float> b{(float*)B.qp, (float*)B.km, (float*)B.wn, (float*)B.u, (float*)B.aqk, B.gam, (float*)B.h,
                (float*)B.vn, nullptr, nullptr, B.pb};
    hipLaunchKernelGGL(kern, dim3(F.NC * F.H), dim3(256), SM::BYTES, st, (const TIn*)F.q, (const TIn*)F.k,
                       (const TIn*)F.v, (const TG*)F.la, (const TG*)F.beta, F.cu, F.N, F.T, F.H, f, b, a.d_o,
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
