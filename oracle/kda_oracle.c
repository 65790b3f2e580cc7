/*
 * CPU oracle for the Kimi Delta Attention (KDA) operator -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load this library. The product path (the HIP library) never calls it.
 *
 * What it computes: the plain token-by-token recurrence, in fp64, for every
 * (sequence, head) of a packed batch:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(log_alpha_t) per key channel
 *
 * written as the four steps of one token (the order follows from the formula):
 *     1. decay:      S <- Diag(alpha_t) S            (row c scaled by alpha_t[c])
 *     2. residual:   u <- beta_t (v_t - S^T k_t)     (against the decayed state)
 *     3. write:      S <- S + k_t u^T
 *     4. read:       o_t <- S^T q_t                  (the post-update state)
 *
 * Sources: the channel-wise (diagonal) forget gate on the delta rule --
 * GeekNews "Kimi Linear" summary (pt.news.hada.io topic 31936), sections
 * "Da atenção linear ao Gated DeltaNet" (delta rule, scalar-gated GDN) and
 * "Controle fino de memória no Kimi Delta Attention" (per-channel gate, DPLR
 * transition consistent with the delta rule); the chunk-to-chunk hand-off of
 * the state -- same page, section "Algoritmo paralelo por chunks". The pages'
 * formulas did not survive extraction; the recurrence above is the one they
 * describe in prose (diagonal gate applied to the state, then the rank-1
 * Householder-type delta correction tied to the key).
 *
 * Conventions (readings where the pages are silent):
 *   - no query scaling; q is used as given;
 *   - log_alpha has one value per (token, head, key channel); beta one per (token, head);
 *   - inputs may be fp32, bf16 (raw 16-bit patterns) or fp64; they are widened
 *     exactly to fp64 before use;
 *   - layouts are token-major: q,k,log_alpha [T_total, H, dk], v [T_total, H, dv],
 *     beta [T_total, H]; states [N, H, dk, dv] (dv fastest).
 *
 * Parallelism: OpenMP over independent units (sequence, head, block of value
 * columns). Columns of S evolve independently (each step touches column j only
 * through v_t[j] and u[j]), so splitting them changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

static inline double load_as_f64(const void* p, int dt, int64_t i) {
    if (dt == ORC_F64) return ((const double*)p)[i];
    if (dt == ORC_F32) return (double)((const float*)p)[i];
    uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int kda_oracle_abi_version(void) { return 1; }

/*
 * Run the recurrence.
 *   cu_seqlens   host int64 [N+1], cu[0] = 0, non-decreasing, cu[N] = T_total
 *   S0           fp64 [N,H,dk,dv] or NULL (zeros)
 *   S_final      fp64 [N,H,dk,dv] or NULL   (only heads in the subset are written)
 *   o            fp64 [T_total,H,dv] or NULL (only heads in the subset are written)
 *   heads        subset of head indices (NULL = all H heads)
 *   rec_pos      sorted global token positions whose outputs are also copied to
 *   o_rec        fp64 [n_rec, n_heads_used, dv] (head order = subset order); may be NULL
 *   col_blocks   number of value-column blocks per (sequence, head) unit (>= 1)
 *   n_threads    OpenMP threads (<= 0: library default)
 * Returns 0 on success, a negative code on bad arguments.
 */
int kda_oracle_forward(int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                       const void* q, const void* k, const void* v, const void* log_alpha,
                       const void* beta, int in_dt, int gate_dt,
                       int32_t N, const int64_t* cu_seqlens,
                       const double* S0, double* S_final, double* o,
                       const int32_t* heads, int32_t n_heads,
                       const int64_t* rec_pos, int64_t n_rec, double* o_rec,
                       int32_t col_blocks, int32_t n_threads) {
    if (H <= 0 || dk <= 0 || dv <= 0 || N < 0 || !cu_seqlens) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return -2;
    for (int32_t i = 0; i < N; ++i)
        if (cu_seqlens[i + 1] < cu_seqlens[i]) return -3;
    if (col_blocks < 1) col_blocks = 1;
    if (col_blocks > dv) col_blocks = dv;
    const int32_t nh = heads ? n_heads : H;
    if (heads)
        for (int32_t i = 0; i < nh; ++i)
            if (heads[i] < 0 || heads[i] >= H) return -4;
    if (n_rec > 0 && !o_rec) return -5;
    const int64_t n_units = (int64_t)N * nh * col_blocks;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* kk = (double*)malloc(sizeof(double) * (size_t)dk * 3);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kk || !u) {
#pragma omp atomic write
            bad = 1;
        } else {
            double* aa = kk + dk;
            double* qq = kk + 2 * dk;
#pragma omp for schedule(dynamic, 1)
            for (int64_t unit = 0; unit < n_units; ++unit) {
                const int32_t cb = (int32_t)(unit % col_blocks);
                const int32_t hi = (int32_t)((unit / col_blocks) % nh);
                const int32_t seq = (int32_t)(unit / ((int64_t)col_blocks * nh));
                const int32_t h = heads ? heads[hi] : hi;
                const int32_t j0 = (int32_t)(((int64_t)dv * cb) / col_blocks);
                const int32_t j1 = (int32_t)(((int64_t)dv * (cb + 1)) / col_blocks);
                const int32_t nc = j1 - j0;
                const int64_t sbase = ((int64_t)seq * H + h) * dk * dv;
                for (int32_t c = 0; c < dk; ++c)
                    for (int32_t j = 0; j < nc; ++j)
                        S[(int64_t)c * nc + j] = S0 ? S0[sbase + (int64_t)c * dv + j0 + j] : 0.0;
                int64_t rp = 0;  /* cursor into rec_pos */
                const int64_t t_begin = cu_seqlens[seq], t_end = cu_seqlens[seq + 1];
                if (n_rec > 0) {
                    int64_t lo = 0, hi2 = n_rec;
                    while (lo < hi2) {
                        int64_t mid = (lo + hi2) / 2;
                        if (rec_pos[mid] < t_begin) lo = mid + 1; else hi2 = mid;
                    }
                    rp = lo;
                }
                for (int64_t t = t_begin; t < t_end; ++t) {
                    const int64_t kb = (t * H + h) * dk;
                    const int64_t vb = (t * H + h) * dv;
                    for (int32_t c = 0; c < dk; ++c) {
                        kk[c] = load_as_f64(k, in_dt, kb + c);
                        qq[c] = load_as_f64(q, in_dt, kb + c);
                        aa[c] = exp(load_as_f64(log_alpha, gate_dt, kb + c));
                    }
                    const double b = load_as_f64(beta, gate_dt, t * H + h);
                    /* 1. decay */
                    for (int32_t c = 0; c < dk; ++c) {
                        double* Sr = S + (int64_t)c * nc;
                        for (int32_t j = 0; j < nc; ++j) Sr[j] *= aa[c];
                    }
                    /* 2. residual against the decayed state: u = beta (v - S^T k) */
                    for (int32_t j = 0; j < nc; ++j) u[j] = 0.0;
                    for (int32_t c = 0; c < dk; ++c) {
                        const double* Sr = S + (int64_t)c * nc;
                        for (int32_t j = 0; j < nc; ++j) u[j] += Sr[j] * kk[c];
                    }
                    for (int32_t j = 0; j < nc; ++j)
                        u[j] = b * (load_as_f64(v, in_dt, vb + j0 + j) - u[j]);
                    /* 3. write: S += k u^T */
                    for (int32_t c = 0; c < dk; ++c) {
                        double* Sr = S + (int64_t)c * nc;
                        for (int32_t j = 0; j < nc; ++j) Sr[j] += kk[c] * u[j];
                    }
                    /* 4. read: o_t = S^T q (post-update state) */
                    const int want_full = (o != NULL);
                    const int want_rec = (rp < n_rec && rec_pos[rp] == t);
                    if (want_full || want_rec) {
                        for (int32_t j = 0; j < nc; ++j) u[j] = 0.0;
                        for (int32_t c = 0; c < dk; ++c) {
                            const double* Sr = S + (int64_t)c * nc;
                            for (int32_t j = 0; j < nc; ++j) u[j] += Sr[j] * qq[c];
                        }
                        if (want_full)
                            for (int32_t j = 0; j < nc; ++j) o[vb + j0 + j] = u[j];
                        if (want_rec) {
                            double* dst = o_rec + (rp * nh + hi) * dv + j0;
                            for (int32_t j = 0; j < nc; ++j) dst[j] = u[j];
                        }
                    }
                    while (rp < n_rec && rec_pos[rp] <= t) ++rp;
                }
                if (S_final)
                    for (int32_t c = 0; c < dk; ++c)
                        for (int32_t j = 0; j < nc; ++j)
                            S_final[sbase + (int64_t)c * dv + j0 + j] = S[(int64_t)c * nc + j];
            }
        }
        free(S);
        free(kk);
        free(u);
    }
    return bad ? -6 : 0;
}

/*
 * General diagonal-plus-low-rank (DPLR) transition -- the comparison operator.
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t
 *
 * with a_t, b_t free per-(token, head) key-space vectors. This is the general
 * transition that KDA specialises (GeekNews "Kimi Linear" summary, section
 * "Menos computação que o DPLR geral": KDA ties both low-rank vectors to the
 * key, a = beta k and b = alpha * k with written key beta k, which is what
 * saves gated matrices and products against the general case). One token, in
 * the order the formula fixes:
 *     1. low-rank read:  u <- S^T b_t              (the state before this token)
 *     2. decay:          S <- Diag(alpha_t) S
 *     3. update:         S <- S - a_t u^T + k_t v_t^T
 *     4. read:           o_t <- S^T q_t
 * Inputs: q, k, a, b, log_alpha [T_total, H, dk] (q, k, v, a, b in in_dt;
 * log_alpha in gate_dt), v [T_total, H, dv]; other arguments as in
 * kda_oracle_forward (no recorded positions). Columns of S stay independent
 * (step 1 reads column j through column j only), so column blocks are exact.
 */
int kda_oracle_dplr_forward(int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                            const void* q, const void* k, const void* v, const void* a,
                            const void* b, const void* log_alpha, int in_dt, int gate_dt,
                            int32_t N, const int64_t* cu_seqlens,
                            const double* S0, double* S_final, double* o,
                            const int32_t* heads, int32_t n_heads,
                            int32_t col_blocks, int32_t n_threads) {
    if (H <= 0 || dk <= 0 || dv <= 0 || N < 0 || !cu_seqlens) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return -2;
    for (int32_t i = 0; i < N; ++i)
        if (cu_seqlens[i + 1] < cu_seqlens[i]) return -3;
    if (col_blocks < 1) col_blocks = 1;
    if (col_blocks > dv) col_blocks = dv;
    const int32_t nh = heads ? n_heads : H;
    if (heads)
        for (int32_t i = 0; i < nh; ++i)
            if (heads[i] < 0 || heads[i] >= H) return -4;
    const int64_t n_units = (int64_t)N * nh * col_blocks;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* vec = (double*)malloc(sizeof(double) * (size_t)dk * 5);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv * 2);
        if (!S || !vec || !u) {
#pragma omp atomic write
            bad = 1;
        } else {
            double *qq = vec, *kk = vec + dk, *aa = vec + 2 * dk, *bb = vec + 3 * dk, *al = vec + 4 * dk;
            double* vv = u + dv;
#pragma omp for schedule(dynamic, 1)
            for (int64_t unit = 0; unit < n_units; ++unit) {
                const int32_t cb = (int32_t)(unit % col_blocks);
                const int32_t hi = (int32_t)((unit / col_blocks) % nh);
                const int32_t seq = (int32_t)(unit / ((int64_t)col_blocks * nh));
                const int32_t h = heads ? heads[hi] : hi;
                const int32_t j0 = (int32_t)(((int64_t)dv * cb) / col_blocks);
                const int32_t j1 = (int32_t)(((int64_t)dv * (cb + 1)) / col_blocks);
                const int32_t nc = j1 - j0;
                const int64_t sbase = ((int64_t)seq * H + h) * dk * dv;
                for (int32_t c = 0; c < dk; ++c)
                    for (int32_t j = 0; j < nc; ++j)
                        S[(int64_t)c * nc + j] = S0 ? S0[sbase + (int64_t)c * dv + j0 + j] : 0.0;
                for (int64_t t = cu_seqlens[seq]; t < cu_seqlens[seq + 1]; ++t) {
                    const int64_t kb = (t * H + h) * dk;
                    const int64_t vb = (t * H + h) * dv;
                    for (int32_t c = 0; c < dk; ++c) {
                        qq[c] = load_as_f64(q, in_dt, kb + c);
                        kk[c] = load_as_f64(k, in_dt, kb + c);
                        aa[c] = load_as_f64(a, in_dt, kb + c);
                        bb[c] = load_as_f64(b, in_dt, kb + c);
                        al[c] = exp(load_as_f64(log_alpha, gate_dt, kb + c));
                    }
                    for (int32_t j = 0; j < nc; ++j) vv[j] = load_as_f64(v, in_dt, vb + j0 + j);
                    /* 1. low-rank read of the previous state: u = S^T b */
                    for (int32_t j = 0; j < nc; ++j) u[j] = 0.0;
                    for (int32_t c = 0; c < dk; ++c) {
                        const double* Sr = S + (int64_t)c * nc;
                        for (int32_t j = 0; j < nc; ++j) u[j] += Sr[j] * bb[c];
                    }
                    /* 2.-3. decay, then subtract a u^T and add k v^T */
                    for (int32_t c = 0; c < dk; ++c) {
                        double* Sr = S + (int64_t)c * nc;
                        for (int32_t j = 0; j < nc; ++j)
                            Sr[j] = al[c] * Sr[j] - aa[c] * u[j] + kk[c] * vv[j];
                    }
                    /* 4. read: o_t = S^T q */
                    if (o) {
                        for (int32_t j = 0; j < nc; ++j) u[j] = 0.0;
                        for (int32_t c = 0; c < dk; ++c) {
                            const double* Sr = S + (int64_t)c * nc;
                            for (int32_t j = 0; j < nc; ++j) u[j] += Sr[j] * qq[c];
                        }
                        for (int32_t j = 0; j < nc; ++j) o[vb + j0 + j] = u[j];
                    }
                }
                if (S_final)
                    for (int32_t c = 0; c < dk; ++c)
                        for (int32_t j = 0; j < nc; ++j)
                            S_final[sbase + (int64_t)c * dv + j0 + j] = S[(int64_t)c * nc + j];
            }
        }
        free(S);
        free(vec);
        free(u);
    }
    return bad ? -6 : 0;
}
