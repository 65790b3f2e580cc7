/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * KDA is a gated delta-rule recurrence with a per-channel (diagonal) forget
 * gate. For one sequence and one head, with a state S of dk x dv:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                       alpha_t = exp(log_alpha_t)
 *
 * The delta rule with a channel-wise gate is described on the GeekNews "Kimi
 * Linear" summary (pt.news.hada.io topic 31936), sections "Da atenção linear ao
 * Gated DeltaNet" and "Controle fino de memória no Kimi Delta Attention";
 * prefill uses the chunkwise-parallel algorithm of sections "Algoritmo paralelo
 * por chunks" and "Menos computação que o DPLR geral" (fixed-size chunks whose
 * final state seeds the next, WY factors from one UT transform built by forward
 * substitution, matrix-form state update, output = inter-chunk recurrent part +
 * intra-chunk parallel part). Decode is one recurrent step with a fixed-size
 * state (remio.ai "Kimi Linear Acabou de Superar a Atenção Completa em Seus
 * Próprios Termos", section "Por Que a Decodificação de Contexto Longo Coloca a
 * Atenção Completa sob Pressão").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (HIP, gfx950) unless marked host.
 *    Every tensor is dense and contiguous in the layout given; base addresses
 *    must be 16-byte aligned, except beta and cu_seqlens, which need only the
 *    alignment of their element type (KDA_ERR_ALIGN otherwise). The layer
 *    entry points (kda_layer_*) state their own, weaker alignment rules.
 *
 * Entry points
 * ------------
 *  - the operator: kda_chunk_fwd (prefill), kda_decode_step, kda_chunk_bwd,
 *    with their workspace sizes, and kda_dplr_chunk_fwd (the general DPLR
 *    transition, for comparison); kda_chunk_fwd_noalloc (the prefill with a
 *    static workspace, for callers that cannot allocate);
 *  - the layer around it: kda_layer_prologue, kda_layer_epilogue,
 *    kda_layer_chunk_fwd (the prologue fused into the prefill),
 *    kda_layer_fwd (the whole layer: prologue and epilogue fused into the
 *    prefill), and for decoding kda_layer_conv_state,
 *    kda_layer_decode_prologue and kda_layer_decode_step (the decode step
 *    with the epilogue fused in);
 *  - kda_status_str, kda_abi_version.
 *  - Layouts are token-major: q, k, log_alpha [T, H, dk]; v [T, H, dv];
 *    beta [T, H]; o [T, H, dv]; states [N, H, dk, dv] fp32 (dv fastest).
 *  - No query scaling is applied (callers pre-scale q if they want 1/sqrt(dk)).
 *  - Supported head sizes: (dk, dv) in {(64, 64), (128, 128)}.
 *  - Size limits (KDA_ERR_SHAPE beyond them): prefill T_total < 2^31,
 *    H <= 65536 and N * H * 8 < 2^31; decode N * H < 2^31.
 *  - Supported dtypes: in_dtype (q, k, v) and gate_dtype (log_alpha, beta) are
 *    each KDA_BF16 or KDA_F32; out_dtype (o) KDA_F32 or KDA_BF16. With
 *    in_dtype == KDA_BF16 the chunk products run on 16-bit matrix cores with
 *    fp32 accumulation and an fp32 state: fp16 operands for the value path,
 *    where the values themselves (beta v in the WY solve, the corrected values
 *    V_new) and the intra-chunk query-key matrix are carried as two fp16 terms
 *    (hi + lo, about 22 bits) and U is kept in fp32; the gated query-key
 *    products use bf16 operands split into a high and a low part. With KDA_F32
 *    they run on fp32 matrix cores.
 *  - Value range with in_dtype == KDA_BF16 (fp16 operands): the accuracy
 *    holds while |v|, the state entries and the corrected values stay below
 *    about 3e4 (fp16 overflows at 65504) and the values are not much smaller
 *    than 1e-4 in magnitude (fp16 loses precision below 6.1e-5). Tested at the
 *    edges: v and the initial state scaled together by 1e-4 and by 1e4 from
 *    N(0,1) values and an N(0, 0.02) state. Outputs dominated by a carried
 *    state up to 100 times larger than the new values' share (v x 1e-2, or the
 *    initial state x 1e2) are tested too; beyond that the fp16 gated queries
 *    round those rows at 2^-12 of their own size. With fp32 inputs the range
 *    is fp32's.
 *  - log_alpha must be finite (<= 0 for the overflow guarantees; 0 is allowed).
 *    Non-finite inputs give undefined (typically NaN) outputs; inputs are not scanned.
 *  - Ownership: the caller owns every buffer. The library never allocates or
 *    frees device memory and keeps no pointer after a call returns (the one
 *    exception is the static workspace of kda_chunk_fwd_noalloc, which the
 *    HIP runtime allocates with the library's code on each device).
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns without synchronising. Buffers must stay
 *    valid until the stream has passed the enqueued work. No host<->device
 *    copies are made; cu_seqlens is read on the device only.
 *  - Errors: arguments are validated on the host before any HIP call and a
 *    status is returned; nothing is enqueued on failure. KDA_ERR_HIP reports
 *    a launch failure. No C++ exception crosses this boundary.
 *  - Thread safety: every entry point may be called from several host threads
 *    at once; calls on one stream run in order. The library holds no mutable
 *    global state besides lazily filled, read-only caches (kernel attributes
 *    set per device; the static scratch's address per device), except the
 *    static scratch of kda_chunk_fwd_noalloc (see there).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1
#define KDA_CHUNK 64 /* fixed chunk length of the prefill algorithm */

/* Element type codes. The entry points take them as int32_t, so any value may
 * be passed; values other than these return KDA_ERR_UNSUPPORTED. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,       /* a size is out of range (<= 0, too large) */
    KDA_ERR_UNSUPPORTED = 3, /* unsupported (dk, dv) or dtype combination */
    KDA_ERR_ALIGN = 4,       /* a base address is not 16-byte aligned */
    KDA_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap */
    KDA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
    KDA_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed */
} kda_status;

/* Version of this ABI (KDA_ABI_VERSION of the built library). */
int kda_abi_version(void);

/* Static, human-readable name of a status code ("KDA_OK", ...). Never NULL. */
const char* kda_status_str(int status);

/*
 * Bytes of device workspace kda_chunk_fwd needs for a batch of N sequences
 * with T_total tokens in all (host call, no device access). The workspace
 * holds the per-chunk factors (gated queries and keys, WY factors, the
 * intra-chunk query-key matrix, the chunk decay; with fp32 inputs also the
 * chunk-entry states and corrected values) for at most
 * floor((T_total + 63*N) / 64) chunks per head.
 *   bytes: host out-pointer, written on KDA_OK.
 */
kda_status kda_chunk_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t dk,
                                        int32_t dv, int32_t in_dtype, size_t* bytes);

/*
 * Chunkwise prefill of a packed batch: kda_chunk_fwd(q, k, v, log_alpha, beta,
 * initial_state, cu_seqlens) -> (o, final_state).
 *
 *   q, k          [T_total, H, dk] in_dtype
 *   v             [T_total, H, dv] in_dtype
 *   log_alpha     [T_total, H, dk] gate_dtype   (natural-log forget gate per key channel)
 *   beta          [T_total, H]     gate_dtype   (delta-rule write strength)
 *   initial_state [N, H, dk, dv] fp32, or NULL for zero states
 *   cu_seqlens    [N+1] int32 device array of sequence starts (cu[0] = 0,
 *                 non-decreasing, cu[N] = T_total), or NULL for one sequence
 *                 (then N must be 1). Zero-length sequences are allowed (their
 *                 final state equals the initial state). It is read only on the
 *                 device, where a first kernel turns it into a sequence table
 *                 at the end of the workspace: sequence i covers tokens
 *                 [s, e) with s = cu[i] clamped into [0, T_total] and e =
 *                 cu[i+1] clamped into [s, T_total], and chunks beyond the
 *                 workspace's floor((T_total + 63*N) / 64) slots are dropped
 *                 (in order of the sequences). A malformed array thus gives
 *                 defined, in-bounds work on those ranges; o rows no range
 *                 covers are not written, and a row two ranges share holds
 *                 either range's result.
 *   o             [T_total, H, dv] out_dtype, written for every token
 *                 (q, k, v, log_alpha, beta and o may be NULL when T_total == 0)
 *   final_state   [N, H, dk, dv] fp32, or NULL if not wanted. It may be the
 *                 same pointer as initial_state (in-place carry); any other
 *                 overlap with an input is KDA_ERR_ALIAS.
 *   workspace     device buffer of at least kda_chunk_fwd_workspace_size()
 *                 bytes, 256-byte aligned; its contents on entry do not matter
 *                 and are clobbered.
 * Chunks of KDA_CHUNK tokens never cross a sequence boundary; a sequence's last
 * chunk may be partial. The call is deterministic (no atomics): the same inputs
 * give bitwise identical outputs.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                         int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                         int32_t in_dtype, int32_t gate_dtype, int32_t out_dtype, void* o,
                         float* final_state, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * kda_chunk_fwd with timing hooks, for profiling and benchmarking. Arguments
 * and behaviour are those of kda_chunk_fwd; in addition, each non-NULL
 * events[i] (a hipEvent_t created by the caller) is recorded on `stream` at
 * stage boundary i: 0 before the per-chunk preparation kernel, 1 between it
 * and the state-recursion kernel, 2 between that and the output kernel, 3
 * after the output kernel. With bf16 inputs the output is computed inside the
 * state-recursion kernel, so events 2 and 3 are recorded back to back.
 * events may be NULL (then this is kda_chunk_fwd).
 * A failed hipEventRecord returns KDA_ERR_HIP.
 */
kda_status kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* initial_state,
                               const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                               int32_t dk, int32_t dv, int32_t in_dtype, int32_t gate_dtype,
                               int32_t out_dtype, void* o, float* final_state, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events);

/* Largest workspace kda_chunk_fwd_noalloc serves from its static scratch: 64 MiB. */
#define KDA_NOALLOC_WORKSPACE_BYTES (64 * 1024 * 1024)

/*
 * kda_chunk_fwd without a caller-supplied workspace and without any device
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * caller still passes every input and output.
 *
 * The workspace is a static device array of KDA_NOALLOC_WORKSPACE_BYTES that
 * the library holds on each device it runs on until the process ends; the
 * current device's copy is used (stream must belong to the current device).
 * Its address is looked up once per device, on the first call there. The
 * call neither allocates nor frees device memory.
 *
 * Arguments, results, validation and determinism are those of kda_chunk_fwd.
 * In addition, KDA_ERR_WORKSPACE is returned, before any device call, when
 * kda_chunk_fwd_workspace_size(N, T_total, H, dk, dv, in_dtype) exceeds
 * KDA_NOALLOC_WORKSPACE_BYTES (with bf16 inputs at dk = dv = 128: 98,816 bytes
 * per chunk-head, so at most 679 chunk-heads, e.g. H = 32 and 21 chunks of
 * 64 tokens; fp32 inputs need about 2.5 times as much per chunk-head).
 * Every call on one device shares that device's scratch, and each call leaves
 * its contents behind; nothing in it needs to start at zero. Calls that
 * overlap in time on one device (on different streams, or from different host
 * threads without ordering) race on the scratch and give undefined results;
 * calls in order on one stream are safe.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                                 const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                                 int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                                 int32_t in_dtype, int32_t gate_dtype, int32_t out_dtype, void* o,
                                 float* final_state, void* stream);

/*
 * The backward's default bound on the chunk-heads (chunk slots x heads) one
 * piece of its work covers; see kda_chunk_bwd_workspace_size.
 */
#define KDA_BWD_PIECE_CHUNK_HEADS 65536

/*
 * Bytes of device workspace kda_chunk_bwd asks for by default (host call, no
 * device access). Per chunk-head of a piece: the forward recomputed with fp32
 * factors (with the gated key products, h_n and V_new), the state-gradient
 * recursion's operand and outputs, its added term and the local kernel's
 * scratch (one region, used in turn): 459,264 bytes at dk = dv = 128, 213,248
 * at 64. The chunk slots are floor((T_total + 63*N) / 64); while slots x H is
 * at most KDA_BWD_PIECE_CHUNK_HEADS one piece covers them all, else each piece
 * covers floor(KDA_BWD_PIECE_CHUNK_HEADS / H) slots (at least one) and one
 * [H, dk, dv] fp32 state per piece is added (the state at the piece's first
 * slot). At N = 1, T_total = 2^20, H = 32, d = 128: 8 pieces, about 30.1 GB.
 *   bytes: host out-pointer, written on KDA_OK.
 */
kda_status kda_chunk_bwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                                        size_t* bytes);

/*
 * Backward of kda_chunk_fwd: given the gradients of o and of the final states,
 * the gradients of q, k, v, log_alpha, beta and of the initial states. The
 * chunkwise form is differentiated chunk by chunk (GeekNews "Kimi Linear"
 * summary, section "Algoritmo paralelo por chunks", presents it as a training
 * algorithm): the forward is recomputed with fp32 factors, the state gradient
 * runs backwards over the chunks, and the chunk-local adjoints (output, state
 * update, UT transform, gated products and scalings, cumulative gate) follow.
 *
 *   q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, T_total, H, dk,
 *   dv, in_dtype, gate_dtype: as for kda_chunk_fwd
 *   d_o             [T_total, H, dv] fp32, gradient of o
 *   d_final_state   [N, H, dk, dv] fp32, gradient of the final states, or NULL (zero)
 *   dq, dk, dlog_alpha [T_total, H, dk] fp32; dv [T_total, H, dv] fp32;
 *   dbeta [T_total, H] fp32  (outputs, written for every token)
 *   d_initial_state [N, H, dk, dv] fp32 or NULL; it may be the same pointer as
 *                   d_final_state (in place), any other overlap is KDA_ERR_ALIAS
 *   workspace       256-byte aligned; contents on entry do not matter. Its
 *                   size sets the pieces: the call takes the largest piece
 *                   (in chunk slots) whose workspace fits in workspace_bytes,
 *                   all slots if they fit. Any size down to one slot per piece
 *                   works; less is KDA_ERR_WORKSPACE.
 * With more than one piece the forward runs twice: once over all pieces but
 * the last for the states at the pieces' first slots, then piece by piece in
 * reverse with the backward of each piece (the state gradient is handed from
 * piece to piece at the same slots, in fp32 as the recursion carries it), so
 * the gradients are bitwise the same for every piece size.
 * Arithmetic is fp32 throughout (bf16 inputs are widened exactly; every
 * product runs on fp32 matrix cores). The same log_alpha condition as
 * kda_chunk_fwd holds (<= 0 for the overflow guarantees). One piece enqueues
 * five kernels (six with cu_seqlens: the sequence table first); each further
 * piece adds seven. Deterministic: every sum has a fixed order, so equal
 * inputs give bitwise equal gradients.
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                         int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                         int32_t in_dtype, int32_t gate_dtype, const float* d_o,
                         const float* d_final_state, float* dq, float* dk_out, float* dv_out,
                         float* dlog_alpha, float* dbeta, float* d_initial_state, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * The layer's prologue: from the pre-activations (the outputs of a KDA layer's
 * q, k, v, gate and beta projections) to kda_chunk_fwd's inputs (GeekNews
 * "Kimi Linear" summary, section "Configuração do modelo Kimi Linear": short
 * convolution and Swish on q, k, v; L2 normalisation of q and k; a per-channel
 * decay gate through a GDN/Mamba-like decay function):
 *
 *   q = L2(swish(conv(xq))), k = L2(swish(conv(xk))), v = swish(conv(xv)),
 *   log_alpha = -exp(A_log[h]) * softplus(xa + dt_bias[h, c]),  beta = sigmoid(xb)
 *
 * conv: causal depthwise filter of width 4, y[t] = sum_i w[h, c, i] x[t - 3 + i],
 * with x = 0 before the first token of t's sequence (per cu_seqlens);
 * swish(x) = x sigmoid(x); L2(x) = x / sqrt(sum_c x^2 + 1e-6).
 *
 *   xq, xk, xv, xa  [T_total, H, d] dtype;  xb [T_total, H] dtype
 *   wq, wk, wv      [H, d, 4] fp32;  A_log [H] fp32;  dt_bias [H, d] fp32
 *   cu_seqlens      as kda_chunk_fwd (NULL = one sequence, N = 1)
 *   q, k, v, log_alpha [T_total, H, d] dtype;  beta [T_total, H] dtype (outputs,
 *                   ready to pass to kda_chunk_fwd with in_dtype = gate_dtype = dtype)
 * d must be 64 or 128; dtype KDA_BF16 or KDA_F32 (fp32 arithmetic, outputs
 * rounded to nearest even for bf16). The [T_total, H, d] tensors must be aligned
 * to two elements, the others to one (KDA_ERR_ALIGN). No output may overlap an
 * input or another output (KDA_ERR_ALIAS). T_total * H < 2^31. One kernel is
 * enqueued: one wave per head and tile of 16 tokens, the filters in registers.
 */
kda_status kda_layer_prologue(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                              const float* wq, const float* wk, const float* wv, const float* A_log,
                              const float* dt_bias, const int32_t* cu_seqlens, int32_t N, int64_t T_total,
                              int32_t H, int32_t d, int32_t dtype, void* q, void* k, void* v,
                              void* log_alpha, void* beta, void* stream);

/*
 * The layer's convolution history after a prefill, for one-token decoding
 * (the short convolution of kda_layer_prologue is causal, so the next token
 * needs the last three pre-activation rows of q, k, v of its sequence):
 *
 *   conv_state[n, h, m, i, :] = x_m[end_n - 3 + i, h, :]   (0 where before start_n)
 *
 *   xq, xk, xv  [T_total, H, d] dtype (the prefill's pre-activations)
 *   cu_seqlens  as kda_chunk_fwd (NULL = one sequence, N = 1)
 *   conv_state  [N, H, 3 (q, k, v), 3 (oldest first), d] dtype (output)
 * The [.., d] tensors must be aligned to two elements (KDA_ERR_ALIGN); the
 * output may not overlap an input (KDA_ERR_ALIAS). One kernel is enqueued.
 */
kda_status kda_layer_conv_state(const void* xq, const void* xk, const void* xv, const int32_t* cu_seqlens,
                                int32_t N, int64_t T_total, int32_t H, int32_t d, int32_t dtype, void* conv_state,
                                void* stream);

/*
 * kda_layer_prologue for one new token per sequence after the history
 * conv_state (kda_layer_conv_state's layout): the convolution reads the
 * history's three rows, then the new row; the history is then shifted by the
 * new row, in place. With kda_decode_step and kda_layer_epilogue (or with
 * kda_layer_decode_step, which does both in one kernel) this is the layer's
 * decode step; the results equal those of kda_layer_prologue over the
 * whole sequence at its last row.
 *
 *   xq, xk, xv, xa  [N, H, d] dtype;  xb [N, H] dtype (one token per sequence)
 *   conv_state      [N, H, 3, 3, d] dtype (in and out)
 *   wq ... dt_bias  as kda_layer_prologue
 *   q, k, v, log_alpha [N, H, d] dtype; beta [N, H] dtype (outputs, ready for
 *                   kda_decode_step)
 * Alignment and aliasing as kda_layer_prologue (conv_state as the [.., d]
 * tensors; it may not overlap any other argument). N * H < 2^31. One kernel is
 * enqueued.
 */
kda_status kda_layer_decode_prologue(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                                     void* conv_state, const float* wq, const float* wk, const float* wv,
                                     const float* A_log, const float* dt_bias, int32_t N, int32_t H, int32_t d,
                                     int32_t dtype, void* q, void* k, void* v, void* log_alpha, void* beta,
                                     void* stream);

/*
 * Bytes of device workspace kda_layer_chunk_fwd needs (host call, no device
 * access): kda_chunk_fwd's for bf16 inputs, plus 32 KiB per chunk-head at
 * d = 128 (16 KiB at d = 64) for the q, k rows of chunks that take the exact
 * path.
 */
kda_status kda_layer_chunk_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t d, size_t* bytes);

/*
 * kda_layer_prologue and kda_chunk_fwd in one pass (bf16 only): the chunk
 * preparation computes the prologue for its own rows (and the three rows before
 * them) in LDS, rounded to bf16 exactly as kda_layer_prologue stores them, so
 * the results equal those of kda_layer_prologue followed by kda_chunk_fwd with
 * bf16 inputs and fp32 o, without q, k, v, log_alpha, beta ever reaching
 * memory. Arguments as kda_layer_prologue (dtype bf16) and kda_chunk_fwd
 * (initial_state, final_state, workspace, o fp32 [T_total, H, d]); the same
 * alignment, aliasing and size rules. Two kernels are enqueued.
 */
kda_status kda_layer_chunk_fwd(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                               const float* wq, const float* wk, const float* wv, const float* A_log,
                               const float* dt_bias, const float* initial_state, const int32_t* cu_seqlens,
                               int32_t N, int64_t T_total, int32_t H, int32_t d, float* o, float* final_state,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The layer's epilogue (same section: a per-head RMSNorm and a data-dependent
 * output gate before the output projection):
 *
 *   y = o / sqrt(mean_c o^2 + 1e-6) * rms_w[c] * sigmoid(xg)
 *
 *   o      [T_total, H, dv] fp32 (kda_chunk_fwd's output)
 *   xg     [T_total, H, dv] dtype (the output gate's pre-activation)
 *   rms_w  [dv] fp32 (one weight per value channel, shared by the heads)
 *   y      [T_total, H, dv] dtype (output; must not overlap an input)
 * dv must be 64 or 128. o, xg and y must be aligned to two elements, rms_w to
 * one (KDA_ERR_ALIGN). One kernel is enqueued: one wave per four rows.
 */
kda_status kda_layer_epilogue(const float* o, const void* xg, const float* rms_w, int64_t T_total, int32_t H,
                              int32_t dv, int32_t dtype, void* y, void* stream);

/*
 * The layer's decode step after kda_layer_decode_prologue: kda_decode_step
 * (fp32 o) and kda_layer_epilogue in one kernel. The workgroup of a (sequence,
 * head) holds the whole row o, so it normalises and gates it before it leaves:
 * o never reaches memory, and y is bitwise that of the two calls.
 *
 *   q, k, v, log_alpha [N, H, d] dtype; beta [N, H] dtype (one token per
 *                   sequence, as kda_layer_decode_prologue leaves them)
 *   state           [N, H, d, d] fp32, updated in place
 *   xg              [N, H, d] dtype (the output gate's pre-activation)
 *   rms_w           [d] fp32
 *   y               [N, H, d] dtype (output)
 * d is 64 or 128; dtype KDA_BF16 or KDA_F32 for every tensor above but the
 * state and rms_w. q, k, v, log_alpha and state must be 16-byte aligned, beta
 * to its element, xg and y to two elements, rms_w to 4 bytes (KDA_ERR_ALIGN).
 * y and state may not overlap an input or each other (KDA_ERR_ALIAS).
 * N * H < 2^31. One kernel is enqueued.
 */
kda_status kda_layer_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                                 const void* beta, float* state, const void* xg, const float* rms_w, int32_t N,
                                 int32_t H, int32_t d, int32_t dtype, void* y, void* stream);

/*
 * Bytes of device workspace kda_layer_fwd needs on the current device (host
 * call; it reads the device's CU count): kda_layer_chunk_fwd's, plus the
 * epilogue's region: per-row partial sums of squares (32 bytes per token-head
 * at d = 128) when the epilogue is fused for these shapes on this device, else
 * room for the operator's fp32 o (4 d bytes per token-head), which is also the
 * answer when no device can be queried. A call on a device with fewer CUs may
 * need the larger size (KDA_ERR_WORKSPACE).
 *   bytes: host out-pointer, written on KDA_OK.
 */
kda_status kda_layer_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t d, size_t* bytes);

/*
 * The whole layer between the projections, in bf16: kda_layer_prologue,
 * kda_chunk_fwd and kda_layer_epilogue in one call, with the prologue fused
 * into the chunk preparation (as kda_layer_chunk_fwd) and the epilogue fused
 * into the recursion's output stage: o never reaches memory. Arguments as
 * kda_layer_chunk_fwd, plus
 *   xg     [T_total, H, d] bf16 (the output gate's pre-activation)
 *   rms_w  [d] fp32
 *   y      [T_total, H, d] bf16 (output, in place of o)
 * xg and y must be 8-byte aligned and rms_w 4-byte aligned (KDA_ERR_ALIGN); y
 * must not overlap an input, the workspace or final_state, and xg and rms_w must
 * not overlap the workspace or final_state (KDA_ERR_ALIAS).
 *
 * A row's RMSNorm needs all d channels, which the recursion spreads over d/16
 * workgroups of one (sequence, head). The epilogue is fused when those
 * workgroups share an XCD's L2 and all fit on the GPU at once: N * H a
 * multiple of 8 (workgroup ids are dispatched round-robin over the 8 XCDs) and
 * N * H * d / 16 at most the device's CU count. Each workgroup then publishes
 * its slab's per-row sums of squares in the workspace and finishes a chunk's y
 * a turn later from every slab's sums, added in one fixed order. A wait for
 * another slab's sums that has not ended after some tens of ms gives up, and
 * the rows it had still to finish are NaN. That needs other work to keep some
 * of the launch's workgroups off the GPU for that long while others wait: in
 * particular two kda_layer_fwd calls running at the same time on different
 * streams can each hold CUs the other's workgroups need. Run such calls on one
 * stream, or use kda_layer_chunk_fwd and kda_layer_epilogue, which never wait
 * on one another's workgroups. (The bound is 65,536 re-reads of the sums; the
 * environment variable KDA_EPI_SPIN_MAX, a non-negative integer read at each
 * call, replaces it: 0 makes every wait give up at once, every y row NaN, which
 * tests use to exercise that path.) Otherwise the operator writes o to
 * the workspace and the epilogue kernel follows; both ways give the same y up
 * to the order of the sum of squares (one rounding of the RMS). Calls that
 * share a workspace must not run concurrently. Three kernels are enqueued
 * (four with the separate epilogue).
 */
kda_status kda_layer_fwd(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                         const void* xg, const float* wq, const float* wk, const float* wv, const float* A_log,
                         const float* dt_bias, const float* rms_w, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H, int32_t d, void* y,
                         float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace kda_dplr_chunk_fwd needs (host call, no device
 * access): seven 16-bit per-chunk factors and the chunk decay, for at most
 * floor((T_total + 63*N) / 64) chunks per head. in_dtype must be KDA_BF16.
 *   bytes: host out-pointer, written on KDA_OK.
 */
kda_status kda_dplr_chunk_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t dk,
                                             int32_t dv, int32_t in_dtype, size_t* bytes);

/*
 * Chunkwise prefill of the general diagonal-plus-low-rank (DPLR) transition,
 * the operator KDA specialises, for comparison with kda_chunk_fwd:
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *
 * with free low-rank vectors a_t, b_t per (token, head). KDA is the case
 * a = beta k, b = alpha * k with written key beta k (GeekNews "Kimi Linear"
 * summary, section "Menos computação que o DPLR geral": tying both vectors
 * to the key saves two of the four gated intra-chunk matrices and three
 * chunk products).
 *
 *   q, k, a, b    [T_total, H, dk] bf16 (in_dtype must be KDA_BF16)
 *   v             [T_total, H, dv] bf16
 *   log_alpha     [T_total, H, dk] gate_dtype
 *   initial_state, cu_seqlens, o, final_state, workspace: as kda_chunk_fwd
 *                 (workspace sized by kda_dplr_chunk_fwd_workspace_size)
 * Same conventions, size limits, error codes and determinism as
 * kda_chunk_fwd; there is no beta input. Two kernels are enqueued (chunk
 * preparation, then the state recursion with the fused output).
 */
kda_status kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                              const void* log_alpha, const float* initial_state,
                              const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                              int32_t dk, int32_t dv, int32_t in_dtype, int32_t gate_dtype,
                              int32_t out_dtype, void* o, float* final_state, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for N independent sequences, one token each:
 * kda_decode_step(q, k, v, log_alpha, beta, state) -> (o, state').
 *
 *   q, k       [N, H, dk] in_dtype;  v [N, H, dv] in_dtype
 *   log_alpha  [N, H, dk] gate_dtype; beta [N, H] gate_dtype
 *   state      [N, H, dk, dv] fp32, read and overwritten in place with S_t
 *   o          [N, H, dv] out_dtype, o = S_t^T q (the updated state)
 * o must not overlap state or any input (KDA_ERR_ALIAS).
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* beta, float* state, int32_t N, int32_t H, int32_t dk,
                           int32_t dv, int32_t in_dtype, int32_t gate_dtype,
                           int32_t out_dtype, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
