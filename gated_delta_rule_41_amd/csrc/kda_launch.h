// Internal launch interface between the C ABI (kda_abi.hip) and the kernels.
// Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v, *la, *beta;
    float* state;
    void* o;
    int N, H, D;
    bool in_f32, gate_f32, out_f32;
    // the layer epilogue fused in (y in place of o; the inputs' dtype throughout)
    bool epi = false;
    const void* xg = nullptr;
    const float* rms_w = nullptr;
    void* y = nullptr;
};

struct SeqMeta;

// A piece of the chunk slots, [g0, g1): the chunk-parallel kernels cover only
// these slots and index the workspace from g0; the recursion walks each
// sequence's chunks inside the piece. A sequence that continues past the
// piece's entry end (g0 for the forward walk, g1 for the reversed one) starts
// from `cin`; one that continues past the exit end leaves its state in `cout`
// (not written when null). Both are [H][D][D] fp32. An empty sequence belongs
// to the piece holding its slot offset (the last piece also takes offset NC).
// g1 == 0: no piece, every slot.
struct Piece {
    int g0 = 0, g1 = 0;
    int last = 1;
    const float* cin = nullptr;
    float* cout = nullptr;
};

// The fused epilogue's default bound on re-reads of another slab's partial
// sums before a wait gives up (some tens of ms).
constexpr int EPI_SPIN_DEFAULT = 1 << 16;

struct ChunkArgs {
    const void *q, *k, *v, *la, *beta;
    const float* s0;        // may be null
    const int32_t* cu;      // may be null (one sequence)
    SeqMeta* tab = nullptr; // the sequence table built from cu (null when cu is)
    float* s_final;         // may be null
    void* o;
    int N, T, H, D;
    int NC;                 // chunk-slot capacity of the workspace
    bool in_f32, gate_f32, out_f32;
    // workspace arrays (element type bf16 bits or fp32, per in_f32)
    void *qp, *km, *wn, *u, *aqk, *h, *vn;
    float* gam;
    // general DPLR transition only: the low-rank vectors a, b [T, H, D] (bf16)
    // and two more workspace arrays (decayed a transposed; A_qk V)
    bool dplr = false;
    const void *lr_a = nullptr, *lr_b = nullptr;
    void *am = nullptr, *oh = nullptr;
    // backward: fp32 factors whatever the input dtype (the forward recompute),
    // and the state-gradient recursion's extra state-independent term
    bool f32_factors = false;
    const float* pb = nullptr;  // [chunk-head][dv/16][dk/16][64 lanes][4] fp32, or null
    // the layer prologue fused into the preparation (bf16 only): pre-activations
    // and the prologue's parameters replace q, k, v, la, beta; qk_scr holds the
    // q, k rows of chunks that take the exact path ([chunk-head][2][64][D] bf16)
    bool pro = false;
    const void *xq = nullptr, *xk = nullptr, *xv = nullptr, *xa = nullptr, *xb = nullptr;
    const float *wq = nullptr, *wk = nullptr, *wv = nullptr, *A_log = nullptr, *dt_bias = nullptr;
    void* qk_scr = nullptr;
    // the layer epilogue fused into the recursion's output stage (with pro, bf16
    // inputs, d x d heads, N H a multiple of 8): y = RMSNorm(o) * rms_w *
    // sigmoid(xg) in bf16 instead of o. The workgroups of one (sequence, head)
    // share each row's sum of squares through epi_part ([chunk-head][dv/16][64]
    // fp32, set to -1 by the preparation kernel of that chunk-head)
    bool epi = false;
    const void* xg = nullptr;
    const float* rms_w = nullptr;
    void* y = nullptr;
    float* epi_part = nullptr;
    int epi_spin_max = EPI_SPIN_DEFAULT;  // the fused epilogue's bounded wait (re-reads)
    Piece piece;
    int slots() const { return piece.g1 > 0 ? piece.g1 - piece.g0 : NC; }  // chunk slots launched
};

// Backward of kda_chunk_fwd (see kda_bwd.hip).
struct BwdArgs {
    ChunkArgs fwd;    // forward recompute: fp32 factors, h_n and V_new kept
    ChunkArgs rec;    // state-gradient recursion: chunks in reverse, the forward factors in swapped roles
    const float* d_o;  // [T, H, dv]
    float *dq, *dk, *dv, *dla, *dbeta;
    float* scr;        // per chunk-head scratch, bwd_scr_floats(D) floats each (dQ+, dK-)
};
// (the gated key products the forward recompute keeps go to fwd.am, [64][64] fp32 per chunk-head;
// the chunk-parallel backward kernels cover fwd.piece's slots)
__host__ __device__ inline int64_t bwd_scr_floats(int D) { return 2LL * 64 * D; }
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_local(const BwdArgs& a, hipStream_t st);

// The layer's prologue and epilogue around the operator (see kda_layer.hip).
struct LayerArgs {
    int N, T, H, D;
    bool f32;  // element type of every pre-activation and output: fp32, else bf16
    const int32_t* cu;
    // prologue
    const void *xq, *xk, *xv, *xa, *xb;
    const float *wq, *wk, *wv, *A_log, *dt_bias;
    void *q, *k, *v, *la, *beta;
    // epilogue
    const float* o;
    const void* g;
    const float* rms_w;
    void* y;
    // decoding: the convolution's history [N][H][q, k, v][3][D]
    void* cs = nullptr;
};
hipError_t launch_layer_conv_state(const LayerArgs& a, hipStream_t st);
hipError_t launch_layer_decode_prologue(const LayerArgs& a, hipStream_t st);
hipError_t launch_layer_prologue(const LayerArgs& a, hipStream_t st);
hipError_t launch_layer_epilogue(const LayerArgs& a, hipStream_t st);

// Workspace carve-up shared by the size query and the launcher.
struct WsPlan {
    size_t off[8];   // qp, km, wn, u, aqk, gam, h, vn
    size_t total;
};
WsPlan plan_workspace(int64_t NC, int H, int D, bool f32);
// general DPLR transition (16-bit factors): qp, km, am, wn, u, aqk, oh, gam
WsPlan plan_workspace_dplr(int64_t NC, int H, int D);
int64_t chunk_capacity(int N, int64_t T, bool have_cu);

// Opt a kernel into more than 64 KiB of dynamic LDS, once per device.
hipError_t allow_dynamic_lds(const void* kernel, int bytes);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// sequence table from cu_seqlens (kda_seq.hip); tab holds N + 1 entries
hipError_t launch_seq_table(const int32_t* cu, int N, int T, int NC, SeqMeta* tab, hipStream_t st);
inline size_t seq_table_bytes(int N) { return ((size_t)(N + 1) * 16 + 255) / 256 * 256; }
hipError_t launch_prep(const ChunkArgs& a, hipStream_t st);
hipError_t launch_recur(const ChunkArgs& a, hipStream_t st);
hipError_t launch_output(const ChunkArgs& a, hipStream_t st);
hipError_t launch_dplr_prep(const ChunkArgs& a, hipStream_t st);

// With 16-bit operands the state-recursion kernel also computes the chunk
// outputs (h_n and V_new stay on chip); with fp32 operands its LDS cannot
// hold the exchange buffers, and a separate output kernel reads h_n and V_new
// from the workspace.
inline bool output_fused(bool in_f32) { return !in_f32; }

}  // namespace kda
