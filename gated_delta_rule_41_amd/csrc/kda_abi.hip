// C ABI of the KDA library: argument validation, workspace carve-up, launches.
// See include/kda.h for the contract of every entry point.
#include "../../include/kda.h"
#include "kda_launch.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <mutex>

namespace kda {

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hipError_t allow_dynamic_lds(const void* kernel, int bytes) {
    // one bit per (kernel, device); the attribute is idempotent, so a race only repeats the call
    struct Entry {
        const void* k;
        std::atomic<uint64_t> devs;
    };
    static Entry table[32];
    static std::atomic<int> used{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const uint64_t bit = 1ull << (dev & 63);
    const int nu = used.load(std::memory_order_acquire);
    for (int i = 0; i < nu; ++i)
        if (table[i].k == kernel && (table[i].devs.load(std::memory_order_acquire) & bit)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    for (int i = 0; i < nu; ++i)
        if (table[i].k == kernel) {
            table[i].devs.fetch_or(bit);
            return hipSuccess;
        }
    static std::mutex mu;
    std::lock_guard<std::mutex> lock(mu);
    const int n2 = used.load();
    for (int i = 0; i < n2; ++i)
        if (table[i].k == kernel) {
            table[i].devs.fetch_or(bit);
            return hipSuccess;
        }
    if (n2 < 32) {
        table[n2].k = kernel;
        table[n2].devs.store(bit);
        used.store(n2 + 1, std::memory_order_release);
    }
    return hipSuccess;
}

int64_t chunk_capacity(int N, int64_t T, bool have_cu) {
    // sum_i ceil(L_i / 64) <= floor((T + 63 N) / 64); one sequence: ceil(T / 64)
    if (!have_cu) return (T + KDA_CHUNK - 1) / KDA_CHUNK;
    return (T + (int64_t)(KDA_CHUNK - 1) * N) / KDA_CHUNK;
}

WsPlan plan_workspace(int64_t NC, int H, int D, bool f32) {
    const size_t es = f32 ? 4 : 2;
    const size_t ch = (size_t)NC * (size_t)H;  // chunk-heads
    const size_t sz[8] = {
        ch * KDA_CHUNK * D * es,       // qp
        ch * D * KDA_CHUNK * es,       // km
        ch * KDA_CHUNK * D * es,       // wn
        ch * KDA_CHUNK * D * 4,        // u (fp32 on both paths)
        ch * KDA_CHUNK * KDA_CHUNK * 4,   // aqk (fp32, or two fp16 planes)
        ch * D * 4,                    // gam
        output_fused(f32) ? 0 : ch * (size_t)D * D * es,   // h (only without the fused output)
        output_fused(f32) ? 0 : ch * KDA_CHUNK * D * es,   // vn
    };
    WsPlan p;
    size_t o = 0;
    for (int i = 0; i < 8; ++i) {
        p.off[i] = o;
        o = align_up(o + sz[i], 256);
    }
    p.total = o;
    return p;
}

WsPlan plan_workspace_dplr(int64_t NC, int H, int D) {
    const size_t ch = (size_t)NC * (size_t)H;
    const size_t f = ch * KDA_CHUNK * D * 2;  // one [64][D] fp16 factor per chunk-head
    const size_t kv = ch * D * (D > KDA_CHUNK ? D : KDA_CHUNK) * 2;  // K-^T V (and the K-^T scratch)
    const size_t sz[8] = {f, kv, f, f, f, ch * KDA_CHUNK * KDA_CHUNK * 2, f, ch * D * 4};
    WsPlan p;
    size_t o = 0;
    for (int i = 0; i < 8; ++i) {
        p.off[i] = o;
        o = align_up(o + sz[i], 256);
    }
    p.total = o;
    return p;
}

}  // namespace kda

using namespace kda;

// Workspace of kda_chunk_fwd_noalloc: one copy per device, allocated by the HIP
// runtime when this code object is loaded and held until the process ends.
// Host code never uses this name as an address (on the host it names a
// stand-in); it uses the device address cached by noalloc_scratch().
static __device__ __align__(256) char scratch[KDA_NOALLOC_WORKSPACE_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per device
// with that device current (each device holds its own copy at its own address).
hipError_t noalloc_scratch(void** out) {
    constexpr int MAXDEV = 64;
    static std::atomic<void*> addr[MAXDEV];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);  // a race stores the same address twice
    }
    *out = p;
    return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned_to(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool dtype_ok(int d) { return d == KDA_F32 || d == KDA_BF16; }
size_t esize(int d) { return d == KDA_F32 ? 4 : 2; }

bool head_ok(int32_t dk, int32_t dv) { return (dk == 64 && dv == 64) || (dk == 128 && dv == 128); }

// T_total < 2^31 tokens and H <= 2^16 heads keep every byte count below 2^64;
// the state recursion launches N * H * dv / 16 <= N * H * 8 workgroups
bool chunk_sizes_ok(int32_t N, int64_t T_total, int32_t H) {
    if (N <= 0 || H <= 0 || H > (1 << 16) || T_total < 0 || T_total >= (int64_t(1) << 31)) return false;
    return (int64_t)N * H * 8 < (int64_t(1) << 31);
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(int s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is out of range";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported head size or dtype";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a base address is not 16-byte aligned";
        case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP call or kernel launch failed";
        default: return "KDA_ERR_UNKNOWN";
    }
}

kda_status kda_chunk_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                                        int32_t in_dtype, size_t* bytes) {
    if (!bytes) return KDA_ERR_NULL;
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv) || !dtype_ok(in_dtype)) return KDA_ERR_UNSUPPORTED;
    // the workspace is sized for the packed case; it also covers one sequence
    const int64_t NC = chunk_capacity(N, T_total, true);
    *bytes = plan_workspace(NC, H, dk, in_dtype == KDA_F32).total + seq_table_bytes(N);
    return KDA_OK;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens, int32_t N, int64_t T_total,
                         int32_t H, int32_t dk, int32_t dv, int32_t in_dtype, int32_t gate_dtype,
                         int32_t out_dtype, void* o, float* final_state, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return kda_chunk_fwd_timed(q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, T_total, H, dk, dv,
                               in_dtype, gate_dtype, out_dtype, o, final_state, workspace, workspace_bytes,
                               stream, nullptr);
}

kda_status kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                               int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                               int32_t in_dtype, int32_t gate_dtype, int32_t out_dtype, void* o,
                               float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                               void* const* events) {
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (T_total > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv) || !dtype_ok(in_dtype) || !dtype_ok(gate_dtype) || !dtype_ok(out_dtype))
        return KDA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(o) ||
        !aligned16(initial_state) || !aligned16(final_state) || !aligned_to(beta, esize(gate_dtype)) ||
        !aligned_to(cu_seqlens, 4))
        return KDA_ERR_ALIGN;
    const size_t T = (size_t)T_total;
    const size_t nqk = T * H * dk * esize(in_dtype), nv = T * H * dv * esize(in_dtype);
    const size_t nla = T * H * dk * esize(gate_dtype), nb = T * H * esize(gate_dtype);
    const size_t no = T * H * dv * esize(out_dtype), ns = (size_t)N * H * dk * dv * 4;
    const size_t ncu = cu_seqlens ? (size_t)(N + 1) * 4 : 0;
    const void* ins[7] = {q, k, v, log_alpha, beta, initial_state, cu_seqlens};
    const size_t nin[7] = {nqk, nqk, nv, nla, nb, ns, ncu};
    for (int i = 0; i < 7; ++i) {
        if (overlaps(o, no, ins[i], nin[i])) return KDA_ERR_ALIAS;
        if (i != 5 && overlaps(final_state, ns, ins[i], nin[i])) return KDA_ERR_ALIAS;
    }
    if (overlaps(o, no, final_state, ns)) return KDA_ERR_ALIAS;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, ns, initial_state, ns))
        return KDA_ERR_ALIAS;

    const bool f32 = in_dtype == KDA_F32;
    const int64_t NC = chunk_capacity(N, T_total, cu_seqlens != nullptr);
    const WsPlan plan = plan_workspace(NC, H, dk, f32);
    const size_t need = plan.total + seq_table_bytes(N);  // the sequence table at the end
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need)
        return KDA_ERR_WORKSPACE;
    for (int i = 0; i < 7; ++i)
        if (overlaps(workspace, need, ins[i], nin[i])) return KDA_ERR_ALIAS;
    if (overlaps(workspace, need, o, no) || overlaps(workspace, need, final_state, ns))
        return KDA_ERR_ALIAS;
    if (NC >= (int64_t(1) << 31) / H) return KDA_ERR_SHAPE;

    char* w = static_cast<char*>(workspace);
    ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.la = log_alpha;
    a.beta = beta;
    a.s0 = initial_state;
    a.cu = cu_seqlens;
    a.s_final = final_state;
    a.o = o;
    a.N = N;
    a.T = (int)T_total;
    a.H = H;
    a.D = dk;
    a.NC = (int)NC;
    a.in_f32 = f32;
    a.gate_f32 = gate_dtype == KDA_F32;
    a.out_f32 = out_dtype == KDA_F32;
    a.qp = w + plan.off[0];
    a.km = w + plan.off[1];
    a.wn = w + plan.off[2];
    a.u = w + plan.off[3];
    a.aqk = w + plan.off[4];
    a.gam = reinterpret_cast<float*>(w + plan.off[5]);
    a.h = w + plan.off[6];
    a.vn = w + plan.off[7];
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        return !events || !events[i] || hipEventRecord(static_cast<hipEvent_t>(events[i]), st) == hipSuccess;
    };
    a.tab = cu_seqlens ? reinterpret_cast<SeqMeta*>(w + plan.total) : nullptr;
    if (!mark(0)) return KDA_ERR_HIP;
    if (cu_seqlens && launch_seq_table(cu_seqlens, N, a.T, a.NC, a.tab, st) != hipSuccess) return KDA_ERR_HIP;
    if (NC > 0 && launch_prep(a, st) != hipSuccess) return KDA_ERR_HIP;
    if (!mark(1)) return KDA_ERR_HIP;
    if (launch_recur(a, st) != hipSuccess) return KDA_ERR_HIP;
    if (!mark(2)) return KDA_ERR_HIP;
    if (NC > 0 && !output_fused(f32) && launch_output(a, st) != hipSuccess) return KDA_ERR_HIP;
    if (!mark(3)) return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status kda_dplr_chunk_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                                             int32_t in_dtype, size_t* bytes) {
    if (!bytes) return KDA_ERR_NULL;
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv) || in_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    *bytes = plan_workspace_dplr(chunk_capacity(N, T_total, true), H, dk).total + seq_table_bytes(N);
    return KDA_OK;
}

kda_status kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                              const void* log_alpha, const float* initial_state, const int32_t* cu_seqlens,
                              int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv, int32_t in_dtype,
                              int32_t gate_dtype, int32_t out_dtype, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (T_total > 0 && (!q || !k || !v || !a || !b || !log_alpha || !o)) return KDA_ERR_NULL;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv) || in_dtype != KDA_BF16 || !dtype_ok(gate_dtype) || !dtype_ok(out_dtype))
        return KDA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) ||
        !aligned16(log_alpha) || !aligned16(o) || !aligned16(initial_state) || !aligned16(final_state) ||
        !aligned_to(cu_seqlens, 4))
        return KDA_ERR_ALIGN;
    const size_t T = (size_t)T_total;
    const size_t nx = T * H * dk * 2, nla = T * H * dk * esize(gate_dtype);
    const size_t no = T * H * dv * esize(out_dtype), ns = (size_t)N * H * dk * dv * 4;
    const size_t ncu = cu_seqlens ? (size_t)(N + 1) * 4 : 0;
    const void* ins[8] = {q, k, v, a, b, log_alpha, initial_state, cu_seqlens};
    const size_t nin[8] = {nx, nx, nx, nx, nx, nla, ns, ncu};
    for (int i = 0; i < 8; ++i) {
        if (overlaps(o, no, ins[i], nin[i])) return KDA_ERR_ALIAS;
        if (i != 6 && overlaps(final_state, ns, ins[i], nin[i])) return KDA_ERR_ALIAS;
    }
    if (overlaps(o, no, final_state, ns)) return KDA_ERR_ALIAS;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, ns, initial_state, ns))
        return KDA_ERR_ALIAS;
    const int64_t NC = chunk_capacity(N, T_total, cu_seqlens != nullptr);
    const WsPlan plan = plan_workspace_dplr(NC, H, dk);
    const size_t need = plan.total + seq_table_bytes(N);  // the sequence table at the end
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need)
        return KDA_ERR_WORKSPACE;
    for (int i = 0; i < 8; ++i)
        if (overlaps(workspace, need, ins[i], nin[i])) return KDA_ERR_ALIAS;
    if (overlaps(workspace, need, o, no) || overlaps(workspace, need, final_state, ns))
        return KDA_ERR_ALIAS;
    if (NC >= (int64_t(1) << 31) / H) return KDA_ERR_SHAPE;

    char* w = static_cast<char*>(workspace);
    ChunkArgs c;
    c.q = q;
    c.k = k;
    c.v = v;
    c.la = log_alpha;
    c.beta = nullptr;
    c.s0 = initial_state;
    c.cu = cu_seqlens;
    c.s_final = final_state;
    c.o = o;
    c.N = N;
    c.T = (int)T_total;
    c.H = H;
    c.D = dk;
    c.NC = (int)NC;
    c.in_f32 = false;
    c.gate_f32 = gate_dtype == KDA_F32;
    c.out_f32 = out_dtype == KDA_F32;
    c.dplr = true;
    c.lr_a = a;
    c.lr_b = b;
    c.qp = w + plan.off[0];
    c.km = w + plan.off[1];
    c.am = w + plan.off[2];
    c.wn = w + plan.off[3];
    c.u = w + plan.off[4];
    c.aqk = w + plan.off[5];
    c.oh = w + plan.off[6];
    c.gam = reinterpret_cast<float*>(w + plan.off[7]);
    c.h = nullptr;
    c.vn = nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c.tab = cu_seqlens ? reinterpret_cast<SeqMeta*>(w + plan.total) : nullptr;
    if (cu_seqlens && launch_seq_table(cu_seqlens, N, c.T, c.NC, c.tab, st) != hipSuccess) return KDA_ERR_HIP;
    if (NC > 0 && launch_dplr_prep(c, st) != hipSuccess) return KDA_ERR_HIP;
    if (launch_recur(c, st) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

// Backward workspace. Per chunk-head of a piece: the forward recomputed with
// fp32 factors (with h_n and V_new), the state-gradient chain's operand U
// (A_qk^T dO) and outputs (its states dh' and dV), the chain's added term
// Q+^T dO (whose room the local kernel's scratch takes over once the chain has
// read it) and the gated key products. With more than one piece, one [H][D][D]
// fp32 state per piece: the forward state at the piece's first slot, later the
// state gradient there. The sequence table last.
struct BwdPlan {
    int64_t pc = 0;  // chunk slots per piece
    int64_t np = 1;  // pieces
    size_t f = 0, ru = 0, rh = 0, rv = 0, pb = 0, pk = 0, ck = 0, tab = 0, total = 0;
};

static BwdPlan plan_bwd(int64_t NC, int H, int D, int N, int64_t pc) {
    BwdPlan p;
    p.pc = pc;
    p.np = NC > 0 ? (NC + pc - 1) / pc : 1;
    const size_t ch = (size_t)pc * H;
    const size_t scr = (size_t)bwd_scr_floats(D) > (size_t)D * D ? (size_t)bwd_scr_floats(D) : (size_t)D * D;
    size_t o = plan_workspace(pc, H, D, true).total;
    p.ru = o;
    o = align_up(o + ch * KDA_CHUNK * D * 4, 256);
    p.rh = o;
    o = align_up(o + ch * D * D * 4, 256);
    p.rv = o;
    o = align_up(o + ch * KDA_CHUNK * D * 4, 256);
    p.pb = o;
    o = align_up(o + ch * scr * 4, 256);
    p.pk = o;
    o = align_up(o + ch * KDA_CHUNK * KDA_CHUNK * 4, 256);
    p.ck = o;
    o = align_up(o + (p.np > 1 ? (size_t)p.np * H * D * D * 4 : 0), 256);
    p.tab = o;
    p.total = o + seq_table_bytes(N);
    return p;
}

// the size query's piece: every slot when the chunk-heads fit the default
// bound, else as many slots as fit it
static int64_t bwd_default_piece(int64_t NC, int H) {
    if (NC * H <= KDA_BWD_PIECE_CHUNK_HEADS) return NC;
    const int64_t pc = KDA_BWD_PIECE_CHUNK_HEADS / H;
    return pc > 0 ? pc : 1;
}

// the largest piece whose plan fits `bytes`; -1 when none does (0 when there
// are no chunk slots)
static int64_t bwd_fit_piece(int64_t NC, int H, int D, int N, size_t bytes) {
    if (NC == 0) return plan_bwd(0, H, D, N, 0).total <= bytes ? 0 : -1;
    const size_t per = plan_bwd(1, H, D, 0, 1).ck;  // bytes per chunk slot (every head)
    int64_t pc = NC;
    while (pc > 0) {
        const BwdPlan p = plan_bwd(NC, H, D, N, pc);
        if (p.total <= bytes) return pc;
        // the bytes that do not scale with the piece at this piece count (a
        // smaller piece only adds boundary states, so the guess never overshoots)
        const size_t fixed = p.total - (size_t)pc * per;
        const int64_t next = fixed < bytes ? (int64_t)((bytes - fixed) / per) : 0;
        pc = next < pc ? next : pc - 1;
    }
    return -1;
}

static void carve(ChunkArgs& a, char* base, int64_t NC, int H, int D) {
    const WsPlan p = plan_workspace(NC, H, D, true);
    a.qp = base + p.off[0];
    a.km = base + p.off[1];
    a.wn = base + p.off[2];
    a.u = base + p.off[3];
    a.aqk = base + p.off[4];
    a.gam = reinterpret_cast<float*>(base + p.off[5]);
    a.h = base + p.off[6];
    a.vn = base + p.off[7];
}

kda_status kda_chunk_bwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                                        size_t* bytes) {
    if (!bytes) return KDA_ERR_NULL;
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    const int64_t NC = chunk_capacity(N, T_total, true);
    *bytes = plan_bwd(NC, H, dk, N, bwd_default_piece(NC, H)).total;
    return KDA_OK;
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens, int32_t N, int64_t T_total,
                         int32_t H, int32_t dk, int32_t dv, int32_t in_dtype, int32_t gate_dtype,
                         const float* d_o, const float* d_final_state, float* dq, float* dk_out, float* dv_out,
                         float* dlog_alpha, float* dbeta, float* d_initial_state, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (T_total > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk_out || !dv_out ||
                        !dlog_alpha || !dbeta))
        return KDA_ERR_NULL;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv) || !dtype_ok(in_dtype) || !dtype_ok(gate_dtype)) return KDA_ERR_UNSUPPORTED;
    const void* al[] = {q, k, v, log_alpha, initial_state, d_o, d_final_state, dq, dk_out, dv_out, dlog_alpha,
                        d_initial_state};
    for (const void* p : al)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    if (!aligned_to(beta, esize(gate_dtype)) || !aligned_to(dbeta, 4) || !aligned_to(cu_seqlens, 4))
        return KDA_ERR_ALIGN;
    const size_t T = (size_t)T_total;
    const size_t nqk = T * H * dk * esize(in_dtype), nv = T * H * dv * esize(in_dtype);
    const size_t nla = T * H * dk * esize(gate_dtype), nb = T * H * esize(gate_dtype);
    const size_t ns = (size_t)N * H * dk * dv * 4, ncu = cu_seqlens ? (size_t)(N + 1) * 4 : 0;
    const size_t ndo = T * H * dv * 4, ng = T * H * dk * 4, ngv = T * H * dv * 4, ngb = T * H * 4;
    const void* ins[8] = {q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_o};
    const size_t nin[8] = {nqk, nqk, nv, nla, nb, ns, ncu, ndo};
    const void* dfin = d_final_state;
    void* outs[6] = {dq, dk_out, dv_out, dlog_alpha, dbeta, d_initial_state};
    const size_t nout[6] = {ng, ng, ngv, ng, ngb, ns};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 8; ++j)
            if (overlaps(outs[i], nout[i], ins[j], nin[j])) return KDA_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], nout[i], outs[j], nout[j])) return KDA_ERR_ALIAS;
        // the initial states' gradient may replace the final states' (in-place)
        if (!(i == 5 && outs[i] == dfin) && overlaps(outs[i], nout[i], dfin, ns)) return KDA_ERR_ALIAS;
    }
    const int64_t NC = chunk_capacity(N, T_total, cu_seqlens != nullptr);
    if (NC >= (int64_t(1) << 31) / H) return KDA_ERR_SHAPE;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return KDA_ERR_WORKSPACE;
    const int64_t pc = bwd_fit_piece(NC, H, dk, N, workspace_bytes);
    if (pc < 0) return KDA_ERR_WORKSPACE;
    const BwdPlan pl = plan_bwd(NC, H, dk, N, pc);
    const size_t need = pl.total;
    for (int j = 0; j < 8; ++j)
        if (overlaps(workspace, need, ins[j], nin[j])) return KDA_ERR_ALIAS;
    for (int i = 0; i < 6; ++i)
        if (overlaps(workspace, need, outs[i], nout[i])) return KDA_ERR_ALIAS;
    if (overlaps(workspace, need, dfin, ns)) return KDA_ERR_ALIAS;

    char* w = static_cast<char*>(workspace);
    BwdArgs b;
    ChunkArgs& F = b.fwd;
    F.q = q;
    F.k = k;
    F.v = v;
    F.la = log_alpha;
    F.beta = beta;
    F.s0 = initial_state;
    F.cu = cu_seqlens;
    F.s_final = nullptr;
    F.o = nullptr;
    F.N = N;
    F.T = (int)T_total;
    F.H = H;
    F.D = dk;
    F.NC = (int)NC;
    F.in_f32 = in_dtype == KDA_F32;
    F.gate_f32 = gate_dtype == KDA_F32;
    F.out_f32 = true;
    F.f32_factors = true;
    carve(F, w, pc, H, dk);
    F.am = w + pl.pk;  // the prep keeps the gated key products there
    ChunkArgs& R = b.rec;
    R = F;
    R.am = nullptr;
    R.s0 = d_final_state;
    R.s_final = d_initial_state;
    // the state-gradient chain reads the forward's factors in swapped roles (K- as
    // its "-W", (-W)^T as its "K-^T", the same gamma) and walks the chunks in reverse;
    // of its own arrays it has U, h and V_new
    R.qp = R.aqk = nullptr;
    R.u = w + pl.ru;
    R.h = w + pl.rh;
    R.vn = w + pl.rv;
    R.wn = F.km;
    R.km = F.wn;
    R.gam = F.gam;
    R.pb = reinterpret_cast<const float*>(w + pl.pb);
    b.d_o = d_o;
    b.dq = dq;
    b.dk = dk_out;
    b.dv = dv_out;
    b.dla = dlog_alpha;
    b.dbeta = dbeta;
    b.scr = reinterpret_cast<float*>(w + pl.pb);  // after the chain has read the added term
    hipStream_t st = static_cast<hipStream_t>(stream);
    F.tab = R.tab = cu_seqlens ? reinterpret_cast<SeqMeta*>(w + pl.tab) : nullptr;
    if (cu_seqlens && launch_seq_table(cu_seqlens, N, F.T, F.NC, F.tab, st) != hipSuccess) return KDA_ERR_HIP;
    if (pl.np <= 1) {
        if (NC > 0 && launch_prep(F, st) != hipSuccess) return KDA_ERR_HIP;
        if (NC > 0 && launch_recur(F, st) != hipSuccess) return KDA_ERR_HIP;
        if (NC > 0 && launch_bwd_prep(b, st) != hipSuccess) return KDA_ERR_HIP;
        if (launch_recur(R, st) != hipSuccess) return KDA_ERR_HIP;
        if (NC > 0 && launch_bwd_local(b, st) != hipSuccess) return KDA_ERR_HIP;
        return KDA_OK;
    }
    // In pieces of pc chunk slots: the forward states at the pieces' first slots
    // (checkpoint p, written by piece p - 1), then the pieces in reverse, each
    // recomputing its forward from its checkpoint and handing the state gradient
    // at its first slot to the piece before it (through the same checkpoint).
    float* ck = reinterpret_cast<float*>(w + pl.ck);
    const size_t cks = (size_t)H * dk * dk;
    auto piece = [&](ChunkArgs& A, int64_t p, const float* cin, float* cout) {
        A.piece.g0 = (int)(p * pc);
        A.piece.g1 = (int)((p + 1) * pc < NC ? (p + 1) * pc : NC);
        A.piece.last = A.piece.g1 == NC;
        A.piece.cin = cin;
        A.piece.cout = cout;
    };
    for (int64_t p = 0; p + 1 < pl.np; ++p) {
        piece(F, p, ck + p * cks, ck + (p + 1) * cks);
        if (launch_prep(F, st) != hipSuccess) return KDA_ERR_HIP;
        if (launch_recur(F, st) != hipSuccess) return KDA_ERR_HIP;
    }
    for (int64_t p = pl.np - 1; p >= 0; --p) {
        piece(F, p, ck + p * cks, nullptr);
        piece(R, p, p + 1 < pl.np ? ck + (p + 1) * cks : nullptr, ck + p * cks);
        if (launch_prep(F, st) != hipSuccess) return KDA_ERR_HIP;
        if (launch_recur(F, st) != hipSuccess) return KDA_ERR_HIP;
        if (launch_bwd_prep(b, st) != hipSuccess) return KDA_ERR_HIP;
        if (launch_recur(R, st) != hipSuccess) return KDA_ERR_HIP;
        if (launch_bwd_local(b, st) != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

kda_status kda_layer_prologue(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                              const float* wq, const float* wk, const float* wv, const float* A_log,
                              const float* dt_bias, const int32_t* cu_seqlens, int32_t N, int64_t T_total,
                              int32_t H, int32_t d, int32_t dtype, void* q, void* k, void* v, void* log_alpha,
                              void* beta, void* stream) {
    if (!chunk_sizes_ok(N, T_total, H) || T_total * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (!head_ok(d, d) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
    if (T_total > 0 && (!xq || !xk || !xv || !xa || !xb || !wq || !wk || !wv || !A_log || !dt_bias || !q || !k ||
                        !v || !log_alpha || !beta))
        return KDA_ERR_NULL;
    const size_t es = esize(dtype), T = (size_t)T_total;
    const size_t nx = T * H * d * es, nb = T * H * es, nw = (size_t)H * d * 4 * 4, nh = (size_t)H * 4,
                 nd = (size_t)H * d * 4, ncu = cu_seqlens ? (size_t)(N + 1) * 4 : 0;
    const void* ins[11] = {xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, cu_seqlens};
    const size_t nin[11] = {nx, nx, nx, nx, nb, nw, nw, nw, nh, nd, ncu};
    void* outs[5] = {q, k, v, log_alpha, beta};
    const size_t nout[5] = {nx, nx, nx, nx, nb};
    // [T, H, d] tensors move in channel pairs: 2 * es bytes
    for (int i = 0; i < 11; ++i)
        if (!aligned_to(ins[i], i < 4 ? 2 * es : i == 4 ? es : 4)) return KDA_ERR_ALIGN;
    for (int i = 0; i < 5; ++i) {
        if (!aligned_to(outs[i], i < 4 ? 2 * es : es)) return KDA_ERR_ALIGN;
        for (int j = 0; j < 11; ++j)
            if (overlaps(outs[i], nout[i], ins[j], nin[j])) return KDA_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], nout[i], outs[j], nout[j])) return KDA_ERR_ALIAS;
    }
    if (T_total == 0) return KDA_OK;
    LayerArgs a{};
    a.N = N;
    a.T = (int)T_total;
    a.H = H;
    a.D = d;
    a.f32 = dtype == KDA_F32;
    a.cu = cu_seqlens;
    a.xq = xq, a.xk = xk, a.xv = xv, a.xa = xa, a.xb = xb;
    a.wq = wq, a.wk = wk, a.wv = wv, a.A_log = A_log, a.dt_bias = dt_bias;
    a.q = q, a.k = k, a.v = v, a.la = log_alpha, a.beta = beta;
    return launch_layer_prologue(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// bytes of the fused layer forward's workspace: the forward's (16-bit factors)
// and the exact path's q, k rows ([chunk-head][2][64][d] bf16)
static size_t layer_fwd_workspace(int64_t NC, int H, int d, size_t* scr_off) {
    const size_t base = plan_workspace(NC, H, d, false).total;
    if (scr_off) *scr_off = base;
    return base + align_up((size_t)NC * H * 2 * KDA_CHUNK * d * 2, 256);
}

kda_status kda_layer_chunk_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t d, size_t* bytes) {
    if (!bytes) return KDA_ERR_NULL;
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (!head_ok(d, d)) return KDA_ERR_UNSUPPORTED;
    *bytes = layer_fwd_workspace(chunk_capacity(N, T_total, true), H, d, nullptr) + seq_table_bytes(N);
    return KDA_OK;
}

// The whole layer's epilogue (kda_layer_fwd): y = RMSNorm(o) rms_w sigmoid(xg).
struct LayerEpi {
    const void* xg;
    const float* rms_w;
    void* y;
};

// The epilogue joins the recursion's output stage when the slab workgroups of
// every (sequence, head) share an XCD (N H a multiple of 8, so that their ids
// are congruent mod 8) and every workgroup of the launch fits on the GPU at once
// (one per CU); otherwise o goes to the workspace and the epilogue kernel follows.
static bool layer_epi_fused(int N, int H, int d) {
    if (((int64_t)N * H) % 8 != 0) return false;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    return (int64_t)N * H * (d / 16) <= cus;
}

// bytes of kda_layer_fwd's own region after the fused layer forward's
// workspace: the fused epilogue's per-row partial sums ([chunk-head][d/16][64]
// fp32), or the operator's fp32 o for the separate epilogue kernel
static size_t layer_epi_bytes(int64_t NC, int64_t T, int H, int d, bool fused) {
    return fused ? align_up((size_t)NC * H * (d / 16) * 64 * 4, 256) : align_up((size_t)T * H * d * 4, 256);
}

// The fused epilogue's bound on re-reads before a wait gives up: the default,
// or KDA_EPI_SPIN_MAX from the environment (a non-negative integer; read at
// each call), which tests set to 0 to take the give-up path.
static int epi_spin_max() {
    const char* e = std::getenv("KDA_EPI_SPIN_MAX");
    if (!e || !*e) return EPI_SPIN_DEFAULT;
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (*end != '\0' || v < 0 || v > (1L << 30)) return EPI_SPIN_DEFAULT;
    return (int)v;
}

static kda_status layer_fwd_impl(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                                 const float* wq, const float* wk, const float* wv, const float* A_log,
                                 const float* dt_bias, const float* initial_state, const int32_t* cu_seqlens,
                                 int32_t N, int64_t T_total, int32_t H, int32_t d, float* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream, const LayerEpi* ep) {
    if (!chunk_sizes_ok(N, T_total, H) || T_total * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (!head_ok(d, d)) return KDA_ERR_UNSUPPORTED;
    if (T_total > 0 && (!xq || !xk || !xv || !xa || !xb || !wq || !wk || !wv || !A_log || !dt_bias ||
                        (ep ? (!ep->xg || !ep->rms_w || !ep->y) : !o)))
        return KDA_ERR_NULL;
    const size_t T = (size_t)T_total;
    const size_t nx = T * H * d * 2, nb = T * H * 2, nw = (size_t)H * d * 4 * 4, nh = (size_t)H * 4,
                 nd = (size_t)H * d * 4, ncu = cu_seqlens ? (size_t)(N + 1) * 4 : 0;
    const size_t no = T * H * d * 4, ns = (size_t)N * H * d * d * 4;
    const void* ins[12] = {xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, cu_seqlens, initial_state};
    const size_t nin[12] = {nx, nx, nx, nx, nb, nw, nw, nw, nh, nd, ncu, ns};
    for (int i = 0; i < 12; ++i)  // [T, H, d] inputs move in bf16 channel pairs
        if (!aligned_to(ins[i], i < 4 ? 4 : i == 4 ? 2 : i == 11 ? 16 : 4)) return KDA_ERR_ALIGN;
    if (!aligned16(o) || !aligned16(final_state)) return KDA_ERR_ALIGN;
    const int64_t NC = chunk_capacity(N, T_total, cu_seqlens != nullptr);
    if (NC >= (int64_t(1) << 31) / H) return KDA_ERR_SHAPE;
    size_t scr_off = 0;
    const size_t wlayer = layer_fwd_workspace(NC, H, d, &scr_off);
    const bool fused_epi = ep && layer_epi_fused(N, H, d);
    const size_t wbase = wlayer + (ep ? layer_epi_bytes(NC, T_total, H, d, fused_epi) : 0);
    const size_t wbytes = wbase + seq_table_bytes(N);  // the sequence table at the end
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < wbytes) return KDA_ERR_WORKSPACE;
    for (int i = 0; i < 12; ++i) {
        if (overlaps(o, no, ins[i], nin[i]) || overlaps(workspace, wbytes, ins[i], nin[i])) return KDA_ERR_ALIAS;
        if (i != 11 && overlaps(final_state, ns, ins[i], nin[i])) return KDA_ERR_ALIAS;
    }
    if (overlaps(o, no, final_state, ns) || overlaps(workspace, wbytes, o, no) ||
        overlaps(workspace, wbytes, final_state, ns))
        return KDA_ERR_ALIAS;
    if (ep) {
        // xg [T, H, d] and y [T, H, d] bf16 move 4 channels (8 bytes) per lane; rms_w [d]
        const size_t ny = T * H * d * 2, nr = (size_t)d * 4;
        if (!aligned_to(ep->xg, 8) || !aligned_to(ep->y, 8) || !aligned_to(ep->rms_w, 4)) return KDA_ERR_ALIGN;
        const void* eins[2] = {ep->xg, ep->rms_w};
        const size_t nein[2] = {ny, nr};
        for (int i = 0; i < 12; ++i)
            if (overlaps(ep->y, ny, ins[i], nin[i])) return KDA_ERR_ALIAS;
        for (int i = 0; i < 2; ++i)
            if (overlaps(ep->y, ny, eins[i], nein[i]) || overlaps(workspace, wbytes, eins[i], nein[i]) ||
                overlaps(final_state, ns, eins[i], nein[i]))
                return KDA_ERR_ALIAS;
        if (overlaps(ep->y, ny, workspace, wbytes) || overlaps(ep->y, ny, final_state, ns)) return KDA_ERR_ALIAS;
    }
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, ns, initial_state, ns))
        return KDA_ERR_ALIAS;
    const WsPlan plan = plan_workspace(NC, H, d, false);
    char* w = static_cast<char*>(workspace);
    ChunkArgs a;
    a.q = a.k = a.v = a.la = a.beta = nullptr;  // computed inside the preparation
    a.s0 = initial_state;
    a.cu = cu_seqlens;
    a.s_final = final_state;
    a.o = o;
    a.N = N;
    a.T = (int)T_total;
    a.H = H;
    a.D = d;
    a.NC = (int)NC;
    a.in_f32 = false;
    a.gate_f32 = false;
    a.out_f32 = true;
    a.qp = w + plan.off[0];
    a.km = w + plan.off[1];
    a.wn = w + plan.off[2];
    a.u = w + plan.off[3];
    a.aqk = w + plan.off[4];
    a.gam = reinterpret_cast<float*>(w + plan.off[5]);
    a.h = w + plan.off[6];
    a.vn = w + plan.off[7];
    a.pro = true;
    a.xq = xq, a.xk = xk, a.xv = xv, a.xa = xa, a.xb = xb;
    a.wq = wq, a.wk = wk, a.wv = wv, a.A_log = A_log, a.dt_bias = dt_bias;
    a.qk_scr = w + scr_off;
    if (fused_epi) {
        a.epi = true;
        a.out_f32 = false;
        a.o = nullptr;
        a.xg = ep->xg, a.rms_w = ep->rms_w, a.y = ep->y;
        a.epi_part = reinterpret_cast<float*>(w + wlayer);
        a.epi_spin_max = epi_spin_max();
    } else if (ep) {
        a.o = w + wlayer;  // the operator's o, then the epilogue kernel
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    a.tab = cu_seqlens ? reinterpret_cast<SeqMeta*>(w + wbase) : nullptr;
    if (cu_seqlens && launch_seq_table(cu_seqlens, N, a.T, a.NC, a.tab, st) != hipSuccess) return KDA_ERR_HIP;
    if (NC > 0 && launch_prep(a, st) != hipSuccess) return KDA_ERR_HIP;
    if (launch_recur(a, st) != hipSuccess) return KDA_ERR_HIP;
    if (ep && !fused_epi && T_total > 0) {
        LayerArgs la{};
        la.N = N, la.T = (int)T_total, la.H = H, la.D = d;
        la.f32 = false;
        la.o = static_cast<const float*>(a.o);
        la.g = ep->xg, la.rms_w = ep->rms_w, la.y = ep->y;
        if (launch_layer_epilogue(la, st) != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

kda_status kda_layer_chunk_fwd(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                               const float* wq, const float* wk, const float* wv, const float* A_log,
                               const float* dt_bias, const float* initial_state, const int32_t* cu_seqlens,
                               int32_t N, int64_t T_total, int32_t H, int32_t d, float* o, float* final_state,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return layer_fwd_impl(xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, initial_state, cu_seqlens, N, T_total, H,
                          d, o, final_state, workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_layer_fwd_workspace_size(int32_t N, int64_t T_total, int32_t H, int32_t d, size_t* bytes) {
    if (!bytes) return KDA_ERR_NULL;
    if (!chunk_sizes_ok(N, T_total, H)) return KDA_ERR_SHAPE;
    if (!head_ok(d, d)) return KDA_ERR_UNSUPPORTED;
    const int64_t NC = chunk_capacity(N, T_total, true);
    *bytes = layer_fwd_workspace(NC, H, d, nullptr) + layer_epi_bytes(NC, T_total, H, d, layer_epi_fused(N, H, d)) +
             seq_table_bytes(N);
    return KDA_OK;
}

kda_status kda_layer_fwd(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                         const void* xg, const float* wq, const float* wk, const float* wv, const float* A_log,
                         const float* dt_bias, const float* rms_w, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H, int32_t d, void* y,
                         float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    const LayerEpi ep{xg, rms_w, y};
    return layer_fwd_impl(xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, initial_state, cu_seqlens, N, T_total, H,
                          d, nullptr, final_state, workspace, workspace_bytes, stream, &ep);
}

kda_status kda_layer_conv_state(const void* xq, const void* xk, const void* xv, const int32_t* cu_seqlens,
                                int32_t N, int64_t T_total, int32_t H, int32_t d, int32_t dtype, void* conv_state,
                                void* stream) {
    if (!chunk_sizes_ok(N, T_total, H) || T_total * H >= (int64_t(1) << 31) || (int64_t)N * H >= (int64_t(1) << 31))
        return KDA_ERR_SHAPE;
    if (!cu_seqlens && N != 1) return KDA_ERR_SHAPE;
    if (!head_ok(d, d) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
    if (!conv_state || (T_total > 0 && (!xq || !xk || !xv))) return KDA_ERR_NULL;
    const size_t es = esize(dtype), nx = (size_t)T_total * H * d * es, ncs = (size_t)N * H * 9 * d * es;
    const size_t ncu = cu_seqlens ? (size_t)(N + 1) * 4 : 0;
    if (!aligned_to(xq, 2 * es) || !aligned_to(xk, 2 * es) || !aligned_to(xv, 2 * es) ||
        !aligned_to(conv_state, 2 * es) || !aligned_to(cu_seqlens, 4))
        return KDA_ERR_ALIGN;
    if (overlaps(conv_state, ncs, xq, nx) || overlaps(conv_state, ncs, xk, nx) || overlaps(conv_state, ncs, xv, nx) ||
        overlaps(conv_state, ncs, cu_seqlens, ncu))
        return KDA_ERR_ALIAS;
    LayerArgs a{};
    a.N = N;
    a.T = (int)T_total;
    a.H = H;
    a.D = d;
    a.f32 = dtype == KDA_F32;
    a.cu = cu_seqlens;
    a.xq = xq, a.xk = xk, a.xv = xv;
    a.cs = conv_state;
    return launch_layer_conv_state(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_layer_decode_prologue(const void* xq, const void* xk, const void* xv, const void* xa, const void* xb,
                                     void* conv_state, const float* wq, const float* wk, const float* wv,
                                     const float* A_log, const float* dt_bias, int32_t N, int32_t H, int32_t d,
                                     int32_t dtype, void* q, void* k, void* v, void* log_alpha, void* beta,
                                     void* stream) {
    if (N <= 0 || H <= 0 || H > 65536 || (int64_t)N * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!head_ok(d, d) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
    if (!xq || !xk || !xv || !xa || !xb || !conv_state || !wq || !wk || !wv || !A_log || !dt_bias || !q || !k ||
        !v || !log_alpha || !beta)
        return KDA_ERR_NULL;
    const size_t es = esize(dtype), NH = (size_t)N * H;
    const size_t nx = NH * d * es, nb = NH * es, ncs = NH * 9 * d * es, nw = (size_t)H * d * 16, nh = (size_t)H * 4,
                 nd = (size_t)H * d * 4;
    const void* ins[11] = {xq, xk, xv, xa, xb, wq, wk, wv, A_log, dt_bias, conv_state};
    const size_t nin[11] = {nx, nx, nx, nx, nb, nw, nw, nw, nh, nd, ncs};
    void* outs[5] = {q, k, v, log_alpha, beta};
    const size_t nout[5] = {nx, nx, nx, nx, nb};
    for (int i = 0; i < 11; ++i)  // [N, H, d] tensors and the history move in channel pairs
        if (!aligned_to(ins[i], i < 4 || i == 10 ? 2 * es : i == 4 ? es : 4)) return KDA_ERR_ALIGN;
    for (int i = 0; i < 10; ++i)  // the history is updated in place
        if (overlaps(conv_state, ncs, ins[i], nin[i])) return KDA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i) {
        if (!aligned_to(outs[i], i < 4 ? 2 * es : es)) return KDA_ERR_ALIGN;
        for (int j = 0; j < 11; ++j)
            if (overlaps(outs[i], nout[i], ins[j], nin[j])) return KDA_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], nout[i], outs[j], nout[j])) return KDA_ERR_ALIAS;
    }
    LayerArgs a{};
    a.N = N;
    a.H = H;
    a.D = d;
    a.f32 = dtype == KDA_F32;
    a.xq = xq, a.xk = xk, a.xv = xv, a.xa = xa, a.xb = xb;
    a.wq = wq, a.wk = wk, a.wv = wv, a.A_log = A_log, a.dt_bias = dt_bias;
    a.q = q, a.k = k, a.v = v, a.la = log_alpha, a.beta = beta;
    a.cs = conv_state;
    return launch_layer_decode_prologue(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_layer_epilogue(const float* o, const void* g, const float* rms_w, int64_t T_total, int32_t H,
                              int32_t dv, int32_t dtype, void* y, void* stream) {
    if (T_total < 0 || T_total >= (int64_t(1) << 31) || H <= 0 || H > 65536 || T_total * H >= (int64_t(1) << 31))
        return KDA_ERR_SHAPE;
    if (!(dv == 64 || dv == 128) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
    if (T_total > 0 && (!o || !g || !rms_w || !y)) return KDA_ERR_NULL;
    const size_t es = esize(dtype), n = (size_t)T_total * H * dv;
    // rows move in channel pairs
    if (!aligned_to(o, 8) || !aligned_to(g, 2 * es) || !aligned_to(rms_w, 4) || !aligned_to(y, 2 * es))
        return KDA_ERR_ALIGN;
    if (overlaps(y, n * es, o, n * 4) || overlaps(y, n * es, g, n * es) || overlaps(y, n * es, rms_w, (size_t)dv * 4))
        return KDA_ERR_ALIAS;
    if (T_total == 0) return KDA_OK;
    LayerArgs a{};
    a.T = (int)T_total;
    a.H = H;
    a.D = dv;
    a.f32 = dtype == KDA_F32;
    a.o = o, a.g = g, a.rms_w = rms_w, a.y = y;
    return launch_layer_epilogue(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                           float* state, int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t in_dtype,
                           int32_t gate_dtype, int32_t out_dtype, void* o, void* stream) {
    if (!q || !k || !v || !log_alpha || !beta || !state || !o) return KDA_ERR_NULL;
    if (N <= 0 || H <= 0 || (int64_t)N * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!head_ok(dk, dv) || !dtype_ok(in_dtype) || !dtype_ok(gate_dtype) || !dtype_ok(out_dtype))
        return KDA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(state) ||
        !aligned16(o) || !aligned_to(beta, esize(gate_dtype)))
        return KDA_ERR_ALIGN;
    const size_t NH = (size_t)N * H;
    const size_t no = NH * dv * esize(out_dtype), ns = NH * dk * dv * 4;
    const void* ins[5] = {q, k, v, log_alpha, beta};
    const size_t nin[5] = {NH * dk * esize(in_dtype), NH * dk * esize(in_dtype), NH * dv * esize(in_dtype),
                           NH * dk * esize(gate_dtype), NH * esize(gate_dtype)};
    for (int i = 0; i < 5; ++i)
        if (overlaps(o, no, ins[i], nin[i]) || overlaps(state, ns, ins[i], nin[i])) return KDA_ERR_ALIAS;
    if (overlaps(o, no, state, ns)) return KDA_ERR_ALIAS;
    DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.la = log_alpha;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.N = N;
    a.H = H;
    a.D = dk;
    a.in_f32 = in_dtype == KDA_F32;
    a.gate_f32 = gate_dtype == KDA_F32;
    a.out_f32 = out_dtype == KDA_F32;
    if (launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status kda_layer_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                                 const void* beta, float* state, const void* xg, const float* rms_w, int32_t N,
                                 int32_t H, int32_t d, int32_t dtype, void* y, void* stream) {
    if (!q || !k || !v || !log_alpha || !beta || !state || !xg || !rms_w || !y) return KDA_ERR_NULL;
    if (N <= 0 || H <= 0 || (int64_t)N * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!head_ok(d, d) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(state) ||
        !aligned_to(beta, es) || !aligned_to(xg, 2 * es) || !aligned_to(y, 2 * es) || !aligned_to(rms_w, 4))
        return KDA_ERR_ALIGN;
    const size_t NH = (size_t)N * H;
    const size_t ny = NH * d * es, ns = NH * d * d * 4;
    const void* ins[7] = {q, k, v, log_alpha, beta, xg, rms_w};
    const size_t nin[7] = {NH * d * es, NH * d * es, NH * d * es, NH * d * es, NH * es, NH * d * es, (size_t)d * 4};
    for (int i = 0; i < 7; ++i)
        if (overlaps(y, ny, ins[i], nin[i]) || overlaps(state, ns, ins[i], nin[i])) return KDA_ERR_ALIAS;
    if (overlaps(y, ny, state, ns)) return KDA_ERR_ALIAS;
    DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.la = log_alpha;
    a.beta = beta;
    a.state = state;
    a.o = nullptr;
    a.N = N;
    a.H = H;
    a.D = d;
    a.in_f32 = a.gate_f32 = dtype == KDA_F32;
    a.out_f32 = true;
    a.epi = true;
    a.xg = xg;
    a.rms_w = rms_w;
    a.y = y;
    if (launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                                 const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                                 int32_t N, int64_t T_total, int32_t H, int32_t dk, int32_t dv,
                                 int32_t in_dtype, int32_t gate_dtype, int32_t out_dtype, void* o,
                                 float* final_state, void* stream) {
    // A call whose workspace would not fit the scratch is refused before any
    // device call. Sizes the workspace query rejects go to kda_chunk_fwd's own
    // validation with no workspace, which reports them exactly as it would.
    size_t need = 0;
    const bool sized = kda_chunk_fwd_workspace_size(N, T_total, H, dk, dv, in_dtype, &need) == KDA_OK;
    if (sized && need > (size_t)KDA_NOALLOC_WORKSPACE_BYTES) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (sized && noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
    return kda_chunk_fwd_timed(q, k, v, log_alpha, beta, initial_state, cu_seqlens, N, T_total, H, dk, dv,
                               in_dtype, gate_dtype, out_dtype, o, final_state, ws,
                               sized ? (size_t)KDA_NOALLOC_WORKSPACE_BYTES : 0, stream, nullptr);
}

}  // extern "C"
