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
// only through column j), so one workgroup owns a 16-wide value-column slab of
// one (sequence, head). Its compute wave keeps the dk x 16 fp32 slab of S in
// accumulator registers for the whole sequence. Thanks to the split k order
// (kda_common.h) the accumulator tiles of S and of V_new are directly the B
// operands of the next product: no LDS round trip and no cross-lane shuffle on
// the dependency chain.
//
// Feeding the chain: two producer waves stream each chunk's factors (-W, K-^T,
// this slab's U, gamma) into a ring of LDS slots with direct global->LDS loads,
// RING - 1 chunks ahead of the compute wave. A wave's vector-memory queue
// returns in order, so keeping these loads off the compute wave means its
// chain never waits behind a memory round trip; producers wait for their own
// loads with an explicit vmcnt and hand slots over at one barrier per chunk.
// Inside a slot, 16-byte granules (one fp16 operand fragment each) are
// XOR-swizzled within each 256-byte segment (granule c stored at
// c ^ ((c >> 4) & 15)) so that the compute wave's operand reads (16 rows x 4
// k-groups per instruction) hit distinct banks.
//
// Workgroup -> work mapping is XCD-aware: workgroups are dispatched round-robin
// over the 8 XCDs, so the dv/16 slabs of one (sequence, head) get ids that are
// congruent mod 8 and land on the same XCD, where they share the L2 copy of
// that head's W and K- factors.
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_prep_util.h"  // split_pos
#include "kda_layer_util.h"  // sigm, LAYER_EPS (the fused layer epilogue)

#include <type_traits>

namespace kda {

template <int D, bool F32, bool FUSED, bool DPLR = false>
struct RecurPlan {
    using E = typename Pol<F32>::E;
    // KDA with 16-bit factors: U is fp32 and the compute wave loads its slab
    // itself, one chunk ahead (it is not in the ring); V_new is two-term fp16
    static constexpr bool HP = FUSED && !DPLR && !F32;
    static constexpr int FB = 64 * D * (int)sizeof(E);   // bytes of -W (and of K-^T) per chunk-head
    static constexpr int UB = HP ? 0 : 64 * 16 * (int)sizeof(E);  // bytes of one slab's U in the ring
    static constexpr int UBG = HP ? 64 * 16 * 4 : UB;    // bytes of one slab's U in the workspace
    static constexpr int GB = D * 4;                     // bytes of gamma
    static constexpr int GPAD = 1024;                    // gamma region rounded up to one whole load
    static constexpr int SLOT = 2 * FB + UB + GPAD;      // one ring slot
    // with the fused output: two buffers of (h_n slab [D x 16], V_new slab [64 x 16],
    // with HP its hi then lo part)
    static constexpr int HVS = (D * 16 + (HP ? 2 : 1) * 64 * 16) * (int)sizeof(E);
    static constexpr int HV = FUSED ? 2 * HVS : 0;
    // DPLR: two buffers of the state-independent update K-^T V of this slab
    // (fp16, accumulator-tile order), by chunk parity
    static constexpr int PBS = (D / 16) * 64 * 4 * 2;
    static constexpr int PB = DPLR ? 2 * PBS : 0;
    static_assert(PBS % 1024 == 0, "K-^T V share in whole 1 KiB loads");
    // target of the L2 warm-up loads (never read); DPLR has no room for it and
    // aims them at the unread tail of ring slot 0's gamma region instead
    static constexpr int WARM = !DPLR ? 256 : 0;
    // unfused (fp32 factors): NCW compute waves exchange their row tiles of the
    // state ([D/16][64 lanes][4]) and of V_new ([4][64][4]) through LDS
    static constexpr int NCW = FUSED ? 1 : 4;
    static constexpr int XCH = FUSED ? 0 : (D / 16 + 4) * 64 * 4 * (int)sizeof(E);
    static constexpr int RING = (4 * SLOT + HV + PB + WARM + XCH <= 160 * 1024) ? 4 : 2;
    static constexpr int LDS = RING * SLOT + HV + PB + WARM + XCH;
    static_assert(!DPLR || (FUSED && GPAD - GB >= 256), "warm-up target in the gamma pad");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    // global->LDS loads per chunk and producer wave (16 bytes per lane, 1 KiB per load)
    static constexpr int OPS_W = FB / 1024, OPS_U = UB / 1024, OPS_G = 1;
    static constexpr int OPS0 = OPS_W + OPS_U;   // producer 0: -W and U
    static constexpr int OPS1 = OPS_W + OPS_G;   // producer 1: K-^T and gamma
    static constexpr int OPS = OPS0 > OPS1 ? OPS0 : OPS1;
    static_assert((RING - 2) * OPS <= 63, "in-flight loads must fit the 6-bit vmcnt");
    static_assert(FB % 1024 == 0 && UB % 1024 == 0 && GB <= GPAD, "slot parts are whole 1 KiB loads");
    // L2 warm-up (fused kernel): the 128-byte lines of one chunk-head's -W, K-^T,
    // Q+ and A_qk are shared out over the head's D/16 slab workgroups; a second
    // load covers this slab's U and the head's gamma
    static constexpr int LINES_W = FB / 128, LINES_A = 64 * 64 * (int)sizeof(E) * (HP ? 2 : 1) / 128;
    static constexpr int LINES = 3 * LINES_W + LINES_A;
    static constexpr int LINES_PER = (LINES + D / 16 - 1) / (D / 16);
    static constexpr int WARM_LOADS = (LINES_PER + 63) / 64;  // first-part loads per lane and chunk
    static constexpr int LINES_U = UBG / 128, LINES_G = GB / 128;
    // DPLR: the second load also covers this slab's A_qk V tiles, a third its K-^T V share
    static constexpr int LINES_O = DPLR ? UB / 128 : 0, LINES_KV = DPLR ? PBS / 128 : 0;
    static constexpr int LINES_2 = LINES_U + LINES_G + LINES_O;
    static_assert(!FUSED || (LINES_PER <= 128 && LINES_2 <= 64 && LINES_KV <= 64), "warm-up loads per chunk");
    static constexpr int AHEAD = 3;  // chunks warmed ahead of the compute wave (2..6 measured; 3 best)
};

// granule swizzle of the ring slots; fp32 fragments span two granules, so the
// fp32 path keeps the plain layout
template <bool F32>
__device__ __forceinline__ int swz(int c) {
    if constexpr (F32) return c;
    return c ^ ((c >> 4) & 15);
}

__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// wait until at most n of this wave's vector-memory operations are outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until this wave's LDS operations have completed
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Workgroup barrier for an LDS exchange between waves: this wave's LDS writes
// complete first (s_barrier alone does not wait for them), and the compiler may
// move no memory access across it (the builtin is not a fence)
__device__ __forceinline__ void lds_exchange_barrier() {
    wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// wait until only the loads of the `after` chunks issued last are outstanding
template <int OPS, int RING>
__device__ __forceinline__ void wait_chunks(int after) {
    if constexpr (RING >= 4) {
        if (after >= 2) {
            wait_vm<2 * OPS>();
            return;
        }
    }
    if constexpr (RING >= 3) {
        if (after >= 1) {
            wait_vm<OPS>();
            return;
        }
    }
    wait_vm<0>();
}

// Producer: issue the global->LDS loads of one chunk (this producer's half).
// Both producers issue exactly OPS loads per chunk, so one vmcnt threshold
// serves both.
template <int D, bool F32, bool FUSED, bool DPLR>
__device__ __forceinline__ void produce(const Ws<typename Pol<F32>::E>& ws, int64_t chh, int ct, int pw, int l,
                                       char* slot) {
    using PL = RecurPlan<D, F32, FUSED, DPLR>;
    if (pw == 0) {
        const char* wp = reinterpret_cast<const char*>(ws.wn + chh * 64 * D);
#pragma unroll
        for (int j = 0; j < PL::OPS_W; ++j) dma16(wp + swz<F32>(64 * j + l) * 16, slot + j * 1024);
        if constexpr (PL::OPS_U > 0) {
            const char* up = reinterpret_cast<const char*>(ws.u + chh * 64 * D + (int64_t)ct * 4 * 64 * 4);
#pragma unroll
            for (int j = 0; j < PL::OPS_U; ++j) dma16(up + (64 * j + l) * 16, slot + 2 * PL::FB + j * 1024);
            // pad to OPS loads: repeat the last U load (same source, same destination)
#pragma unroll
            for (int j = PL::OPS0; j < PL::OPS; ++j)
                dma16(up + (64 * (PL::OPS_U - 1) + l) * 16, slot + 2 * PL::FB + (PL::OPS_U - 1) * 1024);
        } else {
            // pad to OPS loads: repeat the last -W load (same source, same destination)
#pragma unroll
            for (int j = PL::OPS0; j < PL::OPS; ++j)
                dma16(wp + swz<F32>(64 * (PL::OPS_W - 1) + l) * 16, slot + (PL::OPS_W - 1) * 1024);
        }
    } else {
        // the state update's key factor: K-^T (KDA) or A-^T (DPLR)
        const char* kp = reinterpret_cast<const char*>((DPLR ? ws.am : ws.km) + chh * D * 64);
#pragma unroll
        for (int j = 0; j < PL::OPS_W; ++j) dma16(kp + swz<F32>(64 * j + l) * 16, slot + PL::FB + j * 1024);
        // gamma: lanes past its end re-load its first granule into the unread tail of its region
        const char* gp = reinterpret_cast<const char*>(ws.gam + chh * D) + (l * 16 < PL::GB ? l * 16 : 0);
        dma16(gp, slot + 2 * PL::FB + PL::UB);
        // pad to OPS loads: repeat the gamma load (same source, same destination)
#pragma unroll
        for (int j = PL::OPS1; j < PL::OPS; ++j) dma16(gp, slot + 2 * PL::FB + PL::UB);
    }
}

// L2 warm-up: 4-byte global->LDS loads, one per 128-byte line, touch this
// workgroup's share of one chunk's -W, K-^T, Q+, A_qk lines and its own U and
// gamma lines, so that the producers' DMA and the output waves' loads of that
// chunk, a few chain steps later, hit the XCD's L2 instead of HBM. The LDS
// target is a scratch area nobody reads.
template <int D, bool F32, bool FUSED, bool DPLR>
__device__ __forceinline__ void warm_chunk(const Ws<typename Pol<F32>::E>& ws, int64_t chh, int ct, int l,
                                           char* dst) {
    using PL = RecurPlan<D, F32, FUSED, DPLR>;
#pragma unroll
    for (int k = 0; k < PL::WARM_LOADS; ++k) {
        const int li = 64 * k + l;
        int L = ct * PL::LINES_PER + (li < PL::LINES_PER ? li : PL::LINES_PER - 1);
        L = L < PL::LINES ? L : PL::LINES - 1;
        const char* p;
        if (L < PL::LINES_W)
            p = reinterpret_cast<const char*>(ws.wn + chh * 64 * D) + L * 128;
        else if (L < 2 * PL::LINES_W)
            p = reinterpret_cast<const char*>((DPLR ? ws.am : ws.km) + chh * 64 * D) + (L - PL::LINES_W) * 128;
        else if (L < 3 * PL::LINES_W)
            p = reinterpret_cast<const char*>(ws.qp + chh * 64 * D) + (L - 2 * PL::LINES_W) * 128;
        else
            p = reinterpret_cast<const char*>(ws.aqk + chh * 64 * 64 * (PL::HP ? 2 : 1)) + (L - 3 * PL::LINES_W) * 128;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)p,
                                         (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    }
    const int m = l < PL::LINES_2 ? l : 0;
    const char* pu;
    if (m < PL::LINES_U)
        pu = (PL::HP ? reinterpret_cast<const char*>(ws.uf + chh * 64 * D + (int64_t)ct * 4 * 64 * 4)
                     : reinterpret_cast<const char*>(ws.u + chh * 64 * D + (int64_t)ct * 4 * 64 * 4)) +
             m * 128;
    else if (m < PL::LINES_U + PL::LINES_G)
        pu = reinterpret_cast<const char*>(ws.gam + chh * D) + (m - PL::LINES_U) * 128;
    else
        pu = reinterpret_cast<const char*>(ws.oh + chh * 64 * D + (int64_t)ct * 4 * 64 * 4) +
             (m - PL::LINES_U - PL::LINES_G) * 128;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)pu,
                                     (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    if constexpr (DPLR) {
        const int k = l < PL::LINES_KV ? l : 0;
        const char* pk = reinterpret_cast<const char*>(ws.km + chh * D * D) + (int64_t)ct * PL::PBS + k * 128;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)pk,
                                         (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    }
}

// With FUSED, two more waves compute each chunk's output O = Q+ h_n + A_qk V_new
// for this slab's 16 columns, one chunk behind the compute wave: the compute
// wave leaves h_n and V_new in an LDS buffer (two buffers, by chunk parity)
// instead of the workspace, and the output waves, taking alternate chunks,
// fetch Q+ and A_qk into registers one chunk ahead. Waves: 0 compute, 1-2
// output, 3-4 producers, 5 L2 warm-up (6: DPLR state-independent update).
// Every wave executes the same 1 + nch barriers.
//
// Unfused (fp32 factors, 16x16x4 fp32 products): one chain step is 256
// products at d = 128, too many for one wave's matrix core, so four compute
// waves share it (each the state's row tiles of one quarter and one 16-row
// tile of V_new), and the tiles meet in LDS twice per chunk. Waves: 0-3
// compute, 4-5 producers, 6 L2 warm-up; every wave executes 1 + 2 nch
// barriers.
//
// DPLR (the general transition, factors from kda_dplr_prep.hip): the chain is
// the same with -u = -U' + (-W') h in place of V_new and A-^T in place of
// K-^T, plus two state-independent terms: the state update adds K-^T V and the
// output adds A_qk V (from the workspace, as the output accumulators' start).
// The prep kernel computes K-^T V; a seventh wave copies this slab's share of
// it into an LDS buffer (by chunk parity) one chunk ahead of the compute wave.
// The layer epilogue fused into the output stage (GeekNews "Kimi Linear"
// summary, section "Configuração do modelo Kimi Linear": a per-head RMSNorm and
// a data-dependent output gate before the output projection):
//     y = o / sqrt(mean over the head's dv channels of o^2 + eps) * rms_w * sigmoid(xg)
// The dv channels of a row are spread over the dv/16 slab workgroups of the
// (sequence, head). Workgroup ids congruent mod 8 run on one XCD (the dispatch
// is round-robin over the 8 XCDs, and the slab ids of a unit are congruent when
// N H is a multiple of 8), so they share one L2: each output wave publishes the
// per-row sums of squares of its slab there (part, which the preparation kernel
// fills with -1, so a slot's sign bit says whether it has been written yet),
// and finishes that chunk's y in its next free iteration (while the other
// output wave computes), from the sums of every slab, added in one fixed order
// so that every workgroup normalises with the same value. By then the other
// slabs have published: the chain does not wait for them.
struct EpiArgs {
    const uint16_t* xg;  // [T, H, dv] bf16, the output gate's pre-activation
    const float* rms_w;  // [dv]
    uint16_t* y;         // [T, H, dv] bf16
    float* part;         // [chunk-head][dv/16][64] fp32, -1 before the launch
    // Re-reads of a chunk's partial sums before the wait gives up (each an L2
    // round trip and a short sleep; EPI_SPIN_DEFAULT, 65,536, is some tens of ms
    // in all); a wave that gave up once waits no more, and the rows of every
    // chunk it has not normalised are stored as NaN, so a launch whose
    // workgroups cannot meet still ends. The caller runs this path only when
    // every workgroup of the launch fits on the GPU at once, where the slabs of
    // a unit advance together. 0 makes every wait give up at once.
    int spin_max;
};

// The value lane l ^ 16 (l ^ 32) of the wave holds, by gfx950's lane swaps: with
// both operands x, permlane16_swap leaves each odd row of its first result
// holding the even row before it and each even row of its second result the
// odd row after it (permlane32_swap likewise for the two halves). No LDS traffic.
__device__ __forceinline__ float lane_xor16(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(((threadIdx.x >> 5) & 1) ? r[0] : r[1]);
}

template <int D, bool F32, bool FUSED, bool OUT_F32, bool DPLR = false, bool ADDP = false, bool EPI = false>
__global__ __launch_bounds__(FUSED ? (DPLR ? 448 : 384) : 448) void recur_kernel(const float* __restrict__ s0,
                                                                  float* __restrict__ s_final,
                                                                  const SeqMeta* __restrict__ tab, int N, int T,
                                                                  int H, Ws<typename Pol<F32>::E> ws,
                                                                  void* __restrict__ o, Piece pc, EpiArgs ep) {
    using P = Pol<F32>;
    using E = typename P::E;
    using Frag = typename P::Frag;
    using PL = RecurPlan<D, F32, FUSED, DPLR>;
    static_assert(!DPLR || (FUSED && !F32), "the DPLR chain runs on 16-bit factors with the fused output");
    static_assert(!ADDP || (F32 && !FUSED), "the added state term is for the fp32 unfused chain");
    static_assert(!EPI || (FUSED && !F32 && !DPLR && !OUT_F32), "the fused epilogue is for the 16-bit KDA chain");
    constexpr int NS = D / 32;
    constexpr int NT = D / 16;  // row tiles over dk == column slabs over dv
    constexpr int RING = PL::RING;
    constexpr int OPS = PL::OPS;
    // With the fused output the compute wave reads chunk c + 1's -W fragments
    // while chunk c's key-value products run, so the producers keep one more
    // chunk landed ahead of each barrier (the 4-slot ring has room for it).
    constexpr int LOOK = (FUSED && RING >= 4) ? 1 : 0;

    extern __shared__ __align__(16) char ring[];

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
    if (unit >= NU) return;  // uniform over the workgroup
    const int seq = unit / H, h = unit % H;
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;

    const SeqMeta sq = seq_info(tab, T, seq);
    int co = sq.coff, nch = sq.nch;
    // the state the walk starts from and the one it leaves (base of this unit's [D][D])
    const float* s_in = s0 ? s0 + (int64_t)unit * D * D : nullptr;
    float* s_out = s_final ? s_final + (int64_t)unit * D * D : nullptr;
    if (pc.g1 > 0) {
        // only this sequence's chunks inside the piece; a walk that enters or
        // leaves through a cut takes its state from cin or leaves it in cout
        const int lo = co > pc.g0 ? co : pc.g0, hi = co + nch < pc.g1 ? co + nch : pc.g1;
        if (nch == 0 ? !(co >= pc.g0 && (co < pc.g1 || pc.last)) : lo >= hi) return;  // uniform
        const bool cut_lo = nch > 0 && lo > co, cut_hi = nch > 0 && hi < co + nch;
        if (ADDP ? cut_hi : cut_lo) s_in = pc.cin ? pc.cin + (int64_t)h * D * D : nullptr;
        if (ADDP ? cut_lo : cut_hi) s_out = pc.cout ? pc.cout + (int64_t)h * D * D : nullptr;
        co = lo - pc.g0;  // workspace slots count from the piece's start
        nch = nch > 0 ? hi - lo : 0;
    }
    char* hvbase = ring + RING * PL::SLOT;  // h_n / V_new exchange buffers (FUSED)
    char* pbase = hvbase + PL::HV;          // K-^T V buffers (DPLR)

    if (FUSED && (wv == 1 || wv == 2)) {
        // ---------------- output waves: wave 1 + p computes the outputs of the
        // chunks j = p (mod 2) in iteration j + 1, once the compute wave has left
        // h_j and V_j in the exchange buffer j & 1.
        const int p = wv - 1;
        const int tstart = sq.start;
        const int len = sq.len;
        Frag qa[4][NS], aa[4][2];
        Frag al[PL::HP ? 4 : 1][2];  // HP: the low plane of A_qk
        u32x2_t ohr[4];  // DPLR: this slab's A_qk V tiles (fp16)
        u32x2_t xgr[EPI ? 4 : 1];  // EPI: the gate's pre-activation at this lane's 4 columns of rows 16 I + n
        float wc[4];     // EPI: rms_w at this lane's columns 16 ct + 4 g .. + 3
        bool epi_gave_up = false;  // EPI: a wait of this wave gave up (it waits no more)
        if constexpr (EPI) {
#pragma unroll
            for (int i = 0; i < 4; ++i) wc[i] = ep.rms_w[16 * ct + 4 * g + i];
        }
        auto issue = [&](int c) {
            const int64_t chh = (int64_t)(co + c) * H + h;
            if constexpr (EPI) {
                // rows past the sequence's end read its last row (not used)
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int t = tstart + min(64 * c + 16 * I + n, len - 1);
                    xgr[I] = *reinterpret_cast<const u32x2_t*>(ep.xg + ((int64_t)t * H + h) * D + 16 * ct + 4 * g);
                }
            }
            const E* qp = ws.qp + chh * 64 * D;
            const E* ap = ws.aqk + chh * 64 * 64 * (PL::HP ? 2 : 1);
            if constexpr (DPLR) {
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    ohr[I] = *reinterpret_cast<const u32x2_t*>(ws.oh + chh * 64 * D + (((int64_t)ct * 4 + I) * 64 + l) * 4);
            }
            // HP: Q+ and A_qk in fragment order (each fragment a contiguous 1 KiB);
            // DPLR: row-major, split order
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    qa[I][s] = P::load(qp + (PL::HP ? ((I * NS + s) * 64 + l) * 8 : ((16 * I + n) * NS + s) * 32 + g * 8));
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (16 * I + 15 >= 32 * s) {
                        const int at = PL::HP ? ((I * 2 + s) * 64 + l) * 8 : ((16 * I + n) * 2 + s) * 32 + g * 8;
                        aa[I][s] = P::load(ap + at);
                        if constexpr (PL::HP) al[I][s] = P::load(ap + 64 * 64 + at);
                    }
        };
        // chunk c's output tiles from the exchange buffer and the operands in registers
        auto compute = [&](int c, f32x4_t (&acc)[4]) {
            const E* hb = reinterpret_cast<const E*>(hvbase + (c & 1) * PL::HVS);
            const E* vb = hb + D * 16;
            if constexpr (DPLR) {
                // keep the conversion below the barrier that precedes this call:
                // hoisted above it, it would make the wave wait there for every
                // load it has in flight
#pragma unroll
                for (int I = 0; I < 4; ++I) asm volatile("" : "+v"(ohr[I]));
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if constexpr (DPLR)
                    acc[I] = f32x4_t{h2f(ohr[I][0] & 0xffffu), h2f(ohr[I][0] >> 16), h2f(ohr[I][1] & 0xffffu),
                                     h2f(ohr[I][1] >> 16)};
                else
                    acc[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            // HP: the output is formed transposed (each product's operands
            // swapped), so lane n + 16 g holds row 16 I + n at columns 4 g .. 4 g + 3
            // of the slab and stores them as one vector
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const Frag bh = P::load(hb + (s * 64 + l) * 8);
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if constexpr (PL::HP)
                        P::mma(acc[I], bh, qa[I][s]);
                    else
                        P::mma(acc[I], qa[I][s], bh);
                }
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const Frag bv = P::load(vb + (s * 64 + l) * 8);
                if constexpr (PL::HP) {
                    // A_qk V_new with both operands two-term: lo hi + hi lo + hi hi
                    const Frag bvl = P::load(vb + (2 * 64 + s * 64 + l) * 8);
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        if (16 * I + 15 >= 32 * s) {
                            P::mma(acc[I], bv, al[I][s]);
                            P::mma(acc[I], bvl, aa[I][s]);
                            P::mma(acc[I], bv, aa[I][s]);
                        }
                } else {
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        if (16 * I + 15 >= 32 * s) P::mma(acc[I], aa[I][s], bv);
                }
            }
        };
        // only a sequence's last chunk can be partial; every other chunk stores
        // all 64 rows without a per-row branch
        auto store = [&](int c, auto masked, const f32x4_t (&acc)[4]) {
            const int t0 = tstart + 64 * c;
            const int L = min(64, len - 64 * c);
            if constexpr (PL::HP) {
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int rr = 16 * I + n;
                    if (!decltype(masked)::value || rr < L) {
                        const int64_t oi = ((int64_t)(t0 + rr) * H + h) * D + 16 * ct + 4 * g;
                        if constexpr (OUT_F32) {
                            *reinterpret_cast<f32x4_t*>(static_cast<float*>(o) + oi) = acc[I];
                        } else {
                            u32x2_t pk;
                            pk[0] = pack2bf(acc[I][0], acc[I][1]);
                            pk[1] = pack2bf(acc[I][2], acc[I][3]);
                            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o) + oi) = pk;
                        }
                    }
                }
                return;
            }
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * I + 4 * g + i;
                    if (!decltype(masked)::value || rr < L) {
                        const int64_t oi = ((int64_t)(t0 + rr) * H + h) * D + 16 * ct + n;
                        if constexpr (OUT_F32)
                            static_cast<float*>(o)[oi] = acc[I][i];
                        else
                            static_cast<uint16_t*>(o)[oi] = f2bf(acc[I][i]);
                    }
                }
        };
        // EPI: y instead of o. Lane n + 16 g holds row 16 I + n at columns
        // 4 g .. 4 g + 3 of the slab (I = 0..3).
        constexpr int NSL = D / 16;  // slab workgroups per (sequence, head)
        auto prec = [&](int c) { return ep.part + ((int64_t)(co + c) * H + h) * NSL * 64; };  // [slab][64 rows]
        // this slab's sum of squares per row (the lane's 4 columns, then the 4
        // lanes of the row), published as one contiguous 256-byte record: lane
        // n + 16 g writes row 16 g + n
        auto publish = [&](int c, const f32x4_t (&acc)[4]) {
            float ss[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                float x = acc[I][0] * acc[I][0] + acc[I][1] * acc[I][1];
                x += acc[I][2] * acc[I][2] + acc[I][3] * acc[I][3];
                x += lane_xor16(x);
                x += lane_xor32(x);
                ss[I] = x;
            }
            prec(c)[ct * 64 + 16 * g + n] = g == 0 ? ss[0] : g == 1 ? ss[1] : g == 2 ? ss[2] : ss[3];
        };
        // the partial sums this lane adds for its rows: slabs g and g + 4
        auto load_parts = [&](int c, float (&pv)[4][2]) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float* rp = prec(c) + 16 * I + n;
                pv[I][0] = __hip_atomic_load(rp + g * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                pv[I][1] = NSL > 4 ? __hip_atomic_load(rp + (g + 4) * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0.f;
            }
        };
        auto all_in = [&](const float (&pv)[4][2]) {
            uint32_t sgn = 0;
#pragma unroll
            for (int I = 0; I < 4; ++I) sgn |= __float_as_uint(pv[I][0]) | __float_as_uint(pv[I][1]);
            return __all((sgn >> 31) == 0);
        };
        // until every slab's sums of chunk c are in pv (re-read while not)
        auto ensure_in = [&](int c, float (&pv)[4][2]) {
            const int smax = ep.spin_max;
            int it = epi_gave_up ? smax : 0;
            while (it < smax && !all_in(pv)) {
                __builtin_amdgcn_s_sleep(1);
                load_parts(c, pv);
                ++it;
            }
            if (it >= smax) epi_gave_up = true;
        };
        auto finish_y_m = [&](int c, auto masked, const f32x4_t (&acc)[4], const u32x2_t (&xg)[4],
                              const float (&pv)[4][2]) {
            // the sum over every slab of a row in one order for all of them: lane g
            // adds slabs g and g + 4, then xor 16, then xor 32
            float r[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                float a = pv[I][0] + pv[I][1];
                a += lane_xor16(a);
                a += lane_xor32(a);
                r[I] = epi_gave_up ? __builtin_nanf("") : rsqrtf(a * (1.f / D) + LAYER_EPS);
            }
            const int t0 = tstart + 64 * c;
            const int L = min(64, len - 64 * c);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int rr = 16 * I + n;
                if (!decltype(masked)::value || rr < L) {
                    float yv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t gw = xg[I][i >> 1];
                        const float x = __uint_as_float((i & 1) ? (gw & 0xffff0000u) : (gw << 16));
                        yv[i] = acc[I][i] * r[I] * wc[i] * sigm(x);
                    }
                    u32x2_t pk;
                    pk[0] = pack2bf(yv[0], yv[1]);
                    pk[1] = pack2bf(yv[2], yv[3]);
                    *reinterpret_cast<u32x2_t*>(ep.y + ((int64_t)(t0 + rr) * H + h) * D + 16 * ct + 4 * g) = pk;
                }
            }
        };
        // only a sequence's last chunk can be partial
        auto finish_y = [&](int c, const f32x4_t (&acc)[4], const u32x2_t (&xg)[4], const float (&pv)[4][2]) {
            if (64 * c + 64 <= len)
                finish_y_m(c, std::false_type{}, acc, xg, pv);
            else
                finish_y_m(c, std::true_type{}, acc, xg, pv);
        };
        // chunk j's operands are fetched right after chunk j - 2's output is
        // computed and stored (in iteration j - 1), two chain steps before they
        // are used (issuing them before the stores measured slower).
        if (p < nch) issue(p);
        __builtin_amdgcn_s_barrier();
        if (p == 1 && nch > 0) __builtin_amdgcn_s_barrier();  // iteration 0 (chunk 0 is wave 1's)
        if constexpr (EPI) {
            // A wave computes chunk j in iteration j + 1 and publishes its sums;
            // in iteration j + 2, where the other output wave computes chunk
            // j + 1, it finishes y of its previous chunk j - 2, whose sums every
            // slab published an iteration or more before and which it read at
            // the end of its previous finish. The finish thus runs beside the
            // other wave's products instead of after its own.
            f32x4_t pacc[4];
            u32x2_t pxg[4];
            int pj = -1;
            float pv[4][2];
            if (nch > 0) load_parts(p < nch ? p : 0, pv);  // (unused; keeps the loads in flight counted exactly)
            for (int j = p; j < nch; j += 2) {
                __builtin_amdgcn_s_barrier();  // end of iteration j: h_j, V_j are in the buffer
                f32x4_t acc[4];
                compute(j, acc);
                publish(j, acc);
                u32x2_t xgj[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) xgj[I] = xgr[I];  // (the next issue overwrites xgr)
                if (j + 2 < nch) issue(j + 2);
                if (j + 1 < nch) __builtin_amdgcn_s_barrier();  // end of iteration j + 1
                if (pj >= 0) {
                    ensure_in(pj, pv);
                    finish_y(pj, pacc, pxg, pv);
                }
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    pacc[I] = acc[I];
                    pxg[I] = xgj[I];
                }
                pj = j;
                load_parts(pj, pv);  // for the finish in this wave's next free iteration
            }
            if (pj >= 0) {
                ensure_in(pj, pv);
                finish_y(pj, pacc, pxg, pv);
            }
            return;
        }
        for (int j = p; j < nch; j += 2) {
            __builtin_amdgcn_s_barrier();  // end of iteration j: h_j, V_j are in the buffer
            f32x4_t acc[4];
            compute(j, acc);
            if (j + 1 < nch) {
                store(j, std::false_type{}, acc);
                if (j + 2 < nch) issue(j + 2);
                __builtin_amdgcn_s_barrier();  // end of iteration j + 1
            } else {
                store(j, std::true_type{}, acc);
            }
        }
        return;
    }

    if (DPLR && wv == 6) {
        // ---------------- DPLR: the state update's state-independent part K-^T V
        // (computed by the prep kernel) of chunk c + 1, copied into LDS buffer
        // (c + 1) & 1 during iteration c: the compute wave reads it in
        // iteration c + 1, and its last reader of that buffer (chunk c - 1)
        // finished before the barrier that ended iteration c - 1
        auto fetch = [&](int c) {
            const char* src = reinterpret_cast<const char*>(ws.km + ((int64_t)(co + c) * H + h) * D * D) +
                              (int64_t)ct * PL::PBS;
            char* dst = pbase + (c & 1) * PL::PBS;
#pragma unroll
            for (int j = 0; j < PL::PBS / 1024; ++j) dma16(src + j * 1024 + l * 16, dst + j * 1024);
        };
        if (nch > 0) fetch(0);
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) fetch(c + 1);
            wait_vm<0>();
            __builtin_amdgcn_s_barrier();
        }
        return;
    }

    if (!FUSED && wv == PL::NCW + 2) {
        // ---------------- L2 warm-up wave of the fp32 chain: during chunk c, this
        // slab's share of chunk c + AHEAD's -W and K-^T lines (one load per lane)
        // and its own U and gamma lines, so that the producers' DMA hits the L2
        // (ADDP: also its added term's lines, which the compute waves load)
        char* wdst = ring + RING * PL::SLOT + PL::XCH;
        constexpr int LW = PL::FB / 128, LPER = 2 * LW / NT, LU = PL::UB / 128, LG = PL::GB / 128;
        static_assert(LPER <= 64 && LU + LG <= 64, "one warm-up load per lane and part");
        auto warm = [&](int c) {
            const int64_t chh = (int64_t)(co + (ADDP ? nch - 1 - c : c)) * H + h;
            const int L = ct * LPER + (l < LPER ? l : LPER - 1);
            const char* p = L < LW ? reinterpret_cast<const char*>(ws.wn + chh * 64 * D) + L * 128
                                   : reinterpret_cast<const char*>(ws.km + chh * D * 64) + (L - LW) * 128;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)p,
                                             (__attribute__((address_space(3))) void*)wdst, 4, 0, 0);
            const int m = l < LU + LG ? l : 0;
            const char* pu = m < LU ? reinterpret_cast<const char*>(ws.u + chh * 64 * D + (int64_t)ct * 4 * 64 * 4) + m * 128
                                    : reinterpret_cast<const char*>(ws.gam + chh * D) + (m - LU) * 128;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)pu,
                                             (__attribute__((address_space(3))) void*)wdst, 4, 0, 0);
            if constexpr (ADDP) {
                constexpr int LP = NT * 64 * 4 * 4 / 128;  // lines of this slab's added term
                static_assert(LP <= 64, "one warm-up load per lane");
                const char* pp = reinterpret_cast<const char*>(ws.pb + chh * D * D + (int64_t)ct * NT * 64 * 4) +
                                 (l < LP ? l : 0) * 128;
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)pp,
                                                 (__attribute__((address_space(3))) void*)wdst, 4, 0, 0);
            }
        };
        const int pre = nch < PL::AHEAD ? nch : PL::AHEAD;
        for (int c = 0; c < pre; ++c) warm(c);
        __builtin_amdgcn_s_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + PL::AHEAD < nch) warm(c + PL::AHEAD);
            wait_vm<48>();
            __builtin_amdgcn_s_barrier();  // the compute waves' V_new exchange
            __builtin_amdgcn_s_barrier();  // end of chunk
        }
        wait_vm<0>();  // the LDS target stays allocated until the loads have landed
        return;
    }

    if (FUSED && wv == 5) {
        // ---------------- L2 warm-up wave: chunk c + AHEAD during chunk c; it
        // never waits for its loads except to bound the counter and at the end
        char* wdst = DPLR ? ring + 2 * PL::FB + PL::UB + PL::GB : hvbase + PL::HV;
        const int pre = nch < PL::AHEAD ? nch : PL::AHEAD;
        for (int c = 0; c < pre; ++c) warm_chunk<D, F32, FUSED, DPLR>(ws, (int64_t)(co + c) * H + h, ct, l, wdst);
        __builtin_amdgcn_s_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + PL::AHEAD < nch)
                warm_chunk<D, F32, FUSED, DPLR>(ws, (int64_t)(co + c + PL::AHEAD) * H + h, ct, l, wdst);
            wait_vm<48>();
            __builtin_amdgcn_s_barrier();
        }
        wait_vm<0>();  // the LDS target stays allocated until the loads have landed
        return;
    }

    if (wv >= (FUSED ? 1 : PL::NCW)) {
        // ---------------- producers (waves 3 and 4 when fused, else the two after the compute waves)
        const int pw = FUSED ? wv - 3 : wv - PL::NCW;
        const int pre = nch < RING - 1 ? nch : RING - 1;
        for (int c = 0; c < pre; ++c)
            produce<D, F32, FUSED, DPLR>(ws, (int64_t)(co + (ADDP ? nch - 1 - c : c)) * H + h, ct, pw, l,
                                         ring + c * PL::SLOT);
        // chunks 0 .. LOOK have landed once only the chunks issued after them are outstanding
        {
            const int need = nch - 1 < LOOK ? nch - 1 : LOOK;
            wait_chunks<OPS, RING>(pre - 1 - need);
        }
        __builtin_amdgcn_s_barrier();
        for (int c = 0; c < nch; ++c) {
            // slot (c + RING - 1) % RING was last read by the compute wave in chunk
            // c - 1, which it finished before the barrier that ended that chunk
            const int nx = c + RING - 1;
            if (nx < nch)
                produce<D, F32, FUSED, DPLR>(ws, (int64_t)(co + (ADDP ? nch - 1 - nx : nx)) * H + h, ct, pw, l,
                                             ring + (nx % RING) * PL::SLOT);
            if constexpr (!FUSED) __builtin_amdgcn_s_barrier();  // the compute waves' V_new exchange
            // chunk c + 1 + LOOK has landed once only the chunks issued after it are outstanding
            const int last = nch - 1 < nx ? nch - 1 : nx;
            const int need = nch - 1 < c + 1 + LOOK ? nch - 1 : c + 1 + LOOK;
            wait_chunks<OPS, RING>(last - need);
            __builtin_amdgcn_s_barrier();
        }
        return;
    }

    if constexpr (!FUSED) {
        // ---------------- NCW compute waves (fp32 factors). Wave q owns the
        // state's row tiles TH q .. TH q + TH - 1 and V_new's row tile q; both
        // are exchanged as accumulator tiles through LDS and every wave builds
        // the B fragments of the whole state and V_new from them.
        constexpr int NCW = PL::NCW, TH = NT / NCW;
        const int q = wv;
        f32x4_t* XS = reinterpret_cast<f32x4_t*>(ring + RING * PL::SLOT);  // [NT][64 lanes] state tiles
        f32x4_t* XV = XS + NT * 64;                                        // [4][64] V_new tiles
        f32x4_t S[TH];  // rows 16 (TH q + tt) + 4g + i, column 16 ct + n
        const int sbase = 16 * ct + n;
#pragma unroll
        for (int tt = 0; tt < TH; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[tt][i] = s_in ? s_in[sbase + (16 * (TH * q + tt) + 4 * g + i) * D] : 0.f;
        // ADDP: the added term of chunk c + 1 is loaded at the start of chunk c
        f32x4_t pc[ADDP ? TH : 1], pnx[ADDP ? TH : 1];
        auto load_p = [&](int c, f32x4_t (&dst)[ADDP ? TH : 1]) {
            if constexpr (ADDP) {
                const float* pp = ws.pb + ((int64_t)(co + nch - 1 - c) * H + h) * D * D + (int64_t)ct * NT * 64 * 4;
#pragma unroll
                for (int tt = 0; tt < TH; ++tt)
                    dst[tt] = *reinterpret_cast<const f32x4_t*>(pp + ((TH * q + tt) * 64 + l) * 4);
            }
        };
        auto put_s = [&]() {
#pragma unroll
            for (int tt = 0; tt < TH; ++tt) XS[(TH * q + tt) * 64 + l] = S[tt];
        };
        // ADDP (the backward's chain) runs on the forward's own factor arrays with
        // their roles swapped: the slot's "-W" part holds K-^T as the forward stored
        // it ([dk][64], rows split-ordered) and its "K-^T" part holds -W ([64][dk],
        // channels split-ordered), so the operand fragments are read transposed,
        // one element at a time
        auto w_transposed = [&](const char* sl, int s) {  // K- rows 16q + n, channels of slice s
            const float* kt = reinterpret_cast<const float*>(sl);
            const int r = 16 * q + n, pr = 32 * (r >> 5) + split_pos(r);
            Frag f;
#pragma unroll
            for (int j = 0; j < 8; ++j) f.v[j] = kt[(32 * s + kslot(g, j)) * 64 + pr];
            return f;
        };
        auto k_transposed = [&](const char* sl, int t, int s) {  // (-W)^T rows 16t + n, chunk rows of slice s
            const float* wn = reinterpret_cast<const float*>(sl);
            const int c = 16 * t + n, pc = 32 * (c >> 5) + split_pos(c);
            Frag f;
#pragma unroll
            for (int j = 0; j < 8; ++j) f.v[j] = wn[(32 * s + kslot(g, j)) * D + pc];
            return f;
        };
        put_s();
        if (nch > 0) load_p(0, pc);
        lds_exchange_barrier();
        for (int c = 0; c < nch; ++c) {
            const char* slot = ring + (c % RING) * PL::SLOT;
            const char* wsl = slot;
            const char* ksl = slot + PL::FB;
            const E* usl = reinterpret_cast<const E*>(slot + 2 * PL::FB);
            const float* gsl = reinterpret_cast<const float*>(slot + 2 * PL::FB + PL::UB);
            const int64_t chh = (int64_t)(co + (ADDP ? nch - 1 - c : c)) * H + h;
            // (unconditional: the last chunk reloads its own term, unused)
            if (ADDP) load_p(c + 1 < nch ? c + 1 : c, pnx);
            // every LDS operand of the V_new products first (-W of row tile q, the
            // whole state as B fragments), held here by the fence below so that
            // their latencies overlap instead of each product waiting for its own
            Frag wfr[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int gr = ((16 * q + n) * NS + s) * 4 + g;
                wfr[s] = ADDP ? w_transposed(wsl, s) : P::load(reinterpret_cast<const E*>(wsl + gr * 8 * sizeof(E)));
            }
            Frag sb[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) sb[s] = frag_from_acc<F32>(XS[(2 * s) * 64 + l], XS[(2 * s + 1) * 64 + l]);
            // V_new = U + (-W) S on row tile q, starting from U
            f32x4_t V = *reinterpret_cast<const f32x4_t*>(usl + (q * 64 + l) * 4);
            asm volatile("" ::: "memory");
            // h_n out: each wave stores its own state tiles from its registers
            // (tile t is half t & 1 of the B fragment of slice t >> 1). Every wave
            // issues the same global operations in every chunk, with no branch, so
            // the compiler's count of outstanding ones stays exact and the wait
            // for the added term (ADDP) does not also wait for this chunk's stores
            E* hp = ws.h + chh * D * D + (int64_t)ct * NS * 64 * 8;
#pragma unroll
            for (int tt = 0; tt < TH; ++tt) {
                const int t = TH * q + tt;
                *reinterpret_cast<f32x4_t*>(hp + ((t >> 1) * 64 + l) * 8 + (t & 1) * 4) = S[tt];
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) P::mma(V, wfr[s], sb[s]);
            XV[q * 64 + l] = V;
            // V_new out: this wave's row tile q, stored as h_n's tiles above
            E* vp = ws.vn + chh * 64 * D + (int64_t)ct * 2 * 64 * 8;
            *reinterpret_cast<f32x4_t*>(vp + ((q >> 1) * 64 + l) * 8 + (q & 1) * 4) = V;
            // this wave's K-^T fragments and gamma while the other tiles land
            Frag kf[TH][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int tt = 0; tt < TH; ++tt) {
                    const int gr = ((16 * (TH * q + tt) + n) * 2 + s) * 4 + g;
                    kf[tt][s] = ADDP ? k_transposed(ksl, TH * q + tt, s)
                                     : P::load(reinterpret_cast<const E*>(ksl + gr * 8 * sizeof(E)));
                }
            f32x4_t gm[TH];
#pragma unroll
            for (int tt = 0; tt < TH; ++tt) gm[tt] = *reinterpret_cast<const f32x4_t*>(gsl + 16 * (TH * q + tt) + 4 * g);
            lds_exchange_barrier();  // every V_new tile in LDS
            Frag vb[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) vb[s] = frag_from_acc<F32>(XV[(2 * s) * 64 + l], XV[(2 * s + 1) * 64 + l]);
            // S <- Diag(gamma) S (+ the added term) + K-^T V_new on this wave's row tiles
#pragma unroll
            for (int tt = 0; tt < TH; ++tt) {
                if constexpr (ADDP)
                    S[tt] = gm[tt] * S[tt] + pc[tt];
                else
                    S[tt] = gm[tt] * S[tt];
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int tt = 0; tt < TH; ++tt) P::mma(S[tt], kf[tt][s], vb[s]);
            put_s();
            if constexpr (ADDP) {
#pragma unroll
                for (int tt = 0; tt < TH; ++tt) pc[tt] = pnx[tt];
            }
            lds_exchange_barrier();  // end of chunk: slot free, state tiles in LDS
        }
        if (s_out) {
#pragma unroll
            for (int tt = 0; tt < TH; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) s_out[sbase + (16 * (TH * q + tt) + 4 * g + i) * D] = S[tt][i];
        }
        return;
    }

    // ---------------- compute wave (the fused chain; the unfused one returned above)
    f32x4_t S[NT];  // state slab: rows 16t + 4g + i, column 16 ct + n
    const int sbase = 16 * ct + n;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] = s_in ? s_in[sbase + (16 * t + 4 * g + i) * D] : 0.f;

    // HP: this slab's fp32 U of the next chunk, loaded from the workspace one
    // chunk ahead (the compute wave's only global loads in the loop, so the
    // wait before their use finds them landed a whole chain step later)
    f32x4_t un[PL::HP ? 4 : 1];
    auto load_u = [&](int c) {
        if constexpr (PL::HP) {
            const float* up = ws.uf + ((int64_t)(co + c) * H + h) * 64 * D + (int64_t)ct * 4 * 64 * 4;
#pragma unroll
            for (int I = 0; I < 4; ++I) un[I] = *reinterpret_cast<const f32x4_t*>(up + (I * 64 + l) * 4);
        }
    };
    if (PL::HP && nch > 0) load_u(0);
    Frag wf[4][NS];  // -W fragments (with LOOK, of the chunk after the current one once read)
    auto load_w = [&](int c) {
        const char* wsl = ring + (c % RING) * PL::SLOT;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int gr = ((16 * I + n) * NS + s) * 4 + g;  // fragment of -W (row 16I+n, slice s, group g)
                wf[I][s] = P::load(reinterpret_cast<const E*>(wsl + swz<F32>(gr) * 8 * sizeof(E)));
            }
    };
    __builtin_amdgcn_s_barrier();
    if (LOOK && nch > 0) load_w(0);
    for (int c = 0; c < nch; ++c) {
        const char* slot = ring + (c % RING) * PL::SLOT;
        const char* ksl = slot + PL::FB;
        const E* usl = reinterpret_cast<const E*>(slot + 2 * PL::FB);
        const float* gsl = reinterpret_cast<const float*>(slot + 2 * PL::FB + PL::UB);
        const int64_t chh = (int64_t)(co + c) * H + h;

        // every LDS read of this chunk first, so their latencies overlap
        Frag kf[NT][2];
        if (!LOOK) load_w(c);
        f32x4_t V[4];
        if constexpr (PL::HP) {
#pragma unroll
            for (int I = 0; I < 4; ++I) V[I] = un[I];
            if (c + 1 < nch) load_u(c + 1);
            asm volatile("" ::: "memory");  // issue the next chunk's U loads here
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if constexpr (PL::HP) {
            } else if constexpr (F32) {
                V[I] = *reinterpret_cast<const f32x4_t*>(usl + (I * 64 + l) * 4);
            } else {
                const u32x2_t u = *reinterpret_cast<const u32x2_t*>(usl + (I * 64 + l) * 4);
                V[I] = f32x4_t{h2f(u[0] & 0xffffu), h2f(u[0] >> 16), h2f(u[1] & 0xffffu), h2f(u[1] >> 16)};
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int gr = ((16 * t + n) * 2 + s) * 4 + g;  // fragment of K-^T (row 16t+n, slice s, group g)
                kf[t][s] = P::load(reinterpret_cast<const E*>(ksl + swz<F32>(gr) * 8 * sizeof(E)));
            }
        f32x4_t gm[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) gm[t] = *reinterpret_cast<const f32x4_t*>(gsl + 16 * t + 4 * g);
        u32x2_t kv[DPLR ? NT : 1];  // DPLR: K-^T V of this chunk and slab
        if constexpr (DPLR) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                kv[t] = *reinterpret_cast<const u32x2_t*>(pbase + (c & 1) * PL::PBS + (t * 64 + l) * 8);
        }

        // h_n = S as B-operand fragments (also the operand of W S below); to the
        // output wave's LDS buffer when fused, else to the workspace
        Frag sb[NS];
        E* hp = FUSED ? reinterpret_cast<E*>(hvbase + (c & 1) * PL::HVS)
                      : ws.h + chh * D * D + (int64_t)ct * NS * 64 * 8;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            sb[s] = frag_from_acc<F32>(S[2 * s], S[2 * s + 1]);
            P::store(hp + (s * 64 + l) * 8, sb[s]);
        }
        // S <- Diag(gamma) S (+ K-^T V with DPLR) now that h_n is taken: off the
        // V_new products' path
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (DPLR)
                S[t] = gm[t] * S[t] + f32x4_t{h2f(kv[t][0] & 0xffffu), h2f(kv[t][0] >> 16), h2f(kv[t][1] & 0xffffu),
                                              h2f(kv[t][1] >> 16)};
            else
                S[t] = gm[t] * S[t];
        }
        // V_new = U + (-W) S, row tiles 0-1 first: their two-term split and the
        // state products of their half run while tiles 2-3 are still in the matrix core
#pragma unroll
        for (int hv = 0; hv < 2; ++hv)
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int I = 2 * hv; I < 2 * hv + 2; ++I) P::mma(V[I], wf[I][s], sb[s]);
        // the next chunk's -W while this chunk's key-value products run (the
        // last chunk re-reads its own)
        if (LOOK) load_w(c + 1 < nch ? c + 1 : c);
        Frag vb[2];
        Frag vl[PL::HP ? 2 : 1];  // HP: the low terms of V_new
        E* vp = FUSED ? reinterpret_cast<E*>(hvbase + (c & 1) * PL::HVS) + D * 16
                      : ws.vn + chh * 64 * D + (int64_t)ct * 2 * 64 * 8;
        // S += K-^T V_new: with HP the low terms of both halves first, then the high
        // terms (each tile accumulates lo 0, lo 1, hi 0, hi 1 in that order)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (PL::HP) {
                const Frag2 x = split_from_acc(V[2 * s], V[2 * s + 1]);
                vb[s] = x.hi;
                vl[s] = x.lo;
                P::store(vp + (2 * 64 + s * 64 + l) * 8, vl[s]);
#pragma unroll
                for (int t = 0; t < NT; ++t) P::mma(S[t], kf[t][s], vl[s]);
            } else {
                vb[s] = frag_from_acc<F32>(V[2 * s], V[2 * s + 1]);
            }
            P::store(vp + (s * 64 + l) * 8, vb[s]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < NT; ++t) P::mma(S[t], kf[t][s], vb[s]);
        if constexpr (FUSED) wait_lgkm0();  // h_n / V_new in LDS before the hand-over
        __builtin_amdgcn_s_barrier();
    }
    if (s_out) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_out[sbase + (16 * t + 4 * g + i) * D] = S[t][i];
    }
}

template <int D, bool F32, bool FUSED, bool OUT_F32, bool DPLR = false, bool ADDP = false, bool EPI = false>
static hipError_t launch_recur_t(const ChunkArgs& a, hipStream_t st) {
    using E = typename Pol<F32>::E;
    using PL = RecurPlan<D, F32, FUSED, DPLR>;
    Ws<E> ws{(E*)a.qp, (E*)a.km, (E*)a.wn, (E*)a.u, (E*)a.aqk, a.gam, (E*)a.h, (E*)a.vn, (E*)a.am, (E*)a.oh, a.pb};
    ws.uf = static_cast<float*>(a.u);  // KDA with 16-bit factors: U is fp32
    constexpr int NT = D / 16;
    const int NU = a.N * a.H;
    auto kern = recur_kernel<D, F32, FUSED, OUT_F32, DPLR, ADDP, EPI>;
    constexpr int LDS = PL::LDS;
    const hipError_t e = allow_dynamic_lds((const void*)kern, LDS);
    if (e != hipSuccess) return e;
    dim3 grid(NU * NT), block(FUSED ? (DPLR ? 448 : 384) : 64 * (PL::NCW + 3));
    const EpiArgs ep{static_cast<const uint16_t*>(a.xg), a.rms_w, static_cast<uint16_t*>(a.y), a.epi_part,
                     a.epi_spin_max};
    hipLaunchKernelGGL(kern, grid, block, LDS, st, a.s0, a.s_final, a.tab, a.N, a.T, a.H, ws, a.o, a.piece, ep);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_recur_d(const ChunkArgs& a, hipStream_t st) {
    if (a.in_f32 || a.f32_factors)
        return a.pb ? launch_recur_t<D, true, false, true, false, true>(a, st) : launch_recur_t<D, true, false, true>(a, st);
    if (a.epi) return launch_recur_t<D, false, true, false, false, false, true>(a, st);  // (checked by the caller)
    return a.out_f32 ? launch_recur_t<D, false, true, true>(a, st) : launch_recur_t<D, false, true, false>(a, st);
}

hipError_t launch_recur(const ChunkArgs& a, hipStream_t st) {
    if (a.dplr) {  // 16-bit factors only (checked by the caller)
        if (a.D == 128)
            return a.out_f32 ? launch_recur_t<128, false, true, true, true>(a, st)
                             : launch_recur_t<128, false, true, false, true>(a, st);
        return a.out_f32 ? launch_recur_t<64, false, true, true, true>(a, st)
                         : launch_recur_t<64, false, true, false, true>(a, st);
    }
    return a.D == 128 ? launch_recur_d<128>(a, st) : launch_recur_d<64>(a, st);
}

}  // namespace kda
