// Shared device helpers of the KDA HIP library (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions used by every kernel
// -------------------------------------------
// All chunk products run on 16x16 output tiles:
//   half policy: v_mfma_f32_16x16x32_f16 / _bf16 (one instruction per 32-deep slice)
//   fp32 policy: v_mfma_f32_16x16x4_f32   (eight instructions per 32-deep slice)
// Lane l of a wave (n = l & 15, g = l >> 4) holds
//   A operand: row m = n of the 16 x 32 slice, eight k-slots (g, j), j = 0..7
//   B operand: col n of the 32 x 16 slice, the same eight k-slots (g, j)
//   C/D:       col n, rows 4g + i (i = 0..3) of the 16 x 16 tile
// The hardware contracts slot (g, j) of A with slot (g, j) of B, so which
// logical k a slot carries is ours to choose, as long as both operands agree.
// We always use the "split" order
//      k(g, j) = 16 * (j >> 2) + 4 * g + (j & 3)
// because then a B operand made of two stacked accumulator tiles (rows 0-15
// and 16-31 of the slice) is just the lane's own accumulator registers:
// slots j = 0..3 are tile 0 rows 4g..4g+3, slots j = 4..7 are tile 1 rows
// 4g..4g+3. State tiles and corrected values therefore move from one product
// to the next without any cross-lane exchange; operands that come from memory
// are stored pre-permuted in this order so that each lane loads one 16-byte
// (bf16) or 32-byte (fp32) vector per slice.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int CH = 64;   // chunk length
constexpr int SUB = 16;  // secondary-chunk length (one MFMA tile)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
// Two values rounded to nearest even and packed (lo in bits 0-15) by one
// conversion instruction (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32): written as a
// vector conversion, because two scalar conversions joined by shifts compile to
// two conversions plus the joining operations.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
// round-to-nearest-even fp32 <-> fp16
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

// k-slot -> logical k inside a 32-deep slice ("split" order, see above)
__host__ __device__ constexpr int kslot(int g, int j) { return 16 * (j >> 2) + 4 * g + (j & 3); }

// ---------------------------------------------------------------- operands
// Value-path products (WY solve, W S, K-^T V_new, Q+ h, A_qk V_new) take fp16
// operands with fp32 accumulation when the inputs are bf16: fp16 has 3 more
// mantissa bits than bf16 at the same matrix-core rate. Operands that carry
// the values themselves (beta V in the solve, V_new) are two-term fp16 (Frag2
// below), and U is stored in fp32: the error is judged max-abs relative to the
// RMS, and on heavy-tailed values one fp16 rounding of the largest value is
// already a sizeable part of that budget. Every value-path operand is bounded
// by the input magnitudes (|q|, |k| for the gated factors; |v| for U, V_new
// and the state), so the fp16 range holds while |v| and the state stay below
// ~3e4. With fp32 inputs every product runs in fp32.
template <bool F32> struct Pol;
template <> struct Pol<false> {
    using E = uint16_t;  // fp16 bits
    struct Frag { f16x8_t v; };
    static __device__ __forceinline__ float to_f(E x) { return h2f(x); }
    static __device__ __forceinline__ E from_f(float x) { return f2h(x); }
    static __device__ __forceinline__ Frag make(const float (&x)[8]) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = (_Float16)x[j];
        return f;
    }
    static __device__ __forceinline__ Frag zero() {
        Frag f;
        f.v = __builtin_bit_cast(f16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        return f;
    }
    static __device__ __forceinline__ Frag load(const E* p) {  // 16-byte aligned
        Frag f;
        f.v = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(p));
        return f;
    }
    static __device__ __forceinline__ void store(E* p, const Frag& f) {
        *reinterpret_cast<u32x4_t*>(p) = __builtin_bit_cast(u32x4_t, f.v);
    }
    static __device__ __forceinline__ void mma(f32x4_t& acc, const Frag& a, const Frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
    }
};
template <> struct Pol<true> {
    using E = float;
    struct Frag { float v[8]; };
    static __device__ __forceinline__ float to_f(E x) { return x; }
    static __device__ __forceinline__ E from_f(float x) { return x; }
    static __device__ __forceinline__ Frag make(const float (&x)[8]) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = x[j];
        return f;
    }
    static __device__ __forceinline__ Frag zero() {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
        return f;
    }
    static __device__ __forceinline__ Frag load(const E* p) {  // 16-byte aligned
        Frag f;
        const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
        const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f.v[j] = a[j];
            f.v[4 + j] = b[j];
        }
        return f;
    }
    static __device__ __forceinline__ void store(E* p, const Frag& f) {
        reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{f.v[0], f.v[1], f.v[2], f.v[3]};
        reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{f.v[4], f.v[5], f.v[6], f.v[7]};
    }
    static __device__ __forceinline__ void mma(f32x4_t& acc, const Frag& a, const Frag& b) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
    }
};

// Gated intra-chunk products (A_kk, A_qk). Their anchored factors span up to
// 2^100, outside the fp16 range, so with bf16 inputs they run as split bf16:
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi), and
// a b ~= a_hi b_hi + a_lo b_hi + a_hi b_lo (16 mantissa bits, fp32 range).
// The B operand (keys) is kept in LDS as a hi array followed by a lo array.
template <bool F32> struct APol;
template <> struct APol<false> {
    using E = uint16_t;  // bf16 bits
    static constexpr int PLANES = 2;
    struct Frag { bf16x8_t hi, lo; };
    static __device__ __forceinline__ Frag make(const float (&x)[8]) {
        Frag f;
        u32x4_t h, l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t hj = pack2bf(x[2 * j], x[2 * j + 1]);
            h[j] = hj;
            l[j] = pack2bf(x[2 * j] - __uint_as_float(hj << 16), x[2 * j + 1] - __uint_as_float(hj & 0xffff0000u));
        }
        f.hi = __builtin_bit_cast(bf16x8_t, h);
        f.lo = __builtin_bit_cast(bf16x8_t, l);
        return f;
    }
    // planes: hi at p, lo at p + plane
    static __device__ __forceinline__ Frag load(const E* p, int plane) {
        Frag f;
        f.hi = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
        f.lo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p + plane));
        return f;
    }
    static __device__ __forceinline__ void store(E* p, int plane, const Frag& f) {
        *reinterpret_cast<u32x4_t*>(p) = __builtin_bit_cast(u32x4_t, f.hi);
        *reinterpret_cast<u32x4_t*>(p + plane) = __builtin_bit_cast(u32x4_t, f.lo);
    }
    static __device__ __forceinline__ void mma(f32x4_t& acc, const Frag& a, const Frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    }
    // The gated query-key and key-key products of one block, sharing B:
    // cq += xq B in split bf16 (xq split by truncation: hi keeps the top 16
    // bits exactly, lo = x - hi rounded to nearest, about 16 significant bits
    // in all), ck += xk B with xk and B rounded once to bf16 (the key-key
    // matrix only feeds the UT transform, where bf16 operands cost nothing
    // measurable against the fp16 value path). Interleaved so dependent MFMAs
    // of one accumulator are separated by the other's.
    static __device__ __forceinline__ void mma_qk(f32x4_t& cq, const float (&xq)[8], f32x4_t& ck,
                                                  const float (&xk)[8], const Frag& b) {
        u32x4_t qh, ql, kh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b0 = __float_as_uint(xq[2 * j]) & 0xffff0000u;
            const uint32_t b1 = __float_as_uint(xq[2 * j + 1]) & 0xffff0000u;
            qh[j] = (b0 >> 16) | b1;
            ql[j] = pack2bf(xq[2 * j] - __uint_as_float(b0), xq[2 * j + 1] - __uint_as_float(b1));
            kh[j] = pack2bf(xk[2 * j], xk[2 * j + 1]);
        }
        const bf16x8_t qhi = __builtin_bit_cast(bf16x8_t, qh), qlo = __builtin_bit_cast(bf16x8_t, ql);
        const bf16x8_t khi = __builtin_bit_cast(bf16x8_t, kh);
        cq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo, b.hi, cq, 0, 0, 0);
        ck = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khi, b.hi, ck, 0, 0, 0);
        cq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, b.lo, cq, 0, 0, 0);
        cq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, b.hi, cq, 0, 0, 0);
    }
    // The same with the query-key product transposed: cq += (xq B)^T, i.e. B
    // is the A operand and xq the B operand. Its accumulator tile then holds,
    // in lane n + 16 g, row n of xq B at columns 4 g .. 4 g + 3, which is the
    // matrix-core operand layout of xq B: the tile is stored as operand
    // fragments without any exchange between lanes.
    static __device__ __forceinline__ void mma_qk_t(f32x4_t& cq, const float (&xq)[8], f32x4_t& ck,
                                                    const float (&xk)[8], const Frag& b) {
        u32x4_t qh, ql, kh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b0 = __float_as_uint(xq[2 * j]) & 0xffff0000u;
            const uint32_t b1 = __float_as_uint(xq[2 * j + 1]) & 0xffff0000u;
            qh[j] = (b0 >> 16) | b1;
            ql[j] = pack2bf(xq[2 * j] - __uint_as_float(b0), xq[2 * j + 1] - __uint_as_float(b1));
            kh[j] = pack2bf(xk[2 * j], xk[2 * j + 1]);
        }
        const bf16x8_t qhi = __builtin_bit_cast(bf16x8_t, qh), qlo = __builtin_bit_cast(bf16x8_t, ql);
        const bf16x8_t khi = __builtin_bit_cast(bf16x8_t, kh);
        cq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.hi, qlo, cq, 0, 0, 0);
        ck = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khi, b.hi, ck, 0, 0, 0);
        cq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.lo, qhi, cq, 0, 0, 0);
        cq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.hi, qhi, cq, 0, 0, 0);
    }
};
template <> struct APol<true> {
    using E = float;
    static constexpr int PLANES = 1;
    using Frag = Pol<true>::Frag;
    static __device__ __forceinline__ Frag make(const float (&x)[8]) { return Pol<true>::make(x); }
    static __device__ __forceinline__ Frag load(const E* p, int) { return Pol<true>::load(p); }
    static __device__ __forceinline__ void store(E* p, int, const Frag& f) { Pol<true>::store(p, f); }
    static __device__ __forceinline__ void mma(f32x4_t& acc, const Frag& a, const Frag& b) {
        Pol<true>::mma(acc, a, b);
    }
    static __device__ __forceinline__ void mma_qk(f32x4_t& cq, const float (&xq)[8], f32x4_t& ck,
                                                  const float (&xk)[8], const Frag& b) {
        const Frag a0 = make(xq), a1 = make(xk);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            cq = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.v[j], b.v[j], cq, 0, 0, 0);
            ck = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.v[j], b.v[j], ck, 0, 0, 0);
        }
    }
};

// B operand built from two accumulator tiles (rows 0-15 = t0, rows 16-31 = t1)
template <bool F32>
__device__ __forceinline__ typename Pol<F32>::Frag frag_from_acc(const f32x4_t& t0, const f32x4_t& t1) {
    float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    return Pol<F32>::make(x);
}

// ---------------------------------------------------------------- input loads
template <typename T> __device__ __forceinline__ float ld_in(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
template <> __device__ __forceinline__ float ld_in<float>(const float* p, int64_t i) { return p[i]; }

// four consecutive input elements starting at i (i multiple of 4)
template <typename T> __device__ __forceinline__ void ld_in4(const T* p, int64_t i, float (&x)[4]);
template <> __device__ __forceinline__ void ld_in4<uint16_t>(const uint16_t* p, int64_t i, float (&x)[4]) {
    const u32x2_t u = *reinterpret_cast<const u32x2_t*>(p + i);
    x[0] = __uint_as_float(u[0] << 16);
    x[1] = __uint_as_float(u[0] & 0xffff0000u);
    x[2] = __uint_as_float(u[1] << 16);
    x[3] = __uint_as_float(u[1] & 0xffff0000u);
}
template <> __device__ __forceinline__ void ld_in4<float>(const float* p, int64_t i, float (&x)[4]) {
    const f32x4_t u = *reinterpret_cast<const f32x4_t*>(p + i);
    x[0] = u[0];
    x[1] = u[1];
    x[2] = u[2];
    x[3] = u[3];
}

// Sequence table of a packed batch, built on the device from cu_seqlens by
// seq_table_kernel (kda_seq.hip) at the start of every call that has one:
// entry i = {first token, length, first chunk slot, chunk count} of sequence
// i, after sanitising the offsets (each clamped into [0, T], non-decreasing,
// chunks capped at the workspace's capacity), so that a malformed cu_seqlens
// can give wrong results but never an access outside the buffers. Entry N is
// a sentinel {T, 0, total chunks, 0}. Chunk slots of sequence i are
// [coff_i, coff_i + nch_i); they tile [0, total) in order.
struct SeqMeta {
    int32_t start, len, coff, nch;
};

// Chunk slot -> (sequence, first token, length, the sequence's first token).
// tab == nullptr means one sequence of T tokens. Every lane of the calling
// wave must call it with the same gc (the search is uniform).
struct ChunkLoc {
    int seq;
    int t0;
    int L;
    int start;
};
__device__ __forceinline__ bool locate_chunk(const SeqMeta* __restrict__ tab, int N, int T, int gc,
                                             ChunkLoc& out) {
    if (tab == nullptr) {
        const int t0 = gc * CH;
        if (t0 >= T) return false;
        out.seq = 0;
        out.t0 = t0;
        out.L = min(CH, T - t0);
        out.start = 0;
        return true;
    }
    if (gc >= tab[N].coff) return false;
    // the last sequence whose first chunk slot is <= gc (empty sequences share
    // their successor's offset and are skipped by taking the last)
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab[mid].coff <= gc) lo = mid; else hi = mid - 1;
    }
    const SeqMeta m = tab[lo];
    const int lc = gc - m.coff;
    out.seq = lo;
    out.t0 = m.start + lc * CH;
    out.L = min(CH, m.len - lc * CH);
    out.start = m.start;
    return true;
}

// First token, length, first chunk slot and chunk count of sequence `seq`.
__device__ __forceinline__ SeqMeta seq_info(const SeqMeta* __restrict__ tab, int T, int seq) {
    if (tab == nullptr) return SeqMeta{0, T, 0, (T + CH - 1) / CH};
    return tab[seq];
}

// ---------------------------------------------------------------- workspace
// Per (chunk slot, head) intermediates, each array [NC][H][...]:
//   qp   [64][D]   gated queries  Q+ = exp(g) * q, rows in order, k = key channel (split order per 32);
//                  with 16-bit KDA factors in fragment order [4 row blocks][D/32 slices][64 lanes][8]
//                  (lane n + 16 g holds row 16 I + n, channels 32 s + kslot(g, 0..7))
//   km   [D][64]   decayed keys K- = exp(g_last - g) * k, transposed: row = key channel, k = chunk row
//   wn   [64][D]   -W (negated key WY factor), k = key channel (split order)
//   u    [D/16][4][64 lanes][4]   U in accumulator-tile order (value col tile, row tile, lane, i);
//                  fp32 with 16-bit KDA factors (uf), so the values are never rounded to fp16
//   aqk  [64][64]  gated query-key matrix (lower incl. diagonal), k = chunk col (split order);
//                  with 16-bit KDA factors two fp16 planes (x = hi + lo), each in fragment order
//                  [4 row blocks][2 slices][64 lanes][8] like qp
//   gam  [D] fp32  exp(g_last) per key channel
//   h    [D/16][D/32][64 lanes][8]   chunk-entry state as B-operand fragments (value col tile, k slice)
//   vn   [D/16][2][64 lanes][8]      corrected values V_new as B-operand fragments
// The general DPLR transition (16-bit factors only) uses the same arrays for
// its analogues -- qp: Q+, wn: -W', u: -U', aqk: A_qa, gam; km holds the state
// update's state-independent part K-^T V [D/16 col tile][D/16 row tile][64 lanes][4]
// (D x max(D, 64) elements) -- and two more:
//   am   [D][64]   decayed A-vectors A- = exp(g_last - g) * a, transposed like km
//   oh   [D/16][4][64 lanes][4]   the output's state-independent part A_qk V, accumulator-tile order
template <typename E>
struct Ws {
    E* qp;
    E* km;
    E* wn;
    E* u;
    E* aqk;
    float* gam;
    E* h;
    E* vn;
    E* am = nullptr;
    E* oh = nullptr;
    // backward state-gradient recursion: a state-independent term added to the
    // state each chunk, [dv/16][dk/16][64 lanes][4] fp32 per chunk-head
    const float* pb = nullptr;
    // KDA with 16-bit factors: U in fp32 (the same array as u)
    float* uf = nullptr;
};

// Two-term fp16 operand: x = hi + lo with hi = fp16(x) and lo = fp16(x - hi),
// about 22 significant bits. A product a x runs as two matrix-core products,
// a lo + a hi, accumulated in fp32. The bf16 path carries its large-magnitude
// values (beta V inside the WY solve, the corrected values V_new) this way,
// because one fp16 rounding of a heavy-tailed value already costs a sizeable
// fraction of the max-abs error budget.
struct Frag2 {
    Pol<false>::Frag hi, lo;
};
__device__ __forceinline__ Frag2 split_frag(const float (&x)[8]) {
    u32x4_t h, r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // (through a scalar: a bit cast of the vector element itself reads element 0)
        const uint32_t hj = pack2h(x[2 * j], x[2 * j + 1]);
        h[j] = hj;
        const f16x2_t hh = __builtin_bit_cast(f16x2_t, hj);
        r[j] = pack2h(x[2 * j] - (float)hh[0], x[2 * j + 1] - (float)hh[1]);
    }
    Frag2 f;
    f.hi.v = __builtin_bit_cast(f16x8_t, h);
    f.lo.v = __builtin_bit_cast(f16x8_t, r);
    return f;
}
__device__ __forceinline__ Frag2 split_from_acc(const f32x4_t& t0, const f32x4_t& t1) {
    const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    return split_frag(x);
}
// acc += a x for a two-term B operand (the small term first)
__device__ __forceinline__ void mma2(f32x4_t& acc, const Pol<false>::Frag& a, const Frag2& x) {
    Pol<false>::mma(acc, a, x.lo);
    Pol<false>::mma(acc, a, x.hi);
}

}  // namespace kda
