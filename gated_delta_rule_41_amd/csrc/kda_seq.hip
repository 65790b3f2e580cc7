// The sequence table of a packed batch (SeqMeta, kda_common.h) from
// cu_seqlens, once per call, before the kernels that look chunks up in it.
//
// One workgroup walks the N sequences in tiles of 1024: each thread sanitises
// its sequence's offsets (start clamped into [0, T], end into [start, T]),
// counts its chunks, and a block-wide exclusive scan (64-bit, so that no
// malformed input can wrap it) gives each sequence's first chunk slot. Chunk
// counts past the workspace's capacity NC are cut, so slots never exceed it.
// A chunk slot is then found by a binary search over the table (O(log N)
// uniform loads per workgroup) and a sequence's slots by one load, where the
// kernels used to scan cu_seqlens from the start in every workgroup.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

__global__ __launch_bounds__(1024) void seq_table_kernel(const int32_t* __restrict__ cu, int N, int T, int NC,
                                                         SeqMeta* __restrict__ tab) {
    __shared__ long long wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    long long carry = 0;  // chunks of the sequences before this tile (before the cut)
    for (int base = 0; base < N; base += 1024) {
        const int i = base + tid;
        int s = 0, len = 0;
        long long nch = 0;
        if (i < N) {
            s = min(max(cu[i], 0), T);
            const int e = min(max(cu[i + 1], s), T);
            len = e - s;
            nch = (len + CH - 1) / CH;
        }
        long long x = nch;  // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const long long y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[wid] = x;
        __syncthreads();
        long long before = 0, tile = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            before += w < wid ? wsum[w] : 0;
            tile += wsum[w];
        }
        if (i < N) {
            const long long coff = carry + before + x - nch;
            const long long room = (long long)NC - coff;
            const int nc = (int)(room <= 0 ? 0 : (nch < room ? nch : room));
            tab[i] = SeqMeta{s, min(len, nc * CH), (int)(coff < NC ? coff : NC), nc};
        }
        carry += tile;
        __syncthreads();  // wsum is rewritten by the next tile
    }
    if (tid == 0) tab[N] = SeqMeta{T, 0, (int)(carry < NC ? carry : NC), 0};
}

hipError_t launch_seq_table(const int32_t* cu, int N, int T, int NC, SeqMeta* tab, hipStream_t st) {
    hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(1024), 0, st, cu, N, T, NC, tab);
    return hipGetLastError();
}

}  // namespace kda
