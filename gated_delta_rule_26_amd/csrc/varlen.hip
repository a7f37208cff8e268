// Variable-length (packed) batches: the table of chunks that the chunk
// kernels walk, built on the device from the caller's cu_seqlens.
//
// Sequence n holds the packed tokens [cu[n], cu[n+1]).  The table is made
// safe for any values: every entry is clamped to [0, T] and raised to the
// largest entry before it (a prefix maximum), so the sequences are disjoint
// ranges inside [0, T] and the chunk count sum_n ceil(len_n / 64) is at most
// floor((T + 63 N) / 64), the bound the workspace and the grids are sized
// for.  For well-formed cu_seqlens (0 = cu[0] <= ... <= cu[N] = T) the
// clamps change nothing.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kTabThreads = 1024;

// Exclusive scan of one value per thread over the workgroup (max or sum of
// values >= 0, so 0 is the identity of both), Hillis-Steele in LDS.
template <bool MAX>
__device__ int block_scan_excl(int x, int *tmp) {
    const int t = threadIdx.x;
    tmp[t] = x;
    __syncthreads();
    for (int off = 1; off < kTabThreads; off <<= 1) {
        const int y = t >= off ? tmp[t - off] : 0;
        __syncthreads();
        x = MAX ? max(x, y) : x + y;
        tmp[t] = x;
        __syncthreads();
    }
    const int excl = t > 0 ? tmp[t - 1] : 0;
    __syncthreads();  // tmp may be reused
    return excl;
}

__global__ __launch_bounds__(kTabThreads) void seq_table_kernel(const int *__restrict__ cu, int N, int T,
                                                                int *__restrict__ start, int *__restrict__ cbase,
                                                                int *__restrict__ tok, int *__restrict__ seq,
                                                                int *__restrict__ order) {
    __shared__ int tmp[kTabThreads];
    const int t = threadIdx.x;
    // entries i0 .. i1-1 of the N + 1 boundaries belong to this thread
    const int per = (N + 1 + kTabThreads - 1) / kTabThreads;
    const int i0 = min(t * per, N + 1), i1 = min(i0 + per, N + 1);
    auto clampT = [&](int x) { return min(max(x, 0), T); };

    // 1. boundaries: prefix maximum of the clamped entries
    int m = 0;
    for (int i = i0; i < i1; ++i) m = max(m, clampT(cu[i]));
    int excl = block_scan_excl<true>(m, tmp);
    for (int i = i0; i < i1; ++i) {
        excl = max(excl, clampT(cu[i]));
        start[i] = excl;
    }
    __syncthreads();  // start[] is visible to the whole workgroup

    // 2. chunks per sequence and their exclusive prefix sum
    const int n1 = min(i1, N);
    int cnt = 0;
    for (int n = i0; n < n1; ++n) cnt += (start[n + 1] - start[n] + kChunk - 1) / kChunk;
    int c = block_scan_excl<false>(cnt, tmp);
    for (int n = i0; n < n1; ++n) {
        cbase[n] = c;
        c += (start[n + 1] - start[n] + kChunk - 1) / kChunk;
    }
    if (t == kTabThreads - 1) cbase[N] = c;  // the last thread's running sum is the total
    __syncthreads();

    // 3. the chunk table: first token and sequence of every chunk.  Chunk u
    // belongs to the last sequence n with cbase[n] <= u (empty sequences
    // share their successor's cbase and come before it).
    const int total = cbase[N];
    for (int u = t; u < total; u += kTabThreads) {
        int lo = 0, hi = N - 1;  // invariant: cbase[lo] <= u, and the answer is in [lo, hi]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cbase[mid] <= u) lo = mid;
            else hi = mid - 1;
        }
        tok[u] = start[lo] + (u - cbase[lo]) * kChunk;
        seq[u] = lo;
    }

    // 4. the walk order: every walk of a sequence steps through its chunks one after the other, so
    // the call lasts at least as long as the longest walk, and a long walk dispatched late makes it
    // longer.  Sequences by chunk count, longest first, ties in sequence order: a bitonic sort of
    // one key per thread (count above the low 10 bits, kTabThreads - 1 - n in them; padding -1,
    // sorted last) for up to kTabThreads sequences; beyond that the sequence order itself.
    if (N <= kTabThreads) {
        __shared__ long long keys[kTabThreads];
        keys[t] = t < N ? ((long long)((start[t + 1] - start[t] + kChunk - 1) / kChunk) << 10) | (kTabThreads - 1 - t)
                        : -1;
        for (int k = 2; k <= kTabThreads; k <<= 1)
            for (int j = k >> 1; j > 0; j >>= 1) {
                __syncthreads();
                const int ixj = t ^ j;
                if (ixj > t) {
                    const long long a = keys[t], b = keys[ixj];
                    if ((t & k) == 0 ? a < b : a > b) {  // descending within blocks whose bit k is clear
                        keys[t] = b;
                        keys[ixj] = a;
                    }
                }
            }
        __syncthreads();
        if (t < N) order[t] = kTabThreads - 1 - (int)(keys[t] & (kTabThreads - 1));
    } else {
        for (int n = t; n < N; n += kTabThreads) order[n] = n;
    }
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int varlen_max_chunks(int N, int T) { return (int)(((long)T + 63L * N) / kChunk); }

// Table layout (int32): start [N + 1], cbase [N + 1], tok [NCmax], seq [NCmax], order [N].
size_t seq_table_bytes(int N, int NCmax) {
    return align256(sizeof(int) * (2 * ((size_t)N + 1) + 2 * (size_t)NCmax + (size_t)N));
}

SeqTable seq_table(void *ws, int N, int NCmax) {
    int *p = static_cast<int *>(ws);
    SeqTable tb;
    tb.start = p;
    tb.cbase = p + (N + 1);
    tb.tok = p + 2 * (N + 1);
    tb.seq = p + 2 * (N + 1) + NCmax;
    tb.order = p + 2 * (N + 1) + 2 * NCmax;
    return tb;
}

hipError_t launch_seq_table(const int *cu, int N, int T, void *ws, hipStream_t stream) {
    const int NCmax = varlen_max_chunks(N, T);
    int *p = static_cast<int *>(ws);
    hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(kTabThreads), 0, stream, cu, N, T, p, p + (N + 1),
                       p + 2 * (N + 1), p + 2 * (N + 1) + NCmax, p + 2 * (N + 1) + 2 * NCmax);
    return hipGetLastError();
}

}  // namespace gdr
