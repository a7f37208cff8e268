// Fused recurrent schedule of the gated delta rule: decode (one token) and
// short sequences (T tokens per sequence with the state kept in registers).
//
// Blog summary on the DeltaNet family, "Kernel Triton recurrente fusionado":
// the recurrent schedule fuses decay, prediction, residual, rank-1 write and
// read in one pass over the state; it is the schedule for decode.  Each step
// here is the seven-step recurrence of the oracle for one token:
//   S~ = D S;  p = S~^T k;  e = v - p;  S = S~ + beta k e^T;  o = scale S^T q.
//
// The kernel is bound by HBM: per (sequence, head) it moves the fp32 state
// (Dk*Dv*4 bytes) in and out once and a few hundred bytes of q/k/v/g/beta.
// One 256-thread workgroup owns one state.  Each thread holds Dk*Dv/256 fp32
// of it in registers as float4s; a wavefront's float4 load covers whole
// contiguous state rows (512 B per row at Dv = 128), so every access is a
// fully coalesced 128-bit access and the state is read once and written once.
// The column reductions p = S~^T k and r = S~^T q run in the same pass:
// across the lanes of a wavefront with cross-lane swaps, then across the four
// wavefronts through LDS.  The output uses o = scale (r + beta e (k.q)), so no
// second pass over the state is needed.
//
// A run of T tokens keeps the state in registers: it is read before the
// first token and written after the last.  The one-token kernel below loads
// each token's q, k, v and gates while the previous token is computed (it is
// launched for decode, T = 1); runs of several tokens take
// recurrent_tokens_kernel, which stages the inputs of 16 tokens at a time in
// LDS.
//
// Without the delta rule (delta = false: linear attention, RetNet / Mamba-2,
// GLA; textbook page, update table) the write is S = S~ + k v^T: the same
// pass with e = v and beta = 1 (the prediction is formed and not used; the
// pass is bound by the state's bytes either way) and beta never read.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;

// The updated state goes back with non-temporal stores: it is not read again
// within the call, and the next call usually comes after other work, so
// keeping it in the caches only displaces other data.  Measured on the decode
// workload, whose 256 MiB state fills the last-level cache: 83 us per step
// against 80 us with ordinary stores; with 512 sequences (a 512 MiB state,
// twice that cache) 164 us against 216 us.
__device__ __forceinline__ void store_state(float *p, float4 v) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(p));
}

// The token span [t0, end) of sequence n of a packed batch.  Its offsets are
// cu[n] and cu[n+1], each clamped to [0, T] and raised to the largest offset
// before it: t0 = max over i <= n of clamp(cu[i]), end = max(t0,
// clamp(cu[n+1])).  The prefix maximum is a workgroup reduction (each thread
// takes every kThreads-th offset, then the wavefronts and LDS), so a
// workgroup reads about n / kThreads offsets per thread.  Every thread of the
// workgroup must call it (it holds a barrier).
__device__ __forceinline__ int2 packed_span(const int *__restrict__ cu, size_t n, int T, int *red) {
    const int tid = threadIdx.x;
    int m = 0;
    for (size_t i = tid; i <= n; i += kThreads) m = max(m, min(max(cu[i], 0), T));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    int t0 = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) t0 = max(t0, red[w]);
    return make_int2(t0, max(t0, min(max(cu[n + 1], 0), T)));
}

template <int DK, int DV, bool PC, bool KZ, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void recurrent_step_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    void *__restrict__ o, int T, int H, float eps, float scale, bool delta, const int *__restrict__ cu) {
    constexpr int TPR = DV / 4;          // threads per state row (one float4 each)
    constexpr int RPP = kThreads / TPR;  // rows per pass of the workgroup
    constexpr int PASSES = DK / RPP;
    static_assert(DK % RPP == 0, "state rows must tile the workgroup");

    const size_t nh = blockIdx.x;  // flattened (sequence, head)
    const size_t n = nh / H, h = nh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c4 = tid % TPR;      // column quad owned by this thread
    const int r0 = tid / TPR;      // first row owned by this thread

    // Per-token LDS is double-buffered by token parity: token t+1 fills its
    // buffers while token t's are still read, so each token needs two
    // barriers (inputs published; partial sums published).
    __shared__ float sk[2][DK], sq[2][DK], sa[2][PC ? DK : 1];
    __shared__ float4 red[2][2][4][TPR];
    __shared__ float s_kq[2], s_beta[2];

    float *S = state + nh * DK * DV;

    // Issue the state loads first; they dominate the latency.
    float4 s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        s[p] = *reinterpret_cast<const float4 *>(S + (size_t)(p * RPP + r0) * DV + 4 * c4);

    // token t of this (sequence, head): row (n T + t) H + h of q, k, v, g,
    // beta; in a packed batch (cu != NULL, T tokens in all) row (t0 + t) H + h
    // for the sequence's first token t0, its tokens [cu[n], cu[n+1]) with each
    // offset clamped to [0, T] and raised to the largest one before it
    size_t first = (size_t)n * T;
    if (cu) {
        __shared__ int red_cu[kThreads / 64];
        const int2 span = packed_span(cu, n, T, red_cu);
        first = span.x;
        T = span.y - span.x;
    }
    auto row_of = [&](int t) { return (first + t) * H + h; };
    float kin = 0.f, qin = 0.f, gin = 0.f, bin = 1.f, gsc = 0.f;
    float4 vin;
    auto fetch = [&](int t) {  // token t's inputs into registers
        const size_t r = row_of(t);
        if (tid < DK) {
            kin = load_in<IN_BF16>(k, r * DK + tid);
            qin = load_in<IN_BF16>(q, r * DK + tid);
            if constexpr (PC) gin = g[r * DK + tid];
        }
        vin = make_float4(load_in<IN_BF16>(v, r * DV + 4 * c4 + 0), load_in<IN_BF16>(v, r * DV + 4 * c4 + 1),
                          load_in<IN_BF16>(v, r * DV + 4 * c4 + 2), load_in<IN_BF16>(v, r * DV + 4 * c4 + 3));
        if constexpr (!PC) gsc = g[r];
        if (wave == 0 && delta) bin = beta[r];
    };
    if (T > 0) fetch(0);
    for (int t = 0; t < T; ++t) {
        const int b = t & 1;
        if (tid < DK) {
            sk[b][tid] = kin;
            sq[b][tid] = qin;
            if constexpr (PC) sa[b][tid] = __expf(gin);
        }
        const float4 vv = vin;
        const float a_scalar = PC ? 1.0f : __expf(gsc);
        const float bet = bin;
        if (t + 1 < T) fetch(t + 1);  // next token's inputs, in flight during this one
        __syncthreads();

        if (wave == 0) {
            float kq = 0.f, kk = 0.f;
            for (int i = lane; i < DK; i += 64) {
                kq += sk[b][i] * sq[b][i];
                kk += sk[b][i] * sk[b][i];
            }
            kq = wave_sum(kq);
            kk = wave_sum(kk);
            if (lane == 0) {
                s_kq[b] = kq;
                s_beta[b] = KZ ? bet / (kk + eps) : bet;
            }
        }

        // Column partial sums of the decayed state against k (prediction) and q (read).
        float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = p * RPP + r0;
            const float a = PC ? sa[b][row] : a_scalar;
            const float ak = a * sk[b][row], aq = a * sq[b][row];
            pk.x += ak * s[p].x; pk.y += ak * s[p].y; pk.z += ak * s[p].z; pk.w += ak * s[p].w;
            pq.x += aq * s[p].x; pq.y += aq * s[p].y; pq.z += aq * s[p].z; pq.w += aq * s[p].w;
        }
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1) {
            pk.x += __shfl_xor(pk.x, off, 64); pk.y += __shfl_xor(pk.y, off, 64);
            pk.z += __shfl_xor(pk.z, off, 64); pk.w += __shfl_xor(pk.w, off, 64);
            pq.x += __shfl_xor(pq.x, off, 64); pq.y += __shfl_xor(pq.y, off, 64);
            pq.z += __shfl_xor(pq.z, off, 64); pq.w += __shfl_xor(pq.w, off, 64);
        }
        if (lane < TPR) {
            red[b][0][wave][c4] = pk;
            red[b][1][wave][c4] = pq;
        }
        __syncthreads();
        float4 P = red[b][0][0][c4], R = red[b][1][0][c4];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const float4 x = red[b][0][w][c4], y = red[b][1][w][c4];
            P.x += x.x; P.y += x.y; P.z += x.z; P.w += x.w;
            R.x += y.x; R.y += y.y; R.z += y.z; R.w += y.w;
        }
        const float bt = s_beta[b];
        const float4 e = delta ? make_float4(vv.x - P.x, vv.y - P.y, vv.z - P.z, vv.w - P.w) : vv;

        if (r0 == 0) {  // read after write: o = scale (S~^T q + beta e (k.q))
            const float bkq = bt * s_kq[b];
            const size_t ob = row_of(t) * DV + 4 * c4;
            store_out<OUT_BF16>(o, ob + 0, scale * (R.x + bkq * e.x));
            store_out<OUT_BF16>(o, ob + 1, scale * (R.y + bkq * e.y));
            store_out<OUT_BF16>(o, ob + 2, scale * (R.z + bkq * e.z));
            store_out<OUT_BF16>(o, ob + 3, scale * (R.w + bkq * e.w));
        }

#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = p * RPP + r0;
            const float a = PC ? sa[b][row] : a_scalar;
            const float bk = bt * sk[b][row];
            s[p].x = a * s[p].x + bk * e.x;
            s[p].y = a * s[p].y + bk * e.y;
            s[p].z = a * s[p].z + bk * e.z;
            s[p].w = a * s[p].w + bk * e.w;
        }
    }

#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        store_state(S + (size_t)(p * RPP + r0) * DV + 4 * c4, s[p]);
}

// Several tokens per sequence: the same recurrence and thread layout, with
// the tokens' inputs staged in LDS a block of kTokBlock tokens at a time (one
// cooperative load per block, so no token waits on a global load), and one
// barrier per token.  The per-token LDS that crosses that barrier (partial
// sums, k.q, the write strength) is double-buffered by token parity: token
// t+2 rewrites a buffer only after every thread has passed token t+1's
// barrier, i.e. has finished reading token t's.
constexpr int kTokBlock = 16;

template <int DK, int DV, bool PC, bool KZ, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 3) void recurrent_tokens_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    void *__restrict__ o, int T, int H, float eps, float scale, bool delta, const int *__restrict__ cu) {
    constexpr int TPR = DV / 4;
    constexpr int RPP = kThreads / TPR;
    constexpr int PASSES = DK / RPP;
    static_assert(DK % RPP == 0, "state rows must tile the workgroup");

    const size_t nh = blockIdx.x;
    const size_t n = nh / H, h = nh % H;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c4 = tid % TPR;
    const int r0 = tid / TPR;

    __shared__ float sk[kTokBlock][DK], sq[kTokBlock][DK], sa[PC ? kTokBlock : 1][DK];
    __shared__ float4 sv[kTokBlock][TPR];
    __shared__ float sgs[kTokBlock], sbt[kTokBlock];
    __shared__ float4 red[2][2][4][TPR];
    __shared__ float s_kq[2], s_beta[2];

    float *S = state + nh * DK * DV;
    float4 s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        s[p] = *reinterpret_cast<const float4 *>(S + (size_t)(p * RPP + r0) * DV + 4 * c4);

    // token rows as in the one-token kernel (packed batches: offsets clamped
    // to [0, T] and raised to the largest one before them)
    size_t first = (size_t)n * T;
    if (cu) {
        __shared__ int red_cu[kThreads / 64];
        const int2 span = packed_span(cu, n, T, red_cu);
        first = span.x;
        T = span.y - span.x;
    }
    auto row_of = [&](int t) { return (first + t) * H + h; };

    for (int tb0 = 0; tb0 < T; tb0 += kTokBlock) {
        const int nb = min(kTokBlock, T - tb0);
        __syncthreads();  // the previous block's inputs are no longer read
        for (int e = tid; e < nb * DK; e += kThreads) {
            const int tt = e / DK, i = e % DK;
            const size_t r = row_of(tb0 + tt);
            sk[tt][i] = load_in<IN_BF16>(k, r * DK + i);
            sq[tt][i] = load_in<IN_BF16>(q, r * DK + i);
            if constexpr (PC) sa[tt][i] = __expf(g[r * DK + i]);
        }
        for (int e = tid; e < nb * TPR; e += kThreads) {
            const int tt = e / TPR, j = e % TPR;
            const size_t r = row_of(tb0 + tt);
            sv[tt][j] = make_float4(load_in<IN_BF16>(v, r * DV + 4 * j + 0), load_in<IN_BF16>(v, r * DV + 4 * j + 1),
                                    load_in<IN_BF16>(v, r * DV + 4 * j + 2), load_in<IN_BF16>(v, r * DV + 4 * j + 3));
        }
        if (tid < nb) {
            const size_t r = row_of(tb0 + tid);
            sgs[tid] = PC ? 1.0f : __expf(g[r]);
            sbt[tid] = delta ? beta[r] : 1.0f;
        }
        __syncthreads();

        for (int tt = 0; tt < nb; ++tt) {
            const int t = tb0 + tt;
            const int b = t & 1;
            if (wave == 0) {
                float kq = 0.f, kk = 0.f;
                for (int i = lane; i < DK; i += 64) {
                    kq += sk[tt][i] * sq[tt][i];
                    kk += sk[tt][i] * sk[tt][i];
                }
                kq = wave_sum(kq);
                kk = wave_sum(kk);
                if (lane == 0) {
                    s_kq[b] = kq;
                    s_beta[b] = KZ ? sbt[tt] / (kk + eps) : sbt[tt];
                }
            }
            const float a_scalar = sgs[tt];
            float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int row = p * RPP + r0;
                const float a = PC ? sa[tt][row] : a_scalar;
                const float ak = a * sk[tt][row], aq = a * sq[tt][row];
                pk.x += ak * s[p].x; pk.y += ak * s[p].y; pk.z += ak * s[p].z; pk.w += ak * s[p].w;
                pq.x += aq * s[p].x; pq.y += aq * s[p].y; pq.z += aq * s[p].z; pq.w += aq * s[p].w;
            }
#pragma unroll
            for (int off = TPR; off < 64; off <<= 1) {
                pk.x += __shfl_xor(pk.x, off, 64); pk.y += __shfl_xor(pk.y, off, 64);
                pk.z += __shfl_xor(pk.z, off, 64); pk.w += __shfl_xor(pk.w, off, 64);
                pq.x += __shfl_xor(pq.x, off, 64); pq.y += __shfl_xor(pq.y, off, 64);
                pq.z += __shfl_xor(pq.z, off, 64); pq.w += __shfl_xor(pq.w, off, 64);
            }
            if (lane < TPR) {
                red[b][0][wave][c4] = pk;
                red[b][1][wave][c4] = pq;
            }
            __syncthreads();
            float4 P = red[b][0][0][c4], R = red[b][1][0][c4];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const float4 x = red[b][0][w][c4], y = red[b][1][w][c4];
                P.x += x.x; P.y += x.y; P.z += x.z; P.w += x.w;
                R.x += y.x; R.y += y.y; R.z += y.z; R.w += y.w;
            }
            const float bt = s_beta[b];
            const float4 vv = sv[tt][c4];
            const float4 e = delta ? make_float4(vv.x - P.x, vv.y - P.y, vv.z - P.z, vv.w - P.w) : vv;
            if (r0 == 0) {  // read after write: o = scale (S~^T q + beta e (k.q))
                const float bkq = bt * s_kq[b];
                const size_t ob = row_of(t) * DV + 4 * c4;
                store_out<OUT_BF16>(o, ob + 0, scale * (R.x + bkq * e.x));
                store_out<OUT_BF16>(o, ob + 1, scale * (R.y + bkq * e.y));
                store_out<OUT_BF16>(o, ob + 2, scale * (R.z + bkq * e.z));
                store_out<OUT_BF16>(o, ob + 3, scale * (R.w + bkq * e.w));
            }
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int row = p * RPP + r0;
                const float a = PC ? sa[tt][row] : a_scalar;
                const float bk = bt * sk[tt][row];
                s[p].x = a * s[p].x + bk * e.x;
                s[p].y = a * s[p].y + bk * e.y;
                s[p].z = a * s[p].z + bk * e.z;
                s[p].w = a * s[p].w + bk * e.w;
            }
        }
    }

#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        store_state(S + (size_t)(p * RPP + r0) * DV + 4 * c4, s[p]);
}

template <int DK, int DV, bool PC, bool KZ, bool IB, bool OB>
hipError_t launch_t(const StepArgs &a) {
    const unsigned grid = static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H);
    // one token per sequence (decode): the one-token kernel; more: tokens staged in LDS
    const bool many = a.cu ? a.T > a.N : a.T > 1;
    if (many)
        GDR_LAUNCH((recurrent_tokens_kernel<DK, DV, PC, KZ, IB, OB>), dim3(grid), dim3(kThreads), a.stream, a.ev0,
                   a.ev1, a.q, a.k, a.v, a.g, a.beta, a.state, a.o, a.T, a.H, a.eps, a.scale, a.delta, a.cu);
    else
        GDR_LAUNCH((recurrent_step_kernel<DK, DV, PC, KZ, IB, OB>), dim3(grid), dim3(kThreads), a.stream, a.ev0,
                   a.ev1, a.q, a.k, a.v, a.g, a.beta, a.state, a.o, a.T, a.H, a.eps, a.scale, a.delta, a.cu);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_d(const StepArgs &a) {
    const int key = (a.per_channel ? 8 : 0) | (a.kaczmarz ? 4 : 0) | (a.qkv_bf16 ? 2 : 0) | (a.o_bf16 ? 1 : 0);
    switch (key) {
        case 0: return launch_t<DK, DV, false, false, false, false>(a);
        case 1: return launch_t<DK, DV, false, false, false, true>(a);
        case 2: return launch_t<DK, DV, false, false, true, false>(a);
        case 3: return launch_t<DK, DV, false, false, true, true>(a);
        case 4: return launch_t<DK, DV, false, true, false, false>(a);
        case 5: return launch_t<DK, DV, false, true, false, true>(a);
        case 6: return launch_t<DK, DV, false, true, true, false>(a);
        case 7: return launch_t<DK, DV, false, true, true, true>(a);
        case 8: return launch_t<DK, DV, true, false, false, false>(a);
        case 9: return launch_t<DK, DV, true, false, false, true>(a);
        case 10: return launch_t<DK, DV, true, false, true, false>(a);
        case 11: return launch_t<DK, DV, true, false, true, true>(a);
        case 12: return launch_t<DK, DV, true, true, false, false>(a);
        case 13: return launch_t<DK, DV, true, true, false, true>(a);
        case 14: return launch_t<DK, DV, true, true, true, false>(a);
        default: return launch_t<DK, DV, true, true, true, true>(a);
    }
}

}  // namespace

hipError_t launch_recurrent_step(const StepArgs &a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_d<64, 128>(a);
    return launch_d<64, 64>(a);
}

}  // namespace gdr
