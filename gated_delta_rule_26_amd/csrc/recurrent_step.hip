// Fused single-token recurrent step of the gated delta rule (decode).
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
// Without the delta rule (delta = false: linear attention, RetNet / Mamba-2,
// GLA; textbook page, update table) the write is S = S~ + k v^T: the same
// pass with e = v and beta = 1 (the prediction is formed and not used; the
// pass is bound by the state's bytes either way) and beta never read.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;

template <int DK, int DV, bool PC, bool KZ, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void recurrent_step_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    void *__restrict__ o, float eps, float scale, bool delta) {
    constexpr int TPR = DV / 4;          // threads per state row (one float4 each)
    constexpr int RPP = kThreads / TPR;  // rows per pass of the workgroup
    constexpr int PASSES = DK / RPP;
    static_assert(DK % RPP == 0, "state rows must tile the workgroup");

    const size_t nh = blockIdx.x;  // flattened (sequence, head)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c4 = tid % TPR;      // column quad owned by this thread
    const int r0 = tid / TPR;      // first row owned by this thread

    __shared__ float sk[DK], sq[DK], sa[PC ? DK : 1];
    __shared__ float4 red[2][4][TPR];
    __shared__ float s_kq, s_beta;

    float *S = state + nh * DK * DV;

    // Issue the state loads first; they dominate the latency.
    float4 s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        s[p] = *reinterpret_cast<const float4 *>(S + (size_t)(p * RPP + r0) * DV + 4 * c4);

    if (tid < DK) {
        sk[tid] = load_in<IN_BF16>(k, nh * DK + tid);
        sq[tid] = load_in<IN_BF16>(q, nh * DK + tid);
        if constexpr (PC) sa[tid] = __expf(g[nh * DK + tid]);
    }
    const float4 vv = make_float4(load_in<IN_BF16>(v, nh * DV + 4 * c4 + 0),
                                  load_in<IN_BF16>(v, nh * DV + 4 * c4 + 1),
                                  load_in<IN_BF16>(v, nh * DV + 4 * c4 + 2),
                                  load_in<IN_BF16>(v, nh * DV + 4 * c4 + 3));
    const float a_scalar = PC ? 1.0f : __expf(g[nh]);
    __syncthreads();

    if (wave == 0) {
        float kq = 0.f, kk = 0.f;
        for (int i = lane; i < DK; i += 64) {
            kq += sk[i] * sq[i];
            kk += sk[i] * sk[i];
        }
        kq = wave_sum(kq);
        kk = wave_sum(kk);
        if (lane == 0) {
            s_kq = kq;
            const float b = delta ? beta[nh] : 1.f;
            s_beta = KZ ? b / (kk + eps) : b;
        }
    }

    // Column partial sums of the decayed state against k (prediction) and q (read).
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int row = p * RPP + r0;
        const float a = PC ? sa[row] : a_scalar;
        const float ak = a * sk[row], aq = a * sq[row];
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
        red[0][wave][c4] = pk;
        red[1][wave][c4] = pq;
    }
    __syncthreads();
    float4 P = red[0][0][c4], R = red[1][0][c4];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const float4 a = red[0][w][c4], b = red[1][w][c4];
        P.x += a.x; P.y += a.y; P.z += a.z; P.w += a.w;
        R.x += b.x; R.y += b.y; R.z += b.z; R.w += b.w;
    }
    const float bt = s_beta;
    const float4 e = delta ? make_float4(vv.x - P.x, vv.y - P.y, vv.z - P.z, vv.w - P.w) : vv;

    if (r0 == 0) {  // read after write: o = scale (S~^T q + beta e (k.q))
        const float bkq = bt * s_kq;
        const size_t ob = nh * DV + 4 * c4;
        store_out<OUT_BF16>(o, ob + 0, scale * (R.x + bkq * e.x));
        store_out<OUT_BF16>(o, ob + 1, scale * (R.y + bkq * e.y));
        store_out<OUT_BF16>(o, ob + 2, scale * (R.z + bkq * e.z));
        store_out<OUT_BF16>(o, ob + 3, scale * (R.w + bkq * e.w));
    }

#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int row = p * RPP + r0;
        const float a = PC ? sa[row] : a_scalar;
        const float bk = bt * sk[row];
        float4 ns;
        ns.x = a * s[p].x + bk * e.x;
        ns.y = a * s[p].y + bk * e.y;
        ns.z = a * s[p].z + bk * e.z;
        ns.w = a * s[p].w + bk * e.w;
        *reinterpret_cast<float4 *>(S + (size_t)row * DV + 4 * c4) = ns;
    }
}

template <int DK, int DV, bool PC, bool KZ, bool IB, bool OB>
hipError_t launch_t(const StepArgs &a) {
    const unsigned grid = static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H);
    hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, PC, KZ, IB, OB>), dim3(grid), dim3(kThreads),
                       0, a.stream, a.q, a.k, a.v, a.g, a.beta, a.state, a.o, a.eps, a.scale,
                       a.delta);
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
