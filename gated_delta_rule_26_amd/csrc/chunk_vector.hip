// Chunked forward pass on the vector ALUs, fp32 arithmetic throughout.
//
// This is the path for fp32 inputs (on MI355X the fp32 matrix cores and the
// fp32 vector ALUs have the same peak, so fp32 products gain nothing from
// MFMA), and a second implementation of the chunked algebra for bf16 inputs.
//
// The algebra (blog summary on the DeltaNet family, "KDA por chunks"; here
// in the d_k x d_v state orientation): inside a chunk of n <= 64 tokens with
// in-chunk cumulative log-decay G_i = g_0 + ... + g_i,
//   R_ij  = beta_i sum_c k_ic exp(G_ic - G_jc) k_jc        (j < i)
//   A_ij  = scale sum_c q_ic exp(G_ic - G_jc) k_jc         (j <= i)
//   (I + R) W = Diag(beta) Diag(exp G) K,  (I + R) U = Diag(beta) V
// and then, walking the chunks of one sequence in order,
//   E       = U - W S                       (the corrected writes)
//   O       = scale (exp(G) o Q) S + A E    (read of the entering state plus
//                                            the causal in-chunk reads)
//   S_next  = Diag(exp G_{n-1}) S + (exp(G_{n-1} - G) o K)^T E.
// Padded rows of a partial last chunk have k = q = v = 0, g = 0, beta = 0,
// which makes them contribute nothing and keeps G_{63} = G_{n-1}.
// Without the delta rule (the additive write S = D S + k v^T of the textbook
// page's update table) R = 0, beta = 1 and W = 0, so E = U = V: the same
// kernels with those three values.
//
// Two kernels: intra (one workgroup per (sequence, head, chunk), fully
// parallel) writes W, U, A and G to the workspace; state (one workgroup per
// (sequence, head, 32-column slice of the value axis)) walks the chunks in
// order with the fp32 state slice in LDS and writes o and the final state.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int C = kChunk;
constexpr int kThreads = 256;
constexpr int kBV = 32;  // value columns per state workgroup

struct VecWs {  // workspace carve-up, all fp32
    float *W, *U, *A, *G;
};

inline VecWs carve(void *ws, size_t nchunks, int Dk, int Dv, bool pc) {
    float *p = static_cast<float *>(ws);
    VecWs w;
    w.W = p; p += nchunks * C * Dk;
    w.U = p; p += nchunks * C * Dv;
    w.A = p; p += nchunks * C * C;
    w.G = p;
    (void)pc;
    return w;
}

template <int DK, int DV, bool PC, bool KZ, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void intra_vector_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, int T, int H, int NC, float eps,
    float scale, bool delta, float *__restrict__ wsW, float *__restrict__ wsU, float *__restrict__ wsA,
    float *__restrict__ wsG, SeqTable tb) {
    constexpr int GK = PC ? DK : 1;
    const int ci = blockIdx.x;  // (b*H + h)*NC + c; packed batches: u*H + h for chunk u of the table
    if (tb.start && ci >= tb.cbase[tb.N] * H) return;  // past the chunks the table holds
    size_t row0;  // [.., H, D] row of the chunk's token 0; token i is row row0 + i H
    int n;
    {
        const int u = tb.start ? ci / H : 0, hh = tb.start ? ci % H : (ci / NC) % H;
        const int b = ci / NC / H, c = ci % NC;
        if (tb.start) {
            const int t0 = tb.tok[u];
            n = min(C, tb.start[tb.seq[u] + 1] - t0);
            row0 = (size_t)t0 * H + hh;
        } else {
            n = min(C, T - c * C);
            row0 = ((size_t)b * T + c * C) * H + hh;
        }
    }
    const int tid = threadIdx.x;

    __shared__ float sK[C][DK + 1];
    __shared__ float sQ[C][DK + 1];
    __shared__ float sG[C][GK];
    __shared__ __align__(16) float sR[C][C];
    __shared__ float sBeta[C];

    for (int idx = tid; idx < C * DK; idx += kThreads) {
        const int i = idx / DK, cc = idx % DK;
        const size_t off = (row0 + (size_t)i * H) * DK + cc;
        sK[i][cc] = i < n ? load_in<IN_BF16>(k, off) : 0.f;
        sQ[i][cc] = i < n ? load_in<IN_BF16>(q, off) : 0.f;
    }
    if constexpr (PC) {
        for (int idx = tid; idx < C * DK; idx += kThreads) {
            const int i = idx / DK, cc = idx % DK;
            sG[i][cc] = i < n ? g[(row0 + (size_t)i * H) * DK + cc] : 0.f;
        }
    } else {
        if (tid < C) sG[tid][0] = tid < n ? g[row0 + (size_t)tid * H] : 0.f;
    }
    __syncthreads();

    // in-chunk inclusive cumulative sum of the log-decays, one channel per thread
    if (tid < GK) {
        float run = 0.f;
        for (int i = 0; i < C; ++i) {
            run += sG[i][tid];
            sG[i][tid] = run;
        }
    }
    if (tid >= kThreads - C) {  // the last wavefront prepares beta
        const int i = tid - (kThreads - C);
        float bv = 0.f;
        if (i < n && !delta) {
            bv = 1.f;
        } else if (i < n) {
            const float given = beta[row0 + (size_t)i * H];
            if constexpr (KZ) {
                float kk = 0.f;
                for (int cc = 0; cc < DK; ++cc) kk += sK[i][cc] * sK[i][cc];
                bv = given / (kk + eps);
            } else {
                bv = given;
            }
        }
        sBeta[i] = bv;
    }
    __syncthreads();

    // R (strictly lower) and A (lower, diagonal kept): thread -> row i, 16 columns
    {
        const int i = tid >> 2;
        const int jb = (tid & 3) * 16;
        float *Ag = wsA + (size_t)ci * C * C + (size_t)i * C;
        for (int jj = 0; jj < 16; ++jj) {
            const int j = jb + jj;
            float r = 0.f, a = 0.f;
            if (j <= i) {
                if constexpr (PC) {
                    for (int cc = 0; cc < DK; ++cc) {
                        const float gam = __expf(sG[i][cc] - sG[j][cc]);
                        const float kj = sK[j][cc] * gam;
                        r += sK[i][cc] * kj;
                        a += sQ[i][cc] * kj;
                    }
                } else {
                    for (int cc = 0; cc < DK; ++cc) {
                        r += sK[i][cc] * sK[j][cc];
                        a += sQ[i][cc] * sK[j][cc];
                    }
                    const float gam = __expf(sG[i][0] - sG[j][0]);
                    r *= gam;
                    a *= gam;
                }
            }
            sR[i][j] = delta && j < i ? sBeta[i] * r : 0.f;
            Ag[j] = scale * a;
        }
    }
    __syncthreads();

    // Forward substitution, one column of [W | U] per thread:
    //   x_i = rhs_i - sum_{j<i} R_ij x_j   (unit lower-triangular solve)
    // The loops stay rolled: unrolled, the compiler keeps about 2,000 values
    // live across the 64 rows (every register plus 6 KB of spills per lane);
    // rolled, the column x goes to LDS or scratch and the kernel takes half
    // the time (measured on the GDN and KDA prefill shapes).
    if (tid < DK + DV) {
        float x[C];
        const bool isW = tid < DK;
        const int col = isW ? tid : tid - DK;
#pragma unroll 1
        for (int i = 0; i < C; ++i) {
            float rhs;
            if (isW) {
                const float gi = PC ? sG[i][col] : sG[i][0];
                rhs = delta ? sBeta[i] * __expf(gi) * sK[i][col] : 0.f;
            } else {
                rhs = i < n ? sBeta[i] * load_in<IN_BF16>(v, (row0 + (size_t)i * H) * DV + col) : 0.f;
            }
#pragma unroll 1
            for (int j4 = 0; j4 < i / 4; ++j4) {
                const float4 r4 = *reinterpret_cast<const float4 *>(&sR[i][4 * j4]);
                rhs -= r4.x * x[4 * j4] + r4.y * x[4 * j4 + 1] + r4.z * x[4 * j4 + 2] + r4.w * x[4 * j4 + 3];
            }
            for (int j = (i / 4) * 4; j < i; ++j) rhs -= sR[i][j] * x[j];
            x[i] = rhs;
        }
        float *dst = isW ? wsW + (size_t)ci * C * DK : wsU + (size_t)ci * C * DV;
        const int ld = isW ? DK : DV;
#pragma unroll
        for (int i = 0; i < C; ++i) dst[(size_t)i * ld + col] = x[i];
    }

    float *Gg = wsG + (size_t)ci * C * GK;
    for (int idx = tid; idx < C * GK; idx += kThreads) Gg[idx] = sG[idx / GK][idx % GK];
}

template <int DK, int DV, bool PC, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void state_vector_kernel(
    const void *__restrict__ q, const void *__restrict__ k, int T, int H, int NC,
    const float *__restrict__ wsW, const float *__restrict__ wsU, const float *__restrict__ wsA,
    const float *__restrict__ wsG, const float *__restrict__ s0, void *__restrict__ o,
    float *__restrict__ s_final, float scale, SeqTable tb) {
    constexpr int GK = PC ? DK : 1;
    constexpr int NT = DV / kBV;
    const int tile = blockIdx.x % NT;
    const int bh = walk_seq(blockIdx.x / NT, H, tb);  // packed batches: longest sequences first
    const int b = bh / H, h = bh % H;
    const int j0 = tile * kBV;
    // this sequence: [.., H, D] row of its token 0, its length and chunks, and
    // the workspace index of its chunk c (first + c * cstep)
    size_t head0, cfirst, cstep;
    int L, nc;
    if (tb.start) {
        const int s = tb.start[b], cb = tb.cbase[b];
        head0 = (size_t)s * H + h;
        L = tb.start[b + 1] - s;
        nc = tb.cbase[b + 1] - cb;
        cfirst = (size_t)cb * H + h;
        cstep = H;
    } else {
        head0 = (size_t)b * T * H + h;
        L = T;
        nc = NC;
        cfirst = (size_t)bh * NC;
        cstep = 1;
    }
    const int tid = threadIdx.x;
    const int jj = tid % kBV;  // value column within the slice owned by this thread
    const int rr = tid / kBV;  // 0..7

    __shared__ float sS[DK][kBV];
    __shared__ float sX[C][DK + 1];
    __shared__ float sE[C][kBV + 1];
    __shared__ float sG[C][GK];
    __shared__ float sA[C][C + 1];

    const size_t sbase = (size_t)bh * DK * DV;
    for (int idx = tid; idx < DK * kBV; idx += kThreads) {
        const int r = idx / kBV, cc = idx % kBV;
        sS[r][cc] = s0 ? s0[sbase + (size_t)r * DV + j0 + cc] : 0.f;
    }

    for (int c = 0; c < nc; ++c) {
        const size_t ci = cfirst + (size_t)c * cstep;
        const int t0 = c * C;
        const int n = min(C, L - t0);
        const float *W = wsW + ci * C * DK;
        const float *U = wsU + ci * C * DV;
        const float *A = wsA + ci * C * C;
        const float *G = wsG + ci * C * GK;

        for (int idx = tid; idx < C * DK; idx += kThreads) sX[idx / DK][idx % DK] = W[idx];
        for (int idx = tid; idx < C * GK; idx += kThreads) sG[idx / GK][idx % GK] = G[idx];
        for (int idx = tid; idx < C * C; idx += kThreads) sA[idx / C][idx % C] = A[idx];
        __syncthreads();

        // E = U - W S
        for (int i = rr; i < C; i += kThreads / kBV) {
            float acc = U[(size_t)i * DV + j0 + jj];
            for (int cc = 0; cc < DK; ++cc) acc -= sX[i][cc] * sS[cc][jj];
            sE[i][jj] = acc;
        }
        __syncthreads();

        // decayed, scaled queries: scale exp(G_i) q_i
        for (int idx = tid; idx < C * DK; idx += kThreads) {
            const int i = idx / DK, cc = idx % DK;
            const float gi = PC ? sG[i][cc] : sG[i][0];
            sX[i][cc] = i < n ? scale * __expf(gi) * load_in<IN_BF16>(q, (head0 + (size_t)(t0 + i) * H) * DK + cc)
                              : 0.f;
        }
        __syncthreads();

        // O = scale (exp(G) o Q) S + A E
        for (int i = rr; i < n; i += kThreads / kBV) {
            float acc = 0.f;
            for (int cc = 0; cc < DK; ++cc) acc += sX[i][cc] * sS[cc][jj];
            for (int j = 0; j <= i; ++j) acc += sA[i][j] * sE[j][jj];
            store_out<OUT_BF16>(o, (head0 + (size_t)(t0 + i) * H) * DV + j0 + jj, acc);
        }
        __syncthreads();

        // keys decayed to the chunk end: exp(G_63 - G_j) k_j
        for (int idx = tid; idx < C * DK; idx += kThreads) {
            const int i = idx / DK, cc = idx % DK;
            const float gi = PC ? sG[i][cc] : sG[i][0];
            const float ge = PC ? sG[C - 1][cc] : sG[C - 1][0];
            sX[i][cc] = i < n ? __expf(ge - gi) * load_in<IN_BF16>(k, (head0 + (size_t)(t0 + i) * H) * DK + cc)
                              : 0.f;
        }
        __syncthreads();

        // S <- Diag(exp G_63) S + Kend^T E (each thread updates its own entries)
        for (int r = rr; r < DK; r += kThreads / kBV) {
            const float ge = PC ? sG[C - 1][r] : sG[C - 1][0];
            float acc = __expf(ge) * sS[r][jj];
            for (int j = 0; j < C; ++j) acc += sX[j][r] * sE[j][jj];
            sS[r][jj] = acc;
        }
        __syncthreads();
    }

    if (s_final) {
        for (int idx = tid; idx < DK * kBV; idx += kThreads) {
            const int r = idx / kBV, cc = idx % kBV;
            s_final[sbase + (size_t)r * DV + j0 + cc] = sS[r][cc];
        }
    }
}

template <int DK, int DV, bool PC, bool KZ, bool IB, bool OB>
hipError_t launch_t(const ChunkArgs &a, int stage) {
    const size_t nchunks = (size_t)chunk_slots(a);
    VecWs w = carve(a.ws, nchunks, DK, DV, PC);
    if (stage != 1) {
        hipLaunchKernelGGL((intra_vector_kernel<DK, DV, PC, KZ, IB>), dim3((unsigned)nchunks), dim3(kThreads), 0,
                           a.stream, a.q, a.k, a.v, a.g, a.beta, a.T, a.H, a.NC, a.eps, a.scale, a.delta, w.W, w.U,
                           w.A, w.G, a.tab);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || stage == 0) return e;
    }
    const unsigned grid = (unsigned)(a.B * a.H * (DV / kBV));
    hipLaunchKernelGGL((state_vector_kernel<DK, DV, PC, IB, OB>), dim3(grid), dim3(kThreads), 0, a.stream,
                       a.q, a.k, a.T, a.H, a.NC, w.W, w.U, w.A, w.G, a.s0, a.o, a.s_final, a.scale, a.tab);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_d(const ChunkArgs &a, int stage) {
    const int key = (a.per_channel ? 8 : 0) | (a.kaczmarz ? 4 : 0) | (a.qkv_bf16 ? 2 : 0) | (a.o_bf16 ? 1 : 0);
    switch (key) {
        case 0: return launch_t<DK, DV, false, false, false, false>(a, stage);
        case 1: return launch_t<DK, DV, false, false, false, true>(a, stage);
        case 2: return launch_t<DK, DV, false, false, true, false>(a, stage);
        case 3: return launch_t<DK, DV, false, false, true, true>(a, stage);
        case 4: return launch_t<DK, DV, false, true, false, false>(a, stage);
        case 5: return launch_t<DK, DV, false, true, false, true>(a, stage);
        case 6: return launch_t<DK, DV, false, true, true, false>(a, stage);
        case 7: return launch_t<DK, DV, false, true, true, true>(a, stage);
        case 8: return launch_t<DK, DV, true, false, false, false>(a, stage);
        case 9: return launch_t<DK, DV, true, false, false, true>(a, stage);
        case 10: return launch_t<DK, DV, true, false, true, false>(a, stage);
        case 11: return launch_t<DK, DV, true, false, true, true>(a, stage);
        case 12: return launch_t<DK, DV, true, true, false, false>(a, stage);
        case 13: return launch_t<DK, DV, true, true, false, true>(a, stage);
        case 14: return launch_t<DK, DV, true, true, true, false>(a, stage);
        default: return launch_t<DK, DV, true, true, true, true>(a, stage);
    }
}

__global__ void state_init_kernel(float *__restrict__ dst, const float *__restrict__ src, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

size_t chunk_vector_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel) {
    const size_t nchunks = (size_t)B * H * NC;
    const size_t gk = per_channel ? (size_t)Dk : 1;
    return nchunks * C * ((size_t)Dk + Dv + C + gk) * sizeof(float);
}

hipError_t launch_chunk_vector(const ChunkArgs &a, int stage) {
    if (a.Dk == 128 && a.Dv == 128) return launch_d<128, 128>(a, stage);
    if (a.Dk == 128 && a.Dv == 64) return launch_d<128, 64>(a, stage);
    if (a.Dk == 64 && a.Dv == 128) return launch_d<64, 128>(a, stage);
    return launch_d<64, 64>(a, stage);
}

hipError_t launch_state_init(float *dst, const float *src, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(state_init_kernel, dim3(blocks), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace gdr
