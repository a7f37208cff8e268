// Backward pass of the chunked forward pass (training), fp32 vector ALUs.
//
// The pages derive no backward pass (the blog summary on the DeltaNet family
// calls the chunked mode the training mode, "Pipeline Triton por chunks"), so
// it is derived here from the chunk algebra of the forward pass ("KDA por
// chunks", in the d_k x d_v state orientation).  For a chunk with entering
// state S, in-chunk cumulative log-decay G_i (one value, or one per key
// channel c), write strengths beta and P_ijc = exp(G_ic - G_jc):
//   M_ij = sum_c k_ic k_jc P_ijc (j < i),  R = Diag(beta) M,  T = (I + R)^-1
//   A_ij = scale sum_c q_ic k_jc P_ijc (j <= i)
//   K~ = exp(G) k,  Q~ = scale exp(G) q,  K^ = exp(G_63 - G) k,  gam = exp(G_63)
//   X = V - K~ S,  E = T Diag(beta) X,  O = Q~ S + A E,  S' = Diag(gam) S + K^' E.
// Given dO and dS' (the gradient of the chunk-end state), reverse mode gives
//   dE = A' dO + K^ dS',  dX = Diag(beta) T' dE = dV,
//   dS = Diag(gam) dS' + Q~' dO - K~' dX                      (to the chunk before)
//   dQ~ = dO S',  dK~ = -dX S',  dK^ = E dS'',  dgam_c = sum_v dS'_cv S_cv,
//   dA = dO E' (j <= i),  dT'' = dE X' (T'' = T Diag(beta)),
//   dT = dT'' Diag(beta),  dbeta_j += sum_i dT''_ij T_ij,
//   dR = -T' dT T' (j < i),  dbeta_i += sum_j dR_ij M_ij,  dM = Diag(beta) dR,
// and through M, A, K~, Q~, K^, gam to k, q and G; then dg = the reverse
// cumulative sum of dG inside the chunk, and for the Kaczmarz step size
// beta = eta / (|k|^2 + eps): deta = dbeta / (|k|^2 + eps),
// dk += -2 beta dbeta / (|k|^2 + eps) k.
//
// Five kernels:
//  * prep (one workgroup per chunk): G, beta, M, A and T (as the forward
//    vector intra kernel, with T itself instead of W and U);
//  * forward walk (one workgroup per (sequence, head, 32 value columns)): the
//    state entering every chunk, stored;
//  * reverse walk (same grid, chunks in reverse): dS' of every chunk, stored,
//    and the gradient of the initial state;
//  * grads A (one workgroup per chunk): the products over the value axis, in
//    slices of 16 columns: dV, and the parts of dq, dk, dG that come through
//    K~, Q~, K^ and gam; dA and dT'' to the workspace;
//  * grads B (one workgroup per chunk): the triangular algebra (dT, dR, dM,
//    dbeta), the pair terms of M and A, the Kaczmarz step, the reverse
//    cumulative sum; writes dq, dk, dg and dbeta.
// Padded rows of a partial last chunk have k = q = v = g = beta = 0 and
// dO = 0, so they contribute nothing.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int C = kChunk;
constexpr int kThreads = 256;
constexpr int kBV = 32;  // value columns per walk workgroup
constexpr int kBS = 16;  // value columns per slice of grads A

// ---- workspace, per chunk slot ci = (b H + h) NC + c
struct BwdWs {
    float *T, *A, *M, *G, *beta;   // C x C (three), C x GK, C
    float *S, *dS;                 // DK x DV: entering state; gradient of the chunk-end state
    float *dA, *dTT, *dG;          // C x C (two), C x GK
    float *dG63;                   // GK: the chunk-end decay's extra gradient (K^ and gam)
    float *Kt, *Kh, *Qt;           // C x DK each: K~, K^, Q~ (decayed operands, fp32)
};

template <int DK, int DV, bool PC>
BwdWs carve_bwd(void *ws, size_t slots) {
    constexpr int GK = PC ? DK : 1;
    float *p = static_cast<float *>(ws);
    BwdWs w;
    w.T = p; p += slots * C * C;
    w.A = p; p += slots * C * C;
    w.M = p; p += slots * C * C;
    w.G = p; p += slots * C * GK;
    w.beta = p; p += slots * C;
    w.S = p; p += slots * DK * DV;
    w.dS = p; p += slots * DK * DV;
    w.dA = p; p += slots * C * C;
    w.dTT = p; p += slots * C * C;
    w.dG = p; p += slots * C * GK;
    w.dG63 = p; p += slots * GK;
    w.Kt = p; p += slots * C * DK;
    w.Kh = p; p += slots * C * DK;
    w.Qt = p;
    return w;
}

template <int DK, int DV, bool PC>
size_t bwd_bytes(size_t slots) {
    constexpr int GK = PC ? DK : 1;
    return slots * sizeof(float) *
           ((size_t)5 * C * C + 2 * (size_t)C * GK + GK + C + 2 * (size_t)DK * DV + 3 * (size_t)C * DK);
}

// chunk slot ci -> (b, h, c), token row of its token 0, token count
struct Slot {
    int b, h, c, n;
    size_t row0;  // [B, T, H, .] row of token 0; token i is row0 + i H
};
__device__ __forceinline__ Slot slot_of(int ci, int T, int H, int NC) {
    Slot s;
    s.c = ci % NC;
    const int bh = ci / NC;
    s.b = bh / H;
    s.h = bh % H;
    s.n = min(C, T - s.c * C);
    s.row0 = ((size_t)s.b * T + (size_t)s.c * C) * H + s.h;
    return s;
}

// ============================================================ prep
template <int DK, bool PC, bool KZ, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const void *__restrict__ q, const void *__restrict__ k,
                                                            const float *__restrict__ g, const float *__restrict__ beta,
                                                            int T, int H, int NC, float eps, float scale,
                                                            float *__restrict__ wT, float *__restrict__ wA,
                                                            float *__restrict__ wM, float *__restrict__ wG,
                                                            float *__restrict__ wB, float *__restrict__ wKt,
                                                            float *__restrict__ wKh, float *__restrict__ wQt) {
    constexpr int GK = PC ? DK : 1;
    const int ci = blockIdx.x;
    const Slot sl = slot_of(ci, T, H, NC);
    const int n = sl.n;
    const int tid = threadIdx.x;
    __shared__ float sK[C][DK + 1];
    __shared__ float sQ[C][DK + 1];
    __shared__ float sG[C][GK];
    __shared__ __align__(16) float sR[C][C];
    __shared__ float sBeta[C];

    {  // all loads in flight at once, then the LDS stores
        constexpr int NE = C * DK / kThreads, NG = (C * GK + kThreads - 1) / kThreads;
        float kr[NE], qr[NE], gr[NG];
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int idx = tid + u * kThreads, i = idx / DK, cc = idx % DK;
            const size_t off = (sl.row0 + (size_t)i * H) * DK + cc;
            kr[u] = i < n ? load_in<IN_BF16>(k, off) : 0.f;
            qr[u] = i < n ? load_in<IN_BF16>(q, off) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int idx = tid + u * kThreads, i = idx / GK, cc = idx % GK;
            gr[u] = idx < C * GK && i < n ? g[(sl.row0 + (size_t)i * H) * GK + cc] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int idx = tid + u * kThreads;
            sK[idx / DK][idx % DK] = kr[u];
            sQ[idx / DK][idx % DK] = qr[u];
        }
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int idx = tid + u * kThreads;
            if (idx < C * GK) sG[idx / GK][idx % GK] = gr[u];
        }
    }
    __syncthreads();
    if (tid < GK) {  // in-chunk inclusive cumulative sum, one channel per thread
        float run = 0.f;
        for (int i = 0; i < C; ++i) {
            run += sG[i][tid];
            sG[i][tid] = run;
        }
    }
    if (tid >= kThreads - C) {
        const int i = tid - (kThreads - C);
        float bv = 0.f;
        if (i < n) {
            const float given = beta[sl.row0 + (size_t)i * H];
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

    float *Mg = wM + (size_t)ci * C * C, *Ag = wA + (size_t)ci * C * C;
    {  // M (strictly lower), A (lower): thread -> row i, 16 columns
        const int i = tid >> 2, jb = (tid & 3) * 16;
        for (int jj = 0; jj < 16; ++jj) {
            const int j = jb + jj;
            float r = 0.f, a = 0.f;
            if (j <= i) {
                for (int cc = 0; cc < DK; ++cc) {
                    const float p = PC ? __expf(sG[i][cc] - sG[j][cc]) : 1.f;
                    r += sK[i][cc] * sK[j][cc] * p;
                    a += sQ[i][cc] * sK[j][cc] * p;
                }
                if constexpr (!PC) {
                    const float p = __expf(sG[i][0] - sG[j][0]);
                    r *= p;
                    a *= p;
                }
            }
            const float m = j < i ? r : 0.f;
            Mg[i * C + j] = m;
            Ag[i * C + j] = j <= i ? scale * a : 0.f;
            sR[i][j] = sBeta[i] * m;
        }
    }
    __syncthreads();
    // T = (I + R)^-1, one column per thread: x_i = [i == col] - sum_{m<i} R_im x_m
    if (tid < C) {
        const int col = tid;
        float x[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float acc = i == col ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc -= sR[i][m] * x[m];
            x[i] = acc;
        }
        float *Tg = wT + (size_t)ci * C * C;
#pragma unroll
        for (int i = 0; i < C; ++i) Tg[i * C + col] = x[i];
    }
    for (int idx = tid; idx < C * GK; idx += kThreads) wG[(size_t)ci * C * GK + idx] = sG[idx / GK][idx % GK];
    if (tid < C) wB[(size_t)ci * C + tid] = sBeta[tid];
    // the decayed operands: K~ = exp(G) k, K^ = exp(G_63 - G) k, Q~ = scale exp(G) q
    for (int idx = tid; idx < C * DK; idx += kThreads) {
        const int i = idx / DK, cc = idx % DK;
        const float gi = PC ? sG[i][cc] : sG[i][0];
        const float ge = PC ? sG[C - 1][cc] : sG[C - 1][0];
        const float ei = __expf(gi);
        wKt[(size_t)ci * C * DK + idx] = ei * sK[i][cc];
        wKh[(size_t)ci * C * DK + idx] = __expf(ge - gi) * sK[i][cc];
        wQt[(size_t)ci * C * DK + idx] = scale * ei * sQ[i][cc];
    }
}

// decay factors of token i, channel cc from G in LDS
template <bool PC, int GK>
__device__ __forceinline__ float gval(const float (*sG)[GK], int i, int cc) {
    return PC ? sG[i][cc] : sG[i][0];
}

// ============================================================ forward walk: entering states
// Each chunk's operands (T, K~, K^, the v slice, beta, gam) are loaded into
// registers one chunk ahead and moved to LDS at the start of the chunk.
template <int DK, int DV, bool PC, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void bwd_states_kernel(const void *__restrict__ v, int T, int H, int NC,
                                                              const float *__restrict__ wT,
                                                              const float *__restrict__ wG,
                                                              const float *__restrict__ wB,
                                                              const float *__restrict__ wKt,
                                                              const float *__restrict__ wKh,
                                                              const float *__restrict__ s0, float *__restrict__ wS) {
    constexpr int GK = PC ? DK : 1;
    constexpr int NT = DV / kBV;
    constexpr int NTT = C * C / kThreads, NKK = C * DK / kThreads, NVV = C * kBV / kThreads;
    constexpr int RPW = kThreads / kBV;  // rows per pass of the workgroup
    const int tile = blockIdx.x % NT, bh = blockIdx.x / NT;
    const int b = bh / H, h = bh % H;
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, jj = tid % kBV, rr = tid / kBV;
    __shared__ float sS[DK][kBV];
    __shared__ float sKt[C][DK + 1];
    __shared__ float sKh[C][DK + 1];
    __shared__ float sX[C][kBV + 1];  // V, then X
    __shared__ float sE[C][kBV + 1];
    __shared__ float sT[C][C + 1];
    __shared__ float sBeta[C], sGam[DK];

    float rT[NTT], rKt[NKK], rKh[NKK], rV[NVV], rB = 0.f, rGam = 0.f;
    auto fetch = [&](int c) {
        const size_t ci = (size_t)bh * NC + c;
        const int n = min(C, T - c * C);
        const size_t row0 = ((size_t)b * T + (size_t)c * C) * H + h;
#pragma unroll
        for (int u = 0; u < NTT; ++u) rT[u] = wT[ci * C * C + tid + u * kThreads];
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            rKt[u] = wKt[ci * C * DK + tid + u * kThreads];
            rKh[u] = wKh[ci * C * DK + tid + u * kThreads];
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int idx = tid + u * kThreads, i = idx / kBV, cc = idx % kBV;
            rV[u] = i < n ? load_in<IN_BF16>(v, (row0 + (size_t)i * H) * DV + j0 + cc) : 0.f;
        }
        if (tid < C) rB = wB[ci * C + tid];
        if (tid < DK) rGam = __expf(wG[ci * C * GK + (size_t)(C - 1) * GK + (PC ? tid : 0)]);
    };

    const size_t sbase = (size_t)bh * DK * DV;
    for (int idx = tid; idx < DK * kBV; idx += kThreads) {
        const int r = idx / kBV, cc = idx % kBV;
        sS[r][cc] = s0 ? s0[sbase + (size_t)r * DV + j0 + cc] : 0.f;
    }
    if (NC > 0) fetch(0);
    for (int c = 0; c < NC; ++c) {
        const size_t ci = (size_t)bh * NC + c;
        __syncthreads();  // the previous chunk's reads are done
        float *Sg = wS + ci * DK * DV;
        for (int idx = tid; idx < DK * kBV; idx += kThreads) {
            const int r = idx / kBV, cc = idx % kBV;
            Sg[(size_t)r * DV + j0 + cc] = sS[r][cc];
        }
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            const int idx = tid + u * kThreads;
            sT[idx / C][idx % C] = rT[u];
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            const int idx = tid + u * kThreads;
            sKt[idx / DK][idx % DK] = rKt[u];
            sKh[idx / DK][idx % DK] = rKh[u];
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int idx = tid + u * kThreads;
            sX[idx / kBV][idx % kBV] = rV[u];
        }
        if (tid < C) sBeta[tid] = rB;
        if (tid < DK) sGam[tid] = rGam;
        if (c + 1 < NC) fetch(c + 1);
        __syncthreads();
        // X = V - K~ S (each thread its own entries of sX)
        for (int i = rr; i < C; i += RPW) {
            float acc = sX[i][jj];
            for (int cc = 0; cc < DK; ++cc) acc -= sKt[i][cc] * sS[cc][jj];
            sX[i][jj] = acc;
        }
        __syncthreads();
        for (int i = rr; i < C; i += RPW) {  // E = T Diag(beta) X
            float acc = 0.f;
            for (int m = 0; m <= i; ++m) acc += sT[i][m] * sBeta[m] * sX[m][jj];
            sE[i][jj] = acc;
        }
        __syncthreads();
        // S <- Diag(gam) S + K^' E (each thread its own entries)
        constexpr int PER = DK / RPW;
        float acc[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] = sGam[rr + p * RPW] * sS[rr + p * RPW][jj];
        for (int i = 0; i < C; ++i) {
            const float e = sE[i][jj];
#pragma unroll
            for (int p = 0; p < PER; ++p) acc[p] += sKh[i][rr + p * RPW] * e;
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) sS[rr + p * RPW][jj] = acc[p];
    }
}

// ============================================================ reverse walk: dS' per chunk
template <int DK, int DV, bool PC>
__global__ __launch_bounds__(kThreads) void bwd_dstates_kernel(const float *__restrict__ dO, int T, int H, int NC,
                                                               const float *__restrict__ wT,
                                                               const float *__restrict__ wA,
                                                               const float *__restrict__ wG,
                                                               const float *__restrict__ wB,
                                                               const float *__restrict__ wKt,
                                                               const float *__restrict__ wKh,
                                                               const float *__restrict__ wQt,
                                                               const float *__restrict__ ds_final,
                                                               float *__restrict__ wdS, float *__restrict__ ds0) {
    constexpr int GK = PC ? DK : 1;
    constexpr int NT = DV / kBV;
    constexpr int NTT = C * C / kThreads, NKK = C * DK / kThreads, NVV = C * kBV / kThreads;
    constexpr int RPW = kThreads / kBV;
    const int tile = blockIdx.x % NT, bh = blockIdx.x / NT;
    const int b = bh / H, h = bh % H;
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, jj = tid % kBV, rr = tid / kBV;
    __shared__ float sdS[DK][kBV];
    __shared__ float sK1[C][DK + 1];  // K^, then Q~
    __shared__ float sK2[C][DK + 1];  // K~
    __shared__ float sO[C][kBV + 1];  // dO slice
    __shared__ float sdE[C][kBV + 1];
    __shared__ float sdX[C][kBV + 1];
    __shared__ float sT[C][C + 1];
    __shared__ float sA[C][C + 1];
    __shared__ float sBeta[C], sGam[DK];

    float rT[NTT], rA[NTT], rKt[NKK], rKh[NKK], rQt[NKK], rO[NVV], rB = 0.f, rGam = 0.f;
    auto fetch = [&](int c) {
        const size_t ci = (size_t)bh * NC + c;
        const int n = min(C, T - c * C);
        const size_t row0 = ((size_t)b * T + (size_t)c * C) * H + h;
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            rT[u] = wT[ci * C * C + tid + u * kThreads];
            rA[u] = wA[ci * C * C + tid + u * kThreads];
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            rKt[u] = wKt[ci * C * DK + tid + u * kThreads];
            rKh[u] = wKh[ci * C * DK + tid + u * kThreads];
            rQt[u] = wQt[ci * C * DK + tid + u * kThreads];
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int idx = tid + u * kThreads, i = idx / kBV, cc = idx % kBV;
            rO[u] = i < n ? dO[(row0 + (size_t)i * H) * DV + j0 + cc] : 0.f;
        }
        if (tid < C) rB = wB[ci * C + tid];
        if (tid < DK) rGam = __expf(wG[ci * C * GK + (size_t)(C - 1) * GK + (PC ? tid : 0)]);
    };

    const size_t sbase = (size_t)bh * DK * DV;
    for (int idx = tid; idx < DK * kBV; idx += kThreads) {
        const int r = idx / kBV, cc = idx % kBV;
        sdS[r][cc] = ds_final ? ds_final[sbase + (size_t)r * DV + j0 + cc] : 0.f;
    }
    constexpr int PER = DK / RPW;  // dS entries per thread: rows rr + RPW p, column jj
    if (NC > 0) fetch(NC - 1);
    for (int c = NC - 1; c >= 0; --c) {
        const size_t ci = (size_t)bh * NC + c;
        __syncthreads();
        float *dSg = wdS + ci * DK * DV;
        for (int idx = tid; idx < DK * kBV; idx += kThreads) {
            const int r = idx / kBV, cc = idx % kBV;
            dSg[(size_t)r * DV + j0 + cc] = sdS[r][cc];
        }
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            const int idx = tid + u * kThreads;
            sT[idx / C][idx % C] = rT[u];
            sA[idx / C][idx % C] = rA[u];
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            const int idx = tid + u * kThreads;
            sK1[idx / DK][idx % DK] = rKh[u];
            sK2[idx / DK][idx % DK] = rKt[u];
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int idx = tid + u * kThreads;
            sO[idx / kBV][idx % kBV] = rO[u];
        }
        if (tid < C) sBeta[tid] = rB;
        if (tid < DK) sGam[tid] = rGam;
        __syncthreads();
        for (int i = rr; i < C; i += RPW) {  // dE = A' dO + K^ dS'
            float acc = 0.f;
            for (int m = i; m < C; ++m) acc += sA[m][i] * sO[m][jj];
            for (int cc = 0; cc < DK; ++cc) acc += sK1[i][cc] * sdS[cc][jj];
            sdE[i][jj] = acc;
        }
        __syncthreads();
        for (int i = rr; i < C; i += RPW) {  // dX = Diag(beta) T' dE
            float acc = 0.f;
            for (int m = i; m < C; ++m) acc += sT[m][i] * sdE[m][jj];
            sdX[i][jj] = sBeta[i] * acc;
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {  // K^ is no longer read: Q~ in its place
            const int idx = tid + u * kThreads;
            sK1[idx / DK][idx % DK] = rQt[u];
        }
        if (c > 0) fetch(c - 1);
        __syncthreads();
        // dS = Diag(gam) dS' - K~' dX + Q~' dO (each thread its own entries)
        float acc[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] = sGam[rr + p * RPW] * sdS[rr + p * RPW][jj];
        for (int i = 0; i < C; ++i) {
            const float x = sdX[i][jj], o = sO[i][jj];
#pragma unroll
            for (int p = 0; p < PER; ++p) acc[p] += sK1[i][rr + p * RPW] * o - sK2[i][rr + p * RPW] * x;
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) sdS[rr + p * RPW][jj] = acc[p];
    }
    __syncthreads();
    if (ds0) {
        for (int idx = tid; idx < DK * kBV; idx += kThreads) {
            const int r = idx / kBV, cc = idx % kBV;
            ds0[sbase + (size_t)r * DV + j0 + cc] = sdS[r][cc];
        }
    }
}

// ============================================================ grads A: products over the value axis
// Thread t owns row i = t / 4 of the C x DK accumulators (channels
// (t % 4) CPT .. +CPT) and of the C x C accumulators (columns (t % 4) 16 .. +16).
template <int DK, int DV, bool PC, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void bwd_grads_a_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v, const float *__restrict__ dO,
    int T, int H, int NC, float scale, const float *__restrict__ wT, const float *__restrict__ wA,
    const float *__restrict__ wG, const float *__restrict__ wB, const float *__restrict__ wS,
    const float *__restrict__ wdS, const float *__restrict__ wKt, const float *__restrict__ wKh,
    const float *__restrict__ wQt, float *__restrict__ wdA, float *__restrict__ wdTT, float *__restrict__ wdG,
    float *__restrict__ wdG63, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv) {
    constexpr int GK = PC ? DK : 1;
    constexpr int CPT = DK / 4;
    constexpr int NTT = C * C / kThreads, NKK = C * DK / kThreads;
    constexpr int NSS = DK * kBS / kThreads, NVS = C * kBS / kThreads;
    const int ci = blockIdx.x;
    const Slot sl = slot_of(ci, T, H, NC);
    const int n = sl.n;
    const int tid = threadIdx.x;
    const int i = tid >> 2, q4 = tid & 3;
    const int cb = q4 * CPT;
    __shared__ float sKt[C][DK + 1];     // K~
    __shared__ float sKh[C][DK + 1];     // K^
    __shared__ float sT[C][C + 1];
    __shared__ float sA[C][C + 1];
    __shared__ float sS[DK][kBS + 1];    // entering state, this slice
    __shared__ float sdS[DK][kBS + 1];   // dS', this slice
    __shared__ float sX[C][kBS + 1];     // V, then X
    __shared__ float sO[C][kBS + 1];     // dO
    __shared__ float sE[C][kBS + 1];
    __shared__ float sdE[C][kBS + 1];
    __shared__ float sdX[C][kBS + 1];
    __shared__ float sBeta[C];
    // G of token r, channel cc (from the workspace: LDS holds the slices)
    const float *Gc = wG + (size_t)ci * C * GK;
    auto gget = [&](int r, int cc) { return Gc[r * GK + (PC ? cc : 0)]; };

    {  // T, A, K~, K^: all loads in flight, then the LDS stores
        float rT[NTT], rA[NTT], rKt[NKK], rKh[NKK];
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            rT[u] = wT[(size_t)ci * C * C + tid + u * kThreads];
            rA[u] = wA[(size_t)ci * C * C + tid + u * kThreads];
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            rKt[u] = wKt[(size_t)ci * C * DK + tid + u * kThreads];
            rKh[u] = wKh[(size_t)ci * C * DK + tid + u * kThreads];
        }
        if (tid < C) sBeta[tid] = wB[(size_t)ci * C + tid];
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            const int idx = tid + u * kThreads;
            sT[idx / C][idx % C] = rT[u];
            sA[idx / C][idx % C] = rA[u];
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            const int idx = tid + u * kThreads;
            sKt[idx / DK][idx % DK] = rKt[u];
            sKh[idx / DK][idx % DK] = rKh[u];
        }
    }
    (void)k;
    (void)q;

    float dQt[CPT], dKt[CPT], dKh[CPT], dAa[16], dTa[16];
#pragma unroll
    for (int u = 0; u < CPT; ++u) dQt[u] = dKt[u] = dKh[u] = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) dAa[u] = dTa[u] = 0.f;
    float dgam = 0.f;  // channel tid (tid < DK)

    const float *Sg = wS + (size_t)ci * DK * DV;
    const float *dSg = wdS + (size_t)ci * DK * DV;
    const int oi = tid / 4, oj = (tid % 4) * 4;  // C x kBS products: row oi, columns oj .. oj+3
    // the slice's S, dS', v and dO, loaded into registers one slice ahead
    float rS[NSS], rdS[NSS], rV[NVS], rO[NVS];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NSS; ++u) {
            const int idx = tid + u * kThreads, r = idx / kBS, cc = idx % kBS;
            rS[u] = Sg[(size_t)r * DV + j0 + cc];
            rdS[u] = dSg[(size_t)r * DV + j0 + cc];
        }
#pragma unroll
        for (int u = 0; u < NVS; ++u) {
            const int idx = tid + u * kThreads, r = idx / kBS, cc = idx % kBS;
            const size_t row = sl.row0 + (size_t)r * H;
            rV[u] = r < n ? load_in<IN_BF16>(v, row * DV + j0 + cc) : 0.f;
            rO[u] = r < n ? dO[row * DV + j0 + cc] : 0.f;
        }
    };
    fetch(0);
    for (int j0 = 0; j0 < DV; j0 += kBS) {
        __syncthreads();  // the previous slice is no longer read
#pragma unroll
        for (int u = 0; u < NSS; ++u) {
            const int idx = tid + u * kThreads;
            sS[idx / kBS][idx % kBS] = rS[u];
            sdS[idx / kBS][idx % kBS] = rdS[u];
        }
#pragma unroll
        for (int u = 0; u < NVS; ++u) {
            const int idx = tid + u * kThreads;
            sX[idx / kBS][idx % kBS] = rV[u];
            sO[idx / kBS][idx % kBS] = rO[u];
        }
        if (j0 + kBS < DV) fetch(j0 + kBS);
        __syncthreads();
        {  // X = V - K~ S;  dE = A' dO + K^ dS'
            float x[4], de[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = sX[oi][oj + u];
                de[u] = 0.f;
            }
            for (int cc = 0; cc < DK; ++cc) {
                const float kt = sKt[oi][cc], kh = sKh[oi][cc];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    x[u] -= kt * sS[cc][oj + u];
                    de[u] += kh * sdS[cc][oj + u];
                }
            }
            for (int m = oi; m < C; ++m) {
                const float a = sA[m][oi];
#pragma unroll
                for (int u = 0; u < 4; ++u) de[u] += a * sO[m][oj + u];
            }
            __syncthreads();  // every thread has read V
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sX[oi][oj + u] = x[u];
                sdE[oi][oj + u] = de[u];
            }
        }
        __syncthreads();
        {  // E = T Diag(beta) X;  dX = Diag(beta) T' dE (= dV)
            float e[4] = {0.f, 0.f, 0.f, 0.f}, dx[4] = {0.f, 0.f, 0.f, 0.f};
            for (int m = 0; m <= oi; ++m) {
                const float t = sT[oi][m] * sBeta[m];
#pragma unroll
                for (int u = 0; u < 4; ++u) e[u] += t * sX[m][oj + u];
            }
            for (int m = oi; m < C; ++m) {
                const float t = sT[m][oi];
#pragma unroll
                for (int u = 0; u < 4; ++u) dx[u] += t * sdE[m][oj + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sE[oi][oj + u] = e[u];
                sdX[oi][oj + u] = sBeta[oi] * dx[u];
                if (oi < n) dv[(sl.row0 + (size_t)oi * H) * DV + j0 + oj + u] = sBeta[oi] * dx[u];
            }
        }
        __syncthreads();
        // accumulators of row i, one value column at a time
        for (int jj = 0; jj < kBS; ++jj) {
            const float o = sO[i][jj], x = sdX[i][jj], e = sE[i][jj], de = sdE[i][jj];
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const float sv = sS[cb + u][jj];
                dQt[u] += o * sv;
                dKt[u] -= x * sv;
                dKh[u] += e * sdS[cb + u][jj];
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int m = q4 * 16 + u;
                dAa[u] += o * sE[m][jj];
                dTa[u] += de * sX[m][jj];
            }
        }
        if (tid < DK) {
            float s = 0.f;
#pragma unroll
            for (int jj = 0; jj < kBS; ++jj) s += sdS[tid][jj] * sS[tid][jj];
            dgam += s;
        }
    }

    // dA, dT'' (lower triangle incl. the diagonal) to the workspace
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int m = q4 * 16 + u;
        wdA[(size_t)ci * C * C + i * C + m] = m <= i ? dAa[u] : 0.f;
        wdTT[(size_t)ci * C * C + i * C + m] = m <= i ? dTa[u] : 0.f;
    }
    // parts of dq, dk through Q~, K~, K^ (rows past the end are not written);
    // parts of dG: dK~ K~ + dQ~ Q~ - dK^ K^; for G_63 also sum_i dK^ K^ + dgam gam
    const bool valid = i < n;
    const size_t rowi = sl.row0 + (size_t)i * H;
    float gpart = 0.f;  // scalar decay: this thread's share of the sum over channels
    float hh[CPT];      // dK^ K^ of row i, channels cb ..
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int cc = cb + u;
        const float gi = gget(i, cc);
        const float ei = __expf(gi);
        const float qt = wQt[((size_t)ci * C + i) * DK + cc];  // Q~ (zero past the end)
        const float kt = sKt[i][cc], kh = sKh[i][cc];
        if (valid) {
            dq[rowi * DK + cc] = scale * ei * dQt[u];
            dk[rowi * DK + cc] = ei * dKt[u] + __expf(gget(C - 1, cc) - gi) * dKh[u];
        }
        const float part = dKt[u] * kt + dQt[u] * qt - dKh[u] * kh;
        hh[u] = dKh[u] * kh;
        if constexpr (PC) wdG[((size_t)ci * C + i) * GK + cc] = part;
        else gpart += part;
    }
    if constexpr (!PC) {  // the four threads of row i are adjacent lanes
        gpart += __shfl_xor(gpart, 1, 64);
        gpart += __shfl_xor(gpart, 2, 64);
        if (q4 == 0) wdG[(size_t)ci * C + i] = gpart;
    }
    // the chunk-end decay: per channel, the column sum of dK^ K^ (through LDS,
    // fixed order) plus dgam gam; summed over channels for scalar decay
    __syncthreads();  // sKt is no longer read
#pragma unroll
    for (int u = 0; u < CPT; ++u) sKt[i][cb + u] = hh[u];
    __syncthreads();
    if (tid < DK) {
        float s = 0.f;
        for (int r = 0; r < C; ++r) s += sKt[r][tid];
        sKh[0][tid] = s + dgam * __expf(gget(C - 1, tid));
    }
    __syncthreads();
    if constexpr (PC) {
        if (tid < DK) wdG63[(size_t)ci * GK + tid] = sKh[0][tid];
    } else {
        if (tid == 0) {
            float s = 0.f;
            for (int cc = 0; cc < DK; ++cc) s += sKh[0][cc];
            wdG63[ci] = s;
        }
    }
}

// ============================================================ grads B: triangular algebra and pair terms
template <int DK, bool PC, bool KZ, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void bwd_grads_b_kernel(
    const void *__restrict__ q, const void *__restrict__ k, int T, int H, int NC, float eps, float scale,
    const float *__restrict__ wT, const float *__restrict__ wM, const float *__restrict__ wG,
    const float *__restrict__ wB, const float *__restrict__ wdA, const float *__restrict__ wdTT,
    const float *__restrict__ wdG, const float *__restrict__ wdG63, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dg, float *__restrict__ dbeta) {
    constexpr int GK = PC ? DK : 1;
    constexpr int GROUPS = kThreads / DK;      // row groups per channel in the pair terms
    constexpr int RPT = C / GROUPS;            // rows per thread
    const int ci = blockIdx.x;
    const Slot sl = slot_of(ci, T, H, NC);
    const int n = sl.n;
    const int tid = threadIdx.x;
    // phase 1 buffers (C x C) and phase 2 buffers (C x DK) share the space
    __shared__ float smem[3 * C * (C + 1) > 2 * C * (DK + 1) ? 3 * C * (C + 1) : 2 * C * (DK + 1)];
    __shared__ float sD[C][C + 1];      // dA (j <= i) and, in the strict upper part, dM transposed
    __shared__ float sG[C][GK];
    __shared__ float sBeta[C], sdBeta[C], sKK[C];
    __shared__ float sdG[C][GK];

    float(*sT)[C + 1] = reinterpret_cast<float(*)[C + 1]>(smem);
    float(*sX)[C + 1] = reinterpret_cast<float(*)[C + 1]>(smem + C * (C + 1));       // dT, then dR
    float(*sY)[C + 1] = reinterpret_cast<float(*)[C + 1]>(smem + 2 * C * (C + 1));   // T' dT, then M
    const float *Tg = wT + (size_t)ci * C * C;
    const float *dAg = wdA + (size_t)ci * C * C, *dTg = wdTT + (size_t)ci * C * C;
    {  // all loads in flight, then the LDS stores
        constexpr int NTT = C * C / kThreads, NG = (C * GK + kThreads - 1) / kThreads;
        float rT[NTT], rD[NTT], rX[NTT], rG[NG], rdG[NG];
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            const int idx = tid + u * kThreads;
            rT[u] = Tg[idx];
            rD[u] = dAg[idx];
            rX[u] = dTg[idx];
        }
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int idx = tid + u * kThreads;
            rG[u] = idx < C * GK ? wG[(size_t)ci * C * GK + idx] : 0.f;
            rdG[u] = idx < C * GK ? wdG[(size_t)ci * C * GK + idx] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            const int idx = tid + u * kThreads, r = idx / C, cc = idx % C;
            sT[r][cc] = rT[u];
            sD[r][cc] = cc <= r ? rD[u] : 0.f;
            sX[r][cc] = cc <= r ? rX[u] : 0.f;  // dT''
        }
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int idx = tid + u * kThreads;
            if (idx < C * GK) {
                sG[idx / GK][idx % GK] = rG[u];
                sdG[idx / GK][idx % GK] = rdG[u];
            }
        }
    }
    if (tid < C) sBeta[tid] = wB[(size_t)ci * C + tid];
    __syncthreads();
    if (tid < GK) sdG[C - 1][tid] += wdG63[(size_t)ci * GK + tid];  // the chunk-end decay's extra
    // dbeta_j = sum_i dT''_ij T_ij; then dT = dT'' Diag(beta)
    if (tid < C) {
        const int j = tid;
        float s = 0.f;
        for (int r = j; r < C; ++r) s += sX[r][j] * sT[r][j];
        sdBeta[j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, cc = idx % C;
        sX[r][cc] *= sBeta[cc];
    }
    __syncthreads();
    // Y = T' dT:  Y_ab = sum_i T_ia dT_ib
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int a = idx / C, bb = idx % C;
        float s = 0.f;
        for (int r = max(a, bb); r < C; ++r) s += sT[r][a] * sX[r][bb];
        sY[a][bb] = s;
    }
    __syncthreads();
    // dR = -Y T' (strictly lower):  dR_ab = -sum_m Y_am T_bm
    float dr[C * C / kThreads];
#pragma unroll
    for (int u = 0; u < C * C / kThreads; ++u) {
        const int idx = tid + u * kThreads;
        const int a = idx / C, bb = idx % C;
        float s = 0.f;
        if (bb < a) {
            for (int m = 0; m <= bb; ++m) s += sY[a][m] * sT[bb][m];
        }
        dr[u] = -s;
    }
    __syncthreads();
    const float *Mg = wM + (size_t)ci * C * C;
#pragma unroll
    for (int u = 0; u < C * C / kThreads; ++u) {
        const int idx = tid + u * kThreads;
        sX[idx / C][idx % C] = dr[u];
        sY[idx / C][idx % C] = Mg[idx];
    }
    __syncthreads();
    // dbeta_i += sum_{j<i} dR_ij M_ij;  dM_ij = beta_i dR_ij -> sD[j][i] (j < i)
    if (tid < C) {
        const int r = tid;
        float s = 0.f;
        for (int cc = 0; cc < r; ++cc) s += sX[r][cc] * sY[r][cc];
        sdBeta[r] += s;
    }
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, cc = idx % C;
        if (cc < r) sD[cc][r] = sBeta[r] * sX[r][cc];
    }
    __syncthreads();

    // ---- phase 2: raw k, q in LDS; pair terms per (channel, row group)
    float(*sK)[DK + 1] = reinterpret_cast<float(*)[DK + 1]>(smem);
    float(*sQ)[DK + 1] = reinterpret_cast<float(*)[DK + 1]>(smem + C * (DK + 1));
    {
        constexpr int NKK = C * DK / kThreads;
        float rk[NKK], rq[NKK];
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            const int idx = tid + u * kThreads, r = idx / DK, cc = idx % DK;
            const size_t off = (sl.row0 + (size_t)r * H) * DK + cc;
            rk[u] = r < n ? load_in<IN_BF16>(k, off) : 0.f;
            rq[u] = r < n ? load_in<IN_BF16>(q, off) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            const int idx = tid + u * kThreads;
            sK[idx / DK][idx % DK] = rk[u];
            sQ[idx / DK][idx % DK] = rq[u];
        }
    }
    __syncthreads();
    if constexpr (KZ) {  // |k_i|^2
        if (tid < C) {
            float s = 0.f;
            for (int cc = 0; cc < DK; ++cc) s += sK[tid][cc] * sK[tid][cc];
            sKK[tid] = s;
        }
        __syncthreads();
    }
    const int cch = tid % DK, grp = tid / DK;
    float pk[RPT], pq[RPT], pg[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int r = grp + u * GROUPS;  // rows of this thread (interleaved: the triangle is balanced)
        const float gi = gval<PC, GK>(sG, r, cch);
        const float ki = sK[r][cch], qi = sQ[r][cch];
        float ak = 0.f, aq = 0.f, ag = 0.f;
        // as the row of M and A: j <= i
        for (int j = 0; j <= r; ++j) {
            const float p = __expf(gi - gval<PC, GK>(sG, j, cch));
            const float kj = sK[j][cch];
            const float a = j < r ? sD[j][r] : 0.f;  // dM_ij
            const float bq = scale * sD[r][j];       // scale dA_ij
            ak += a * kj * p;
            aq += bq * kj * p;
            ag += (a * ki + bq * qi) * kj * p;
        }
        // as the column of M and A: i >= j (here j = r)
        for (int i2 = r; i2 < C; ++i2) {
            const float p = __expf(gval<PC, GK>(sG, i2, cch) - gi);
            const float a = i2 > r ? sD[r][i2] : 0.f;  // dM_{i2, r}
            const float bq = scale * sD[i2][r];        // scale dA_{i2, r}
            const float w = (a * sK[i2][cch] + bq * sQ[i2][cch]) * p;
            ak += w;
            ag -= w * ki;
        }
        pk[u] = ak;
        pq[u] = aq;
        pg[u] = ag;
    }
    __syncthreads();  // sK, sQ are read below only at this thread's own entries
    if constexpr (PC) {  // dG per channel: each thread its own entries
#pragma unroll
        for (int u = 0; u < RPT; ++u) sdG[grp + u * GROUPS][cch] += pg[u];
    }
    // dq, dk: add the parts written by grads A; the Kaczmarz step size
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int r = grp + u * GROUPS;
        if (r < n) {
            const size_t off = (sl.row0 + (size_t)r * H) * DK + cch;
            float dkv = dk[off] + pk[u];
            if constexpr (KZ) dkv += -2.f * sBeta[r] * sdBeta[r] / (sKK[r] + eps) * sK[r][cch];
            dk[off] = dkv;
            dq[off] += pq[u];
        }
    }
    if constexpr (!PC) {
        // scalar decay: dG_i = sum over channels; pg to LDS (sK space is free now), summed per row
        __syncthreads();
#pragma unroll
        for (int u = 0; u < RPT; ++u) sK[grp + u * GROUPS][cch] = pg[u];
        __syncthreads();
        if (tid < C) {
            float s = 0.f;
            for (int cc = 0; cc < DK; ++cc) s += sK[tid][cc];
            sdG[tid][0] += s;
        }
    }
    __syncthreads();
    // dg = reverse cumulative sum of dG over the chunk's tokens; dbeta (deta)
    if (tid < GK) {
        float run = 0.f;
        for (int r = C - 1; r >= 0; --r) {
            run += sdG[r][tid];
            if (r < n) dg[(sl.row0 + (size_t)r * H) * GK + tid] = run;
        }
    }
    if (tid < C && tid < n) {
        float db = sdBeta[tid];
        if constexpr (KZ) db /= (sKK[tid] + eps);
        dbeta[sl.row0 + (size_t)tid * H] = db;
    }
}

// ============================================================ launch
template <int DK, int DV, bool PC, bool KZ, bool IB>
hipError_t launch_bwd_t(const BwdArgs &a) {
    const size_t slots = (size_t)a.B * a.H * a.NC;
    BwdWs w = carve_bwd<DK, DV, PC>(a.ws, slots);
    const unsigned nslot = (unsigned)slots;
    const unsigned nwalk = (unsigned)(a.B * a.H * (DV / kBV));
    hipLaunchKernelGGL((bwd_prep_kernel<DK, PC, KZ, IB>), dim3(nslot), dim3(kThreads), 0, a.stream, a.q, a.k, a.g,
                       a.beta, a.T, a.H, a.NC, a.eps, a.scale, w.T, w.A, w.M, w.G, w.beta, w.Kt, w.Kh, w.Qt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_states_kernel<DK, DV, PC, IB>), dim3(nwalk), dim3(kThreads), 0, a.stream, a.v, a.T, a.H,
                       a.NC, w.T, w.G, w.beta, w.Kt, w.Kh, a.s0, w.S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dstates_kernel<DK, DV, PC>), dim3(nwalk), dim3(kThreads), 0, a.stream, a.dO, a.T, a.H,
                       a.NC, w.T, w.A, w.G, w.beta, w.Kt, w.Kh, w.Qt, a.ds_final, w.dS, a.ds0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grads_a_kernel<DK, DV, PC, IB>), dim3(nslot), dim3(kThreads), 0, a.stream, a.q, a.k, a.v,
                       a.dO, a.T, a.H, a.NC, a.scale, w.T, w.A, w.G, w.beta, w.S, w.dS, w.Kt, w.Kh, w.Qt, w.dA,
                       w.dTT, w.dG, w.dG63, a.dq, a.dk, a.dv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grads_b_kernel<DK, PC, KZ, IB>), dim3(nslot), dim3(kThreads), 0, a.stream, a.q, a.k,
                       a.T, a.H, a.NC, a.eps, a.scale, w.T, w.M, w.G, w.beta, w.dA, w.dTT, w.dG, w.dG63, a.dq, a.dk,
                       a.dg, a.dbeta);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd_d(const BwdArgs &a) {
    const int key = (a.per_channel ? 4 : 0) | (a.kaczmarz ? 2 : 0) | (a.qkv_bf16 ? 1 : 0);
    switch (key) {
        case 0: return launch_bwd_t<DK, DV, false, false, false>(a);
        case 1: return launch_bwd_t<DK, DV, false, false, true>(a);
        case 2: return launch_bwd_t<DK, DV, false, true, false>(a);
        case 3: return launch_bwd_t<DK, DV, false, true, true>(a);
        case 4: return launch_bwd_t<DK, DV, true, false, false>(a);
        case 5: return launch_bwd_t<DK, DV, true, false, true>(a);
        case 6: return launch_bwd_t<DK, DV, true, true, false>(a);
        default: return launch_bwd_t<DK, DV, true, true, true>(a);
    }
}

}  // namespace

size_t chunk_bwd_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel) {
    const size_t slots = (size_t)B * H * NC;
    if (Dk == 128 && Dv == 128) return per_channel ? bwd_bytes<128, 128, true>(slots) : bwd_bytes<128, 128, false>(slots);
    if (Dk == 128 && Dv == 64) return per_channel ? bwd_bytes<128, 64, true>(slots) : bwd_bytes<128, 64, false>(slots);
    if (Dk == 64 && Dv == 128) return per_channel ? bwd_bytes<64, 128, true>(slots) : bwd_bytes<64, 128, false>(slots);
    return per_channel ? bwd_bytes<64, 64, true>(slots) : bwd_bytes<64, 64, false>(slots);
}

hipError_t launch_chunk_bwd(const BwdArgs &a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bwd_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bwd_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bwd_d<64, 128>(a);
    return launch_bwd_d<64, 64>(a);
}

}  // namespace gdr
