// Chunked forward pass on the matrix cores (bf16 MFMA, fp32 accumulation),
// bf16 q/k/v, d_k = d_v = 128, scalar (per token and head) decay.
//
// Algebra (blog summary on the DeltaNet family, "KDA por chunks", written
// for the d_k x d_v state; G_i is the in-chunk inclusive cumulative log-decay,
// Gam_i = exp(G_i), gend = exp(G_63), Gend_i = exp(G_63 - G_i)):
//   R_ij = beta_i exp(G_i - G_j) (K K^T)_ij          j < i   (strictly lower)
//   A_ij = scale exp(G_i - G_j) (Q K^T)_ij           j <= i  (read after write)
//   T    = (I + R)^{-1}                               unit lower triangular
//   W    = T Diag(beta Gam) K,   U = T Diag(beta) V   (WY-like form of the writes)
//   E    = U - W S                                    corrected writes
//   O    = scale Diag(Gam) Q S + A E                  outputs of the chunk
//   S   <- gend S + K^T Diag(Gend) E                  chunk-end state
// Padded rows of a partial last chunk are zero (k = q = v = g = beta = 0).
//
// One workgroup (4 wavefronts) owns one (sequence, head, BV-column slice of
// the value axis) and walks the chunks in order; there is no workspace and no
// second kernel, so q, k, v are read from HBM once and o is written once.
// The per-chunk matrices that do not depend on the state (R, A, T, W, U) are
// recomputed by each slice's workgroup: that costs matrix-core time but
// saves a round trip of W, U and A through HBM.
//
// Precision.  Products of two exact bf16 inputs (K K^T, Q K^T, W = T'K with K
// exact, U = T''V, Q S with S split, K^T E' with E' split) accumulate in fp32.
// Every fp32-derived operand (T', T'', S, E, A) is split into bf16 hi + lo
// and multiplied as hi*x + lo*x (and hi*hi + hi*lo + lo*hi when both sides
// are split), which carries ~16 significant bits; W is stored as plain bf16.
// The triangular inverse is fp32 on the vector ALUs: the four 16x16 diagonal
// blocks by forward substitution, then the off-diagonal blocks by
// T_IJ = -T_II sum_{J<=M<I} R_IM T_MJ, one block level at a time.
//
// MFMA used: v_mfma_f32_16x16x32_bf16 with lane l holding A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] (e = 0..7) and D[4(l/16)+r][l%16] (r = 0..3).  Every
// operand sits in LDS with its reduction index contiguous, so each fragment is
// one 16-byte LDS read.
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;      // 64 tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int kThreads = 256;
constexpr int LDQ = DK + 8;    // bf16 row stride of Q, K, W (token-major)
constexpr int LDT = C + 8;     // bf16 row stride of K^T, V^T, E^T (token index contiguous)
constexpr int LDF = C + 4;     // fp32 row stride of R, T, A
constexpr int LDS_ = DK + 8;   // bf16 row stride of S^T (d_k contiguous)

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x32 fragment of a bf16 matrix stored row-major with the reduction index
// contiguous: rows r0 .. r0+15, reduction k0 .. k0+31.
__device__ __forceinline__ bf16x8 frag(const __bf16 *base, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// Same from an fp32 matrix, each element multiplied by colscale[k], split
// into bf16 hi and lo parts.
__device__ __forceinline__ void frag_split(const float *base, int ld, int r0, int k0, int lane,
                                           const float *colscale, bf16x8 &hi, bf16x8 &lo) {
    const float *p = base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
    const float4 x0 = *reinterpret_cast<const float4 *>(p);
    const float4 x1 = *reinterpret_cast<const float4 *>(p + 4);
    float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (colscale) {
        const float *cs = colscale + k0 + 8 * (lane >> 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= cs[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Off-diagonal block of the unit lower-triangular inverse, by one wavefront:
// T_IJ = -T_II * sum_{M=J}^{I-1} R_IM T_MJ  (16x16 fp32 blocks in LDS).
__device__ void inverse_block(float *sT, const float *sR, float *scratch, int I, int J, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    for (int M = J; M < I; ++M) {
#pragma unroll 4
        for (int mm = 0; mm < 16; ++mm) {
            const float t = sT[(16 * M + mm) * LDF + 16 * J + lr];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] += sR[(16 * I + 4 * lg + r) * LDF + 16 * M + mm] * t;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) scratch[(4 * lg + r) * 16 + lr] = p[r];
    wave_lds_sync();
    float out[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int mm = 0; mm < 16; ++mm) {
        const float pv = scratch[mm * 16 + lr];
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] -= sT[(16 * I + 4 * lg + r) * LDF + 16 * I + mm] * pv;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * lg + r) * LDF + 16 * J + lr] = out[r];
}

template <int BV>
struct alignas(16) Smem {
    __bf16 Q[C * LDQ];            // q, token-major
    __bf16 KW[C * LDQ];           // k token-major; then W (bf16) token-major
    __bf16 KT[DK * LDT];          // k^T: d_k-major, token contiguous
    __bf16 VT[BV * LDT];          // v^T of the slice
    float A[C * LDF];             // causal read matrix (fp32)
    float T[C * LDF];             // (I + R)^{-1} (fp32)
    union {
        float R[C * LDF];         // strictly lower beta.decay-weighted K K^T (fp32)
        __bf16 E[4][BV * LDT];    // E^T hi, lo and (Gend E)^T hi, lo
    } re;
    __bf16 ST[2][BV * LDS_];      // S^T hi, lo of the slice
    float G[C];                   // in-chunk cumulative log-decay
    float beta[C];
    float cw[C];                  // beta_j exp(G_j): column scale of T for W
    float scratch[4][256];        // per-wavefront 16x16 scratch of the inverse
};

template <int BV, bool KZ, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void chunk_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ s0,
    void *__restrict__ o, float *__restrict__ s_final, int T, int H, int NC, int BH, float eps,
    float scale) {
    constexpr int NS = DV / BV;   // slices per (sequence, head)
    constexpr int NT = BV / 16;   // 16-column tiles per slice
    __shared__ Smem<BV> sm;

    // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
    // the slices of one (sequence, head) get ids that are equal modulo 8 and
    // share that XCD's L2 for q, k and v.
    const int x = blockIdx.x;
    int bh, slice;
    if ((BH & 7) == 0) {
        const int xcd = x & 7, r = x >> 3;
        bh = (r / NS) * 8 + xcd;
        slice = r % NS;
    } else {
        bh = x / NS;
        slice = x % NS;
    }
    const int b = bh / H, h = bh % H;
    const int j0 = slice * BV;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // State slice in registers: wavefront w owns rows 32w + 16m + 4lg + r,
    // columns j0 + 16nt + lr.
    f32x4 S[2][NT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 32 * w + 16 * m + 4 * lg + r;
                S[m][nt][r] = s0 ? s0[sbase + (size_t)row * DV + j0 + 16 * nt + lr] : 0.f;
            }

    auto write_state_lds = [&]() {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                __bf16 hv[4], lv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hv[r] = static_cast<__bf16>(S[m][nt][r]);
                    lv[r] = static_cast<__bf16>(S[m][nt][r] - static_cast<float>(hv[r]));
                }
                const int col = 16 * nt + lr, row = 32 * w + 16 * m + 4 * lg;
                __bf16 *ph = &sm.ST[0][col * LDS_ + row];
                __bf16 *pl = &sm.ST[1][col * LDS_ + row];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ph[r] = hv[r];
                    pl[r] = lv[r];
                }
            }
    };
    write_state_lds();

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * C;
        const int n = min(C, T - t0);
        const size_t row0 = ((size_t)b * T + t0) * H + h;  // (b, t0, h) token-head row

        // ---- stage the chunk: q, k token-major, k^T, v^T of the slice, gates
        for (int idx = tid; idx < C * (DK / 8); idx += kThreads) {
            const int i = idx >> 4, seg = idx & 15;
            uint4 qv = make_uint4(0, 0, 0, 0), kv = qv;
            if (i < n) {
                const size_t off = (row0 + (size_t)i * H) * DK + 8 * seg;
                qv = *reinterpret_cast<const uint4 *>(q + off);
                kv = *reinterpret_cast<const uint4 *>(k + off);
            }
            *reinterpret_cast<uint4 *>(&sm.Q[i * LDQ + 8 * seg]) = qv;
            *reinterpret_cast<uint4 *>(&sm.KW[i * LDQ + 8 * seg]) = kv;
            const __bf16 *ke = reinterpret_cast<const __bf16 *>(&kv);
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.KT[(8 * seg + e) * LDT + i] = ke[e];
        }
        for (int idx = tid; idx < C * (BV / 8); idx += kThreads) {
            const int i = idx / (BV / 8), seg = idx % (BV / 8);
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (i < n) vv = *reinterpret_cast<const uint4 *>(v + (row0 + (size_t)i * H) * DV + j0 + 8 * seg);
            const __bf16 *ve = reinterpret_cast<const __bf16 *>(&vv);
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.VT[(8 * seg + e) * LDT + i] = ve[e];
        }
        if (tid < C) {
            const bool ok = tid < n;
            sm.G[tid] = ok ? g[row0 + (size_t)tid * H] : 0.f;
            sm.beta[tid] = ok ? beta[row0 + (size_t)tid * H] : 0.f;
        }
        __syncthreads();

        // ---- gates: cumulative log-decay (wavefront 0), Kaczmarz beta
        if (w == 0) {
            float gv = sm.G[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gv, off, 64);
                if (lane >= off) gv += up;
            }
            sm.G[lane] = gv;
        }
        if constexpr (KZ) {
            const int i = tid >> 2, part = tid & 3;
            float kk = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float kvf = static_cast<float>(sm.KW[i * LDQ + 32 * part + e]);
                kk += kvf * kvf;
            }
            kk += __shfl_xor(kk, 1, 64);
            kk += __shfl_xor(kk, 2, 64);
            if (part == 0) sm.beta[i] = i < n ? sm.beta[i] / (kk + eps) : 0.f;
        }
        __syncthreads();
        if (tid < C) sm.cw[tid] = sm.beta[tid] * __expf(sm.G[tid]);

        // ---- K K^T -> R and Q K^T -> A on the lower 16x16 tiles; zero the
        // upper tiles of A and T (their fragments are read below)
        for (int job = w; job < 32; job += 4) {
            if (job < 20) {
                const bool isA = job >= 10;
                const int t = isA ? job - 10 : job;
                // lower tiles (I, J), J <= I, in the order (0,0) (1,0) (1,1) (2,0) ...
                const int I = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
                const int J = t - (I * (I + 1)) / 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const bf16x8 a = frag(isA ? sm.Q : sm.KW, LDQ, 16 * I, 32 * kb, lane);
                    const bf16x8 bb = frag(sm.KW, LDQ, 16 * J, 32 * kb, lane);
                    acc = mma(a, bb, acc);
                }
                const int j = 16 * J + lr;
                const float gj = sm.G[j];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * lg + r;
                    const float dec = j <= i ? __expf(sm.G[i] - gj) : 0.f;
                    if (isA) sm.A[i * LDF + j] = scale * dec * acc[r];
                    else sm.re.R[i * LDF + j] = j < i ? sm.beta[i] * dec * acc[r] : 0.f;
                }
            } else if (job < 26) {
                const int t = job - 20;  // upper tiles (I, J), J > I
                const int I = t < 3 ? 0 : t < 5 ? 1 : 2;
                const int J = I + 1 + (t < 3 ? t : t < 5 ? t - 3 : 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * lg + r, j = 16 * J + lr;
                    sm.A[i * LDF + j] = 0.f;
                    sm.T[i * LDF + j] = 0.f;
                }
            }
        }
        __syncthreads();

        // ---- T = (I + R)^{-1}: diagonal blocks by forward substitution
        if (lane < 16) {
            const int cc = lane, base = 16 * w;
            float xcol[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = i == cc ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc -= sm.re.R[(base + i) * LDF + base + m] * xcol[m];
                xcol[i] = i < cc ? 0.f : acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.T[(base + i) * LDF + base + cc] = xcol[i];
        }
        __syncthreads();
        if (w < 3) inverse_block(sm.T, sm.re.R, sm.scratch[w], w + 1, w, lane);
        __syncthreads();
        if (w < 2) inverse_block(sm.T, sm.re.R, sm.scratch[w], w + 2, w, lane);
        __syncthreads();
        if (w == 0) inverse_block(sm.T, sm.re.R, sm.scratch[0], 3, 0, lane);
        __syncthreads();

        // ---- W = T Diag(beta Gam) K (wavefront w: d_k tiles 2w, 2w+1) and the
        // wavefront's own rows of U = T Diag(beta) V
        f32x4 U[NT];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 accw[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kb = 0; kb <= (I >> 1); ++kb) {
                bf16x8 ahi, alo;
                frag_split(sm.T, LDF, 16 * I, 32 * kb, lane, sm.cw, ahi, alo);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const bf16x8 bk = frag(sm.KT, LDT, 16 * (2 * w + u), 32 * kb, lane);
                    accw[u] = mma(ahi, bk, accw[u]);
                    accw[u] = mma(alo, bk, accw[u]);
                }
            }
            // K (token-major) was last read before the inverse: W may overwrite it
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.KW[(16 * I + 4 * lg + r) * LDQ + 16 * (2 * w + u) + lr] = static_cast<__bf16>(accw[u][r]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) U[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb > (w >> 1)) break;
            bf16x8 ahi, alo;
            frag_split(sm.T, LDF, 16 * w, 32 * kb, lane, sm.beta, ahi, alo);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 bv = frag(sm.VT, LDT, 16 * nt, 32 * kb, lane);
                U[nt] = mma(ahi, bv, U[nt]);
                U[nt] = mma(alo, bv, U[nt]);
            }
        }
        __syncthreads();

        // ---- E = U - W S and the read of the entering state, rows 16w..16w+15
        f32x4 P[NT], Oa[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            P[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            Oa[nt] = P[nt];
        }
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            const bf16x8 aw = frag(sm.KW, LDQ, 16 * w, 32 * kb, lane);
            const bf16x8 aq = frag(sm.Q, LDQ, 16 * w, 32 * kb, lane);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 shi = frag(sm.ST[0], LDS_, 16 * nt, 32 * kb, lane);
                const bf16x8 slo = frag(sm.ST[1], LDS_, 16 * nt, 32 * kb, lane);
                P[nt] = mma(aw, shi, P[nt]);
                P[nt] = mma(aw, slo, P[nt]);
                Oa[nt] = mma(aq, shi, Oa[nt]);
                Oa[nt] = mma(aq, slo, Oa[nt]);
            }
        }
        const float gend = sm.G[C - 1];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            __bf16 eh[4], el[4], ph[4], pl[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r;
                const float e = U[nt][r] - P[nt][r];
                const float ep = e * __expf(gend - sm.G[i]);
                Oa[nt][r] *= scale * __expf(sm.G[i]);
                eh[r] = static_cast<__bf16>(e);
                el[r] = static_cast<__bf16>(e - static_cast<float>(eh[r]));
                ph[r] = static_cast<__bf16>(ep);
                pl[r] = static_cast<__bf16>(ep - static_cast<float>(ph[r]));
            }
            const int off = (16 * nt + lr) * LDT + 16 * w + 4 * lg;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sm.re.E[0][off + r] = eh[r];
                sm.re.E[1][off + r] = el[r];
                sm.re.E[2][off + r] = ph[r];
                sm.re.E[3][off + r] = pl[r];
            }
        }
        __syncthreads();

        // ---- S <- gend S + K^T (Gend E), rows 32w .. 32w+31
        const float gscale = __expf(gend);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 acc = S[m][nt] * gscale;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 ak = frag(sm.KT, LDT, 32 * w + 16 * m, 32 * kb, lane);
                    acc = mma(ak, frag(sm.re.E[2], LDT, 16 * nt, 32 * kb, lane), acc);
                    acc = mma(ak, frag(sm.re.E[3], LDT, 16 * nt, 32 * kb, lane), acc);
                }
                S[m][nt] = acc;
            }

        // ---- O += A E (causal in-chunk reads), rows 16w .. 16w+15
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb > (w >> 1)) break;
            bf16x8 ahi, alo;
            frag_split(sm.A, LDF, 16 * w, 32 * kb, lane, nullptr, ahi, alo);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 ehi = frag(sm.re.E[0], LDT, 16 * nt, 32 * kb, lane);
                const bf16x8 elo = frag(sm.re.E[1], LDT, 16 * nt, 32 * kb, lane);
                Oa[nt] = mma(ahi, ehi, Oa[nt]);
                Oa[nt] = mma(ahi, elo, Oa[nt]);
                Oa[nt] = mma(alo, ehi, Oa[nt]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r;
                if (i < n) store_out<OUT_BF16>(o, (row0 + (size_t)i * H) * DV + j0 + 16 * nt + lr, Oa[nt][r]);
            }

        // every wavefront has read S^T (above, before the E barrier): publish the new state
        write_state_lds();
        __syncthreads();
    }

    if (s_final) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 32 * w + 16 * m + 4 * lg + r;
                    s_final[sbase + (size_t)row * DV + j0 + 16 * nt + lr] = S[m][nt][r];
                }
    }
}

template <int BV, bool KZ, bool OB>
hipError_t launch_t(const ChunkArgs &a) {
    const int BH = a.B * a.H;
    const unsigned grid = (unsigned)(BH * (DV / BV));
    hipLaunchKernelGGL((chunk_matrix_kernel<BV, KZ, OB>), dim3(grid), dim3(kThreads), 0, a.stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.v), a.g, a.beta, a.s0, a.o, a.s_final, a.T, a.H, a.NC,
                       BH, a.eps, a.scale);
    return hipGetLastError();
}

template <int BV>
hipError_t launch_bv(const ChunkArgs &a) {
    const int key = (a.kaczmarz ? 2 : 0) | (a.o_bf16 ? 1 : 0);
    switch (key) {
        case 0: return launch_t<BV, false, false>(a);
        case 1: return launch_t<BV, false, true>(a);
        case 2: return launch_t<BV, true, false>(a);
        default: return launch_t<BV, true, true>(a);
    }
}

}  // namespace

size_t chunk_matrix_workspace_bytes(int, int, int, int, int, bool) { return 0; }

bool chunk_matrix_supported(int Dk, int Dv, bool qkv_bf16, bool per_channel) {
    return qkv_bf16 && Dk == DK && Dv == DV && !per_channel;
}

// Slice width: 32 value columns when that already gives one workgroup per
// compute unit, else 16 (twice the workgroups, less reuse of q/k per slice).
hipError_t launch_chunk_matrix(const ChunkArgs &a, int stage) {
    if (stage == 0) return hipSuccess;  // single fused kernel: everything runs in the state stage
    const long wg32 = (long)a.B * a.H * (DV / 32);
    if (wg32 >= 256) return launch_bv<32>(a);
    return launch_bv<16>(a);
}

}  // namespace gdr
