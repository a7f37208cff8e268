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
// The state-independent matrices (R, A, T, W, U) are recomputed by each
// slice's workgroup: matrix-core time traded for an HBM round trip of them.
//
// Layout.  v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] (e = 0..7) and D[4(l/16)+r][l%16] (r = 0..3).  A sum
// over tokens may take its 32 terms in any order shared by both operands;
// here the 8 terms of lane group p = l/16 within a 32-token block are tokens
// {4p..4p+3} and {16+4p..16+4p+3}, which is exactly what two stacked D tiles
// hold.  So a D tile is directly a token-reduction operand, and K^T, V^T
// (needed for W, U and the state update) are produced in registers by one
// MFMA against a 0/1 selector instead of transposed LDS writes.  W is formed
// as W^T = K^T T'^T, whose D layout lets it be stored token-major with 8-byte
// writes.  The off-diagonal 16x16 blocks of T use v_mfma_f32_16x16x4f32
// (fp32 operands, same D layout).  The next chunk's q, k, v, g and beta are
// loaded into registers while the current chunk is processed.
//
// Precision.  Products of two exact bf16 inputs accumulate in fp32.  Every
// fp32-derived operand (T', T'', S, E, A) is split into bf16 hi + lo and
// multiplied as hi*x + lo*x (hi*hi + hi*lo + lo*hi when both sides are
// split), which carries ~16 significant bits; W is stored as plain bf16.
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;      // 64 tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int kThreads = 256;
constexpr int LDQ = DK + 8;    // bf16 row stride of Q, K, W (token-major)
constexpr int LDV = 32 + 8;    // bf16 row stride of the value slice (token-major, 32 columns)
constexpr int LDE = C + 8;     // bf16 row stride of E^T (token index contiguous)
constexpr int LDF = C + 4;     // fp32 row stride of R, T, A
constexpr int LDS_ = DK + 8;   // bf16 row stride of S^T (d_k contiguous)

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x32 fragment of a bf16 matrix stored with the reduction index contiguous
// (rows r0 .. r0+15, reduction k0 .. k0+31, natural order).
__device__ __forceinline__ bf16x8 frag(const __bf16 *base, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// Token-reduction fragment (tokens 32kb .. 32kb+31 in the lane-group order
// above) of a bf16 matrix with the token index contiguous.
__device__ __forceinline__ bf16x8 frag_tok(const __bf16 *base, int ld, int r0, int kb, int lane) {
    const __bf16 *p = base + (r0 + (lane & 15)) * ld + 32 * kb + 4 * (lane >> 4);
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p + 16);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Same from an fp32 matrix, times an optional per-token scale, split into
// bf16 hi and lo parts.
__device__ __forceinline__ void frag_tok_split(const float *base, int ld, int r0, int kb, int lane,
                                               const float *tokscale, bf16x8 &hi, bf16x8 &lo) {
    const int off = 32 * kb + 4 * (lane >> 4);
    const float *p = base + (r0 + (lane & 15)) * ld + off;
    const float4 x0 = *reinterpret_cast<const float4 *>(p);
    const float4 x1 = *reinterpret_cast<const float4 *>(p + 16);
    float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (tokscale) {
        const float4 s0 = *reinterpret_cast<const float4 *>(tokscale + off);
        const float4 s1 = *reinterpret_cast<const float4 *>(tokscale + off + 16);
        x[0] *= s0.x; x[1] *= s0.y; x[2] *= s0.z; x[3] *= s0.w;
        x[4] *= s1.x; x[5] *= s1.y; x[6] *= s1.z; x[7] *= s1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
}

// Two stacked D tiles (tokens 32kb .. +15 and 32kb+16 .. +31) as one
// token-reduction operand in bf16.
__device__ __forceinline__ bf16x8 pack_tok(f32x4 t0, f32x4 t1) {
    return bf16x8{static_cast<__bf16>(t0[0]), static_cast<__bf16>(t0[1]), static_cast<__bf16>(t0[2]),
                  static_cast<__bf16>(t0[3]), static_cast<__bf16>(t1[0]), static_cast<__bf16>(t1[1]),
                  static_cast<__bf16>(t1[2]), static_cast<__bf16>(t1[3])};
}

// 0/1 selector: MFMA(X rows, selector(u)) = columns 16u .. 16u+15 of a
// 32-wide block of X, as a D tile (one column per lane, four consecutive
// rows).  Exact: bf16 values times 1 summed with zeros in fp32.
__device__ __forceinline__ bf16x8 selector(int u, int lane) {
    bf16x8 s;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        s[e] = static_cast<__bf16>((8 * (lane >> 4) + e) == ((lane & 15) + 16 * u) ? 1.0f : 0.0f);
    return s;
}

// Off-diagonal 16x16 block of the unit lower-triangular inverse, by one
// wavefront on fp32 MFMA:  T_IJ = -T_II * sum_{M=J}^{I-1} R_IM T_MJ.
// Reduction index k = 4 (lane/16) + s at step s, so the partial product P
// (a D tile) is the B operand of the second product without any exchange.
__device__ __forceinline__ void inverse_block(float *sT, const float *sR, int I, int J, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 P = {0.f, 0.f, 0.f, 0.f};
    for (int M = J; M < I; ++M) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            P = mma32(sR[(16 * I + lr) * LDF + 16 * M + 4 * lg + s], sT[(16 * M + 4 * lg + s) * LDF + 16 * J + lr], P);
    }
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) out = mma32(sT[(16 * I + lr) * LDF + 16 * I + 4 * lg + s], P[s], out);
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * lg + r) * LDF + 16 * J + lr] = -out[r];
}

// One thread's share of a chunk's inputs, loaded ahead of use.
struct Pref {
    uint4 q0, q1, q2, q3, k0, k1, k2, k3, v;
    float g, b;
};

__device__ __forceinline__ uint4 ld16(const __bf16 *p, bool ok) {
    return ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
}

// Piece `it` of the q/k tile is token (tid + 256 it) / 16, 16-byte segment tid % 16.
template <int BV>
__device__ __forceinline__ Pref load_chunk(const __bf16 *q, const __bf16 *k, const __bf16 *v, const float *g,
                                           const float *beta, int c, int T, int H, int b, int h, int j0, int tid) {
    constexpr int VSEG = BV / 8;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    const int seg = tid & 15, i0 = tid >> 4, lane = tid & 63;
    Pref p;
    const size_t o0 = (row0 + (size_t)(i0 + 0) * H) * DK + 8 * seg;
    const size_t o1 = (row0 + (size_t)(i0 + 16) * H) * DK + 8 * seg;
    const size_t o2 = (row0 + (size_t)(i0 + 32) * H) * DK + 8 * seg;
    const size_t o3 = (row0 + (size_t)(i0 + 48) * H) * DK + 8 * seg;
    p.q0 = ld16(q + o0, i0 < n);
    p.q1 = ld16(q + o1, i0 + 16 < n);
    p.q2 = ld16(q + o2, i0 + 32 < n);
    p.q3 = ld16(q + o3, i0 + 48 < n);
    p.k0 = ld16(k + o0, i0 < n);
    p.k1 = ld16(k + o1, i0 + 16 < n);
    p.k2 = ld16(k + o2, i0 + 32 < n);
    p.k3 = ld16(k + o3, i0 + 48 < n);
    const int vi = tid / VSEG, vs = tid % VSEG;
    p.v = ld16(v + (row0 + (size_t)vi * H) * DV + j0 + 8 * vs, tid < C * VSEG && vi < n);
    p.g = lane < n ? g[row0 + (size_t)lane * H] : 0.f;
    p.b = lane < n ? beta[row0 + (size_t)lane * H] : 0.f;
    return p;
}

__device__ __forceinline__ float sumsq8(uint4 x) {
    const __bf16 *e = reinterpret_cast<const __bf16 *>(&x);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += static_cast<float>(e[i]) * static_cast<float>(e[i]);
    return s;
}

template <int BV>
struct alignas(16) Smem {
    __bf16 Q[C * LDQ];            // q, token-major
    __bf16 KW[C * LDQ];           // k token-major; then W (bf16) token-major
    __bf16 V[C * LDV];            // v slice token-major (columns BV..31 stay zero)
    float A[C * LDF];             // causal read matrix
    float T[C * LDF];             // (I + R)^{-1}
    union {
        float R[C * LDF];         // strictly lower beta.decay-weighted K K^T
        __bf16 E[4][BV * LDE];    // E^T hi, lo and (Gend E)^T hi, lo
    } re;
    __bf16 ST[2][BV * LDS_];      // S^T hi, lo of the slice
    float cw[C];                  // beta_j exp(G_j): token scale of T for W
    float cb[C];                  // beta_j: token scale of T for U
    float kk[C];                  // ||k_j||^2 (Kaczmarz)
};

template <int BV, bool KZ, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void chunk_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ s0,
    void *__restrict__ o, float *__restrict__ s_final, int T, int H, int NC, int BH, float eps,
    float scale) {
    constexpr int NS = DV / BV;   // slices per (sequence, head)
    constexpr int NT = BV / 16;   // 16-column tiles per slice
    constexpr int VSEG = BV / 8;  // 16-byte segments per token row of the slice
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

    // Entries never written inside the chunk loop stay zero: the upper 16x16
    // tiles of A and T, and the value columns BV .. 31.
    for (int idx = tid; idx < C * LDF; idx += kThreads) {
        sm.A[idx] = 0.f;
        sm.T[idx] = 0.f;
    }
    for (int idx = tid; idx < C * LDV; idx += kThreads) sm.V[idx] = static_cast<__bf16>(0.f);

    // State slice in registers: wavefront w owns rows 32w + 16u + 4lg + r,
    // columns j0 + 16nt + lr.
    f32x4 S[2][NT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 32 * w + 16 * u + 4 * lg + r;
                S[u][nt][r] = s0 ? s0[sbase + (size_t)row * DV + j0 + 16 * nt + lr] : 0.f;
            }
    auto publish_state = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                bf16x4 hv, lv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hv[r] = static_cast<__bf16>(S[u][nt][r]);
                    lv[r] = static_cast<__bf16>(S[u][nt][r] - static_cast<float>(hv[r]));
                }
                const int off = (16 * nt + lr) * LDS_ + 32 * w + 16 * u + 4 * lg;
                *reinterpret_cast<bf16x4 *>(&sm.ST[0][off]) = hv;
                *reinterpret_cast<bf16x4 *>(&sm.ST[1][off]) = lv;
            }
    };
    publish_state();

    const bf16x8 sel0 = selector(0, lane), sel1 = selector(1, lane);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // Prefetch registers: this thread's 16-byte pieces of a chunk.
    Pref pf = load_chunk<BV>(q, k, v, g, beta, 0, T, H, b, h, j0, tid);
    __syncthreads();  // zero fills and the first state publication are visible

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * C;
        const int n = min(C, T - t0);
        const size_t row0 = ((size_t)b * T + t0) * H + h;

        // ---- stage the prefetched chunk; per-wavefront gates in registers
        {
            const int seg = tid & 15, i0 = tid >> 4;
            *reinterpret_cast<uint4 *>(&sm.Q[(i0 + 0) * LDQ + 8 * seg]) = pf.q0;
            *reinterpret_cast<uint4 *>(&sm.Q[(i0 + 16) * LDQ + 8 * seg]) = pf.q1;
            *reinterpret_cast<uint4 *>(&sm.Q[(i0 + 32) * LDQ + 8 * seg]) = pf.q2;
            *reinterpret_cast<uint4 *>(&sm.Q[(i0 + 48) * LDQ + 8 * seg]) = pf.q3;
            *reinterpret_cast<uint4 *>(&sm.KW[(i0 + 0) * LDQ + 8 * seg]) = pf.k0;
            *reinterpret_cast<uint4 *>(&sm.KW[(i0 + 16) * LDQ + 8 * seg]) = pf.k1;
            *reinterpret_cast<uint4 *>(&sm.KW[(i0 + 32) * LDQ + 8 * seg]) = pf.k2;
            *reinterpret_cast<uint4 *>(&sm.KW[(i0 + 48) * LDQ + 8 * seg]) = pf.k3;
            if (tid < C * VSEG) *reinterpret_cast<uint4 *>(&sm.V[(tid / VSEG) * LDV + 8 * (tid % VSEG)]) = pf.v;
            if constexpr (KZ) {
                float s2[4] = {sumsq8(pf.k0), sumsq8(pf.k1), sumsq8(pf.k2), sumsq8(pf.k3)};
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    s2[it] += __shfl_xor(s2[it], 1, 64);
                    s2[it] += __shfl_xor(s2[it], 2, 64);
                    s2[it] += __shfl_xor(s2[it], 4, 64);
                    s2[it] += __shfl_xor(s2[it], 8, 64);
                }
                if (seg == 0) {
                    sm.kk[i0 + 0] = s2[0];
                    sm.kk[i0 + 16] = s2[1];
                    sm.kk[i0 + 32] = s2[2];
                    sm.kk[i0 + 48] = s2[3];
                }
            }
        }
        // inclusive scan of the log-decays, lane = token (every wavefront)
        float Gl = pf.g;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(Gl, off, 64);
            if (lane >= off) Gl += up;
        }
        const float given = pf.b;
        if (c + 1 < NC) pf = load_chunk<BV>(q, k, v, g, beta, c + 1, T, H, b, h, j0, tid);
        __syncthreads();

        float Bl = given;  // beta of token `lane`
        if constexpr (KZ) Bl = lane < n ? given / (sm.kk[lane] + eps) : 0.f;
        if (w == 0) {
            sm.cw[lane] = Bl * __expf(Gl);
            sm.cb[lane] = Bl;
        }

        // ---- K K^T -> R (wavefronts 0, 1) and Q K^T -> A (2, 3), lower tiles;
        // even wavefronts take row blocks {0, 3}, odd ones {1, 2}: five each
        {
            const __bf16 *X = w >= 2 ? sm.Q : sm.KW;
            f32x4 acc[5];
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = zero4;
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
#pragma unroll
                for (int t = 0; t < 5; ++t) {
                    const int I = (w & 1) ? (t < 2 ? 1 : 2) : (t < 1 ? 0 : 3);
                    const int J = (w & 1) ? (t < 2 ? t : t - 2) : (t < 1 ? 0 : t - 1);
                    acc[t] = mma(frag(X, LDQ, 16 * I, 32 * kb, lane), frag(sm.KW, LDQ, 16 * J, 32 * kb, lane), acc[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < 5; ++t) {
                const int I = (w & 1) ? (t < 2 ? 1 : 2) : (t < 1 ? 0 : 3);
                const int J = (w & 1) ? (t < 2 ? t : t - 2) : (t < 1 ? 0 : t - 1);
                const int j = 16 * J + lr;
                const float gj = __shfl(Gl, j, 64);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * lg + r;
                    const float gi = __shfl(Gl, i, 64);
                    const float bi = __shfl(Bl, i, 64);
                    const float dec = j <= i ? __expf(gi - gj) : 0.f;
                    if (w >= 2) sm.A[i * LDF + j] = scale * dec * acc[t][r];
                    else sm.re.R[i * LDF + j] = j < i ? bi * dec * acc[t][r] : 0.f;
                }
            }
        }

        __syncthreads();

        // ---- T = (I + R)^{-1}: diagonal 16x16 blocks by forward substitution,
        // then three levels of off-diagonal blocks
        if (lane < 16) {
            const int cc = lane, base = 16 * w;
            float xcol[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float accv = i == cc ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) accv -= sm.re.R[(base + i) * LDF + base + m] * xcol[m];
                xcol[i] = i < cc ? 0.f : accv;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.T[(base + i) * LDF + base + cc] = xcol[i];
        }
        __syncthreads();
        if (w < 3) inverse_block(sm.T, sm.re.R, w + 1, w, lane);
        __syncthreads();
        if (w < 2) inverse_block(sm.T, sm.re.R, w + 2, w, lane);
        __syncthreads();
        if (w == 0) inverse_block(sm.T, sm.re.R, 3, 0, lane);
        __syncthreads();

        // ---- K^T (d_k tiles 2w, 2w+1) and V^T of the slice, in registers.  Wavefront
        // w reads exactly the K columns 32w .. 32w+31 that it overwrites with W below.
        bf16x8 KTf[2][2];  // [u][kb]: d_k rows 32w + 16u + lr, tokens of block kb
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 tr[4];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau)
                tr[tau] = mma(frag(sm.KW, LDQ, 16 * tau, 32 * w, lane), u ? sel1 : sel0, zero4);
            KTf[u][0] = pack_tok(tr[0], tr[1]);
            KTf[u][1] = pack_tok(tr[2], tr[3]);
        }
        bf16x8 VTf[NT][2];  // [nt][kb]: value columns 16nt + lr, tokens of block kb
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const f32x4 t0v = mma(frag(sm.V, LDV, 32 * kb, 0, lane), nt ? sel1 : sel0, zero4);
                const f32x4 t1v = mma(frag(sm.V, LDV, 32 * kb + 16, 0, lane), nt ? sel1 : sel0, zero4);
                VTf[nt][kb] = pack_tok(t0v, t1v);
            }

        // ---- W^T = K^T (T Diag(beta Gam))^T for d_k tiles 2w, 2w+1, stored
        // token-major; the wavefront's own rows of U = T Diag(beta) V
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 accw[2] = {zero4, zero4};
#pragma unroll
            for (int kb = 0; kb <= (I >> 1); ++kb) {
                bf16x8 thi, tlo;
                frag_tok_split(sm.T, LDF, 16 * I, kb, lane, sm.cw, thi, tlo);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    accw[u] = mma(KTf[u][kb], thi, accw[u]);
                    accw[u] = mma(KTf[u][kb], tlo, accw[u]);
                }
            }
            // lane holds W[token 16I + lr][d_k 32w + 16u + 4lg + r], r = 0..3
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x4 wv = {static_cast<__bf16>(accw[u][0]), static_cast<__bf16>(accw[u][1]),
                                   static_cast<__bf16>(accw[u][2]), static_cast<__bf16>(accw[u][3])};
                *reinterpret_cast<bf16x4 *>(&sm.KW[(16 * I + lr) * LDQ + 32 * w + 16 * u + 4 * lg]) = wv;
            }
        }
        f32x4 U[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) U[nt] = zero4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb > (w >> 1)) break;
            bf16x8 thi, tlo;
            frag_tok_split(sm.T, LDF, 16 * w, kb, lane, sm.cb, thi, tlo);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                U[nt] = mma(thi, VTf[nt][kb], U[nt]);
                U[nt] = mma(tlo, VTf[nt][kb], U[nt]);
            }
        }
        __syncthreads();

        // ---- E = U - W S and the read of the entering state, rows 16w..16w+15
        f32x4 P[NT], Oa[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            P[nt] = zero4;
            Oa[nt] = zero4;
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
        const float Gend = __shfl(Gl, C - 1, 64);
        float rowG[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rowG[r] = __shfl(Gl, 16 * w + 4 * lg + r, 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            bf16x4 eh, el, ph, pl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = U[nt][r] - P[nt][r];
                const float ep = e * __expf(Gend - rowG[r]);
                Oa[nt][r] *= scale * __expf(rowG[r]);
                eh[r] = static_cast<__bf16>(e);
                el[r] = static_cast<__bf16>(e - static_cast<float>(eh[r]));
                ph[r] = static_cast<__bf16>(ep);
                pl[r] = static_cast<__bf16>(ep - static_cast<float>(ph[r]));
            }
            const int off = (16 * nt + lr) * LDE + 16 * w + 4 * lg;
            *reinterpret_cast<bf16x4 *>(&sm.re.E[0][off]) = eh;
            *reinterpret_cast<bf16x4 *>(&sm.re.E[1][off]) = el;
            *reinterpret_cast<bf16x4 *>(&sm.re.E[2][off]) = ph;
            *reinterpret_cast<bf16x4 *>(&sm.re.E[3][off]) = pl;
        }
        __syncthreads();

        // ---- S <- gend S + K^T (Gend E), rows 32w .. 32w+31
        const float gscale = __expf(Gend);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 acc = S[u][nt] * gscale;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    acc = mma(KTf[u][kb], frag_tok(sm.re.E[2], LDE, 16 * nt, kb, lane), acc);
                    acc = mma(KTf[u][kb], frag_tok(sm.re.E[3], LDE, 16 * nt, kb, lane), acc);
                }
                S[u][nt] = acc;
            }

        // ---- O += A E (causal in-chunk reads), rows 16w .. 16w+15
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb > (w >> 1)) break;
            bf16x8 ahi, alo;
            frag_tok_split(sm.A, LDF, 16 * w, kb, lane, nullptr, ahi, alo);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 ehi = frag_tok(sm.re.E[0], LDE, 16 * nt, kb, lane);
                const bf16x8 elo = frag_tok(sm.re.E[1], LDE, 16 * nt, kb, lane);
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

        // every wavefront has read S^T (before the E barrier): publish the new state
        publish_state();
        __syncthreads();
    }

    if (s_final) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 32 * w + 16 * u + 4 * lg + r;
                    s_final[sbase + (size_t)row * DV + j0 + 16 * nt + lr] = S[u][nt][r];
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
