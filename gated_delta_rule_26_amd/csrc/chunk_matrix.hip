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
// Two kernels, as in the blog summary's "Pipeline Triton por chunks" (an
// intra-chunk kernel, then the state walk that also produces the outputs):
//  * intra: one workgroup per chunk, all chunks in parallel: gates, K K^T and
//    Q K^T on the lower 16x16 tiles, R, A and T = (I + R)^{-1}.  Writes to the
//    workspace, as bf16 hi + lo pairs of their lower 16x16 tiles, the three
//    operands the state walk needs -- T' = T Diag(beta Gam), T'' = T Diag(beta)
//    and A -- plus G (30 KiB per chunk).  Small LDS, so several workgroups
//    share a compute unit and hide each other's latencies.
//  * state: one 8-wavefront workgroup per (sequence, head, BV-column value
//    slice), chunks in order, the fp32 state slice in registers:
//    W^T = K^T T'^T, U = T'' V, E = U - W S, O and the state update.  Two
//    wavefronts per SIMD: one wavefront per SIMD reaches only about half of
//    the LDS read bandwidth (measured 134 vs 256 B/clk per CU).  Everything a
//    chunk needs from HBM is loaded into registers during the previous chunk.
//
// Layout.  v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] (e = 0..7) and D[4(l/16)+r][l%16] (r = 0..3).  A sum
// over tokens may take its 32 terms in any order shared by both operands;
// here the 8 terms of lane group p = l/16 within a 32-token block are tokens
// {4p..4p+3} and {16+4p..16+4p+3}, which is exactly what two stacked D tiles
// hold.  So a D tile is directly a token-reduction operand, and K^T, V^T are
// produced in registers by one MFMA against a 0/1 selector instead of
// transposed LDS writes.  W^T's D layout lets W be stored token-major with
// 8-byte writes.  The off-diagonal 16x16 blocks of T use
// v_mfma_f32_16x16x4f32 (fp32 operands, same D layout).
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



// Lower 16x16 tile t (0..9) of a 64x64 matrix: (0,0) (1,0) (1,1) (2,0) ...
__host__ __device__ constexpr int lower_I(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__host__ __device__ constexpr int lower_J(int t) { return t - lower_I(t) * (lower_I(t) + 1) / 2; }

// Per-chunk workspace record.  Six packed bf16 matrices (T' hi, T' lo,
// T'' hi, T'' lo, A hi, A lo), each as its ten lower 16x16 tiles, a tile
// row-major (512 B per tile, 5120 B per matrix), then G of the 64 tokens.
constexpr int kPackBytes = 10 * 256 * 2;
constexpr int kRecGOffsetFloats = 6 * kPackBytes / 4;
constexpr int kRecFloats = kRecGOffsetFloats + C;

// 16-byte piece p (0..319) of a packed matrix: tile t, row rr, half hf.
__device__ __forceinline__ void packed_piece(int p, int &row, int &col, int &byte_off) {
    const int t = p >> 5, rr = (p >> 1) & 15, hf = p & 1;
    row = 16 * lower_I(t) + rr;
    col = 16 * lower_J(t) + 8 * hf;
    byte_off = t * 512 + rr * 32 + hf * 16;
}

__device__ __forceinline__ uint4 ld16(const void *p, bool ok) {
    return ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ float sumsq8(uint4 x) {
    const __bf16 *e = reinterpret_cast<const __bf16 *>(&x);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += static_cast<float>(e[i]) * static_cast<float>(e[i]);
    return s;
}

// 8 fp32 values times 8 scales, split into bf16 hi and lo (16 bytes each).
__device__ __forceinline__ void split8(const float *x, const float *sc, uint4 &hi, uint4 &lo) {
    __bf16 h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float y = sc ? x[e] * sc[e] : x[e];
        h[e] = static_cast<__bf16>(y);
        l[e] = static_cast<__bf16>(y - static_cast<float>(h[e]));
    }
    hi = *reinterpret_cast<const uint4 *>(h);
    lo = *reinterpret_cast<const uint4 *>(l);
}

// ============================================================ intra kernel
constexpr int kIntraThreads = 256;

struct alignas(16) IntraSmem {
    union {
        __bf16 Q[C * LDQ];        // q token-major ...
        float T[C * LDF];         // ... then (I + R)^{-1}
    } qt;
    union {
        __bf16 K[C * LDQ];        // k token-major ...
        float A[C * LDF];         // ... then the causal read matrix
    } ka;
    float R[C * LDF];
    float kk[C];
    float cw[C];                  // beta_j exp(G_j)
    float cb[C];                  // beta_j
};

template <bool KZ>
__global__ __launch_bounds__(kIntraThreads) void intra_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, int T, int H, int NC, float eps, float scale, float *__restrict__ ws) {
    __shared__ IntraSmem sm;
    const int ci = blockIdx.x;  // (b*H + h)*NC + c
    const int c = ci % NC;
    const int bh = ci / NC;
    const int b = bh / H, h = bh % H;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    float *rec = ws + (size_t)ci * kRecFloats;
    char *recb = reinterpret_cast<char *>(rec);

    // ---- stage q, k token-major; gates of token `lane` in every wavefront
    {
        const int seg = tid & 15, i0 = tid >> 4;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = i0 + 16 * it;
            const size_t off = (row0 + (size_t)i * H) * DK + 8 * seg;
            const uint4 qv = ld16(q + off, i < n);
            const uint4 kv = ld16(k + off, i < n);
            *reinterpret_cast<uint4 *>(&sm.qt.Q[i * LDQ + 8 * seg]) = qv;
            *reinterpret_cast<uint4 *>(&sm.ka.K[i * LDQ + 8 * seg]) = kv;
            if constexpr (KZ) {
                float s2 = sumsq8(kv);
                s2 += __shfl_xor(s2, 1, 64);
                s2 += __shfl_xor(s2, 2, 64);
                s2 += __shfl_xor(s2, 4, 64);
                s2 += __shfl_xor(s2, 8, 64);
                if (seg == 0) sm.kk[i] = s2;
            }
        }
    }
    float Gl = lane < n ? g[row0 + (size_t)lane * H] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_up(Gl, off, 64);
        if (lane >= off) Gl += up;
    }
    const float given = lane < n ? beta[row0 + (size_t)lane * H] : 0.f;
    __syncthreads();
    float Bl = given;
    if constexpr (KZ) Bl = lane < n ? given / (sm.kk[lane] + eps) : 0.f;
    if (w == 0) {
        rec[kRecGOffsetFloats + lane] = Gl;
        sm.cw[lane] = Bl * __expf(Gl);
        sm.cb[lane] = Bl;
    }

    // ---- K K^T -> R (wavefronts 0, 1) and Q K^T (2, 3) on the lower tiles:
    // even wavefronts take row blocks {0, 3}, odd ones {1, 2}
    f32x4 acc[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const __bf16 *X = w >= 2 ? sm.qt.Q : sm.ka.K;
        const int Ia = (w & 1) ? 1 : 0, Ib = (w & 1) ? 2 : 3;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            const bf16x8 xa = frag(X, LDQ, 16 * Ia, 32 * kb, lane);
            const bf16x8 xb = frag(X, LDQ, 16 * Ib, 32 * kb, lane);
            const bf16x8 k0 = frag(sm.ka.K, LDQ, 0, 32 * kb, lane);
            const bf16x8 k1 = frag(sm.ka.K, LDQ, 16, 32 * kb, lane);
            const bf16x8 k2 = frag(sm.ka.K, LDQ, 32, 32 * kb, lane);
            if (w & 1) {  // tiles (1,0) (1,1) (2,0) (2,1) (2,2)
                acc[0] = mma(xa, k0, acc[0]);
                acc[1] = mma(xa, k1, acc[1]);
                acc[2] = mma(xb, k0, acc[2]);
                acc[3] = mma(xb, k1, acc[3]);
                acc[4] = mma(xb, k2, acc[4]);
            } else {      // tiles (0,0) (3,0) (3,1) (3,2) (3,3)
                const bf16x8 k3 = frag(sm.ka.K, LDQ, 48, 32 * kb, lane);
                acc[0] = mma(xa, k0, acc[0]);
                acc[1] = mma(xb, k0, acc[1]);
                acc[2] = mma(xb, k1, acc[2]);
                acc[3] = mma(xb, k2, acc[3]);
                acc[4] = mma(xb, k3, acc[4]);
            }
        }
    }
    // decay (and beta for R) applied in fp32; R to LDS now, A after the barrier
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
            const float dec = j <= i ? __expf(gi - gj) : 0.f;
            if (w >= 2) {
                acc[t][r] = scale * dec * acc[t][r];
            } else {
                const float bi = __shfl(Bl, i, 64);
                sm.R[i * LDF + j] = j < i ? bi * dec * acc[t][r] : 0.f;
            }
        }
    }
    __syncthreads();  // R complete; q and k no longer read: their space now holds T and A

    if (w >= 2) {
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            const int I = (w & 1) ? (t < 2 ? 1 : 2) : (t < 1 ? 0 : 3);
            const int J = (w & 1) ? (t < 2 ? t : t - 2) : (t < 1 ? 0 : t - 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.ka.A[(16 * I + 4 * lg + r) * LDF + 16 * J + lr] = acc[t][r];
        }
    }

    // ---- T = (I + R)^{-1}: diagonal 16x16 blocks by forward substitution,
    // then three levels of off-diagonal blocks on fp32 MFMA
    if (lane < 16) {
        const int cc = lane, base = 16 * w;
        float xcol[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float accv = i == cc ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) accv -= sm.R[(base + i) * LDF + base + m] * xcol[m];
            xcol[i] = i < cc ? 0.f : accv;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.qt.T[(base + i) * LDF + base + cc] = xcol[i];
    }
    __syncthreads();
    if (w < 3) inverse_block(sm.qt.T, sm.R, w + 1, w, lane);
    __syncthreads();
    if (w < 2) inverse_block(sm.qt.T, sm.R, w + 2, w, lane);
    __syncthreads();
    if (w == 0) inverse_block(sm.qt.T, sm.R, 3, 0, lane);
    __syncthreads();

    // ---- packed bf16 hi/lo operands: T' = T Diag(cw), T'' = T Diag(cb), A
    for (int u = tid; u < 640; u += kIntraThreads) {
        const int p = u < 320 ? u : u - 320;
        int row, col, boff;
        packed_piece(p, row, col, boff);
        uint4 hi, lo;
        if (u < 320) {
            const float *x = &sm.qt.T[row * LDF + col];
            split8(x, &sm.cw[col], hi, lo);
            *reinterpret_cast<uint4 *>(recb + 0 * kPackBytes + boff) = hi;
            *reinterpret_cast<uint4 *>(recb + 1 * kPackBytes + boff) = lo;
            split8(x, &sm.cb[col], hi, lo);
            *reinterpret_cast<uint4 *>(recb + 2 * kPackBytes + boff) = hi;
            *reinterpret_cast<uint4 *>(recb + 3 * kPackBytes + boff) = lo;
        } else {
            split8(&sm.ka.A[row * LDF + col], nullptr, hi, lo);
            *reinterpret_cast<uint4 *>(recb + 4 * kPackBytes + boff) = hi;
            *reinterpret_cast<uint4 *>(recb + 5 * kPackBytes + boff) = lo;
        }
    }
}

// ============================================================ state kernel
constexpr int kStateThreads = 512;  // 8 wavefronts

template <int BV>
struct alignas(16) StateSmem {
    __bf16 Q[C * LDQ];            // q, token-major
    __bf16 K[C * LDQ];            // k, token-major
    __bf16 W[C * LDQ];            // W (bf16), token-major
    __bf16 V[C * LDV];            // v slice token-major (columns BV..31 stay zero)
    __bf16 P6[6][C * LDE];        // T' hi, lo; T'' hi, lo; A hi, lo (upper tiles stay zero)
    __bf16 E[4][BV * LDE];        // E^T hi, lo and (Gend E)^T hi, lo
    __bf16 ST[2][BV * LDS_];      // S^T hi, lo of the slice
};

// This thread's share of a chunk's state-kernel inputs, loaded ahead of use.
struct StatePref {
    uint4 q0, q1, k0, k1, v, p0, p1, p2, p3;
    float g;
};

template <int BV>
__device__ __forceinline__ StatePref load_state_chunk(const __bf16 *q, const __bf16 *k, const __bf16 *v,
                                                      const float *ws, int c, int T, int H, int NC, int b,
                                                      int h, int bh, int j0, int tid) {
    constexpr int VSEG = BV / 8;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    const int seg = tid & 15, i0 = tid >> 4;  // i0 < 32
    const float *rec = ws + ((size_t)bh * NC + c) * kRecFloats;
    const char *recb = reinterpret_cast<const char *>(rec);
    StatePref p;
    const size_t o0 = (row0 + (size_t)i0 * H) * DK + 8 * seg;
    const size_t o1 = (row0 + (size_t)(i0 + 32) * H) * DK + 8 * seg;
    p.q0 = ld16(q + o0, i0 < n);
    p.q1 = ld16(q + o1, i0 + 32 < n);
    p.k0 = ld16(k + o0, i0 < n);
    p.k1 = ld16(k + o1, i0 + 32 < n);
    const int vi = tid / VSEG, vs = tid % VSEG;
    p.v = ld16(v + (row0 + (size_t)vi * H) * DV + j0 + 8 * vs, tid < C * VSEG && vi < n);
    // packed pieces tid + 512 m of the six matrices (1920 pieces)
    {
        int row, col, boff;
        const int m0 = tid, m1 = tid + 512, m2 = tid + 1024, m3 = tid + 1536;
        packed_piece(m0 % 320, row, col, boff);
        p.p0 = *reinterpret_cast<const uint4 *>(recb + (m0 / 320) * kPackBytes + boff);
        packed_piece(m1 % 320, row, col, boff);
        p.p1 = *reinterpret_cast<const uint4 *>(recb + (m1 / 320) * kPackBytes + boff);
        packed_piece(m2 % 320, row, col, boff);
        p.p2 = *reinterpret_cast<const uint4 *>(recb + (m2 / 320) * kPackBytes + boff);
        if (m3 < 1920) {
            packed_piece(m3 % 320, row, col, boff);
            p.p3 = *reinterpret_cast<const uint4 *>(recb + (m3 / 320) * kPackBytes + boff);
        } else {
            p.p3 = make_uint4(0, 0, 0, 0);
        }
    }
    p.g = rec[kRecGOffsetFloats + (tid & 63)];
    return p;
}

template <int BV>
__device__ __forceinline__ void stage_packed(StateSmem<BV> &sm, int m, uint4 val) {
    int row, col, boff;
    packed_piece(m % 320, row, col, boff);
    *reinterpret_cast<uint4 *>(&sm.P6[m / 320][row * LDE + col]) = val;
}

template <int BV, bool OUT_BF16>
__global__ __launch_bounds__(kStateThreads) void state_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ ws, const float *__restrict__ s0, void *__restrict__ o,
    float *__restrict__ s_final, int T, int H, int NC, int BH, float scale) {
    constexpr int NS = DV / BV;   // slices per (sequence, head)
    constexpr int NT = BV / 16;   // 16-column tiles per slice
    constexpr int VSEG = BV / 8;  // 16-byte segments per token row of the slice
    __shared__ StateSmem<BV> sm;

    // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
    // the slices of one (sequence, head) get ids that are equal modulo 8 and
    // share that XCD's L2 for q, k, v and the chunk records.
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
    const int lane = tid & 63, w = tid >> 6;  // w = 0..7
    const int lr = lane & 15, lg = lane >> 4;
    const int M = w >> 1, mt = w & 1;        // (token tile, value tile) of this wavefront
    const bool has_mt = mt < NT;

    // Never written inside the chunk loop, so they stay zero: the upper tiles
    // of the packed operands and the value columns BV .. 31.
    for (int idx = tid; idx < 6 * C * LDE; idx += kStateThreads) (&sm.P6[0][0])[idx] = static_cast<__bf16>(0.f);
    for (int idx = tid; idx < C * LDV; idx += kStateThreads) sm.V[idx] = static_cast<__bf16>(0.f);

    // State slice in registers: wavefront w owns rows 16w + 4lg + r (d_k
    // tile w), columns j0 + 16nt + lr.
    f32x4 S[NT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * w + 4 * lg + r;
            S[nt][r] = s0 ? s0[sbase + (size_t)row * DV + j0 + 16 * nt + lr] : 0.f;
        }
    auto publish_state = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            bf16x4 hv, lv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hv[r] = static_cast<__bf16>(S[nt][r]);
                lv[r] = static_cast<__bf16>(S[nt][r] - static_cast<float>(hv[r]));
            }
            const int off = (16 * nt + lr) * LDS_ + 16 * w + 4 * lg;
            *reinterpret_cast<bf16x4 *>(&sm.ST[0][off]) = hv;
            *reinterpret_cast<bf16x4 *>(&sm.ST[1][off]) = lv;
        }
    };

    const bf16x8 sel0 = selector(0, lane), sel1 = selector(1, lane);
    const bf16x8 selw = (w & 1) ? sel1 : sel0;   // K^T: d_k columns 16w .. 16w+15
    const bf16x8 selv = mt ? sel1 : sel0;        // V^T: value columns 16mt .. 16mt+15
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    StatePref pf = load_state_chunk<BV>(q, k, v, ws, 0, T, H, NC, b, h, bh, j0, tid);
    __syncthreads();  // zero fills done before the first staging writes
    publish_state();

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * C;
        const int n = min(C, T - t0);
        const size_t row0 = ((size_t)b * T + t0) * H + h;

        // ---- stage this chunk from the prefetch registers
        {
            const int seg = tid & 15, i0 = tid >> 4;
            *reinterpret_cast<uint4 *>(&sm.Q[i0 * LDQ + 8 * seg]) = pf.q0;
            *reinterpret_cast<uint4 *>(&sm.Q[(i0 + 32) * LDQ + 8 * seg]) = pf.q1;
            *reinterpret_cast<uint4 *>(&sm.K[i0 * LDQ + 8 * seg]) = pf.k0;
            *reinterpret_cast<uint4 *>(&sm.K[(i0 + 32) * LDQ + 8 * seg]) = pf.k1;
            if (tid < C * VSEG) *reinterpret_cast<uint4 *>(&sm.V[(tid / VSEG) * LDV + 8 * (tid % VSEG)]) = pf.v;
            stage_packed(sm, tid, pf.p0);
            stage_packed(sm, tid + 512, pf.p1);
            stage_packed(sm, tid + 1024, pf.p2);
            if (tid + 1536 < 1920) stage_packed(sm, tid + 1536, pf.p3);
        }
        const float Gl = pf.g;  // G of token `lane`
        __syncthreads();

        // ---- next chunk's inputs: loads in flight until the next staging
        if (c + 1 < NC) pf = load_state_chunk<BV>(q, k, v, ws, c + 1, T, H, NC, b, h, bh, j0, tid);

        // ---- K^T of d_k tile w (both token blocks) and V^T of value tile mt
        bf16x8 KTf[2];
        {
            f32x4 tr[4];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) tr[tau] = mma(frag(sm.K, LDQ, 16 * tau, 32 * (w >> 1), lane), selw, zero4);
            KTf[0] = pack_tok(tr[0], tr[1]);
            KTf[1] = pack_tok(tr[2], tr[3]);
        }
        // ---- W^T = K^T T'^T for d_k tile w (all token tiles), stored token-major
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 aw = zero4;
#pragma unroll
            for (int kb = 0; kb <= (I >> 1); ++kb) {
                aw = mma(KTf[kb], frag_tok(sm.P6[0], LDE, 16 * I, kb, lane), aw);
                aw = mma(KTf[kb], frag_tok(sm.P6[1], LDE, 16 * I, kb, lane), aw);
            }
            const bf16x4 wv = {static_cast<__bf16>(aw[0]), static_cast<__bf16>(aw[1]),
                               static_cast<__bf16>(aw[2]), static_cast<__bf16>(aw[3])};
            *reinterpret_cast<bf16x4 *>(&sm.W[(16 * I + lr) * LDQ + 16 * w + 4 * lg]) = wv;
        }
        // ---- U = T'' V for (token tile M, value tile mt)
        f32x4 U = zero4;
        if (has_mt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb > (M >> 1)) break;
                const f32x4 t0v = mma(frag(sm.V, LDV, 32 * kb, 0, lane), selv, zero4);
                const f32x4 t1v = mma(frag(sm.V, LDV, 32 * kb + 16, 0, lane), selv, zero4);
                const bf16x8 vt = pack_tok(t0v, t1v);
                U = mma(frag_tok(sm.P6[2], LDE, 16 * M, kb, lane), vt, U);
                U = mma(frag_tok(sm.P6[3], LDE, 16 * M, kb, lane), vt, U);
            }
        }
        __syncthreads();

        // ---- E = U - W S and the read of the entering state, (M, mt)
        f32x4 Oa = zero4;
        const float Gend = __shfl(Gl, C - 1, 64);
        if (has_mt) {
            f32x4 P = zero4;
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const bf16x8 aw = frag(sm.W, LDQ, 16 * M, 32 * kb, lane);
                const bf16x8 aq = frag(sm.Q, LDQ, 16 * M, 32 * kb, lane);
                const bf16x8 shi = frag(sm.ST[0], LDS_, 16 * mt, 32 * kb, lane);
                const bf16x8 slo = frag(sm.ST[1], LDS_, 16 * mt, 32 * kb, lane);
                P = mma(aw, shi, P);
                P = mma(aw, slo, P);
                Oa = mma(aq, shi, Oa);
                Oa = mma(aq, slo, Oa);
            }
            bf16x4 eh, el, ph, pl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gi = __shfl(Gl, 16 * M + 4 * lg + r, 64);
                const float e = U[r] - P[r];
                const float ep = e * __expf(Gend - gi);
                Oa[r] *= scale * __expf(gi);
                eh[r] = static_cast<__bf16>(e);
                el[r] = static_cast<__bf16>(e - static_cast<float>(eh[r]));
                ph[r] = static_cast<__bf16>(ep);
                pl[r] = static_cast<__bf16>(ep - static_cast<float>(ph[r]));
            }
            const int off = (16 * mt + lr) * LDE + 16 * M + 4 * lg;
            *reinterpret_cast<bf16x4 *>(&sm.E[0][off]) = eh;
            *reinterpret_cast<bf16x4 *>(&sm.E[1][off]) = el;
            *reinterpret_cast<bf16x4 *>(&sm.E[2][off]) = ph;
            *reinterpret_cast<bf16x4 *>(&sm.E[3][off]) = pl;
        }
        __syncthreads();

        // ---- S <- gend S + K^T (Gend E), d_k tile w
        const float gscale = __expf(Gend);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = S[nt] * gscale;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                acc = mma(KTf[kb], frag_tok(sm.E[2], LDE, 16 * nt, kb, lane), acc);
                acc = mma(KTf[kb], frag_tok(sm.E[3], LDE, 16 * nt, kb, lane), acc);
            }
            S[nt] = acc;
        }

        // ---- O += A E (causal in-chunk reads), (M, mt)
        if (has_mt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb > (M >> 1)) break;
                const bf16x8 ahi = frag_tok(sm.P6[4], LDE, 16 * M, kb, lane);
                const bf16x8 alo = frag_tok(sm.P6[5], LDE, 16 * M, kb, lane);
                const bf16x8 ehi = frag_tok(sm.E[0], LDE, 16 * mt, kb, lane);
                const bf16x8 elo = frag_tok(sm.E[1], LDE, 16 * mt, kb, lane);
                Oa = mma(ahi, ehi, Oa);
                Oa = mma(ahi, elo, Oa);
                Oa = mma(alo, ehi, Oa);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * M + 4 * lg + r;
                if (i < n) store_out<OUT_BF16>(o, (row0 + (size_t)i * H) * DV + j0 + 16 * mt + lr, Oa[r]);
            }
        }

        // every wavefront has read S^T (before the E barrier): publish the new state
        publish_state();
        __syncthreads();
    }

    if (s_final) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * w + 4 * lg + r;
                s_final[sbase + (size_t)row * DV + j0 + 16 * nt + lr] = S[nt][r];
            }
    }
}

// ============================================================ launchers
template <bool KZ>
hipError_t launch_intra(const ChunkArgs &a) {
    const unsigned grid = (unsigned)((size_t)a.B * a.H * a.NC);
    hipLaunchKernelGGL((intra_matrix_kernel<KZ>), dim3(grid), dim3(kIntraThreads), 0, a.stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), a.g, a.beta, a.T, a.H,
                       a.NC, a.eps, a.scale, static_cast<float *>(a.ws));
    return hipGetLastError();
}

template <int BV, bool OB>
hipError_t launch_state(const ChunkArgs &a) {
    const int BH = a.B * a.H;
    const unsigned grid = (unsigned)(BH * (DV / BV));
    hipLaunchKernelGGL((state_matrix_kernel<BV, OB>), dim3(grid), dim3(kStateThreads), 0, a.stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.v), static_cast<const float *>(a.ws), a.s0, a.o, a.s_final,
                       a.T, a.H, a.NC, BH, a.scale);
    return hipGetLastError();
}

}  // namespace

size_t chunk_matrix_workspace_bytes(int B, int H, int NC, int, int, bool) {
    return (size_t)B * H * NC * kRecFloats * sizeof(float);
}

bool chunk_matrix_supported(int Dk, int Dv, bool qkv_bf16, bool per_channel) {
    return qkv_bf16 && Dk == DK && Dv == DV && !per_channel;
}

// Slice width of the state kernel: 32 value columns when that already gives
// one workgroup per compute unit, else 16 (twice the workgroups).
hipError_t launch_chunk_matrix(const ChunkArgs &a, int stage) {
    if (stage != 1) {
        const hipError_t e = a.kaczmarz ? launch_intra<true>(a) : launch_intra<false>(a);
        if (e != hipSuccess || stage == 0) return e;
    }
    const bool wide = (long)a.B * a.H * (DV / 32) >= 256;
    if (wide) return a.o_bf16 ? launch_state<32, true>(a) : launch_state<32, false>(a);
    return a.o_bf16 ? launch_state<16, true>(a) : launch_state<16, false>(a);
}

}  // namespace gdr
