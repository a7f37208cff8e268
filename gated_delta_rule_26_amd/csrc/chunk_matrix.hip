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
// W is never formed: E = U - W S = T'' (V - Diag(Gam) K S) with
// T'' = T Diag(beta), so the walk multiplies K by the state (the same work as
// W S) and applies the 64 x 64 triangle T'' to the 64 x 16 result.
//
// Two kernels, as in the blog summary's "Pipeline Triton por chunks" (an
// intra-chunk kernel, then the state walk that also produces the outputs):
//  * intra: one workgroup per chunk, all chunks in parallel: gates, K K^T and
//    Q K^T on the lower 16x16 tiles, R, A and T = (I + R)^{-1}.  Writes T'' and
//    A, each split into bf16 hi + lo and laid out as the exact MFMA operand
//    fragments the walk loads (one 16-byte load per lane per fragment), and G.
//  * state: one workgroup per (sequence, head, 32 value columns), chunks in
//    order.  Two "chain" wavefronts each own the fp32 state of 16 value
//    columns in registers and do the dependent work of a chunk:
//    P = K S, X = V - Gam P, E = T'' X, S <- gend S + K^T (Gend E).  Their
//    operands stay in registers from one product to the next (see Layout),
//    so a chunk needs no exchange between chain wavefronts.  They also form
//    the read Q S, which shares the state operand with K S.  Two "helper"
//    wavefronts stage the next chunk's q, k, v and decays in LDS and, one
//    chunk behind, finish the outputs O = scale Gam (Q S) + A E from the
//    chain's Q S and E, passed through LDS.  One barrier per chunk; every LDS
//    buffer that crosses it is doubled.
//
// Layout.  v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] (e = 0..7) and D[4(l/16)+r][l%16] (r = 0..3).  A
// reduction may take its 32 terms (per 32-block) in any order shared by
// both operands; here the 8 terms of lane group p = l/16 are indices
// {4p..4p+3} and {16+4p..16+4p+3} of the block, which is exactly what two
// stacked D tiles hold.  So a D tile (the state, X, E) is directly the B
// operand of the next product, and the other operand (k, k^T, T'', A, q) is
// stored or loaded in that permuted order.  The off-diagonal 16x16 blocks of
// T use v_mfma_f32_16x16x4f32 (fp32 operands, same D layout).
//
// Precision.  Products of two exact bf16 inputs accumulate in fp32.  Every
// fp32-derived operand (T'', A, S, X, E) is split into bf16 hi + lo and
// multiplied as hi*x + lo*x (hi*hi + hi*lo + lo*hi when both sides are
// split), which carries ~16 significant bits.
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;      // 64 tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Index, inside a 32-block, of term e (0..7) of lane group p (0..3).
__host__ __device__ constexpr int kperm(int p, int e) { return e < 4 ? 4 * p + e : 12 + 4 * p + e; }

// Two stacked D tiles (block rows 0..15 and 16..31) as one permuted operand,
// split into bf16 hi and lo.
__device__ __forceinline__ void pair_split(f32x4 t0, f32x4 t1, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        hi[r] = static_cast<__bf16>(t0[r]);
        lo[r] = static_cast<__bf16>(t0[r] - static_cast<float>(hi[r]));
        hi[4 + r] = static_cast<__bf16>(t1[r]);
        lo[4 + r] = static_cast<__bf16>(t1[r] - static_cast<float>(hi[4 + r]));
    }
}

// ---- per-chunk workspace record
// T'' hi, T'' lo, A hi, A lo: each the six 16x32 operand fragments (M, kb) of
// its lower triangle -- (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), rows 16M ..
// 16M+15, tokens 32kb .. 32kb+31 in the permuted order -- as 64 lanes x
// 16 bytes; then, for the 64 tokens, Gam = exp(G) and Gend = exp(G_63 - G)
// (fp32), so the walk needs no exponentials.
constexpr int kFragBytes = 64 * 16;
constexpr int kRecTH = 0;
constexpr int kRecTL = 6 * kFragBytes;
constexpr int kRecAH = 12 * kFragBytes;
constexpr int kRecAL = 18 * kFragBytes;
constexpr int kRecGam = 24 * kFragBytes;
constexpr int kRecGend = kRecGam + C * 4;
constexpr int kRecBytes = kRecGend + C * 4;  // 25088, a multiple of 256
__host__ __device__ constexpr int lower_frag(int M, int kb) { return M < 2 ? M : 2 * M - 2 + kb; }
__host__ __device__ constexpr int frag_M(int f) { return f < 2 ? f : 2 + ((f - 2) >> 1); }
__host__ __device__ constexpr int frag_kb(int f) { return f < 2 ? 0 : (f - 2) & 1; }

// Raw buffer resource over `rows` rows of `row_bytes` bytes spaced `stride`
// bytes apart, starting at `base`: loads past the last row return zero and
// stores past it are dropped, with no branch in the instruction stream
// (0x00020000 is the gfx9-family descriptor word for untyped 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *base, int rows, int stride, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (rows - 1) * stride + row_bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ============================================================ intra kernel
constexpr int kIntraThreads = 256;
constexpr int LT = 20;                  // fp32 row stride of a 16x16 tile in LDS (16-byte aligned rows)
constexpr int LQK = DK + 8;             // bf16 row stride of the staged q, k (token-major)
constexpr int kTile = 16 * LT;          // floats per tile
__host__ __device__ constexpr int tile_id(int I, int J) { return I * (I + 1) / 2 + J; }  // lower tiles 0..9
__host__ __device__ constexpr int offdiag_id(int I, int J) { return I * (I - 1) / 2 + J; }  // J < I: 0..5

// q and k are staged token-major for the K K^T and Q K^T products; the same
// space then holds the lower 16x16 tiles of R, T and A.  T's diagonal blocks
// overwrite R's (R_II is not needed once T_II is known; R_IJ with J < I is).
struct alignas(16) IntraSmem {
    union {
        struct {
            __bf16 Q[C * LQK];
            __bf16 K[C * LQK];
        } qk;
        struct {
            float R[10 * kTile];
            float Toff[6 * kTile];
            float A[10 * kTile];
        } t;
    } u;
    float G[C];                 // in-chunk cumulative log-decay
    float eta[C];               // beta, or eta for the Kaczmarz step size (0 past the end)
    float kk[C];                // |k_i|^2 (Kaczmarz only)
};

template <bool KZ>
__global__ __launch_bounds__(kIntraThreads, 4) void intra_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, int T, int H, int NC, int total, float eps, float scale,
    char *__restrict__ ws) {
    __shared__ IntraSmem sm;
    const int qk_stride = H * DK * 2;
    auto Tb = [&](int I, int J) -> float * {  // block (I, J) of T, J <= I
        return I == J ? &sm.u.t.R[tile_id(I, I) * kTile] : &sm.u.t.Toff[offdiag_id(I, J) * kTile];
    };
    const int seg = threadIdx.x & 15, i0 = threadIdx.x >> 4;
    const int lane0 = threadIdx.x & 63;

    // Persistent: the workgroup takes chunks ci = blockIdx.x + k gridDim.x
    // ((b*H + h)*NC + c) and loads the next one's q, k and gates into
    // registers while it computes the current one.
    uint4 qv[4], kv[4];
    float gv, ev;
    auto prefetch = [&](int cj) {
        const int cc = cj % NC, bhj = cj / NC;
        const int tt = cc * C, nn = min(C, T - tt);
        const size_t r0 = ((size_t)(bhj / H) * T + tt) * H + bhj % H;
        const auto rk = rows_rsrc(k + r0 * DK, nn, qk_stride, DK * 2);
        const auto rq = rows_rsrc(q + r0 * DK, nn, qk_stride, DK * 2);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int off = (i0 + 16 * it) * qk_stride + 16 * seg;
            qv[it] = buf_ld16(rq, off);
            kv[it] = buf_ld16(rk, off);
        }
        gv = g[r0 + (size_t)min(lane0, nn - 1) * H];
        ev = beta[r0 + (size_t)min(lane0, nn - 1) * H];
    };
    prefetch(min((int)blockIdx.x, total - 1));
    for (int ci = blockIdx.x; ci < total; ci += gridDim.x) {
    // The thread index passes through an empty asm each chunk, so the many
    // per-lane LDS addresses below are recomputed per chunk instead of being
    // hoisted out of the loop and kept live (which would spill).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int c = ci % NC;
    const int bh = ci / NC;
    const int b = bh / H, h = bh % H;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    char *recb = ws + (size_t)ci * kRecBytes;
    __syncthreads();  // the previous chunk's tiles are no longer read

    // ---- gates of token `lane`: cumulative log-decay and beta (eta)
    float Gl = lane < n ? gv : 0.f;
    const float El = lane < n ? ev : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_up(Gl, off, 64);
        if (lane >= off) Gl += up;
    }
    if (w == 0) {
        sm.G[lane] = Gl;
        sm.eta[lane] = El;
        reinterpret_cast<float *>(recb + kRecGam)[lane] = __expf(Gl);
        reinterpret_cast<float *>(recb + kRecGend)[lane] = __expf(__shfl(Gl, C - 1, 64) - Gl);
    }

    // ---- stage q, k token-major (rows past the chunk read as zero), then
    // start loading the next chunk
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        *reinterpret_cast<uint4 *>(&sm.u.qk.Q[(i0 + 16 * it) * LQK + 8 * seg]) = qv[it];
        *reinterpret_cast<uint4 *>(&sm.u.qk.K[(i0 + 16 * it) * LQK + 8 * seg]) = kv[it];
    }
    prefetch(min(ci + (int)gridDim.x, total - 1));
    __syncthreads();

    // ---- K K^T (wavefronts 0, 1) and Q K^T (2, 3) on the lower tiles: even
    // wavefronts take row blocks {0, 3}, odd ones {1, 2}
    const int Ia = (w & 1) ? 1 : 0, Ib = (w & 1) ? 2 : 3;
    f32x4 acc[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const __bf16 *X = w >= 2 ? sm.u.qk.Q : sm.u.qk.K;
        const __bf16 *Kt = sm.u.qk.K;
        auto fr = [&](const __bf16 *base, int row, int kb) {
            return *reinterpret_cast<const bf16x8 *>(base + row * LQK + 32 * kb + 8 * lg);
        };
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            const bf16x8 xa = fr(X, 16 * Ia + lr, kb);
            const bf16x8 xb = fr(X, 16 * Ib + lr, kb);
            const bf16x8 k0 = fr(Kt, lr, kb);
            const bf16x8 k1 = fr(Kt, 16 + lr, kb);
            const bf16x8 k2 = fr(Kt, 32 + lr, kb);
            if (w & 1) {  // tiles (1,0) (1,1) (2,0) (2,1) (2,2)
                acc[0] = mma(xa, k0, acc[0]);
                acc[1] = mma(xa, k1, acc[1]);
                acc[2] = mma(xb, k0, acc[2]);
                acc[3] = mma(xb, k1, acc[3]);
                acc[4] = mma(xb, k2, acc[4]);
            } else {      // tiles (0,0) (3,0) (3,1) (3,2) (3,3)
                const bf16x8 k3 = fr(Kt, 48 + lr, kb);
                acc[0] = mma(xa, k0, acc[0]);
                acc[1] = mma(xb, k0, acc[1]);
                acc[2] = mma(xb, k1, acc[2]);
                acc[3] = mma(xb, k2, acc[3]);
                acc[4] = mma(xb, k3, acc[4]);
            }
        }
    }
    auto tileI = [&](int t) { return (w & 1) ? (t < 2 ? 1 : 2) : (t < 1 ? 0 : 3); };
    auto tileJ = [&](int t) { return (w & 1) ? (t < 2 ? t : t - 2) : (t < 1 ? 0 : t - 1); };
    if constexpr (KZ) {  // |k_i|^2 is the diagonal of K K^T
        if (w < 2) {
#pragma unroll
            for (int t = 0; t < 5; ++t) {
                if (tileI(t) != tileJ(t)) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (lr == 4 * lg + r) sm.kk[16 * tileI(t) + lr] = acc[t][r];
            }
        }
    }
    __syncthreads();  // G, eta (and |k|^2) in LDS; q and k no longer read

    // ---- decay (and beta for R) applied in fp32; R and A tiles to LDS
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        const int I = tileI(t), J = tileJ(t);
        const int j = 16 * J + lr;
        const float gj = sm.G[j];
        const f32x4 gi4 = *reinterpret_cast<const f32x4 *>(&sm.G[16 * I + 4 * lg]);
        float *dst = (w >= 2 ? sm.u.t.A : sm.u.t.R) + tile_id(I, J) * kTile;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * lg + r;
            const float dec = j <= i ? __expf(gi4[r] - gj) : 0.f;
            float val;
            if (w >= 2) {
                val = scale * dec * acc[t][r];
            } else {
                float bi = sm.eta[i];
                if constexpr (KZ) bi = i < n ? bi / (sm.kk[i] + eps) : 0.f;
                val = j < i ? bi * dec * acc[t][r] : 0.f;
            }
            dst[(4 * lg + r) * LT + lr] = val;
        }
    }
    __syncthreads();

    // ---- T = (I + R)^{-1}: diagonal 16x16 blocks by forward substitution
    // (one column per lane), then three levels of off-diagonal blocks on
    // fp32 MFMA:  T_IJ = -T_II sum_{M=J}^{I-1} R_IM T_MJ
    if (lane < 16) {
        const int cc = lane;
        float *blk = &sm.u.t.R[tile_id(w, w) * kTile];
        float xcol[16];
        f32x4 row[2][4];  // R row i (broadcast to every lane), the next row read ahead
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) row[0][q4] = *reinterpret_cast<const f32x4 *>(&blk[4 * q4]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int cur = i & 1;
            if (i + 1 < 16) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    if (4 * q4 < i + 1) row[cur ^ 1][q4] = *reinterpret_cast<const f32x4 *>(&blk[(i + 1) * LT + 4 * q4]);
            }
            float a0 = i == cc ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) {
                if (m & 1) a1 -= row[cur][m >> 2][m & 3] * xcol[m];
                else a0 -= row[cur][m >> 2][m & 3] * xcol[m];
            }
            xcol[i] = i < cc ? 0.f : a0 + a1;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) blk[i * LT + cc] = xcol[i];
    }
    __syncthreads();
    auto inverse_tile = [&](int I, int J) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        for (int M = J; M < I; ++M) {
            const float *Rt = &sm.u.t.R[tile_id(I, M) * kTile];
            const float *Tt = Tb(M, J);
#pragma unroll
            for (int s = 0; s < 4; ++s) P = mma32(Rt[lr * LT + 4 * lg + s], Tt[(4 * lg + s) * LT + lr], P);
        }
        const float *Tii = Tb(I, I);
        f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) out = mma32(Tii[lr * LT + 4 * lg + s], P[s], out);
        float *dst = Tb(I, J);
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * lg + r) * LT + lr] = -out[r];
    };
    if (w < 3) inverse_tile(w + 1, w);
    __syncthreads();
    if (w < 2) inverse_tile(w + 2, w);
    __syncthreads();
    if (w == 0) inverse_tile(3, 0);
    __syncthreads();

    // ---- operand fragments: T'' = T Diag(beta) and A, lower triangle only,
    // bf16 hi + lo.  Terms 0..3 of lane group p are tile columns 4p .. 4p+3
    // of tile (M, 2kb), terms 4..7 the same columns of tile (M, 2kb + 1).
    for (int u = tid; u < 2 * 6 * 64; u += kIntraThreads) {
        const int mat = u / 384, f = (u >> 6) % 6, l = u & 63;
        const int M = frag_M(f), kb = frag_kb(f), rr = l & 15, p = l >> 4;
        bf16x8 hv, lv;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int J = 2 * kb + half;
            f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
            if (J <= M) {
                const float *tile = mat == 0 ? Tb(M, J) : &sm.u.t.A[tile_id(M, J) * kTile];
                x4 = *reinterpret_cast<const f32x4 *>(&tile[rr * LT + 4 * p]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 4 * p + e;
                float x = (J < M || (J == M && col <= rr)) ? x4[e] : 0.f;
                if (mat == 0) {
                    const int jt = 16 * J + col;
                    float bj = sm.eta[jt];
                    if constexpr (KZ) bj = jt < n ? bj / (sm.kk[jt] + eps) : 0.f;
                    x *= bj;
                }
                hv[4 * half + e] = static_cast<__bf16>(x);
                lv[4 * half + e] = static_cast<__bf16>(x - static_cast<float>(hv[4 * half + e]));
            }
        }
        char *dst = recb + (mat == 0 ? kRecTH : kRecAH) + f * kFragBytes + l * 16;
        *reinterpret_cast<bf16x8 *>(dst) = hv;
        *reinterpret_cast<bf16x8 *>(dst + 6 * kFragBytes) = lv;
    }
    }  // chunk loop
}

// ============================================================ state kernel
constexpr int kStateThreads = 256;  // chain wavefronts 0, 1; helper wavefronts 2, 3
constexpr int BV = 32;              // value columns per workgroup
constexpr int NS = DV / BV;         // workgroups per (sequence, head)
constexpr int LDK = DK + 8;         // bf16 row stride of the token-major q, k
constexpr int LDV = BV + 8;         // bf16 row stride of the token-major v slice
constexpr int kXFrags = 8;          // chain -> helper: scale Gam Q S and E (4 fp32 tiles each)

struct alignas(16) StateSmem {
    __bf16 K[2][C * LDK];          // k, token-major, key channels permuted within 32-blocks
    __bf16 Q[2][C * LDK];          // q, the same layout
    __bf16 V[2][C * LDV];          // v slice, token-major
    float Gam[2][C];               // exp(G_i)
    float Gend[2][C];              // exp(G_63 - G_i)
    uint4 X[2][2][kXFrags][64];    // per chain wavefront and chunk parity
    float Ost[2][C * 20];          // per helper: its fp32 output tile, token-major, for 16-byte stores
};

// Workgroup barrier for data exchanged through LDS only: waits for this
// wavefront's LDS operations, not for its global loads, so loads issued for a
// later chunk stay in flight across it (a full __syncthreads also waits for
// every outstanding global load).  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ds_read_b64_tr_b16 (gfx950): every lane names 8 bytes (four bf16) of LDS;
// within each group of 16 lanes, element e of lane i of the result is element
// i % 4 of the 8 bytes named by lane 4e + i / 4 of the group.  So if lane j of
// group p names elements c0 + 4 (j % 4) .. +3 of row r0 + 4p + j / 4 of a
// row-major matrix, lane (i, p) receives rows r0 + 4p + e, e = 0..3, of column
// c0 + i: a transposed 4x16 block, as MFMA fragments and D tiles hold it.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Column, in the permuted token-major layout, of the 8-byte half hh (0, 1)
// of key-channel segment seg (8 channels, 0..15).
__device__ __forceinline__ int kperm_col(int seg, int hh) {
    const int s = seg & 3;
    return 32 * (seg >> 2) + 8 * ((2 * s + hh) & 3) + 4 * (s >> 1);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kStateThreads) void state_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const char *__restrict__ ws, const float *__restrict__ s0, void *__restrict__ o,
    float *__restrict__ s_final, int T, int H, int NC, int BH, float scale) {
    __shared__ StateSmem sm;

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
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const char *recs = ws + (size_t)bh * NC * kRecBytes;
    const size_t sbase = (size_t)bh * DK * DV;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    if (NC == 0) {  // empty sequence: the final state is the initial one
        if (s_final && w < 2) {
            const int jt = j0 + 16 * w;
            for (int i = 0; i < 8; ++i)
                for (int r = 0; r < 4; ++r) {
                    const size_t idx = sbase + (size_t)(16 * i + 4 * lg + r) * DV + jt + lr;
                    s_final[idx] = s0 ? s0[idx] : 0.f;
                }
        }
        return;
    }

    // The two roles run separate loops with the same number of barriers (one
    // before the first chunk, then one after each of the steps c = 0 .. NC),
    // so neither role's registers are live in the other's code.  Inside the
    // loops every global load and store is issued unconditionally (chunk
    // indices are clamped instead): the compiler's wait counts are exact only
    // when the number of memory operations between a load and its use does
    // not depend on a branch; otherwise it waits for all of them.
    if (w < 2) {
        // ================= chain wavefront: value columns jt .. jt+15
        const int jt = j0 + 16 * w;
        f32x4 S[8];  // S[i][r] = S[16i + 4lg + r][jt + lr]
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[i][r] = s0 ? s0[sbase + (size_t)(16 * i + 4 * lg + r) * DV + jt + lr] : 0.f;
        // T'' fragments of even chunks in tA, of odd chunks in tB: each chunk
        // loads the next one's into the other set (no register copies).
        bf16x8 tAh[6], tAl[6], tBh[6], tBl[6];
#pragma unroll
        for (int f = 0; f < 6; ++f) {
            tAh[f] = *reinterpret_cast<const bf16x8 *>(recs + kRecTH + f * kFragBytes + lane * 16);
            tAl[f] = *reinterpret_cast<const bf16x8 *>(recs + kRecTL + f * kFragBytes + lane * 16);
        }
        auto step = [&](int c, const bf16x8 *th, const bf16x8 *tl, bf16x8 *thn, bf16x8 *tln)
                        __attribute__((always_inline)) {
            const int buf = c & 1;
            // next chunk's T'' fragments, in flight during this chunk
            {
                const char *rn = recs + (size_t)min(c + 1, NC - 1) * kRecBytes;
#pragma unroll
                for (int f = 0; f < 6; ++f) {
                    thn[f] = *reinterpret_cast<const bf16x8 *>(rn + kRecTH + f * kFragBytes + lane * 16);
                    tln[f] = *reinterpret_cast<const bf16x8 *>(rn + kRecTL + f * kFragBytes + lane * 16);
                }
            }
            uint4 *xo = &sm.X[buf][w][0][0];
            // S as the B operand over key channels (hi, lo)
            bf16x8 SH[4], SL[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) pair_split(S[2 * kb], S[2 * kb + 1], SH[kb], SL[kb]);
            // P = K S and Q S (token tile M, this wavefront's 16 value columns,
            // sharing the state operand); the fragments of the next 32 key
            // channels are read during the products of the current ones
            f32x4 P[4] = {zero4, zero4, zero4, zero4};
            f32x4 QS[4] = {zero4, zero4, zero4, zero4};
            const __bf16 *sK = sm.K[buf];
            const __bf16 *sQ = sm.Q[buf];
            bf16x8 ka[2][4], qa[2][4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                ka[0][M] = *reinterpret_cast<const bf16x8 *>(&sK[(16 * M + lr) * LDK + 8 * lg]);
                qa[0][M] = *reinterpret_cast<const bf16x8 *>(&sQ[(16 * M + lr) * LDK + 8 * lg]);
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cur = kb & 1;
                if (kb + 1 < 4) {
#pragma unroll
                    for (int M = 0; M < 4; ++M) {
                        ka[cur ^ 1][M] = *reinterpret_cast<const bf16x8 *>(&sK[(16 * M + lr) * LDK + 32 * (kb + 1) + 8 * lg]);
                        qa[cur ^ 1][M] = *reinterpret_cast<const bf16x8 *>(&sQ[(16 * M + lr) * LDK + 32 * (kb + 1) + 8 * lg]);
                    }
                }
#pragma unroll
                for (int M = 0; M < 4; ++M) P[M] = mma(ka[cur][M], SH[kb], P[M]);
#pragma unroll
                for (int M = 0; M < 4; ++M) P[M] = mma(ka[cur][M], SL[kb], P[M]);
#pragma unroll
                for (int M = 0; M < 4; ++M) QS[M] = mma(qa[cur][M], SH[kb], QS[M]);
#pragma unroll
                for (int M = 0; M < 4; ++M) QS[M] = mma(qa[cur][M], SL[kb], QS[M]);
            }
            // decays and this wavefront's v columns
            f32x4 gam[4], gnd[4];
            bf16x4 vv[4];
            const float gs = sm.Gam[buf][C - 1];  // exp(G_63), the chunk's state decay
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                gam[M] = *reinterpret_cast<const f32x4 *>(&sm.Gam[buf][16 * M + 4 * lg]);
                gnd[M] = *reinterpret_cast<const f32x4 *>(&sm.Gend[buf][16 * M + 4 * lg]);
                // V[16M + 4lg + r][16w + lr], r = 0..3
                vv[M] = lds_read_tr(&sm.V[buf][(16 * M + 4 * lg + (lr >> 2)) * LDV + 16 * w + 4 * (lr & 3)]);
            }
            // X = V - Gam P, rows 16M + 4lg + r; the read scale Gam Q S to the helper
            f32x4 Xv[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Xv[M][r] = static_cast<float>(vv[M][r]) - gam[M][r] * P[M][r];
                    QS[M][r] *= scale * gam[M][r];
                }
                xo[M * 64 + lane] = *reinterpret_cast<const uint4 *>(&QS[M]);
            }
            bf16x8 XH[2], XL[2];
            pair_split(Xv[0], Xv[1], XH[0], XL[0]);
            pair_split(Xv[2], Xv[3], XH[1], XL[1]);
            // k^T fragments (key-channel tile i, token block kb) for the update,
            // read transposed from the token-major k: term e of lane group lg is
            // token 32kb + kperm(lg, e), key channel 16i + lr.  Tile 0 now.
            auto kt_frag = [&](int i, int kb) {
                const int col = 32 * (i >> 1) + 8 * (lr & 3) + 4 * (i & 1);  // 16i + 4(lr%4), permuted
                const int row = 32 * kb + 4 * lg + (lr >> 2);
                const bf16x4 a = lds_read_tr(&sK[row * LDK + col]);
                const bf16x4 c = lds_read_tr(&sK[(row + 16) * LDK + col]);
                return bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
            };
            bf16x8 kt[2][2];
            kt[0][0] = kt_frag(0, 0);
            kt[0][1] = kt_frag(0, 1);
            // E = T'' X
            f32x4 E[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                E[M] = zero4;
#pragma unroll
                for (int kb = 0; kb <= (M >> 1); ++kb) {
                    const int f = lower_frag(M, kb);
                    E[M] = mma(th[f], XH[kb], E[M]);
                    E[M] = mma(th[f], XL[kb], E[M]);
                    E[M] = mma(tl[f], XH[kb], E[M]);
                }
            }
            // E to the helper; Gend E as the update's B operand
            f32x4 Ep[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                xo[(4 + M) * 64 + lane] = *reinterpret_cast<const uint4 *>(&E[M]);
#pragma unroll
                for (int r = 0; r < 4; ++r) Ep[M][r] = E[M][r] * gnd[M][r];
            }
            bf16x8 PH[2], PL[2];
            pair_split(Ep[0], Ep[1], PH[0], PL[0]);
            pair_split(Ep[2], Ep[3], PH[1], PL[1]);
            // S <- gend S + K^T (Gend E), key-channel tile i (tile i+1's
            // fragments are read during tile i's products)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int cur = i & 1;
                if (i + 1 < 8) {
                    kt[cur ^ 1][0] = kt_frag(i + 1, 0);
                    kt[cur ^ 1][1] = kt_frag(i + 1, 1);
                }
                f32x4 acc = S[i] * gs;
                acc = mma(kt[cur][0], PH[0], acc);
                acc = mma(kt[cur][0], PL[0], acc);
                acc = mma(kt[cur][1], PH[1], acc);
                acc = mma(kt[cur][1], PL[1], acc);
                S[i] = acc;
            }
        };
        barrier_lds();
        int c = 0;
        for (; c + 1 < NC; c += 2) {
            step(c, tAh, tAl, tBh, tBl);
            barrier_lds();
            step(c + 1, tBh, tBl, tAh, tAl);
            barrier_lds();
        }
        if (c < NC) {
            step(c, tAh, tAl, tBh, tBl);
            barrier_lds();
        }
        barrier_lds();  // step NC: the helpers finish the last chunk's outputs
        if (s_final) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s_final[sbase + (size_t)(16 * i + 4 * lg + r) * DV + jt + lr] = S[i][r];
        }
    } else {
        // ================= helper wavefront: stages chunk c+1, outputs of chunk c-1
        const int vt = w - 2;
        const int jt = j0 + 16 * vt;
        const int ht = tid - 128;  // 0..127
        // Rows past the end of a partial last chunk read as zero (buffer
        // bounds); T'' and A are zero in those rows and columns anyway.
        uint4 kreg[8], qreg[8], vreg[2];
        float gam_reg, gnd_reg;
        const size_t head0 = (size_t)b * T * H + h;  // row of token 0 of this head
        const int qk_stride = H * DK * 2, v_stride = H * DV * 2;
        // byte offsets, inside a chunk, of this thread's q/k and v pieces
        int qk_off[8], v_off[2];
#pragma unroll
        for (int u = 0; u < 8; ++u) qk_off[u] = (8 * (ht >> 4) + u) * qk_stride + 16 * (ht & 15);
#pragma unroll
        for (int u = 0; u < 2; ++u) v_off[u] = (2 * (ht >> 2) + u) * v_stride + 2 * (j0 + 8 * (ht & 3));
        auto load_stage = [&](int cc) {  // chunk cc's q, k, v slice and G into registers
            const int t0 = cc * C;
            const int n = min(C, T - t0);
            const size_t row0 = head0 + (size_t)t0 * H;
            const auto rk = rows_rsrc(k + row0 * DK, n, qk_stride, DK * 2);
            const auto rq = rows_rsrc(q + row0 * DK, n, qk_stride, DK * 2);
            const auto rv = rows_rsrc(v + row0 * DV, n, v_stride, DV * 2);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                kreg[u] = buf_ld16(rk, qk_off[u]);
                qreg[u] = buf_ld16(rq, qk_off[u]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) vreg[u] = buf_ld16(rv, v_off[u]);
            const char *rec = recs + (size_t)cc * kRecBytes;
            gam_reg = reinterpret_cast<const float *>(rec + kRecGam)[ht & 63];
            gnd_reg = reinterpret_cast<const float *>(rec + kRecGend)[ht & 63];
        };
        auto store_stage = [&](int cc) {  // registers -> LDS buffers of chunk cc
            const int buf = cc & 1;
            const int seg = ht & 15, tg = ht >> 4;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = 8 * tg + u;
                const uint2 *kh = reinterpret_cast<const uint2 *>(&kreg[u]);
                const uint2 *qh = reinterpret_cast<const uint2 *>(&qreg[u]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int col = kperm_col(seg, hh);
                    *reinterpret_cast<uint2 *>(&sm.K[buf][i * LDK + col]) = kh[hh];
                    *reinterpret_cast<uint2 *>(&sm.Q[buf][i * LDK + col]) = qh[hh];
                }
            }
            {
                const int sv = ht & 3, tq = ht >> 2;
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    *reinterpret_cast<uint4 *>(&sm.V[buf][(2 * tq + u) * LDV + 8 * sv]) = vreg[u];
            }
            if (ht < C) {
                sm.Gam[buf][ht] = gam_reg;
                sm.Gend[buf][ht] = gnd_reg;
            }
        };
        bf16x8 ah[6], al[6];
        auto load_out_ops = [&](int cc) {  // chunk cc's A fragments
            const char *rec = recs + (size_t)cc * kRecBytes;
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                ah[f] = *reinterpret_cast<const bf16x8 *>(rec + kRecAH + f * kFragBytes + lane * 16);
                al[f] = *reinterpret_cast<const bf16x8 *>(rec + kRecAL + f * kFragBytes + lane * 16);
            }
        };
        // outputs of chunk cp: O = (scale Gam Q S, from the chain) + A E; rows
        // past the end of the sequence are dropped by the buffer bounds
        auto outputs = [&](int cp) __attribute__((always_inline)) {
            const uint4 *xi = &sm.X[cp & 1][vt][0][0];
            f32x4 O[4], E[4];
            bf16x8 eh[2], el[2];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                *reinterpret_cast<uint4 *>(&O[M]) = xi[M * 64 + lane];
                *reinterpret_cast<uint4 *>(&E[M]) = xi[(4 + M) * 64 + lane];
            }
            pair_split(E[0], E[1], eh[0], el[0]);
            pair_split(E[2], E[3], eh[1], el[1]);
#pragma unroll
            for (int M = 0; M < 4; ++M)
#pragma unroll
                for (int kb = 0; kb <= (M >> 1); ++kb) {
                    const int f = lower_frag(M, kb);
                    O[M] = mma(ah[f], eh[kb], O[M]);
                    O[M] = mma(ah[f], el[kb], O[M]);
                    O[M] = mma(al[f], eh[kb], O[M]);
                }
            const int t0 = cp * C;
            const int n = min(C, T - t0);
            const size_t row0 = head0 + (size_t)t0 * H;
            constexpr int es = OUT_BF16 ? 2 : 4;
            const auto ro = rows_rsrc(static_cast<char *>(o) + row0 * DV * es, n, H * DV * es, DV * es);
            if constexpr (OUT_BF16) {
#pragma unroll
                for (int M = 0; M < 4; ++M)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int off = ((16 * M + 4 * lg + r) * H * DV + jt + lr) * es;
                        const __bf16 hv = static_cast<__bf16>(O[M][r]);
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hv), ro, off, 0, 0);
                    }
            } else {
                // the tile through this wavefront's LDS area: one 16-byte store per
                // lane covers 4 output columns (same wavefront, so no barrier)
                float *ost = sm.Ost[vt];
#pragma unroll
                for (int M = 0; M < 4; ++M)
#pragma unroll
                    for (int r = 0; r < 4; ++r) ost[(16 * M + 4 * lg + r) * 20 + lr] = O[M][r];
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = 16 * it + (lane >> 2), c4 = 4 * (lane & 3);
                    const uint4 val = *reinterpret_cast<const uint4 *>(&ost[row * 20 + c4]);
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, val), ro,
                        (row * H * DV + jt + c4) * 4, 0, 0);
                }
            }
        };
        // step 0: stage chunk 0 (and 1); step c >= 1: outputs of chunk c-1
        load_stage(0);
        store_stage(0);
        load_stage(min(1, NC - 1));
        barrier_lds();
        if (NC > 1) store_stage(1);
        load_stage(min(2, NC - 1));
        load_out_ops(0);
        barrier_lds();
        for (int c = 1; c < NC; ++c) {
            if (c + 1 < NC) store_stage(c + 1);
            load_stage(min(c + 2, NC - 1));
            outputs(c - 1);
            load_out_ops(c);
            barrier_lds();
        }
        outputs(NC - 1);
        barrier_lds();
    }
}

// ============================================================ launchers
// Workgroups of the persistent intra kernel: four per compute unit (its LDS
// allows four), or one per chunk when there are fewer chunks.
int intra_grid(long total) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (int)std::min<long>(total, 4L * cus);
}

template <bool KZ>
hipError_t launch_intra(const ChunkArgs &a) {
    const long total = (long)a.B * a.H * a.NC;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((intra_matrix_kernel<KZ>), dim3(intra_grid(total)), dim3(kIntraThreads), 0, a.stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), a.g, a.beta, a.T, a.H,
                       a.NC, (int)total, a.eps, a.scale, static_cast<char *>(a.ws));
    return hipGetLastError();
}

template <bool OB>
hipError_t launch_state(const ChunkArgs &a) {
    const int BH = a.B * a.H;
    const unsigned grid = (unsigned)(BH * NS);
    hipLaunchKernelGGL((state_matrix_kernel<OB>), dim3(grid), dim3(kStateThreads), 0, a.stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.v), static_cast<const char *>(a.ws), a.s0, a.o, a.s_final,
                       a.T, a.H, a.NC, BH, a.scale);
    return hipGetLastError();
}

}  // namespace

size_t chunk_matrix_workspace_bytes(int B, int H, int NC, int, int, bool) {
    return (size_t)B * H * NC * kRecBytes;
}

bool chunk_matrix_supported(int Dk, int Dv, bool qkv_bf16, bool per_channel) {
    return qkv_bf16 && Dk == DK && Dv == DV && !per_channel;
}

hipError_t launch_chunk_matrix(const ChunkArgs &a, int stage) {
    if (stage != 1) {
        const hipError_t e = a.kaczmarz ? launch_intra<true>(a) : launch_intra<false>(a);
        if (e != hipSuccess || stage == 0) return e;
    }
    return a.o_bf16 ? launch_state<true>(a) : launch_state<false>(a);
}

}  // namespace gdr
