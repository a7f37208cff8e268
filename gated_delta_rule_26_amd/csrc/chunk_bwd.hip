// Backward pass of the chunked forward pass (training).  For bf16 q/k/v at
// d_k = d_v = 128 with scalar decay the products run on bf16 matrix-core
// tiles with every fp32 operand split into hi + lo, as in the forward pass
// (launch_bwd16: the forward intra kernel and walk of chunk_matrix.hip with
// backward outputs, the reverse walk and one gradient kernel below); for
// every other input on fp32 tiles (v_mfma_f32_16x16x4_f32), in the five
// kernels listed further down.
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
// Five kernels on fp32 tiles:
//  * prep (one workgroup per chunk): G, beta, M, A and T (as the forward
//    vector intra kernel, with T itself instead of W and U);
//  * forward walk (one workgroup per (sequence, head, 32 value columns)): the
//    state entering every chunk, stored;
//  * reverse walk (same grid, chunks in reverse): dS' of every chunk, stored,
//    and the gradient of the initial state (it reads no entering state, so
//    the two walks run in one launch, side by side when they fit the compute
//    units together);
//  * grads A (one workgroup per chunk): the products over the value axis, in
//    slices of 16 columns: dV, and the parts of dq, dk, dG that come through
//    K~, Q~, K^ and gam; dA and dT'' to the workspace;
//  * grads B (one workgroup per chunk): the triangular algebra (dT, dR, dM,
//    dbeta), the pair terms of M and A, the Kaczmarz step, the reverse
//    cumulative sum; writes dq, dk, dg and dbeta.
// Padded rows of a partial last chunk have k = q = v = g = beta = 0 and
// dO = 0, so they contribute nothing.
// Without the delta rule (delta = false: S = D S + k v^T) the same kernels run
// with M = 0, beta = 1 (so T'' = I), X = V (no K~ S, no K~' dX) and no
// gradient of beta.
#include "gdr_internal.h"
#include "matrix_common.h"

namespace gdr {
namespace {

using mx::state_slot;
using mx::kRevTH;
using mx::kRevTL;
using mx::kRevAH;
using mx::kRevAL;
using mx::kRevBytes;
using mx::upper_frag;
constexpr int C = kChunk;
constexpr int kThreads = 256;
constexpr int kBV = 32;  // value columns per walk workgroup
constexpr int kBS = 16;  // value columns per slice of grads A

// ---- workspace, per chunk slot ci (fixed-length: (b H + h) NC + c; packed: u H + h)
struct BwdWs {
    float *T, *A, *M, *G, *beta;   // C x C (three), C x GK, C
    float *S, *dS;                 // DK x DV: entering state; gradient of the chunk-end state
    float *dA, *dTT, *dG;          // C x C (two), C x GK
    float *dG63;                   // GK: the chunk-end decay's extra gradient (K^ and gam)
    float *Kt, *Kh, *Qt;           // C x DK each: K~, K^, Q~ (decayed operands, fp32), or null
    void *rec;                     // the bf16 walks' chunk records (forward, then reverse), or null
    void *rrev;
};

// Whether the decayed operands are stored: not for scalar decay with bf16
// inputs, whose kernels form them from k and q (exact in bf16) and the token
// factors where they use them.
constexpr bool bwd_stores_ops(bool per_channel, bool qkv_bf16) { return per_channel || !qkv_bf16; }
// Whether the entering states come from the forward pass's bf16 walk (bf16
// products with hi/lo split fp32 operands, as the forward pass computes them):
// scalar decay with bf16 inputs at d_k = d_v = 128.  Its chunk records lead
// the workspace.
constexpr bool bwd_walk16(bool ops, int Dk, int Dv) { return !ops && Dk == 128 && Dv == 128; }

// The bf16 path's records lead the workspace: the forward walk's, the segment spaces of the two walks
// (time segments of long sequences: the forward chunk maps and entering states, then the reverse walk's N'
// and entering gradients), the reverse walk's records.
size_t rev_segment_bytes(int BH, int NC) {
    const int P = chunk_walk_segments(BH, NC);
    return P > 1 ? (size_t)BH * P * 2 * mx::DK * mx::DV * sizeof(float) : 0;
}
template <int DK, int DV, bool PC>
BwdWs carve_bwd(void *ws, size_t slots, bool ops, int BH, int NC) {
    constexpr int GK = PC ? DK : 1;
    BwdWs w;
    w.rec = w.rrev = nullptr;
    if (bwd_walk16(ops, DK, DV)) {
        w.rec = ws;
        w.rrev = static_cast<char *>(ws) + slots * mx::kRecBytes + chunk_states_segment_bytes(BH, NC) +
                 rev_segment_bytes(BH, NC);
        ws = static_cast<char *>(w.rrev) + slots * kRevBytes;
    }
    float *p = static_cast<float *>(ws);
    w.T = p; p += slots * C * C;
    w.A = w.M = nullptr;
    if (!bwd_walk16(ops, DK, DV)) {  // the bf16 path forms M and A where it uses them
        w.A = p; p += slots * C * C;
        w.M = p; p += slots * C * C;
    }
    w.G = p; p += slots * C * GK;
    w.beta = p; p += slots * C;
    w.S = p; p += slots * DK * DV;
    w.dS = p; p += slots * DK * DV;
    w.dA = w.dTT = w.dG = w.dG63 = nullptr;
    if (!bwd_walk16(ops, DK, DV)) {  // the bf16 path keeps these on the workgroup that forms them
        w.dA = p; p += slots * C * C;
        w.dTT = p; p += slots * C * C;
        w.dG = p; p += slots * C * GK;
        w.dG63 = p; p += slots * GK;
    }
    w.Kt = w.Kh = w.Qt = nullptr;
    if (ops) {
        w.Kt = p; p += slots * C * DK;
        w.Kh = p; p += slots * C * DK;
        w.Qt = p;
    }
    return w;
}

template <int DK, int DV, bool PC>
size_t bwd_bytes(size_t slots, bool ops, int BH, int NC) {
    constexpr int GK = PC ? DK : 1;
    const bool walk16 = bwd_walk16(ops, DK, DV);
    const size_t grads = walk16 ? 0 : (size_t)4 * C * C + (size_t)C * GK + GK;  // A, M, dA, dT'', dG, dG63
    return slots * sizeof(float) *
               ((size_t)C * C + (size_t)C * GK + C + 2 * (size_t)DK * DV + grads + (ops ? 3 * (size_t)C * DK : 0)) +
           (walk16 ? slots * (mx::kRecBytes + kRevBytes) + chunk_states_segment_bytes(BH, NC) + rev_segment_bytes(BH, NC)
                   : 0);
}

// chunk slot ci -> token row of its token 0 and token count.  Fixed-length
// batch: ci = (b H + h) NC + c; packed batch: ci = u H + h for chunk u of the
// sequence table (its slots past the table's chunks are not used).
struct Slot {
    int n;
    size_t row0;  // [.., H, .] row of token 0; token i is row0 + i H
};
__device__ __forceinline__ Slot slot_of(int ci, int T, int H, int NC, const SeqTable &tb) {
    Slot s;
    if (tb.start) {
        const int u = ci / H, h = ci - u * H;
        const int t0 = tb.tok[u];
        s.n = min(C, tb.start[tb.seq[u] + 1] - t0);
        s.row0 = (size_t)t0 * H + h;
    } else {
        const int c = ci % NC, bh = ci / NC;
        s.n = min(C, T - c * C);
        s.row0 = ((size_t)(bh / H) * T + (size_t)c * C) * H + bh % H;
    }
    return s;
}
// Chunk slots of a launch over every chunk: packed batches have fewer than
// the grid (the chunk bound); the workgroups past them return.
__device__ __forceinline__ bool slot_used(int ci, int H, const SeqTable &tb) {
    return !tb.start || ci < tb.cbase[tb.N] * H;
}

// The chunks one walk covers: sequence b = bh / H, head h = bh % H; chunk c
// of it has slot slot(c), token row row0(c) and count(c) tokens.  A
// sequence's chunks are consecutive in its tokens and in the slot order
// (stride 1 in a fixed-length batch, H in a packed one), so after the
// sequence's start and end are read once these are arithmetic on scalars.
struct BwdWalk {
    int nc;        // chunks of the sequence
    int tok0, tend;  // its first token and one past its last (relative to its batch row)
    size_t slot0, sstride;  // slot of chunk 0 and the slot stride
    size_t row00, rstride;  // token row of chunk 0's first token and the row stride of a chunk
    __device__ __forceinline__ size_t slot(int c) const { return slot0 + (size_t)c * sstride; }
    __device__ __forceinline__ size_t row0(int c) const { return row00 + (size_t)c * rstride; }
    __device__ __forceinline__ int count(int c) const { return min(C, tend - (tok0 + c * C)); }
};
__device__ __forceinline__ BwdWalk bwd_walk(int bh, int T, int H, int NC, const SeqTable &tb) {
    BwdWalk w;
    const int b = bh / H, h = bh % H;
    w.rstride = (size_t)C * H;
    if (tb.start) {
        const int cb = tb.cbase[b];
        w.nc = tb.cbase[b + 1] - cb;
        w.tok0 = tb.start[b];
        w.tend = tb.start[b + 1];
        w.slot0 = (size_t)cb * H + h;
        w.sstride = H;
        w.row00 = (size_t)w.tok0 * H + h;
    } else {
        w.nc = NC;
        w.tok0 = 0;
        w.tend = T;
        w.slot0 = (size_t)bh * NC;
        w.sstride = 1;
        w.row00 = (size_t)b * T * H + h;
    }
    return w;
}

// ============================================================ fp32 matrix-core tiles
// v_mfma_f32_16x16x4_f32: lane l (lr = l % 16, lg = l / 16) gives A[lr][lg]
// and B[lg][lr] of a 16 x 4 by 4 x 16 product and holds D[4 lg + r][lr] in
// d[r].  A 16 x 16 tile with K = 4 m is m such steps; in step s lane l takes
// reduction index k = 4 s + lg, so every k is taken once.  fp32 operands, fp32
// accumulation: the same precision class as the vector-ALU products.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// One element of a token-major input through a raw buffer resource (rows past
// the resource's end read as zero, with no branch), at element offset `off`.
template <bool BF16>
__device__ __forceinline__ float buf_in(__amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (BF16) return bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off * 2, 0, 0));
    else return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off * 4, 0, 0));
}
using mx::barrier_lds;
using mx::rows_rsrc;
// The input elements in 16 loaded bytes, as fp32: eight bf16 or four fp32.
template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4 &r, float *dst) {
    const unsigned wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
            dst[2 * e] = __uint_as_float(wd[e] << 16);
            dst[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
        } else {
            dst[e] = __uint_as_float(wd[e]);
        }
    }
}
// A value the same in every lane, in scalar registers (so that a buffer
// resource built from it is uniform and needs no per-lane loop).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ size_t uniform(size_t x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
    return ((size_t)hi << 32) | lo;
}

// Workgroup barrier that first waits until at most N of this wavefront's
// vector memory operations are outstanding (its global-to-LDS copies
// included) and its LDS operations are done.
template <int N>
__device__ __forceinline__ void barrier_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Rows w, w + 4, .. of a C x NCOL fp32 matrix (row-major, in global memory)
// to LDS rows LD floats apart, 64 values per copy instruction.
// (A rolled loop: unrolled, the compiler would keep every copy's address live.)
template <int NCOL, int LD>
__device__ __forceinline__ void dma_rows(const float *src, float *dst, int w, int lane) {
    const float *s = src + w * NCOL + lane;
    unsigned d = mx::lds_addr(dst + w * LD);
#pragma unroll 1
    for (int i = 0; i < C / 4; ++i) {
#pragma unroll
        for (int hh = 0; hh < NCOL / 64; ++hh) mx::lds_dma4(s + 64 * hh, d + 256 * hh);
        s += 4 * NCOL;
        d += 16 * LD;
    }
}

// Swizzled fp32 matrices in LDS, rows of NCOL values (no padding): the
// 16-byte piece q of row r sits at piece q ^ (r % 16).  A float4 read of the
// same four columns of 16 consecutive rows, and a one-value read of four rows
// 4 apart by 16 consecutive columns, then fall in distinct banks, and the rows
// stay contiguous, so 1 KiB global-to-LDS copies fill them.
template <int NCOL>
__device__ __forceinline__ int lds_swz(int r, int col) {
    return r * NCOL + ((((col >> 2) ^ (r & 15))) << 2) + (col & 3);
}
// Copy instructions per wavefront for one C x NCOL matrix.
template <int NCOL>
constexpr int swz_copies() { return C * NCOL * 4 / 1024 / 4; }
// A C x NCOL fp32 matrix (row-major, in global memory) into LDS in the
// swizzled layout: 1 KiB per copy instruction (lane l moves the 16 bytes that
// belong at piece l of it), instructions w, w + 4, .. on wavefront w.
template <int NCOL>
__device__ __forceinline__ void dma_swz(const float *src, float *dst, int w, int lane) {
    constexpr int RPI = 1024 / (NCOL * 4);  // rows per instruction
    constexpr int SPR = NCOL / 4;           // 16-byte pieces per row
    static_assert(SPR >= 16 && C % RPI == 0, "the swizzle needs at least 16 pieces per row");
    const int rr = lane / SPR, q = lane % SPR;
#pragma unroll
    for (int i = 0; i < C / RPI / 4; ++i) {
        const int ins = 4 * i + w, row = ins * RPI + rr;
        mx::lds_dma16(src + row * NCOL + 4 * (q ^ (row & 15)), mx::lds_addr(dst + ins * 256));
    }
}

// LDS row strides (floats) of the fp32-tile forward walk.  A
// row-indexed-by-lane read (rows lr, columns lg) is free of bank conflicts at
// a stride of 2 mod 32, a column-indexed one (rows lg, columns lr) at 16 mod
// 32.
constexpr int kLK = 130;  // C x DK operands read row-wise (K~ in X = V - K~ S, K^ in dE)
constexpr int kLKT = 144; // C x DK operands read column-wise (K^' , K~', Q~')
constexpr int kLT = 66;   // C x C read row-wise (T'' in E = T'' X)
constexpr int kLB = 48;   // B operands of 32 columns, read column-wise

// ============================================================ prep
// One workgroup per chunk.  M and A on fp32 matrix-core tiles (wavefront w
// takes lower tiles w, w + 4, w + 8 of the list; the upper tiles are zero).
// Scalar decay: the products K K' and Q K', then the one decay factor of the
// pair.  Per-channel decay: row block I takes the reference token r = 16 I
// and the factors exp(G_ic - G_rc) (rows, <= 1) and exp(G_rc - G_jc)
// (columns, <= 1 left of the diagonal) go into the operands; a diagonal
// tile whose span max_c (G_rc - G_{r+15,c}) exceeds kSpanMax would overflow
// the column factor and is summed term by term instead.  The decayed operands
// K~, K^, Q~ are written next; then the LDS that held k and q holds R as
// 16x16 tiles and T = (I + R)^-1 is formed by the block inverse of the
// forward pass's intra kernel (forward substitution on the diagonal blocks,
// matrix-core products for the others).
constexpr float kSpanMax = 64.f;

template <int DK, bool PC, bool KZ, bool IN_BF16>
__global__ __launch_bounds__(kThreads, PC ? 1 : 2) void bwd_prep_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, int T, int H, int NC, float eps, float scale, float *__restrict__ wT,
    float *__restrict__ wA, float *__restrict__ wM, float *__restrict__ wG, float *__restrict__ wB,
    float *__restrict__ wKt, float *__restrict__ wKh, float *__restrict__ wQt, bool delta, SeqTable tb) {
    constexpr int GK = PC ? DK : 1;
    static_assert(2 * C * (DK + 1) >= 16 * mx::kTile, "the R and T tiles must fit where k and q were");
    const int ci = blockIdx.x;
    if (!slot_used(ci, H, tb)) return;
    const Slot sl = slot_of(ci, T, H, NC, tb);
    const int n = sl.n;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    __shared__ __align__(16) float sKQ[2][C][DK + 1];  // k, q; later the R and T tiles
    float (*sK)[DK + 1] = sKQ[0];
    float (*sQ)[DK + 1] = sKQ[1];
    __shared__ float sG[C][GK];
    __shared__ float sBeta[C];
    __shared__ float sE[2][C];  // scalar decay: exp(G_i), exp(G_63 - G_i)

    {  // all loads in flight at once (16 bytes per lane, rows past the chunk's end read as zero through
       // the buffer bounds), then the LDS stores
        constexpr int es = IN_BF16 ? 2 : 4, EPL = 16 / es;   // input elements per 16-byte load
        constexpr int NL = C * DK / EPL / kThreads;           // loads per thread and matrix
        constexpr int NG4 = (C * GK / 4 + kThreads - 1) / kThreads;
        const size_t row0u = uniform(sl.row0);
        const int nu = uniform(n);
        const auto rk = rows_rsrc(static_cast<const char *>(k) + row0u * DK * es, nu, H * DK * es, DK * es);
        const auto rq = rows_rsrc(static_cast<const char *>(q) + row0u * DK * es, nu, H * DK * es, DK * es);
        const auto rg = rows_rsrc(g + row0u * GK, nu, H * GK * 4, GK * 4);
        uint4 kr[NL], qr[NL];
        f32x4 gr[NG4];
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int idx = tid + u * kThreads, i = idx / (DK / EPL), c0 = (idx % (DK / EPL)) * EPL;
            kr[u] = mx::buf_ld16(rk, (i * H * DK + c0) * es);
            qr[u] = mx::buf_ld16(rq, (i * H * DK + c0) * es);
        }
#pragma unroll
        for (int u = 0; u < NG4; ++u) {
            const int idx4 = tid + u * kThreads, i = idx4 / ((GK + 3) / 4), c0 = (idx4 % ((GK + 3) / 4)) * 4;
            if constexpr (PC) {
                gr[u] = __builtin_bit_cast(f32x4, mx::buf_ld16(rg, (i * H * GK + c0) * 4));
            } else {  // one value per token: thread i < C takes token i
                gr[u] = f32x4{idx4 < C ? mx::buf_ld4f(rg, idx4 * H * 4) : 0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int idx = tid + u * kThreads, i = idx / (DK / EPL), c0 = (idx % (DK / EPL)) * EPL;
            float kv[EPL], qv[EPL];
            unpack16<IN_BF16>(kr[u], kv);
            unpack16<IN_BF16>(qr[u], qv);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                sK[i][c0 + e] = kv[e];
                sQ[i][c0 + e] = qv[e];
            }
        }
#pragma unroll
        for (int u = 0; u < NG4; ++u) {
            const int idx4 = tid + u * kThreads;
            if constexpr (PC) {
                const int i = idx4 / (GK / 4), c0 = (idx4 % (GK / 4)) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) sG[i][c0 + e] = gr[u][e];
            } else {
                if (idx4 < C) sG[idx4][0] = gr[u][0];
            }
        }
    }
    __syncthreads();
    __shared__ float sKn[KZ ? C : 1];  // |k_i|^2 (Kaczmarz step size)
    if constexpr (KZ) {  // four lanes per token, then a sum over the quad
        const int r = tid >> 2, q = tid & 3;
        float sq = 0.f;
        for (int cc = q; cc < DK; cc += 4) sq += sK[r][cc] * sK[r][cc];
        sq += __shfl_xor(sq, 1, 64);
        sq += __shfl_xor(sq, 2, 64);
        if (q == 0) sKn[r] = sq;
        barrier_lds();
    }
    if constexpr (PC) {  // in-chunk inclusive cumulative sum, one channel per thread
        if (tid < GK) {
            float run = 0.f;
            for (int i = 0; i < C; ++i) {
                run += sG[i][tid];
                sG[i][tid] = run;
            }
        }
    } else if (w == 0) {  // one token per lane: an inclusive scan across the wavefront
        float run = sG[lane][0];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(run, off, 64);
            if (lane >= off) run += up;
        }
        sG[lane][0] = run;
    }
    if (tid >= kThreads - C) {
        const int i = tid - (kThreads - C);
        float bv = 0.f;
        if (i < n && !delta) {
            bv = 1.f;
        } else if (i < n) {
            const float given = beta[sl.row0 + (size_t)i * H];
            if constexpr (KZ) {
                bv = given / (sKn[i] + eps);
            } else {
                bv = given;
            }
        }
        sBeta[i] = bv;
    }
    __syncthreads();
    if constexpr (!PC) {
        if (tid < C) {
            sE[0][tid] = __expf(sG[tid][0]);
            sE[1][tid] = __expf(sG[C - 1][0] - sG[tid][0]);
        }
    }

    // ---- M and A; this wavefront's R = Diag(beta) M values stay in registers
    float *Mg = wM + (size_t)ci * C * C, *Ag = wA + (size_t)ci * C * C;
    f32x4 rv[3];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int t = w + 4 * s4;
        // tile t as 4 I + J in nibble t: the lower tiles (J <= I) row by row, then the upper ones
        const int code = (int)((0xB76321FEDCA98540ull >> (4 * t)) & 15);
        const int I = code >> 2, J = code & 3;
        f32x4 mm = {0.f, 0.f, 0.f, 0.f}, aa = mm;
        if (t < 10) {
            if constexpr (!PC) {
                for (int kk = 0; kk < DK; kk += 4) {
                    const float kb = sK[16 * J + lr][kk + lg];
                    mm = mfma4(sK[16 * I + lr][kk + lg], kb, mm);
                    aa = mfma4(sQ[16 * I + lr][kk + lg], kb, aa);
                }
            } else {
                const int r0 = 16 * I, ir = 16 * I + lr, jc = 16 * J + lr;
                float span = 0.f;
                if (I == J) {  // max over channels of G_r - G_{r+15}: a wavefront reduction
                    for (int cc = lane; cc < DK; cc += 64) span = fmaxf(span, sG[r0][cc] - sG[r0 + 15][cc]);
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
                }
                if (span <= kSpanMax) {
                    for (int kk = 0; kk < DK; kk += 4) {
                        const int cc = kk + lg;
                        const float er = __expf(sG[ir][cc] - sG[r0][cc]);
                        const float kb = sK[jc][cc] * __expf(sG[r0][cc] - sG[jc][cc]);
                        mm = mfma4(sK[ir][cc] * er, kb, mm);
                        aa = mfma4(sQ[ir][cc] * er, kb, aa);
                    }
                } else {  // every entry j <= i directly
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * I + 4 * lg + r;
                        float sm_ = 0.f, sa = 0.f;
                        if (jc <= i) {
                            for (int cc = 0; cc < DK; ++cc) {
                                const float d = __expf(sG[i][cc] - sG[jc][cc]) * sK[jc][cc];
                                sm_ += d * sK[i][cc];
                                sa += d * sQ[i][cc];
                            }
                        }
                        mm[r] = sm_;
                        aa[r] = sa;
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * lg + r, j = 16 * J + lr;
            const float pp = PC ? (j <= i ? 1.f : 0.f) : (j <= i ? __expf(sG[i][0] - sG[j][0]) : 0.f);
            const float m = delta && j < i ? mm[r] * pp : 0.f;
            Mg[i * C + j] = m;
            Ag[i * C + j] = scale * aa[r] * pp;
            if (s4 < 3 && t < 10) rv[s4 < 3 ? s4 : 0][r] = sBeta[i] * m;
        }
    }
    for (int idx = tid; idx < C * GK; idx += kThreads) wG[(size_t)ci * C * GK + idx] = sG[idx / GK][idx % GK];
    if (tid < C) wB[(size_t)ci * C + tid] = sBeta[tid];
    // the decayed operands: K~ = exp(G) k, K^ = exp(G_63 - G) k, Q~ = scale exp(G) q (four channels
    // per thread and step, 16-byte stores), when the caller keeps them
    for (int idx4 = tid; wKt && idx4 < C * DK / 4; idx4 += kThreads) {
        const int i = idx4 / (DK / 4), c0 = (idx4 % (DK / 4)) * 4;
        f32x4 kt, kh, qt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cc = c0 + e;
            float ei, eh;
            if constexpr (PC) {
                ei = __expf(sG[i][cc]);
                eh = __expf(sG[C - 1][cc] - sG[i][cc]);
            } else {
                ei = sE[0][i];
                eh = sE[1][i];
            }
            kt[e] = ei * sK[i][cc];
            kh[e] = eh * sK[i][cc];
            qt[e] = scale * ei * sQ[i][cc];
        }
        reinterpret_cast<f32x4 *>(wKt + (size_t)ci * C * DK)[idx4] = kt;
        reinterpret_cast<f32x4 *>(wKh + (size_t)ci * C * DK)[idx4] = kh;
        reinterpret_cast<f32x4 *>(wQt + (size_t)ci * C * DK)[idx4] = qt;
    }
    __syncthreads();  // k and q are no longer read

    // ---- T = (I + R)^-1 on 16x16 tiles in the LDS of k and q
    float *tiles = &sKQ[0][0][0];
    const mx::TriTiles tri{tiles, tiles + 10 * mx::kTile, nullptr};
#pragma unroll
    for (int s4 = 0; s4 < 3; ++s4) {
        const int t = w + 4 * s4;
        if (t < 10) {
            const int code = (int)((0xB76321FEDCA98540ull >> (4 * t)) & 15);
            const int I = code >> 2, J = code & 3;
            float *dst = &tri.R[mx::tile_id(I, J) * mx::kTile];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * lg + r) * mx::LT + lr] = rv[s4][r];
        }
    }
    __syncthreads();
    mx::invert_unit_lower(tri, lane, w, lr, lg);  // ends with a barrier
    float *Tg = wT + (size_t)ci * C * C;
    for (int idx4 = tid; idx4 < C * C / 4; idx4 += kThreads) {  // 16-byte stores
        const int i = idx4 / (C / 4), j = (idx4 % (C / 4)) * 4, I = i >> 4, J = j >> 4;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<f32x4 *>(Tg)[idx4] =
            J <= I ? *reinterpret_cast<const f32x4 *>(&tri.Tb(I, J)[(i & 15) * mx::LT + (j & 15)]) : z;
    }
}

// decay factors of token i, channel cc from G in LDS
template <bool PC, int GK>
__device__ __forceinline__ float gval(const float (*sG)[GK], int i, int cc) {
    return PC ? sG[i][cc] : sG[i][0];
}

// ============================================================ forward walk: entering states
// One workgroup per (sequence, head, 32 value columns), four wavefronts in two
// pairs; pair p owns value columns j0 + 16p .. +15 and its wavefront h owns
// key channels h DK/2 .. of the state, kept in registers in the layout of a
// product's D tile.  That layout is also the B operand of the next product
// when the reduction runs over the tile's rows with index 16 t + 4 lg + e
// (step e of block t, lane group lg), so the state, X and E pass from one
// product to the next without leaving the registers.  Per chunk:
//   P_h = K~[:, half h] S_h          (each wavefront its half of the channels)
//   X = V - (P_0 + P_1)              (the pair exchanges P through LDS)
//   E = T (beta X)                   (= T'' X; both wavefronts of the pair)
//   S_h <- Diag(gam_h) S_h + K^[:, half h]' E.
// The A operands come from LDS: rows of K~ and T as float4 (four steps of one
// lane group), columns of K^ one value per step, in the swizzled layout of
// lds_swz.  The operands move from the workspace to LDS by 1 KiB
// global-to-LDS copies (no registers): K~, T, beta and G_63 of the next chunk
// into the other half of double buffers at the start of a chunk, K^ of this
// chunk into its single buffer at the same time (used last, in the update).
// Per chunk three barriers: the pair exchange; before the update, after this
// chunk's K^ has landed; at the end, after the next chunk's operands have.
// Only v goes through registers, one chunk ahead.
// The walk's LDS (a struct, so that the launch below can overlay the reverse walk's on it).
template <int DK>
struct alignas(16) BwdStatesSmem {
    float sKt[2][C * DK];
    float sT[2][C * C];
    float sKh[C * DK];
    float sB[2][C];            // beta of the chunk's tokens
    float sG[2][DK];           // G_63 per channel (scalar decay: the one value, repeated)
    f32x4 sP[2][2][4][64];     // per pair and half: the partial K~ S tiles
};
// Workgroup `blk` of `nblk` (the walk's own numbering) in LDS `sm`.
template <int DK, int DV, bool PC, bool IN_BF16>
__device__ __forceinline__ void bwd_states_body(const void *__restrict__ v, int T, int H, int NC,
                                                const float *__restrict__ wT, const float *__restrict__ wG,
                                                const float *__restrict__ wB, const float *__restrict__ wKt,
                                                const float *__restrict__ wKh, const float *__restrict__ s0,
                                                float *__restrict__ wS, bool delta, SeqTable tb,
                                                BwdStatesSmem<DK> &sm, int blk, int nblk) {
    constexpr int GK = PC ? DK : 1;
    constexpr int NT = DV / kBV;
    constexpr int HK = DK / 2, NTH = HK / 16;  // channels per wavefront of a pair, their 16-blocks
    // copy instructions per wavefront issued after K^'s: K~ and T of the next chunk and one small copy
    constexpr int kAfterKh = swz_copies<DK>() + swz_copies<C>() + 1;
    // XCD-aware placement: the value slices of one (sequence, head) share an XCD, so its L2 serves the
    // chunk operands they all read
    int bh, tile;
    state_slot(blk, nblk / NT, NT, bh, tile);
    bh = walk_seq(bh, H, tb);  // packed batches: longest sequences first
    const BwdWalk wk = bwd_walk(bh, T, H, NC, tb);
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int p = w >> 1, h = w & 1;
    const int jc = j0 + 16 * p + lr;  // this lane's value column
    const int kh0 = h * HK;           // first key channel of this wavefront's half
    auto &sKt = sm.sKt;
    auto &sT = sm.sT;
    auto &sKh = sm.sKh;
    auto &sB = sm.sB;
    auto &sG = sm.sG;
    auto &sP = sm.sP;

    // the next chunk's K~, T, beta and G_63 into buffer `b` (one small copy per wavefront: beta on
    // wavefronts 0 and 3, G_63 in 64-channel pieces on 1 and 2, beta again when there is one piece)
    auto copy_next = [&](size_t ci, int b) __attribute__((always_inline)) {
        dma_swz<DK>(wKt + ci * C * DK, sKt[b], w, lane);
        dma_swz<C>(wT + ci * C * C, sT[b], w, lane);
        if (w == 1 || (w == 2 && DK > 64))
            mx::lds_dma4(wG + ci * C * GK + (size_t)(C - 1) * GK + (PC ? 64 * (w - 1) + lane : 0),
                         mx::lds_addr(sG[b] + 64 * (w - 1)));
        else
            mx::lds_dma4(wB + ci * C + lane, mx::lds_addr(sB[b]));
    };
    f32x4 gV[4];  // v of a chunk: rows 16 M + 4 lg + r, column jc
    auto load_v = [&](int c) __attribute__((always_inline)) {
        const int n = uniform(wk.count(c));
        const size_t row0 = uniform(wk.row0(c));
        constexpr int es = IN_BF16 ? 2 : 4;
        const auto rv = rows_rsrc(static_cast<const char *>(v) + row0 * DV * es, n, H * DV * es, DV * es);
#pragma unroll
        for (int M = 0; M < 4; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) gV[M][r] = buf_in<IN_BF16>(rv, (16 * M + 4 * lg + r) * H * DV + jc);
    };

    const size_t sbase = (size_t)bh * DK * DV;
    f32x4 sv[NTH];  // S[kh0 + 16 t + 4 lg + e][jc]
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[t][e] = s0 ? s0[sbase + (size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] : 0.f;
    if (wk.nc <= 0) return;
    copy_next(uniform(wk.slot(0)), 0);
    load_v(0);
    barrier_vm<0>();
    for (int c = 0; c < wk.nc; ++c) {
        const int b = c & 1;
        const size_t ci = uniform(wk.slot(c));
        const bool more = c + 1 < wk.nc;
        const size_t cn = uniform(wk.slot(more ? c + 1 : c));
        const f32x4 vv[4] = {gV[0], gV[1], gV[2], gV[3]};
        // the state entering this chunk, to the workspace
        float *Sg = wS + ci * DK * DV;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sg[(size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] = sv[t][e];
        load_v(more ? c + 1 : c);
        dma_swz<DK>(wKh + ci * C * DK, sKh, w, lane);  // this chunk's K^ (its buffer's last reader was the previous update)
        if (more) copy_next(cn, b ^ 1);
        // P_h = K~[:, half h] S_h (X = V without the delta rule)
        const float *kt = sKt[b];
        f32x4 pp[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if (delta) {
#pragma unroll
            for (int t = 0; t < NTH; ++t)
#pragma unroll
                for (int M = 0; M < 4; ++M) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&kt[lds_swz<DK>(16 * M + lr, kh0 + 16 * t + 4 * lg)]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pp[M] = mfma4(a4[e], sv[t][e], pp[M]);
                }
        }
#pragma unroll
        for (int M = 0; M < 4; ++M) sP[p][h][M][lane] = pp[M];
        barrier_lds();  // both partial tiles of each pair
        f32x4 x[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) x[M] = vv[M] - (pp[M] + sP[p][h ^ 1][M][lane]);  // the same sum in both
        // E = T (beta X) (T lower triangular)
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] *= *reinterpret_cast<const f32x4 *>(&sB[b][16 * t + 4 * lg]);
        const float *tt = sT[b];
        f32x4 e4[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t <= M; ++t) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&tt[lds_swz<C>(16 * M + lr, 16 * t + 4 * lg)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(a4[e], x[t][e], acc);
            }
            e4[M] = acc;
        }
        // this chunk's K^ has landed (the next chunk's copies, issued after it, may still be in flight)
        if (more) barrier_vm<kAfterKh>();
        else barrier_vm<0>();
        // S_h <- Diag(gam) S_h + K^[:, half h]' E
#pragma unroll
        for (int J = 0; J < NTH; ++J) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __expf(sG[b][PC ? kh0 + 16 * J + 4 * lg + e : 0]) * sv[J][e];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * t + 4 * lg + e;
                    acc = mfma4(sKh[lds_swz<DK>(row, kh0 + 16 * J + lr)], e4[t][e], acc);
                }
            sv[J] = acc;
        }
        barrier_vm<0>();  // the next chunk's K~, T, beta, G_63 have landed; K^ is free
    }
}

// ---- forward walk, scalar decay with bf16 q and k
// The forward walk above for scalar decay and bf16 inputs: K~ = exp(G) k and
// K^ = exp(G_63 - G) k are k scaled per token, so the walk stages the chunk's
// bf16 k (exact) and applies the token factors to the product's result or to
// the other operand:
//   P_h = k[:, half h] S_h,   X = V - exp(G) (P_0 + P_1),   E = T (beta X),
//   S_h <- gam S_h + k[:, half h]' (exp(G_63 - G) E).
// Rows of k are read as 8-byte pieces, its columns by transposing reads.
// Every operand of the next chunk is staged while this chunk is processed
// (double buffers): T, G and beta by global-to-LDS copies, k and v through
// registers.  (With the decayed operands in the workspace the fp32 walk above
// is faster, 380 against 396 us on the GDN workload; this one runs when they
// are not stored.)
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void bwd_states_kq16_kernel(const __bf16 *__restrict__ v,
                                                                   const __bf16 *__restrict__ k, int T, int H, int NC,
                                                                   const float *__restrict__ wT,
                                                                   const float *__restrict__ wG,
                                                                   const float *__restrict__ wB,
                                                                   const float *__restrict__ s0, float *__restrict__ wS,
                                                                   bool delta, SeqTable tb) {
    constexpr int NT = DV / kBV;
    constexpr int HK = DK / 2, NTH = HK / 16;
    constexpr int LKB = DK + 16;                // bf16 row stride of k (rows 8 banks apart)
    constexpr int LTR = C + 8;                  // T: rows read as float4
    constexpr int NKQ = C * DK / 8 / kThreads;  // 16-byte pieces per thread of the chunk's k
    // XCD-aware placement: the value slices of one (sequence, head) share an XCD, so its L2 serves the
    // chunk operands they all read
    int bh, tile;
    state_slot(blockIdx.x, gridDim.x / NT, NT, bh, tile);
    bh = walk_seq(bh, H, tb);  // packed batches: longest sequences first
    const BwdWalk wk = bwd_walk(bh, T, H, NC, tb);
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int p = w >> 1, h = w & 1;
    const int jc = j0 + 16 * p + lr;
    const int kh0 = h * HK;
    __shared__ __align__(16) __bf16 sK[2][C * LKB];
    __shared__ __align__(16) float sT[2][C * LTR];
    __shared__ __align__(16) float sGc[2][C];  // in-chunk cumulative log-decay per token
    __shared__ __align__(16) float sB[2][C];   // beta
    __shared__ f32x4 sP[2][2][4][64];          // per pair and half: the partial k S tiles

    auto copy_at = [&](size_t ci, int b) __attribute__((always_inline)) {  // T, G, beta into buffer b
        dma_rows<C, LTR>(wT + ci * C * C, sT[b], w, lane);
        if (w == 0) mx::lds_dma4(wG + ci * C + lane, mx::lds_addr(sGc[b]));
        else if (w == 1) mx::lds_dma4(wB + ci * C + lane, mx::lds_addr(sB[b]));
    };
    uint4 gk[NKQ];  // a chunk's k, this thread's 16-byte pieces
    f32x4 gV[4];    // v of a chunk: rows 16 M + 4 lg + r, column jc
    auto load_kv = [&](int c) __attribute__((always_inline)) {
        const int n = uniform(wk.count(c));
        const size_t row0 = uniform(wk.row0(c));
        const auto rk = rows_rsrc(k + row0 * DK, n, H * DK * 2, DK * 2);
#pragma unroll
        for (int u = 0; u < NKQ; ++u) {
            const int idx = tid + u * kThreads, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            gk[u] = mx::buf_ld16(rk, (r * H * DK + c8) * 2);
        }
        const auto rv = rows_rsrc(v + row0 * DV, n, H * DV * 2, DV * 2);
#pragma unroll
        for (int M = 0; M < 4; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) gV[M][r] = buf_in<true>(rv, (16 * M + 4 * lg + r) * H * DV + jc);
    };
    auto store_k = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NKQ; ++u) {
            const int idx = tid + u * kThreads, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            *reinterpret_cast<uint4 *>(&sK[b][r * LKB + c8]) = gk[u];
        }
    };
    auto bf16lo = [](unsigned x) { return __uint_as_float(x << 16); };
    auto bf16hi = [](unsigned x) { return __uint_as_float(x & 0xffff0000u); };

    const size_t sbase = (size_t)bh * DK * DV;
    f32x4 sv[NTH];  // S[kh0 + 16 t + 4 lg + e][jc]
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[t][e] = s0 ? s0[sbase + (size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] : 0.f;
    if (wk.nc <= 0) return;
    copy_at(uniform(wk.slot(0)), 0);
    load_kv(0);
    store_k(0);
    barrier_vm<0>();
    for (int c = 0; c < wk.nc; ++c) {
        const int b = c & 1, nb = b ^ 1;
        const size_t ci = uniform(wk.slot(c));
        const bool more = c + 1 < wk.nc;
        const size_t cn = uniform(wk.slot(more ? c + 1 : c));
        const f32x4 vv[4] = {gV[0], gV[1], gV[2], gV[3]};  // this chunk's v (loaded a chunk ago)
        // the state entering this chunk, to the workspace
        float *Sg = wS + ci * DK * DV;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sg[(size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] = sv[t][e];
        // the next chunk's operands (buffer nb was last read in the iteration before this one)
        if (more) copy_at(cn, nb);
        load_kv(more ? c + 1 : c);
        // P_h = k[:, half h] S_h
        const __bf16 *kb = sK[b];
        f32x4 pp[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if (delta) {
#pragma unroll
            for (int t = 0; t < NTH; ++t)
#pragma unroll
                for (int M = 0; M < 4; ++M) {
                    const uint2 raw = *reinterpret_cast<const uint2 *>(&kb[(16 * M + lr) * LKB + kh0 + 16 * t + 4 * lg]);
                    const float a4[4] = {bf16lo(raw.x), bf16hi(raw.x), bf16lo(raw.y), bf16hi(raw.y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) pp[M] = mfma4(a4[e], sv[t][e], pp[M]);
                }
        }
#pragma unroll
        for (int M = 0; M < 4; ++M) sP[p][h][M][lane] = pp[M];
        barrier_lds();  // both partial tiles of each pair
        // token factors of this lane's rows 16 M + 4 lg + r: exp(G) and exp(G_63 - G)
        const float gend = sGc[b][C - 1];
        f32x4 fe[4], fh[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&sGc[b][16 * M + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                fe[M][r] = __expf(g4[r]);
                fh[M][r] = __expf(gend - g4[r]);
            }
        }
        // X = V - exp(G) (P_0 + P_1), then beta X
        f32x4 x[4];
#pragma unroll
        for (int M = 0; M < 4; ++M)
            x[M] = (vv[M] - fe[M] * (pp[M] + sP[p][h ^ 1][M][lane])) *
                   *reinterpret_cast<const f32x4 *>(&sB[b][16 * M + 4 * lg]);  // the same in both
        // E = T (beta X) (T lower triangular), then exp(G_63 - G) E for the update
        const float *tt = sT[b];
        f32x4 es[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t <= M; ++t) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&tt[(16 * M + lr) * LTR + 16 * t + 4 * lg]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(a4[e], x[t][e], acc);
            }
            es[M] = fh[M] * acc;
        }
        // S_h <- gam S_h + k[:, half h]' (exp(G_63 - G) E)
        const float gam = __expf(gend);
#pragma unroll
        for (int J = 0; J < NTH; ++J) {
            f32x4 acc = gam * sv[J];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const mx::bf16x4 k4 =
                    mx::lds_read_tr(&kb[(16 * t + 4 * lg + (lr >> 2)) * LKB + kh0 + 16 * J + 4 * (lr & 3)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(static_cast<float>(k4[e]), es[t][e], acc);
            }
            sv[J] = acc;
        }
        store_k(nb);       // the next chunk's k (the compiler waits for its loads)
        barrier_vm<16>();  // its T, G, beta copies and k have landed (its v may still be in flight)
    }
}

// ============================================================ reverse walk: dS' per chunk
// One workgroup per (sequence, head, 32 value columns), chunks in reverse, in
// the layout of the forward walk above: pair p owns value columns j0 + 16p ..
// +15, its wavefront h key channels h DK/2 .. of dS' (in registers).  Per
// chunk, with dO (this lane's column, rows as a D tile) in registers:
//   P_h = K^[:, half h] dS'_h            (the pair sums the halves through LDS)
//   dE = P_0 + P_1 + A' dO
//   dX = Diag(beta) T' dE                (= T''' dE; both wavefronts of the pair)
//   dS_h = Diag(gam_h) dS'_h + Q~[:, half h]' dO - K~[:, half h]' dX.
// Rows of K^ are read from LDS as float4, the columns of A, T, Q~ and K~ one
// value per lane and step.  The operands move to LDS by global-to-LDS copies
// as in the forward walk: K^ and A after the exchange barrier, T, Q~, K~, beta
// and G_63 after the chunk's last barrier; dO goes through registers one chunk
// ahead.
template <int DK>
struct alignas(16) BwdDstatesSmem {
    static constexpr int LKR = DK + 8;  // K^: rows read as float4
    static constexpr int LKC = DK + 4;  // Q~, K~: columns read one value per lane (4 lane groups in 4 bank quarters)
    static constexpr int LTC = C + 4;   // A, T: columns
    float sKh[C * LKR];
    float sQt[C * LKC];
    float sKt[C * LKC];
    float sA[C * LTC];
    float sT[C * LTC];
    float sB[C];               // beta of the chunk's tokens
    float sG[DK];              // G_63 per channel (scalar decay: the one value, repeated)
    f32x4 sP[2][2][4][64];     // per pair and half: the partial dE tiles
};
template <int DK, int DV, bool PC>
__device__ __forceinline__ void bwd_dstates_body(const float *__restrict__ dO, int T, int H, int NC,
                                                 const float *__restrict__ wT, const float *__restrict__ wA,
                                                 const float *__restrict__ wG, const float *__restrict__ wB,
                                                 const float *__restrict__ wKt, const float *__restrict__ wKh,
                                                 const float *__restrict__ wQt, const float *__restrict__ ds_final,
                                                 float *__restrict__ wdS, float *__restrict__ ds0, bool delta,
                                                 SeqTable tb, BwdDstatesSmem<DK> &sm, int blk, int nblk) {
    constexpr int GK = PC ? DK : 1;
    constexpr int NT = DV / kBV;
    constexpr int HK = DK / 2, NTH = HK / 16;
    constexpr int LKR = BwdDstatesSmem<DK>::LKR, LKC = BwdDstatesSmem<DK>::LKC, LTC = BwdDstatesSmem<DK>::LTC;
    // XCD-aware placement: the value slices of one (sequence, head) share an XCD, so its L2 serves the
    // chunk operands they all read
    int bh, tile;
    state_slot(blk, nblk / NT, NT, bh, tile);
    bh = walk_seq(bh, H, tb);  // packed batches: longest sequences first
    const BwdWalk wk = bwd_walk(bh, T, H, NC, tb);
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int p = w >> 1, h = w & 1;
    const int jc = j0 + 16 * p + lr;
    const int kh0 = h * HK;
    auto &sKh = sm.sKh;
    auto &sQt = sm.sQt;
    auto &sKt = sm.sKt;
    auto &sA = sm.sA;
    auto &sT = sm.sT;
    auto &sB = sm.sB;
    auto &sG = sm.sG;
    auto &sP = sm.sP;

    auto copy_ka = [&](size_t ci) __attribute__((always_inline)) {
        dma_rows<DK, LKR>(wKh + ci * C * DK, sKh, w, lane);
        dma_rows<C, LTC>(wA + ci * C * C, sA, w, lane);
    };
    auto copy_rest = [&](size_t ci) __attribute__((always_inline)) {
        dma_rows<C, LTC>(wT + ci * C * C, sT, w, lane);
        dma_rows<DK, LKC>(wQt + ci * C * DK, sQt, w, lane);
        dma_rows<DK, LKC>(wKt + ci * C * DK, sKt, w, lane);
        if (w == 0) mx::lds_dma4(wB + ci * C + lane, mx::lds_addr(sB));
        if (w >= 1 && w <= DK / 64)
            mx::lds_dma4(wG + ci * C * GK + (size_t)(C - 1) * GK + (PC ? 64 * (w - 1) + lane : 0),
                         mx::lds_addr(sG + 64 * (w - 1)));
    };
    f32x4 gO[4];  // dO of a chunk: rows 16 t + 4 lg + e, column jc
    auto load_do = [&](int c) __attribute__((always_inline)) {
        const int n = uniform(wk.count(c));
        const size_t row0 = uniform(wk.row0(c));
        const auto ro = rows_rsrc(dO + row0 * DV, n, H * DV * 4, DV * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) gO[t][e] = buf_in<false>(ro, (16 * t + 4 * lg + e) * H * DV + jc);
    };

    const size_t sbase = (size_t)bh * DK * DV;
    f32x4 dsv[NTH];  // dS'[kh0 + 16 t + 4 lg + e][jc]
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dsv[t][e] = ds_final ? ds_final[sbase + (size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] : 0.f;
    if (wk.nc > 0) {
        const size_t cl = uniform(wk.slot(wk.nc - 1));
        copy_ka(cl);
        copy_rest(cl);
        load_do(wk.nc - 1);
        barrier_vm<0>();
    }
    for (int c = wk.nc - 1; c >= 0; --c) {
        const size_t ci = uniform(wk.slot(c));
        const bool more = c > 0;
        const size_t cn = uniform(wk.slot(more ? c - 1 : c));
        // dS' of this chunk to the workspace
        float *dSg = wdS + ci * DK * DV;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) dSg[(size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] = dsv[t][e];
        // P_h = K^[:, half h] dS'_h
        f32x4 pp[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&sKh[(16 * M + lr) * LKR + kh0 + 16 * t + 4 * lg]);
#pragma unroll
                for (int e = 0; e < 4; ++e) pp[M] = mfma4(a4[e], dsv[t][e], pp[M]);
            }
#pragma unroll
        for (int M = 0; M < 4; ++M) sP[p][h][M][lane] = pp[M];
        barrier_vm<0>();  // partial tiles; this chunk's T, Q~, K~, beta, G_63 and dO have landed
        const f32x4 ov[4] = {gO[0], gO[1], gO[2], gO[3]};
        // dE = P_0 + P_1 + A' dO (A' upper triangular: blocks t >= M); A is read before K^ and A are
        // refilled below, so the copies wait for these reads
        f32x4 de[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = pp[M] + sP[p][h ^ 1][M][lane];  // the same sum in both
#pragma unroll
            for (int t = M; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(sA[(16 * t + 4 * lg + e) * LTC + 16 * M + lr], ov[t][e], acc);
            de[M] = acc;
        }
        barrier_vm<0>();  // every wavefront's reads of K^ and A are done
        if (more) copy_ka(cn);
        load_do(more ? c - 1 : c);  // the last 16 loads: the barrier below may leave them in flight
        // dX = Diag(beta) T' dE (T' upper triangular)
        f32x4 dx[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = M; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(sT[(16 * t + 4 * lg + e) * LTC + 16 * M + lr], de[t][e], acc);
            dx[M] = acc * *reinterpret_cast<const f32x4 *>(&sB[16 * M + 4 * lg]);
        }
        // dS_h = Diag(gam) dS'_h + Q~[:, half h]' dO - K~[:, half h]' dX (no K~ term without the delta
        // rule: X does not depend on S then)
#pragma unroll
        for (int J = 0; J < NTH; ++J) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __expf(sG[PC ? kh0 + 16 * J + 4 * lg + e : 0]) * dsv[J][e];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = mfma4(sQt[(16 * t + 4 * lg + e) * LKC + kh0 + 16 * J + lr], ov[t][e], acc);
            if (delta) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc = mfma4(-sKt[(16 * t + 4 * lg + e) * LKC + kh0 + 16 * J + lr], dx[t][e], acc);
            }
            dsv[J] = acc;
        }
        barrier_vm<16>();  // the previous chunk's K^ and A have landed; T, Q~, K~, beta, G_63 are free
        if (more) copy_rest(cn);
    }
    if (ds0) {
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) ds0[sbase + (size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] = dsv[t][e];
    }
}

// ---- both walks in one launch.  The reverse walk reads no entering state,
// so the two are independent: workgroups 0 .. nwalk-1 walk forward and
// nwalk .. 2 nwalk-1 in reverse, each in its own layout of one LDS block
// (a union of the two).  With at most half as many walks as compute units (a few heads per
// batch) the two run side by side instead of one after the other; otherwise
// the workgroups are dispatched in order and the forward ones start first.
// A walk's value slices keep workgroup ids equal mod 8 (one XCD), as their
// offset by nwalk is the same for all of them.
template <int DK>
union BwdWalksSmem {
    BwdStatesSmem<DK> fwd;
    BwdDstatesSmem<DK> rev;
};
template <int DK, int DV, bool PC, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void bwd_walks_kernel(
    const void *__restrict__ v, const float *__restrict__ dO, int T, int H, int NC, const float *__restrict__ wT,
    const float *__restrict__ wA, const float *__restrict__ wG, const float *__restrict__ wB,
    const float *__restrict__ wKt, const float *__restrict__ wKh, const float *__restrict__ wQt,
    const float *__restrict__ s0, float *__restrict__ wS, const float *__restrict__ ds_final,
    float *__restrict__ wdS, float *__restrict__ ds0, bool delta, SeqTable tb, int nwalk) {
    __shared__ BwdWalksSmem<DK> sm;
    const int blk = blockIdx.x;
    if (blk < nwalk)
        bwd_states_body<DK, DV, PC, IN_BF16>(v, T, H, NC, wT, wG, wB, wKt, wKh, s0, wS, delta, tb, sm.fwd, blk,
                                             nwalk);
    else
        bwd_dstates_body<DK, DV, PC>(dO, T, H, NC, wT, wA, wG, wB, wKt, wKh, wQt, ds_final, wdS, ds0, delta, tb,
                                     sm.rev, blk - nwalk, nwalk);
}

// ---- reverse walk, scalar decay with bf16 q and k
// The reverse walk above for scalar decay and bf16 inputs.  There
// K~ = exp(G) k, K^ = exp(G_63 - G) k and Q~ = scale exp(G) q are k and q
// scaled per token, so the walk stages the chunk's bf16 k and q (exact) and
// applies the token factors to the other operand of each product or to its
// result:
//   P_h = k[:, half h] dS'_h,   dE = exp(G_63 - G) (P_0 + P_1) + A' dO,
//   dX = Diag(beta) T' dE,
//   dS_h = gam dS'_h + q[:, half h]' (scale exp(G) dO) - k[:, half h]' (exp(G) dX).
// Rows of k are read as 8-byte pieces (a lane group's four bf16), columns of
// q and k by transposing reads (tokens 16 t + 4 lg + e of one column in one
// read).  With bf16 k and q every operand of the previous chunk fits a second
// buffer, so it is staged while this chunk is processed: A, T, G and beta by
// global-to-LDS copies, k and q through registers, dO through registers.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void bwd_dstates_kq16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ dO, int T, int H, int NC,
    float scale, const float *__restrict__ wT, const float *__restrict__ wA, const float *__restrict__ wG,
    const float *__restrict__ wB, const float *__restrict__ ds_final, float *__restrict__ wdS,
    float *__restrict__ ds0, bool delta, SeqTable tb) {
    constexpr int NT = DV / kBV;
    constexpr int HK = DK / 2, NTH = HK / 16;
    constexpr int LKB = DK + 16;                // bf16 row stride of k and q (rows 8 banks apart)
    constexpr int LTC = C + 4;                  // A, T: columns read one value per lane
    constexpr int NKQ = C * DK / 8 / kThreads;  // 16-byte pieces per thread of the chunk's k (and of q)
    // XCD-aware placement: the value slices of one (sequence, head) share an XCD, so its L2 serves the
    // chunk operands they all read
    int bh, tile;
    state_slot(blockIdx.x, gridDim.x / NT, NT, bh, tile);
    bh = walk_seq(bh, H, tb);  // packed batches: longest sequences first
    const BwdWalk wk = bwd_walk(bh, T, H, NC, tb);
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int p = w >> 1, h = w & 1;
    const int jc = j0 + 16 * p + lr;
    const int kh0 = h * HK;
    __shared__ __align__(16) __bf16 sK[2][C * LKB];
    __shared__ __align__(16) __bf16 sQ[2][C * LKB];
    __shared__ float sA[2][C * LTC];
    __shared__ float sT[2][C * LTC];
    __shared__ __align__(16) float sGc[2][C];  // in-chunk cumulative log-decay per token
    __shared__ __align__(16) float sB[2][C];   // beta
    __shared__ f32x4 sP[2][2][4][64];          // per pair and half: the partial k dS' tiles

    auto copy_at = [&](size_t ci, int b) __attribute__((always_inline)) {  // A, T, G, beta into buffer b
        dma_rows<C, LTC>(wA + ci * C * C, sA[b], w, lane);
        dma_rows<C, LTC>(wT + ci * C * C, sT[b], w, lane);
        if (w == 0) mx::lds_dma4(wG + ci * C + lane, mx::lds_addr(sGc[b]));
        else if (w == 1) mx::lds_dma4(wB + ci * C + lane, mx::lds_addr(sB[b]));
    };
    uint4 gk[NKQ], gq[NKQ];  // a chunk's k and q, this thread's 16-byte pieces
    auto load_kq = [&](int c) __attribute__((always_inline)) {
        const int n = uniform(wk.count(c));
        const size_t row0 = uniform(wk.row0(c));
        const auto rk = rows_rsrc(k + row0 * DK, n, H * DK * 2, DK * 2);
        const auto rq = rows_rsrc(q + row0 * DK, n, H * DK * 2, DK * 2);
#pragma unroll
        for (int u = 0; u < NKQ; ++u) {
            const int idx = tid + u * kThreads, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            gk[u] = mx::buf_ld16(rk, (r * H * DK + c8) * 2);
            gq[u] = mx::buf_ld16(rq, (r * H * DK + c8) * 2);
        }
    };
    auto store_kq = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NKQ; ++u) {
            const int idx = tid + u * kThreads, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            *reinterpret_cast<uint4 *>(&sK[b][r * LKB + c8]) = gk[u];
            *reinterpret_cast<uint4 *>(&sQ[b][r * LKB + c8]) = gq[u];
        }
    };
    f32x4 gO[4];  // dO of a chunk: rows 16 t + 4 lg + e, column jc
    auto load_do = [&](int c) __attribute__((always_inline)) {
        const int n = uniform(wk.count(c));
        const size_t row0 = uniform(wk.row0(c));
        const auto ro = rows_rsrc(dO + row0 * DV, n, H * DV * 4, DV * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) gO[t][e] = buf_in<false>(ro, (16 * t + 4 * lg + e) * H * DV + jc);
    };
    auto bf16lo = [](unsigned x) { return __uint_as_float(x << 16); };
    auto bf16hi = [](unsigned x) { return __uint_as_float(x & 0xffff0000u); };

    const size_t sbase = (size_t)bh * DK * DV;
    f32x4 dsv[NTH];  // dS'[kh0 + 16 t + 4 lg + e][jc]
#pragma unroll
    for (int t = 0; t < NTH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dsv[t][e] = ds_final ? ds_final[sbase + (size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] : 0.f;
    if (wk.nc > 0) {
        const int cl = wk.nc - 1;
        copy_at(uniform(wk.slot(cl)), cl & 1);
        load_kq(cl);
        load_do(cl);
        store_kq(cl & 1);
        barrier_vm<0>();
    }
    for (int c = wk.nc - 1; c >= 0; --c) {
        const int b = c & 1, nb = b ^ 1;
        const size_t ci = uniform(wk.slot(c));
        const bool more = c > 0;
        const size_t cn = uniform(wk.slot(more ? c - 1 : c));
        const f32x4 ov[4] = {gO[0], gO[1], gO[2], gO[3]};  // this chunk's dO (loaded a chunk ago)
        // dS' of this chunk to the workspace
        float *dSg = wdS + ci * DK * DV;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) dSg[(size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] = dsv[t][e];
        // the previous chunk's operands (buffer nb was last read in the iteration before this one)
        if (more) copy_at(cn, nb);
        load_kq(more ? c - 1 : c);
        load_do(more ? c - 1 : c);
        // P_h = k[:, half h] dS'_h
        const __bf16 *kb = sK[b];
        f32x4 pp[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                const uint2 raw = *reinterpret_cast<const uint2 *>(&kb[(16 * M + lr) * LKB + kh0 + 16 * t + 4 * lg]);
                const float a4[4] = {bf16lo(raw.x), bf16hi(raw.x), bf16lo(raw.y), bf16hi(raw.y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) pp[M] = mfma4(a4[e], dsv[t][e], pp[M]);
            }
#pragma unroll
        for (int M = 0; M < 4; ++M) sP[p][h][M][lane] = pp[M];
        barrier_lds();  // both partial tiles of each pair
        // token factors of this lane's rows 16 M + 4 lg + r: exp(G) and exp(G_63 - G)
        const float gend = sGc[b][C - 1];
        f32x4 fe[4], fh[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&sGc[b][16 * M + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                fe[M][r] = __expf(g4[r]);
                fh[M][r] = __expf(gend - g4[r]);
            }
        }
        // dE = exp(G_63 - G) (P_0 + P_1) + A' dO (A' upper triangular: blocks t >= M)
        f32x4 de[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = fh[M] * (pp[M] + sP[p][h ^ 1][M][lane]);  // the same in both
#pragma unroll
            for (int t = M; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(sA[b][(16 * t + 4 * lg + e) * LTC + 16 * M + lr], ov[t][e], acc);
            de[M] = acc;
        }
        // dX = Diag(beta) T' dE (T' upper triangular)
        f32x4 dx[4];
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = M; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(sT[b][(16 * t + 4 * lg + e) * LTC + 16 * M + lr], de[t][e], acc);
            dx[M] = acc * *reinterpret_cast<const f32x4 *>(&sB[b][16 * M + 4 * lg]);
        }
        // dS_h = gam dS'_h + q[:, half h]' (scale exp(G) dO) - k[:, half h]' (exp(G) dX) (no k term without
        // the delta rule: X does not depend on S then)
        f32x4 os[4], xs[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            os[t] = scale * fe[t] * ov[t];
            xs[t] = -(fe[t] * dx[t]);
        }
        const float gam = __expf(gend);
        const __bf16 *qb = sQ[b];
#pragma unroll
        for (int J = 0; J < NTH; ++J) {
            f32x4 acc = gam * dsv[J];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int at = (16 * t + 4 * lg + (lr >> 2)) * LKB + kh0 + 16 * J + 4 * (lr & 3);
                const mx::bf16x4 q4 = mx::lds_read_tr(&qb[at]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma4(static_cast<float>(q4[e]), os[t][e], acc);
                if (delta) {
                    const mx::bf16x4 k4 = mx::lds_read_tr(&kb[at]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = mfma4(static_cast<float>(k4[e]), xs[t][e], acc);
                }
            }
            dsv[J] = acc;
        }
        store_kq(nb);      // the previous chunk's k and q (the compiler waits for their loads)
        barrier_vm<16>();  // its A, T, G, beta copies and k, q have landed (its dO may still be in flight)
    }
    if (ds0) {
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) ds0[sbase + (size_t)(kh0 + 16 * t + 4 * lg + e) * DV + jc] = dsv[t][e];
    }
}

// ---- the same walk on bf16 tiles (scalar decay, bf16 inputs, d_k = d_v = 128), as the forward pass's
// walk computes the states: bf16 products with every fp32 operand split into hi + lo (matrix_common.h).
// Per chunk c, from the last, with dS' the gradient of its end state (stored first):
//   P = k dS',  dE = A' dO + Diag(exp(G_63 - G)) P,  dX = T''' dE,
//   dS = exp(G_63) dS' + q' (scale Diag(exp(G)) dO) - k' (Diag(exp(G)) dX)
// (dS is the earlier chunk's dS').  One workgroup per (sequence, head, 32 value columns), chunks in
// reverse.  Chain wavefronts 0, 1 keep dS of 16 value columns in registers as D tiles, the B operand of
// the next product, and do the dependent products: k dS' (k rows from LDS in the permuted channel
// order), T''' dE (upper-triangular fragments from the reverse record, loaded a chunk ahead) and the
// update (k' by transposing LDS reads).  Helper wavefronts 2, 3 stage k, q and the decays in LDS and,
// one chunk ahead of their chain wavefront, form the chain-independent A' dO (4 token tiles) and
// q'(scale exp(G) dO) (8 channel tiles), which reach the chain through LDS.  One barrier per chunk;
// q is staged one chunk earlier than k (the helpers read it before the chain reads k).
struct alignas(16) RevSmem {
    __bf16 K[2][C * (mx::DK + 16)];  // k, token-major, channels permuted (chunk parity)
    __bf16 Q[2][C * (mx::DK + 16)];  // q, the same
    f32x4 At[2][2][4][64];           // A' dO per chunk parity and chain wavefront, 4 token tiles
    f32x4 Qd[2][2][8][64];           // q'(scale exp(G) dO), 8 channel tiles
    float Gam[2][C], Gend[2][C];     // exp(G_i), exp(G_63 - G_i)
};

// Time segments (fixed-length batches, P > 1): workgroup g = bh P + p walks chunks [p seg, (p+1) seg) of
// its sequence.  With NPASS it starts from zero and writes only the gradient it reaches at the segment's
// first chunk, to d_end[g] (the segment's N' of dS_start = M' dS_end + N'); otherwise it starts from
// ds_final (last segment) or d_start[g], stores dS' of every chunk, and the first segment writes ds0.
template <bool DELTA, bool NPASS>
__global__ __launch_bounds__(kThreads, 1) void bwd_dstates_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ dO, int T, int H, int NC,
    float scale, const char *__restrict__ rec, const char *__restrict__ rrev, const float *__restrict__ ds_final,
    float *__restrict__ wdS, float *__restrict__ ds0, int P, int seg, const float *__restrict__ d_start,
    float *__restrict__ d_end, SeqTable tb) {
    using mx::bf16x8;
    constexpr int DK = mx::DK, DV = mx::DV, LDK = DK + 16, NT = DV / kBV;
    __shared__ RevSmem sm;
    int g, tile;
    state_slot(blockIdx.x, gridDim.x / NT, NT, g, tile);
    g = walk_seq(g, H, tb);  // packed batches (P = 1): longest sequences first
    const int bh = g / P, p = g % P;
    const BwdWalk wk = bwd_walk(bh, T, H, NC, tb);
    const int c_lo = min(p * seg, wk.nc), c_hi = min(c_lo + seg, wk.nc);
    const int nc = c_hi - c_lo, L = c_hi - 1;
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    if (w < 2) {
        // ================= chain wavefront: value columns jt .. jt+15
        const int jt = j0 + 16 * w;
        f32x4 S[8];  // dS'[16 i + 4 lg + r][jt + lr]
        const float *sfin = NPASS ? nullptr
                            : p < P - 1 ? d_start + (size_t)g * DK * DV
                                        : (ds_final ? ds_final + (size_t)bh * DK * DV : nullptr);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[i][r] = sfin ? sfin[(size_t)(16 * i + 4 * lg + r) * DV + jt + lr] : 0.f;
        if (nc > 0) {
            // T''' fragments of even chunks in tA, of odd ones in tB (each step loads the next)
            bf16x8 tAh[6], tAl[6], tBh[6], tBl[6];
            auto load_t = [&](int c, bf16x8 *th, bf16x8 *tl) __attribute__((always_inline)) {
                if constexpr (DELTA) {
                    const char *r = rrev + wk.slot(max(c, c_lo)) * kRevBytes;
#pragma unroll
                    for (int f = 0; f < 6; ++f) {
                        th[f] = *reinterpret_cast<const bf16x8 *>(r + kRevTH + f * mx::kFragBytes + lane * 16);
                        tl[f] = *reinterpret_cast<const bf16x8 *>(r + kRevTL + f * mx::kFragBytes + lane * 16);
                    }
                }
            };
            if (L & 1) load_t(L, tBh, tBl);
            else load_t(L, tAh, tAl);
            auto step = [&](int c, const bf16x8 *th, const bf16x8 *tl, bf16x8 *thn, bf16x8 *tln)
                            __attribute__((always_inline)) {
                const int buf = c & 1;
                if constexpr (!NPASS) {  // the gradient of chunk c's end state
                    float *d = wdS + wk.slot(c) * DK * DV;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) d[(size_t)(16 * i + 4 * lg + r) * DV + jt + lr] = S[i][r];
                }
                load_t(c - 1, thn, tln);
                const float gs = sm.Gam[buf][C - 1];
                bf16x8 PH[2], PL[2];  // -exp(G) dX as the update's B operand
                if constexpr (DELTA) {
                    bf16x8 SH[4], SL[4];
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) mx::pair_split(S[2 * kb], S[2 * kb + 1], SH[kb], SL[kb]);
                    // P = k dS' (token tile M); the next 32 channels' k fragments read during the products
                    const __bf16 *sK = sm.K[buf];
                    f32x4 P[4] = {z4, z4, z4, z4};
                    bf16x8 ka[2][4];
#pragma unroll
                    for (int M = 0; M < 4; ++M) ka[0][M] = *reinterpret_cast<const bf16x8 *>(&sK[(16 * M + lr) * LDK + 8 * lg]);
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const int cur = kb & 1;
                        if (kb + 1 < 4) {
#pragma unroll
                            for (int M = 0; M < 4; ++M)
                                ka[cur ^ 1][M] = *reinterpret_cast<const bf16x8 *>(
                                    &sK[(16 * M + lr) * LDK + 32 * (kb + 1) + 8 * lg]);
                        }
#pragma unroll
                        for (int M = 0; M < 4; ++M) P[M] = mx::mma(ka[cur][M], SH[kb], P[M]);
#pragma unroll
                        for (int M = 0; M < 4; ++M) P[M] = mx::mma(ka[cur][M], SL[kb], P[M]);
                    }
                    // dE = A' dO + exp(G_63 - G) P
                    f32x4 dE[4];
#pragma unroll
                    for (int M = 0; M < 4; ++M) {
                        const f32x4 gnd = *reinterpret_cast<const f32x4 *>(&sm.Gend[buf][16 * M + 4 * lg]);
                        const f32x4 at = sm.At[buf][w][M][lane];
#pragma unroll
                        for (int r = 0; r < 4; ++r) dE[M][r] = at[r] + gnd[r] * P[M][r];
                    }
                    bf16x8 EH[2], EL[2];
                    mx::pair_split(dE[0], dE[1], EH[0], EL[0]);
                    mx::pair_split(dE[2], dE[3], EH[1], EL[1]);
                    // dX = T''' dE (upper triangle: token blocks kb >= M / 2), then -exp(G) dX
                    f32x4 Ep[4];
#pragma unroll
                    for (int M = 0; M < 4; ++M) {
                        f32x4 dx = z4;
#pragma unroll
                        for (int kb = M >> 1; kb < 2; ++kb) {
                            const int f = upper_frag(M, kb);
                            dx = mx::mma(th[f], EH[kb], dx);
                            dx = mx::mma(th[f], EL[kb], dx);
                            dx = mx::mma(tl[f], EH[kb], dx);
                        }
                        const f32x4 gm = *reinterpret_cast<const f32x4 *>(&sm.Gam[buf][16 * M + 4 * lg]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) Ep[M][r] = -gm[r] * dx[r];
                    }
                    mx::pair_split(Ep[0], Ep[1], PH[0], PL[0]);
                    mx::pair_split(Ep[2], Ep[3], PH[1], PL[1]);
                }
                // dS = exp(G_63) dS' + q'(scale exp(G) dO) - k'(exp(G) dX), key-channel tile i
                const __bf16 *sK = sm.K[buf];
                bf16x8 kt[2][2];
                if constexpr (DELTA) {
                    kt[0][0] = mx::kt_operand(sK, LDK, 0, 0, lr, lg);
                    kt[0][1] = mx::kt_operand(sK, LDK, 0, 1, lr, lg);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int cur = i & 1;
                    if (DELTA && i + 1 < 8) {
                        kt[cur ^ 1][0] = mx::kt_operand(sK, LDK, i + 1, 0, lr, lg);
                        kt[cur ^ 1][1] = mx::kt_operand(sK, LDK, i + 1, 1, lr, lg);
                    }
                    f32x4 acc = S[i] * gs + sm.Qd[buf][w][i][lane];
                    if constexpr (DELTA) {
                        acc = mx::mma(kt[cur][0], PH[0], acc);
                        acc = mx::mma(kt[cur][0], PL[0], acc);
                        acc = mx::mma(kt[cur][1], PH[1], acc);
                        acc = mx::mma(kt[cur][1], PL[1], acc);
                    }
                    S[i] = acc;
                }
            };
            barrier_lds();
            barrier_lds();
            int c = L;
            if (L & 1) {  // odd chunks use tB: the last chunk first when it is odd
                step(c, tBh, tBl, tAh, tAl);
                barrier_lds();
                --c;
            }
            for (; c - 1 >= c_lo; c -= 2) {
                step(c, tAh, tAl, tBh, tBl);
                barrier_lds();
                step(c - 1, tBh, tBl, tAh, tAl);
                barrier_lds();
            }
            if (c >= c_lo) {  // the first chunk, even
                step(c, tAh, tAl, tBh, tBl);
                barrier_lds();
            }
        }
        float *d = NPASS ? d_end + (size_t)g * DK * DV : (ds0 && p == 0 ? ds0 + (size_t)bh * DK * DV : nullptr);
        if (d) {  // the gradient at the segment's start: N' of the segment, or of the initial state
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) d[(size_t)(16 * i + 4 * lg + r) * DV + jt + lr] = S[i][r];
        }
    } else if (nc > 0) {
        // ================= helper wavefront: stages k, q; A' dO and q'(scale exp(G) dO) a chunk ahead
        const int vt = w - 2, jt = j0 + 16 * vt, ht = tid - 128;
        const int qk_stride = H * DK * 2;
        uint4 kreg[8], qreg[8];
        float gam_reg = 0.f, gnd_reg = 0.f;
        f32x4 dor[4], gmr[4];   // dO[16 t + 4 lg + e][jt + lr] and exp(G) of those tokens
        bf16x8 ath[6], atl[6];  // A' fragments
        auto qk_rsrc = [&](const __bf16 *base, int c) __attribute__((always_inline)) {
            return rows_rsrc(base + uniform(wk.row0(c)) * DK, uniform(wk.count(c)), qk_stride, DK * 2);
        };
        auto load_k = [&](int c) __attribute__((always_inline)) {
            c = max(c, c_lo);
            const auto rk = qk_rsrc(k, c);
#pragma unroll
            for (int u = 0; u < 8; ++u) kreg[u] = mx::buf_ld16(rk, (8 * (ht >> 4) + u) * qk_stride + 16 * (ht & 15));
            const char *r = rec + wk.slot(c) * mx::kRecBytes;
            gam_reg = reinterpret_cast<const float *>(r + mx::kRecGam)[ht & 63];
            gnd_reg = reinterpret_cast<const float *>(r + mx::kRecGend)[ht & 63];
        };
        auto load_q = [&](int c) __attribute__((always_inline)) {
            const auto rq = qk_rsrc(q, max(c, c_lo));
#pragma unroll
            for (int u = 0; u < 8; ++u) qreg[u] = mx::buf_ld16(rq, (8 * (ht >> 4) + u) * qk_stride + 16 * (ht & 15));
        };
        auto load_d = [&](int c) __attribute__((always_inline)) {
            c = max(c, c_lo);
            const auto ro = rows_rsrc(dO + uniform(wk.row0(c)) * DV, uniform(wk.count(c)), H * DV * 4, DV * 4);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) dor[t][e] = buf_in<false>(ro, (16 * t + 4 * lg + e) * H * DV + jt + lr);
            const char *r = rec + wk.slot(c) * mx::kRecBytes;
#pragma unroll
            for (int t = 0; t < 4; ++t) gmr[t] = *reinterpret_cast<const f32x4 *>(r + mx::kRecGam + (16 * t + 4 * lg) * 4);
            if constexpr (DELTA) {
                const char *rr = rrev + wk.slot(c) * kRevBytes;
#pragma unroll
                for (int f = 0; f < 6; ++f) {
                    ath[f] = *reinterpret_cast<const bf16x8 *>(rr + kRevAH + f * mx::kFragBytes + lane * 16);
                    atl[f] = *reinterpret_cast<const bf16x8 *>(rr + kRevAL + f * mx::kFragBytes + lane * 16);
                }
            }
        };
        // into the buffers of chunk parity b (the data: the chunk last loaded)
        auto store_rows = [&](__bf16 *dst, const uint4 *src) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = 8 * (ht >> 4) + u;
                const uint2 *h2 = reinterpret_cast<const uint2 *>(&src[u]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    *reinterpret_cast<uint2 *>(&dst[i * LDK + mx::kperm_col(ht & 15, hh)]) = h2[hh];
            }
        };
        auto store_k = [&](int b) __attribute__((always_inline)) {
            store_rows(sm.K[b], kreg);
            if (ht < C) {
                sm.Gam[b][ht] = gam_reg;
                sm.Gend[b][ht] = gnd_reg;
            }
        };
        auto store_q = [&](int b) __attribute__((always_inline)) { store_rows(sm.Q[b], qreg); };
        // A' dO and q'(scale exp(G) dO) of the chunk whose dO was last loaded, q in Q[b], to buffers b
        auto compute = [&](int b) __attribute__((always_inline)) {
            if constexpr (DELTA) {
                bf16x8 OH[2], OL[2];
                mx::pair_split(dor[0], dor[1], OH[0], OL[0]);
                mx::pair_split(dor[2], dor[3], OH[1], OL[1]);
#pragma unroll
                for (int M = 0; M < 4; ++M) {
                    f32x4 acc = z4;
#pragma unroll
                    for (int kb = M >> 1; kb < 2; ++kb) {
                        const int f = upper_frag(M, kb);
                        acc = mx::mma(ath[f], OH[kb], acc);
                        acc = mx::mma(ath[f], OL[kb], acc);
                        acc = mx::mma(atl[f], OH[kb], acc);
                    }
                    sm.At[b][vt][M][lane] = acc;
                }
            }
            f32x4 sd[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) sd[t] = scale * gmr[t] * dor[t];
            bf16x8 DH[2], DL[2];
            mx::pair_split(sd[0], sd[1], DH[0], DL[0]);
            mx::pair_split(sd[2], sd[3], DH[1], DL[1]);
            const __bf16 *sQ = sm.Q[b];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bf16x8 q0 = mx::kt_operand(sQ, LDK, i, 0, lr, lg), q1 = mx::kt_operand(sQ, LDK, i, 1, lr, lg);
                f32x4 acc = mx::mma(q0, DH[0], z4);
                acc = mx::mma(q0, DL[0], acc);
                acc = mx::mma(q1, DH[1], acc);
                acc = mx::mma(q1, DL[1], acc);
                sm.Qd[b][vt][i][lane] = acc;
            }
        };
        // before the first barrier: k, q of chunk L staged; then q of L - 1 and dO of L loaded
        load_k(L);
        load_q(L);
        store_k(L & 1);
        store_q(L & 1);
        load_q(L - 1);
        load_d(L);
        barrier_lds();
        // before the second: chunk L's products; q of L - 1 staged
        compute(L & 1);
        store_q((L - 1) & 1);
        load_k(L - 1);
        load_q(L - 2);
        load_d(L - 1);
        barrier_lds();
        // during the chain's step on chunk c: k of c - 1 and q of c - 2 staged, chunk c - 1's products
        for (int c = L; c >= c_lo; --c) {
            store_k((c - 1) & 1);
            store_q((c - 2) & 1);
            compute((c - 1) & 1);
            load_k(c - 2);
            load_q(c - 3);
            load_d(c - 2);
            barrier_lds();
        }
    }
}

// ============================================================ grads A: products over the value axis
// One workgroup per chunk, four wavefronts; wavefront w owns rows 16w .. 16w+15
// of every C-row product.  Over the value axis in slices of 16 columns:
//   X = V - K~ S,  dE = A' dO + K^ dS',  E = T'' X,  dX = transpose(T'') dE (= dV),
// and, accumulated over the slices in matrix-core accumulators,
//   dQ~ += dO S',  dK~ -= dX S',  dK^ += E dS'',  dA += dO E',  dT'' += dE X'.
// Then the parts of dq, dk, dG through K~, Q~, K^ and gam; dA and dT'' to the
// workspace.  Every product takes reduction index 16 t + 4 lg + e in step
// (t, e) from lane group lg, so that each operand gives a lane its four values
// as one float4 of a row: the wavefront's rows of K~ and K^ stay in registers
// in that order, and the LDS holds the other operands in the orientation that
// makes the reduction index run along rows (T'' and its transpose, A
// transposed, the slices of S, dS' and dO both ways, X and dE both ways).  The
// slice operands are loaded one slice ahead; the barriers wait for LDS
// operations only, so those loads stay in flight across them.  With KQ (scalar
// decay, bf16 inputs) K~, K^ and Q~ are not in the workspace: their values are
// formed here from k, q and the token factors, as the prep kernel forms them.
template <int DK, int DV, bool PC, bool IN_BF16, bool KQ>
__global__ __launch_bounds__(kThreads) void bwd_grads_a_kernel(
    const void *__restrict__ v, const float *__restrict__ dO, int T, int H, int NC, float scale,
    const float *__restrict__ wT, const float *__restrict__ wA, const float *__restrict__ wG,
    const float *__restrict__ wB, const float *__restrict__ wS, const float *__restrict__ wdS,
    const float *__restrict__ wKt, const float *__restrict__ wKh, const float *__restrict__ wQt,
    const __bf16 *__restrict__ kin, const __bf16 *__restrict__ qin, float *__restrict__ wdA,
    float *__restrict__ wdTT, float *__restrict__ wdG, float *__restrict__ wdG63, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv, bool delta, SeqTable tb) {
    constexpr int GK = PC ? DK : 1;
    constexpr int JK = DK / 16;   // column tiles of the C x DK accumulators, and reduction blocks over channels
    constexpr int LR = kBS + 4;   // rows of a 16-column slice (16-byte aligned)
    constexpr int LSt = DK + 4;   // rows of a transposed DK x 16 slice
    constexpr int LCt = C + 4;    // rows of C x C operands and of transposed C x 16 tiles
    constexpr int NT4 = C * C / 4 / kThreads;       // float4s per thread of a C x C operand
    constexpr int NS4 = DK * kBS / 4 / kThreads;    // float4s per thread of a DK x 16 slice
    const int ci = blockIdx.x;
    if (!slot_used(ci, H, tb)) return;
    const Slot sl = slot_of(ci, T, H, NC, tb);
    const int n = sl.n;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    __shared__ float sT[C * LCt];     // T'' = T Diag(beta)
    __shared__ float sTt[C * LCt];    // transpose(T'')
    __shared__ float sAt[C * LCt];    // transpose(A)
    __shared__ float sS[DK * LR], sdS[DK * LR];         // slices of S and dS', channel rows
    __shared__ float sSt[kBS * LSt], sdSt[kBS * LSt];   // the same, column rows
    __shared__ float sO[C * LR], sOt[kBS * LCt];        // slice of dO, token rows and column rows
    __shared__ float sX[C * LR], sXt[kBS * LCt];
    __shared__ float sdE[C * LR], sdEt[kBS * LCt];
    __shared__ float sE[C * LR], sdX[C * LR];
    __shared__ float sBeta[C];
    __shared__ float sH[4][DK];       // per wavefront: column sums of dK^ K^

    // this wavefront's rows of K~ and K^: kt[t][e] = K~[16w + lr][16t + 4lg + e]
    f32x4 kt[JK], kh[JK];
    if constexpr (KQ) {  // exp(G_r) k_r and exp(G_63 - G_r) k_r, k read 8 bytes (four bf16) at a time
        static_assert(!PC && IN_BF16, "k and q scaled per token: scalar decay, bf16 inputs");
        const int r = 16 * w + lr;
        const float gr = wG[(size_t)ci * C + r], gend = wG[(size_t)ci * C + C - 1];
        const float fe = __expf(gr), fh = __expf(gend - gr);
        const auto rk = rows_rsrc(kin + uniform(sl.row0) * DK, uniform(n), H * DK * 2, DK * 2);
#pragma unroll
        for (int t = 0; t < JK; ++t) {
            const auto raw = __builtin_amdgcn_raw_buffer_load_b64(rk, (r * H * DK + 16 * t + 4 * lg) * 2, 0, 0);
            const f32x4 k4 = {__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                              __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
            kt[t] = fe * k4;
            kh[t] = fh * k4;
        }
    } else {
        const float *ktr = wKt + ((size_t)ci * C + 16 * w + lr) * DK + 4 * lg;
        const float *khr = wKh + ((size_t)ci * C + 16 * w + lr) * DK + 4 * lg;
#pragma unroll
        for (int t = 0; t < JK; ++t) {
            kt[t] = *reinterpret_cast<const f32x4 *>(ktr + 16 * t);
            kh[t] = *reinterpret_cast<const f32x4 *>(khr + 16 * t);
        }
    }
    {  // T'' both ways and A transposed: all loads in flight (16 bytes per lane), then the LDS stores
        f32x4 rT[NT4], rA[NT4];
        const f32x4 *t4 = reinterpret_cast<const f32x4 *>(wT + (size_t)ci * C * C);
        const f32x4 *a4 = reinterpret_cast<const f32x4 *>(wA + (size_t)ci * C * C);
#pragma unroll
        for (int u = 0; u < NT4; ++u) {
            rT[u] = t4[tid + u * kThreads];
            rA[u] = a4[tid + u * kThreads];
        }
        // the columns of this thread's pieces: beta[m0 .. m0 + 3]
        const f32x4 b4 = reinterpret_cast<const f32x4 *>(wB + (size_t)ci * C)[tid % (C / 4)];
        if (tid < C) sBeta[tid] = wB[(size_t)ci * C + tid];
#pragma unroll
        for (int u = 0; u < NT4; ++u) {
            const int idx4 = tid + u * kThreads, i = idx4 / (C / 4), m0 = (idx4 % (C / 4)) * 4;
            const f32x4 tt = rT[u] * b4;
            *reinterpret_cast<f32x4 *>(&sT[i * LCt + m0]) = tt;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sTt[(m0 + e) * LCt + i] = tt[e];
                sAt[(m0 + e) * LCt + i] = rA[u][e];
            }
        }
    }

    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 aQ[JK], aKt[JK], aKh[JK], aA[4], aT[4];
#pragma unroll
    for (int J = 0; J < JK; ++J) aQ[J] = aKt[J] = aKh[J] = z4;
#pragma unroll
    for (int J = 0; J < 4; ++J) aA[J] = aT[J] = z4;
    float dgam = 0.f;  // channel tid (tid < DK)

    const float *Sg = wS + (size_t)ci * DK * DV;
    const float *dSg = wdS + (size_t)ci * DK * DV;
    const size_t row0u = uniform(sl.row0);
    const int nu = uniform(n);
    constexpr int es = IN_BF16 ? 2 : 4;
    const auto r_o = rows_rsrc(dO + row0u * DV, nu, H * DV * 4, DV * 4);
    const auto r_v = rows_rsrc(static_cast<const char *>(v) + row0u * DV * es, nu, H * DV * es, DV * es);
    const auto r_dv = rows_rsrc(dv + row0u * DV, nu, H * DV * 4, DV * 4);
    f32x4 rS[NS4], rdS[NS4], rO;  // this thread's four-column pieces of the slice
    f32x4 rV;                      // v in the layout of this wavefront's X tile
    // every load and store in the slice loop is issued unconditionally (buffer bounds drop the rows past
    // the chunk's end), which keeps the compiler's wait counts exact
    auto fetch = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NS4; ++u) {
            const int idx4 = tid + u * kThreads, r = idx4 / (kBS / 4), c0 = (idx4 % (kBS / 4)) * 4;
            rS[u] = *reinterpret_cast<const f32x4 *>(&Sg[(size_t)r * DV + j0 + c0]);
            rdS[u] = *reinterpret_cast<const f32x4 *>(&dSg[(size_t)r * DV + j0 + c0]);
        }
        {
            const int r = tid / (kBS / 4), c0 = (tid % (kBS / 4)) * 4;  // C x 16 = 256 float4s
            rO = __builtin_bit_cast(f32x4, mx::buf_ld16(r_o, (r * H * DV + j0 + c0) * 4));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) rV[r] = buf_in<IN_BF16>(r_v, (16 * w + 4 * lg + r) * H * DV + j0 + lr);
    };
    fetch(0);
    for (int j0 = 0; j0 < DV; j0 += kBS) {
        barrier_lds();  // the previous slice's reads are done (and, first time, T'', A staged)
#pragma unroll
        for (int u = 0; u < NS4; ++u) {
            const int idx4 = tid + u * kThreads, r = idx4 / (kBS / 4), c0 = (idx4 % (kBS / 4)) * 4;
            *reinterpret_cast<f32x4 *>(&sS[r * LR + c0]) = rS[u];
            *reinterpret_cast<f32x4 *>(&sdS[r * LR + c0]) = rdS[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sSt[(c0 + e) * LSt + r] = rS[u][e];
                sdSt[(c0 + e) * LSt + r] = rdS[u][e];
            }
        }
        {
            const int r = tid / (kBS / 4), c0 = (tid % (kBS / 4)) * 4;
            *reinterpret_cast<f32x4 *>(&sO[r * LR + c0]) = rO;
#pragma unroll
            for (int e = 0; e < 4; ++e) sOt[(c0 + e) * LCt + r] = rO[e];
        }
        const f32x4 vv = rV;
        fetch(min(j0 + kBS, DV - kBS));
        barrier_lds();
        // X = V - K~ S;  dE = K^ dS' + A' dO (A' upper triangular: token blocks t >= w)
        f32x4 x = z4, de = z4;
#pragma unroll
        for (int t = 0; t < JK; ++t) {
            const f32x4 bs = *reinterpret_cast<const f32x4 *>(&sSt[lr * LSt + 16 * t + 4 * lg]);
            const f32x4 bd = *reinterpret_cast<const f32x4 *>(&sdSt[lr * LSt + 16 * t + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x = mfma4(kt[t][e], bs[e], x);
                de = mfma4(kh[t][e], bd[e], de);
            }
        }
        x = delta ? vv - x : vv;  // without the delta rule X = V
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < w) continue;
            const f32x4 aa = *reinterpret_cast<const f32x4 *>(&sAt[(16 * w + lr) * LCt + 16 * t + 4 * lg]);
            const f32x4 bo = *reinterpret_cast<const f32x4 *>(&sOt[lr * LCt + 16 * t + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) de = mfma4(aa[e], bo[e], de);
        }
        *reinterpret_cast<f32x4 *>(&sXt[lr * LCt + 16 * w + 4 * lg]) = x;
        *reinterpret_cast<f32x4 *>(&sdEt[lr * LCt + 16 * w + 4 * lg]) = de;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sX[(16 * w + 4 * lg + r) * LR + lr] = x[r];
            sdE[(16 * w + 4 * lg + r) * LR + lr] = de[r];
        }
        barrier_lds();
        // E = T'' X (token blocks t <= w);  dX = transpose(T'') dE (blocks t >= w)
        f32x4 ee = z4, dx = z4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t <= w) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sT[(16 * w + lr) * LCt + 16 * t + 4 * lg]);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(&sXt[lr * LCt + 16 * t + 4 * lg]);
#pragma unroll
                for (int e = 0; e < 4; ++e) ee = mfma4(a[e], b[e], ee);
            }
            if (t >= w) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sTt[(16 * w + lr) * LCt + 16 * t + 4 * lg]);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(&sdEt[lr * LCt + 16 * t + 4 * lg]);
#pragma unroll
                for (int e = 0; e < 4; ++e) dx = mfma4(a[e], b[e], dx);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lg + r;
            sE[i * LR + lr] = ee[r];
            sdX[i * LR + lr] = dx[r];
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dx[r]), r_dv, (i * H * DV + j0 + lr) * 4, 0, 0);
        }
        barrier_lds();
        // accumulators of rows 16w .. (reduction over this slice's 16 value columns; step e of lane
        // group lg takes column 4 lg + e)
        {
            const int ka = (16 * w + lr) * LR + 4 * lg;
            // without the delta rule X does not depend on K~, and T'' (so beta) is fixed
            const f32x4 ao = *reinterpret_cast<const f32x4 *>(&sO[ka]);
            const f32x4 ae = *reinterpret_cast<const f32x4 *>(&sE[ka]);
            const f32x4 ax = delta ? -*reinterpret_cast<const f32x4 *>(&sdX[ka]) : z4;
            const f32x4 ade = delta ? *reinterpret_cast<const f32x4 *>(&sdE[ka]) : z4;
#pragma unroll
            for (int J = 0; J < JK; ++J) {
                const int kb = (16 * J + lr) * LR + 4 * lg;
                const f32x4 bs = *reinterpret_cast<const f32x4 *>(&sS[kb]);
                const f32x4 bd = *reinterpret_cast<const f32x4 *>(&sdS[kb]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    aQ[J] = mfma4(ao[e], bs[e], aQ[J]);
                    aKt[J] = mfma4(ax[e], bs[e], aKt[J]);
                    aKh[J] = mfma4(ae[e], bd[e], aKh[J]);
                }
            }
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                const int kb = (16 * J + lr) * LR + 4 * lg;
                const f32x4 be = *reinterpret_cast<const f32x4 *>(&sE[kb]);
                const f32x4 bx = *reinterpret_cast<const f32x4 *>(&sX[kb]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    aA[J] = mfma4(ao[e], be[e], aA[J]);
                    aT[J] = mfma4(ade[e], bx[e], aT[J]);
                }
            }
        }
        if (tid < DK) {
            const f32x4 *s4 = reinterpret_cast<const f32x4 *>(&sS[tid * LR]);
            const f32x4 *d4 = reinterpret_cast<const f32x4 *>(&sdS[tid * LR]);
            f32x4 acc = z4;
#pragma unroll
            for (int q = 0; q < kBS / 4; ++q) acc += d4[q] * s4[q];
            dgam += (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
    }

    // dA, dT'' (lower triangle incl. the diagonal) to the workspace
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lg + r, m = 16 * J + lr;
            wdA[(size_t)ci * C * C + i * C + m] = m <= i ? aA[J][r] : 0.f;
            wdTT[(size_t)ci * C * C + i * C + m] = m <= i ? aT[J][r] : 0.f;
        }
    // parts of dq, dk through Q~, K~, K^ (rows past the end are not written);
    // parts of dG: dK~ K~ + dQ~ Q~ - dK^ K^; for G_63 also sum_i dK^ K^ + dgam gam
    const float *Gc = wG + (size_t)ci * C * GK;
    float rowpart[4] = {0.f, 0.f, 0.f, 0.f};  // scalar decay: sums over this lane's channels
    [[maybe_unused]] const size_t kq0 = KQ ? uniform(sl.row0) * DK : 0;
    [[maybe_unused]] const auto rkq = rows_rsrc(kin + kq0, KQ ? uniform(n) : 0, H * DK * 2, DK * 2);
    [[maybe_unused]] const auto rqq = rows_rsrc(qin + kq0, KQ ? uniform(n) : 0, H * DK * 2, DK * 2);
    float colh[JK];                           // per channel 16J + lr: sum over this lane's rows of dK^ K^
#pragma unroll
    for (int J = 0; J < JK; ++J) {
        colh[J] = 0.f;
        const int ch = 16 * J + lr;
        const float ge = Gc[(C - 1) * GK + (PC ? ch : 0)];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lg + r;
            const float gi = Gc[i * GK + (PC ? ch : 0)];
            const float ei = __expf(gi);
            float ktv, khv, qt;
            if constexpr (KQ) {
                const float kv = buf_in<true>(rkq, i * H * DK + ch), qv = buf_in<true>(rqq, i * H * DK + ch);
                ktv = ei * kv;
                khv = __expf(ge - gi) * kv;
                qt = scale * ei * qv;
            } else {
                ktv = wKt[((size_t)ci * C + i) * DK + ch];
                khv = wKh[((size_t)ci * C + i) * DK + ch];
                qt = wQt[((size_t)ci * C + i) * DK + ch];
            }
            if (i < n) {
                const size_t off = (sl.row0 + (size_t)i * H) * DK + ch;
                dq[off] = scale * ei * aQ[J][r];
                dk[off] = ei * aKt[J][r] + __expf(ge - gi) * aKh[J][r];
            }
            const float part = aKt[J][r] * ktv + aQ[J][r] * qt - aKh[J][r] * khv;
            colh[J] += aKh[J][r] * khv;
            if constexpr (PC) wdG[((size_t)ci * C + i) * GK + ch] = part;
            else rowpart[r] += part;
        }
    }
    if constexpr (!PC) {  // sum over the 16 lanes of a row group (lr), then one lane writes each row
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sum = rowpart[r];
            sum += __shfl_xor(sum, 1, 64);
            sum += __shfl_xor(sum, 2, 64);
            sum += __shfl_xor(sum, 4, 64);
            sum += __shfl_xor(sum, 8, 64);
            if (lr == 0) wdG[(size_t)ci * C + 16 * w + 4 * lg + r] = sum;
        }
    }
    // the chunk-end decay: per channel the column sum of dK^ K^ (lanes lg, then
    // wavefronts, in a fixed order) plus dgam gam; summed over channels for scalar decay
#pragma unroll
    for (int J = 0; J < JK; ++J) {
        float sum = colh[J];
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        if (lg == 0) sH[w][16 * J + lr] = sum;
    }
    __syncthreads();
    if (tid < DK) {
        const float ge = Gc[(C - 1) * GK + (PC ? tid : 0)];
        const float extra = ((sH[0][tid] + sH[1][tid]) + (sH[2][tid] + sH[3][tid])) + dgam * __expf(ge);
        if constexpr (PC) wdG63[(size_t)ci * GK + tid] = extra;
        else sH[0][tid] = extra;
    }
    if constexpr (!PC) {  // the sum over channels, on one wavefront
        __syncthreads();
        if (w == 0) {
            float s = 0.f;
            for (int cc = lane; cc < DK; cc += 64) s += sH[0][cc];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
            if (lane == 0) wdG63[ci] = s;
        }
    }
}

// Entering gradients of the reverse walk's time segments: D_P = ds_final (or zero), D_p = M_p' D_{p+1} +
// N'_p for p = P-1 .. 1, with M_p the forward chunk map of segment p (S_end = M_p S_start + N_p, from the
// states walk's transfer walk: the reverse map of a segment is its transpose) and N'_p the reverse walk
// from zero over it; segment p walks from D_{p+1}, stored at d_start[bh P + p].  One workgroup per
// (sequence, head, 16 value columns); thread t forms row t / 2, columns 8 (t % 2) .. +7 of its slice.
__global__ __launch_bounds__(256) void rev_segment_combine_kernel(const float *__restrict__ tr,
                                                                  const float *__restrict__ nrev,
                                                                  const float *__restrict__ ds_final,
                                                                  float *__restrict__ d_start, int P) {
    constexpr int DK = mx::DK, DV = mx::DV, CC = 16, LM = DK + 1, NCS = DV / CC;
    __shared__ float Ds[DK][CC];
    __shared__ float Ms[DK * LM];  // M_p transposed: Ms[i][k] = M_p[k][i]
    const int bh = blockIdx.x / NCS, cs = blockIdx.x % NCS;
    const int t = threadIdx.x, i = t >> 1, jl = 8 * (t & 1), jb = cs * CC + jl;
    const size_t mat = (size_t)DK * DV;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) Ds[i][jl + jj] = ds_final ? ds_final[bh * mat + i * DV + jb + jj] : 0.f;
    for (int pp = P - 1; pp >= 1; --pp) {
        const float *N = nrev + (size_t)(bh * P + pp) * mat;
        const float *M = tr + ((size_t)(bh * P + pp) * 2 + 1) * mat;
        constexpr int PER = DK * DK / 256;
        float mr[PER], acc[8];
#pragma unroll
        for (int u = 0; u < PER; ++u) mr[u] = M[t + u * 256];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[jj] = N[i * DV + jb + jj];
        __syncthreads();  // the previous step's reads of Ms and Ds are done
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = t + u * 256;
            Ms[(idx % DK) * LM + idx / DK] = mr[u];
        }
        __syncthreads();
        for (int kk = 0; kk < DK; ++kk) {
            const float m = Ms[i * LM + kk];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) acc[jj] = fmaf(m, Ds[kk][jl + jj], acc[jj]);
        }
        __syncthreads();
        float *out = d_start + (size_t)(bh * P + pp - 1) * mat;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            Ds[i][jl + jj] = acc[jj];
            out[i * DV + jb + jj] = acc[jj];
        }
    }
}

// ---- grads A on bf16 tiles (scalar decay, bf16 inputs, d_k = d_v = 128): the products of the kernel
// above with every fp32 operand split into bf16 hi + lo (hi*hi + hi*lo + lo*hi; k and v exact), in
// slices of 32 value columns.  A slice's operands live in LDS as bf16 hi and lo arrays: the S, dS' and dO
// slices as they are in memory ([row][value], 16-byte loads), X, dE, E and dX, which arrive as D tiles, in
// [value][row] orientation.  Every operand read is then one of two kinds: 8-byte reads along an array's
// rows (rows_operand), or transposing reads across them (vals_operand), whichever orientation the product
// reduces over.  This wavefront's rows of
// k (A operand over channels, exact), of T'' (lower) and of T''' and A' (upper) stay in registers, the
// fragments from the walks' records.  Four barriers per slice: slice operands staged; X, dE; E, dX; the
// value-axis accumulations done.  Eight wavefronts: wavefront w takes token rows 16 (w % 4) .., value
// tile w / 4 of each slice's 32 columns, channel tiles 4 (w / 4) .. of the value-axis accumulations, and
// dA (w < 4) or dT'' (w >= 4).
constexpr int kSW = 32;           // value columns per slice
constexpr int kLSV = kSW + 8;     // bf16 pitch of the [row][value] arrays
constexpr int kLST = C + 8;       // bf16 pitch of the [value][token] arrays

constexpr int kLCB = C + 1;       // fp32 pitch of the C x C arrays of the triangular algebra
constexpr int kLQB = mx::DK + 16;  // bf16 pitch of k and q there

struct alignas(16) GradsSmem {
    union {
        struct {  // the value-axis products
            __bf16 S[2][mx::DK * kLSV], dS[2][mx::DK * kLSV];  // [hi, lo][key channel][value]
            __bf16 O[2][C * kLSV];                              // [hi, lo][token][value]
            __bf16 X[2][kSW * kLST], dE[2][kSW * kLST], E[2][kSW * kLST], dX[2][kSW * kLST];  // [value][token]
        } a;
        struct {  // the triangular algebra and the pair terms
            float T[C * kLCB], X[C * kLCB], Y[C * kLCB], D[C * kLCB], M[C * kLCB], A[C * kLCB];
            __bf16 K[C * kLQB], Q[C * kLQB];
        } b;
    } u;
    float gsum[mx::DK];  // per key channel: sum over values of dS' S
    float H[4][mx::DK];  // per token block: column sums of dK^ K^
    float rowp[2][C];    // per half of the channels: the token rows' parts of dG
    float G[C], beta[C], dbeta[C], kk[C], dG[C];
};

// Along the rows of an array (pitch ld): row 16 vt + lr, columns 32 kb + kperm(lg, e).
__device__ __forceinline__ mx::bf16x8 rows_operand(const __bf16 *s, int ld, int vt, int kb, int lr, int lg) {
    const __bf16 *p = s + (16 * vt + lr) * ld + 32 * kb + 4 * lg;
    const uint2 a = *reinterpret_cast<const uint2 *>(p), b = *reinterpret_cast<const uint2 *>(p + 16);
    return __builtin_bit_cast(mx::bf16x8, uint4{a.x, a.y, b.x, b.y});
}
// Across the rows, by transposing reads: column 16 m + lr, rows kperm(lg, e) of the 32 from s.  As an A
// operand, rows 16 m .. of the transpose; as a B operand, reduction over the rows.
__device__ __forceinline__ mx::bf16x8 vals_operand(const __bf16 *s, int ld, int m, int lr, int lg) {
    const __bf16 *p = s + (4 * lg + (lr >> 2)) * ld + 16 * m + 4 * (lr & 3);
    const mx::bf16x4 a = mx::lds_read_tr(p), c = mx::lds_read_tr(p + 16 * ld);
    return mx::bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
}
// A D tile (rows 16 m + 4 lg + r, value column 16 vt + lr) into a [value][row] array as bf16 hi and lo.
__device__ __forceinline__ void store_tile(__bf16 *hi, __bf16 *lo, int m, int vt, f32x4 d, int lr, int lg) {
    uint32_t h0, l0, h1, l1;
    mx::split2(d[0], d[1], h0, l0);
    mx::split2(d[2], d[3], h1, l1);
    const int off = (16 * vt + lr) * kLST + 16 * m + 4 * lg;
    *reinterpret_cast<uint2 *>(hi + off) = uint2{h0, h1};
    *reinterpret_cast<uint2 *>(lo + off) = uint2{l0, l1};
}
__device__ __forceinline__ f32x4 mma3(mx::bf16x8 ah, mx::bf16x8 al, mx::bf16x8 bh, mx::bf16x8 bl, f32x4 c) {
    c = mx::mma(ah, bh, c);
    c = mx::mma(ah, bl, c);
    return mx::mma(al, bh, c);
}
__device__ __forceinline__ mx::bf16x8 neg8(mx::bf16x8 x) {
    uint4 u = __builtin_bit_cast(uint4, x);
    u.x ^= 0x80008000u;
    u.y ^= 0x80008000u;
    u.z ^= 0x80008000u;
    u.w ^= 0x80008000u;
    return __builtin_bit_cast(mx::bf16x8, u);
}

constexpr int kThreads16 = 512;  // eight wavefronts

__global__ __launch_bounds__(kThreads16, 1) void bwd_grads16_kernel(
    const __bf16 *__restrict__ v, const float *__restrict__ dO, const __bf16 *__restrict__ kin,
    const __bf16 *__restrict__ qin, int T, int H, int NC, float eps, float scale, const float *__restrict__ wT,
    const float *__restrict__ wG, const float *__restrict__ wB, const char *__restrict__ rec,
    const char *__restrict__ rrev,
    const float *__restrict__ wS, const float *__restrict__ wdS, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta, bool delta, bool kaczmarz,
    SeqTable tb) {
    using mx::bf16x8;
    constexpr int DK = mx::DK, DV = mx::DV, JH = DK / 32;  // channel tiles per half
    const int ci = blockIdx.x;
    if (!slot_used(ci, H, tb)) return;
    const Slot sl = slot_of(ci, T, H, NC, tb);
    const int n = sl.n;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wv & 3, h = wv >> 2;  // token rows 16 w .., value tile h of a slice, channel tiles 4 h ..
    const int lr = lane & 15, lg = lane >> 4;
    __shared__ GradsSmem sm;
    const size_t row0u = uniform(sl.row0);
    const int nu = uniform(n);
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    // this wavefront's k rows as the A operand over channels: kA[kb] = k[16 w + lr][32 kb + kperm(lg, e)]
    bf16x8 kA[4];
    {
        const auto rk = rows_rsrc(kin + row0u * DK, nu, H * DK * 2, DK * 2);
        const int base = (16 * w + lr) * H * DK + 4 * lg;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const auto a = __builtin_amdgcn_raw_buffer_load_b64(rk, (base + 32 * kb) * 2, 0, 0);
            const auto b = __builtin_amdgcn_raw_buffer_load_b64(rk, (base + 32 * kb + 16) * 2, 0, 0);
            kA[kb] = __builtin_bit_cast(bf16x8, uint4{a[0], a[1], b[0], b[1]});
        }
    }
    // token factors of this lane's D-tile rows and the record fragments of rows 16 w ..: T'' (lower,
    // token blocks kb <= w / 2), T''' and A' (upper, kb >= w / 2); every load issued, unused ones unread
    const char *rc = rec + (size_t)ci * mx::kRecBytes;
    const char *rr = rrev + (size_t)ci * kRevBytes;
    const f32x4 gam = *reinterpret_cast<const f32x4 *>(rc + mx::kRecGam + (16 * w + 4 * lg) * 4);
    const f32x4 gnd = *reinterpret_cast<const f32x4 *>(rc + mx::kRecGend + (16 * w + 4 * lg) * 4);
    bf16x8 tlh[2], tll[2], tuh[2], tul[2], auh[2], aul[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int fl = mx::lower_frag(w, min(kb, w >> 1)), fu = upper_frag(w, max(kb, w >> 1));
        tlh[kb] = *reinterpret_cast<const bf16x8 *>(rc + mx::kRecTH + fl * mx::kFragBytes + lane * 16);
        tll[kb] = *reinterpret_cast<const bf16x8 *>(rc + mx::kRecTL + fl * mx::kFragBytes + lane * 16);
        tuh[kb] = *reinterpret_cast<const bf16x8 *>(rr + kRevTH + fu * mx::kFragBytes + lane * 16);
        tul[kb] = *reinterpret_cast<const bf16x8 *>(rr + kRevTL + fu * mx::kFragBytes + lane * 16);
        auh[kb] = *reinterpret_cast<const bf16x8 *>(rr + kRevAH + fu * mx::kFragBytes + lane * 16);
        aul[kb] = *reinterpret_cast<const bf16x8 *>(rr + kRevAL + fu * mx::kFragBytes + lane * 16);
    }

    // channel tiles 4 h + J of dQ~, dK~, dK^; dA (h = 0) or dT'' (h = 1), token tiles J <= w
    f32x4 aQ[JH], aKt[JH], aKh[JH], aM[4];
#pragma unroll
    for (int J = 0; J < JH; ++J) aQ[J] = aKt[J] = aKh[J] = z4;
#pragma unroll
    for (int J = 0; J < 4; ++J) aM[J] = z4;

    // slice loads, 16 bytes per lane: thread t takes values j0 + 4 (t % 8) .. +3 of key channels t / 8 and
    // 64 + t / 8 (S, dS') and of token t / 8 (dO); v in this wavefront's D-tile layout (value tile h)
    const int sq = 4 * (tid & 7), sr = tid >> 3;
    const float *Sg = wS + (size_t)ci * DK * DV, *dSg = wdS + (size_t)ci * DK * DV;
    const auto r_o = rows_rsrc(dO + row0u * DV, nu, H * DV * 4, DV * 4);
    const auto r_v = rows_rsrc(v + row0u * DV, nu, H * DV * 2, DV * 2);
    const auto r_dv = rows_rsrc(dv + row0u * DV, nu, H * DV * 4, DV * 4);
    f32x4 rS[2], rdS[2], rO, rV;
    float gpart[2] = {0.f, 0.f};
    auto fetch = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            rS[u] = *reinterpret_cast<const f32x4 *>(&Sg[(sr + 64 * u) * DV + j0 + sq]);
            rdS[u] = *reinterpret_cast<const f32x4 *>(&dSg[(sr + 64 * u) * DV + j0 + sq]);
        }
        rO = __builtin_bit_cast(f32x4, mx::buf_ld16(r_o, (sr * H * DV + j0 + sq) * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) rV[r] = buf_in<true>(r_v, (16 * w + 4 * lg + r) * H * DV + j0 + 16 * h + lr);
    };
    auto stage4 = [&](__bf16 *hi, __bf16 *lo, int off, f32x4 x) __attribute__((always_inline)) {
        uint32_t h0, l0, h1, l1;
        mx::split2(x[0], x[1], h0, l0);
        mx::split2(x[2], x[3], h1, l1);
        *reinterpret_cast<uint2 *>(hi + off) = uint2{h0, h1};
        *reinterpret_cast<uint2 *>(lo + off) = uint2{l0, l1};
    };
    fetch(0);
    for (int j0 = 0; j0 < DV; j0 += kSW) {
        if (j0) barrier_lds();  // the previous slice's operands are no longer read
        // ---- the slice's S, dS' and dO to LDS as bf16 hi, lo; the next slice's loads
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int off = (sr + 64 * u) * kLSV + sq;
            stage4(sm.u.a.S[0], sm.u.a.S[1], off, rS[u]);
            stage4(sm.u.a.dS[0], sm.u.a.dS[1], off, rdS[u]);
            const f32x4 pr = rdS[u] * rS[u];
            gpart[u] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        }
        stage4(sm.u.a.O[0], sm.u.a.O[1], sr * kLSV + sq, rO);
        const f32x4 vv = rV;
        fetch(min(j0 + kSW, DV - kSW));
        barrier_lds();
        // ---- X = V - exp(G) (k S),  dE = exp(G_63 - G) (k dS') + A' dO  (value tile h)
        f32x4 x, de;
        {
            const int vt = h;
            f32x4 ps = z4, pd = z4;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int rb = 32 * kb * kLSV;  // key channels 32 kb ..
                if (delta) {
                    ps = mx::mma(kA[kb], vals_operand(sm.u.a.S[0] + rb, kLSV, vt, lr, lg), ps);
                    ps = mx::mma(kA[kb], vals_operand(sm.u.a.S[1] + rb, kLSV, vt, lr, lg), ps);
                }
                pd = mx::mma(kA[kb], vals_operand(sm.u.a.dS[0] + rb, kLSV, vt, lr, lg), pd);
                pd = mx::mma(kA[kb], vals_operand(sm.u.a.dS[1] + rb, kLSV, vt, lr, lg), pd);
            }
            de = gnd * pd;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb >= (w >> 1))
                    de = mma3(auh[kb], aul[kb], vals_operand(sm.u.a.O[0] + 32 * kb * kLSV, kLSV, vt, lr, lg),
                              vals_operand(sm.u.a.O[1] + 32 * kb * kLSV, kLSV, vt, lr, lg), de);
            x = vv - gam * ps;
            store_tile(sm.u.a.X[0], sm.u.a.X[1], w, vt, x, lr, lg);
            store_tile(sm.u.a.dE[0], sm.u.a.dE[1], w, vt, de, lr, lg);
        }
        barrier_lds();
        // ---- E = T'' X (token blocks kb <= w / 2),  dX = T''' dE (kb >= w / 2) = dV  (value tile h);
        // without the delta rule T'' = I (E = X = V, dX = dE)
        {
            const int vt = h;
            f32x4 ee = delta ? z4 : x, dx = delta ? z4 : de;
#pragma unroll
            for (int kb = 0; kb < 2 && delta; ++kb) {
                if (kb <= (w >> 1))
                    ee = mma3(tlh[kb], tll[kb], rows_operand(sm.u.a.X[0], kLST, vt, kb, lr, lg),
                              rows_operand(sm.u.a.X[1], kLST, vt, kb, lr, lg), ee);
                if (kb >= (w >> 1))
                    dx = mma3(tuh[kb], tul[kb], rows_operand(sm.u.a.dE[0], kLST, vt, kb, lr, lg),
                              rows_operand(sm.u.a.dE[1], kLST, vt, kb, lr, lg), dx);
            }
            store_tile(sm.u.a.E[0], sm.u.a.E[1], w, vt, ee, lr, lg);
            store_tile(sm.u.a.dX[0], sm.u.a.dX[1], w, vt, dx, lr, lg);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dx[r]), r_dv,
                                                      ((16 * w + 4 * lg + r) * H * DV + j0 + 16 * vt + lr) * 4, 0, 0);
        }
        barrier_lds();
        // ---- over the slice's values: dQ~ += dO S',  dK~ -= dX S',  dK^ += E dS'' (channel tiles 4 h ..);
        // dA += dO E' (h = 0) or dT'' += dE X' (h = 1)
        {
            const bf16x8 oh = rows_operand(sm.u.a.O[0], kLSV, w, 0, lr, lg), ol = rows_operand(sm.u.a.O[1], kLSV, w, 0, lr, lg);
            const bf16x8 eh = vals_operand(sm.u.a.E[0], kLST, w, lr, lg), el = vals_operand(sm.u.a.E[1], kLST, w, lr, lg);
            const bf16x8 xh = neg8(vals_operand(sm.u.a.dX[0], kLST, w, lr, lg));
            const bf16x8 xl = neg8(vals_operand(sm.u.a.dX[1], kLST, w, lr, lg));
#pragma unroll
            for (int J = 0; J < JH; ++J) {
                const int jc = JH * h + J;
                const bf16x8 sh = rows_operand(sm.u.a.S[0], kLSV, jc, 0, lr, lg), slo = rows_operand(sm.u.a.S[1], kLSV, jc, 0, lr, lg);
                const bf16x8 th = rows_operand(sm.u.a.dS[0], kLSV, jc, 0, lr, lg), tl = rows_operand(sm.u.a.dS[1], kLSV, jc, 0, lr, lg);
                aQ[J] = mma3(oh, ol, sh, slo, aQ[J]);
                if (delta) aKt[J] = mma3(xh, xl, sh, slo, aKt[J]);
                aKh[J] = mma3(eh, el, th, tl, aKh[J]);
            }
            if (h == 0) {
#pragma unroll
                for (int J = 0; J < 4; ++J)
                    if (J <= w)
                        aM[J] = mma3(oh, ol, vals_operand(sm.u.a.E[0], kLST, J, lr, lg),
                                     vals_operand(sm.u.a.E[1], kLST, J, lr, lg), aM[J]);
            } else if (delta) {
                const bf16x8 dh = vals_operand(sm.u.a.dE[0], kLST, w, lr, lg), dl = vals_operand(sm.u.a.dE[1], kLST, w, lr, lg);
#pragma unroll
                for (int J = 0; J < 4; ++J)
                    if (J <= w)
                        aM[J] = mma3(dh, dl, vals_operand(sm.u.a.X[0], kLST, J, lr, lg),
                                     vals_operand(sm.u.a.X[1], kLST, J, lr, lg), aM[J]);
            }
        }
    }
    // dgam per channel: this thread's sums over its values, then over the eight threads of a channel
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float s = gpart[u];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        if (sq == 0) sm.gsum[sr + 64 * u] = s;
    }

    // ===================== the chunk's triangular algebra and pair terms, on this workgroup
    // (in LDS from here on: T, dT'' -> dT -> dR -> W2, Y, dA with dM' above the diagonal, M, A -> W1 in T's
    // place once T is read, the bf16 rows of k and q; G, beta, dbeta, |k|^2, dG)
    constexpr int NCC = C * C / kThreads16;  // C x C values per thread
    float rT[NCC];
    uint4 rk[2], rq[2];
    {
        const float *Tg = wT + (size_t)ci * C * C;
#pragma unroll
        for (int u = 0; u < NCC; ++u) rT[u] = Tg[tid + u * kThreads16];
        const auto rkb = rows_rsrc(kin + row0u * DK, nu, H * DK * 2, DK * 2);
        const auto rqb = rows_rsrc(qin + row0u * DK, nu, H * DK * 2, DK * 2);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = tid + u * kThreads16, r = idx >> 4, c0 = (idx & 15) * 8;
            rk[u] = mx::buf_ld16(rkb, (r * H * DK + c0) * 2);
            rq[u] = mx::buf_ld16(rqb, (r * H * DK + c0) * 2);
        }
    }
    barrier_lds();  // every wavefront is done with the slice operands
    float *sT = sm.u.b.T, *sX = sm.u.b.X, *sY = sm.u.b.Y, *sD = sm.u.b.D, *sMm = sm.u.b.M, *sAa = sm.u.b.A;
    __bf16 *sKb = sm.u.b.K, *sQb = sm.u.b.Q;
#pragma unroll
    for (int J = 0; J < 4; ++J)  // dA (h = 0) into sD, dT'' (h = 1) into sX: lower triangle incl. the diagonal
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lg + r, m = 16 * J + lr;
            (h == 0 ? sD : sX)[i * kLCB + m] = m <= i ? aM[J][r] : 0.f;
        }
#pragma unroll
    for (int u = 0; u < NCC; ++u) {
        const int idx = tid + u * kThreads16, r = idx / C, cc = idx % C;
        sT[r * kLCB + cc] = rT[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int idx = tid + u * kThreads16, r = idx >> 4, c0 = (idx & 15) * 8;
        *reinterpret_cast<uint4 *>(&sKb[r * kLQB + c0]) = rk[u];
        *reinterpret_cast<uint4 *>(&sQb[r * kLQB + c0]) = rq[u];
    }
    if (tid < C) {
        sm.G[tid] = wG[(size_t)ci * C + tid];
        sm.beta[tid] = wB[(size_t)ci * C + tid];
    }
    barrier_lds();
    {  // M_ij = (k k')_ij exp(G_i - G_j), j < i (h = 0), and A_ij = scale (q k')_ij exp(G_i - G_j), j <= i
       // (h = 1): rows 16 w .., column tiles J <= w; exact bf16 products (only the lower parts are read)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J > w) continue;
            f32x4 acc = z4;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc = mx::mma(h == 0 ? kA[kb] : rows_operand(sQb, kLQB, w, kb, lr, lg),
                              rows_operand(sKb, kLQB, J, kb, lr, lg), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r, j = 16 * J + lr;
                const float p = j <= i ? __expf(sm.G[i] - sm.G[j]) : 0.f;
                if (h == 0) sMm[i * kLCB + j] = delta && j < i ? acc[r] * p : 0.f;
                else sAa[i * kLCB + j] = scale * acc[r] * p;
            }
        }
    }
    // parts of dG through Q~, K~, K^ (rows 16 w .., channel tiles 4 h ..): dK~ K~ + dQ~ Q~ - dK^ K^ summed
    // over the channels, and for G_63 the column sums of dK^ K^; dbeta_j = sum_i dT''_ij T_ij
    auto kval = [&](int r, int c) { return static_cast<float>(sKb[r * kLQB + c]); };
    {
        float rowpart[4] = {0.f, 0.f, 0.f, 0.f};
        float colh[JH];
#pragma unroll
        for (int J = 0; J < JH; ++J) {
            colh[J] = 0.f;
            const int ch = 16 * (JH * h + J) + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r;
                const float ei = gam[r], eh = gnd[r];
                const float kv = kval(i, ch), qv = static_cast<float>(sQb[i * kLQB + ch]);
                const float khv = eh * kv;
                rowpart[r] += aKt[J][r] * (ei * kv) + aQ[J][r] * (scale * ei * qv) - aKh[J][r] * khv;
                colh[J] += aKh[J][r] * khv;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // sum over the 16 lanes of a row group; the halves meet in LDS
            float sum = rowpart[r];
            sum += __shfl_xor(sum, 1, 64);
            sum += __shfl_xor(sum, 2, 64);
            sum += __shfl_xor(sum, 4, 64);
            sum += __shfl_xor(sum, 8, 64);
            if (lr == 0) sm.rowp[h][16 * w + 4 * lg + r] = sum;
        }
#pragma unroll
        for (int J = 0; J < JH; ++J) {
            float sum = colh[J];
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            if (lg == 0) sm.H[w][16 * (JH * h + J) + lr] = sum;
        }
        if (tid < kThreads) {  // four lanes per column (every fourth row each), then a sum over the quad
            const int j = tid >> 2, q4 = tid & 3;
            float s = 0.f;
            for (int r = j + q4; r < C; r += 4) s += sX[r * kLCB + j] * sT[r * kLCB + j];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if (q4 == 0) sm.dbeta[j] = s;
        }
    }
    barrier_lds();
    // dG of the tokens; the chunk-end decay's extra (per channel, then over channels below); dT = dT'' Diag(beta)
    if (tid < C) sm.dG[tid] = sm.rowp[0][tid] + sm.rowp[1][tid];
    if (tid < DK) {
        const float ge = sm.G[C - 1];
        sm.H[0][tid] = ((sm.H[0][tid] + sm.H[1][tid]) + (sm.H[2][tid] + sm.H[3][tid])) + sm.gsum[tid] * __expf(ge);
    }
    for (int idx = tid; idx < C * C; idx += kThreads16) {
        const int r = idx / C, cc = idx % C;
        sX[r * kLCB + cc] *= sm.beta[cc];
    }
    barrier_lds();
    if (wv == 0) {  // the sum over channels, to the last token's dG
        float s = 0.f;
        for (int cc = lane; cc < DK; cc += 64) s += sm.H[0][cc];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (lane == 0) sm.dG[C - 1] += s;
    }
    {  // Y = T' dT: rows 16 w .., column tiles 2 h, 2 h + 1
        f32x4 y[2] = {z4, z4};
        for (int kk = 0; kk < C; kk += 4) {
            const float a = sT[(kk + lg) * kLCB + 16 * w + lr];
#pragma unroll
            for (int J = 0; J < 2; ++J) y[J] = mfma4(a, sX[(kk + lg) * kLCB + 16 * (2 * h + J) + lr], y[J]);
        }
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) sY[(16 * w + 4 * lg + r) * kLCB + 16 * (2 * h + J) + lr] = y[J][r];
    }
    barrier_lds();
    {  // -dR = Y T': rows 16 w .., column tiles 2 h, 2 h + 1; dR (strictly lower) over dT
        f32x4 d[2] = {z4, z4};
        for (int kk = 0; kk < C; kk += 4) {
            const float a = sY[(16 * w + lr) * kLCB + kk + lg];
#pragma unroll
            for (int J = 0; J < 2; ++J) d[J] = mfma4(a, sT[(16 * (2 * h + J) + lr) * kLCB + kk + lg], d[J]);
        }
        barrier_lds();  // dT and Y no longer read
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r, j = 16 * (2 * h + J) + lr;
                sX[i * kLCB + j] = j < i ? -d[J][r] : 0.f;
            }
    }
    barrier_lds();
    // dbeta_i += sum_{j<i} dR_ij M_ij;  dM_ij = beta_i dR_ij -> sD[j][i] (j < i)
    if (tid < kThreads) {
        const int r = tid >> 2, q4 = tid & 3;
        float s = 0.f;
        for (int cc = q4; cc < r; cc += 4) s += sX[r * kLCB + cc] * sMm[r * kLCB + cc];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q4 == 0) sm.dbeta[r] += s;
    }
    for (int idx = tid; idx < C * C; idx += kThreads16) {
        const int r = idx / C, cc = idx % C;
        if (cc < r) sD[cc * kLCB + r] = sm.beta[r] * sX[r * kLCB + cc];
    }
    barrier_lds();
    // dG_i += rowsum_i(Z) - colsum_i(Z), Z = dM o M + dA o A;  W1 = dM o P over T, W2 = scale dA o P over
    // dR (P_ij = exp(G_i - G_j), j <= i);  |k_i|^2 for the Kaczmarz step size
    if (tid < kThreads) {
        const int r = tid >> 2, q4 = tid & 3;
        float s = 0.f;
        for (int j = q4; j < r; j += 4) s += sD[j * kLCB + r] * sMm[r * kLCB + j];
        for (int j = q4; j <= r; j += 4) s += sD[r * kLCB + j] * sAa[r * kLCB + j];
        for (int i = r + 1 + q4; i < C; i += 4) s -= sD[r * kLCB + i] * sMm[i * kLCB + r];
        for (int i = r + q4; i < C; i += 4) s -= sD[i * kLCB + r] * sAa[i * kLCB + r];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q4 == 0) sm.dG[r] += s;
    } else if (kaczmarz) {
        const int r = (tid - kThreads) >> 2, q4 = tid & 3;
        float s = 0.f;
        for (int cc = q4; cc < DK; cc += 4) s += kval(r, cc) * kval(r, cc);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q4 == 0) sm.kk[r] = s;
    }
    for (int idx = tid; idx < C * C; idx += kThreads16) {
        const int i = idx / C, j = idx % C;
        const float p = j <= i ? __expf(sm.G[i] - sm.G[j]) : 0.f;
        sT[i * kLCB + j] = j < i ? sD[j * kLCB + i] * p : 0.f;
        sX[i * kLCB + j] = scale * sD[i * kLCB + j] * p;  // zero above the diagonal
    }
    barrier_lds();
    // pair terms, rows 16 w .., channel tiles 4 h ..: dk += W1 K + W1' K + W2' Q, dq += W2 K, on bf16 tiles
    // (W1 + W1', W2', W2 split into hi + lo over token block kb; k, q exact, by transposing reads)
    {
        f32x4 pk[JH], pq[JH];
#pragma unroll
        for (int J = 0; J < JH; ++J) pk[J] = pq[J] = z4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float ak[8], aq[8], ad[8];
            const int i = 16 * w + lr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 32 * kb + mx::kperm(lg, e);
                ak[e] = sT[i * kLCB + j] + sT[j * kLCB + i];  // W1 + W1'
                aq[e] = sX[j * kLCB + i];                     // W2'
                ad[e] = sX[i * kLCB + j];                     // W2
            }
            bf16x8 akh, akl, aqh, aql, adh, adl;
            mx::split8(ak, akh, akl);
            mx::split8(aq, aqh, aql);
            mx::split8(ad, adh, adl);
#pragma unroll
            for (int J = 0; J < JH; ++J) {
                const int jc = JH * h + J;
                const bf16x8 k8 = vals_operand(sKb + 32 * kb * kLQB, kLQB, jc, lr, lg);
                const bf16x8 q8 = vals_operand(sQb + 32 * kb * kLQB, kLQB, jc, lr, lg);
                pk[J] = mx::mma(akh, k8, pk[J]);
                pk[J] = mx::mma(akl, k8, pk[J]);
                pk[J] = mx::mma(aqh, q8, pk[J]);
                pk[J] = mx::mma(aql, q8, pk[J]);
                pq[J] = mx::mma(adh, k8, pq[J]);
                pq[J] = mx::mma(adl, k8, pq[J]);
            }
        }
        // dq, dk: the parts through Q~, K~, K^ and the pair terms (rows past the end are not written)
#pragma unroll
        for (int J = 0; J < JH; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r, ch = 16 * (JH * h + J) + lr;
                if (i < n) {
                    const size_t off = (sl.row0 + (size_t)i * H) * DK + ch;
                    float dkv = gam[r] * aKt[J][r] + gnd[r] * aKh[J][r] + pk[J][r];
                    if (kaczmarz) dkv += -2.f * sm.beta[i] * sm.dbeta[i] / (sm.kk[i] + eps) * kval(i, ch);
                    dk[off] = dkv;
                    dq[off] = scale * gam[r] * aQ[J][r] + pq[J][r];
                }
            }
    }
    // dg = the reverse cumulative sum of dG over the chunk's tokens (a suffix sum across one wavefront);
    // dbeta (deta for the Kaczmarz step size)
    if (wv == 0) {
        float run = sm.dG[lane];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_down(run, off, 64);
            if (lane + off < 64) run += up;
        }
        if (lane < n) dg[sl.row0 + (size_t)lane * H] = run;
    } else if (wv == 1 && dbeta && lane < n) {  // no beta without the delta rule
        float db = sm.dbeta[lane];
        if (kaczmarz) db /= (sm.kk[lane] + eps);
        dbeta[sl.row0 + (size_t)lane * H] = db;
    }
}

// ============================================================ grads B: triangular algebra and pair terms
// One workgroup per chunk, four wavefronts (wavefront w: rows 16w .. of the
// C x C and C x DK products, on fp32 matrix-core tiles).  dbeta from dT'';
// Y = T' dT, dR = -Y T' (strictly lower), dbeta += rowsum(dR o M), dM =
// Diag(beta) dR.  The pair terms of M and A: for scalar decay P_ij =
// exp(G_i - G_j) is one factor per pair, so with W1 = dM o P and W2 = scale
// dA o P they are products, dk += W1 K + W1' K + W2' Q, dq += W2 K, and dG_i
// = rowsum_i(Z) - colsum_i(Z) with Z = dM o M + dA o A; for per-channel decay
// P is split at a reference token per row block, as in the prep kernel.  Then the Kaczmarz step size and
// the reverse cumulative sum of dG.
template <int DK, bool PC, bool KZ, bool IN_BF16>
__global__ __launch_bounds__(kThreads, IN_BF16 && !PC ? 2 : 1) void bwd_grads_b_kernel(
    const void *__restrict__ q, const void *__restrict__ k, int T, int H, int NC, float eps, float scale,
    const float *__restrict__ wT, const float *__restrict__ wM, const float *__restrict__ wA,
    const float *__restrict__ wG, const float *__restrict__ wB, const float *__restrict__ wdA,
    const float *__restrict__ wdTT, const float *__restrict__ wdG, const float *__restrict__ wdG63,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dg, float *__restrict__ dbeta,
    SeqTable tb) {
    constexpr int GK = PC ? DK : 1;
    constexpr int LC = C + 1;                  // row stride of the C x C buffers
    constexpr int LQ = DK + 1;                 // row stride of the C x DK buffers
    constexpr int R0 = 0, R1 = C * LC, R2 = 2 * C * LC;  // three C x C regions
    // per-channel decay: k and q over the C x C regions once those are free; scalar decay: W1, W2
    // in regions 0 and 1, k from region 2 on, then q
    constexpr int KOFF = PC ? 0 : R2, QOFF = KOFF + C * LQ;
    // scalar decay with bf16 inputs: dA / dM' is a fourth C x C region, and k, q (exact in bf16) are
    // kept as bf16 over regions 2 and 3 once those are free, so two workgroups share a unit
    constexpr bool KQ16 = IN_BF16 && !PC;
    constexpr int LQB = DK + 16;  // bf16 row stride: rows 8 banks apart
    constexpr int R3 = 3 * C * LC;
    constexpr int KQ16_END = R2 + (C * LQB > 2 * C * LC ? C * LQB : 2 * C * LC);
    constexpr int kSmem = KQ16 ? KQ16_END : (QOFF + C * LQ > 3 * C * LC ? QOFF + C * LQ : 3 * C * LC);
    const int ci = blockIdx.x;
    if (!slot_used(ci, H, tb)) return;
    const Slot sl = slot_of(ci, T, H, NC, tb);
    const int n = sl.n;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    __shared__ float smem[kSmem];
    __shared__ float sDarr[KQ16 ? 1 : C * LC];
    float *sD = KQ16 ? smem + R3 : sDarr;  // dA (j <= i) and, in the strict upper part, dM transposed
    __shared__ float sG[C][GK];
    __shared__ float sBeta[C], sdBeta[C], sKK[C];
    __shared__ float sdG[C][GK];

    float *sT = smem + R0;   // T, then (scalar decay) A, then W1
    float *sX = smem + R1;   // dT'', dT, dR, then (scalar decay) W2
    float *sY = smem + R2;   // T' dT, then M
    const float *Tg = wT + (size_t)ci * C * C;
    const float *dAg = wdA + (size_t)ci * C * C, *dTg = wdTT + (size_t)ci * C * C;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
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
            sT[r * LC + cc] = rT[u];
            sD[r * LC + cc] = cc <= r ? rD[u] : 0.f;
            sX[r * LC + cc] = cc <= r ? rX[u] : 0.f;  // dT''
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
    {  // four lanes per column (every fourth row each), then a sum over the quad
        const int j = tid >> 2, q = tid & 3;
        float s = 0.f;
        for (int r = j + q; r < C; r += 4) s += sX[r * LC + j] * sT[r * LC + j];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q == 0) sdBeta[j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, cc = idx % C;
        sX[r * LC + cc] *= sBeta[cc];
    }
    __syncthreads();
    {  // Y = T' dT (rows 16w ..)
        f32x4 y[4] = {z4, z4, z4, z4};
        for (int kk = 0; kk < C; kk += 4) {
            const float a = sT[(kk + lg) * LC + 16 * w + lr];
#pragma unroll
            for (int J = 0; J < 4; ++J) y[J] = mfma4(a, sX[(kk + lg) * LC + 16 * J + lr], y[J]);
        }
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) sY[(16 * w + 4 * lg + r) * LC + 16 * J + lr] = y[J][r];
    }
    __syncthreads();
    f32x4 d[4] = {z4, z4, z4, z4};  // -dR = Y T' (rows 16w ..)
    for (int kk = 0; kk < C; kk += 4) {
        const float a = sY[(16 * w + lr) * LC + kk + lg];
#pragma unroll
        for (int J = 0; J < 4; ++J) d[J] = mfma4(a, sT[(16 * J + lr) * LC + kk + lg], d[J]);
    }
    __syncthreads();  // Y, T and dT no longer read
    const float *Mg = wM + (size_t)ci * C * C;
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lg + r, j = 16 * J + lr;
            sX[i * LC + j] = j < i ? -d[J][r] : 0.f;  // dR, strictly lower
        }
    for (int idx = tid; idx < C * C; idx += kThreads) sY[(idx / C) * LC + idx % C] = Mg[idx];
    if constexpr (!PC) {  // A for the pair terms of scalar decay, in T's place
        const float *Ag = wA + (size_t)ci * C * C;
        for (int idx = tid; idx < C * C; idx += kThreads) sT[(idx / C) * LC + idx % C] = Ag[idx];
    }
    __syncthreads();
    // dbeta_i += sum_{j<i} dR_ij M_ij;  dM_ij = beta_i dR_ij -> sD[j][i] (j < i)
    {  // four lanes per row, then a sum over the quad
        const int r = tid >> 2, q = tid & 3;
        float s = 0.f;
        for (int cc = q; cc < r; cc += 4) s += sX[r * LC + cc] * sY[r * LC + cc];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q == 0) sdBeta[r] += s;
    }
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, cc = idx % C;
        if (cc < r) sD[cc * LC + r] = sBeta[r] * sX[r * LC + cc];
    }
    __syncthreads();

    float(*sK)[LQ] = reinterpret_cast<float(*)[LQ]>(smem + KOFF);
    float(*sQ)[LQ] = reinterpret_cast<float(*)[LQ]>(smem + QOFF);
    __bf16 *sKb = reinterpret_cast<__bf16 *>(smem + R2), *sQb = sKb + C * LQB;
    auto kv = [&](int r, int c) -> float {
        if constexpr (KQ16) return static_cast<float>(sKb[r * LQB + c]);
        else return sK[r][c];
    };
    auto qv = [&](int r, int c) -> float {
        if constexpr (KQ16) return static_cast<float>(sQb[r * LQB + c]);
        else return sQ[r][c];
    };
    // raw k, q: the loads (16 bytes per lane, rows past the chunk's end zero through the buffer bounds)
    // are issued here and stored to LDS below
    constexpr int es = IN_BF16 ? 2 : 4, EPL = 16 / es, NL = C * DK / EPL / kThreads;
    uint4 rk[NL], rq[NL];
    {
        const size_t row0u = uniform(sl.row0);
        const int nu = uniform(n);
        const auto rkb = rows_rsrc(static_cast<const char *>(k) + row0u * DK * es, nu, H * DK * es, DK * es);
        const auto rqb = rows_rsrc(static_cast<const char *>(q) + row0u * DK * es, nu, H * DK * es, DK * es);
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int idx = tid + u * kThreads, r = idx / (DK / EPL), c0 = (idx % (DK / EPL)) * EPL;
            rk[u] = mx::buf_ld16(rkb, (r * H * DK + c0) * es);
            rq[u] = mx::buf_ld16(rqb, (r * H * DK + c0) * es);
        }
    }
    if constexpr (!PC) {
        // dG_i = rowsum_i(Z) - colsum_i(Z), Z = dM o M + dA o A (M in sY, A in sT)
        {  // four lanes per token r (every fourth term each), then a sum over the quad
            const int r = tid >> 2, q = tid & 3;
            float s = 0.f;
            for (int j = q; j < r; j += 4) s += sD[j * LC + r] * sY[r * LC + j];              // dM_rj M_rj
            for (int j = q; j <= r; j += 4) s += sD[r * LC + j] * sT[r * LC + j];             // dA_rj A_rj
            for (int i = r + 1 + q; i < C; i += 4) s -= sD[r * LC + i] * sY[i * LC + r];      // dM_ir M_ir
            for (int i = r + q; i < C; i += 4) s -= sD[i * LC + r] * sT[i * LC + r];          // dA_ir A_ir
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if (q == 0) sdG[r][0] += s;
        }
        __syncthreads();  // M, A no longer read
        // W1 = dM o P (region 0), W2 = scale dA o P (region 1), P_ij = exp(G_i - G_j), j <= i
        for (int idx = tid; idx < C * C; idx += kThreads) {
            const int i = idx / C, j = idx % C;
            const float p = j <= i ? __expf(sG[i][0] - sG[j][0]) : 0.f;
            sT[i * LC + j] = j < i ? sD[j * LC + i] * p : 0.f;
            sX[i * LC + j] = scale * sD[i * LC + j] * p;  // zero above the diagonal
        }
    }
    if constexpr (KQ16) {
        __syncthreads();  // M and dA / dM' are no longer read
#pragma unroll
        for (int u = 0; u < NL; ++u) {  // the bf16 rows as loaded (16-byte aligned: 288-byte rows)
            const int idx = tid + u * kThreads, r = idx / (DK / EPL), c0 = (idx % (DK / EPL)) * EPL;
            *reinterpret_cast<uint4 *>(&sKb[r * LQB + c0]) = rk[u];
            *reinterpret_cast<uint4 *>(&sQb[r * LQB + c0]) = rq[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int idx = tid + u * kThreads, r = idx / (DK / EPL), c0 = (idx % (DK / EPL)) * EPL;
            float kf[EPL], qf[EPL];
            unpack16<IN_BF16>(rk[u], kf);
            unpack16<IN_BF16>(rq[u], qf);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                sK[r][c0 + e] = kf[e];
                sQ[r][c0 + e] = qf[e];
            }
        }
    }
    __syncthreads();
    if constexpr (KZ) {  // |k_i|^2
        {  // four lanes per token, then a sum over the quad
            const int r = tid >> 2, q = tid & 3;
            float s = 0.f;
            for (int cc = q; cc < DK; cc += 4) s += kv(r, cc) * kv(r, cc);
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if (q == 0) sKK[r] = s;
        }
        __syncthreads();
    }
    if constexpr (!PC) {
        // dk += W1 K + W1' K + W2' Q,  dq += W2 K (rows 16w .., all channels)
        constexpr int JK = DK / 16;
        f32x4 pk[JK], pq[JK];
#pragma unroll
        for (int J = 0; J < JK; ++J) pk[J] = pq[J] = z4;
        if constexpr (KQ16) {
            // token j = 16 t + 4 lg + e in step (t, e): the four tokens of a lane group are one
            // transposing read of the bf16 rows of k and q (rows 16 t + 4 lg + e, column 16 J + lr), and
            // W1 + W1' is formed once per operand
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float ak[4], aq[4], ad[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * t + 4 * lg + e;
                    ak[e] = sT[(16 * w + lr) * LC + j] + sT[j * LC + 16 * w + lr];  // W1 + W1'
                    aq[e] = sX[j * LC + 16 * w + lr];                                 // W2'
                    ad[e] = sX[(16 * w + lr) * LC + j];                               // W2
                }
#pragma unroll
                for (int J = 0; J < JK; ++J) {
                    const int at = (16 * t + 4 * lg + (lr >> 2)) * LQB + 16 * J + 4 * (lr & 3);
                    const mx::bf16x4 k4 = mx::lds_read_tr(&sKb[at]);
                    const mx::bf16x4 q4 = mx::lds_read_tr(&sQb[at]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float kb = static_cast<float>(k4[e]), qb = static_cast<float>(q4[e]);
                        pk[J] = mfma4(ak[e], kb, pk[J]);
                        pk[J] = mfma4(aq[e], qb, pk[J]);
                        pq[J] = mfma4(ad[e], kb, pq[J]);
                    }
                }
            }
        } else {
            for (int kk = 0; kk < C; kk += 4) {
                const float w1 = sT[(16 * w + lr) * LC + kk + lg], w1t = sT[(kk + lg) * LC + 16 * w + lr];
                const float w2 = sX[(16 * w + lr) * LC + kk + lg], w2t = sX[(kk + lg) * LC + 16 * w + lr];
#pragma unroll
                for (int J = 0; J < JK; ++J) {
                    const float kb = kv(kk + lg, 16 * J + lr), qb = qv(kk + lg, 16 * J + lr);
                    pk[J] = mfma4(w1 + w1t, kb, pk[J]);
                    pk[J] = mfma4(w2t, qb, pk[J]);
                    pq[J] = mfma4(w2, kb, pq[J]);
                }
            }
        }
#pragma unroll
        for (int J = 0; J < JK; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r, ch = 16 * J + lr;
                if (i < n) {
                    const size_t off = (sl.row0 + (size_t)i * H) * DK + ch;
                    float dkv = dk[off] + pk[J][r];
                    if constexpr (KZ) dkv += -2.f * sBeta[i] * sdBeta[i] / (sKK[i] + eps) * kv(i, ch);
                    dk[off] = dkv;
                    dq[off] += pq[J][r];
                }
            }
    } else {
        // Per-channel pair terms on matrix-core tiles.  Wavefront w takes the rows i of block w and all
        // channels c:  U_ic = sum_{j<i} dM_ij k_jc P_ijc  and  V_ic = scale sum_{j<=i} dA_ij k_jc P_ijc  (its
        // rows of M and A), and Cl_ic = sum_{i2>=i} (dM_{i2 i} k_{i2 c} + scale dA_{i2 i} q_{i2 c}) P_{i2 i c}
        // (its columns); then dk += U + Cl, dq += V, dG += k (U - Cl) + q V.  P_ijc = exp(G_ic - G_jc) is
        // split at the reference token r = 16 I of the row block I of i: exp(G_ic - G_rc) (<= 1) scales the
        // product's rows (U, V) or operand (Cl), exp(G_rc - G_jc) its operand (U, V) or rows (Cl); both are
        // <= 1 off the diagonal, and the diagonal block is summed term by term when its span would overflow.
        constexpr int JC = DK / 16;
        const f32x4 zero = z4;
        f32x4 U[JC], V[JC], Cl[JC];
#pragma unroll
        for (int jc = 0; jc < JC; ++jc) U[jc] = V[jc] = Cl[jc] = zero;
        const int rw = 16 * w;  // first row of this wavefront's block
        float span = 0.f;
        for (int cc = lane; cc < DK; cc += 64) span = fmaxf(span, sG[rw][cc] - sG[rw + 15][cc]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
        const bool direct = span > kSpanMax;
        // U, V over the column blocks J <= w
        for (int J = 0; J <= w; ++J) {
            if (J == w && direct) continue;
            for (int kk = 0; kk < 16; kk += 4) {
                const int i = rw + lr, j = 16 * J + kk + lg;
                const float a1 = j < i ? sD[j * LC + i] : 0.f;           // dM_ij
                const float a2 = j <= i ? scale * sD[i * LC + j] : 0.f;  // scale dA_ij
#pragma unroll
                for (int jc = 0; jc < JC; ++jc) {
                    const int c = 16 * jc + lr;
                    const float b = sK[j][c] * __expf(sG[rw][c] - sG[j][c]);
                    U[jc] = mfma4(a1, b, U[jc]);
                    V[jc] = mfma4(a2, b, V[jc]);
                }
            }
        }
#pragma unroll
        for (int jc = 0; jc < JC; ++jc)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rw + 4 * lg + r, c = 16 * jc + lr;
                const float e = __expf(sG[i][c] - sG[rw][c]);
                U[jc][r] *= e;
                V[jc][r] *= e;
            }
        // Cl over the row blocks I >= w
        for (int I = w; I < 4; ++I) {
            if (I == w && direct) continue;
            const int ri = 16 * I;
            f32x4 Ck[JC];
#pragma unroll
            for (int jc = 0; jc < JC; ++jc) Ck[jc] = zero;
            for (int kk = 0; kk < 16; kk += 4) {
                const int j = rw + lr, i = ri + kk + lg;
                const float a1 = i > j ? sD[j * LC + i] : 0.f;           // dM_ij
                const float a2 = i >= j ? scale * sD[i * LC + j] : 0.f;  // scale dA_ij
#pragma unroll
                for (int jc = 0; jc < JC; ++jc) {
                    const int c = 16 * jc + lr;
                    const float e = __expf(sG[i][c] - sG[ri][c]);
                    Ck[jc] = mfma4(a1, sK[i][c] * e, Ck[jc]);
                    Ck[jc] = mfma4(a2, sQ[i][c] * e, Ck[jc]);
                }
            }
#pragma unroll
            for (int jc = 0; jc < JC; ++jc)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = rw + 4 * lg + r, c = 16 * jc + lr;
                    Cl[jc][r] += Ck[jc][r] * __expf(sG[ri][c] - sG[j][c]);
                }
        }
        if (direct) {  // the diagonal block term by term
#pragma unroll
            for (int jc = 0; jc < JC; ++jc)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = rw + 4 * lg + r, c = 16 * jc + lr;
                    const float gi = sG[i][c];
                    float u = 0.f, vq = 0.f, cl = 0.f;
                    for (int j = rw; j < rw + 16; ++j) {
                        if (j <= i) {  // i's row of M and A
                            const float p = __expf(gi - sG[j][c]) * sK[j][c];
                            if (j < i) u += sD[j * LC + i] * p;
                            vq += scale * sD[i * LC + j] * p;
                        }
                        if (j >= i) {  // i's column
                            const float p = __expf(sG[j][c] - gi);
                            const float a = j > i ? sD[i * LC + j] * sK[j][c] : 0.f;
                            cl += (a + scale * sD[j * LC + i] * sQ[j][c]) * p;
                        }
                    }
                    U[jc][r] += u;
                    V[jc][r] += vq;
                    Cl[jc][r] += cl;
                }
        }
#pragma unroll
        for (int jc = 0; jc < JC; ++jc)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rw + 4 * lg + r, c = 16 * jc + lr;
                const float ki = sK[i][c];
                sdG[i][c] += ki * (U[jc][r] - Cl[jc][r]) + sQ[i][c] * V[jc][r];  // each lane its own entries
                if (i < n) {
                    const size_t off = (sl.row0 + (size_t)i * H) * DK + c;
                    float dkv = dk[off] + U[jc][r] + Cl[jc][r];
                    if constexpr (KZ) dkv += -2.f * sBeta[i] * sdBeta[i] / (sKK[i] + eps) * ki;
                    dk[off] = dkv;
                    dq[off] += V[jc][r];
                }
            }
    }
    __syncthreads();
    // dg = reverse cumulative sum of dG over the chunk's tokens; dbeta (deta)
    if constexpr (PC) {  // one channel per thread
        if (tid < GK) {
            float run = 0.f;
            for (int r = C - 1; r >= 0; --r) {
                run += sdG[r][tid];
                if (r < n) dg[(sl.row0 + (size_t)r * H) * GK + tid] = run;
            }
        }
    } else if (w == 0) {  // one token per lane: a suffix sum across the wavefront
        float run = sdG[lane][0];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_down(run, off, 64);
            if (lane + off < 64) run += up;
        }
        if (lane < n) dg[sl.row0 + (size_t)lane * H] = run;
    }
    if (dbeta && tid < C && tid < n) {  // no beta without the delta rule
        float db = sdBeta[tid];
        if constexpr (KZ) db /= (sKK[tid] + eps);
        dbeta[sl.row0 + (size_t)tid * H] = db;
    }
}

// ============================================================ forward pass on fp32 tiles
// The chunked forward pass for the inputs the bf16 matrix-core kernels do not
// take (fp32 q/k/v, or d_k or d_v = 64): the prep kernel above forms the
// per-chunk T, A and decayed operands, then this walk, which is the forward
// walk above with the chunk's outputs O = Q~ S + A E formed before the state
// moves on (Q~ S with the entering state, the diagonal of A kept: read after
// write), and the final state written once instead of every entering state.
// fp32 operands and accumulation throughout, as the vector-ALU kernels.
// Q~ and A come straight from the workspace into registers at the start of
// each chunk (the LDS holds the walk's own operands): lane (lr, lg) of
// wavefront w holds row 16 w + lr of each, columns 16 t + 4 lg + e
// (t = 0.., e = 0..3) as float4s, which is the reduction order of its
// products: step (t, e) of a product takes reduction index 16 t + 4 lg + e
// from lane group lg on both operands.
template <int DK, int DV, bool PC, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void fwd_tile_walk_kernel(
    const void *__restrict__ v, int T, int H, int NC, const float *__restrict__ wT, const float *__restrict__ wA,
    const float *__restrict__ wG, const float *__restrict__ wB, const float *__restrict__ wKt,
    const float *__restrict__ wKh, const float *__restrict__ wQt, const float *__restrict__ s0,
    void *__restrict__ o, float *__restrict__ s_final, bool delta, SeqTable tb) {
    constexpr int GK = PC ? DK : 1;
    constexpr int NT = DV / kBV;
    constexpr int NTT = C * C / kThreads, NKK = C * DK / kThreads;
    constexpr int SRB = DK / 64;  // state row blocks per wavefront
    constexpr int NQ = DK / 16;   // float4 groups of a Q~ row per lane
    // XCD-aware placement: the value slices of one (sequence, head) share an XCD, so its L2 serves the
    // chunk operands they all read
    int bh, tile;
    state_slot(blockIdx.x, gridDim.x / NT, NT, bh, tile);
    bh = walk_seq(bh, H, tb);  // packed batches: longest sequences first
    const BwdWalk wk = bwd_walk(bh, T, H, NC, tb);
    const int j0 = tile * kBV;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    __shared__ float sS[DK * kLB];
    __shared__ float sKt[C * kLK];
    __shared__ float sKh[C * kLKT];
    __shared__ float sT[C * kLT];     // T'' = T Diag(beta)
    __shared__ float sX[C * kLB];
    __shared__ float sE[C * kLB];
    __shared__ float sBeta[C], sGam[DK];

    float rT[NTT], rKt[NKK], rKh[NKK], rB = 0.f, rGam = 0.f;
    f32x4 rV[2];  // the v slice in the layout of this wavefront's X tiles
    auto fetch = [&](int c) {
        const size_t ci = wk.slot(c);
        const int n = wk.count(c);
        const size_t row0 = wk.row0(c);
#pragma unroll
        for (int u = 0; u < NTT; ++u) rT[u] = wT[ci * C * C + tid + u * kThreads];
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            rKt[u] = wKt[ci * C * DK + tid + u * kThreads];
            rKh[u] = wKh[ci * C * DK + tid + u * kThreads];
        }
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r;
                rV[J][r] = i < n ? load_in<IN_BF16>(v, (row0 + (size_t)i * H) * DV + j0 + 16 * J + lr) : 0.f;
            }
        if (tid < C) rB = wB[ci * C + tid];
        if (tid < DK) rGam = __expf(wG[ci * C * GK + (size_t)(C - 1) * GK + (PC ? tid : 0)]);
    };

    const size_t sbase = (size_t)bh * DK * DV;
    for (int idx = tid; idx < DK * kBV; idx += kThreads) {
        const int r = idx / kBV, cc = idx % kBV;
        sS[r * kLB + cc] = s0 ? s0[sbase + (size_t)r * DV + j0 + cc] : 0.f;
    }
    if (wk.nc > 0) fetch(0);
    for (int c = 0; c < wk.nc; ++c) {
        const size_t ci = wk.slot(c);
        const int n = wk.count(c);
        const size_t row0 = wk.row0(c);
        // this chunk's Q~ and A rows (only the blocks on or below the diagonal of A)
        f32x4 rQ[NQ], rA[4];
        const float *qrow = wQt + ci * C * DK + (size_t)(16 * w + lr) * DK + 4 * lg;
        const float *arow = wA + ci * C * C + (size_t)(16 * w + lr) * C + 4 * lg;
#pragma unroll
        for (int t = 0; t < NQ; ++t) rQ[t] = *reinterpret_cast<const f32x4 *>(qrow + 16 * t);
#pragma unroll
        for (int t = 0; t < 4; ++t) rA[t] = t <= w ? *reinterpret_cast<const f32x4 *>(arow + 16 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();  // the previous chunk's reads are done; sS holds the entering state
        if (tid < C) sBeta[tid] = rB;
        if (tid < DK) sGam[tid] = rGam;
#pragma unroll
        for (int u = 0; u < NKK; ++u) {
            const int idx = tid + u * kThreads;
            sKt[(idx / DK) * kLK + idx % DK] = rKt[u];
            sKh[(idx / DK) * kLKT + idx % DK] = rKh[u];
        }
        __syncthreads();  // sBeta
#pragma unroll
        for (int u = 0; u < NTT; ++u) {
            const int idx = tid + u * kThreads, i = idx / C, m = idx % C;
            sT[i * kLT + m] = rT[u] * sBeta[m];
        }
        f32x4 x[2] = {rV[0], rV[1]};
        if (c + 1 < wk.nc) fetch(c + 1);
        // X = V - K~ S (rows 16w ..; X = V without the delta rule)
        for (int kk = 0; delta && kk < DK; kk += 4) {
            const float a = -sKt[(16 * w + lr) * kLK + kk + lg];
#pragma unroll
            for (int J = 0; J < 2; ++J) x[J] = mfma4(a, sS[(kk + lg) * kLB + 16 * J + lr], x[J]);
        }
        // the read of the entering state, Q~ S (rows 16w ..)
        f32x4 oo[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < NQ; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int J = 0; J < 2; ++J)
                    oo[J] = mfma4(rQ[t][e], sS[(16 * t + 4 * lg + e) * kLB + 16 * J + lr], oo[J]);
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[(16 * w + 4 * lg + r) * kLB + 16 * J + lr] = x[J][r];
        __syncthreads();  // X, T''
        f32x4 e[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        for (int kk = 0; kk < 16 * (w + 1); kk += 4) {  // T'' is lower triangular
            const float a = sT[(16 * w + lr) * kLT + kk + lg];
#pragma unroll
            for (int J = 0; J < 2; ++J) e[J] = mfma4(a, sX[(kk + lg) * kLB + 16 * J + lr], e[J]);
        }
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) sE[(16 * w + 4 * lg + r) * kLB + 16 * J + lr] = e[J][r];
        __syncthreads();  // E
        // the in-chunk read A E (A lower triangular, diagonal kept), then the outputs
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t > w) break;
#pragma unroll
            for (int ee = 0; ee < 4; ++ee)
#pragma unroll
                for (int J = 0; J < 2; ++J)
                    oo[J] = mfma4(rA[t][ee], sE[(16 * t + 4 * lg + ee) * kLB + 16 * J + lr], oo[J]);
        }
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lg + r;
                if (i < n) store_out<OUT_BF16>(o, (row0 + (size_t)i * H) * DV + j0 + 16 * J + lr, oo[J][r]);
            }
        // S <- Diag(gam) S + K^' E (this wavefront's state rows; nobody else reads them now)
#pragma unroll
        for (int t = 0; t < SRB; ++t) {
            const int I = w + 4 * t;
            f32x4 acc[2];
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * I + 4 * lg + r;
                    acc[J][r] = sGam[row] * sS[row * kLB + 16 * J + lr];
                }
            for (int kk = 0; kk < C; kk += 4) {
                const float a = sKh[(kk + lg) * kLKT + 16 * I + lr];
#pragma unroll
                for (int J = 0; J < 2; ++J) acc[J] = mfma4(a, sE[(kk + lg) * kLB + 16 * J + lr], acc[J]);
            }
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[(16 * I + 4 * lg + r) * kLB + 16 * J + lr] = acc[J][r];
        }
    }
    if (!s_final) return;
    __syncthreads();  // the last update's rows, from every wavefront
    for (int idx = tid; idx < DK * kBV; idx += kThreads) {
        const int r = idx / kBV, cc = idx % kBV;
        s_final[sbase + (size_t)r * DV + j0 + cc] = sS[r * kLB + cc];
    }
}

// ============================================================ launch
// bf16 q, k at d = 128 with scalar decay: the forward intra kernel's per-chunk work with its backward outputs,
// the forward pass's bf16 walk storing the entering states, the bf16 reverse walk, then every per-chunk
// gradient in one kernel.
hipError_t launch_bwd16(const BwdArgs &a, const BwdWs &w, unsigned nslot, unsigned nwalk) {
    ChunkArgs f{};
    f.B = a.B;
    f.T = a.T;
    f.H = a.H;
    f.Dk = mx::DK;
    f.Dv = mx::DV;
    f.NC = a.NC;
    f.tab = a.tab;
    f.qkv_bf16 = true;
    f.kaczmarz = a.kaczmarz;
    f.delta = a.delta;
    f.eps = a.eps;
    f.scale = a.scale;
    f.q = a.q;
    f.k = a.k;
    f.v = a.v;
    f.g = a.g;
    f.beta = a.beta;
    f.s0 = a.s0;
    f.ws = w.rec;
    f.stream = a.stream;
    hipError_t e = launch_chunk_prep_bwd(f, w.T, w.G, w.beta, static_cast<char *>(w.rrev));
    if (e != hipSuccess || (e = launch_chunk_states(f, w.S)) != hipSuccess) return e;
    const __bf16 *qb = static_cast<const __bf16 *>(a.q), *kb = static_cast<const __bf16 *>(a.k);
    const char *rec = static_cast<const char *>(w.rec), *rrev = static_cast<const char *>(w.rrev);
    // the reverse walk, in the states walk's time segments (fixed-length batches)
    const int BH = a.B * a.H;
    const int P = a.tab.start ? 1 : chunk_walk_segments(BH, a.NC);
    const int seg = (a.NC + P - 1) / P;
    const float *d_start = nullptr;
    if (P > 1) {
        constexpr size_t mat = (size_t)mx::DK * mx::DV;
        const float *tr = reinterpret_cast<const float *>(rec + (size_t)BH * a.NC * mx::kRecBytes);
        float *nrev = const_cast<float *>(tr) + (size_t)BH * P * 3 * mat;  // after the forward's maps and states
        float *dst = nrev + (size_t)BH * P * mat;
        auto npass = a.delta ? bwd_dstates_bf16_kernel<true, true> : bwd_dstates_bf16_kernel<false, true>;
        hipLaunchKernelGGL(npass, dim3(nwalk * P), dim3(kThreads), 0, a.stream, qb, kb, a.dO, a.T, a.H, a.NC, a.scale,
                           rec, rrev, a.ds_final, w.dS, a.ds0, P, seg, nullptr, nrev, a.tab);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(rev_segment_combine_kernel, dim3((unsigned)(BH * (mx::DV / 16))), dim3(256), 0, a.stream,
                           tr, nrev, a.ds_final, dst, P);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        d_start = dst;
    }
    auto walk = a.delta ? bwd_dstates_bf16_kernel<true, false> : bwd_dstates_bf16_kernel<false, false>;
    hipLaunchKernelGGL(walk, dim3(nwalk * P), dim3(kThreads), 0, a.stream, qb, kb, a.dO, a.T, a.H, a.NC, a.scale, rec,
                       rrev, a.ds_final, w.dS, a.ds0, P, seg, d_start, nullptr, a.tab);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_grads16_kernel, dim3(nslot), dim3(kThreads16), 0, a.stream, static_cast<const __bf16 *>(a.v),
                       a.dO, kb, qb, a.T, a.H, a.NC, a.eps, a.scale, w.T, w.G, w.beta, rec, rrev, w.S, w.dS, a.dq, a.dk,
                       a.dv, a.dg, a.dbeta, a.delta, a.kaczmarz, a.tab);
    return hipGetLastError();
}

template <int DK, int DV, bool PC, bool KZ, bool IB>
hipError_t launch_bwd_t(const BwdArgs &a) {
    // packed batch: a.NC is the chunk bound of all sequences together
    const size_t slots = (size_t)(a.tab.start ? 1 : a.B) * a.H * a.NC;
    constexpr bool ops = bwd_stores_ops(PC, IB);  // K~, K^, Q~ in the workspace
    BwdWs w = carve_bwd<DK, DV, PC>(a.ws, slots, ops, (a.tab.start ? 1 : a.B) * a.H, a.NC);
    const unsigned nslot = (unsigned)slots;
    const unsigned nwalk = (unsigned)(a.B * a.H * (DV / kBV));
    if constexpr (bwd_walk16(ops, DK, DV)) return launch_bwd16(a, w, nslot, nwalk);
    hipLaunchKernelGGL((bwd_prep_kernel<DK, PC, KZ, IB>), dim3(nslot), dim3(kThreads), 0, a.stream, a.q, a.k, a.g,
                       a.beta, a.T, a.H, a.NC, a.eps, a.scale, w.T, w.A, w.M, w.G, w.beta, w.Kt, w.Kh, w.Qt, a.delta,
                       a.tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (ops) {  // both walks in one launch (independent: side by side when they fit)
        hipLaunchKernelGGL((bwd_walks_kernel<DK, DV, PC, IB>), dim3(2 * nwalk), dim3(kThreads), 0, a.stream, a.v,
                           a.dO, a.T, a.H, a.NC, w.T, w.A, w.G, w.beta, w.Kt, w.Kh, w.Qt, a.s0, w.S, a.ds_final, w.dS,
                           a.ds0, a.delta, a.tab, (int)nwalk);
    } else {  // scalar decay with bf16 inputs: the walks on k and q themselves
        hipLaunchKernelGGL((bwd_states_kq16_kernel<DK, DV>), dim3(nwalk), dim3(kThreads), 0, a.stream,
                           static_cast<const __bf16 *>(a.v), static_cast<const __bf16 *>(a.k), a.T, a.H, a.NC, w.T,
                           w.G, w.beta, a.s0, w.S, a.delta, a.tab);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_dstates_kq16_kernel<DK, DV>), dim3(nwalk), dim3(kThreads), 0, a.stream,
                           static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), a.dO, a.T, a.H, a.NC,
                           a.scale, w.T, w.A, w.G, w.beta, a.ds_final, w.dS, a.ds0, a.delta, a.tab);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grads_a_kernel<DK, DV, PC, IB, !ops>), dim3(nslot), dim3(kThreads), 0, a.stream, a.v,
                       a.dO, a.T, a.H, a.NC, a.scale, w.T, w.A, w.G, w.beta, w.S, w.dS, w.Kt, w.Kh, w.Qt,
                       static_cast<const __bf16 *>(a.k), static_cast<const __bf16 *>(a.q), w.dA, w.dTT, w.dG, w.dG63,
                       a.dq, a.dk, a.dv, a.delta, a.tab);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grads_b_kernel<DK, PC, KZ, IB>), dim3(nslot), dim3(kThreads), 0, a.stream, a.q, a.k,
                       a.T, a.H, a.NC, a.eps, a.scale, w.T, w.M, w.A, w.G, w.beta, w.dA, w.dTT, w.dG, w.dG63, a.dq,
                       a.dk, a.dg, a.dbeta, a.tab);
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

// ---- the forward pass on fp32 tiles: prep (stage 0), then the walk with outputs (stage 1).  Its
// workspace is the prep kernel's part of the backward's: T, A, M, G, beta, K~, K^, Q~ per chunk slot.
template <int DK, bool PC>
size_t tile_fwd_bytes(size_t slots) {
    constexpr int GK = PC ? DK : 1;
    return slots * sizeof(float) * ((size_t)3 * C * C + (size_t)C * GK + C + 3 * (size_t)C * DK);
}

template <int DK, int DV, bool PC, bool KZ, bool IB, bool OB>
hipError_t launch_tile_fwd_t(const ChunkArgs &a, int stage) {
    constexpr int GK = PC ? DK : 1;
    const size_t slots = (size_t)chunk_slots(a);
    float *p = static_cast<float *>(a.ws);
    float *wT = p, *wA = wT + slots * C * C, *wM = wA + slots * C * C, *wG = wM + slots * C * C;
    float *wB = wG + slots * C * GK, *wKt = wB + slots * C, *wKh = wKt + slots * C * DK, *wQt = wKh + slots * C * DK;
    if (stage != 1) {
        GDR_LAUNCH((bwd_prep_kernel<DK, PC, KZ, IB>), dim3((unsigned)slots), dim3(kThreads), a.stream, a.ev0,
                   stage == 0 ? a.ev1 : nullptr, a.q, a.k, a.g, a.beta, a.T, a.H, a.NC, a.eps, a.scale, wT, wA, wM, wG,
                   wB, wKt, wKh, wQt, a.delta, a.tab);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || stage == 0) return e;
    }
    const unsigned nwalk = (unsigned)(a.B * a.H * (DV / kBV));
    GDR_LAUNCH((fwd_tile_walk_kernel<DK, DV, PC, IB, OB>), dim3(nwalk), dim3(kThreads), a.stream,
               stage == 1 ? a.ev0 : nullptr, a.ev1, a.v, a.T, a.H, a.NC, wT, wA, wG, wB, wKt, wKh, wQt, a.s0, a.o,
               a.s_final, a.delta, a.tab);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_tile_fwd_d(const ChunkArgs &a, int stage) {
    const int key = (a.per_channel ? 8 : 0) | (a.kaczmarz ? 4 : 0) | (a.qkv_bf16 ? 2 : 0) | (a.o_bf16 ? 1 : 0);
    switch (key) {
        case 0: return launch_tile_fwd_t<DK, DV, false, false, false, false>(a, stage);
        case 1: return launch_tile_fwd_t<DK, DV, false, false, false, true>(a, stage);
        case 2: return launch_tile_fwd_t<DK, DV, false, false, true, false>(a, stage);
        case 3: return launch_tile_fwd_t<DK, DV, false, false, true, true>(a, stage);
        case 4: return launch_tile_fwd_t<DK, DV, false, true, false, false>(a, stage);
        case 5: return launch_tile_fwd_t<DK, DV, false, true, false, true>(a, stage);
        case 6: return launch_tile_fwd_t<DK, DV, false, true, true, false>(a, stage);
        case 7: return launch_tile_fwd_t<DK, DV, false, true, true, true>(a, stage);
        case 8: return launch_tile_fwd_t<DK, DV, true, false, false, false>(a, stage);
        case 9: return launch_tile_fwd_t<DK, DV, true, false, false, true>(a, stage);
        case 10: return launch_tile_fwd_t<DK, DV, true, false, true, false>(a, stage);
        case 11: return launch_tile_fwd_t<DK, DV, true, false, true, true>(a, stage);
        case 12: return launch_tile_fwd_t<DK, DV, true, true, false, false>(a, stage);
        case 13: return launch_tile_fwd_t<DK, DV, true, true, false, true>(a, stage);
        case 14: return launch_tile_fwd_t<DK, DV, true, true, true, false>(a, stage);
        default: return launch_tile_fwd_t<DK, DV, true, true, true, true>(a, stage);
    }
}

}  // namespace

size_t chunk_tile_workspace_bytes(int B, int H, int NC, int Dk, int, bool per_channel) {
    const size_t slots = (size_t)B * H * NC;
    if (Dk == 128) return per_channel ? tile_fwd_bytes<128, true>(slots) : tile_fwd_bytes<128, false>(slots);
    return per_channel ? tile_fwd_bytes<64, true>(slots) : tile_fwd_bytes<64, false>(slots);
}

hipError_t launch_chunk_tile(const ChunkArgs &a, int stage) {
    if (a.Dk == 128 && a.Dv == 128) return launch_tile_fwd_d<128, 128>(a, stage);
    if (a.Dk == 128 && a.Dv == 64) return launch_tile_fwd_d<128, 64>(a, stage);
    if (a.Dk == 64 && a.Dv == 128) return launch_tile_fwd_d<64, 128>(a, stage);
    return launch_tile_fwd_d<64, 64>(a, stage);
}

size_t chunk_bwd_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel, bool qkv_bf16) {
    const size_t slots = (size_t)B * H * NC;
    const bool ops = bwd_stores_ops(per_channel, qkv_bf16);
    const int BH = B * H;
    if (Dk == 128 && Dv == 128)
        return per_channel ? bwd_bytes<128, 128, true>(slots, ops, BH, NC) : bwd_bytes<128, 128, false>(slots, ops, BH, NC);
    if (Dk == 128 && Dv == 64)
        return per_channel ? bwd_bytes<128, 64, true>(slots, ops, BH, NC) : bwd_bytes<128, 64, false>(slots, ops, BH, NC);
    if (Dk == 64 && Dv == 128)
        return per_channel ? bwd_bytes<64, 128, true>(slots, ops, BH, NC) : bwd_bytes<64, 128, false>(slots, ops, BH, NC);
    return per_channel ? bwd_bytes<64, 64, true>(slots, ops, BH, NC) : bwd_bytes<64, 64, false>(slots, ops, BH, NC);
}

hipError_t launch_chunk_bwd(const BwdArgs &a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bwd_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bwd_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bwd_d<64, 128>(a);
    return launch_bwd_d<64, 64>(a);
}

}  // namespace gdr
