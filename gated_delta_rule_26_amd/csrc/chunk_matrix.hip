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
//    operands stay in registers from one product to the next (the layout in
//    matrix_common.h), so a chunk needs no exchange between chain wavefronts.  They also form
//    the read Q S, which shares the state operand with K S.  Two "helper"
//    wavefronts stage the next chunk's q, k, v and decays in LDS and, one
//    chunk behind, finish the outputs O = scale Gam (Q S) + A E from the
//    chain's Q S and E, passed through LDS.  One barrier per chunk; every LDS
//    buffer that crosses it is doubled (exp(G) tripled: the helpers read it
//    one chunk after the chain).
//
// Without the delta rule (DELTA = false: the additive write S = D S + k v^T
// of the textbook page's update table; linear attention, RetNet / Mamba-2)
// there is no prediction and no solve: E = V, so the intra kernel forms only
// A (no K K^T, no inverse, no T'' in the record) and the walk skips K S and
// the T'' product.
//
// The operand layout (a D tile is directly the B operand of the next
// product) and the bf16 hi/lo precision scheme are described in
// matrix_common.h.
#include <cmath>
#include <type_traits>

#include "matrix_common.h"

namespace gdr {
namespace {

using namespace mx;

// The per-chunk workspace record of scalar decay (kRecBytes, matrix_common.h):
// the T'' and A fragments, then exp(G) and exp(G_63 - G) of the 64 tokens, so
// the walk needs no exponentials.

// ============================================================ intra kernel
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
    float eta[C];               // beta, or eta for the Kaczmarz step size (0 past the end), then the write strengths
    float kk[C];                // |k_i|^2 (Kaczmarz only)
};

// With BWD (the backward pass's per-chunk inputs) the kernel also writes, per chunk, T itself (fp32, zero
// above the diagonal; the identity without the delta rule), G and the write strengths to bT, bG, bB, and
// the reverse record (the transposes of T'' and A as bf16 hi/lo fragments) to brev.
template <bool KZ, bool DELTA, bool BWD = false>
__global__ __launch_bounds__(kIntraThreads, 4) void intra_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, int T, int H, int NC, int total, float eps, float scale,
    char *__restrict__ ws, SeqTable tb, float *__restrict__ bT, float *__restrict__ bG, float *__restrict__ bB,
    char *__restrict__ brev) {
    __shared__ IntraSmem sm;
    if (tb.start) total = tb.cbase[tb.N] * H;  // packed batch: the chunks the table holds
    if (total <= 0) return;
    const int qk_stride = H * DK * 2;
    const TriTiles tri{sm.u.t.R, sm.u.t.Toff, sm.u.t.A};
    const int seg = threadIdx.x & 15, i0 = threadIdx.x >> 4;
    const int lane0 = threadIdx.x & 63;

    // Persistent: the workgroup takes chunks ci = blockIdx.x + k gridDim.x
    // ((b*H + h)*NC + c) and loads the next one's q, k and gates into
    // registers while it computes the current one.
    uint4 qv[4], kv[4];
    float gv, ev;
    auto prefetch = [&](int cj) {
        size_t r0;
        int nn;
        chunk_place(cj, T, H, NC, tb, r0, nn);
        const auto rk = rows_rsrc(k + r0 * DK, nn, qk_stride, DK * 2);
        const auto rq = rows_rsrc(q + r0 * DK, nn, qk_stride, DK * 2);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int off = (i0 + 16 * it) * qk_stride + 16 * seg;
            qv[it] = buf_ld16(rq, off);
            kv[it] = buf_ld16(rk, off);
        }
        gv = g[r0 + (size_t)min(lane0, nn - 1) * H];
        ev = DELTA ? beta[r0 + (size_t)min(lane0, nn - 1) * H] : 0.f;
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
    size_t r0_unused;
    int n;
    chunk_place(ci, T, H, NC, tb, r0_unused, n);
    char *recb = ws + (size_t)ci * kRecBytes;
    barrier_lds();  // the previous chunk's tiles are no longer read

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
    barrier_lds();

    // ---- K K^T (wavefronts 0, 1) and Q K^T (2, 3) on the lower tiles: even
    // wavefronts take row blocks {0, 3}, odd ones {1, 2}
    const int Ia = (w & 1) ? 1 : 0, Ib = (w & 1) ? 2 : 3;
    f32x4 acc[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (DELTA || w >= 2) {
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
    barrier_lds();  // G, eta (and |k|^2) in LDS; q and k no longer read
    if constexpr (KZ) {
        write_strength<KZ>(sm.eta, sm.kk, n, eps, w, lane);
        barrier_lds();
    }

    // ---- decay (and beta for R) applied in fp32; R and A tiles to LDS (no R
    // without the delta rule)
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        if (!DELTA && w < 2) continue;
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
                val = j < i ? sm.eta[i] * dec * acc[t][r] : 0.f;
            }
            dst[(4 * lg + r) * LT + lr] = val;
        }
    }
    barrier_lds();

    // ---- T = (I + R)^{-1}, then the T'' and A operand fragments
    if constexpr (DELTA) invert_unit_lower(tri, lane, w, lr, lg);
    pack_T_A<DELTA>(tri, sm.eta, recb, tid);
    if constexpr (BWD) {
        float *Tg = bT + (size_t)ci * C * C;
        for (int idx4 = tid; idx4 < C * C / 4; idx4 += kIntraThreads) {  // 16-byte stores
            const int i = idx4 / (C / 4), j = (idx4 % (C / 4)) * 4, I = i >> 4, J = j >> 4;
            f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
            if (DELTA && J <= I) t4 = *reinterpret_cast<const f32x4 *>(&tri.Tb(I, J)[(i & 15) * LT + (j & 15)]);
            else if (!DELTA && (i >> 2) == (j >> 2)) t4[i & 3] = 1.f;  // the identity
            reinterpret_cast<f32x4 *>(Tg)[idx4] = t4;
        }
        if (tid < C) {
            bG[(size_t)ci * C + tid] = sm.G[tid];
            bB[(size_t)ci * C + tid] = sm.eta[tid];
        }
        pack_reverse<DELTA>(tri, sm.eta, brev + (size_t)ci * kRevBytes, tid);
    }
    }  // chunk loop
}

// ============================================================ state kernel
// bf16 row stride of the token-major q, k: 288 bytes keeps both the 16-byte
// fragment reads and the transposing 8-byte reads of four rows free of LDS
// bank conflicts (272 bytes costs the transposing reads a third more, 320
// bytes doubles the 16-byte reads; measured on gfx950)
constexpr int LDK = DK + 16;

struct alignas(16) StateSmem {
    __bf16 K[2][C * LDK];          // k, token-major, key channels permuted within 32-blocks
    __bf16 Q[2][C * LDK];          // q, the same layout
    __bf16 V[2][C * LDV];          // v slice, token-major
    float Gam[3][C];               // exp(G_i); chunk c in buffer c % 3 (read one chunk later by the helpers)
    float Gend[2][C];              // exp(G_63 - G_i)
    uint4 X[2][2][kXFrags][64];    // per chunk parity and chain wavefront; once a helper has read its
                                   // chunk's Q S and E, the same 8 KB hold its fp32 output tile
                                   // (token-major, 20-float rows) for 16-byte stores
};
static_assert(C * 20 * sizeof(float) <= kXFrags * 64 * sizeof(uint4), "output tile must fit one X buffer");
// The transfer walk (no outputs, no Q S) needs only the k and v staging and the decays.
struct alignas(16) TransferSmem {
    __bf16 K[2][C * LDK];
    __bf16 V[2][C * LDV];
    float Gam[3][C];
    float Gend[2][C];
};

// The walk over the chunks of G = BH * P groups (sequence, head, time
// segment p): group g = bh * P + p covers chunks [p seg, min(NC, (p+1) seg)).
// With P = 1 this is the whole sequence.
//  * TRANSFER = false: s0 (or zero) holds the entering state of every group
//    ([G][DK][DV]); the last segment of each sequence writes its final state
//    to s_out[bh]; outputs are written.
//  * TRANSFER = true: the group's chunk map S -> M S + N (substituting
//    E = T''(V - Gam K S) into the chunk-end state, [P2] "KDA por chunks",
//    chunk-end state): slices 0 .. NS-1 walk N (zero start, v), slices NS ..
//    2NS-1 walk the columns of M (identity start, v = 0); N and M go to
//    s_out[g][0] and s_out[g][1].  No outputs, so the LDS holds only the
//    k, v staging and the decays (48 KB) and two workgroups share a unit.
//  * STATES (with TRANSFER's staging, P = 1): the walk of S itself from s0
//    (or zero), no outputs; the state entering every chunk goes to s_out at
//    the chunk's record index ([DK][DV] each), for the backward pass.
// DELTA = false: E = V (no K S, no T''), records without T''.
template <bool OUT_BF16, bool TRANSFER, bool DELTA, bool STATES = false>
__global__ __launch_bounds__(kStateThreads, TRANSFER ? 2 : 1) void state_matrix_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const char *__restrict__ ws, const float *__restrict__ s0, void *__restrict__ o,
    float *__restrict__ s_out, int T, int H, int NC, int G, int P, int seg, float scale, SeqTable tb) {
    static_assert(!STATES || TRANSFER, "the states walk uses the transfer walk's staging");
    constexpr bool MAPS = TRANSFER && !STATES;  // the walk of a chunk map
    __shared__ std::conditional_t<TRANSFER, TransferSmem, StateSmem> sm;

    int g, slice;
    state_slot(blockIdx.x, G, MAPS ? 2 * NS : NS, g, slice);
    g = walk_seq(g, H, tb);  // packed batches (P = 1): longest sequences first
    const int bh = g / P, p = g % P;
    const int kind = MAPS ? slice / NS : 0;      // transfer: 0 = N, 1 = M
    const int c0 = p * seg;
    const WalkPlace wp = walk_place(bh, c0, seg, T, H, NC, tb, ws, kRecBytes);
    const int nc = wp.nc;                        // chunks of this segment
    const int L = wp.L;                          // tokens of this sequence
    const size_t rstride = wp.rstride;           // bytes from one chunk's record to the next
    const int j0 = (slice % NS) * BV;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const char *recs = wp.recs;
    const float *s_in = MAPS || !s0 ? nullptr : s0 + (size_t)g * DK * DV;
    float *s_end = STATES ? nullptr
                   : TRANSFER ? s_out + ((size_t)g * 2 + kind) * DK * DV
                              : (s_out && p == P - 1 ? s_out + (size_t)bh * DK * DV : nullptr);
    // STATES: record index of the segment's first chunk and from one chunk to the next
    const size_t slot0 = (size_t)(recs - ws) / kRecBytes, slot_step = rstride / kRecBytes;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    if (nc <= 0) {  // empty sequence: the final state is the initial one
        if (s_end && w < 2) {
            const int jt = j0 + 16 * w;
            for (int i = 0; i < 8; ++i)
                for (int r = 0; r < 4; ++r) {
                    const size_t idx = (size_t)(16 * i + 4 * lg + r) * DV + jt + lr;
                    s_end[idx] = s_in ? s_in[idx] : 0.f;
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
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * lg + r;
                if constexpr (MAPS) S[i][r] = kind == 1 && row == jt + lr ? 1.f : 0.f;
                else S[i][r] = s_in ? s_in[(size_t)row * DV + jt + lr] : 0.f;
            }
        // T'' fragments of even chunks in tA, of odd chunks in tB: each chunk
        // loads the next one's into the other set (no register copies).
        bf16x8 tAh[6], tAl[6], tBh[6], tBl[6];
        if constexpr (DELTA) {
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                tAh[f] = *reinterpret_cast<const bf16x8 *>(recs + kRecTH + f * kFragBytes + lane * 16);
                tAl[f] = *reinterpret_cast<const bf16x8 *>(recs + kRecTL + f * kFragBytes + lane * 16);
            }
        }
        auto step = [&](int c, const bf16x8 *th, const bf16x8 *tl, bf16x8 *thn, bf16x8 *tln)
                        __attribute__((always_inline)) {
            const int buf = c & 1;
            if constexpr (STATES) {  // the state entering chunk c
                float *Sc = s_out + (slot0 + (size_t)c * slot_step) * (DK * DV);
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sc[(size_t)(16 * i + 4 * lg + r) * DV + jt + lr] = S[i][r];
            }
            // next chunk's T'' fragments, in flight during this chunk
            if constexpr (DELTA) {
                const char *rn = recs + (size_t)min(c + 1, nc - 1) * rstride;
#pragma unroll
                for (int f = 0; f < 6; ++f) {
                    thn[f] = *reinterpret_cast<const bf16x8 *>(rn + kRecTH + f * kFragBytes + lane * 16);
                    tln[f] = *reinterpret_cast<const bf16x8 *>(rn + kRecTL + f * kFragBytes + lane * 16);
                }
            }
            uint4 *xo = nullptr;
            if constexpr (!TRANSFER) xo = &sm.X[buf][w][0][0];
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
            const __bf16 *sQ = nullptr;
            if constexpr (!TRANSFER) sQ = sm.Q[buf];
            bf16x8 ka[2][4], qa[2][4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                if constexpr (DELTA) ka[0][M] = *reinterpret_cast<const bf16x8 *>(&sK[(16 * M + lr) * LDK + 8 * lg]);
                if constexpr (!TRANSFER) qa[0][M] = *reinterpret_cast<const bf16x8 *>(&sQ[(16 * M + lr) * LDK + 8 * lg]);
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cur = kb & 1;
                if (kb + 1 < 4) {
#pragma unroll
                    for (int M = 0; M < 4; ++M) {
                        if constexpr (DELTA)
                            ka[cur ^ 1][M] = *reinterpret_cast<const bf16x8 *>(&sK[(16 * M + lr) * LDK + 32 * (kb + 1) + 8 * lg]);
                        if constexpr (!TRANSFER)
                            qa[cur ^ 1][M] = *reinterpret_cast<const bf16x8 *>(&sQ[(16 * M + lr) * LDK + 32 * (kb + 1) + 8 * lg]);
                    }
                }
                if constexpr (DELTA) {
#pragma unroll
                    for (int M = 0; M < 4; ++M) P[M] = mma(ka[cur][M], SH[kb], P[M]);
#pragma unroll
                    for (int M = 0; M < 4; ++M) P[M] = mma(ka[cur][M], SL[kb], P[M]);
                }
                if constexpr (!TRANSFER) {  // the read Q S (no outputs in a transfer walk)
#pragma unroll
                    for (int M = 0; M < 4; ++M) QS[M] = mma(qa[cur][M], SH[kb], QS[M]);
#pragma unroll
                    for (int M = 0; M < 4; ++M) QS[M] = mma(qa[cur][M], SL[kb], QS[M]);
                }
            }
            // decays and this wavefront's v columns
            f32x4 gam[4], gnd[4];
            bf16x4 vv[4];
            const float *gamc = sm.Gam[c % 3];
            const float gs = gamc[C - 1];  // exp(G_63), the chunk's state decay
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                gam[M] = *reinterpret_cast<const f32x4 *>(&gamc[16 * M + 4 * lg]);
                gnd[M] = *reinterpret_cast<const f32x4 *>(&sm.Gend[buf][16 * M + 4 * lg]);
                // V[16M + 4lg + r][16w + lr], r = 0..3
                vv[M] = lds_read_tr(&sm.V[buf][(16 * M + 4 * lg + (lr >> 2)) * LDV + 16 * w + 4 * (lr & 3)]);
            }
            // X = V - Gam P, rows 16M + 4lg + r; the read Q S to the helper
            // (which applies scale Gam)
            f32x4 Xv[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Xv[M][r] = DELTA ? static_cast<float>(vv[M][r]) - gam[M][r] * P[M][r] : static_cast<float>(vv[M][r]);
                if constexpr (!TRANSFER) xo[M * 64 + lane] = *reinterpret_cast<const uint4 *>(&QS[M]);
            }
            bf16x8 XH[2], XL[2];
            if constexpr (DELTA) {
                pair_split(Xv[0], Xv[1], XH[0], XL[0]);
                pair_split(Xv[2], Xv[3], XH[1], XL[1]);
            }
            // k^T fragments (key-channel tile i, token block kb) for the update,
            // read transposed from the token-major k: term e of lane group lg is
            // token 32kb + kperm(lg, e), key channel 16i + lr.  Tile 0 now.
            auto kt_frag = [&](int i, int kb) { return kt_operand(sK, LDK, i, kb, lr, lg); };
            bf16x8 kt[2][2];
            kt[0][0] = kt_frag(0, 0);
            kt[0][1] = kt_frag(0, 1);
            // E = T'' X (E = X = V without the delta rule)
            f32x4 E[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                E[M] = DELTA ? zero4 : Xv[M];
                if constexpr (DELTA) {
#pragma unroll
                    for (int kb = 0; kb <= (M >> 1); ++kb) {
                        const int f = lower_frag(M, kb);
                        E[M] = mma(th[f], XH[kb], E[M]);
                        E[M] = mma(th[f], XL[kb], E[M]);
                        E[M] = mma(tl[f], XH[kb], E[M]);
                    }
                }
            }
            // E to the helper; Gend E as the update's B operand
            f32x4 Ep[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                if constexpr (!TRANSFER) xo[(4 + M) * 64 + lane] = *reinterpret_cast<const uint4 *>(&E[M]);
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
        for (; c + 1 < nc; c += 2) {
            step(c, tAh, tAl, tBh, tBl);
            barrier_lds();
            step(c + 1, tBh, tBl, tAh, tAl);
            barrier_lds();
        }
        if (c < nc) {
            step(c, tAh, tAl, tBh, tBl);
            barrier_lds();
        }
        barrier_lds();  // step nc: the helpers finish the last chunk's outputs
        if (s_end) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) s_end[(size_t)(16 * i + 4 * lg + r) * DV + jt + lr] = S[i][r];
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
        const size_t head0 = wp.head0;  // row of token 0 of this sequence and head
        const int qk_stride = H * DK * 2, v_stride = H * DV * 2;
        // byte offsets, inside a chunk, of this thread's q/k and v pieces
        int qk_off[8], v_off[2];
#pragma unroll
        for (int u = 0; u < 8; ++u) qk_off[u] = (8 * (ht >> 4) + u) * qk_stride + 16 * (ht & 15);
#pragma unroll
        for (int u = 0; u < 2; ++u) v_off[u] = (2 * (ht >> 2) + u) * v_stride + 2 * (j0 + 8 * (ht & 3));
        auto load_stage = [&](int cc) {  // chunk cc's q, k, v slice and G into registers
            const int t0 = (c0 + cc) * C;
            const int n = min(C, L - t0);
            const size_t row0 = head0 + (size_t)t0 * H;
            const auto rk = rows_rsrc(k + row0 * DK, n, qk_stride, DK * 2);
            const auto rq = rows_rsrc(q + row0 * DK, n, qk_stride, DK * 2);
            const auto rv = rows_rsrc(v + row0 * DV, kind == 1 ? 0 : n, v_stride, DV * 2);  // M columns: v = 0
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                kreg[u] = buf_ld16(rk, qk_off[u]);
                if constexpr (!TRANSFER) qreg[u] = buf_ld16(rq, qk_off[u]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) vreg[u] = buf_ld16(rv, v_off[u]);
            const char *rec = recs + (size_t)cc * rstride;
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
                    if constexpr (!TRANSFER) *reinterpret_cast<uint2 *>(&sm.Q[buf][i * LDK + col]) = qh[hh];
                }
            }
            {
                const int sv = ht & 3, tq = ht >> 2;
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    *reinterpret_cast<uint4 *>(&sm.V[buf][(2 * tq + u) * LDV + 8 * sv]) = vreg[u];
            }
            if (ht < C) {
                sm.Gam[cc % 3][ht] = gam_reg;
                sm.Gend[buf][ht] = gnd_reg;
            }
        };
        bf16x8 ah[6], al[6];
        auto load_out_ops = [&](int cc) {  // chunk cc's A fragments
            const char *rec = recs + (size_t)cc * rstride;
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                ah[f] = *reinterpret_cast<const bf16x8 *>(rec + kRecAH + f * kFragBytes + lane * 16);
                al[f] = *reinterpret_cast<const bf16x8 *>(rec + kRecAL + f * kFragBytes + lane * 16);
            }
        };
        // outputs of chunk cp: O = scale Gam (Q S, from the chain) + A E (none
        // for a transfer walk)
        auto outputs = [&](int cp) __attribute__((always_inline)) {
            if constexpr (!TRANSFER) {
                const int t0 = (c0 + cp) * C;
                uint4 *xv = &sm.X[cp & 1][vt][0][0];  // not written by the chain before the next barrier
                chunk_outputs<OUT_BF16, true>(xv, sm.Gam[cp % 3], scale, ah, al, reinterpret_cast<float *>(xv),
                                              o, head0 + (size_t)t0 * H, min(C, L - t0), H, jt, lane);
            }
        };
        auto load_outputs_operands = [&](int cc) {
            if constexpr (!TRANSFER) load_out_ops(cc);
        };
        // step 0: stage chunk 0 (and 1); step c >= 1: outputs of chunk c-1
        load_stage(0);
        store_stage(0);
        load_stage(min(1, nc - 1));
        barrier_lds();
        if (nc > 1) store_stage(1);
        load_stage(min(2, nc - 1));
        load_outputs_operands(0);
        barrier_lds();
        for (int c = 1; c < nc; ++c) {
            if (c + 1 < nc) store_stage(c + 1);
            load_stage(min(c + 2, nc - 1));
            outputs(c - 1);
            load_outputs_operands(c);
            barrier_lds();
        }
        outputs(nc - 1);
        barrier_lds();
    }
}

// ============================================================ segment combine
// Entering state of every time segment of a sequence: S_0 = s0 (or zero),
// S_{p+1} = M_p S_p + N_p, from the chunk maps of the transfer walk.  The
// columns of S are independent, so one workgroup takes (sequence, head, 16
// value columns); per step it stages M_p in LDS (rows padded to 129 floats,
// so the rows a wavefront reads fall in different banks), and thread t forms
// row t / 2, columns 8 (t % 2) .. +7 of its slice in fp32.
constexpr int kCombineCols = 16;
__global__ __launch_bounds__(256) void segment_combine_kernel(const float *__restrict__ tr,
                                                              const float *__restrict__ s0,
                                                              float *__restrict__ seg_state, int P) {
    constexpr int LM = DK + 1, NCS = DV / kCombineCols;
    __shared__ float Ss[DK][kCombineCols];
    __shared__ float Ms[DK * LM];
    const int bh = blockIdx.x / NCS, cs = blockIdx.x % NCS;
    const int t = threadIdx.x, i = t >> 1, jl = 8 * (t & 1), jb = cs * kCombineCols + jl;
    const size_t mat = (size_t)DK * DV;
    const float *sin = s0 ? s0 + bh * mat : nullptr;
    float *out0 = seg_state + (size_t)bh * P * mat;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const float x = sin ? sin[i * DV + jb + jj] : 0.f;
        Ss[i][jl + jj] = x;
        out0[i * DV + jb + jj] = x;
    }
    for (int pp = 0; pp + 1 < P; ++pp) {
        const float *N = tr + ((size_t)(bh * P + pp) * 2 + 0) * mat;
        const float *M = tr + ((size_t)(bh * P + pp) * 2 + 1) * mat;
        constexpr int PER = DK * DK / 256;  // M entries per thread
        float mr[PER], acc[8];
#pragma unroll
        for (int u = 0; u < PER; ++u) mr[u] = M[t + u * 256];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[jj] = N[i * DV + jb + jj];
        __syncthreads();  // the previous step's reads of Ms and Ss are done
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = t + u * 256;
            Ms[(idx / DK) * LM + idx % DK] = mr[u];
        }
        __syncthreads();
        for (int kk = 0; kk < DK; ++kk) {
            const float m = Ms[i * LM + kk];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) acc[jj] = fmaf(m, Ss[kk][jl + jj], acc[jj]);
        }
        __syncthreads();
        float *out = seg_state + ((size_t)bh * P + pp + 1) * mat;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            Ss[i][jl + jj] = acc[jj];
            out[i * DV + jb + jj] = acc[jj];
        }
    }
}

// ============================================================ launchers
template <bool KZ, bool DELTA>
hipError_t launch_intra(const ChunkArgs &a) {
    const long total = chunk_slots(a);
    if (total == 0) return hipSuccess;
    GDR_LAUNCH((intra_matrix_kernel<KZ, DELTA>), dim3(intra_grid(total, 4)), dim3(kIntraThreads), a.stream, a.ev0,
               a.ev1, static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), a.g, a.beta, a.T, a.H, a.NC,
               (int)total, a.eps, a.scale, static_cast<char *>(a.ws), a.tab, nullptr, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

// Time segments of the walk.  Each walk is one workgroup per (group, 32 value
// columns) and the walk is latency-bound, so a few long sequences leave most
// compute units idle; splitting each sequence into P segments costs a
// transfer walk of twice the columns plus a walk per segment.  The transfer
// walk keeps no outputs and fits two workgroups per compute unit, and a round
// of those takes about as long as a round of walks with outputs (one per
// unit), so the cost is (ceil(2 P BH NS / 2 CUs) + ceil(P BH NS / CUs)) / P
// of the single walk's time.  P is the smallest power of two that minimises
// that (planned for 256 compute units so that the workspace size does not
// depend on the device), with at least 32 chunks per segment.
int walk_segments(int BH, int NC) {
    constexpr double kPlanCUs = 256.0;
    int best = 1;
    double best_cost = std::ceil(BH * NS / kPlanCUs);
    for (int P = 2; P <= 16; P *= 2) {
        if (NC < 32 * P) break;
        const double cost =
            (std::ceil(2.0 * P * BH * NS / (2 * kPlanCUs)) + std::ceil(1.0 * P * BH * NS / kPlanCUs)) / P;
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = P;
        }
    }
    return best;
}

size_t segment_bytes(int BH, int NC) {
    const int P = walk_segments(BH, NC);
    return P > 1 ? (size_t)BH * P * 3 * DK * DV * sizeof(float) : 0;
}

template <bool OB, bool DELTA>
hipError_t launch_state(const ChunkArgs &a) {
    const int BH = a.B * a.H;
    const int P = a.tab.start ? 1 : walk_segments(BH, a.NC);  // packed batches: one walk per sequence
    const __bf16 *q = static_cast<const __bf16 *>(a.q), *k = static_cast<const __bf16 *>(a.k),
                 *v = static_cast<const __bf16 *>(a.v);
    const char *ws = static_cast<const char *>(a.ws);
    if (P == 1) {
        GDR_LAUNCH((state_matrix_kernel<OB, false, DELTA>), dim3((unsigned)(BH * NS)), dim3(kStateThreads), a.stream,
                   a.ev0, a.ev1, q, k, v, ws, a.s0, a.o, a.s_final, a.T, a.H, a.NC, BH, 1, a.NC, a.scale, a.tab);
        return hipGetLastError();
    }
    // segments: chunk maps, entering states, then the walks with outputs
    const int seg = (a.NC + P - 1) / P;
    float *tr = reinterpret_cast<float *>(static_cast<char *>(a.ws) + (size_t)BH * a.NC * kRecBytes);
    float *seg_state = tr + (size_t)BH * P * 2 * DK * DV;
    GDR_LAUNCH((state_matrix_kernel<false, true, DELTA>), dim3((unsigned)(BH * P * 2 * NS)), dim3(kStateThreads),
               a.stream, a.ev0, nullptr, q, k, v, ws, nullptr, nullptr, tr, a.T, a.H, a.NC, BH * P, P, seg, a.scale,
               SeqTable{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(segment_combine_kernel, dim3((unsigned)(BH * (DV / kCombineCols))), dim3(256), 0, a.stream, tr,
                       a.s0, seg_state, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GDR_LAUNCH((state_matrix_kernel<OB, false, DELTA>), dim3((unsigned)(BH * P * NS)), dim3(kStateThreads), a.stream,
               nullptr, a.ev1, q, k, v, ws, seg_state, a.o, a.s_final, a.T, a.H, a.NC, BH * P, P, seg, a.scale,
               SeqTable{});
    return hipGetLastError();
}

// The backward pass's walk: one workgroup per (sequence, head, time segment,
// 32 value columns), the entering states to `states`.  Time segments as in
// launch_state (fixed-length batches): the chunk maps, the entering state of
// every segment, then the segments' walks.
template <bool DELTA>
hipError_t launch_states_walk(const ChunkArgs &a, float *states) {
    if (chunk_slots(a) == 0) return hipSuccess;
    const int BH = a.B * a.H;
    const int P = a.tab.start ? 1 : walk_segments(BH, a.NC);
    const __bf16 *q = static_cast<const __bf16 *>(a.q), *k = static_cast<const __bf16 *>(a.k),
                 *v = static_cast<const __bf16 *>(a.v);
    const char *ws = static_cast<const char *>(a.ws);
    const int seg = (a.NC + P - 1) / P;
    const float *s_in = a.s0;
    if (P > 1) {
        float *tr = reinterpret_cast<float *>(static_cast<char *>(a.ws) + (size_t)BH * a.NC * kRecBytes);
        float *seg_state = tr + (size_t)BH * P * 2 * DK * DV;
        hipLaunchKernelGGL((state_matrix_kernel<false, true, DELTA>), dim3((unsigned)(BH * P * 2 * NS)),
                           dim3(kStateThreads), 0, a.stream, q, k, v, ws, nullptr, nullptr, tr, a.T, a.H, a.NC, BH * P,
                           P, seg, a.scale, SeqTable{});
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(segment_combine_kernel, dim3((unsigned)(BH * (DV / kCombineCols))), dim3(256), 0, a.stream,
                           tr, a.s0, seg_state, P);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        s_in = seg_state;
    }
    hipLaunchKernelGGL((state_matrix_kernel<false, true, DELTA, true>), dim3((unsigned)(BH * P * NS)),
                       dim3(kStateThreads), 0, a.stream, q, k, v, ws, s_in, nullptr, states, a.T, a.H, a.NC, BH * P, P,
                       seg, a.scale, a.tab);
    return hipGetLastError();
}

// The backward pass's per-chunk inputs for bf16 q, k at d = 128 and scalar decay: the intra kernel with its
// backward outputs.
template <bool KZ, bool DELTA>
hipError_t launch_intra_bwd(const ChunkArgs &a, float *bT, float *bG, float *bB, char *brev) {
    const long total = chunk_slots(a);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((intra_matrix_kernel<KZ, DELTA, true>), dim3(intra_grid(total, 4)), dim3(kIntraThreads), 0,
                       a.stream, static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), a.g, a.beta, a.T,
                       a.H, a.NC, (int)total, a.eps, a.scale, static_cast<char *>(a.ws), a.tab, bT, bG, bB, brev);
    return hipGetLastError();
}

}  // namespace

size_t chunk_states_segment_bytes(int BH, int NC) { return segment_bytes(BH, NC); }
int chunk_walk_segments(int BH, int NC) { return walk_segments(BH, NC); }

hipError_t launch_chunk_states(const ChunkArgs &a, float *states) {
    return a.delta ? launch_states_walk<true>(a, states) : launch_states_walk<false>(a, states);
}

hipError_t launch_chunk_prep_bwd(const ChunkArgs &a, float *T, float *G, float *beta, char *rrev) {
    return !a.delta ? launch_intra_bwd<false, false>(a, T, G, beta, rrev)
           : a.kaczmarz ? launch_intra_bwd<true, true>(a, T, G, beta, rrev)
                        : launch_intra_bwd<false, true>(a, T, G, beta, rrev);
}

int mx::intra_grid(long total, int per_cu) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (int)std::min<long>(total, (long)per_cu * cus);
}

// The bf16 kernels of this file (and of chunk_matrix_pc.hip) take bf16 q/k/v at
// d_k = d_v = 128; every other input runs on the fp32-tile kernels.
static bool bf16_kernels(int Dk, int Dv, bool qkv_bf16) { return qkv_bf16 && Dk == DK && Dv == DV; }

size_t chunk_matrix_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel, bool packed,
                                    bool qkv_bf16) {
    if (!bf16_kernels(Dk, Dv, qkv_bf16)) return chunk_tile_workspace_bytes(B, H, NC, Dk, Dv, per_channel);
    if (per_channel) return chunk_matrix_pc_workspace_bytes(B, H, NC);
    return (size_t)B * H * NC * kRecBytes + (packed ? 0 : segment_bytes(B * H, NC));
}

bool chunk_matrix_supported(int, int, bool, bool) { return true; }

hipError_t launch_chunk_matrix(const ChunkArgs &a, int stage) {
    if (!bf16_kernels(a.Dk, a.Dv, a.qkv_bf16)) return launch_chunk_tile(a, stage);
    if (a.per_channel) return launch_chunk_matrix_pc(a, stage);
    if (stage != 1) {
        const hipError_t e = !a.delta ? launch_intra<false, false>(a)
                             : a.kaczmarz ? launch_intra<true, true>(a) : launch_intra<false, true>(a);
        if (e != hipSuccess || stage == 0) return e;
    }
    if (!a.delta) return a.o_bf16 ? launch_state<true, false>(a) : launch_state<false, false>(a);
    return a.o_bf16 ? launch_state<true, true>(a) : launch_state<false, true>(a);
}

}  // namespace gdr
