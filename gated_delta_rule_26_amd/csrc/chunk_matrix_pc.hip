// Chunked forward pass on the matrix cores for per-channel decay (one decay
// rate per token, head and key channel, as in Kimi Delta Attention), bf16
// q/k/v, d_k = d_v = 128, fp32 state.
//
// Algebra (blog summary on the DeltaNet family, "KDA por chunks", written for
// the d_k x d_v state; G_i in R^{d_k} is the in-chunk inclusive cumulative
// log-decay of token i, exponentials and (.) are elementwise):
//   R_ij = beta_i sum_c k_ic exp(G_ic - G_jc) k_jc     j < i   (strictly lower)
//   A_ij = scale sum_c q_ic exp(G_ic - G_jc) k_jc      j <= i  (read after write)
//   T    = (I + R)^{-1},  T'' = T Diag(beta)
//   K~   = exp(G) (.) K,  Q~ = scale exp(G) (.) Q,  K^ = exp(G_63 - G) (.) K
//   E    = T'' (V - K~ S)                               corrected writes
//   O    = Q~ S + A E                                    outputs of the chunk
//   S   <- Diag(exp(G_63)) S + K^^T E                    chunk-end state
// With one decay rate for all channels this is the scalar-decay form of
// chunk_matrix.hip (there the factors multiply rows of K S and Q S instead).
// Without the delta rule (DELTA = false: GLA's additive write
// S = Diag(exp g) S + k v^T, textbook page, update table) E = V: no R, no
// inverse and no T'' in the record, and the walk skips K~ S and T''.
//
// Two kernels, as for scalar decay:
//  * intra (persistent, two workgroups per compute unit): the gate scan, R
//    and A on the matrix cores, T, and the chunk record: the T'' and A
//    fragments of the common head, then K~, Q~ and K^ as bf16 hi + lo MFMA
//    operand fragments, and exp(G_63).  The decayed operands are not exact in
//    bf16, so every product with them is split (hi*hi + hi*lo + lo*hi).
//  * state (one workgroup per (sequence, head, 32 value columns)): two chain
//    wavefronts as for scalar decay; two helper wavefronts move the decayed
//    operand fragments of a chunk from the record, and the v slice, straight
//    into LDS (global loads that write LDS, no registers) and form
//    O = Q~ S + A E one chunk behind.  Two barriers per chunk; key block 0 of
//    K~, Q~ is double-buffered so that the copies split evenly between the
//    two halves of a chunk.
//
// R and A with per-channel decay.  exp(G_i - G_j) does not factor into a row
// term times a column term that is bounded for every i, j, so row block I
// (tokens 16I .. 16I+15) takes the reference token r = 16I:
//   exp(G_ic - G_jc) = exp(G_ic - G_rc) exp(G_rc - G_jc).
// The row factor is <= 1 (i >= r, g <= 0); the column factor is <= 1 for the
// tiles left of the diagonal (j < r) and at most exp(span_I) in the diagonal
// tile, span_I = max_c (G_rc - G_{r+15,c}).  A diagonal tile whose span
// exceeds kSpanMax is computed term by term in fp32 instead.
#include "matrix_common.h"

namespace gdr {
namespace {

using namespace mx;

// ---- per-chunk record (per-channel decay): the common head (T'' and A
// fragments), then the decayed operands of the walk, each fragment 64 lanes x
// 16 bytes: K~ and Q~ as 64 fragments ordered by key block kb, then kind
// (K~ hi, K~ lo, Q~ hi, Q~ lo), then token tile M (f = 16kb + 4kind + M; term
// e of lane group p = key channel 32kb + kperm(p,e)), so each key block is
// one contiguous 16 KiB group; K^ hi, K^ lo (16 fragments each, f = 2i + kb:
// key tile i, token block kb, term e of lane group p = token 32kb +
// kperm(p,e)); then exp(G_63) per key channel (fp32).
constexpr int kPcKq = kRecHead;
constexpr int kPcKu = kPcKq + 64 * kFragBytes;
constexpr int kPcGend = kPcKu + 32 * kFragBytes;
constexpr int kPcBytes = kPcGend + DK * 4;  // 123392, a multiple of 256

constexpr int LG = DK + 4;        // fp32 row stride of the per-channel G in LDS (16-byte aligned rows)
constexpr float kSpanMax = 64.f;  // largest diagonal-tile span taken on the matrix cores

// ============================================================ intra kernel
struct alignas(16) IntraPcSmem {
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
    float G[C * LG];   // in-chunk cumulative log-decay, token-major
    float eta[C];      // beta, or eta for the Kaczmarz step size (0 past the end), then the write strengths
    float kk[C];       // |k_i|^2 (Kaczmarz only)
    float carry[DK];   // G of token 31, added to tokens 32 .. 63
    unsigned span[4];  // span_I as fp32 bits (>= 0, so integer order is float order)
};

template <bool KZ, bool DELTA>
__global__ __launch_bounds__(kIntraThreads, 2) void intra_pc_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, int T, int H, int NC, int total, float eps, float scale,
    char *__restrict__ ws, SeqTable tb) {
    __shared__ IntraPcSmem sm;
    if (tb.start) total = tb.cbase[tb.N] * H;  // packed batch: the chunks the table holds
    if (total <= 0) return;
    const int qk_stride = H * DK * 2, g_stride = H * DK * 4;
    const TriTiles tri{sm.u.t.R, sm.u.t.Toff, sm.u.t.A};
    const int seg = threadIdx.x & 15, i0 = threadIdx.x >> 4;
    const int lane0 = threadIdx.x & 63;
    const int gc = threadIdx.x & 127, gh = threadIdx.x >> 7;  // gate scan: key channel, token half

    // Persistent: the workgroup takes chunks ci = blockIdx.x + k gridDim.x
    // ((b*H + h)*NC + c) and loads the next one's q, k and gates into
    // registers while it computes the current one.  Rows past the end of the
    // sequence read as zero.
    uint4 qv[4], kv[4];
    float gv[32];
    float ev;
    auto prefetch = [&](int cj) {
        size_t r0;
        int nn;
        chunk_place(cj, T, H, NC, tb, r0, nn);
        const auto rk = rows_rsrc(k + r0 * DK, nn, qk_stride, DK * 2);
        const auto rq = rows_rsrc(q + r0 * DK, nn, qk_stride, DK * 2);
        const auto rg = rows_rsrc(g + r0 * DK, nn, g_stride, DK * 4);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int off = (i0 + 16 * it) * qk_stride + 16 * seg;
            qv[it] = buf_ld16(rq, off);
            kv[it] = buf_ld16(rk, off);
        }
#pragma unroll
        for (int m = 0; m < 32; ++m) gv[m] = buf_ld4f(rg, (32 * gh + m) * g_stride + 4 * gc);
        ev = DELTA ? beta[r0 + (size_t)min(lane0, nn - 1) * H] : 0.f;
    };
    prefetch(min((int)blockIdx.x, total - 1));
    for (int ci = blockIdx.x; ci < total; ci += gridDim.x) {
    // The thread index passes through an empty asm each chunk, so per-lane
    // LDS addresses are recomputed per chunk instead of being kept live.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    size_t r0_unused;
    int n;
    chunk_place(ci, T, H, NC, tb, r0_unused, n);
    char *recb = ws + (size_t)ci * kPcBytes;
    barrier_lds();  // the previous chunk's tiles and G are no longer read

    // ---- gates: thread (gc, gh) scans tokens 32gh .. 32gh+31 of key channel gc
    float gl[32];
#pragma unroll
    for (int m = 0; m < 32; ++m) gl[m] = gv[m];
#pragma unroll
    for (int m = 1; m < 32; ++m) gl[m] += gl[m - 1];
    if (gh == 0) sm.carry[gc] = gl[31];
    if (w == 0) sm.eta[lane] = lane < n ? ev : 0.f;
    if (tid < 4) sm.span[tid] = 0u;

    // ---- stage q, k token-major, then start loading the next chunk
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        *reinterpret_cast<uint4 *>(&sm.u.qk.Q[(i0 + 16 * it) * LQK + 8 * seg]) = qv[it];
        *reinterpret_cast<uint4 *>(&sm.u.qk.K[(i0 + 16 * it) * LQK + 8 * seg]) = kv[it];
    }
    prefetch(min(ci + (int)gridDim.x, total - 1));
    barrier_lds();

    if (gh == 1) {
        const float cr = sm.carry[gc];
#pragma unroll
        for (int m = 0; m < 32; ++m) gl[m] += cr;
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) sm.G[(32 * gh + m) * LG + gc] = gl[m];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
        atomicMax(&sm.span[2 * gh + bb], __float_as_uint(fmaxf(gl[16 * bb] - gl[16 * bb + 15], 0.f)));
    if constexpr (KZ) {  // |k_i|^2: four lanes per token, 32 key channels each
        const int i = tid >> 2, qd = tid & 3;
        float s = 0.f;
#pragma unroll
        for (int e8 = 0; e8 < 4; ++e8) {
            const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(&sm.u.qk.K[i * LQK + 32 * qd + 8 * e8]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += static_cast<float>(k8[e]) * static_cast<float>(k8[e]);
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (qd == 0) sm.kk[i] = s;
    }
    barrier_lds();  // G, spans, eta (and |k|^2) in LDS
    if constexpr (KZ) {
        write_strength<KZ>(sm.eta, sm.kk, n, eps, w, lane);
        barrier_lds();
    }

    // ---- decayed operands of the walk into the record
    // K~ and Q~: row i = 16M + l%16, key channels c0 .. c0+3 and c0+16 .. c0+19
    for (int u = tid; u < 16 * 64; u += kIntraThreads) {
        const int f = u >> 6, l = u & 63, M = f >> 2, kb = f & 3, p = l >> 4;
        const int i = 16 * M + (l & 15), c0 = 32 * kb + 4 * p;
        const bf16x4 k0 = *reinterpret_cast<const bf16x4 *>(&sm.u.qk.K[i * LQK + c0]);
        const bf16x4 k1 = *reinterpret_cast<const bf16x4 *>(&sm.u.qk.K[i * LQK + c0 + 16]);
        const bf16x4 q0 = *reinterpret_cast<const bf16x4 *>(&sm.u.qk.Q[i * LQK + c0]);
        const bf16x4 q1 = *reinterpret_cast<const bf16x4 *>(&sm.u.qk.Q[i * LQK + c0 + 16]);
        const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&sm.G[i * LG + c0]);
        const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&sm.G[i * LG + c0 + 16]);
        float kx[8], qx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a0 = __expf(g0[e]), a1 = __expf(g1[e]);
            kx[e] = a0 * static_cast<float>(k0[e]);
            kx[4 + e] = a1 * static_cast<float>(k1[e]);
            qx[e] = scale * a0 * static_cast<float>(q0[e]);
            qx[4 + e] = scale * a1 * static_cast<float>(q1[e]);
        }
        bf16x8 hv, lv;
        char *dst = recb + kPcKq + (16 * kb + M) * kFragBytes + l * 16;
        split8(kx, hv, lv);
        *reinterpret_cast<bf16x8 *>(dst) = hv;
        *reinterpret_cast<bf16x8 *>(dst + 4 * kFragBytes) = lv;
        split8(qx, hv, lv);
        *reinterpret_cast<bf16x8 *>(dst + 8 * kFragBytes) = hv;
        *reinterpret_cast<bf16x8 *>(dst + 12 * kFragBytes) = lv;
    }
    // K^: key channel 16i + l%16, tokens 32kb + kperm(p, e)
    for (int u = tid; u < 16 * 64; u += kIntraThreads) {
        const int f = u >> 6, l = u & 63, ti = f >> 1, kb = f & 1, p = l >> 4;
        const int ch = 16 * ti + (l & 15);
        const float gend = sm.G[(C - 1) * LG + ch];
        float kx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tok = 32 * kb + kperm(p, e);
            kx[e] = __expf(gend - sm.G[tok * LG + ch]) * static_cast<float>(sm.u.qk.K[tok * LQK + ch]);
        }
        bf16x8 hv, lv;
        split8(kx, hv, lv);
        char *dst = recb + kPcKu + f * kFragBytes + l * 16;
        *reinterpret_cast<bf16x8 *>(dst) = hv;
        *reinterpret_cast<bf16x8 *>(dst + 16 * kFragBytes) = lv;
    }
    if (tid < DK) reinterpret_cast<float *>(recb + kPcGend)[tid] = __expf(sm.G[(C - 1) * LG + tid]);

    // ---- R and A on the lower tiles, each wavefront both products of its
    // tiles (I, J): w0 (3,0) (3,1); w1 (3,2) (3,3) (0,0); w2 (2,0) (2,1);
    // w3 (1,0) (1,1) (2,2).  Tiles 0 and 1 have row block Ia, tile 2 row
    // block Ib.
    const int Ia = w < 2 ? 3 : 4 - w;
    const int Ib = w == 1 ? 0 : 2;
    const bool three = (w & 1) != 0;
    const int J0 = w == 1 ? 2 : 0;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 accR[3] = {zero4, zero4, zero4}, accA[3] = {zero4, zero4, zero4};
    {
        // row operands of block I (reference r = 16I): k_i and q_i times exp(G_i - G_r)
        auto row_ops = [&](int I, int kb, bf16x8 &kh, bf16x8 &kl, bf16x8 &qh, bf16x8 &ql) {
            const int i = 16 * I + lr, r = 16 * I, c0 = 32 * kb + 8 * lg;
            const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(&sm.u.qk.K[i * LQK + c0]);
            const bf16x8 q8 = *reinterpret_cast<const bf16x8 *>(&sm.u.qk.Q[i * LQK + c0]);
            float kx[8], qx[8];
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const f32x4 gi = *reinterpret_cast<const f32x4 *>(&sm.G[i * LG + c0 + 4 * h4]);
                const f32x4 gr = *reinterpret_cast<const f32x4 *>(&sm.G[r * LG + c0 + 4 * h4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = __expf(gi[e] - gr[e]);
                    kx[4 * h4 + e] = d * static_cast<float>(k8[4 * h4 + e]);
                    qx[4 * h4 + e] = d * static_cast<float>(q8[4 * h4 + e]);
                }
            }
            split8(kx, kh, kl);
            split8(qx, qh, ql);
        };
        // column operand of tile (I, J): k_j times exp(G_r - G_j), r = 16I
        auto col_ops = [&](int I, int J, int kb, bf16x8 &bh, bf16x8 &bl) {
            const int j = 16 * J + lr, r = 16 * I, c0 = 32 * kb + 8 * lg;
            const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(&sm.u.qk.K[j * LQK + c0]);
            float bx[8];
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const f32x4 gj = *reinterpret_cast<const f32x4 *>(&sm.G[j * LG + c0 + 4 * h4]);
                const f32x4 gr = *reinterpret_cast<const f32x4 *>(&sm.G[r * LG + c0 + 4 * h4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) bx[4 * h4 + e] = __expf(gr[e] - gj[e]) * static_cast<float>(k8[4 * h4 + e]);
            }
            split8(bx, bh, bl);
        };
        auto both = [&](int t, const bf16x8 &kh, const bf16x8 &kl, const bf16x8 &qh, const bf16x8 &ql,
                        const bf16x8 &bh, const bf16x8 &bl) {
            if constexpr (DELTA) {
                accR[t] = mma(kh, bh, accR[t]);
                accR[t] = mma(kh, bl, accR[t]);
                accR[t] = mma(kl, bh, accR[t]);
            }
            accA[t] = mma(qh, bh, accA[t]);
            accA[t] = mma(qh, bl, accA[t]);
            accA[t] = mma(ql, bh, accA[t]);
        };
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            bf16x8 kh, kl, qh, ql, bh, bl;
            row_ops(Ia, kb, kh, kl, qh, ql);
            col_ops(Ia, J0, kb, bh, bl);
            both(0, kh, kl, qh, ql, bh, bl);
            col_ops(Ia, J0 + 1, kb, bh, bl);
            both(1, kh, kl, qh, ql, bh, bl);
            if (three) {
                row_ops(Ib, kb, kh, kl, qh, ql);
                col_ops(Ib, Ib, kb, bh, bl);
                both(2, kh, kl, qh, ql, bh, bl);
            }
        }
    }
    // diagonal tiles whose span is too large for the factored form: every
    // entry j <= i directly, sum_c k_jc exp(G_ic - G_jc) times k_ic (R) and q_ic (A)
    auto direct_tile = [&](int I, f32x4 &aR, f32x4 &aA) {
        const int j = 16 * I + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * lg + r;
            float sR = 0.f, sA = 0.f;
            if (j <= i) {
                for (int c = 0; c < DK; ++c) {
                    const float d = __expf(sm.G[i * LG + c] - sm.G[j * LG + c]) * static_cast<float>(sm.u.qk.K[j * LQK + c]);
                    sR += d * static_cast<float>(sm.u.qk.K[i * LQK + c]);
                    sA += d * static_cast<float>(sm.u.qk.Q[i * LQK + c]);
                }
            }
            aR[r] = sR;
            aA[r] = sA;
        }
    };
    if (three) {  // tile 1 is (Ia, Ia), tile 2 is (Ib, Ib)
        if (__uint_as_float(sm.span[Ia]) > kSpanMax) direct_tile(Ia, accR[1], accA[1]);
        if (__uint_as_float(sm.span[Ib]) > kSpanMax) direct_tile(Ib, accR[2], accA[2]);
    }
    barrier_lds();  // q, k no longer read: the tiles may overwrite them

    // ---- beta (R) and the output scale (A); strictly lower R, lower A
    auto put = [&](int I, int J, const f32x4 &aR, const f32x4 &aA) {
        const int j = 16 * J + lr;
        float *dR = sm.u.t.R + tile_id(I, J) * kTile;
        float *dA = sm.u.t.A + tile_id(I, J) * kTile;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * lg + r;
            dR[(4 * lg + r) * LT + lr] = j < i ? sm.eta[i] * aR[r] : 0.f;
            dA[(4 * lg + r) * LT + lr] = j <= i ? scale * aA[r] : 0.f;
        }
    };
    put(Ia, J0, accR[0], accA[0]);
    put(Ia, J0 + 1, accR[1], accA[1]);
    if (three) put(Ib, Ib, accR[2], accA[2]);
    barrier_lds();

    // ---- T = (I + R)^{-1}, then the T'' and A operand fragments
    if constexpr (DELTA) invert_unit_lower(tri, lane, w, lr, lg);
    pack_T_A<DELTA>(tri, sm.eta, recb, tid);
    }  // chunk loop
}

// ============================================================ state kernel
struct alignas(16) StatePcSmem {
    uint4 Kq0[2][16 * 64];       // key block 0 of K~, Q~ (hi, lo), by chunk parity
    uint4 Kq123[48 * 64];        // key blocks 1..3 of K~, Q~ (hi, lo) of the current chunk
    uint4 Ku[32 * 64];           // K^ hi, K^ lo fragments of the current chunk
    float Gend[DK];              // exp(G_63) per key channel
    __bf16 V[2][C * BV];         // v slice, token-major, 64-byte rows
    uint4 X[2][2][kXFrags][64];  // per chain wavefront and chunk parity: Q~ S, then E
    float Ost[C * 20];           // a helper's fp32 output tile, token-major, for 16-byte stores (the
                                 // helpers form outputs in turn, never at the same time)
};

// PIECES 1 KiB pieces, split over the two helper wavefronts (vt = 0, 1).
template <int PIECES>
__device__ __forceinline__ void copy_to_lds(const char *src, unsigned dst, int vt, int lane) {
#pragma unroll
    for (int j = 0; j < PIECES / 2; ++j) {
        const int p = 2 * j + vt;
        lds_dma16(src + p * 1024 + lane * 16, dst + p * 1024);
    }
}

// Barrier after which data a helper moved into LDS is visible: waits for
// all of this wavefront's global loads (those writing LDS included) and LDS
// operations.
__device__ __forceinline__ void barrier_after_loads() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool OUT_BF16, bool DELTA>
__global__ __launch_bounds__(kStateThreads) void state_pc_kernel(
    const __bf16 *__restrict__ v, const char *__restrict__ ws, const float *__restrict__ s0, void *__restrict__ o,
    float *__restrict__ s_final, int T_all, int H, int NC_all, int BH, SeqTable tb) {
    __shared__ StatePcSmem sm;
    int bh, slice;
    state_slot(blockIdx.x, BH, NS, bh, slice);
    bh = walk_seq(bh, H, tb);  // packed batches: longest sequences first
    const WalkPlace wp = walk_place(bh, 0, NC_all, T_all, H, NC_all, tb, ws, kPcBytes);
    const int NC = wp.nc;                 // chunks of this sequence
    const int T = wp.L;                   // tokens of this sequence
    const size_t rstride = wp.rstride;    // bytes from one chunk's record to the next
    const int j0 = slice * BV;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const char *recs = wp.recs;
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

    // Per chunk c two barriers: A(c) after the chain has read K~, Q~ (the
    // helpers then move key blocks 1..3 of chunk c+1's), B(c) at the end of
    // the chunk (K^, exp(G_63) of chunk c and key block 0 of chunk c+1 are
    // moved between B(c-1) and A(c)).  Every role passes 2 NC + 3 barriers.
    if (w < 2) {
        // ================= chain wavefront: value columns jt .. jt+15
        const int jt = j0 + 16 * w;
        f32x4 S[8];  // S[i][r] = S[16i + 4lg + r][jt + lr]
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[i][r] = s0 ? s0[sbase + (size_t)(16 * i + 4 * lg + r) * DV + jt + lr] : 0.f;
        bf16x8 tAh[6], tAl[6], tBh[6], tBl[6];
        if constexpr (DELTA) {
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                tAh[f] = *reinterpret_cast<const bf16x8 *>(recs + kRecTH + f * kFragBytes + lane * 16);
                tAl[f] = *reinterpret_cast<const bf16x8 *>(recs + kRecTL + f * kFragBytes + lane * 16);
            }
        }
        auto frag = [&](const uint4 *base, int f) { return __builtin_bit_cast(bf16x8, base[f * 64 + lane]); };
        auto step = [&](int c, const bf16x8 *th, const bf16x8 *tl, bf16x8 *thn, bf16x8 *tln)
                        __attribute__((always_inline)) {
            const int buf = c & 1;
            if constexpr (DELTA) {  // next chunk's T'' fragments, in flight during this chunk
                const char *rn = recs + (size_t)min(c + 1, NC - 1) * rstride;
#pragma unroll
                for (int f = 0; f < 6; ++f) {
                    thn[f] = *reinterpret_cast<const bf16x8 *>(rn + kRecTH + f * kFragBytes + lane * 16);
                    tln[f] = *reinterpret_cast<const bf16x8 *>(rn + kRecTL + f * kFragBytes + lane * 16);
                }
            }
            uint4 *xo = &sm.X[buf][w][0][0];
            bf16x8 SH[4], SL[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) pair_split(S[2 * kb], S[2 * kb + 1], SH[kb], SL[kb]);
            // P = K~ S and Q~ S; key block kb+1's fragments are read during
            // block kb's products
            f32x4 P[4] = {zero4, zero4, zero4, zero4};
            f32x4 QS[4] = {zero4, zero4, zero4, zero4};
            bf16x8 fa[2][4][4];  // [stage][K~ hi, K~ lo, Q~ hi, Q~ lo][M]
#pragma unroll
            for (int m4 = DELTA ? 0 : 2; m4 < 4; ++m4)
#pragma unroll
                for (int M = 0; M < 4; ++M) fa[0][m4][M] = frag(sm.Kq0[buf], 4 * m4 + M);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cur = kb & 1;
                if (kb + 1 < 4) {
#pragma unroll
                    for (int m4 = DELTA ? 0 : 2; m4 < 4; ++m4)
#pragma unroll
                        for (int M = 0; M < 4; ++M) fa[cur ^ 1][m4][M] = frag(sm.Kq123, 16 * kb + 4 * m4 + M);
                }
                if constexpr (DELTA) {
#pragma unroll
                    for (int M = 0; M < 4; ++M) {
                        P[M] = mma(fa[cur][0][M], SH[kb], P[M]);
                        P[M] = mma(fa[cur][0][M], SL[kb], P[M]);
                        P[M] = mma(fa[cur][1][M], SH[kb], P[M]);
                    }
                }
#pragma unroll
                for (int M = 0; M < 4; ++M) {
                    QS[M] = mma(fa[cur][2][M], SH[kb], QS[M]);
                    QS[M] = mma(fa[cur][2][M], SL[kb], QS[M]);
                    QS[M] = mma(fa[cur][3][M], SH[kb], QS[M]);
                }
            }
            barrier_lds();  // A(c): key blocks 1..3 of K~, Q~ are no longer read
            // X = V - K~ S (rows 16M + 4lg + r); Q~ S to the helper
            f32x4 Xv[4];
#pragma unroll
            for (int M = 0; M < 4; ++M) {
                // V[16M + 4lg + r][16w + lr], r = 0..3
                const bf16x4 vv = lds_read_tr(&sm.V[buf][(16 * M + 4 * lg + (lr >> 2)) * BV + 16 * w + 4 * (lr & 3)]);
#pragma unroll
                for (int r = 0; r < 4; ++r) Xv[M][r] = DELTA ? static_cast<float>(vv[r]) - P[M][r] : static_cast<float>(vv[r]);
                xo[M * 64 + lane] = *reinterpret_cast<const uint4 *>(&QS[M]);
            }
            bf16x8 XH[2], XL[2];
            if constexpr (DELTA) {
                pair_split(Xv[0], Xv[1], XH[0], XL[0]);
                pair_split(Xv[2], Xv[3], XH[1], XL[1]);
            }
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
                xo[(4 + M) * 64 + lane] = *reinterpret_cast<const uint4 *>(&E[M]);
            }
            bf16x8 EH[2], EL[2];
            pair_split(E[0], E[1], EH[0], EL[0]);
            pair_split(E[2], E[3], EH[1], EL[1]);
            // S <- Diag(exp(G_63)) S + K^^T E, key-channel tile i
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 gd = *reinterpret_cast<const f32x4 *>(&sm.Gend[16 * i + 4 * lg]);
                const bf16x8 u0h = frag(sm.Ku, 2 * i), u1h = frag(sm.Ku, 2 * i + 1);
                const bf16x8 u0l = frag(sm.Ku, 16 + 2 * i), u1l = frag(sm.Ku, 16 + 2 * i + 1);
                f32x4 acc = S[i] * gd;
                acc = mma(u0h, EH[0], acc);
                acc = mma(u0h, EL[0], acc);
                acc = mma(u0l, EH[0], acc);
                acc = mma(u1h, EH[1], acc);
                acc = mma(u1h, EL[1], acc);
                acc = mma(u1l, EH[1], acc);
                S[i] = acc;
            }
            barrier_lds();  // B(c)
        };
        barrier_lds();  // chunk 0's K~, Q~ and v staged
        int c = 0;
        for (; c + 1 < NC; c += 2) {
            step(c, tAh, tAl, tBh, tBl);
            step(c + 1, tBh, tBl, tAh, tAl);
        }
        if (c < NC) step(c, tAh, tAl, tBh, tBl);
        barrier_lds();  // the helpers finish the last chunk's outputs, in turn
        barrier_lds();
        if (s_final) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s_final[sbase + (size_t)(16 * i + 4 * lg + r) * DV + jt + lr] = S[i][r];
        }
    } else {
        // ================= helper wavefronts (vt = 0, 1): both move the
        // decayed operands and the v slice into LDS by global -> LDS copies,
        // half each, and wait for them before each barrier; helper vt forms
        // O = Q~ S + A E of chunk c-1 for the value columns of chain
        // wavefront vt, helper 0 between B(c-1) and A(c), helper 1 between
        // A(c) and B(c).
        const int vt = __builtin_amdgcn_readfirstlane(w - 2);
        const size_t head0 = wp.head0;  // row of token 0 of this sequence and head
        const unsigned lds_kq0 = lds_addr(sm.Kq0), lds_kq123 = lds_addr(sm.Kq123), lds_ku = lds_addr(sm.Ku);
        const unsigned lds_gend = lds_addr(sm.Gend), lds_v = lds_addr(sm.V);
        // v slice of chunk cc, 16 rows per copy (lane l: row l/4, 16-byte
        // segment l%4); rows past the end repeat the last row (any finite
        // value works there: those rows and columns of T'' and A are zero,
        // and so are those tokens' rows of K^, which meet them directly
        // without the delta rule)
        auto copy_v = [&](int cc) {
            const int t0 = cc * C, n = min(C, T - t0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int i = 2 * j + vt;
                const int row = min(16 * i + (lane >> 2), n - 1);
                lds_dma16(v + (head0 + (size_t)(t0 + row) * H) * DV + j0 + 8 * (lane & 3),
                          lds_v + (cc & 1) * (C * BV * 2) + i * 1024);
            }
        };
        auto kq0 = [&](int cc) { return lds_kq0 + (cc & 1) * (16 * 1024); };
        bf16x8 ah[6], al[6], ahn[6], aln[6];
        auto load_out_ops = [&](int cc) {  // chunk cc's A fragments
            const char *rec = recs + (size_t)cc * rstride;
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                ahn[f] = *reinterpret_cast<const bf16x8 *>(rec + kRecAH + f * kFragBytes + lane * 16);
                aln[f] = *reinterpret_cast<const bf16x8 *>(rec + kRecAL + f * kFragBytes + lane * 16);
            }
        };
        auto outputs = [&](int cp) __attribute__((always_inline)) {
            const int t0 = cp * C;
            chunk_outputs<OUT_BF16, false>(&sm.X[cp & 1][vt][0][0], nullptr, 1.f, ah, al, sm.Ost, o,
                                           head0 + (size_t)t0 * H, min(C, T - t0), H, j0 + 16 * vt, lane);
        };
        copy_to_lds<16>(recs + kPcKq, kq0(0), vt, lane);
        copy_to_lds<48>(recs + kPcKq + 16 * 1024, lds_kq123, vt, lane);
        copy_v(0);
        barrier_after_loads();
        for (int c = 0; c < NC; ++c) {
            // chain: K~ S, Q~ S of chunk c (key block 0 from its own buffer)
            const char *rc = recs + (size_t)c * rstride;
            const char *rn = recs + (size_t)min(c + 1, NC - 1) * rstride;
            load_out_ops(c);
            copy_to_lds<32>(rc + kPcKu, lds_ku, vt, lane);
            lds_dma4(rc + kPcGend + vt * 256 + lane * 4, lds_gend + vt * 256);
            copy_to_lds<16>(rn + kPcKq, kq0(c + 1), vt, lane);
            if (c + 1 < NC) copy_v(c + 1);
            if (vt == 0 && c >= 1) outputs(c - 1);
            barrier_after_loads();  // A(c)
            // chain: E and the state update of chunk c
            copy_to_lds<48>(rn + kPcKq + 16 * 1024, lds_kq123, vt, lane);
            if (vt == 1 && c >= 1) outputs(c - 1);
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                ah[f] = ahn[f];
                al[f] = aln[f];
            }
            barrier_after_loads();  // B(c)
        }
        if (vt == 0) outputs(NC - 1);
        barrier_lds();
        if (vt == 1) outputs(NC - 1);
        barrier_lds();
    }
}

// ============================================================ launchers
template <bool KZ, bool DELTA>
hipError_t launch_intra_pc(const ChunkArgs &a) {
    const long total = chunk_slots(a);
    if (total == 0) return hipSuccess;
    GDR_LAUNCH((intra_pc_kernel<KZ, DELTA>), dim3(intra_grid(total, 2)), dim3(kIntraThreads), a.stream, a.ev0, a.ev1,
               static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), a.g, a.beta, a.T, a.H, a.NC,
               (int)total, a.eps, a.scale, static_cast<char *>(a.ws), a.tab);
    return hipGetLastError();
}

template <bool OB, bool DELTA>
hipError_t launch_state_pc(const ChunkArgs &a) {
    const int BH = a.B * a.H;
    GDR_LAUNCH((state_pc_kernel<OB, DELTA>), dim3((unsigned)(BH * NS)), dim3(kStateThreads), a.stream, a.ev0, a.ev1,
               static_cast<const __bf16 *>(a.v), static_cast<const char *>(a.ws), a.s0, a.o, a.s_final, a.T, a.H, a.NC,
               BH, a.tab);
    return hipGetLastError();
}

}  // namespace

size_t chunk_matrix_pc_workspace_bytes(int B, int H, int NC) { return (size_t)B * H * NC * kPcBytes; }

hipError_t launch_chunk_matrix_pc(const ChunkArgs &a, int stage) {
    if (stage != 1) {
        const hipError_t e = !a.delta ? launch_intra_pc<false, false>(a)
                             : a.kaczmarz ? launch_intra_pc<true, true>(a) : launch_intra_pc<false, true>(a);
        if (e != hipSuccess || stage == 0) return e;
    }
    if (!a.delta) return a.o_bf16 ? launch_state_pc<true, false>(a) : launch_state_pc<false, false>(a);
    return a.o_bf16 ? launch_state_pc<true, true>(a) : launch_state_pc<false, true>(a);
}

}  // namespace gdr
