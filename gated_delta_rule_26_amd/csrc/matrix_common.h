// Device pieces shared by the matrix-core chunked kernels (scalar decay in
// chunk_matrix.hip, per-channel decay in chunk_matrix_pc.hip): MFMA operand
// layout, bf16 hi/lo splitting, raw buffer access, the triangular inverse of
// a chunk and the packing of T'' and A into MFMA operand fragments, and the
// output stage of the state walk.
//
// Layout.  v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] (e = 0..7) and D[4(l/16)+r][l%16] (r = 0..3).  A
// reduction may take its 32 terms (per 32-block) in any order shared by
// both operands; the walk uses, for lane group p = l/16, indices
// {4p..4p+3} and {16+4p..16+4p+3} of the block, which is exactly what two
// stacked D tiles hold.  So a D tile (the state, X, E) is directly the B
// operand of the next product, and the other operand is stored or loaded in
// that permuted order.
//
// Precision.  Every fp32-derived operand is split into bf16 hi + lo and
// multiplied as hi*x + lo*x (hi*hi + hi*lo + lo*hi when both sides are
// split), which carries ~16 significant bits.
#pragma once

#include "gdr_internal.h"

namespace gdr {
namespace mx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;  // 64 tokens per chunk
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

// Two fp32 values as bf16 hi (round to nearest even) and lo (the rounded
// residual), each pair packed in one 32-bit word: element 0 in the low half.
// The hi values are recovered from the packed word by a shift and a mask,
// so a pair costs two conversions, two bit operations and two subtractions.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    const bf16x2 h = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
    hi = __builtin_bit_cast(uint32_t, h);
    const bf16x2 l = {static_cast<__bf16>(x0 - __uint_as_float(hi << 16)),
                      static_cast<__bf16>(x1 - __uint_as_float(hi & 0xffff0000u))};
    lo = __builtin_bit_cast(uint32_t, l);
}

// Two stacked D tiles (block rows 0..15 and 16..31) as one permuted operand,
// split into bf16 hi and lo.
__device__ __forceinline__ void pair_split(f32x4 t0, f32x4 t1, bf16x8 &hi, bf16x8 &lo) {
    uint4 h, l;
    split2(t0[0], t0[1], h.x, l.x);
    split2(t0[2], t0[3], h.y, l.y);
    split2(t1[0], t1[1], h.z, l.z);
    split2(t1[2], t1[3], h.w, l.w);
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Eight fp32 values as bf16 hi + lo.
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
    uint4 h, l;
    split2(x[0], x[1], h.x, l.x);
    split2(x[2], x[3], h.y, l.y);
    split2(x[4], x[5], h.z, l.z);
    split2(x[6], x[7], h.w, l.w);
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// ---- per-chunk record, common head: T'' hi, T'' lo, A hi, A lo, each the six
// 16x32 operand fragments (M, kb) of its lower triangle -- (0,0) (1,0) (2,0)
// (2,1) (3,0) (3,1), rows 16M .. 16M+15, tokens 32kb .. 32kb+31 in the
// permuted order -- as 64 lanes x 16 bytes.
constexpr int kFragBytes = 64 * 16;
constexpr int kRecTH = 0;
constexpr int kRecTL = 6 * kFragBytes;
constexpr int kRecAH = 12 * kFragBytes;
constexpr int kRecAL = 18 * kFragBytes;
constexpr int kRecHead = 24 * kFragBytes;
// The record of scalar decay: the head, then exp(G_i) and exp(G_63 - G_i) of
// the 64 tokens (fp32; past the end of a partial chunk G stays at its last
// value).  Written by the forward intra kernel and by the backward's prep.
constexpr int kRecGam = kRecHead;
constexpr int kRecGend = kRecGam + C * 4;
constexpr int kRecBytes = kRecGend + C * 4;  // 25088, a multiple of 256
__host__ __device__ constexpr int lower_frag(int M, int kb) { return M < 2 ? M : 2 * M - 2 + kb; }
__host__ __device__ constexpr int frag_M(int f) { return f < 2 ? f : 2 + ((f - 2) >> 1); }
__host__ __device__ constexpr int frag_kb(int f) { return f < 2 ? 0 : (f - 2) & 1; }

// Raw buffer resource over `rows` rows of `row_bytes` bytes spaced `stride`
// bytes apart, starting at `base`: loads past the last row return zero and
// stores past it are dropped, with no branch in the instruction stream
// (0x00020000 is the gfx9-family descriptor word for untyped 32-bit data).
// With rows <= 0 every load returns zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *base, int rows, int stride, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             rows > 0 ? (rows - 1) * stride + row_bytes : 0, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// ---- chunk triangle in LDS: 16x16 fp32 tiles, row stride LT
constexpr int kIntraThreads = 256;

// Chunk ci of the intra kernels' order: the [.., H, D] row of its first token
// and its token count.  Fixed-length batch: ci = (b H + h) NC + c; packed
// batch: ci = u H + h for chunk u of the table.
__device__ __forceinline__ void chunk_place(int ci, int T, int H, int NC, const SeqTable &tb, size_t &row0, int &n) {
    if (tb.start) {
        const int u = ci / H, h = ci - u * H;
        const int t0 = tb.tok[u];
        n = min(C, tb.start[tb.seq[u] + 1] - t0);
        row0 = (size_t)t0 * H + h;
    } else {
        const int c = ci % NC, bh = ci / NC;
        const int t0 = c * C;
        n = min(C, T - t0);
        row0 = ((size_t)(bh / H) * T + t0) * H + bh % H;
    }
}

// The chunks one walk covers: sequence `bh / H` (head bh % H), chunks c0 ..
// c0 + nc - 1 of it, the [.., H, D] row of its token 0, its length L, and
// the byte address and stride of its chunk records (rec_bytes each).
struct WalkPlace {
    size_t head0;
    int L, nc;
    const char *recs;
    size_t rstride;
};
__device__ __forceinline__ WalkPlace walk_place(int bh, int c0, int seg, int T, int H, int NC, const SeqTable &tb,
                                                const char *ws, size_t rec_bytes) {
    const int b = bh / H, h = bh - b * H;
    WalkPlace w;
    if (tb.start) {
        const int s = tb.start[b], cb = tb.cbase[b];
        w.L = tb.start[b + 1] - s;
        w.head0 = (size_t)s * H + h;
        w.nc = min(seg, tb.cbase[b + 1] - cb - c0);
        w.rstride = (size_t)H * rec_bytes;
        w.recs = ws + ((size_t)(cb + c0) * H + h) * rec_bytes;
    } else {
        w.L = T;
        w.head0 = (size_t)b * T * H + h;
        w.nc = min(seg, NC - c0);
        w.rstride = rec_bytes;
        w.recs = ws + ((size_t)bh * NC + c0) * rec_bytes;
    }
    return w;
}
constexpr int LT = 20;           // fp32 row stride of a 16x16 tile in LDS (16-byte aligned rows)
constexpr int LQK = DK + 8;      // bf16 row stride of the staged q, k (token-major)
constexpr int kTile = 16 * LT;   // floats per tile
__host__ __device__ constexpr int tile_id(int I, int J) { return I * (I + 1) / 2 + J; }     // lower tiles 0..9
__host__ __device__ constexpr int offdiag_id(int I, int J) { return I * (I - 1) / 2 + J; }  // J < I: 0..5

// The lower tiles of R (strictly lower part used), T and A.  T's diagonal
// blocks overwrite R's (R_II is not needed once T_II is known; R_IJ with
// J < I is).
struct TriTiles {
    float *R;     // 10 tiles
    float *Toff;  // 6 strictly lower tiles of T
    float *A;     // 10 tiles
    __device__ __forceinline__ float *Tb(int I, int J) const {
        return I == J ? &R[tile_id(I, I) * kTile] : &Toff[offdiag_id(I, J) * kTile];
    }
};

// Workgroup barrier for data exchanged through LDS only: waits for this
// wavefront's LDS operations, not for its global loads, so loads issued for a
// later chunk stay in flight across it (a full __syncthreads also waits for
// every outstanding global load).  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// T = (I + R)^{-1} for the unit lower-triangular I + R of one chunk, by all
// 256 threads: the 16x16 diagonal blocks by forward substitution (wavefront w
// takes block w, one column per lane, rows read ahead with 16-byte reads),
// then three levels of off-diagonal blocks on fp32 MFMA,
//   T_IJ = -T_II sum_{M=J}^{I-1} R_IM T_MJ.
// Starts after a barrier that published R; ends with a barrier.
__device__ __forceinline__ void invert_unit_lower(const TriTiles &t, int lane, int w, int lr, int lg) {
    if (lane < 16) {
        const int cc = lane;
        float *blk = &t.R[tile_id(w, w) * kTile];
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
    barrier_lds();
    auto inverse_tile = [&](int I, int J) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        for (int M = J; M < I; ++M) {
            const float *Rt = &t.R[tile_id(I, M) * kTile];
            const float *Tt = t.Tb(M, J);
#pragma unroll
            for (int s = 0; s < 4; ++s) P = mma32(Rt[lr * LT + 4 * lg + s], Tt[(4 * lg + s) * LT + lr], P);
        }
        const float *Tii = t.Tb(I, I);
        f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) out = mma32(Tii[lr * LT + 4 * lg + s], P[s], out);
        float *dst = t.Tb(I, J);
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * lg + r) * LT + lr] = -out[r];
    };
    if (w < 3) inverse_tile(w + 1, w);
    barrier_lds();
    if (w < 2) inverse_tile(w + 2, w);
    barrier_lds();
    if (w == 0) inverse_tile(3, 0);
    barrier_lds();
}

// The write strength of the chunk's tokens in place: beta stays; for the
// Kaczmarz step size eta_j becomes eta_j / (|k_j|^2 + eps) (zero past the
// end of a partial chunk).  One wavefront, one token per lane; the caller
// synchronises before and after.
template <bool KZ>
__device__ __forceinline__ void write_strength(float *eta, const float *kk, int n, float eps, int w, int lane) {
    if constexpr (KZ) {
        if (w == 0) eta[lane] = lane < n ? eta[lane] / (kk[lane] + eps) : 0.f;
    }
}

// Operand fragments of T'' = T Diag(beta) and A, lower triangle only, bf16
// hi + lo, into the record's head (beta: the chunk's write strengths; A only
// when WITH_T is false).  Terms 0..3 of lane group p are tile columns
// 4p .. 4p+3 of tile (M, 2kb), terms 4..7 the same columns of tile (M, 2kb + 1).
template <bool WITH_T = true>
__device__ __forceinline__ void pack_T_A(const TriTiles &t, const float *beta, char *recb, int tid) {
    for (int u = tid + (WITH_T ? 0 : 6 * 64); u < 2 * 6 * 64; u += kIntraThreads) {
        const int mat = u / 384, f = (u >> 6) % 6, l = u & 63;
        const int M = frag_M(f), kb = frag_kb(f), rr = l & 15, p = l >> 4;
        bf16x8 hv, lv;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int J = 2 * kb + half;
            f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
            if (J <= M) {
                const float *tile = mat == 0 ? t.Tb(M, J) : &t.A[tile_id(M, J) * kTile];
                x4 = *reinterpret_cast<const f32x4 *>(&tile[rr * LT + 4 * p]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 4 * p + e;
                float x = (J < M || (J == M && col <= rr)) ? x4[e] : 0.f;
                if (mat == 0) x *= beta[16 * J + col];
                hv[4 * half + e] = static_cast<__bf16>(x);
                lv[4 * half + e] = static_cast<__bf16>(x - static_cast<float>(hv[4 * half + e]));
            }
        }
        char *dst = recb + (mat == 0 ? kRecTH : kRecAH) + f * kFragBytes + l * 16;
        *reinterpret_cast<bf16x8 *>(dst) = hv;
        *reinterpret_cast<bf16x8 *>(dst + 6 * kFragBytes) = lv;
    }
}

// ---- the backward pass's reverse record of a chunk (scalar decay): the transposes of T'' and A as
// bf16 hi + lo A-operand fragments of their upper triangles, for the reverse walk and the gradients.
constexpr int kRevTH = 0;                    // T''' hi, lo; A' hi, lo: six fragments each
constexpr int kRevTL = 6 * kFragBytes;
constexpr int kRevAH = 12 * kFragBytes;
constexpr int kRevAL = 18 * kFragBytes;
constexpr int kRevBytes = 24 * kFragBytes;
// Upper-triangular fragment f (M, kb): rows 16 M .. of a 64 x 64 matrix, columns 32 kb + kperm(p, e).
__host__ __device__ constexpr int upper_frag(int M, int kb) { return M < 2 ? 2 * M + kb : M + 2; }
__host__ __device__ constexpr int ufrag_M(int f) { return f < 4 ? f >> 1 : f - 2; }
__host__ __device__ constexpr int ufrag_kb(int f) { return f < 4 ? f & 1 : 1; }

// The reverse record from a chunk's tiles (T, A in LDS as the intra kernels keep them): T''' = Diag(beta) T'
// and A' (A' only when WITH_T is false), by kIntraThreads threads.
template <bool WITH_T>
__device__ __forceinline__ void pack_reverse(const TriTiles &t, const float *beta, char *dst, int tid) {
    for (int u = tid + (WITH_T ? 0 : 6 * 64); u < 2 * 6 * 64; u += kIntraThreads) {
        const int mat = u / 384, f = (u >> 6) % 6, l = u & 63;
        const int i = 16 * ufrag_M(f) + (l & 15), p = l >> 4, kb = ufrag_kb(f);
        bf16x8 hv, lv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 32 * kb + kperm(p, e);
            float x = 0.f;
            if (j >= i) {
                const int I = i >> 4, J = j >> 4, at = (j & 15) * LT + (i & 15);
                x = mat == 0 ? t.Tb(J, I)[at] * beta[i] : t.A[tile_id(J, I) * kTile + at];
            }
            hv[e] = static_cast<__bf16>(x);
            lv[e] = static_cast<__bf16>(x - static_cast<float>(hv[e]));
        }
        char *d = dst + (mat == 0 ? kRevTH : kRevAH) + f * kFragBytes + l * 16;
        *reinterpret_cast<bf16x8 *>(d) = hv;
        *reinterpret_cast<bf16x8 *>(d + 6 * kFragBytes) = lv;
    }
}

// ---- state walk
constexpr int kStateThreads = 256;  // chain wavefronts 0, 1; helper wavefronts 2, 3
constexpr int BV = 32;              // value columns per workgroup
constexpr int NS = DV / BV;         // workgroups per (sequence, head)
constexpr int LDV = BV + 8;         // bf16 row stride of the token-major v slice
constexpr int kXFrags = 8;          // chain -> helper: the read Q S and E (4 fp32 tiles each)


// ds_read_b64_tr_b16 (gfx950): every lane names 8 bytes (four bf16) of LDS;
// within each group of 16 lanes, element e of lane i of the result is element
// i % 4 of the 8 bytes named by lane 4e + i / 4 of the group.  So if lane j of
// group p names elements c0 + 4 (j % 4) .. +3 of row r0 + 4p + j / 4 of a
// row-major matrix, lane (i, p) receives rows r0 + 4p + e, e = 0..3, of column
// c0 + i: a transposed 4x16 block, as MFMA fragments and D tiles hold it.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// k and q staged token-major in LDS (rows of ld bf16) with the key channels
// of each 32-block permuted, so that a 16-byte read at row r, column 32 kb +
// 8 p holds channels 32 kb + kperm(p, 0..7): the A operand of a product over
// key channels.  kperm_col: the column of the 8-byte half hh (0, 1) of key
// channel segment seg (8 channels, 0..15).
__device__ __forceinline__ int kperm_col(int seg, int hh) {
    const int s = seg & 3;
    return 32 * (seg >> 2) + 8 * ((2 * s + hh) & 3) + 4 * (s >> 1);
}
// The transposed A operand of that layout (key channel tile i, token block
// kb): term e of lane group lg is token 32 kb + kperm(lg, e), key channel
// 16 i + lr, by transposing reads.
__device__ __forceinline__ bf16x8 kt_operand(const __bf16 *s, int ld, int i, int kb, int lr, int lg) {
    const int col = 32 * (i >> 1) + 8 * (lr & 3) + 4 * (i & 1);  // 16 i + 4 (lr % 4), permuted
    const int row = 32 * kb + 4 * lg + (lr >> 2);
    const bf16x4 a = lds_read_tr(&s[row * ld + col]);
    const bf16x4 c = lds_read_tr(&s[(row + 16) * ld + col]);
    return bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
}

// Global -> LDS copies without registers (global_load_lds, gfx950): every
// lane moves 16 (or 4) bytes from its own global address to LDS address
// M0 + 16 lane (4 lane).  Issued from inline asm, which saves and restores M0:
// the compiler then does not make later LDS accesses of this wavefront wait
// for the copy (they touch other buffers); the copies complete at an explicit
// s_waitcnt vmcnt before the barrier that publishes them.  The hardware
// counts them in vmcnt, so the compiler's own wait counts for other loads can
// only get stricter.  One wait state separates the M0 write from the copy
// that reads it.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)(p))));
}
__device__ __forceinline__ void lds_dma16(const void *src, unsigned lds) {
    int saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void *src, unsigned lds) {
    int saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src) : "memory");
}

// XCD-aware placement of the state walk's workgroups: consecutive workgroup
// ids go to different XCDs, so the nsl slices of one group (sequence, head,
// time segment) get ids that are equal modulo 8 and share that XCD's L2 for
// q, k, v and the chunk records.
__device__ __forceinline__ void state_slot(int x, int groups, int nsl, int &g, int &slice) {
    if ((groups & 7) == 0) {
        const int xcd = x & 7, r = x >> 3;
        g = (r / nsl) * 8 + xcd;
        slice = r % nsl;
    } else {
        g = x / nsl;
        slice = x % nsl;
    }
}

// Outputs of one chunk on a helper wavefront: O = QS + A E, where QS (the
// read of the state) and E (fp32) come from the chain wavefront of value
// columns jt .. jt+15 through LDS (xi: 8 tiles of 64 lanes x 16 bytes) and
// ah, al are the A fragments.  With ROW_SCALE, QS still lacks the output
// scale and the decay of its token (row i is multiplied by scale
// row_scale[i] here); otherwise it is final.  Rows past the end of the
// sequence are dropped by the buffer bounds.  The output tile goes through
// the LDS area `ost` (rows of 20 floats, or of 24 bf16 elements; it may be xi
// itself, and holds at least 5,120 bytes) so that each lane stores 16-byte
// pieces of rows.
template <bool OUT_BF16, bool ROW_SCALE>
__device__ __forceinline__ void chunk_outputs(const uint4 *xi, const float *row_scale, float scale,
                                              const bf16x8 *ah, const bf16x8 *al, float *ost, void *o, size_t row0,
                                              int n, int H, int jt, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 O[4], E[4];
    bf16x8 eh[2], el[2];
#pragma unroll
    for (int M = 0; M < 4; ++M) {
        *reinterpret_cast<uint4 *>(&O[M]) = xi[M * 64 + lane];
        *reinterpret_cast<uint4 *>(&E[M]) = xi[(4 + M) * 64 + lane];
        if constexpr (ROW_SCALE) {
            const f32x4 rs = *reinterpret_cast<const f32x4 *>(&row_scale[16 * M + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) O[M][r] *= scale * rs[r];
        }
    }
    // ost may overlay xi (a caller whose xi is free once read): no LDS store
    // below may be moved above these loads (one wavefront's LDS operations
    // complete in order, so the hardware keeps them apart).
    __asm__ volatile("" ::: "memory");
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
    constexpr int es = OUT_BF16 ? 2 : 4;
    const auto ro = rows_rsrc(static_cast<char *>(o) + row0 * DV * es, n, H * DV * es, DV * es);
    if constexpr (OUT_BF16) {
        // the same through a bf16 tile (rows of 24 elements, 48 bytes): each
        // lane stores two 16-byte half rows of 8 output columns
        __bf16 *ob = reinterpret_cast<__bf16 *>(ost);
#pragma unroll
        for (int M = 0; M < 4; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) ob[(16 * M + 4 * lg + r) * 24 + lr] = static_cast<__bf16>(O[M][r]);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int row = 32 * it + (lane >> 1), c8 = 8 * (lane & 1);
            const uint4 val = *reinterpret_cast<const uint4 *>(&ob[row * 24 + c8]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, val),
                                                   ro, (row * H * DV + jt + c8) * es, 0, 0);
        }
    } else {
        // one 16-byte store per lane covers 4 output columns (same wavefront,
        // so no barrier)
#pragma unroll
        for (int M = 0; M < 4; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) ost[(16 * M + 4 * lg + r) * 20 + lr] = O[M][r];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = 16 * it + (lane >> 2), c4 = 4 * (lane & 3);
            const uint4 val = *reinterpret_cast<const uint4 *>(&ost[row * 20 + c4]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, val),
                                                   ro, (row * H * DV + jt + c4) * 4, 0, 0);
        }
    }
}

// Workgroups of a persistent intra kernel: `per_cu` per compute unit, or one
// per chunk when there are fewer chunks.
int intra_grid(long total, int per_cu);

}  // namespace mx
}  // namespace gdr
