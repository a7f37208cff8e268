// Internal declarations shared by the libgdr sources (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdr.h"

namespace gdr {

constexpr int kChunk = 64;

// The sequences of a variable-length (packed) batch, as device tables built
// from cu_seqlens by launch_seq_table at the start of the workspace.  With
// start == nullptr the batch has B sequences of T tokens each.
struct SeqTable {
    const int *start = nullptr;  // [N+1] first token of sequence n (clamped, non-decreasing; start[N] <= T)
    const int *cbase = nullptr;  // [N+1] first chunk of sequence n; cbase[N] = number of chunks
    const int *tok = nullptr;    // [chunk bound] first token of chunk u
    const int *seq = nullptr;    // [chunk bound] sequence of chunk u
    const int *order = nullptr;  // [N] the sequence walked at rank r: longest first (see seq_table_kernel)
    int N = 0;
};
// Chunk bound of N packed sequences of T tokens in all: floor((T + 63 N) / 64).
int varlen_max_chunks(int N, int T);
size_t seq_table_bytes(int N, int NCmax);
SeqTable seq_table(void *ws, int N, int NCmax);
hipError_t launch_seq_table(const int *cu, int N, int T, void *ws, hipStream_t stream);

// Validated arguments of gdr_chunk_fwd, as the launchers see them.  For a
// packed batch B = N sequences, T = tokens in all, NC = the chunk bound, ws
// = the workspace after the table, and the records of chunk u of head h are
// record u * H + h (for a fixed-length batch: (b * H + h) * NC + c).
struct ChunkArgs {
    int B, T, H, Dk, Dv;
    int NC;                  // chunks per sequence, ceil(T / 64) (packed: the chunk bound)
    SeqTable tab;            // packed batches only
    bool qkv_bf16, o_bf16, per_channel, kaczmarz;
    bool delta;              // false: additive write S = D S + k v^T (beta is NULL)
    float eps, scale;
    const void *q, *k, *v;
    const float *g, *beta;
    const float *s0;         // may be NULL (zero start)
    void *o;
    float *s_final;          // may be NULL
    void *ws;
    hipStream_t stream;
    hipEvent_t ev0 = nullptr;  // a timed stage: recorded when its first kernel begins
    hipEvent_t ev1 = nullptr;  //   and when its last kernel ends
};

// Kernel launch that records E0 when the kernel begins and E1 when it ends
// (hipExtLaunchKernelGGL) if either is non-null; otherwise a plain launch.
#define GDR_LAUNCH(K, GRID, BLOCK, STREAM, E0, E1, ...)                                        \
    do {                                                                                       \
        if ((E0) || (E1))                                                                      \
            hipExtLaunchKernelGGL(K, GRID, BLOCK, 0, STREAM, E0, E1, 0, __VA_ARGS__);          \
        else                                                                                   \
            hipLaunchKernelGGL(K, GRID, BLOCK, 0, STREAM, __VA_ARGS__);                        \
    } while (0)

// Number of chunk records (chunks times heads) the kernels are launched for.
inline long chunk_slots(const ChunkArgs &a) {
    return a.tab.start ? (long)a.NC * a.H : (long)a.B * a.H * a.NC;
}

// Validated arguments of gdr_recurrent_step (T = 1) and gdr_recurrent_fwd.
struct StepArgs {
    int N, T, H, Dk, Dv;
    bool qkv_bf16, o_bf16, per_channel, kaczmarz;
    bool delta;              // false: additive write S = D S + k v^T (beta is NULL)
    float eps, scale;
    const void *q, *k, *v;
    const float *g, *beta;
    float *state;
    void *o;
    hipStream_t stream;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;  // a timed step: recorded when the kernel begins and ends
    const int *cu = nullptr;  // packed batch: N + 1 token offsets (device), T = tokens in all
};

// Vector-ALU chunked path (fp32 arithmetic, any input dtype).
size_t chunk_vector_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel);
// stage: -1 = both kernels, 0 = intra kernel only, 1 = state kernel only
hipError_t launch_chunk_vector(const ChunkArgs &a, int stage);

// Matrix-core chunked path: bf16 MFMA with fp32 accumulation for bf16 inputs
// at Dk = Dv = 128, fp32 MFMA tiles for every other input (see below).
// packed: records only (a packed batch is walked one sequence per walk, no time segments)
size_t chunk_matrix_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel, bool packed,
                                    bool qkv_bf16);
bool chunk_matrix_supported(int Dk, int Dv, bool qkv_bf16, bool per_channel);
hipError_t launch_chunk_matrix(const ChunkArgs &a, int stage);
// Its fp32-tile kernels (fp32 q/k/v, or a width of 64): the backward pass's
// per-chunk prep, then a walk that forms the outputs (chunk_bwd.hip).
size_t chunk_tile_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel);
hipError_t launch_chunk_tile(const ChunkArgs &a, int stage);
// The state entering every chunk, for the backward pass (bf16 inputs at
// Dk = Dv = 128, scalar decay): the bf16 walk without outputs over the chunk
// records at a.ws (mx::kRecBytes each, in the intra kernel's format, written
// by the caller), the states to `states` at the records' indices ([Dk][Dv]
// fp32 each).  Long sequences of a fixed-length batch walk in time segments,
// whose chunk maps and entering states take chunk_states_segment_bytes(B H,
// NC) right after the records.
size_t chunk_states_segment_bytes(int BH, int NC);
int chunk_walk_segments(int BH, int NC);  // the time segments of those walks (1: none)
hipError_t launch_chunk_states(const ChunkArgs &a, float *states);
// Its per-chunk inputs (the same case): the intra kernel's records into a.ws and, per chunk, T (fp32, 64 x
// 64), G and the write strengths (64 each) and the reverse record (the transposes of T'' and A as bf16
// hi/lo fragments, mx::kRevBytes) at the records' indices.
hipError_t launch_chunk_prep_bwd(const ChunkArgs &a, float *T, float *G, float *beta, char *rrev);
// Its per-channel-decay kernels (called by the two functions above).
size_t chunk_matrix_pc_workspace_bytes(int B, int H, int NC);
hipError_t launch_chunk_matrix_pc(const ChunkArgs &a, int stage);

// Validated arguments of gdr_chunk_bwd (fixed-length batches).
struct BwdArgs {
    int B, T, H, Dk, Dv, NC;     // packed batch: B = N sequences, T = tokens in all, NC = the chunk bound
    SeqTable tab;                // packed batches only
    bool qkv_bf16, per_channel, kaczmarz;
    bool delta;                                  // false: additive write (beta and dbeta are NULL)
    float eps, scale;
    const void *q, *k, *v;
    const float *g, *beta, *s0, *dO, *ds_final;  // s0, ds_final may be NULL (zero)
    float *dq, *dk, *dv, *dg, *dbeta, *ds0;      // ds0 may be NULL
    void *ws;
    hipStream_t stream;
};
// Backward pass (fp32 vector kernels).
size_t chunk_bwd_workspace_bytes(int B, int H, int NC, int Dk, int Dv, bool per_channel, bool qkv_bf16);
hipError_t launch_chunk_bwd(const BwdArgs &a);

// T == 0: s_final = s0 (or zero).
hipError_t launch_state_init(float *dst, const float *src, size_t n, hipStream_t stream);

// Fused recurrent steps over T >= 1 tokens per sequence.
hipError_t launch_recurrent_step(const StepArgs &a);

}  // namespace gdr

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
namespace gdr {

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (quiet NaN kept).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_in(const void *p, size_t i) {
    if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_out(void *p, size_t i, float x) {
    if constexpr (BF16) static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(x);
    else static_cast<float *>(p)[i] = x;
}

// The (sequence, head) that walk slot x (= rank * H + head) takes in a packed
// batch: sequences in the table's walk order, longest first, so that the
// longest walks are dispatched first; fixed-length batches (no table) and
// the identity order leave x as it is.
__device__ __forceinline__ int walk_seq(int x, int H, const SeqTable &tb) {
    return tb.order ? tb.order[x / H] * H + x % H : x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace gdr
#endif
