// libgdr C ABI: argument validation (pure host code, before any HIP call)
// and dispatch to the kernels.  See include/gdr.h for the contract.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "gdr_internal.h"

namespace {

using gdr::ChunkArgs;
constexpr size_t kChunkRows = gdr::kChunk;
using gdr::StepArgs;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

Range range_of(const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a*b*... with overflow detection (all factors >= 0)
bool mul_ok(size_t &acc, size_t f) {
    if (f != 0 && acc > SIZE_MAX / f) return false;
    acc *= f;
    return true;
}

struct Sizes {
    size_t qk, v, g, beta, state, o;  // element counts
};

// Shared descriptor validation.  `step` selects the recurrent readings (no
// chunk constraint; T = 1 for the single step when `one_token`); `packed`
// the packed batch (B sequences sharing T tokens in all).
int check_desc(const gdr_desc *d, bool step, Sizes *sz, bool one_token = true, bool packed = false) {
    if (!d) return GDR_E_NULL;
    if (d->delta_mode != GDR_DELTA_RULE && d->delta_mode != GDR_DELTA_OFF) return GDR_E_MODE;
    const bool delta = d->delta_mode == GDR_DELTA_RULE;  // beta_mode and eps matter only then
    if (d->qkv_dtype != GDR_F32 && d->qkv_dtype != GDR_BF16) return GDR_E_MODE;
    if (d->o_dtype != GDR_F32 && d->o_dtype != GDR_BF16) return GDR_E_MODE;
    if (d->decay_mode != GDR_DECAY_SCALAR && d->decay_mode != GDR_DECAY_PER_CHANNEL) return GDR_E_MODE;
    if (delta && d->beta_mode != GDR_BETA_GIVEN && d->beta_mode != GDR_BETA_KACZMARZ) return GDR_E_MODE;
    if (d->algo != GDR_ALGO_AUTO && d->algo != GDR_ALGO_VECTOR && d->algo != GDR_ALGO_MATRIX) return GDR_E_MODE;
    if (!std::isfinite(d->scale)) return GDR_E_MODE;
    if (delta && d->beta_mode == GDR_BETA_KACZMARZ && !(std::isfinite(d->eps) && d->eps >= 0.f))
        return GDR_E_MODE;
    const int T = step && one_token ? 1 : d->T;
    if (d->B < 0 || d->H < 0 || T < 0 || d->Dk < 0 || d->Dv < 0) return GDR_E_SHAPE;
    if (!(d->Dk == 64 || d->Dk == 128) || !(d->Dv == 64 || d->Dv == 128)) return GDR_E_UNSUPPORTED;
    if (!step && d->chunk != gdr::kChunk) return GDR_E_UNSUPPORTED;
    size_t tok = 1;  // B*T*H (packed: T*H)
    if (!mul_ok(tok, packed ? 1 : (size_t)d->B) || !mul_ok(tok, (size_t)T) || !mul_ok(tok, (size_t)d->H))
        return GDR_E_SHAPE;
    size_t qk = tok, vv = tok, st = (size_t)d->B;
    if (!mul_ok(qk, (size_t)d->Dk) || !mul_ok(vv, (size_t)d->Dv)) return GDR_E_SHAPE;
    if (!mul_ok(st, (size_t)d->H) || !mul_ok(st, (size_t)d->Dk) || !mul_ok(st, (size_t)d->Dv)) return GDR_E_SHAPE;
    // byte counts and 64-bit kernel offsets must fit comfortably
    const size_t lim = (size_t)1 << 60;
    if (qk > lim || vv > lim || st > lim) return GDR_E_SHAPE;
    // grid-size limits of the launches (blocks per dimension < 2^31)
    if ((size_t)d->B * d->H * 2 >= ((size_t)1 << 31)) return GDR_E_SHAPE;
    // the chunk kernels address the rows of one chunk ([64 tokens, H, D], up to 4-byte elements) with
    // 32-bit byte offsets
    if (!step && (size_t)kChunkRows * d->H * (size_t)(d->Dk > d->Dv ? d->Dk : d->Dv) * 4 >= ((size_t)1 << 31))
        return GDR_E_SHAPE;
    if (sz) {
        sz->qk = qk;
        sz->v = vv;
        sz->g = d->decay_mode == GDR_DECAY_PER_CHANNEL ? qk : tok;
        sz->beta = delta ? tok : 0;  // beta_or_eta is not read without the delta rule
        sz->state = st;
        sz->o = vv;
    }
    return GDR_OK;
}

// AUTO takes the matrix-core kernels: bf16 MFMA for bf16 q/k/v at d128, fp32
// MFMA tiles for every other input.
int resolve_algo(const gdr_desc *d) { return d->algo == GDR_ALGO_AUTO ? GDR_ALGO_MATRIX : d->algo; }

bool matrix_path_available(const gdr_desc *d) {
    return gdr::chunk_matrix_supported(d->Dk, d->Dv, d->qkv_dtype == GDR_BF16,
                                       d->decay_mode == GDR_DECAY_PER_CHANNEL);
}

// Chunks per sequence (fixed length), or the chunk bound of a packed batch.
long chunk_count(const gdr_desc *d, bool packed) {
    return packed ? ((long)d->T + 63L * d->B) / gdr::kChunk : ((long)d->T + gdr::kChunk - 1) / gdr::kChunk;
}

// Workspace bytes; for a packed batch *table is the size of the sequence
// table at its start (the records follow it).
int chunk_workspace(const gdr_desc *d, bool packed, size_t *bytes, size_t *table = nullptr) {
    const long NC = chunk_count(d, packed);
    // one workgroup per (sequence, head, chunk) or (chunk, head): the grid must stay below 2^31
    if ((size_t)(packed ? 1 : d->B) * d->H * (size_t)NC >= ((size_t)1 << 31)) return GDR_E_SHAPE;
    const bool pc = d->decay_mode == GDR_DECAY_PER_CHANNEL;
    int algo = resolve_algo(d);
    if (algo == GDR_ALGO_MATRIX && !matrix_path_available(d)) {
        if (d->algo == GDR_ALGO_MATRIX) return GDR_E_UNSUPPORTED;
        algo = GDR_ALGO_VECTOR;
    }
    const int Bw = packed ? 1 : d->B;  // the records of a packed batch: NC chunks x H heads
    const size_t tab = packed ? gdr::seq_table_bytes(d->B, (int)NC) : 0;
    *bytes = tab + (algo == GDR_ALGO_MATRIX
                        ? gdr::chunk_matrix_workspace_bytes(Bw, d->H, (int)NC, d->Dk, d->Dv, pc, packed,
                                                            d->qkv_dtype == GDR_BF16)
                        : gdr::chunk_vector_workspace_bytes(Bw, d->H, (int)NC, d->Dk, d->Dv, pc));
    if (table) *table = tab;
    return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_status_string(int status) {
    switch (status) {
        case GDR_OK: return "GDR_OK: success (work enqueued)";
        case GDR_E_NULL: return "GDR_E_NULL: a required pointer is NULL";
        case GDR_E_SHAPE: return "GDR_E_SHAPE: negative size or element count overflow";
        case GDR_E_UNSUPPORTED: return "GDR_E_UNSUPPORTED: unsupported Dk/Dv/chunk or algorithm";
        case GDR_E_ALIGN: return "GDR_E_ALIGN: misaligned pointer";
        case GDR_E_WORKSPACE: return "GDR_E_WORKSPACE: workspace missing or too small";
        case GDR_E_HIP: return "GDR_E_HIP: a HIP launch failed";
        case GDR_E_ALIAS: return "GDR_E_ALIAS: an output overlaps an input";
        case GDR_E_MODE: return "GDR_E_MODE: bad mode, dtype, eps or scale";
        default: return "unknown gdr status";
    }
}

int gdr_chunk_fwd_workspace_size(const gdr_desc *desc, size_t *bytes) {
    if (!bytes) return GDR_E_NULL;
    Sizes sz;
    const int rc = check_desc(desc, false, &sz);
    if (rc != GDR_OK) return rc;
    return chunk_workspace(desc, false, bytes);
}

int gdr_chunk_fwd_varlen_workspace_size(const gdr_desc *desc, size_t *bytes) {
    if (!bytes) return GDR_E_NULL;
    Sizes sz;
    const int rc = check_desc(desc, false, &sz, true, true);
    if (rc != GDR_OK) return rc;
    return chunk_workspace(desc, true, bytes);
}

}  // extern "C"

namespace {

// stage: -1 = the whole chunked pass, 0 = intra kernel, 1 = state kernel.
// cu_seqlens != NULL: a packed batch (the varlen entry point).  ev0, ev1: a
// timed stage (recorded when its first kernel begins and its last ends).
int chunk_fwd_impl(int stage, const gdr_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                   const void *v, const float *g, const float *beta_or_eta, const float *s0, void *o,
                   float *s_final, void *workspace, size_t workspace_bytes, void *stream, bool packed = false,
                   hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    Sizes sz;
    int rc = check_desc(d, false, &sz, true, packed);
    if (rc != GDR_OK) return rc;
    size_t need = 0, table = 0;
    rc = chunk_workspace(d, packed, &need, &table);
    if (rc != GDR_OK) return rc;
    if (d->B == 0 || d->H == 0) return GDR_OK;
    const bool pc = d->decay_mode == GDR_DECAY_PER_CHANNEL;
    const size_t in_es = d->qkv_dtype == GDR_BF16 ? 2 : 4;
    const size_t out_es = d->o_dtype == GDR_BF16 ? 2 : 4;
    const bool have_tokens = d->T > 0;
    const bool delta = d->delta_mode == GDR_DELTA_RULE;
    if (!delta) beta_or_eta = nullptr;

    if (packed && !cu_seqlens) return GDR_E_NULL;
    if (packed && !aligned(cu_seqlens, 4)) return GDR_E_ALIGN;
    if (have_tokens) {
        if (!q || !k || !v || !g || (delta && !beta_or_eta) || !o) return GDR_E_NULL;
        if (need > 0 && !workspace) return GDR_E_WORKSPACE;
        if (workspace_bytes < need) return GDR_E_WORKSPACE;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GDR_E_ALIGN;
        if (!aligned(g, pc ? 16 : 4) || !aligned(beta_or_eta, 4)) return GDR_E_ALIGN;
        if (workspace && !aligned(workspace, 16)) return GDR_E_ALIGN;
    }
    if (s0 && !aligned(s0, 16)) return GDR_E_ALIGN;
    if (s_final && !aligned(s_final, 16)) return GDR_E_ALIGN;

    const Range rq = range_of(q, sz.qk * in_es), rk = range_of(k, sz.qk * in_es), rv = range_of(v, sz.v * in_es);
    const Range rg = range_of(g, sz.g * 4), rb = range_of(beta_or_eta, sz.beta * 4);
    const Range ro = range_of(o, have_tokens ? sz.o * out_es : 0);
    const Range rs0 = range_of(s0, s0 ? sz.state * 4 : 0);
    const Range rsf = range_of(s_final, s_final ? sz.state * 4 : 0);
    const Range rws = range_of(workspace, have_tokens ? need : 0);
    const Range rcu = range_of(cu_seqlens, packed ? ((size_t)d->B + 1) * 4 : 0);
    const Range ins[] = {rq, rk, rv, rg, rb, rcu};
    for (const Range &r : ins) {
        if (have_tokens && (overlap(r, ro) || overlap(r, rws))) return GDR_E_ALIAS;
        if (overlap(r, rsf)) return GDR_E_ALIAS;
    }
    if (overlap(ro, rsf) || overlap(ro, rws) || overlap(rsf, rws) || overlap(rs0, ro) || overlap(rs0, rws))
        return GDR_E_ALIAS;
    if (s0 && s_final && s0 != s_final && overlap(rs0, rsf)) return GDR_E_ALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    // a timed stage that does not go through the matrix-core launchers: the
    // events bracket its launches on the stream
    auto bracket = [&](hipEvent_t e) { return !e || hipEventRecord(e, st) == hipSuccess; };
    if (!have_tokens) {
        if (!bracket(ev0)) return GDR_E_HIP;
        if (stage != 0 && s_final && s_final != s0 &&
            gdr::launch_state_init(s_final, s0, sz.state, st) != hipSuccess)
            return GDR_E_HIP;
        return bracket(ev1) ? GDR_OK : GDR_E_HIP;
    }

    ChunkArgs a;
    a.B = d->B; a.T = d->T; a.H = d->H; a.Dk = d->Dk; a.Dv = d->Dv;
    a.NC = (int)chunk_count(d, packed);
    a.qkv_bf16 = d->qkv_dtype == GDR_BF16;
    a.o_bf16 = d->o_dtype == GDR_BF16;
    a.per_channel = pc;
    a.delta = delta;
    a.kaczmarz = delta && d->beta_mode == GDR_BETA_KACZMARZ;
    a.eps = a.kaczmarz ? d->eps : 0.f;
    a.scale = d->scale;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta_or_eta;
    a.s0 = s0; a.o = o; a.s_final = s_final;
    a.ws = workspace;
    a.stream = st;
    if (packed) {  // the sequence table first; the records after it
        if (gdr::launch_seq_table(cu_seqlens, d->B, d->T, workspace, st) != hipSuccess) return GDR_E_HIP;
        a.tab = gdr::seq_table(workspace, d->B, a.NC);
        a.tab.N = d->B;
        a.ws = static_cast<char *>(workspace) + table;
    }
    int algo = resolve_algo(d);
    if (algo == GDR_ALGO_MATRIX && !matrix_path_available(d)) algo = GDR_ALGO_VECTOR;
    if (algo == GDR_ALGO_MATRIX) {
        a.ev0 = ev0;
        a.ev1 = ev1;
        return gdr::launch_chunk_matrix(a, stage) == hipSuccess ? GDR_OK : GDR_E_HIP;
    }
    if (!bracket(ev0)) return GDR_E_HIP;
    if (gdr::launch_chunk_vector(a, stage) != hipSuccess) return GDR_E_HIP;
    return bracket(ev1) ? GDR_OK : GDR_E_HIP;
}

// The recurrent schedule: one token (gdr_recurrent_step, desc->T ignored) or
// desc->T tokens per sequence (gdr_recurrent_fwd).
int recurrent_impl(const gdr_desc *d, bool one_token, const void *q, const void *k, const void *v, const float *g,
                   const float *beta_or_eta, float *state, void *o, void *stream, hipEvent_t ev0 = nullptr,
                   hipEvent_t ev1 = nullptr, const int32_t *cu_seqlens = nullptr, bool packed = false) {
    Sizes sz;
    const int rc = check_desc(d, true, &sz, one_token, packed);
    if (rc != GDR_OK) return rc;
    const int T = one_token ? 1 : d->T;
    if (d->B > 0 && d->H > 0 && packed) {
        if (!cu_seqlens) return GDR_E_NULL;
        if (!aligned(cu_seqlens, 4)) return GDR_E_ALIGN;
    }
    if (d->B == 0 || d->H == 0 || T == 0) {  // nothing to launch: a timed call still records its events
        hipStream_t st = static_cast<hipStream_t>(stream);
        if (ev0 && hipEventRecord(ev0, st) != hipSuccess) return GDR_E_HIP;
        if (ev1 && hipEventRecord(ev1, st) != hipSuccess) return GDR_E_HIP;
        return GDR_OK;
    }
    const bool delta = d->delta_mode == GDR_DELTA_RULE;
    if (!delta) beta_or_eta = nullptr;
    if (!q || !k || !v || !g || (delta && !beta_or_eta) || !state || !o) return GDR_E_NULL;
    const bool pc = d->decay_mode == GDR_DECAY_PER_CHANNEL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state, 16))
        return GDR_E_ALIGN;
    if (!aligned(g, pc ? 16 : 4) || !aligned(beta_or_eta, 4)) return GDR_E_ALIGN;
    const size_t in_es = d->qkv_dtype == GDR_BF16 ? 2 : 4;
    const size_t out_es = d->o_dtype == GDR_BF16 ? 2 : 4;
    const Range rq = range_of(q, sz.qk * in_es), rk = range_of(k, sz.qk * in_es), rv = range_of(v, sz.v * in_es);
    const Range rg = range_of(g, sz.g * 4), rb = range_of(beta_or_eta, sz.beta * 4);
    const Range rs = range_of(state, sz.state * 4), ro = range_of(o, sz.o * out_es);
    const Range rcu = range_of(cu_seqlens, packed ? ((size_t)d->B + 1) * 4 : 0);
    const Range ins[] = {rq, rk, rv, rg, rb, rcu};
    for (const Range &r : ins)
        if (overlap(r, rs) || overlap(r, ro)) return GDR_E_ALIAS;
    if (overlap(rs, ro)) return GDR_E_ALIAS;

    StepArgs a;
    a.N = d->B; a.T = T; a.H = d->H; a.Dk = d->Dk; a.Dv = d->Dv;
    a.qkv_bf16 = d->qkv_dtype == GDR_BF16;
    a.o_bf16 = d->o_dtype == GDR_BF16;
    a.per_channel = pc;
    a.delta = delta;
    a.kaczmarz = delta && d->beta_mode == GDR_BETA_KACZMARZ;
    a.eps = a.kaczmarz ? d->eps : 0.f;
    a.scale = d->scale;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta_or_eta;
    a.state = state; a.o = o;
    a.stream = static_cast<hipStream_t>(stream);
    a.ev0 = ev0;
    a.ev1 = ev1;
    a.cu = packed ? cu_seqlens : nullptr;
    return gdr::launch_recurrent_step(a) == hipSuccess ? GDR_OK : GDR_E_HIP;
}

}  // namespace

extern "C" {

int gdr_chunk_fwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                  const float *beta_or_eta, const float *s0, void *o, float *s_final, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return chunk_fwd_impl(-1, d, nullptr, q, k, v, g, beta_or_eta, s0, o, s_final, workspace, workspace_bytes,
                          stream);
}

int gdr_chunk_fwd_varlen(const gdr_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                         const void *v, const float *g, const float *beta_or_eta, const float *s0, void *o,
                         float *s_final, void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_fwd_impl(-1, d, cu_seqlens, q, k, v, g, beta_or_eta, s0, o, s_final, workspace, workspace_bytes,
                          stream, true);
}

// Workspace of the backward pass: for a packed batch the sequence table
// first, then the per-chunk records of the chunk bound times H slots.
static int bwd_workspace(const gdr_desc *d, bool packed, size_t *bytes, size_t *table) {
    if (!bytes) return GDR_E_NULL;
    Sizes sz;
    const int rc = check_desc(d, false, &sz, true, packed);
    if (rc != GDR_OK) return rc;
    const long NC = chunk_count(d, packed);
    const int Bw = packed ? 1 : d->B;
    if ((size_t)Bw * d->H * (size_t)NC >= ((size_t)1 << 31)) return GDR_E_SHAPE;
    const size_t tab = packed ? gdr::seq_table_bytes(d->B, (int)NC) : 0;
    *bytes = tab + gdr::chunk_bwd_workspace_bytes(Bw, d->H, (int)NC, d->Dk, d->Dv,
                                                  d->decay_mode == GDR_DECAY_PER_CHANNEL,
                                                  d->qkv_dtype == GDR_BF16);
    if (table) *table = tab;
    return GDR_OK;
}

int gdr_chunk_bwd_workspace_size(const gdr_desc *d, size_t *bytes) { return bwd_workspace(d, false, bytes, nullptr); }

int gdr_chunk_bwd_varlen_workspace_size(const gdr_desc *d, size_t *bytes) {
    return bwd_workspace(d, true, bytes, nullptr);
}

static int chunk_bwd_impl(const gdr_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                          const void *v, const float *g, const float *beta_or_eta, const float *s0, const float *d_o,
                          const float *ds_final, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                          void *workspace, size_t workspace_bytes, void *stream, bool packed) {
    Sizes sz;
    int rc = check_desc(d, false, &sz, true, packed);
    if (rc != GDR_OK) return rc;
    size_t need = 0, table = 0;
    rc = bwd_workspace(d, packed, &need, &table);
    if (rc != GDR_OK) return rc;
    if (d->B == 0 || d->H == 0) return GDR_OK;
    if (packed && !cu_seqlens) return GDR_E_NULL;
    if (packed && !aligned(cu_seqlens, 4)) return GDR_E_ALIGN;
    const bool pc = d->decay_mode == GDR_DECAY_PER_CHANNEL;
    const size_t in_es = d->qkv_dtype == GDR_BF16 ? 2 : 4;
    const bool have_tokens = d->T > 0;
    const bool delta = d->delta_mode == GDR_DELTA_RULE;
    if (!delta) beta_or_eta = dbeta = nullptr;  // no beta without the delta rule
    if (have_tokens) {
        if (!q || !k || !v || !g || !d_o || !dq || !dk || !dv || !dg) return GDR_E_NULL;
        if (delta && (!beta_or_eta || !dbeta)) return GDR_E_NULL;
        if (!workspace) return GDR_E_WORKSPACE;
        if (workspace_bytes < need) return GDR_E_WORKSPACE;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) || !aligned(dq, 16) ||
            !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16))
            return GDR_E_ALIGN;
        if (!aligned(g, pc ? 16 : 4) || !aligned(dg, pc ? 16 : 4) || !aligned(beta_or_eta, 4) || !aligned(dbeta, 4))
            return GDR_E_ALIGN;
    }
    if ((s0 && !aligned(s0, 16)) || (ds_final && !aligned(ds_final, 16)) || (ds0 && !aligned(ds0, 16)))
        return GDR_E_ALIGN;
    const size_t tq = have_tokens ? sz.qk * in_es : 0, tv = have_tokens ? sz.v * in_es : 0;
    const Range ins[] = {range_of(q, tq), range_of(k, tq), range_of(v, tv),
                         range_of(g, have_tokens ? sz.g * 4 : 0), range_of(beta_or_eta, have_tokens ? sz.beta * 4 : 0),
                         range_of(d_o, have_tokens ? sz.o * 4 : 0), range_of(s0, s0 ? sz.state * 4 : 0),
                         range_of(ds_final, ds_final ? sz.state * 4 : 0),
                         range_of(cu_seqlens, packed ? ((size_t)d->B + 1) * 4 : 0)};
    const Range outs[] = {range_of(dq, have_tokens ? sz.qk * 4 : 0), range_of(dk, have_tokens ? sz.qk * 4 : 0),
                          range_of(dv, have_tokens ? sz.v * 4 : 0), range_of(dg, have_tokens ? sz.g * 4 : 0),
                          range_of(dbeta, have_tokens ? sz.beta * 4 : 0), range_of(ds0, ds0 ? sz.state * 4 : 0),
                          range_of(workspace, have_tokens ? need : 0)};
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlap(o, i)) return GDR_E_ALIAS;
        for (const Range &o2 : outs)
            if (&o2 != &o && overlap(o, o2)) return GDR_E_ALIAS;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!have_tokens) {  // the final state is the initial one: ds0 = ds_final
        if (!ds0) return GDR_OK;
        return gdr::launch_state_init(ds0, ds_final, sz.state, st) == hipSuccess ? GDR_OK : GDR_E_HIP;
    }
    gdr::BwdArgs a;
    a.B = d->B; a.T = d->T; a.H = d->H; a.Dk = d->Dk; a.Dv = d->Dv;
    a.NC = (int)chunk_count(d, packed);
    a.qkv_bf16 = d->qkv_dtype == GDR_BF16;
    a.per_channel = pc;
    a.delta = delta;
    a.kaczmarz = delta && d->beta_mode == GDR_BETA_KACZMARZ;
    a.eps = a.kaczmarz ? d->eps : 0.f;
    a.scale = d->scale;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta_or_eta; a.s0 = s0; a.dO = d_o; a.ds_final = ds_final;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.ds0 = ds0;
    a.ws = workspace;
    a.stream = st;
    if (packed) {  // the sequence table first; the records after it
        if (gdr::launch_seq_table(cu_seqlens, d->B, d->T, workspace, st) != hipSuccess) return GDR_E_HIP;
        a.tab = gdr::seq_table(workspace, d->B, a.NC);
        a.tab.N = d->B;
        a.ws = static_cast<char *>(workspace) + table;
    }
    return gdr::launch_chunk_bwd(a) == hipSuccess ? GDR_OK : GDR_E_HIP;
}

int gdr_chunk_bwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                  const float *beta_or_eta, const float *s0, const float *d_o, const float *ds_final, float *dq,
                  float *dk, float *dv, float *dg, float *dbeta, float *ds0, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return chunk_bwd_impl(d, nullptr, q, k, v, g, beta_or_eta, s0, d_o, ds_final, dq, dk, dv, dg, dbeta, ds0,
                          workspace, workspace_bytes, stream, false);
}

int gdr_chunk_bwd_varlen(const gdr_desc *d, const int32_t *cu_seqlens, const void *q, const void *k, const void *v,
                         const float *g, const float *beta_or_eta, const float *s0, const float *d_o,
                         const float *ds_final, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *ds0,
                         void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_bwd_impl(d, cu_seqlens, q, k, v, g, beta_or_eta, s0, d_o, ds_final, dq, dk, dv, dg, dbeta, ds0,
                          workspace, workspace_bytes, stream, true);
}

int gdr_chunk_fwd_stage(int stage, const gdr_desc *d, const void *q, const void *k, const void *v,
                        const float *g, const float *beta_or_eta, const float *s0, void *o, float *s_final,
                        void *workspace, size_t workspace_bytes, void *stream) {
    if (stage != GDR_STAGE_INTRA && stage != GDR_STAGE_STATE) return GDR_E_MODE;
    return chunk_fwd_impl(stage, d, nullptr, q, k, v, g, beta_or_eta, s0, o, s_final, workspace,
                          workspace_bytes, stream);
}

int gdr_chunk_fwd_stage_timed(int stage, const gdr_desc *d, const void *q, const void *k, const void *v,
                              const float *g, const float *beta_or_eta, const float *s0, void *o, float *s_final,
                              void *workspace, size_t workspace_bytes, void *stream, void *start_event,
                              void *stop_event) {
    if (stage != GDR_STAGE_INTRA && stage != GDR_STAGE_STATE) return GDR_E_MODE;
    if (!start_event || !stop_event) return GDR_E_NULL;
    return chunk_fwd_impl(stage, d, nullptr, q, k, v, g, beta_or_eta, s0, o, s_final, workspace,
                          workspace_bytes, stream, false, static_cast<hipEvent_t>(start_event),
                          static_cast<hipEvent_t>(stop_event));
}

int gdr_recurrent_step(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                       const float *beta_or_eta, float *state, void *o, void *stream) {
    return recurrent_impl(d, true, q, k, v, g, beta_or_eta, state, o, stream);
}

int gdr_recurrent_step_timed(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                             const float *beta_or_eta, float *state, void *o, void *stream, void *start_event,
                             void *stop_event) {
    if (!start_event || !stop_event) return GDR_E_NULL;
    return recurrent_impl(d, true, q, k, v, g, beta_or_eta, state, o, stream, static_cast<hipEvent_t>(start_event),
                          static_cast<hipEvent_t>(stop_event));
}

int gdr_recurrent_fwd(const gdr_desc *d, const void *q, const void *k, const void *v, const float *g,
                      const float *beta_or_eta, float *state, void *o, void *stream) {
    return recurrent_impl(d, false, q, k, v, g, beta_or_eta, state, o, stream);
}

int gdr_recurrent_fwd_varlen(const gdr_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                             const void *v, const float *g, const float *beta_or_eta, float *state, void *o,
                             void *stream) {
    return recurrent_impl(d, false, q, k, v, g, beta_or_eta, state, o, stream, nullptr, nullptr, cu_seqlens, true);
}

}  // extern "C"
