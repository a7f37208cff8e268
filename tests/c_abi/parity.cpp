// The C ABI on its own: a host program (no Python, no torch) that allocates
// device memory with the HIP runtime, calls libgdr through include/gdr.h and
// checks the results against the fp64 oracle (liboracle, test
// infrastructure).  Cases: chunked prefill with scalar decay (Gated DeltaNet)
// and per-channel decay (KDA) on the matrix-core path, one decode step, and a
// packed batch of sequences of different lengths (one empty) through the
// chunked and the recurrent entry points for packed batches.
// Inputs are seeded synthetic data drawn here with SplitMix64 (Steele, Lea
// and Flood 2014) and Box-Muller normals; both sides read the same values.
// Exit status 0 when every case is within the relative L2 bar for bf16
// inputs (2e-3), else 1.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdr.h"

extern "C" int gdr_oracle_fwd(long B, long T, long H, long Dk, long Dv, const float *q, const float *k,
                              const float *v, const float *g, const float *beta_or_eta, int per_channel,
                              int kaczmarz, double eps, double scale, int delta_off, const float *s0, double *o,
                              double *s_final, const long *bh_list, long n_bh, int n_threads);

namespace {

struct SplitMix64 {
    uint64_t x;
    uint64_t next() {
        uint64_t z = (x += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }  // (0, 1)
    double normal() { return std::sqrt(-2.0 * std::log(uniform())) * std::cos(6.283185307179586 * uniform()); }
};

// float -> bf16 bits, round to nearest even (finite inputs)
uint16_t to_bf16(float f) {
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return static_cast<uint16_t>((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
float from_bf16(uint16_t h) {
    const uint32_t b = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &b, 4);
    return f;
}

bool hip_ok(hipError_t e, const char *what) {
    if (e != hipSuccess) std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return e == hipSuccess;
}

template <typename T>
struct Dev {
    T *p = nullptr;
    size_t n = 0;
    explicit Dev(size_t count) : n(count) {
        if (!hip_ok(hipMalloc(reinterpret_cast<void **>(&p), std::max<size_t>(count, 1) * sizeof(T)),
                    "hipMalloc"))
            p = nullptr;
    }
    ~Dev() {
        if (p) (void)hipFree(p);
    }
    bool put(const std::vector<T> &h) {
        return hip_ok(hipMemcpy(p, h.data(), n * sizeof(T), hipMemcpyHostToDevice), "copy in");
    }
    bool get(std::vector<T> &h) {
        h.resize(n);
        return hip_ok(hipMemcpy(h.data(), p, n * sizeof(T), hipMemcpyDeviceToHost), "copy out");
    }
};

double rel_l2(const std::vector<float> &a, const std::vector<double> &b) {
    double num = 0, den = 0;
    for (size_t i = 0; i < b.size(); ++i) {
        num += (a[i] - b[i]) * (a[i] - b[i]);
        den += b[i] * b[i];
    }
    return den > 0 ? std::sqrt(num / den) : std::sqrt(num);
}

struct Inputs {
    std::vector<uint16_t> q, k, v;  // bf16 bits
    std::vector<float> qf, kf, vf;  // the same values as floats (the oracle's inputs)
    std::vector<float> g, beta, s0;
};

// q, v ~ N(0, 1); k ~ N(0, I) scaled to unit norm per (b, t, h); log-decays
// log U(0.9, 0.999) (one per key channel when per_channel); beta = sigmoid(N(0, 1));
// s0 ~ N(0, 0.1^2)
Inputs make_inputs(uint64_t seed, int B, int T, int H, int D, bool per_channel) {
    SplitMix64 r{seed};
    Inputs x;
    const size_t rows = (size_t)B * T * H;
    auto store = [](std::vector<uint16_t> &bits, std::vector<float> &vals, float f) {
        bits.push_back(to_bf16(f));
        vals.push_back(from_bf16(bits.back()));
    };
    for (size_t i = 0; i < rows * D; ++i) store(x.q, x.qf, (float)r.normal());
    for (size_t row = 0; row < rows; ++row) {
        std::vector<double> z(D);
        double nn = 0;
        for (int c = 0; c < D; ++c) nn += (z[c] = r.normal()) * z[c];
        for (int c = 0; c < D; ++c) store(x.k, x.kf, (float)(z[c] / std::sqrt(nn)));
    }
    for (size_t i = 0; i < rows * D; ++i) store(x.v, x.vf, (float)r.normal());
    for (size_t i = 0; i < rows * (per_channel ? D : 1); ++i)
        x.g.push_back((float)std::log(0.9 + 0.099 * r.uniform()));
    for (size_t i = 0; i < rows; ++i) x.beta.push_back((float)(1.0 / (1.0 + std::exp(-r.normal()))));
    for (size_t i = 0; i < (size_t)B * H * D * D; ++i) x.s0.push_back((float)(0.1 * r.normal()));
    return x;
}

gdr_desc make_desc(int B, int T, int H, int D, bool per_channel, int algo) {
    gdr_desc d{};
    d.B = B; d.T = T; d.H = H; d.Dk = D; d.Dv = D; d.chunk = 64;
    d.qkv_dtype = GDR_BF16; d.o_dtype = GDR_F32;
    d.decay_mode = per_channel ? GDR_DECAY_PER_CHANNEL : GDR_DECAY_SCALAR;
    d.beta_mode = GDR_BETA_GIVEN; d.algo = algo; d.delta_mode = GDR_DELTA_RULE;
    d.eps = 0.f; d.scale = 1.f;
    return d;
}

bool prefill_case(const char *name, bool per_channel) {
    const int B = 2, T = 200, H = 2, D = 128;
    const Inputs x = make_inputs(per_channel ? 2 : 1, B, T, H, D, per_channel);
    const gdr_desc d = make_desc(B, T, H, D, per_channel, GDR_ALGO_MATRIX);
    size_t ws_bytes = 0;
    if (gdr_chunk_fwd_workspace_size(&d, &ws_bytes) != GDR_OK) return false;
    Dev<uint16_t> q(x.q.size()), k(x.k.size()), v(x.v.size());
    Dev<float> g(x.g.size()), beta(x.beta.size()), s0(x.s0.size()), o((size_t)B * T * H * D), sf(x.s0.size());
    Dev<unsigned char> ws(ws_bytes);
    if (!q.p || !k.p || !v.p || !g.p || !beta.p || !s0.p || !o.p || !sf.p || !ws.p) return false;
    if (!q.put(x.q) || !k.put(x.k) || !v.put(x.v) || !g.put(x.g) || !beta.put(x.beta) || !s0.put(x.s0)) return false;
    const int rc = gdr_chunk_fwd(&d, q.p, k.p, v.p, g.p, beta.p, s0.p, o.p, sf.p, ws.p, ws_bytes, nullptr);
    if (rc != GDR_OK) {
        std::fprintf(stderr, "%s: gdr_chunk_fwd: %s\n", name, gdr_status_string(rc));
        return false;
    }
    if (!hip_ok(hipDeviceSynchronize(), "sync")) return false;
    std::vector<float> oh, sh;
    if (!o.get(oh) || !sf.get(sh)) return false;
    std::vector<double> oref(oh.size()), sref(sh.size());
    if (gdr_oracle_fwd(B, T, H, D, D, x.qf.data(), x.kf.data(), x.vf.data(), x.g.data(), x.beta.data(),
                       per_channel, 0, 0.0, 1.0, 0, x.s0.data(), oref.data(), sref.data(), nullptr, 0, 0) != 0)
        return false;
    const double eo = rel_l2(oh, oref), es = rel_l2(sh, sref);
    std::printf("c-abi %s: rel-L2 o %.2e, S %.2e\n", name, eo, es);
    return eo < 2e-3 && es < 2e-3;
}

bool decode_case() {
    const int N = 4, H = 2, D = 128;
    const Inputs x = make_inputs(3, N, 1, H, D, false);
    gdr_desc d = make_desc(N, 1, H, D, false, GDR_ALGO_AUTO);
    Dev<uint16_t> q(x.q.size()), k(x.k.size()), v(x.v.size());
    Dev<float> g(x.g.size()), beta(x.beta.size()), state(x.s0.size()), o((size_t)N * H * D);
    if (!q.p || !k.p || !v.p || !g.p || !beta.p || !state.p || !o.p) return false;
    if (!q.put(x.q) || !k.put(x.k) || !v.put(x.v) || !g.put(x.g) || !beta.put(x.beta) || !state.put(x.s0))
        return false;
    const int rc = gdr_recurrent_step(&d, q.p, k.p, v.p, g.p, beta.p, state.p, o.p, nullptr);
    if (rc != GDR_OK) {
        std::fprintf(stderr, "decode: gdr_recurrent_step: %s\n", gdr_status_string(rc));
        return false;
    }
    if (!hip_ok(hipDeviceSynchronize(), "sync")) return false;
    std::vector<float> oh, sh;
    if (!o.get(oh) || !state.get(sh)) return false;
    std::vector<double> oref(oh.size()), sref(sh.size());
    if (gdr_oracle_fwd(N, 1, H, D, D, x.qf.data(), x.kf.data(), x.vf.data(), x.g.data(), x.beta.data(), 0, 0, 0.0,
                       1.0, 0, x.s0.data(), oref.data(), sref.data(), nullptr, 0, 0) != 0)
        return false;
    const double eo = rel_l2(oh, oref), es = rel_l2(sh, sref);
    std::printf("c-abi decode step: rel-L2 o %.2e, S %.2e\n", eo, es);
    return eo < 2e-3 && es < 2e-3;
}

// Packed batch: N sequences with cu_seqlens in device memory, token tensors
// [T, H, D], states [N, H, D, D]; each sequence against the oracle run on its
// own tokens and initial state.
bool varlen_case(bool recurrent) {
    const int N = 4, H = 2, D = 128;
    const std::vector<int32_t> cu = {0, 0, 70, 71, 200};  // lengths 0, 70, 1, 129
    const int T = cu.back();
    const Inputs x = make_inputs(recurrent ? 5 : 4, 1, T, H, D, false);
    const std::vector<float> s0 = make_inputs(recurrent ? 7 : 6, N, 1, H, D, false).s0;  // [N, H, D, D]
    gdr_desc d = make_desc(N, T, H, D, false, recurrent ? GDR_ALGO_AUTO : GDR_ALGO_MATRIX);
    size_t ws_bytes = 0;
    if (!recurrent && gdr_chunk_fwd_varlen_workspace_size(&d, &ws_bytes) != GDR_OK) return false;
    Dev<uint16_t> q(x.q.size()), k(x.k.size()), v(x.v.size());
    Dev<float> g(x.g.size()), beta(x.beta.size()), st(s0.size()), o((size_t)T * H * D), sf(s0.size());
    Dev<int32_t> cud(cu.size());
    Dev<unsigned char> ws(ws_bytes);
    if (!q.p || !k.p || !v.p || !g.p || !beta.p || !st.p || !o.p || !sf.p || !cud.p || !ws.p) return false;
    if (!q.put(x.q) || !k.put(x.k) || !v.put(x.v) || !g.put(x.g) || !beta.put(x.beta) || !st.put(s0) || !cud.put(cu))
        return false;
    const int rc = recurrent
                       ? gdr_recurrent_fwd_varlen(&d, cud.p, q.p, k.p, v.p, g.p, beta.p, st.p, o.p, nullptr)
                       : gdr_chunk_fwd_varlen(&d, cud.p, q.p, k.p, v.p, g.p, beta.p, st.p, o.p, sf.p, ws.p, ws_bytes,
                                              nullptr);
    if (rc != GDR_OK) {
        std::fprintf(stderr, "varlen: %s\n", gdr_status_string(rc));
        return false;
    }
    if (!hip_ok(hipDeviceSynchronize(), "sync")) return false;
    std::vector<float> oh, sh;
    if (!o.get(oh) || !(recurrent ? st.get(sh) : sf.get(sh))) return false;
    bool ok = true;
    const size_t ss = (size_t)H * D * D;
    for (int n = 0; n < N; ++n) {
        const long L = cu[n + 1] - cu[n];
        const size_t t0 = (size_t)cu[n] * H * D;
        std::vector<double> oref((size_t)L * H * D), sref(ss);
        if (L > 0 && gdr_oracle_fwd(1, L, H, D, D, x.qf.data() + t0, x.kf.data() + t0, x.vf.data() + t0,
                                    x.g.data() + (size_t)cu[n] * H, x.beta.data() + (size_t)cu[n] * H, 0, 0, 0.0,
                                    1.0, 0, s0.data() + n * ss, oref.data(), sref.data(), nullptr, 0, 0) != 0)
            return false;
        if (L == 0)
            for (size_t i = 0; i < ss; ++i) sref[i] = s0[n * ss + i];
        const std::vector<float> on(oh.begin() + t0, oh.begin() + t0 + (size_t)L * H * D);
        const std::vector<float> sn(sh.begin() + n * ss, sh.begin() + (n + 1) * ss);
        const double eo = L > 0 ? rel_l2(on, oref) : 0.0, es = rel_l2(sn, sref);
        std::printf("c-abi %s varlen, sequence %d (%ld tokens): rel-L2 o %.2e, S %.2e\n",
                    recurrent ? "recurrent" : "chunked", n, L, eo, es);
        ok = ok && eo < 2e-3 && es < 2e-3;
    }
    return ok;
}

}  // namespace

int main() {
    if (gdr_abi_version() != GDR_ABI_VERSION) {
        std::fprintf(stderr, "ABI version %d, header %d\n", gdr_abi_version(), GDR_ABI_VERSION);
        return 1;
    }
    bool ok = prefill_case("prefill GDN B2 T200 H2 d128", false);
    ok = prefill_case("prefill KDA B2 T200 H2 d128", true) && ok;
    ok = decode_case() && ok;
    ok = varlen_case(false) && ok;
    ok = varlen_case(true) && ok;
    std::printf("c-abi: %s\n", ok ? "ok" : "FAILED");
    return ok ? 0 : 1;
}
