"""Pins of the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes a forward callable with the signature of
``oracle.oracle_fwd`` and raises AssertionError when it disagrees with the
pages.  ``tests/test_oracle_pins.py`` runs them on the oracle;
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies of
the oracle and requires that every mutant fails at least one pin.

Page references: page 1 = textbook section "Scrivere meglio nella memoria:
gate e delta rule"; page 2 = blog summary "Revisando las variantes de
atencion lineal de la familia DeltaNet"; page 3 = "Riepilogo Tecnico:
Attenzione Lineare Kaczmarz (KLA)".
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import hadamard
from scipy.optimize import minimize_scalar


# ---------------------------------------------------------------- helpers
def run1(fwd, q, k, v, g, beta, s0=None, **kw):
    """One (batch, head) pair: q,k [T,Dk]; v [T,Dv]; g [T] or [T,Dk]; beta [T]."""
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    g = np.asarray(g, np.float32)
    beta = np.asarray(beta, np.float32)
    T = q.shape[0]
    s0_ = None if s0 is None else np.asarray(s0, np.float32)[None, None]
    o, s = fwd(q[None, :, None], k[None, :, None], v[None, :, None],
               g[None, :, None], beta[None, :, None], s0=s0_, **kw)
    assert o.shape[1] == T
    return o[0, :, 0], s[0, 0]


def hadamard_rows(d):
    """Rows of a d x d Hadamard matrix scaled to unit length: exactly
    orthonormal in float32 when d is a power of 4."""
    return hadamard(d).astype(np.float64) / np.sqrt(d)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- decay
def pin_forget_gate_ten_steps(fwd, golden):
    """Page 1, 'Dimenticare: i gate': factor 0.9 for ten steps leaves ~0.35;
    page 1, scalar-decay unrolling: a write at step j weighs prod_{i>j} alpha_i."""
    fx = golden["forget_gate"]
    n = fx["steps"]
    T = n + 1
    g = np.zeros(T)
    g[1:] = np.log(fx["alpha"])
    beta = np.zeros(T)
    beta[0] = 1.0                      # one write of 1 at token 0, then decay only
    one = np.ones((T, 1))
    o, s = run1(fwd, one, one, one, g, beta)
    alpha32 = float(np.exp(np.float64(np.float32(np.log(fx["alpha"])))))
    assert abs(o[n] - fx["printed_value"]) < fx["printed_digits_tolerance"], o[n]
    assert abs(o[n] - alpha32 ** n) < 1e-14
    for t in range(T):
        assert abs(o[t] - alpha32 ** t) < 1e-14


def pin_per_zone_decay(fwd, golden):
    """Page 1, per-zone paragraph: channel factors 0.99 and 0.5 act on their own
    channel only (0.5 halves every step); an undecayed channel stays put.
    Page 2, KDA section: the per-channel decay acts on the key channels."""
    a_keep, a_half = golden["per_zone_decay"]["alphas"]
    T, Dk, Dv = 10, 3, 2
    s0 = np.array([[1.0, 2.0], [1.0, -4.0], [3.0, 5.0]])
    g = np.tile(np.log([a_keep, a_half, 1.0]), (T, 1))
    zeros_k = np.zeros((T, Dk))
    for c in range(Dk):
        q = np.zeros((T, Dk))
        q[:, c] = 1.0                  # read row c of the state
        o, s = run1(fwd, q, zeros_k, np.zeros((T, Dv)), g, np.zeros(T), s0=s0, per_channel=True)
        a = float(np.exp(np.float64(np.float32(g[0, c]))))
        for t in range(T):
            np.testing.assert_allclose(o[t], s0[c] * a ** (t + 1), rtol=1e-13, atol=0)
    # the halving channel halves at every step (to the float32 storage of log 0.5)
    q = np.zeros((T, Dk))
    q[:, 1] = 1.0
    o, _ = run1(fwd, q, zeros_k, np.zeros((T, Dv)), g, np.zeros(T), s0=s0, per_channel=True)
    np.testing.assert_allclose(o[-1], s0[1] * 0.5 ** T, rtol=1e-6)


def pin_beta_zero_no_write(fwd):
    """Page 1, Gated DeltaNet section: beta -> 0 leaves S_t = alpha_t S_{t-1}
    (the write is switched off together with the correction)."""
    rng = np.random.default_rng(11)
    T, Dk, Dv = 7, 4, 3
    s0 = rng.standard_normal((Dk, Dv))
    g = np.log(rng.uniform(0.5, 1.0, T))
    q = rng.standard_normal((T, Dk))
    k = rng.standard_normal((T, Dk))
    v = rng.standard_normal((T, Dv))
    o, s = run1(fwd, q, k, v, g, np.zeros(T), s0=s0)
    a = np.exp(np.float32(g).astype(np.float64))
    np.testing.assert_allclose(s, np.prod(a) * np.float32(s0), rtol=1e-13)


# ---------------------------------------------------------------- delta rule
def pin_phone_book(fwd, golden):
    """Page 1, phone-book example (7 read, 10 target; beta 0.5 -> 8.5, 1 -> 10,
    0 -> 7), and the erase-half/write-half reading (3.5 + 5 = 8.5)."""
    fx = golden["phone_book"]
    one = np.ones((1, 1))
    for case in fx["cases"]:
        o, s = run1(fwd, one, one, [[fx["target"]]], [0.0], [case["beta"]], s0=[[fx["read"]]])
        assert abs(o[0, 0] - case["answer_after"]) < 1e-12, (case, o)
        assert abs((s[0, 0] - fx["read"]) - case["written"]) < 1e-12
    eh = golden["erase_half_write_half"]
    o, _ = run1(fwd, one, one, [[fx["target"]]], [0.0], [0.5], s0=[[fx["read"]]])
    assert abs(o[0, 0] - (eh["erase_kept"] + eh["written"])) < 1e-12
    assert abs(o[0, 0] - eh["answer_after"]) < 1e-12


def pin_double_weight_key(fwd, golden):
    """Page 1: a key that weighs double (||k||^2 = 2) with beta = 1 swings
    7 -> 13 -> 7 forever; page 3: the Kaczmarz step 1/||k||^2 lands on 10."""
    fx = golden["double_weight_key"]
    n = len(fx["answers"])
    kv = np.float32(np.sqrt(fx["key_weight"]))
    kk = float(kv) ** 2                                    # ||k||^2 of the stored key
    k = np.full((n, 1), kv)
    s0 = [[fx["read"] / float(kv)]]                         # so that S^T k = 7
    v = np.full((n, 1), fx["target"])
    o, _ = run1(fwd, k, k, v, np.zeros(n), np.full(n, fx["beta"]), s0=s0)
    for t, want in enumerate(fx["answers"]):
        assert abs(o[t, 0] - want) < 1e-5 * max(1.0, abs(kk)), (t, o[t, 0], want)
    ks = golden["kaczmarz_step"]
    o, _ = run1(fwd, k, k, v, np.zeros(n), np.full(n, ks["eta"]), s0=s0,
                kaczmarz=True, eps=ks["eps"])
    np.testing.assert_allclose(o[:, 0], fx["target"], rtol=1e-13)


def pin_forget_before_predict(fwd):
    """Page 2, Gated DeltaNet section: forget -> predict -> correct -> write.
    Hand arithmetic: S=7, alpha=0.5, k=1, v=10, beta=0.5: S~ = 3.5, prediction
    3.5, correction 0.5*(10-3.5) = 3.25, new state 6.75 (predicting before the
    forget step would give 3.5 + 0.5*(10-7) = 5)."""
    one = np.ones((1, 1))
    o, s = run1(fwd, one, one, [[10.0]], [np.log(0.5)], [0.5], s0=[[7.0]])
    assert abs(s[0, 0] - 6.75) < 1e-7 and abs(o[0, 0] - 6.75) < 1e-7, s


def pin_read_after_write(fwd):
    """Page 2, KDA step 5 and the in-chunk output subsection: the token reads
    after its own write, so with S0 = 0 the first output is already k.q times
    the write."""
    q = np.array([[1.0, 2.0]])
    k = np.array([[1.0, 0.0]])
    o, _ = run1(fwd, q, k, [[4.0, -2.0]], [0.0], [0.5])
    np.testing.assert_allclose(o[0], [2.0, -1.0], rtol=1e-15)   # 0.5*[4,-2]*(k.q=1)


def pin_constraint_unit_keys(fwd):
    """Page 2, DeltaNet section: re-reading with the same key after a beta = 1
    write returns v_t exactly (unit keys), whatever the decay."""
    rng = np.random.default_rng(3)
    T, Dk, Dv = 40, 16, 8
    H = hadamard_rows(Dk)                                    # exact unit rows in float32
    k = H[rng.integers(0, Dk, T)] * rng.choice([-1.0, 1.0], (T, 1))
    v = rng.standard_normal((T, Dv))
    g = np.log(rng.uniform(0.3, 1.0, T))
    o, _ = run1(fwd, k, k, v, g, np.ones(T), s0=rng.standard_normal((Dk, Dv)))
    np.testing.assert_allclose(o, np.float32(v), rtol=0, atol=1e-12)
    # generic unit keys rounded to float32: met to float32 accuracy of ||k||
    kr = rng.standard_normal((T, Dk))
    kr /= np.linalg.norm(kr, axis=1, keepdims=True)
    o, _ = run1(fwd, kr, kr, v, g, np.ones(T))
    np.testing.assert_allclose(o, np.float32(v), rtol=0, atol=1e-5)


def pin_reread_interpolates(fwd):
    """Page 2, DeltaNet section: after a write of strength beta, re-reading with
    the same unit key gives (1 - beta) S~^T k + beta v."""
    rng = np.random.default_rng(5)
    Dk, Dv = 16, 5
    k = hadamard_rows(Dk)[3:4]
    s0 = np.float32(rng.standard_normal((Dk, Dv)))
    v = np.float32(rng.standard_normal((1, Dv)))
    for beta in (0.0, 0.25, 0.5, 0.9, 1.0):
        g = np.float32(np.log(0.7))
        o, _ = run1(fwd, k, k, v, [g], [beta], s0=s0)
        St = np.exp(np.float64(g)) * s0.astype(np.float64)
        b32 = float(np.float32(beta))                      # the stored beta
        want = (1 - b32) * (St.T @ k[0]) + b32 * v[0].astype(np.float64)
        np.testing.assert_allclose(o[0], want, rtol=1e-13, atol=1e-14)


def pin_locality(fwd):
    """Page 2, DeltaNet section: directions orthogonal to the current key read
    exactly what the decayed state read before the write."""
    rng = np.random.default_rng(7)
    Dk, Dv = 16, 6
    Hm = hadamard_rows(Dk)
    s0 = np.float32(rng.standard_normal((Dk, Dv)))
    g = np.float32(np.log(0.8))
    St = np.exp(np.float64(g)) * s0.astype(np.float64)
    for qi in (1, 5, 15):
        o, _ = run1(fwd, Hm[qi:qi + 1], Hm[0:1], rng.standard_normal((1, Dv)), [g], [0.8], s0=s0)
        np.testing.assert_allclose(o[0], St.T @ Hm[qi], rtol=1e-13, atol=1e-14)


def pin_transition_spectrum(fwd):
    """Page 1, delta-rule section and page 2, structured transition: the
    transition alpha (I - beta k k^T) has eigenvalue alpha (1 - beta ||k||^2)
    along k and alpha elsewhere; with unit k and beta = 1 it is a projector and
    its spectral norm is exactly 1.  With v = 0 and S0 = I the oracle's new
    state IS that transition (d_k x d_v orientation: it acts on the rows)."""
    rng = np.random.default_rng(9)
    D = 8
    k = np.float32(rng.standard_normal((1, D)) * 0.4)
    kk = float(np.sum(k.astype(np.float64) ** 2))
    beta, alpha = 0.6, 0.9
    g = np.float32(np.log(alpha))
    a = float(np.exp(np.float64(g)))
    o, M = run1(fwd, np.zeros((1, D)), k, np.zeros((1, D)), [g], [beta], s0=np.eye(D))
    ev = np.sort(np.linalg.eigvalsh((M + M.T) / 2))
    want = np.sort(np.r_[a * (1 - np.float64(np.float32(beta)) * kk), np.full(D - 1, a)])
    np.testing.assert_allclose(ev, want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(M @ k[0], a * (1 - np.float64(np.float32(beta)) * kk) * k[0], rtol=1e-12)
    # unit key, beta = 1, no decay: projector with spectral norm 1
    ku = hadamard_rows(16)[2:3]
    _, P = run1(fwd, np.zeros((1, 16)), ku, np.zeros((1, 16)), [0.0], [1.0], s0=np.eye(16))
    np.testing.assert_allclose(P @ P, P, atol=1e-14)
    assert abs(np.linalg.norm(P, 2) - 1.0) < 1e-13


# ---------------------------------------------------------------- online regression / KLA
def pin_gradient_step(fwd):
    """Page 1, 'Tutto e regressione online' and page 2, loss derivation: the
    delta-rule write is one gradient step of rate beta on
    L(S) = 1/2 ||S^T k - v||^2 taken at the decayed state; the Kaczmarz write
    is the same step with rate 1/||k||^2 (page 3, normalised-SGD property).
    The gradient here is taken by central finite differences."""
    rng = np.random.default_rng(13)
    Dk, Dv = 4, 3
    s0 = np.float32(rng.standard_normal((Dk, Dv)))
    k = np.float32(rng.standard_normal((1, Dk)))
    v = np.float32(rng.standard_normal((1, Dv)))
    g = np.float32(np.log(0.75))
    St = np.exp(np.float64(g)) * s0.astype(np.float64)
    kd, vd = k[0].astype(np.float64), v[0].astype(np.float64)

    def loss(S):
        r = S.T @ kd - vd
        return 0.5 * float(r @ r)

    h = 1e-6
    grad = np.zeros_like(St)
    for i in range(Dk):
        for j in range(Dv):
            E = np.zeros_like(St)
            E[i, j] = h
            grad[i, j] = (loss(St + E) - loss(St - E)) / (2 * h)
    beta = np.float32(0.35)
    _, s = run1(fwd, np.zeros((1, Dk)), k, v, [g], [beta], s0=s0)
    np.testing.assert_allclose(s, St - float(beta) * grad, rtol=0, atol=1e-8)
    _, s = run1(fwd, np.zeros((1, Dk)), k, v, [g], [1.0], s0=s0, kaczmarz=True, eps=0.0)
    np.testing.assert_allclose(s, St - grad / float(kd @ kd), rtol=0, atol=1e-8)


def pin_kaczmarz_constraint(fwd):
    """Page 3, 'Derivazione Teorica' / 'Proprieta Chiave': with eta = 1, eps = 0
    every write meets S_t^T k_t = v_t exactly for unnormalised keys."""
    rng = np.random.default_rng(17)
    T, Dk, Dv = 50, 12, 7
    k = rng.standard_normal((T, Dk)) * rng.lognormal(0, 0.5, (T, 1))
    v = rng.standard_normal((T, Dv))
    g = np.log(rng.uniform(0.5, 1.0, T))
    o, _ = run1(fwd, k, k, v, g, np.ones(T), kaczmarz=True, eps=0.0,
                s0=rng.standard_normal((Dk, Dv)))
    np.testing.assert_allclose(o, np.float32(v), rtol=0, atol=1e-11)


def pin_kaczmarz_min_norm(fwd):
    """Page 3, 'Derivazione Teorica': the Kaczmarz write is the minimum-Frobenius
    change of the decayed state that meets the constraint; compared with the
    minimum-norm least-squares solution of X^T k = v - S~^T k (numpy lstsq)."""
    rng = np.random.default_rng(19)
    Dk, Dv = 10, 6
    s0 = np.float32(rng.standard_normal((Dk, Dv)))
    k = np.float32(rng.standard_normal((1, Dk)) * 1.7)
    v = np.float32(rng.standard_normal((1, Dv)))
    g = np.float32(np.log(0.6))
    St = np.exp(np.float64(g)) * s0.astype(np.float64)
    _, s = run1(fwd, np.zeros((1, Dk)), k, v, [g], [1.0], s0=s0, kaczmarz=True, eps=0.0)
    resid = v[0].astype(np.float64) - St.T @ k[0].astype(np.float64)
    X, *_ = np.linalg.lstsq(k.astype(np.float64), resid[None, :], rcond=None)   # min-norm
    np.testing.assert_allclose(s - St, X, rtol=1e-12, atol=1e-13)


def pin_kaczmarz_line_search(fwd):
    """Page 3, 'Proprieta Chiave' 2: along the update direction k e^T the
    Kaczmarz step minimises the per-token loss (found with scipy's bounded
    scalar minimiser), and eps > 0 shrinks it to eta / (||k||^2 + eps)."""
    rng = np.random.default_rng(23)
    Dk, Dv = 9, 4
    s0 = np.float32(rng.standard_normal((Dk, Dv)))
    k = np.float32(rng.standard_normal((1, Dk)) * 0.6)
    v = np.float32(rng.standard_normal((1, Dv)))
    St = s0.astype(np.float64)
    kd, vd = k[0].astype(np.float64), v[0].astype(np.float64)
    e = vd - St.T @ kd

    def loss(b):
        r = (St + b * np.outer(kd, e)).T @ kd - vd
        return 0.5 * float(r @ r)

    best = minimize_scalar(loss, bounds=(0.0, 50.0), method="bounded",
                           options={"xatol": 1e-12}).x
    _, s = run1(fwd, np.zeros((1, Dk)), k, v, [0.0], [1.0], s0=s0, kaczmarz=True, eps=0.0)
    np.testing.assert_allclose(s, St + best * np.outer(kd, e), rtol=1e-6, atol=1e-7)
    # relaxation and stabiliser
    eta, eps = np.float32(0.4), 0.3
    _, s = run1(fwd, np.zeros((1, Dk)), k, v, [0.0], [eta], s0=s0, kaczmarz=True, eps=eps)
    step = float(eta) / (float(kd @ kd) + eps)
    np.testing.assert_allclose(s, St + step * np.outer(kd, e), rtol=1e-13)


def pin_accumulate_vs_delta(fwd):
    """Page 1, 'Tutto e regressione online': with orthonormal keys and S0 = 0
    the delta rule writes beta v k^T where accumulation writes v k^T (a factor 2
    at the first token for beta = 0.5); with beta = 1 the two coincide."""
    rng = np.random.default_rng(29)
    D = 16
    T = 16
    k = hadamard_rows(D)[rng.permutation(D)]
    v = rng.standard_normal((T, D))
    q = rng.standard_normal((T, D))
    g = np.zeros(T)
    _, s_acc1 = run1(fwd, q[:1], k[:1], v[:1], g[:1], np.ones(1), delta_off=True)
    _, s_dl1 = run1(fwd, q[:1], k[:1], v[:1], g[:1], np.full(1, 0.5))
    np.testing.assert_allclose(s_acc1, 2.0 * s_dl1, rtol=1e-14, atol=1e-15)
    o_acc, s_acc = run1(fwd, q, k, v, g, np.ones(T), delta_off=True)
    o_dl, s_dl = run1(fwd, q, k, v, g, np.ones(T))
    np.testing.assert_allclose(o_dl, o_acc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s_dl, s_acc, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- read arithmetic
def pin_linear_attention_bruteforce(fwd):
    """Page 2, from quadratic attention to a linear state: without softmax,
    o_t = S_t q_t with S_t = sum_{i<=t} v_i k_i^T equals the causal,
    unnormalised (Q K^T masked to i <= t) V -- diagonal included."""
    rng = np.random.default_rng(31)
    T, Dk, Dv = 33, 8, 5
    q = np.float32(rng.standard_normal((T, Dk)))
    k = np.float32(rng.standard_normal((T, Dk)))
    v = np.float32(rng.standard_normal((T, Dv)))
    o, _ = run1(fwd, q, k, v, np.zeros(T), np.zeros(T), delta_off=True)
    A = np.tril(q.astype(np.float64) @ k.astype(np.float64).T)
    np.testing.assert_allclose(o, A @ v.astype(np.float64), rtol=1e-12, atol=1e-12)


def pin_decayed_attention_bruteforce(fwd):
    """Page 1, scalar decay (a write at step j weighs prod_{i=j+1..t} alpha_i at
    step t) and the GLA per-channel gate: delta off, brute force over pairs."""
    rng = np.random.default_rng(37)
    T, Dk, Dv = 21, 6, 4
    q = np.float32(rng.standard_normal((T, Dk)))
    k = np.float32(rng.standard_normal((T, Dk)))
    v = np.float32(rng.standard_normal((T, Dv)))
    for per_channel in (False, True):
        shape = (T, Dk) if per_channel else (T,)
        g = np.float32(np.log(rng.uniform(0.6, 1.0, shape)))
        a = np.exp(g.astype(np.float64))
        o, _ = run1(fwd, q, k, v, g, np.zeros(T), delta_off=True, per_channel=per_channel)
        want = np.zeros((T, Dv))
        for t in range(T):
            for j in range(t + 1):
                w = np.prod(a[j + 1:t + 1], axis=0) if t > j else (np.ones(Dk) if per_channel else 1.0)
                coef = float(np.sum(q[t].astype(np.float64) * w * k[j].astype(np.float64)))
                want[t] += coef * v[j].astype(np.float64)
        np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-12)


def pin_table_transition_form(fwd):
    """Page 1, update table (Gated DeltaNet row) and page 2, DPLR subsection
    (KDA: A_t = D_t (I - beta_t k_t k_t^T)), both in the pages' own d_v x d_k
    orientation with o_t = S_t q_t: S_t = S_{t-1} A_t + beta_t v_t k_t^T."""
    rng = np.random.default_rng(41)
    T, Dk, Dv = 25, 6, 5
    q = np.float32(rng.standard_normal((T, Dk)))
    k = np.float32(rng.standard_normal((T, Dk)) * 0.5)
    v = np.float32(rng.standard_normal((T, Dv)))
    beta = np.float32(rng.uniform(0, 1, T))
    s0 = np.float32(rng.standard_normal((Dk, Dv)))
    for per_channel in (False, True):
        shape = (T, Dk) if per_channel else (T,)
        g = np.float32(np.log(rng.uniform(0.7, 1.0, shape)))
        o, s = run1(fwd, q, k, v, g, beta, s0=s0, per_channel=per_channel)
        S = s0.astype(np.float64).T                      # d_v x d_k
        want_o = np.zeros((T, Dv))
        for t in range(T):
            kt = k[t].astype(np.float64)
            D = np.diag(np.exp(g[t].astype(np.float64))) if per_channel else \
                np.exp(np.float64(g[t])) * np.eye(Dk)
            A = D @ (np.eye(Dk) - float(beta[t]) * np.outer(kt, kt))
            S = S @ A + float(beta[t]) * np.outer(v[t].astype(np.float64), kt)
            want_o[t] = S @ q[t].astype(np.float64)
        np.testing.assert_allclose(o, want_o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s, S.T, rtol=1e-11, atol=1e-12)


def pin_output_scale(fwd):
    """Page 2, KDA step 5 reads with d_k^{-1/2} q_t; the scale multiplies the
    read only, never the state."""
    rng = np.random.default_rng(43)
    T, Dk, Dv = 9, 16, 4
    q = np.float32(rng.standard_normal((T, Dk)))
    k = np.float32(rng.standard_normal((T, Dk)) * 0.25)
    v = np.float32(rng.standard_normal((T, Dv)))
    g = np.float32(np.log(rng.uniform(0.8, 1.0, T)))
    beta = np.float32(rng.uniform(0, 1, T))
    o1, s1 = run1(fwd, q, k, v, g, beta)
    os_, ss = run1(fwd, q, k, v, g, beta, scale=Dk ** -0.5)
    oq, sq = run1(fwd, q * np.float32(0.25), k, v, g, beta)      # d_k^{-1/2} = 1/4 exactly
    np.testing.assert_allclose(os_, oq, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(os_, o1 / 4, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(ss, s1)


ALL_PINS = [
    pin_forget_gate_ten_steps, pin_per_zone_decay, pin_beta_zero_no_write,
    pin_phone_book, pin_double_weight_key, pin_forget_before_predict, pin_read_after_write,
    pin_constraint_unit_keys, pin_reread_interpolates, pin_locality, pin_transition_spectrum,
    pin_gradient_step, pin_kaczmarz_constraint, pin_kaczmarz_min_norm, pin_kaczmarz_line_search,
    pin_accumulate_vs_delta, pin_linear_attention_bruteforce, pin_decayed_attention_bruteforce,
    pin_table_transition_form, pin_output_scale,
]


def needs_golden(pin) -> bool:
    return pin.__code__.co_argcount == 2
