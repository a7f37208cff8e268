"""The chunked form of the gated delta rule, in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This is a second CPU
formulation, written from the blog summary's section "KDA por chunks" (the
subsections on cumulative decay and provisional error, restoring the causal
dependence, the chunk-end state and the in-chunk outputs).  It shares no code
with the token recurrence in ``gdr_oracle.c``; the two agreeing to rounding is
one of the pins of the oracle, since the page states that the chunked schedule
yields exactly the state and outputs of the token-by-token one.

The page writes the state as d_v x d_k; here it is d_k x d_v (the Kaczmarz
page's orientation), so every product is transposed accordingly:

* cumulative decay inside a chunk: D_{0:i} = D_0 ... D_i, stored as
  G_i = sum_{m<=i} g_m (log domain), D_{j+1:i} = exp(G_i - G_j);
* provisional errors  ebar_i = beta_i (v_i - S_c^T D_{0:i} k_i);
* rho_ij = beta_i k_j^T D_{j+1:i} k_i for j < i (strictly lower R);
  the true errors solve (I + R) E = Ebar, one unit-lower triangular system
  per value channel;
* chunk-end state  S_{c+1} = D_{0:n-1} S_c + (K^end)^T E with
  K^end_j = D_{j+1:n-1} k_j;
* outputs  o_i = s S_c^T D_{0:i} q_i + sum_{j<=i} chi_ij e_j with
  chi_ij = s k_j^T D_{j+1:i} q_i (diagonal kept: the read follows the write).

Here the errors e carry the factor beta (the blog's e_t = beta_t (v_t - ...));
the Kaczmarz page's e excludes it -- the update is the same.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_fwd(q, k, v, g, beta, *, chunk: int = 64, per_channel: bool = False,
              kaczmarz: bool = False, eps: float = 0.0, scale: float = 1.0, s0=None):
    """Chunked forward pass for all (b, h); returns (o, s_final) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    o = np.zeros((B, T, H, Dv))
    s_final = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                n = t1 - t0
                Q = q[b, t0:t1, h]            # [n, Dk]
                K = k[b, t0:t1, h]            # [n, Dk]
                V = v[b, t0:t1, h]            # [n, Dv]
                if per_channel:
                    gc = g[b, t0:t1, h]       # [n, Dk]
                else:
                    gc = np.repeat(g[b, t0:t1, h][:, None], Dk, axis=1)
                if kaczmarz:
                    bc = beta[b, t0:t1, h] / (np.sum(K * K, axis=1) + eps)
                else:
                    bc = beta[b, t0:t1, h]
                G = np.cumsum(gc, axis=0)                     # [n, Dk], G_i = log D_{0:i}
                # D_{j+1:i} for j <= i as exp(G_i - G_j); masked above the diagonal
                diff = G[:, None, :] - G[None, :, :]          # [i, j, c]
                lower_incl = np.tril(np.ones((n, n), dtype=bool))
                Dij = np.where(lower_incl[:, :, None], np.exp(np.where(lower_incl[:, :, None], diff, 0.0)), 0.0)

                Ebar = bc[:, None] * (V - (np.exp(G) * K) @ S)                 # [n, Dv]
                R = bc[:, None] * np.einsum("jc,ijc,ic->ij", K, Dij, K)
                R = np.tril(R, k=-1)
                E = solve_triangular(np.eye(n) + R, Ebar, lower=True, unit_diagonal=True)

                chi = scale * np.einsum("jc,ijc,ic->ij", K, Dij, Q)           # j <= i
                o[b, t0:t1, h] = scale * (np.exp(G) * Q) @ S + chi @ E

                Kend = np.exp(G[n - 1][None, :] - G) * K                       # [n, Dk]
                S = np.exp(G[n - 1])[:, None] * S + Kend.T @ E
            s_final[b, h] = S
    return o, s_final
