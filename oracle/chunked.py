"""Naive chunkwise form of the gated delta rule, numpy fp64 -- TEST INFRASTRUCTURE ONLY.

A second formulation of the same layer, derived by hand from the token
recurrence, used to pin the token-by-token oracle (and never by the HIP
library).  The prefill on the "2080 Ti runs Qwen3.8-27B: a vLLM plugin"
page (section 2, "GDN prefill") runs the layer chunk by chunk with chunk
length 64, in three stages: an intra-chunk preparation, the inter-chunk
state recurrence and the output.  Written in the state-transposed form
H = S^T (d_k x d_v), one chunk of length C with incoming state H0 is:

  G_r   = g_1 + ... + g_r                      (within-chunk decay cumsum)
  A_rs  = beta_r exp(G_r - G_s) (k_r . k_s)   for s < r, else 0
  Tm    = (I + A)^{-1}                         (unit lower triangular)
  W     = Tm diag(beta * exp(G)) K             (C x d_k)
  U     = Tm diag(beta) V                      (C x d_v)
  U'    = U - W H0                             (corrected writes)
  O     = diag(exp(G)) Q H0 + (M o Q K^T) U',  M_rs = exp(G_r - G_s) for s <= r
  H_C   = exp(G_C) H0 + K^T diag(exp(G_C - G)) U'

Derivation sketch: with H_t = alpha_t H_{t-1} + k_t u_t^T and
u_t = beta_t (v_t - alpha_t H_{t-1}^T k_t), unrolling H_{t-1} inside the chunk
gives u_r + beta_r sum_{s<r} exp(G_r - G_s)(k_r . k_s) u_s
= beta_r (v_r - exp(G_r) H0^T k_r), i.e. (I + A) U' = diag(beta) V
- diag(beta exp(G)) K H0, whose solution is U' = U - W H0.  The state and
output follow by summing the unrolled rank-one terms.

The matrix inverse is numpy's (a library primitive); nothing is blocked,
fused or reordered beyond these equations.
"""

from __future__ import annotations

import numpy as np


def chunk_step(Q, K, V, g, beta, H0):
    """One chunk.  Q, K: [C, d_k]; V: [C, d_v]; g, beta: [C]; H0: [d_k, d_v].

    Returns dict with G, A, Tm, W, U, Up (U'), P (M o Q K^T), O and H (outgoing state).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    C = K.shape[0]
    G = np.cumsum(g)
    diff = G[:, None] - G[None, :]
    lower = np.tril(np.ones((C, C), dtype=bool), -1)
    causal = np.tril(np.ones((C, C), dtype=bool), 0)
    # exp(G_r - G_s) only where s <= r, so every exponent is <= 0 when g <= 0
    decay = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    A = np.where(lower, beta[:, None] * decay * (K @ K.T), 0.0)
    Tm = np.linalg.inv(np.eye(C) + A)
    W = (Tm * (beta * np.exp(G))[None, :]) @ K
    U = (Tm * beta[None, :]) @ V
    Up = U - W @ H0
    P = decay * (Q @ K.T)
    O = np.exp(G)[:, None] * (Q @ H0) + P @ Up
    H = np.exp(G[-1]) * H0 + K.T @ (np.exp(G[-1] - G)[:, None] * Up)
    return {"G": G, "A": A, "Tm": Tm, "W": W, "U": U, "Up": Up, "P": P, "O": O, "H": H}


def chunked_forward(q, k, v, g, beta, cu_seqlens, initial_state=None, chunk: int = 64):
    """Whole packed batch, chunk by chunk.  Same layouts as the token oracle.

    Chunks never cross a sequence boundary; a sequence's last chunk may be short.
    Returns (out [T,H_v,d_v], final_state [N,H_v,d_k,d_v]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    group = h_v // h_qk
    n = cu.shape[0] - 1
    out = np.zeros((T, h_v, d_v))
    fin = np.zeros((n, h_v, d_k, d_v))
    for s in range(n):
        for h in range(h_v):
            j = h // group
            H = (np.zeros((d_k, d_v)) if initial_state is None
                 else np.asarray(initial_state[s, h], np.float64).copy())
            for c0 in range(int(cu[s]), int(cu[s + 1]), chunk):
                c1 = min(int(cu[s + 1]), c0 + chunk)
                r = chunk_step(q[c0:c1, j], k[c0:c1, j], v[c0:c1, h], g[c0:c1, h],
                               beta[c0:c1, h], H)
                out[c0:c1, h] = r["O"]
                H = r["H"]
            fin[s, h] = H
    return out, fin
