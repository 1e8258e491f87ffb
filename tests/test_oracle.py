"""Pins for the CPU oracle (runs on CPU, no GPU).

The pages print no GDN values, so the oracle is pinned by facts the
mathematics fixes: closed forms, identities of the gated delta rule, an
exact rational brute force of the literal matrix formula on tiny inputs,
agreement with an independently derived chunkwise form, and the state
hand-off property that prefix caching relies on (the "Qwen3.8-27B on one RTX
3090" page, section on prefix caching, stores the recurrent state and resumes
from it).  Each pin is chosen so that a plausible slip in the oracle (decay
applied after the write, transposed state, output from the old state, a
dropped beta, a wrong head mapping) fails at least one of them.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle import chunked


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def small(T=24, h_qk=2, h_v=4, d_k=8, d_v=6, seed=3, state_std=0.5, lengths=None, **kw):
    if lengths is None:
        lengths = [T]
    return gi.make_inputs(lengths, h_qk, h_v, d_k, d_v, seed=seed, bf16=False,
                          state_std=state_std, **kw)


# ---------------------------------------------------------------- closed forms

def test_beta_zero_is_pure_decay():
    """beta == 0: S_t = exp(G_t) S_0 and o_t = exp(G_t) S_0 q_t."""
    x = small()
    x.beta[:] = 0.0
    out, fin, states = oracle.forward_inputs(x, record_states=True)
    G = np.cumsum(x.g.astype(np.float64), axis=0)            # [T, H_v]
    group = x.h_v // x.h_qk
    for h in range(x.h_v):
        S0 = x.initial_state[0, h].astype(np.float64)          # [d_k, d_v]
        for t in range(x.total_tokens):
            f = math.exp(G[t, h])
            np.testing.assert_allclose(states[t, h], f * S0, rtol=1e-13, atol=1e-300)
            o = f * (x.q[t, h // group].astype(np.float64) @ S0)
            np.testing.assert_allclose(out[t, h], o, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(fin[0], states[-1])


def test_identity_step_keeps_state_bitwise():
    """alpha == 1 and beta == 0: the state never changes, o_t = S_0 q_t."""
    x = small()
    x.beta[:] = 0.0
    x.g[:] = 0.0
    out, fin, _ = oracle.forward_inputs(x)
    np.testing.assert_array_equal(fin, x.initial_state.astype(np.float64))
    group = x.h_v // x.h_qk
    for h in range(x.h_v):
        ref = x.q[:, h // group].astype(np.float64) @ x.initial_state[0, h].astype(np.float64)
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("g_mean", [0.0, -3.0])
def test_unit_key_full_write_recalls_value(g_mean):
    """beta == 1 with unit k_t: the state maps k_t to v_t exactly, whatever alpha."""
    x = small(g_mean=g_mean)
    x.beta[:] = 1.0
    _, _, states = oracle.forward_inputs(x, record_states=True)
    group = x.h_v // x.h_qk
    for t in range(x.total_tokens):
        for h in range(x.h_v):
            k = x.k[t, h // group].astype(np.float64)
            assert abs(np.linalg.norm(k) - 1.0) < 1e-6
            # S_t k_t in the stored orientation state[a][c] = S[c][a]
            recalled = k @ states[t, h]
            # k is only float32-unit-norm, so allow for |k|^2 != 1 at 1e-7
            np.testing.assert_allclose(recalled, x.v[t, h], rtol=0, atol=1e-6 * np.abs(x.v[t, h]).max())


def test_unit_key_recall_is_exact_with_exact_norm():
    """Same identity with k scaled to unit norm in float64 arithmetic: error at rounding level."""
    x = small(T=10)
    x.beta[:] = 1.0
    # entries +-1/2 on four coordinates: exactly unit norm in binary arithmetic
    signs = np.random.default_rng(7).choice([-0.5, 0.5], size=(x.total_tokens, 4)).astype(np.float32)
    x.k[:] = 0.0
    x.k[:, :, 2:6] = signs[:, None, :]
    _, _, states = oracle.forward_inputs(x, record_states=True)
    group = x.h_v // x.h_qk
    for t in range(x.total_tokens):
        for h in range(x.h_v):
            k = x.k[t, h // group].astype(np.float64)
            np.testing.assert_allclose(k @ states[t, h], x.v[t, h], rtol=0, atol=1e-14)


def test_single_token_closed_form():
    """T = 1, S_0 = 0: S_1 = beta v k^T and o_1 = beta (k . q) v."""
    x = small(T=1, state_std=None)
    out, fin, _ = oracle.forward_inputs(x)
    group = x.h_v // x.h_qk
    for h in range(x.h_v):
        q = x.q[0, h // group].astype(np.float64)
        k = x.k[0, h // group].astype(np.float64)
        v = x.v[0, h].astype(np.float64)
        b = float(x.beta[0, h])
        np.testing.assert_allclose(fin[0, h], b * np.outer(k, v), rtol=1e-15, atol=0)
        np.testing.assert_allclose(out[0, h], b * float(k @ q) * v, rtol=1e-14, atol=1e-16)


def _exact_literal(q, k, v, alpha, beta, S0):
    """S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T, o_t = S_t q_t, in exact rationals.

    S is d_v x d_k as in the formula (not the stored transpose)."""
    F = Fraction
    T, dk = k.shape
    dv = v.shape[1]
    S = [[F(float(S0[c][a])) for a in range(dk)] for c in range(dv)]
    outs = []
    for t in range(T):
        kt = [F(float(e)) for e in k[t]]
        qt = [F(float(e)) for e in q[t]]
        vt = [F(float(e)) for e in v[t]]
        al, be = F(float(alpha[t])), F(float(beta[t]))
        # P = I - beta k k^T
        P = [[(F(1) if a == b else F(0)) - be * kt[a] * kt[b] for b in range(dk)] for a in range(dk)]
        SP = [[sum(S[c][a] * P[a][b] for a in range(dk)) for b in range(dk)] for c in range(dv)]
        S = [[al * SP[c][b] + be * vt[c] * kt[b] for b in range(dk)] for c in range(dv)]
        outs.append([sum(S[c][a] * qt[a] for a in range(dk)) for c in range(dv)])
    return outs, S


def test_exact_rational_brute_force_of_literal_formula():
    """The oracle's loop equals the literal matrix formula evaluated exactly."""
    x = small(T=5, h_qk=1, h_v=1, d_k=3, d_v=2, seed=11)
    out, fin, _ = oracle.forward_inputs(x)
    alpha = [math.exp(float(gv)) for gv in x.g[:, 0]]   # same libm exp the C oracle calls
    exact_out, exact_S = _exact_literal(x.q[:, 0], x.k[:, 0], x.v[:, 0], alpha, x.beta[:, 0],
                                        x.initial_state[0, 0].T)
    eo = np.array([[float(e) for e in row] for row in exact_out])
    eS = np.array([[float(e) for e in row] for row in exact_S])     # [d_v, d_k]
    np.testing.assert_allclose(out[:, 0], eo, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin[0, 0], eS.T, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- structure

def test_linear_in_values_and_initial_state():
    """For fixed q, k, g, beta the map (V, S_0) -> (out, S_T) is linear."""
    a = small(seed=5)
    b = small(seed=6)
    b.q, b.k, b.g, b.beta = a.q, a.k, a.g, a.beta
    # bfloat16-valued V and S_0 so that the float32 sums below are exact
    for x in (a, b):
        x.v = gi.bf16_round(x.v)
        x.initial_state = gi.bf16_round(x.initial_state)
    c = small(seed=5)
    c.v = a.v + b.v
    c.initial_state = a.initial_state + b.initial_state
    assert np.array_equal(c.v.astype(np.float64), a.v.astype(np.float64) + b.v)
    assert np.array_equal(c.initial_state.astype(np.float64),
                          a.initial_state.astype(np.float64) + b.initial_state)
    oa, fa, _ = oracle.forward_inputs(a)
    ob, fb, _ = oracle.forward_inputs(b)
    oc, fc, _ = oracle.forward_inputs(c)
    assert rel(oa + ob, oc) < 1e-13
    assert rel(fa + fb, fc) < 1e-13


def test_split_invariance_every_point_tiny():
    """Running [0, s) then [s, T) with the handed-off state equals the unsplit run."""
    x = gi.tiny()
    out, fin, _ = oracle.forward_inputs(x)
    T = x.total_tokens
    for s in range(1, T):
        o1, f1, _ = oracle.forward(x.q[:s], x.k[:s], x.v[:s], x.g[:s], x.beta[:s], [0, s])
        o2, f2, _ = oracle.forward(x.q[s:], x.k[s:], x.v[s:], x.g[s:], x.beta[s:], [0, T - s], f1)
        np.testing.assert_array_equal(np.concatenate([o1, o2]), out)
        np.testing.assert_array_equal(f2, fin)


def test_packed_varlen_equals_separate_runs():
    x = small(lengths=[7, 0, 19, 1, 33], seed=9)
    out, fin, _ = oracle.forward_inputs(x)
    for n in range(x.n_seqs):
        y = x.slice_seq(n)
        o, f, _ = oracle.forward_inputs(y)
        a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
        np.testing.assert_array_equal(out[a:b], o)
        np.testing.assert_array_equal(fin[n], f[0])
    # zero-length sequence hands its initial state straight through
    np.testing.assert_array_equal(fin[1], x.initial_state[1].astype(np.float64))


def test_value_heads_share_qk_heads_in_contiguous_groups():
    """Value head h reads q/k head h // (H_v / H_qk): same as repeating q, k per group."""
    x = small(h_qk=2, h_v=6)
    out, fin, _ = oracle.forward_inputs(x)
    rep = np.repeat(np.arange(2), 3)
    o2, f2, _ = oracle.forward(x.q[:, rep], x.k[:, rep], x.v, x.g, x.beta, x.cu_seqlens, x.initial_state)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(fin, f2)


@pytest.mark.parametrize("C", [1, 7, 16, 64, 128])
def test_chunkwise_form_agrees_with_token_recurrence(C):
    """An independently derived chunk form gives the same result in fp64."""
    x = gi.tiny()
    x.initial_state = (0.3 * np.random.default_rng(1).standard_normal((1, 1, 32, 32))).astype(np.float32)
    out, fin, _ = oracle.forward_inputs(x)
    oc, fc = chunked.chunked_forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, chunk=C)
    assert rel(oc, out) < 1e-12
    assert rel(fc, fin) < 1e-12


def test_chunkwise_form_agrees_on_packed_multihead_batch():
    x = small(lengths=[70, 3, 130], h_qk=2, h_v=4, d_k=16, d_v=8, seed=4)
    out, fin, _ = oracle.forward_inputs(x)
    oc, fc = chunked.chunked_forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, chunk=64)
    assert rel(oc, out) < 1e-12
    assert rel(fc, fin) < 1e-12


def test_chunk_pieces_satisfy_their_defining_equations():
    """(I + A) Tm = I, and U' solves (I + A) U' = diag(beta) V - diag(beta e^G) K H0."""
    x = small(T=64, h_qk=1, h_v=1, d_k=16, d_v=8)
    H0 = x.initial_state[0, 0].astype(np.float64)
    r = chunked.chunk_step(x.q[:, 0], x.k[:, 0], x.v[:, 0], x.g[:, 0], x.beta[:, 0], H0)
    I = np.eye(64)
    np.testing.assert_allclose((I + r["A"]) @ r["Tm"], I, atol=1e-12)
    b = x.beta[:, 0].astype(np.float64)
    rhs = b[:, None] * x.v[:, 0] - (b * np.exp(r["G"]))[:, None] * (x.k[:, 0].astype(np.float64) @ H0)
    np.testing.assert_allclose((I + r["A"]) @ r["Up"], rhs, atol=1e-12)
    assert np.all(np.triu(r["A"]) == 0)


def test_padding_with_identity_tokens_changes_nothing():
    """Appending tokens with g = 0, beta = 0 leaves the final state unchanged."""
    x = small(T=40)
    _, fin, _ = oracle.forward_inputs(x)
    pad = 24
    q = np.concatenate([x.q, np.zeros((pad,) + x.q.shape[1:], np.float32)])
    k = np.concatenate([x.k, np.zeros((pad,) + x.k.shape[1:], np.float32)])
    v = np.concatenate([x.v, np.zeros((pad,) + x.v.shape[1:], np.float32)])
    g = np.concatenate([x.g, np.zeros((pad, x.h_v), np.float32)])
    b = np.concatenate([x.beta, np.zeros((pad, x.h_v), np.float32)])
    _, fin2, _ = oracle.forward(q, k, v, g, b, [0, 64], x.initial_state)
    np.testing.assert_array_equal(fin2, fin)


# ---------------------------------------------------------------- precision

def test_fp32_instantiation_close_to_fp64():
    x = gi.tiny()
    o64, f64, _ = oracle.forward_inputs(x, precision="f64")
    o32, f32, _ = oracle.forward_inputs(x, precision="f32")
    assert rel(o32, o64) < 1e-5
    assert rel(f32, f64) < 1e-5


def test_fp32_close_to_fp64_on_full_width_heads():
    x = gi.make_inputs([300, 200], 2, 4, 128, 128, seed=2, state_std=0.02)
    o64, f64, _ = oracle.forward_inputs(x, precision="f64")
    o32, f32, _ = oracle.forward_inputs(x, precision="f32")
    assert rel(o32, o64) < 1e-5
    assert rel(f32, f64) < 1e-5


def test_record_states_last_equals_final():
    x = small(lengths=[5, 9])
    _, fin, st = oracle.forward_inputs(x, record_states=True)
    np.testing.assert_array_equal(st[4], fin[0])
    np.testing.assert_array_equal(st[13], fin[1])


def test_oracle_rejects_inconsistent_cu_seqlens():
    x = small()
    with pytest.raises(ValueError):
        oracle.forward(x.q, x.k, x.v, x.g, x.beta, [0, x.total_tokens - 1])


def test_golden_tiny_regression():
    """Stored oracle output for the tiny workload (written by tests/golden/make_golden.py)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_f64.txt")
    ref = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, vals = line.split("=", 1)
            ref[key.strip()] = np.array([float(s) for s in vals.split()])
    x = gi.tiny()
    out, fin, _ = oracle.forward_inputs(x)
    np.testing.assert_allclose(out[::16, 0, :4].ravel(), ref["out[::16,0,:4]"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(fin[0, 0, ::8, ::8].ravel(), ref["final[0,0,::8,::8]"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(out), ref["norm(out)"][0], rtol=1e-12)
