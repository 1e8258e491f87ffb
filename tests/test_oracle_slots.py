"""Pins of the slot-pool oracle (``oracle.slots.slots_step``), CPU only.

Each test checks the bookkeeping against a fact that does not come from the
bookkeeping itself: the packed recurrence over whole sequences (rollback ==
resuming from the accepted prefix), a closed form for one token, identity
steps, and the documented handling of bad indices.
"""

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle.slots import slots_step


def small(lengths, seed=0, state_std=0.3):
    return gi.make_inputs(lengths, 1, 2, 16, 16, seed=seed, state_std=state_std)


def test_contiguous_table_reproduces_recorded_states():
    x = small([4, 1, 3])
    R, M = 3, 4
    pool = gi.state_pool(x, R * M)
    table = gi.slot_table_contiguous(R, M, R)
    out, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    ref_out, ref_fin, states = oracle.forward_inputs(x, record_states=True)
    np.testing.assert_array_equal(out, ref_out)
    for r in range(R):
        t0, t1 = x.cu_seqlens[r], x.cu_seqlens[r + 1]
        for t in range(t1 - t0):
            np.testing.assert_array_equal(new_pool[table[r, 1 + t]], states[t0 + t].astype(np.float32))
        for t in range(t1 - t0, M):   # rows past the request's tokens are untouched
            np.testing.assert_array_equal(new_pool[table[r, 1 + t]], pool[table[r, 1 + t]])
    np.testing.assert_array_equal(new_pool[:R], pool[:R])   # incoming slots only read


@pytest.mark.parametrize("accepted", [[1, 3, 5], [5, 1, 2], [2, 2, 2]])
def test_rollback_equals_resume_from_accepted_prefix(accepted):
    """Call 1 verifies 5 tokens per request; call 2 reads column accepted[r].
    That must equal one uninterrupted run over the first accepted[r] tokens of
    call 1 followed by the tokens of call 2 (the rejected drafts never happened)."""
    R, M = 3, 5
    x1 = small([M] * R, seed=1)
    x2 = small([4, 2, 3], seed=2)
    pool = gi.state_pool(x1, R * M)
    table = gi.slot_table_contiguous(R, M, R)
    _, pool1 = slots_step(x1.q, x1.k, x1.v, x1.g, x1.beta, x1.cu_seqlens, pool, table)
    acc = np.array(accepted, np.int32)
    out2, pool2 = slots_step(x2.q, x2.k, x2.v, x2.g, x2.beta, x2.cu_seqlens, pool1, table, acc)
    for r in range(R):
        a = accepted[r]
        s1 = slice(x1.cu_seqlens[r], x1.cu_seqlens[r] + a)
        s2 = slice(x2.cu_seqlens[r], x2.cu_seqlens[r + 1])
        cat = lambda f: np.concatenate([getattr(x1, f)[s1], getattr(x2, f)[s2]])
        n2 = s2.stop - s2.start
        o, fin, _ = oracle.forward(cat("q"), cat("k"), cat("v"), cat("g"), cat("beta"),
                                   np.array([0, a + n2], np.int32), pool[r:r + 1].astype(np.float64))
        # call 1 stored its states in an fp32 pool: agreement to fp32 rounding
        np.testing.assert_allclose(out2[s2], o[a:], rtol=0, atol=1e-7)
        # the state after the last token of call 2 sits in column n2
        np.testing.assert_allclose(pool2[table[r, n2]], fin[0], rtol=0, atol=1e-6)


def test_in_place_incoming_slot():
    """A request may name its incoming slot as a write slot (decode in place)."""
    x = small([1, 1])
    pool = gi.state_pool(x, 0)
    table = np.array([[0, 0], [1, 1]], np.int32)
    out, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    ref_out, ref_fin, _ = oracle.forward_inputs(x)
    np.testing.assert_array_equal(out, ref_out)
    np.testing.assert_array_equal(new_pool, ref_fin.astype(np.float32))


def test_fp16_identity_steps_keep_pool_bitwise():
    """g = 0, beta = 0: every stored state equals the incoming one exactly, so an
    fp16 pool is copied bit for bit, and o_t = S0 q_t."""
    x = small([3, 2])
    x.g[:] = 0.0
    x.beta[:] = 0.0
    pool = gi.state_pool(x, 10, f16=True)
    table = gi.slot_table_contiguous(2, 3, 2)
    out, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    for r, n in enumerate([3, 2]):
        for t in range(n):
            assert np.array_equal(new_pool[table[r, 1 + t]].view(np.uint16), pool[r].view(np.uint16))
        t0 = x.cu_seqlens[r]
        j = 0
        for t in range(n):
            for h in range(2):
                expect = pool[r, h].astype(np.float64).T @ x.q[t0 + t, j].astype(np.float64)
                np.testing.assert_allclose(out[t0 + t, h], expect, rtol=1e-12, atol=1e-14)


def test_fp16_single_token_closed_form():
    """T = 1 from a zero state: S_1 = beta v k^T, stored as its fp16 rounding."""
    x = small([1], state_std=None)
    pool = np.zeros((2, 2, 16, 16), np.float16)
    table = np.array([[0, 1]], np.int32)
    out, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    for h in range(2):
        b = np.float64(x.beta[0, h])
        kk = x.k[0, 0].astype(np.float64)
        vv = x.v[0, h].astype(np.float64)
        H = b * np.outer(kk, vv)        # H = S^T: [d_k][d_v]
        assert np.array_equal(new_pool[1, h], H.astype(np.float16))
        np.testing.assert_allclose(out[0, h], b * (kk @ x.q[0, 0].astype(np.float64)) * vv,
                                   rtol=1e-12, atol=1e-15)


def test_negative_write_slot_is_not_stored():
    x = small([3])
    pool = gi.state_pool(x, 3)
    table = np.array([[0, 1, -1, 3]], np.int32)
    _, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    np.testing.assert_array_equal(new_pool[2], pool[2])
    assert not np.array_equal(new_pool[1], pool[1])
    assert not np.array_equal(new_pool[3], pool[3])


@pytest.mark.parametrize("case", ["read_slot", "write_slot", "accepted_col"])
def test_bad_index_gives_nan_and_no_state_change(case):
    x = small([2, 2])
    pool = gi.state_pool(x, 4)
    table = gi.slot_table_contiguous(2, 2, 2)
    acc = None
    if case == "read_slot":
        table[1, 0] = 6
    elif case == "write_slot":
        table[1, 2] = 99
    else:
        acc = np.array([0, 3], np.int32)
    out, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table, acc)
    assert np.isnan(out[2:4]).all() and np.isfinite(out[0:2]).all()
    np.testing.assert_array_equal(new_pool[table[1, 1]], pool[table[1, 1]])
    assert not np.array_equal(new_pool[table[0, 1]], pool[table[0, 1]])


def test_bad_token_range_is_skipped():
    x = small([2, 2])
    pool = gi.state_pool(x, 4)
    table = gi.slot_table_contiguous(2, 2, 2)
    cu = np.array([0, 2, 7], np.int32)          # request 1 runs past T = 4
    out, new_pool = slots_step(x.q, x.k, x.v, x.g, x.beta, cu, pool, table)
    assert (out[2:4] == 0).all()
    np.testing.assert_array_equal(new_pool[4:6], pool[4:6])
