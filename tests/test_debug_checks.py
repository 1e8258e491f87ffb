"""CPU tests of the device-content precondition checks (what GDN_DEBUG_CHECKS
runs inside every entry point, here on host arrays): each condition is
violated once, on an otherwise valid seeded batch, and must be reported with
the offending element named."""

import numpy as np
import pytest

import gdn_inputs as gi
import hybrid_linear_attention_gdn_amd as gdn


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(gdn.LIB_PATH):
        import hybrid_linear_attention_gdn_amd.build as b
        b.build()


def batch():
    return gi.make_inputs([70, 0, 5], 2, 4, 128, 128, seed=3, state_std=0.02)


def check_chunk(x, **over):
    a = dict(q=x.q, k=x.k, v=x.v, g=x.g, beta=x.beta, cu_seqlens=x.cu_seqlens, initial_state=x.initial_state)
    a.update(over)
    gdn.gdn_check_chunk_inputs_host(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                                    a["initial_state"], h_qk=x.h_qk, h_v=x.h_v)


def expect_invalid(fn, needle):
    with pytest.raises(gdn.GDNError) as ei:
        fn()
    assert ei.value.status == gdn.GDN_ERR_INVALID_VALUE
    assert needle in str(ei.value), str(ei.value)


def test_valid_batch_passes():
    x = batch()
    check_chunk(x)
    check_chunk(x, initial_state=None)
    gdn.gdn_check_step_inputs_host(x.q, x.k, x.v, x.g, x.beta, x.initial_state, n_requests=3, h_qk=2, h_v=4)


def test_cu_seqlens_must_start_at_zero():
    x = batch()
    cu = x.cu_seqlens.copy()
    cu[0] = 1
    expect_invalid(lambda: gdn.gdn_check_chunk_inputs_host(
        x.q, x.k, x.v, x.g, x.beta, cu, None, h_qk=2, h_v=4), "cu_seqlens[0] = 1")


def test_cu_seqlens_must_not_decrease():
    x = batch()
    cu = x.cu_seqlens.copy()
    cu[1], cu[2] = 71, 70       # 0, 71, 70, 75: decreases at 1, ends at T
    expect_invalid(lambda: check_chunk(x, cu_seqlens=cu), "decreases at 1")


def test_cu_seqlens_must_end_at_total_tokens():
    from ctypes import byref
    x = batch()
    lib = gdn.load_library()
    dims = gdn.make_dims(3, 74, 2, 4)                 # one token fewer than cu[N] = 75
    bq = gdn._host_bits(x.q)
    bk = gdn._host_bits(x.k)
    bv = gdn._host_bits(x.v)
    st = lib.gdn_check_chunk_inputs_host(bq.ctypes.data, bk.ctypes.data, bv.ctypes.data, x.g.ctypes.data,
                                         x.beta.ctypes.data, x.cu_seqlens.ctypes.data, None, byref(dims))
    assert st == gdn.GDN_ERR_INVALID_VALUE
    assert b"differs from total_tokens = 74" in lib.gdn_get_last_error()


@pytest.mark.parametrize("bad", [1e-3, float("nan"), float("inf")])
def test_log_decay_must_be_finite_and_nonpositive(bad):
    x = batch()
    g = x.g.copy()
    g[7, 3] = bad
    expect_invalid(lambda: check_chunk(x, g=g), "g[31]")
    expect_invalid(lambda: gdn.gdn_check_step_inputs_host(x.q, x.k, x.v, g, x.beta, None,
                                                          n_requests=3, h_qk=2, h_v=4), "g[31]")


def test_beta_must_be_finite():
    x = batch()
    b = x.beta.copy()
    b[74, 0] = float("nan")
    expect_invalid(lambda: check_chunk(x, beta=b), "beta[296]")


@pytest.mark.parametrize("name", ["q", "k", "v"])
def test_operands_must_fit_fp16(name):
    x = batch()
    a = getattr(x, name).copy()
    a[2, 1, 5] = 65536.0                               # exact in bf16, past fp16's 65504
    idx = (2 * a.shape[1] + 1) * 128 + 5
    expect_invalid(lambda: check_chunk(x, **{name: a}), f"{name}[{idx}]")
    a[2, 1, 5] = -65280.0                              # the largest bf16 magnitude below it passes
    check_chunk(x, **{name: a})
    a[2, 1, 5] = float("inf")
    expect_invalid(lambda: check_chunk(x, **{name: a}), f"{name}[{idx}]")


def test_initial_state_must_be_finite_and_fit_fp16():
    x = batch()
    s = x.initial_state.copy()
    s[2, 3, 127, 127] = 7e4
    last = s.size - 1
    expect_invalid(lambda: check_chunk(x, initial_state=s), f"initial_state[{last}]")
    # the recurrent step keeps states in fp32: only finiteness is required there
    gdn.gdn_check_step_inputs_host(x.q, x.k, x.v, x.g, x.beta, s, n_requests=3, h_qk=2, h_v=4)
    s[0, 0, 0, 1] = float("nan")
    expect_invalid(lambda: gdn.gdn_check_step_inputs_host(x.q, x.k, x.v, x.g, x.beta, s,
                                                          n_requests=3, h_qk=2, h_v=4), "state_in[1]")


def test_bad_dims_come_back_as_the_entry_points_report_them():
    x = batch()
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_check_chunk_inputs_host(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, None, h_qk=3, h_v=4)
    assert ei.value.status == gdn.GDN_ERR_INVALID_VALUE
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_check_chunk_inputs_host(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, None, h_qk=2, h_v=4, d_k=64)
    assert ei.value.status == gdn.GDN_ERR_NOT_SUPPORTED
