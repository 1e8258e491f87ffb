"""GPU parity of gdn_recurrent_step_slots (state pool, slot table, accepted
counts, fp32 or fp16 storage) against the slot-pool oracle.

Tolerances: relative L2 <= 2e-3 on outputs, <= 1e-3 on every stored state.
An fp16 pool is compared with the oracle's fp16-rounded states.  Slots the
call must not write are compared bit for bit with their previous contents.
"""

import numpy as np
import pytest

import gdn_inputs as gi
from oracle.slots import slots_step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import hybrid_linear_attention_gdn_amd as gdn  # noqa: E402
from gpu_util import OUT_TOL, STATE_TOL, DevInputs, recurrent_step, rel_l2  # noqa: E402

SENTINEL = 7.0


def run_slots(x, pool_np, table_np, acc_np=None, cu_np=None):
    """One call on the GPU; returns (out, pool) as numpy."""
    d = DevInputs(x)
    pool = torch.from_numpy(np.ascontiguousarray(pool_np)).cuda()
    table = torch.from_numpy(np.ascontiguousarray(table_np, np.int32)).cuda()
    acc = None if acc_np is None else torch.from_numpy(np.asarray(acc_np, np.int32)).cuda()
    cu = d.cu if cu_np is None else torch.from_numpy(np.asarray(cu_np, np.int32)).cuda()
    out = torch.full((x.total_tokens, x.h_v, x.d_v), SENTINEL, dtype=torch.float32, device="cuda")
    R = cu.shape[0] - 1
    print(f"[case] slots R={R} T={x.total_tokens} pool={tuple(pool.shape)} {pool.dtype} "
          f"max_tokens={table.shape[1] - 1} accepted={acc_np}", flush=True)
    gdn.gdn_recurrent_step_slots(d.q, d.k, d.v, d.g, d.beta, cu, R, table.shape[1] - 1,
                                 pool, table, acc, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), pool.cpu().numpy()


def check_pool(gpu_pool, ref_pool, old_pool, written):
    """Written slots within the state bound, all others bitwise unchanged."""
    for s in range(old_pool.shape[0]):
        if s in written:
            e = rel_l2(gpu_pool[s].astype(np.float64), ref_pool[s].astype(np.float64))
            assert e <= STATE_TOL, (s, e)
        else:
            assert np.array_equal(gpu_pool[s].view(np.uint8), old_pool[s].view(np.uint8)), s


def written_slots(table, cu, acc=None):
    out = set()
    for r in range(table.shape[0]):
        n = int(cu[r + 1] - cu[r])
        out.update(int(s) for s in table[r, 1:1 + n] if s >= 0)
    return out


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_slots_variable_tokens(f16):
    lengths = [6, 1, 4, 6, 2, 5, 3, 6]
    x = gi.verify_variable(lengths, seed=21)
    R, M = len(lengths), 6
    pool = gi.state_pool(x, R * M, f16=f16, seed=21)
    table = gi.slot_table_contiguous(R, M, R)
    out, gpool = run_slots(x, pool, table)
    ro, rpool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    e = rel_l2(out, ro)
    print(f"[result] out rel-L2 {e:.3e}", flush=True)
    assert e <= OUT_TOL
    check_pool(gpool, rpool, pool, written_slots(table, x.cu_seqlens))


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_slots_rollback_by_accepted_count(f16):
    """Call 1 verifies 6 tokens per request; call 2 reads the column that the
    device-side accepted counts name and writes into the same slot row."""
    R, M = 8, 6
    x1 = gi.verify_variable([M] * R, seed=31)
    x2 = gi.verify_variable([3, 6, 1, 2, 6, 4, 5, 2], seed=32)
    pool = gi.state_pool(x1, R * M, f16=f16, seed=31)
    table = gi.slot_table_contiguous(R, M, R)
    acc = np.array([1, 6, 3, 2, 5, 4, 6, 1], np.int32)
    _, gpool1 = run_slots(x1, pool, table)
    _, rpool1 = slots_step(x1.q, x1.k, x1.v, x1.g, x1.beta, x1.cu_seqlens, pool, table)
    out2, gpool2 = run_slots(x2, gpool1, table, acc)
    # the oracle continues from its own pool: errors of the two calls add up
    ro2, rpool2 = slots_step(x2.q, x2.k, x2.v, x2.g, x2.beta, x2.cu_seqlens, rpool1, table, acc)
    e = rel_l2(out2, ro2)
    print(f"[result] out rel-L2 {e:.3e}", flush=True)
    assert e <= OUT_TOL
    check_pool(gpool2, rpool2, gpool1, written_slots(table, x2.cu_seqlens))


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_slots_decode_in_place_chain(f16):
    """Decode: one token per request, read and write the same slot, four calls."""
    R = 16
    pool = None
    ref = None
    table = np.stack([np.arange(R), np.arange(R)], axis=1).astype(np.int32)
    for step in range(4):
        x = gi.verify_variable([1] * R, seed=40 + step)
        if pool is None:
            pool = gi.state_pool(x, 0, f16=f16, seed=40)
            ref = pool.copy()
        out, pool = run_slots(x, pool, table)
        ro, ref = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, ref, table)
        assert rel_l2(out, ro) <= OUT_TOL
        assert rel_l2(pool.astype(np.float64), ref.astype(np.float64)) <= STATE_TOL


def test_slots_fp32_contiguous_equals_fixed_layout_bitwise():
    """An fp32 pool with the contiguous table runs the same arithmetic as
    gdn_recurrent_step with snapshots: identical bits."""
    x = gi.verify_8x6(seed=3)
    R, M = 8, 6
    pool = gi.state_pool(x, R * M, seed=3)
    table = gi.slot_table_contiguous(R, M, R)
    out_s, pool_s = run_slots(x, pool, table)
    d = DevInputs(x)
    out_f, s_out, inter = recurrent_step(d, R, M, save=True)
    np.testing.assert_array_equal(out_s, out_f.cpu().numpy())
    np.testing.assert_array_equal(pool_s[R:].reshape(R, M, *pool.shape[1:]), inter.cpu().numpy())


def test_slots_bad_indices_are_contained():
    """Request 1: incoming slot past the pool; 2: a write slot past the pool;
    3: accepted column past the table; 4: token range past T.  Requests 1-3
    get NaN outputs and no state change, request 4 is skipped, request 0 runs."""
    lengths = [3, 2, 2, 2, 2]
    x = gi.verify_variable(lengths, seed=51)
    R, M = 5, 3
    pool = gi.state_pool(x, R * M, f16=True, seed=51)
    P = pool.shape[0]
    table = gi.slot_table_contiguous(R, M, R)
    table[1, 0] = P
    table[2, 2] = P + 5
    acc = np.zeros(R, np.int32)
    acc[3] = M + 1
    cu = x.cu_seqlens.copy()
    cu[5] = x.total_tokens + 3
    out, gpool = run_slots(x, pool, table, acc, cu)
    c = x.cu_seqlens
    assert np.isfinite(out[c[0]:c[1]]).all()
    for r in (1, 2, 3):
        assert np.isnan(out[c[r]:c[r + 1]]).all(), r
    assert (out[c[4]:] == SENTINEL).all()
    ro, rpool = slots_step(x.q, x.k, x.v, x.g, x.beta, cu, pool, table, acc)
    assert rel_l2(out[c[0]:c[1]], ro[c[0]:c[1]]) <= OUT_TOL
    check_pool(gpool, rpool, pool, {int(s) for s in table[0, 1:4]})


def test_slots_zero_token_requests():
    lengths = [0, 3, 0, 1]
    x = gi.verify_variable(lengths, seed=61)
    R, M = 4, 3
    pool = gi.state_pool(x, R * M, f16=True, seed=61)
    table = gi.slot_table_contiguous(R, M, R)
    out, gpool = run_slots(x, pool, table)
    ro, rpool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    assert rel_l2(out, ro) <= OUT_TOL
    check_pool(gpool, rpool, pool, written_slots(table, x.cu_seqlens))


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_slots_requests_longer_than_a_staging_block(f16):
    """Requests of 9..20 tokens: token inputs are staged 16 at a time, k and q
    in two passes of 8 tokens; the last request spans two staging blocks."""
    lengths = [9, 12, 16, 20]
    x = gi.verify_variable(lengths, seed=71)
    R, M = len(lengths), max(lengths)
    pool = gi.state_pool(x, R * M, f16=f16, seed=71)
    table = gi.slot_table_contiguous(R, M, R)
    out, gpool = run_slots(x, pool, table)
    ro, rpool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table)
    e = rel_l2(out, ro)
    print(f"[result] out rel-L2 {e:.3e}", flush=True)
    assert e <= OUT_TOL
    check_pool(gpool, rpool, pool, written_slots(table, x.cu_seqlens))
