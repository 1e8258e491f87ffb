"""GPU parity over seeded random batches.

Each case draws a batch shape from a fixed seed: head layout, number of
sequences, lengths (with empty, one-token and chunk-boundary lengths mixed
in), decay strength, whether q alone or q and k carry the 1/sqrt(d_k)
scale, and whether there is an initial state.  The chunked prefill and the
recurrent step are checked against the fp64 oracle with the same gates as
the named workloads: whole-tensor, per (sequence, value head) and per
boundary row.  The slot-pool step is checked against the slot-pool oracle
with the gates of its own tests: stored states within the state bound, every
slot the call must not write unchanged bit for bit.
"""

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import (OUT_TOL, STATE_TOL, DevInputs, check_detail, chunk_fwd,  # noqa: E402
                      recurrent_step, rel_l2)
from oracle.slots import slots_step  # noqa: E402
from test_gpu_parity import _segmented, _snapshots  # noqa: E402
from test_gpu_slots import check_pool, run_slots  # noqa: E402

# (q/k heads, value heads): one, two, three, four and eight value heads per
# q/k head, including the odd groupings that run one value head per prep
# workgroup
HEADS = [(1, 1), (2, 4), (4, 8), (2, 6), (1, 3), (16, 32), (2, 16), (3, 12)]
SPECIAL = [0, 1, 2, 63, 64, 65, 127, 128, 129]


def _draw(seed, heads=HEADS, max_seqs=10, max_len=600):
    rng = np.random.default_rng(7000 + seed)
    hqk, hv = heads[seed % len(heads)]
    n = int(rng.integers(1, max_seqs + 1))
    lengths = [int(rng.choice(SPECIAL)) if rng.random() < 0.35 else int(rng.integers(1, max_len))
               for _ in range(n)]
    g_mean = float(rng.choice([0.0, -2.0, 2.0]))
    state = bool(rng.random() < 0.6)
    k_scale = bool(rng.random() < 0.25)
    x = gi.make_inputs(lengths, hqk, hv, 128, 128, seed=7000 + seed, g_mean=g_mean,
                       state_std=0.02 if state else None, k_scale=k_scale, name=f"sweep{seed}")
    return x, dict(heads=(hqk, hv), lengths=lengths, g_mean=g_mean, state=state, k_scale=k_scale)


@pytest.mark.parametrize("seed", range(96))
def test_chunk_random_batch(seed):
    x, desc = _draw(seed)
    print(f"[case] sweep chunk {seed}: {desc}", flush=True)
    out, fin = chunk_fwd(DevInputs(x), poison=True)
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o, f = out.cpu().numpy(), fin.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(f).all()
    eo, ef = rel_l2(o, ro), rel_l2(f, rf)
    print(f"[result] sweep chunk {seed}: out {eo:.3e} state {ef:.3e}", flush=True)
    assert eo <= OUT_TOL and ef <= STATE_TOL
    check_detail(f"sweep{seed}", o, ro, f, rf, x.cu_seqlens)


@pytest.mark.parametrize("seed", range(48))
def test_recurrent_random_batch(seed):
    """R requests of n tokens each (the step's fixed tokens per request), with
    every per-token state saved, against the oracle's per-token states."""
    rng = np.random.default_rng(8000 + seed)
    hqk, hv = HEADS[seed % len(HEADS)]
    R, n = int(rng.integers(1, 11)), int(rng.integers(1, 9))
    x = gi.make_inputs([n] * R, hqk, hv, 128, 128, seed=8000 + seed, state_std=0.02,
                       g_mean=float(rng.choice([0.0, -2.0])), name=f"sweep_step{seed}")
    print(f"[case] sweep step {seed}: heads {hqk}/{hv} R={R} n={n}", flush=True)
    d = DevInputs(x)
    out, s_out, inter = recurrent_step(d, R, n, save=True)
    ro, rf, rs = oracle.forward_inputs(x, precision="f64", record_states=True)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(s_out.cpu().numpy(), rf) <= STATE_TOL
    snaps = inter.cpu().numpy().reshape(rs.shape)
    for t in range(R * n):
        assert rel_l2(snaps[t], rs[t]) <= STATE_TOL, t
    check_detail(f"sweep_step{seed}", out.cpu().numpy(), ro, s_out.cpu().numpy(), rf, x.cu_seqlens)


@pytest.mark.parametrize("seed", range(32))
def test_slots_random_batch(seed):
    """R requests of 0..M tokens (M up to 20: two staging blocks) over a pool
    whose read and write slots are a random permutation of its slots, some
    writes skipped (-1), the incoming column given by random device-side
    accepted counts or column 0, fp32 or fp16 storage."""
    rng = np.random.default_rng(9000 + seed)
    hqk, hv = HEADS[seed % len(HEADS)]
    R, M = int(rng.integers(1, 11)), int(rng.integers(1, 21))
    lengths = [int(rng.integers(0, M + 1)) for _ in range(R)]
    if sum(lengths) == 0:
        lengths[0] = 1
    f16 = bool(rng.random() < 0.5)
    x = gi.make_inputs(lengths, hqk, hv, 128, 128, seed=9000 + seed, state_std=0.02,
                       g_mean=float(rng.choice([0.0, -2.0])), name=f"sweep_slots{seed}")
    P = R * (M + 1) + int(rng.integers(0, 8))
    pool = gi.state_pool(x, P - R, f16=f16, seed=9000 + seed)
    table = rng.permutation(P)[:R * (M + 1)].reshape(R, M + 1).astype(np.int32)
    table[:, 1:][rng.random((R, M)) < 0.15] = -1
    acc = None
    if rng.random() < 0.7:
        acc = rng.integers(0, M + 1, size=R).astype(np.int32)
        acc[table[np.arange(R), acc] < 0] = 0       # the incoming column names a slot
    print(f"[case] sweep slots {seed}: heads {hqk}/{hv} lengths {lengths} M={M} P={P} "
          f"f16={f16} accepted={acc}", flush=True)
    out, gpool = run_slots(x, pool, table, acc)
    ro, rpool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool, table, acc)
    assert np.isfinite(out).all()
    e = rel_l2(out, ro)
    print(f"[result] sweep slots {seed}: out {e:.3e}", flush=True)
    assert e <= OUT_TOL
    written = set()
    for r in range(R):
        written.update(int(t) for t in table[r, 1:1 + lengths[r]] if t >= 0)
    check_pool(gpool, rpool, pool, written)


@pytest.mark.parametrize("seed", range(24))
def test_segmented_random_batch(seed):
    """gdn_chunk_fwd_segmented on a random batch with a random segment length
    (1 chunk up to one segment per sequence)."""
    x, desc = _draw(200 + seed)
    sc = int(np.random.default_rng(7500 + seed).choice([1, 2, 3, 5, 8, 16, 64]))
    print(f"[case] sweep segmented {seed}: sc={sc} {desc}", flush=True)
    out, fin = _segmented(x, DevInputs(x), sc)
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o, f = out.cpu().numpy(), fin.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(f).all()
    eo, ef = rel_l2(o, ro), rel_l2(f, rf)
    print(f"[result] sweep segmented {seed}: out {eo:.3e} state {ef:.3e}", flush=True)
    assert eo <= OUT_TOL and ef <= STATE_TOL
    check_detail(f"sweep_seg{seed}", o, ro, f, rf, x.cu_seqlens)


@pytest.mark.parametrize("seed", range(16))
def test_snapshots_random_batch(seed):
    """gdn_chunk_fwd_snapshots on a random batch (at most six value heads and
    six sequences, so that the oracle's per-token states fit in host memory):
    every chunk's state against the oracle's state after the same token, the
    last one equal to the final state bit for bit, every slot no chunk maps
    to left untouched."""
    x, desc = _draw(300 + seed, heads=[(1, 1), (2, 4), (1, 3), (2, 6)], max_seqs=6, max_len=300)
    print(f"[case] sweep snapshots {seed}: {desc}", flush=True)
    out, fin, cs = _snapshots(x, DevInputs(x))
    _, _, rs = oracle.forward_inputs(x, precision="f64", record_states=True)
    cs_np, fin_np = cs.cpu().numpy(), fin.cpu().numpy()
    written = set()
    for n, L in enumerate(x.lengths):
        start, L = int(x.cu_seqlens[n]), int(L)
        nch = (L + 63) // 64
        for c in range(nch):
            slot = n + start // 64 + c
            t_end = start + min(64 * (c + 1), L) - 1
            assert rel_l2(cs_np[slot], rs[t_end]) <= STATE_TOL, (n, c)
            written.add(slot)
        if nch:
            np.testing.assert_array_equal(cs_np[n + start // 64 + nch - 1], fin_np[n])
    for slot in range(cs_np.shape[0]):
        if slot not in written:
            assert np.isnan(cs_np[slot]).all(), slot
