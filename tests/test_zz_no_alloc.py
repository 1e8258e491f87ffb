"""gdn_chunk_fwd_noalloc through the C ABI: the prefill with the library's
fixed per-GPU scratch as its workspace gives the results of gdn_chunk_fwd
with a caller workspace, bit for bit (same kernels, same workspace layout),
on two calls in a row, the second on a smaller batch, so that whatever the
first call left in the scratch cannot leak into the second; both also match
the oracle.  One long sequence runs range by range inside the scratch.
Batches beyond the scratch are refused."""

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import hybrid_linear_attention_gdn_amd as gdn  # noqa: E402
from gpu_util import OUT_TOL, STATE_TOL, DevInputs, chunk_fwd, rel_l2  # noqa: E402


def _noalloc(d, s0, final=True):
    x = d.x
    out = torch.full((x.total_tokens, x.h_v, 128), float("nan"), device="cuda")
    fin = torch.full((x.n_seqs, x.h_v, 128, 128), float("nan"), device="cuda") if final else None
    print(f"[case] noalloc N={x.n_seqs} T={x.total_tokens} Hv={x.h_v} lengths={list(map(int, x.lengths))}",
          flush=True)
    gdn.gdn_chunk_fwd_noalloc(d.q, d.k, d.v, d.g, d.beta, d.cu, s0, out, fin)
    torch.cuda.synchronize()
    return out, fin


def test_noalloc_matches_workspace_prefill_on_two_calls():
    big = gi.prefill_4000()
    small = gi.make_inputs([700, 1, 64, 0, 130], 16, 32, 128, 128, seed=5, state_std=0.02)
    for x in (big, small):
        d = DevInputs(x)
        o1, f1 = _noalloc(d, d.s0)
        o2, f2 = chunk_fwd(d, poison=True)
        assert torch.equal(o1, o2) and torch.equal(f1, f2)
        ro, rf, _ = oracle.forward_inputs(x, precision="f64")
        eo, ef = rel_l2(o1.cpu().numpy(), ro), rel_l2(f1.cpu().numpy(), rf)
        print(f"[result] noalloc {x.name}: out {eo:.3e} state {ef:.3e}", flush=True)
        assert eo <= OUT_TOL and ef <= STATE_TOL


def test_noalloc_in_place_state_and_rejects_oversized_batches():
    x = gi.make_inputs([333, 65], 2, 4, 128, 128, seed=6, state_std=0.02)
    d = DevInputs(x)
    ref_out, ref_fin = chunk_fwd(d)
    s = d.s0.clone()
    out = torch.empty_like(ref_out)
    gdn.gdn_chunk_fwd_noalloc(d.q, d.k, d.v, d.g, d.beta, d.cu, s, out, s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(s, ref_fin)
    y = gi.make_inputs([9400], 16, 32, 128, 128, seed=1)
    dy = DevInputs(y)
    yo = torch.full((9400, 32, 128), 7.0, device="cuda")
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_chunk_fwd_noalloc(dy.q, dy.k, dy.v, dy.g, dy.beta, dy.cu, None, yo, None)
    assert ei.value.status == gdn.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(yo == 7.0))


def test_noalloc_runs_one_long_sequence_range_by_range():
    """One sequence of 12037 tokens has 173 MB of intermediates, more than the
    scratch, but gdn_chunk_fwd runs it range by range in a workspace of one
    range (62 MB), which the scratch holds: the no-allocation call gives the
    bits of gdn_chunk_fwd with a full caller workspace, then a small batch
    after it still matches."""
    x = gi.make_inputs([12037], 16, 32, 128, 128, seed=9, state_std=0.02)
    assert gdn.gdn_chunk_fwd_workspace_size(1, 12037, 16, 32) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    assert gdn.gdn_chunk_fwd_min_workspace_size(1, 12037, 16, 32) <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    d = DevInputs(x)
    o1, f1 = _noalloc(d, d.s0)
    o2, f2 = chunk_fwd(d, poison=True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    y = gi.make_inputs([300, 65], 16, 32, 128, 128, seed=10, state_std=0.02)
    dy = DevInputs(y)
    o3, f3 = _noalloc(dy, dy.s0)
    o4, f4 = chunk_fwd(dy, poison=True)
    assert torch.equal(o3, o4) and torch.equal(f3, f4)
