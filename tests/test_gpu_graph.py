"""The entry points inside HIP graphs.

They allocate nothing and launch only on the caller's stream, so a serving
loop can capture them once and replay them.  Each test captures a call with
torch's graph capture, replays it several times with eager work and
synchronisations in between (buffers refilled with NaN, eager calls of the
same entry point), and checks every replay bit for bit against the eager
result.
"""

import numpy as np
import pytest

import gdn_inputs as gi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import hybrid_linear_attention_gdn_amd as gdn  # noqa: E402
from gpu_util import DevInputs, workspace_for  # noqa: E402


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_verify_step_graph_replays_match_eager():
    y = gi.verify_8x6()
    d = DevInputs(y)
    R, n_tok, hv = 8, 6, y.h_v
    print(f"[case] graph verify {R}x{n_tok}", flush=True)

    def buffers():
        return (torch.empty((R * n_tok, hv, 128), device="cuda"),
                torch.empty((R, n_tok, hv, 128, 128), device="cuda"))

    out_e, inter_e = buffers()
    gdn.gdn_recurrent_step(d.q, d.k, d.v, d.g, d.beta, R, n_tok, d.s0, None, out_e, inter_e, True)
    torch.cuda.synchronize()

    out_g, inter_g = buffers()
    g = _capture(lambda: gdn.gdn_recurrent_step(d.q, d.k, d.v, d.g, d.beta, R, n_tok, d.s0, None,
                                                out_g, inter_g, True))
    out_x, inter_x = buffers()
    for rep in range(3):
        out_g.fill_(float("nan"))
        inter_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(inter_g, inter_e), rep
        # eager work of the program between replays
        gdn.gdn_recurrent_step(d.q, d.k, d.v, d.g, d.beta, R, n_tok, d.s0, None, out_x, inter_x, True)
        torch.cuda.synchronize()
        assert torch.equal(out_x, out_e), rep


def test_in_place_decode_graph_replays_match_eager():
    y = gi.verify_8x6()
    d = DevInputs(y)
    R, hv = 8, y.h_v
    print(f"[case] graph decode {R}x1 in place", flush=True)
    pick = slice(None, None, 6)      # the first token of each request
    q, k, v = (t[pick].contiguous() for t in (d.q, d.k, d.v))
    gg, bb = d.g[pick].contiguous(), d.beta[pick].contiguous()

    st_e = d.s0.clone()
    st_g = d.s0.clone()
    out_e = torch.empty((R, hv, 128), device="cuda")
    out_g = torch.empty((R, hv, 128), device="cuda")
    g = _capture(lambda: gdn.gdn_recurrent_step(q, k, v, gg, bb, R, 1, st_g, st_g, out_g, None, False))
    # the warm-up call advanced the state once (the capture itself runs
    # nothing): start the graph's state where the eager one starts
    st_g.copy_(d.s0)
    torch.cuda.synchronize()
    for rep in range(4):
        gdn.gdn_recurrent_step(q, k, v, gg, bb, R, 1, st_e, st_e, out_e, None, False)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(st_g, st_e), rep


@pytest.mark.parametrize("case", ["prefill_4000", "ranges_12037"])
def test_prefill_graph_replays_match_eager(case):
    """The T = 4000 prefill (two launches), and one 12037-token sequence with
    an initial state, whose 173 MB of intermediates make gdn_chunk_fwd run
    it range by range (three ranges: six launches and the carried state)."""
    x = (gi.prefill_4000() if case == "prefill_4000"
         else gi.make_inputs([12037], 16, 32, 128, 128, seed=43, state_std=0.02))
    d = DevInputs(x)
    print(f"[case] graph prefill {case} T={x.total_tokens}", flush=True)
    shape_o = (x.total_tokens, x.h_v, 128)
    shape_f = (x.n_seqs, x.h_v, 128, 128)
    ws = workspace_for(x)
    out_e, fin_e = torch.empty(shape_o, device="cuda"), torch.empty(shape_f, device="cuda")
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out_e, fin_e, ws)
    torch.cuda.synchronize()

    out_g, fin_g = torch.empty(shape_o, device="cuda"), torch.empty(shape_f, device="cuda")
    ws_g = workspace_for(x)
    g = _capture(lambda: gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out_g, fin_g, ws_g))
    for rep in range(3):
        out_g.fill_(float("nan"))
        fin_g.fill_(float("nan"))
        ws_g.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(fin_g, fin_e), rep
        # eager work between replays, on the same workspace the graph uses
        gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out_e, fin_e, ws_g)
        torch.cuda.synchronize()
    assert np.isfinite(out_g.cpu().numpy()).all()
