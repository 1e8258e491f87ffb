"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances: relative L2 <= 2e-3 on outputs and <= 1e-3 on states (final and
per-token snapshots), with bf16 q, k, v shared by both sides.  The oracle runs
in fp64 on the same bf16-rounded inputs.
"""

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import (OUT_TOL, STATE_TOL, DevInputs, check_detail, chunk_fwd,  # noqa: E402
                      recurrent_step, rel_l2)


def _print_case(name, x):
    print(f"[case] {name}: N={x.n_seqs} T={x.total_tokens} Hqk={x.h_qk} Hv={x.h_v} "
          f"lengths={list(map(int, x.lengths))[:12]}", flush=True)


def check_chunk(x, name, poison=True, **kw):
    _print_case(name, x)
    d = DevInputs(x)
    out, fin = chunk_fwd(d, poison=poison, **kw)
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o, f = out.cpu().numpy(), fin.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(f).all()
    eo, ef = rel_l2(o, ro), rel_l2(f, rf)
    print(f"[result] {name}: out rel-L2 {eo:.3e}  state rel-L2 {ef:.3e}", flush=True)
    assert eo <= OUT_TOL, eo
    assert ef <= STATE_TOL, ef
    check_detail(name, o, ro, f, rf, x.cu_seqlens)
    return out, fin


# ------------------------------------------------------------ recurrent step

def test_verify_8req_6tok_with_snapshots():
    x = gi.verify_8x6()
    _print_case("verify_8x6", x)
    d = DevInputs(x)
    out, s_out, inter = recurrent_step(d, 8, 6, save=True)
    ro, rf, rs = oracle.forward_inputs(x, precision="f64", record_states=True)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(s_out.cpu().numpy(), rf) <= STATE_TOL
    snaps = inter.cpu().numpy().reshape(48, x.h_v, 128, 128)
    assert rel_l2(snaps, rs) <= STATE_TOL
    # every rollback slot individually
    for t in range(48):
        assert rel_l2(snaps[t], rs[t]) <= STATE_TOL
    # the last snapshot of each request is its final state, bitwise
    np.testing.assert_array_equal(inter[:, -1].cpu().numpy(), s_out.cpu().numpy())
    check_detail("verify_8x6", out.cpu().numpy(), ro, s_out.cpu().numpy(), rf, x.cu_seqlens)


def test_decode_single_token_in_place():
    x = gi.make_inputs([1] * 16, 16, 32, 128, 128, seed=5, state_std=0.02)
    d = DevInputs(x)
    s_ref = d.s0.clone()
    out = torch.empty((16, 32, 128), dtype=torch.float32, device="cuda")
    import hybrid_linear_attention_gdn_amd as gdn
    gdn.gdn_recurrent_step(d.q, d.k, d.v, d.g, d.beta, 16, 1, d.s0, d.s0, out, None, False)
    torch.cuda.synchronize()
    ro, rf, _ = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, s_ref.cpu().numpy())
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(d.s0.cpu().numpy(), rf) <= STATE_TOL


@pytest.mark.parametrize("hqk,hv", [(1, 1), (2, 8), (4, 4)])
def test_recurrent_step_head_groupings(hqk, hv):
    x = gi.make_inputs([4] * 3, hqk, hv, 128, 128, seed=8, state_std=0.02)
    d = DevInputs(x)
    out, s_out, inter = recurrent_step(d, 3, 4, save=True)
    ro, rf, rs = oracle.forward_inputs(x, record_states=True)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(s_out.cpu().numpy(), rf) <= STATE_TOL
    assert rel_l2(inter.cpu().numpy().reshape(rs.shape), rs) <= STATE_TOL


# ------------------------------------------------------------ chunked prefill

@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 128, 200, 257])
def test_chunk_small_lengths(T):
    x = gi.make_inputs([T], 2, 4, 128, 128, seed=T, state_std=0.02)
    check_chunk(x, f"small_T{T}")


@pytest.mark.parametrize("hqk,hv", [(1, 1), (1, 4), (3, 6), (2, 6)])
def test_chunk_head_groupings(hqk, hv):
    x = gi.make_inputs([150, 64, 3], hqk, hv, 128, 128, seed=hv, state_std=0.02)
    check_chunk(x, f"groups_{hqk}x{hv}")


def test_chunk_many_short_sequences_eight_heads_per_qk_head():
    """40 sequences of 1..200 tokens at 16 value / 2 q-k heads: 640 (sequence,
    head) units, more than one XCD round of the state kernel's unit map, odd
    chunk counts, and eight value heads sharing one q/k head's K^T and Q."""
    rng = np.random.default_rng(91)
    lengths = [int(n) for n in rng.integers(1, 201, size=40)]
    x = gi.make_inputs(lengths, 2, 16, 128, 128, seed=91, state_std=0.02)
    check_chunk(x, "many_short_group8")


def test_chunk_prefill_4000():
    x = gi.prefill_4000()
    out, fin = check_chunk(x, "prefill_4000")
    # NULL initial state and an explicit zero state give identical bits
    d = DevInputs(x)
    zeros = torch.zeros((1, 32, 128, 128), dtype=torch.float32, device="cuda")
    out2, fin2 = chunk_fwd(d, initial_state=zeros)
    assert torch.equal(out, out2) and torch.equal(fin, fin2)


def test_chunk_varlen_8():
    x = gi.varlen_8()
    check_chunk(x, "varlen_8")


def test_chunk_slow_decay():
    check_chunk(gi.slow_decay(4000), "slow_decay_T4000")


def test_chunk_no_decay_small_beta():
    check_chunk(gi.no_decay_small_beta(4000), "no_decay_T4000")


def test_chunk_strong_decay_and_extreme_beta():
    """g = -softplus(N(4, 1)) (chunk log-decays near -260, so most cross-position
    factors underflow to zero in fp32), with beta forced to 0 or 1 on a third of
    the tokens each: nothing may turn into inf or NaN, and the gate holds."""
    x = gi.make_inputs([700, 130], 4, 8, 128, 128, seed=17, g_mean=4.0, state_std=0.02)
    rb = np.random.default_rng(170)
    pick = rb.integers(0, 3, size=x.beta.shape)
    x.beta[pick == 0] = 0.0
    x.beta[pick == 1] = 1.0
    check_chunk(x, "strong_decay_extreme_beta")


def test_chunk_k_scaled_reading():
    """The alternative input reading (k also scaled by 1/sqrt(d_k)) passes the same gate."""
    x = gi.make_inputs([1000, 300], 16, 32, 128, 128, seed=4, state_std=0.02, k_scale=True)
    check_chunk(x, "k_scaled")


def test_chunk_zero_length_sequences():
    x = gi.make_inputs([0, 70, 0, 5, 0], 2, 4, 128, 128, seed=12, state_std=0.02)
    out, fin = check_chunk(x, "zero_length")
    f = fin.cpu().numpy()
    for n in (0, 2, 4):
        np.testing.assert_array_equal(f[n], x.initial_state[n])


def test_chunk_all_sequences_empty():
    x = gi.make_inputs([0, 0], 2, 4, 128, 128, seed=1, state_std=0.02)
    d = DevInputs(x)
    import hybrid_linear_attention_gdn_amd as gdn
    fin = torch.full((2, 4, 128, 128), float("nan"), device="cuda")
    out = torch.empty((0, 4, 128), device="cuda")
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(2, 0, 2, 4), dtype=torch.uint8, device="cuda")
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out, fin, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fin.cpu().numpy(), x.initial_state)


def test_chunk_packed_equals_separate_bitwise():
    x = gi.make_inputs([130, 64, 1, 700], 16, 32, 128, 128, seed=21, state_std=0.02)
    out, fin = chunk_fwd(DevInputs(x))
    for n in range(x.n_seqs):
        y = x.slice_seq(n)
        o, f = chunk_fwd(DevInputs(y))
        a, b = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        assert torch.equal(out[a:b], o)
        assert torch.equal(fin[n:n + 1], f)


def test_chunk_deterministic():
    x = gi.make_inputs([1000, 77], 16, 32, 128, 128, seed=3, state_std=0.02)
    d = DevInputs(x)
    o1, f1 = chunk_fwd(d)
    o2, f2 = chunk_fwd(d, poison=True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_chunk_final_state_may_alias_initial():
    x = gi.make_inputs([333, 65], 2, 4, 128, 128, seed=6, state_std=0.02)
    d = DevInputs(x)
    ref_out, ref_fin = chunk_fwd(d)
    import hybrid_linear_attention_gdn_amd as gdn
    from gpu_util import workspace_for
    s = d.s0.clone()
    out = torch.empty_like(ref_out)
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, s, out, s, workspace_for(x))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(s, ref_fin)


def test_chunk_without_final_state():
    x = gi.make_inputs([100], 2, 4, 128, 128, seed=9, state_std=0.02)
    d = DevInputs(x)
    ref_out, _ = chunk_fwd(d)
    out, fin = chunk_fwd(d, want_final=False)
    assert fin is None and torch.equal(out, ref_out)


def test_chunk_writes_stay_in_bounds():
    """Guard bands around out and final_state stay untouched (NaN-free, bit pattern kept)."""
    x = gi.make_inputs([190, 3], 2, 4, 128, 128, seed=2, state_std=0.02)
    d = DevInputs(x)
    import hybrid_linear_attention_gdn_amd as gdn
    from gpu_util import workspace_for
    G = 4096
    out_buf = torch.full((G + x.total_tokens * 4 * 128 + G,), 7.0, device="cuda")
    fin_buf = torch.full((G + 2 * 4 * 128 * 128 + G,), 7.0, device="cuda")
    out = out_buf[G:G + x.total_tokens * 4 * 128].view(x.total_tokens, 4, 128)
    fin = fin_buf[G:G + 2 * 4 * 128 * 128].view(2, 4, 128, 128)
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out, fin, workspace_for(x))
    torch.cuda.synchronize()
    for buf, n in ((out_buf, out.numel()), (fin_buf, fin.numel())):
        assert torch.all(buf[:G] == 7.0) and torch.all(buf[G + n:] == 7.0)
    ro, rf, _ = oracle.forward_inputs(x)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(fin.cpu().numpy(), rf) <= STATE_TOL


def test_recurrent_chain_matches_chunked():
    """Two independent GPU paths agree on short sequences."""
    x = gi.make_inputs([256], 16, 32, 128, 128, seed=14, state_std=0.02)
    d = DevInputs(x)
    co, cf = chunk_fwd(d)
    ro, rf, _ = recurrent_step(d, 1, 256, save=False)
    assert rel_l2(co.cpu().numpy(), ro.cpu().numpy()) <= OUT_TOL
    assert rel_l2(cf.cpu().numpy(), rf.cpu().numpy()) <= STATE_TOL


@pytest.fixture(scope="module")
def long_ref():
    """The fp64 oracle over the whole long-context workload, all 32 value heads,
    run 8 q/k heads (16 value heads) at a time to bound host memory; kept as
    fp32 (rounding adds ~3e-8 relative, far below the gates)."""
    x = gi.long_131072()
    T, hv = x.total_tokens, x.h_v
    ro = np.empty((T, hv, x.d_v), np.float32)
    rf = np.empty((1, hv, x.d_k, x.d_v), np.float32)
    grp = hv // x.h_qk
    step = 8
    for j0 in range(0, x.h_qk, step):
        js = slice(j0, j0 + step)
        hs = slice(j0 * grp, (j0 + step) * grp)
        o, f, _ = oracle.forward(x.q[:, js], x.k[:, js], x.v[:, hs], x.g[:, hs], x.beta[:, hs],
                                 x.cu_seqlens, None, precision="f64", n_threads=16)
        ro[:, hs] = o
        rf[:, hs] = f
        print(f"[oracle] long_131072 q/k heads {j0}..{j0 + step - 1} done", flush=True)
        del o, f
    return x, ro, rf


def _check_long(name, out, fin, x, ro, rf):
    o = out.cpu().numpy()
    f = fin.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(f).all()
    eo, ef = rel_l2(o, ro), rel_l2(f, rf)
    print(f"[result] {name} all heads: out {eo:.3e} state {ef:.3e}", flush=True)
    assert eo <= OUT_TOL and ef <= STATE_TOL
    check_detail(name, o, ro, f, rf, x.cu_seqlens)
    return o, f


def test_long_context_131072_all_heads(long_ref):
    """Full-size long-context prefill: every value head's output over all
    131072 tokens and every final state against the oracle."""
    x, ro, rf = long_ref
    _print_case("long_131072", x)
    out, fin = chunk_fwd(DevInputs(x))
    _check_long("long_131072", out, fin, x, ro, rf)


# ------------------------------------------------------------ state snapshots at chunk boundaries

def _snapshots(x, d, poison=True):
    import hybrid_linear_attention_gdn_amd as gdn
    from gpu_util import workspace_for
    n_slots = gdn.gdn_chunk_state_slots(x.n_seqs, x.total_tokens, x.h_qk, x.h_v)
    cs = torch.full((n_slots, x.h_v, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.empty((x.total_tokens, x.h_v, x.d_v), dtype=torch.float32, device="cuda")
    fin = torch.empty((x.n_seqs, x.h_v, 128, 128), dtype=torch.float32, device="cuda")
    ws = workspace_for(x)
    if poison:
        ws.fill_(0xFF)
    gdn.gdn_chunk_fwd_snapshots(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out, fin, cs, ws)
    torch.cuda.synchronize()
    return out, fin, cs


def test_chunk_snapshots_varlen():
    """State after every chunk of every sequence, in slot n + cu[n] // 64 + c;
    slots no chunk maps to stay untouched; outputs and final states are those
    of gdn_chunk_fwd, bit for bit."""
    lengths = [200, 64, 1, 130, 0, 65]
    x = gi.make_inputs(lengths, 2, 4, 128, 128, seed=77, state_std=0.02)
    _print_case("snapshots_varlen", x)
    d = DevInputs(x)
    out, fin, cs = _snapshots(x, d)
    _, _, rs = oracle.forward_inputs(x, precision="f64", record_states=True)
    cs_np, fin_np = cs.cpu().numpy(), fin.cpu().numpy()
    written = set()
    for n, L in enumerate(lengths):
        start = int(x.cu_seqlens[n])
        nch = (L + 63) // 64
        for c in range(nch):
            slot = n + start // 64 + c
            t_end = start + min(64 * (c + 1), L) - 1
            e = rel_l2(cs_np[slot], rs[t_end])
            assert e <= STATE_TOL, (n, c, e)
            assert slot not in written
            written.add(slot)
        if nch:
            np.testing.assert_array_equal(cs_np[n + start // 64 + nch - 1], fin_np[n])
    for slot in range(cs_np.shape[0]):
        if slot not in written:
            assert np.isnan(cs_np[slot]).all(), slot
    out2, fin2 = chunk_fwd(d)
    np.testing.assert_array_equal(out.cpu().numpy(), out2.cpu().numpy())
    np.testing.assert_array_equal(fin_np, fin2.cpu().numpy())


def test_chunk_snapshots_prefill_4000_sampled():
    """Full-size prefill with snapshots: sampled chunk boundaries against the
    oracle's state after the same prefix."""
    x = gi.prefill_4000()
    _print_case("snapshots_prefill_4000", x)
    d = DevInputs(x)
    out, fin, cs = _snapshots(x, d, poison=False)
    cs_np = cs.cpu().numpy()
    assert cs_np.shape[0] == 64 and np.isnan(cs_np[63]).all()
    for c in (0, 1, 30, 62):
        t = min(64 * (c + 1), 4000)
        _, rf, _ = oracle.forward(x.q[:t], x.k[:t], x.v[:t], x.g[:t], x.beta[:t], np.array([0, t], np.int32))
        e = rel_l2(cs_np[c], rf[0])
        print(f"[result] snapshot chunk {c}: state rel-L2 {e:.3e}", flush=True)
        assert e <= STATE_TOL
    np.testing.assert_array_equal(cs_np[62], fin.cpu().numpy()[0])


# ------------------------------------------------------------ segment-parallel recurrence (affine scan)

def _segmented(x, d, sc, initial_state="default"):
    import hybrid_linear_attention_gdn_amd as gdn
    s0 = d.s0 if isinstance(initial_state, str) else initial_state
    nbytes = gdn.gdn_chunk_fwd_segmented_workspace_size(x.n_seqs, x.total_tokens, x.h_qk, x.h_v, sc)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")     # fp16 / fp32 NaN poison
    out = torch.full((x.total_tokens, x.h_v, x.d_v), float("nan"), dtype=torch.float32, device="cuda")
    fin = torch.full((x.n_seqs, x.h_v, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_chunk_fwd_segmented(d.q, d.k, d.v, d.g, d.beta, d.cu, s0, out, fin, sc, ws)
    torch.cuda.synchronize()
    return out, fin


@pytest.mark.parametrize("sc", [1, 3, 4, 16, 1000])
def test_segmented_varlen(sc):
    """Segments of sc chunks (1 = every chunk its own segment; 1000 = one
    segment) over a ragged batch with an empty sequence and random states."""
    lengths = [300, 1, 700, 64, 0, 200]
    x = gi.make_inputs(lengths, 2, 4, 128, 128, seed=90 + sc, state_std=0.02)
    _print_case(f"segmented_varlen_sc{sc}", x)
    d = DevInputs(x)
    out, fin = _segmented(x, d, sc)
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o, f = out.cpu().numpy(), fin.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(f).all()
    eo, ef = rel_l2(o, ro), rel_l2(f, rf)
    print(f"[result] segmented sc={sc}: out {eo:.3e} state {ef:.3e}", flush=True)
    assert eo <= OUT_TOL and ef <= STATE_TOL
    # the empty sequence keeps its initial state exactly
    np.testing.assert_array_equal(f[4], x.initial_state[4])


def test_segmented_prefill_4000():
    x = gi.prefill_4000()
    _print_case("segmented_prefill_4000", x)
    d = DevInputs(x)
    out, fin = _segmented(x, d, 8)
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    eo, ef = rel_l2(out.cpu().numpy(), ro), rel_l2(fin.cpu().numpy(), rf)
    print(f"[result] segmented prefill_4000 sc=8: out {eo:.3e} state {ef:.3e}", flush=True)
    assert eo <= OUT_TOL and ef <= STATE_TOL


def test_segmented_long_131072_all_heads(long_ref):
    """Full-size long context, 8 segments of 256 chunks: every value head's
    output over the whole sequence and every final state against the oracle,
    and the whole output against the serial GPU path."""
    x, ro, rf = long_ref
    _print_case("segmented_long_131072", x)
    d = DevInputs(x)
    out, fin = _segmented(x, d, 256)
    o, f = _check_long("segmented_long_131072", out, fin, x, ro, rf)
    del out, fin
    so, sf = chunk_fwd(d, poison=False)
    assert rel_l2(o, so.cpu().numpy()) <= OUT_TOL
    assert rel_l2(f, sf.cpu().numpy()) <= STATE_TOL


def test_batch_with_more_tiles_than_cus_matches_separate_runs_bitwise():
    """Nine sequences at 32 value heads are 2304 column tiles, more than the
    CUs, so the state kernel runs them as tile pairs (two chain waves sharing
    one copy ring); one sequence alone is 256 tiles and runs one tile per
    workgroup.  The arithmetic per tile is the same either way: every output
    row and final state of the batch equals the separate run's bit for bit,
    and the batch matches the oracle."""
    lengths = [300, 1, 129, 64, 700, 0, 65, 200, 33]
    x = gi.make_inputs(lengths, 16, 32, 128, 128, seed=23, state_std=0.02)
    out, fin = check_chunk(x, "batch_tile_pairs")
    out, fin = out.cpu(), fin.cpu()
    for n in range(len(lengths)):
        xs = x.slice_seq(n)
        _print_case(f"batch_tile_pairs[{n}] alone", xs)
        o1, f1 = chunk_fwd(DevInputs(xs), poison=True)
        a, b = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        assert torch.equal(o1.cpu(), out[a:b]), n
        assert torch.equal(f1.cpu()[0], fin[n]), n


def test_streaming_prep_matches_ordinary_prep_bitwise():
    """Prep writes its intermediates with non-temporal stores once they exceed
    160 MiB, and with ordinary stores below.  The store kind changes no value:
    the eight-sequence varlen batch (~0.5 GB of intermediates, streaming prep)
    equals each of its sequences run alone (at most ~0.11 GB, ordinary prep)
    bit for bit, outputs and final states."""
    import hybrid_linear_attention_gdn_amd as gdn
    x = gi.varlen_8()
    big = gdn.gdn_chunk_fwd_workspace_size(x.n_seqs, x.total_tokens, x.h_qk, x.h_v)
    assert big > 170 << 20, big
    _print_case("varlen_8 streaming prep", x)
    out, fin = chunk_fwd(DevInputs(x), poison=True)
    out, fin = out.cpu(), fin.cpu()
    for n in range(x.n_seqs):
        xs = x.slice_seq(n)
        small = gdn.gdn_chunk_fwd_workspace_size(1, xs.total_tokens, xs.h_qk, xs.h_v)
        assert small < 150 << 20, small
        _print_case(f"varlen_8[{n}] alone, ordinary prep", xs)
        o1, f1 = chunk_fwd(DevInputs(xs), poison=True)
        a, b = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        assert torch.equal(o1.cpu(), out[a:b]), n
        assert torch.equal(f1.cpu()[0], fin[n]), n


@pytest.mark.parametrize("hqk,hv,T,init,final", [
    (16, 32, 12037, True, True),      # 189 chunks: ranges of 64, 64, 61 (two value heads per prep workgroup)
    (16, 32, 12288, True, True),      # 192 chunks: three full ranges
    (16, 32, 12289, True, True),      # 193 chunks: the last range is one chunk of one token
    (16, 32, 12037, False, False),    # zero initial state; no final state wanted (the carry still runs)
    (8, 16, 24000, True, True),       # ranges of 128 chunks
    (2, 6, 76013, True, True),        # three value heads per q/k head: one per prep workgroup, ranges of 168
])
def test_long_sequence_ranges_match_single_pass_bitwise(hqk, hv, T, init, final):
    """One sequence whose intermediates exceed 160 MiB runs range by range
    (prep of a range of chunk slots, then the recurrence over them, the state
    carried in fp32 from range to range), in a workspace of one range's
    size, which the single pass would refuse; the stage-by-stage call runs
    the single pass (streaming prep over all slots, then one recurrence) in
    the full workspace.  The arithmetic is the same: outputs and final states
    equal bit for bit."""
    import hybrid_linear_attention_gdn_amd as gdn
    from gpu_util import workspace_for
    x = gi.make_inputs([T], hqk, hv, 128, 128, seed=41, state_std=0.02 if init else None)
    _print_case(f"ranges vs single pass H_qk={hqk} H_v={hv} T={T}", x)
    d = DevInputs(x)
    small = gdn.gdn_chunk_fwd_min_workspace_size(1, T, hqk, hv)
    assert small < gdn.gdn_chunk_fwd_workspace_size(1, T, hqk, hv)
    ws_r = torch.full((small,), 0xFF, dtype=torch.uint8, device="cuda")
    out_r = torch.full((T, hv, 128), float("nan"), device="cuda")
    fin_r = torch.full((1, hv, 128, 128), float("nan"), device="cuda") if final else None
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out_r, fin_r, ws_r)
    torch.cuda.synchronize()
    ws = workspace_for(x)
    ws.fill_(0xFF)
    out_s = torch.full((T, hv, 128), float("nan"), device="cuda")
    fin_s = torch.full((1, hv, 128, 128), float("nan"), device="cuda") if final else None
    gdn.gdn_chunk_fwd_stages(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out_s, fin_s, ws, 1)
    gdn.gdn_chunk_fwd_stages(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out_s, fin_s, ws, 2)
    torch.cuda.synchronize()
    assert torch.isfinite(out_r).all()
    assert torch.equal(out_r, out_s)
    if final:
        assert torch.isfinite(fin_r).all()
        assert torch.equal(fin_r, fin_s)
    # and the oracle over the whole sequence
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o = out_r.cpu().numpy()
    assert rel_l2(o, ro) <= OUT_TOL
    if final:
        assert rel_l2(fin_r.cpu().numpy(), rf) <= STATE_TOL


def test_long_sequence_ranges_final_state_may_alias_initial():
    """Range by range, the initial state is read by the first range's
    launch only and the final state written by the last one's, so an
    in-place update (final_state aliasing initial_state) gives the same bits
    as separate buffers."""
    import hybrid_linear_attention_gdn_amd as gdn
    from gpu_util import workspace_for
    x = gi.make_inputs([12037], 16, 32, 128, 128, seed=47, state_std=0.02)
    _print_case("ranges, final state aliasing the initial state", x)
    d = DevInputs(x)
    ws = workspace_for(x)
    out1 = torch.empty((x.total_tokens, 32, 128), device="cuda")
    fin1 = torch.empty((1, 32, 128, 128), device="cuda")
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out1, fin1, ws)
    s = d.s0.clone()
    out2 = torch.empty_like(out1)
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, s, out2, s, ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(fin1, s)


def test_segmented_tile_pairs_match_single_tiles_bitwise():
    """At 32 value heads in segments of 8 chunks, the map and segment passes
    have more tiles than CUs and run as tile pairs; one head alone runs them
    one tile per workgroup.  Heads are independent and the arithmetic per tile
    is the same: each head's output rows and final states in the batch equal
    the one-head run's bit for bit."""
    import dataclasses
    lengths = [3000, 1700]
    x = gi.make_inputs(lengths, 16, 32, 128, 128, seed=31, state_std=0.02)
    _print_case("segmented sc=8, tile pairs", x)
    out, fin = _segmented(x, DevInputs(x), 8)
    out, fin = out.cpu(), fin.cpu()
    assert torch.isfinite(out).all() and torch.isfinite(fin).all()
    for h in (0, 1, 17, 31):
        j = h // 2
        xh = dataclasses.replace(
            x, name=f"{x.name}_head{h}", q=x.q[:, j:j + 1].copy(), k=x.k[:, j:j + 1].copy(),
            v=x.v[:, h:h + 1].copy(), g=x.g[:, h:h + 1].copy(), beta=x.beta[:, h:h + 1].copy(),
            initial_state=x.initial_state[:, h:h + 1].copy())
        _print_case(f"segmented sc=8, head {h} alone", xh)
        oh, fh = _segmented(xh, DevInputs(xh), 8)
        assert torch.equal(oh.cpu()[:, 0], out[:, h]), h
        assert torch.equal(fh.cpu()[:, 0], fin[:, h]), h
