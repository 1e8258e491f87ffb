"""GPU checks beyond end-to-end parity, through the C ABI:

* the segment-parallel prefill with final_state aliasing initial_state;
* inputs scaled toward the fp16 operand range (v and states x 1024);
* guard bands around every output of the recurrent step, the slot pool and
  the chunk-boundary snapshots (nothing written outside its tensor);
* the prepared (checked-once) step calls against the plain ones, bit for bit;
* the intra-chunk preparation checked on its own, kernel by kernel as the
  "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page does in its section on
  precision (each kernel against an fp32-or-better reference): its
  workspace intermediates (TU = Tm diag(beta), P = M o Q K^T, the decay
  vectors, the fp16 K^T and Q fragments) decoded from matrix-core fragment
  order and compared with the chunkwise oracle's, chunk by chunk and head by
  head.

Gates as elsewhere: relative L2 <= 2e-3 on outputs, <= 1e-3 on states.
"""

import dataclasses

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle.chunked import chunk_step
from oracle.slots import slots_step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import hybrid_linear_attention_gdn_amd as gdn  # noqa: E402
from gpu_util import (OUT_TOL, STATE_TOL, DevInputs, check_detail, chunk_fwd,  # noqa: E402
                      recurrent_step, rel_l2, workspace_for)

GUARD = 4096
SENT = 7.0


def _case(name, x):
    print(f"[case] {name}: N={x.n_seqs} T={x.total_tokens} Hqk={x.h_qk} Hv={x.h_v} "
          f"lengths={list(map(int, x.lengths))[:12]}", flush=True)


def _guarded(shape, dtype=torch.float32, fill=SENT):
    """A tensor of `shape` inside a buffer with GUARD elements of `fill` on each side."""
    n = int(np.prod(shape))
    buf = torch.full((GUARD + n + GUARD,), fill, dtype=dtype, device="cuda")
    return buf, buf[GUARD:GUARD + n].view(shape)


def _guards_intact(buf, n, fill=SENT):
    return bool(torch.all(buf[:GUARD] == fill)) and bool(torch.all(buf[GUARD + n:] == fill))


# ------------------------------------------------------------ segmented, in place

@pytest.mark.parametrize("hqk,hv", [(2, 4), (16, 32)], ids=["single_tiles", "tile_pairs"])
def test_segmented_final_state_aliases_initial(hqk, hv):
    """Segments of 3 chunks with nonzero initial states, final_state == initial_state:
    segment 0 must still start from the initial state although the last segment
    of the same sequence writes the final state in the same launch."""
    lengths = [300, 1, 700, 64, 0, 200]
    x = gi.make_inputs(lengths, hqk, hv, 128, 128, seed=41, state_std=0.02)
    _case(f"segmented_aliased_{hqk}x{hv}", x)
    d = DevInputs(x)
    sc = 3
    nbytes = gdn.gdn_chunk_fwd_segmented_workspace_size(x.n_seqs, x.total_tokens, x.h_qk, x.h_v, sc)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    s = d.s0.clone()
    out = torch.full((x.total_tokens, x.h_v, 128), float("nan"), device="cuda")
    gdn.gdn_chunk_fwd_segmented(d.q, d.k, d.v, d.g, d.beta, d.cu, s, out, s, sc, ws)
    torch.cuda.synchronize()
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o, f = out.cpu().numpy(), s.cpu().numpy()
    eo, ef = rel_l2(o, ro), rel_l2(f, rf)
    print(f"[result] aliased segmented: out {eo:.3e} state {ef:.3e}", flush=True)
    assert eo <= OUT_TOL and ef <= STATE_TOL
    check_detail("segmented_aliased", o, ro, f, rf, x.cu_seqlens)
    np.testing.assert_array_equal(f[4], x.initial_state[4])


# ------------------------------------------------------------ fp16 operand range

def _scaled(x, factor):
    """v and the initial states times a power of two (exact in bf16 and fp32):
    outputs and states scale by the same factor (the layer is linear in (V, S0))."""
    return dataclasses.replace(x, name=f"{x.name}_x{factor}", v=x.v * np.float32(factor),
                               initial_state=None if x.initial_state is None
                               else x.initial_state * np.float32(factor))


def test_chunk_fp16_range_v_times_1024():
    x = _scaled(gi.make_inputs([1000, 300], 16, 32, 128, 128, seed=55, state_std=0.02), 1024)
    _case("chunk_v_x1024", x)
    out, fin = chunk_fwd(DevInputs(x), poison=True)
    ro, rf, _ = oracle.forward_inputs(x, precision="f64")
    o, f = out.cpu().numpy(), fin.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(f).all()
    print(f"[result] max |state| {np.abs(rf).max():.1f}, max |out| {np.abs(ro).max():.1f}", flush=True)
    assert rel_l2(o, ro) <= OUT_TOL and rel_l2(f, rf) <= STATE_TOL
    check_detail("chunk_v_x1024", o, ro, f, rf, x.cu_seqlens)


def test_recurrent_fp16_range_v_times_1024():
    x = _scaled(gi.verify_8x6(seed=3), 1024)
    _case("verify_v_x1024", x)
    out, s_out, inter = recurrent_step(DevInputs(x), 8, 6, save=True)
    ro, rf, rs = oracle.forward_inputs(x, precision="f64", record_states=True)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(s_out.cpu().numpy(), rf) <= STATE_TOL
    assert rel_l2(inter.cpu().numpy().reshape(rs.shape), rs) <= STATE_TOL


# ------------------------------------------------------------ guard bands

@pytest.mark.parametrize("save", [True, False], ids=["snapshots", "state_only"])
def test_recurrent_step_writes_stay_in_bounds(save):
    x = gi.make_inputs([5] * 3, 2, 4, 128, 128, seed=61, state_std=0.02)
    _case(f"recurrent_guards_save{int(save)}", x)
    d = DevInputs(x)
    R, n = 3, 5
    ob, out = _guarded((R * n, 4, 128))
    sb, s_out = _guarded((R, 4, 128, 128))
    ib, inter = _guarded((R, n, 4, 128, 128)) if save else (None, None)
    gdn.gdn_recurrent_step(d.q, d.k, d.v, d.g, d.beta, R, n, d.s0, s_out, out, inter, save)
    torch.cuda.synchronize()
    assert _guards_intact(ob, out.numel()) and _guards_intact(sb, s_out.numel())
    ro, rf, rs = oracle.forward_inputs(x, record_states=True)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    assert rel_l2(s_out.cpu().numpy(), rf) <= STATE_TOL
    if save:
        assert _guards_intact(ib, inter.numel())
        assert rel_l2(inter.cpu().numpy().reshape(rs.shape), rs) <= STATE_TOL


@pytest.mark.parametrize("f16", [False, True], ids=["f32", "f16"])
def test_slots_writes_stay_in_bounds(f16):
    """The pool and out inside guard bands: only the slots the table names change."""
    lengths = [3, 0, 5, 1]
    x = gi.verify_variable(lengths, seed=62)
    R, M = len(lengths), 5
    pool_np = gi.state_pool(x, R * M, f16=f16, seed=62)
    table_np = gi.slot_table_contiguous(R, M, R)
    dt = torch.float16 if f16 else torch.float32
    pb, pool = _guarded(pool_np.shape, dt)
    pool.copy_(torch.from_numpy(pool_np))
    ob, out = _guarded((x.total_tokens, x.h_v, 128))
    d = DevInputs(x)
    table = torch.from_numpy(table_np).cuda()
    _case(f"slots_guards_{'f16' if f16 else 'f32'}", x)
    gdn.gdn_recurrent_step_slots(d.q, d.k, d.v, d.g, d.beta, d.cu, R, M, pool, table, None, out)
    torch.cuda.synchronize()
    assert _guards_intact(pb, pool.numel()) and _guards_intact(ob, out.numel())
    ro, rpool = slots_step(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool_np, table_np)
    assert rel_l2(out.cpu().numpy(), ro) <= OUT_TOL
    gp = pool.cpu().numpy()
    written = {int(s) for r in range(R) for s in table_np[r, 1:1 + lengths[r]]}
    for s in range(pool_np.shape[0]):
        if s in written:
            assert rel_l2(gp[s].astype(np.float64), rpool[s].astype(np.float64)) <= STATE_TOL, s
        else:
            assert np.array_equal(gp[s].view(np.uint8), pool_np[s].view(np.uint8)), s


def test_snapshots_write_stay_in_bounds():
    """chunk_states inside guard bands, NaN-filled: the chunk slots fill in, every
    other slot and both guard bands stay as they were."""
    lengths = [130, 0, 64, 7]
    x = gi.make_inputs(lengths, 2, 4, 128, 128, seed=63, state_std=0.02)
    _case("snapshots_guards", x)
    d = DevInputs(x)
    n_slots = gdn.gdn_chunk_state_slots(x.n_seqs, x.total_tokens, x.h_qk, x.h_v)
    cb, cs = _guarded((n_slots, 4, 128, 128), fill=float("nan"))
    ob, out = _guarded((x.total_tokens, 4, 128))
    fb, fin = _guarded((x.n_seqs, 4, 128, 128))
    ws = workspace_for(x)
    ws.fill_(0xFF)
    gdn.gdn_chunk_fwd_snapshots(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out, fin, cs, ws)
    torch.cuda.synchronize()
    n = cs.numel()
    assert bool(torch.isnan(cb[:GUARD]).all()) and bool(torch.isnan(cb[GUARD + n:]).all())
    assert _guards_intact(ob, out.numel()) and _guards_intact(fb, fin.numel())
    _, _, rs = oracle.forward_inputs(x, precision="f64", record_states=True)
    c = cs.cpu().numpy()
    written = set()
    for s, L in enumerate(lengths):
        a = int(x.cu_seqlens[s])
        for ch in range((L + 63) // 64):
            slot = s + a // 64 + ch
            written.add(slot)
            assert rel_l2(c[slot], rs[a + min(64 * (ch + 1), L) - 1]) <= STATE_TOL, (s, ch)
    for slot in range(n_slots):
        if slot not in written:
            assert np.isnan(c[slot]).all(), slot


# ------------------------------------------------------------ prep, kernel by kernel

def _workspace_regions(n_seqs, T, h_qk, h_v):
    """Byte offsets of the prefill workspace's regions, in the order and
    256-byte rounding the library carves them (region, per-unit elements, item bytes)."""
    slots = n_seqs + T // 64 + 1
    spec = [("tu", h_v, 6 * 64 * 8, 2), ("p", h_v, 6 * 64 * 8, 2),
            ("dg", h_v, 128, 4), ("kt", h_qk, 8 * 2 * 64 * 8, 2), ("qf", h_qk, 4 * 4 * 64 * 8, 2)]
    off, regions = 0, {}
    for name, heads, elems, isz in spec:
        regions[name] = (off, heads, elems, isz)
        off += (slots * heads * elems * isz + 255) // 256 * 256
    return regions


def _unit(ws, regions, name, slot, head):
    off, heads, elems, isz = regions[name]
    dt = np.float16 if isz == 2 else np.float32
    base = off + (slot * heads + head) * elems * isz
    return ws[base:base + elems * isz].view(dt).astype(np.float64)


# Decoders from matrix-core fragment order to [position or row, column]
# matrices.  Lane l = 16 gq + ln; contraction slot s of K-step qq holds index
# 32 qq + 16 (s // 4) + 4 gq + s % 4.
_GQ, _LN, _S = np.meshgrid(np.arange(4), np.arange(16), np.arange(8), indexing="ij")
_LANE = 16 * _GQ + _LN
_SLOT = 16 * (_S // 4) + 4 * _GQ + _S % 4


def _dec_rowfrag(frag, n_row_tiles, n_ksteps, order):
    """A fragments [f][lane][8] -> M[16 rt + ln][32 qq + slot]; order(rt, qq) gives f."""
    f = frag.reshape(-1, 64, 8)
    m = np.zeros((16 * n_row_tiles, 32 * n_ksteps))
    for rt in range(n_row_tiles):
        for qq in range(n_ksteps):
            fi = order(rt, qq)
            if fi is None:
                continue
            m[16 * rt + _LN, 32 * qq + _SLOT] = f[fi][_LANE, _S]
    return m


_P_BLOCKS = {(0, 0): 0, (1, 0): 1, (2, 0): 2, (2, 1): 3, (3, 0): 4, (3, 1): 5}


@pytest.mark.parametrize("hqk,hv", [(2, 4), (1, 4), (2, 6)],
                         ids=["pairs", "pairs_of_four_per_qk_head", "single_heads_of_three_per_qk_head"])
def test_prep_intermediates_against_chunkwise_oracle(hqk, hv):
    """Prep serves two value heads per workgroup when a q/k head has an even
    number of them (4 / 2, 4 / 1: there the second pair does not write the
    shared K^T and Q fragments), one otherwise (6 / 2)."""
    lengths = [200, 64, 1, 130]
    x = gi.make_inputs(lengths, hqk, hv, 128, 128, seed=71, state_std=0.02)
    _case(f"prep_stage_{hqk}x{hv}", x)
    d = DevInputs(x)
    ws = workspace_for(x)
    ws.fill_(0xFF)
    out = torch.empty((x.total_tokens, x.h_v, 128), device="cuda")
    gdn.gdn_chunk_fwd_stages(d.q, d.k, d.v, d.g, d.beta, d.cu, d.s0, out, None, ws, 1)
    torch.cuda.synchronize()
    w_np = ws.cpu().numpy()
    regions = _workspace_regions(x.n_seqs, x.total_tokens, x.h_qk, x.h_v)
    grp = x.h_v // x.h_qk
    worst = {"TU": 0.0, "P": 0.0, "dg": 0.0}
    sq = {k: [0.0, 0.0] for k in ("TU", "P")}
    for s, L in enumerate(lengths):
        a = int(x.cu_seqlens[s])
        for ch in range((L + 63) // 64):
            slot = s + a // 64 + ch
            t0, n = a + 64 * ch, min(64, L - 64 * ch)
            for j in range(x.h_qk):
                # K^T and Q fragments: the fp16 conversions of the bf16 inputs, exactly
                kt = _dec_rowfrag(_unit(w_np, regions, "kt", slot, j), 8, 2, lambda i, qq: 2 * i + qq)
                kref = np.zeros((64, 128))
                kref[:n] = x.k[t0:t0 + n, j].astype(np.float16)
                np.testing.assert_array_equal(kt.T, kref)
                qf = _dec_rowfrag(_unit(w_np, regions, "qf", slot, j), 4, 4, lambda p, qq: 4 * p + qq)
                qref = np.zeros((64, 128))
                qref[:n] = x.q[t0:t0 + n, j].astype(np.float16)
                np.testing.assert_array_equal(qf, qref)
            for h in range(x.h_v):
                j = h // grp
                r = chunk_step(x.q[t0:t0 + n, j], x.k[t0:t0 + n, j], x.v[t0:t0 + n, h],
                               x.g[t0:t0 + n, h], x.beta[t0:t0 + n, h], np.zeros((128, 128)))
                # TU = Tm diag(beta): what the state kernel forms W = TU diag(e^G) K
                # and U = TU V from
                tudec = _dec_rowfrag(_unit(w_np, regions, "tu", slot, h), 4, 2,
                                     lambda p, qq: _P_BLOCKS.get((p, qq)))
                pdec = _dec_rowfrag(_unit(w_np, regions, "p", slot, h), 4, 2,
                                    lambda p, qq: _P_BLOCKS.get((p, qq)))
                tu_ref = r["Tm"] * np.asarray(x.beta[t0:t0 + n, h], np.float64)[None, :]
                for name, dec, ref in (("TU", tudec, tu_ref), ("P", pdec, r["P"])):
                    e = rel_l2(dec[:n, :n], ref)
                    worst[name] = max(worst[name], e)
                    sq[name][0] += float(((dec[:n, :n] - ref) ** 2).sum())
                    sq[name][1] += float((ref ** 2).sum())
                    assert e <= OUT_TOL, (name, s, ch, h, e)
                    # pad rows and columns of a short chunk, and everything
                    # above the diagonal, are exactly zero
                    assert not np.any(dec[n:]) and not np.any(dec[:n, n:]), (name, s, ch, h)
                    assert not np.any(np.triu(dec, 1)), (name, "upper triangle", s, ch, h)
                # decay vectors: e^{G_C - G_r} (r < 63; entry 63 = e^{G_C}), then e^{G_r};
                # pad positions carry G_C (their g reads as 0)
                dg = _unit(w_np, regions, "dg", slot, h)
                G = np.concatenate([r["G"], np.full(64 - n, r["G"][-1])])
                want = np.concatenate([np.exp(G[-1] - G[:63]), [np.exp(G[-1])], np.exp(G)])
                # G is an fp32 prefix sum of at most 64 terms: its absolute error is
                # below 63 * 2^-24 * max|G| (2.3e-4 at this workload's |G| <= 60),
                # and that is the relative error it leaves in e^G
                e = float(np.max(np.abs(dg - want) / np.maximum(np.abs(want), 1e-30)))
                bound = 63 * 2.0 ** -24 * max(1.0, float(np.abs(G).max())) + 1e-5
                worst["dg"] = max(worst["dg"], e)
                assert e <= bound, ("decay vectors", s, ch, h, e, bound)
    tot = {k: (v[0] / v[1]) ** 0.5 for k, v in sq.items()}
    print(f"[result] prep stage: worst per (chunk, head) {worst}; whole-tensor {tot}", flush=True)
    for k in tot:
        assert tot[k] <= 1e-3, (k, tot[k])


# ------------------------------------------------------------ GDN_DEBUG_CHECKS on the device path

def test_debug_checks_reject_bad_device_contents(monkeypatch):
    """With GDN_DEBUG_CHECKS set, the entry points copy their inputs to the host
    and refuse a violated precondition before any launch (nothing written);
    valid inputs give the results of an unchecked call, bit for bit."""
    x = gi.make_inputs([70, 5], 2, 4, 128, 128, seed=81, state_std=0.02)
    _case("debug_checks", x)
    d = DevInputs(x)
    ref_out, ref_fin = chunk_fwd(d)
    monkeypatch.setenv("GDN_DEBUG_CHECKS", "1")
    out, fin = chunk_fwd(d)
    assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)
    bad_g = d.g.clone()
    bad_g[71, 2] = 0.5
    out = torch.full_like(ref_out, SENT)
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_chunk_fwd(d.q, d.k, d.v, bad_g, d.beta, d.cu, d.s0, out, None, workspace_for(x))
    assert ei.value.status == gdn.GDN_ERR_INVALID_VALUE and "g[286]" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out == SENT))
    bad_cu = torch.tensor([0, 76, 75], dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, bad_cu, d.s0, out, None, workspace_for(x))
    assert "decreases" in str(ei.value)
    y = gi.verify_8x6(seed=2)
    dy = DevInputs(y)
    s_bad = dy.s0.clone()
    s_bad[3, 5, 7, 9] = float("nan")
    vout = torch.empty((48, 32, 128), device="cuda")
    with pytest.raises(gdn.GDNError) as ei:
        gdn.gdn_recurrent_step(dy.q, dy.k, dy.v, dy.g, dy.beta, 8, 6, s_bad, s_bad, vout, None, False)
    assert "state_in" in str(ei.value)
    monkeypatch.delenv("GDN_DEBUG_CHECKS")


# ------------------------------------------------------------ prepared calls

def test_prepared_steps_match_the_plain_calls_bitwise():
    """prepare_recurrent_step / prepare_recurrent_step_slots check and marshal
    their arguments once; each later call must compute what the plain call
    computes on the buffers' contents at that time, bit for bit: decode in
    place over three steps with new tokens written into the same buffers,
    verify with snapshots on an explicit stream, and an fp16 slot-pool step."""
    R = 8
    xs = [gi.make_inputs([1] * R, 16, 32, 128, 128, seed=90 + i, state_std=0.02) for i in range(3)]
    _case("prepared_decode", xs[0])
    d0 = DevInputs(xs[0])
    s_a, s_b = d0.s0.clone(), d0.s0.clone()
    out_a = torch.full((R, 32, 128), float("nan"), device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    step = gdn.prepare_recurrent_step(d0.q, d0.k, d0.v, d0.g, d0.beta, R, 1, s_a, s_a, out_a, None, False)
    for x in xs:
        dx = DevInputs(x)
        for name in ("q", "k", "v", "g", "beta"):
            getattr(d0, name).copy_(getattr(dx, name))
        step()
        gdn.gdn_recurrent_step(d0.q, d0.k, d0.v, d0.g, d0.beta, R, 1, s_b, s_b, out_b, None, False)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b) and torch.equal(s_a, s_b)

    y = gi.verify_8x6(seed=3)
    dy = DevInputs(y)
    inter_a = torch.full((R, 6, 32, 128, 128), float("nan"), device="cuda")
    inter_b = torch.full_like(inter_a, float("nan"))
    vo_a = torch.empty((R * 6, 32, 128), device="cuda")
    vo_b = torch.empty_like(vo_a)
    side = torch.cuda.Stream()
    vstep = gdn.prepare_recurrent_step(dy.q, dy.k, dy.v, dy.g, dy.beta, R, 6, dy.s0, None, vo_a, inter_a, True)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        vstep(side)
    side.synchronize()
    gdn.gdn_recurrent_step(dy.q, dy.k, dy.v, dy.g, dy.beta, R, 6, dy.s0, None, vo_b, inter_b, True)
    torch.cuda.synchronize()
    assert torch.equal(vo_a, vo_b) and torch.equal(inter_a, inter_b)

    pool_np = gi.state_pool(y, R * 6, f16=True)
    pool_a = torch.from_numpy(pool_np).to("cuda")
    pool_b = pool_a.clone()
    table = torch.from_numpy(gi.slot_table_contiguous(R, 6, R)).to("cuda")
    cu_tok = torch.from_numpy(y.cu_seqlens).to("cuda")
    so_a = torch.empty((R * 6, 32, 128), device="cuda")
    so_b = torch.empty_like(so_a)
    sstep = gdn.prepare_recurrent_step_slots(dy.q, dy.k, dy.v, dy.g, dy.beta, cu_tok, R, 6, pool_a, table, None, so_a)
    sstep()
    gdn.gdn_recurrent_step_slots(dy.q, dy.k, dy.v, dy.g, dy.beta, cu_tok, R, 6, pool_b, table, None, so_b)
    torch.cuda.synchronize()
    assert torch.equal(so_a, so_b) and torch.equal(pool_a, pool_b)
