"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

Only failing-validation paths are exercised here (plus the pure host
workspace-size query and the zero-sequence no-op); no call in this file
reaches a kernel launch, so fake device addresses are safe.
"""

import ctypes
import os
import re

import pytest

import hybrid_linear_attention_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

FAKE = 0x7f0000000000          # 16-byte aligned fake device address (never dereferenced)
MIS = FAKE + 4                 # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        import hybrid_linear_attention_gdn_amd.build as b
        b.build()
    return gdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(gdn.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exported_symbols_have_c_linkage():
    out = os.popen(f"nm -D --defined-only {gdn.LIB_PATH}").read()
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in names, f"{name} not exported unmangled"


def test_status_strings(lib):
    for s in range(6):
        assert lib.gdn_status_string(s)
    assert lib.gdn_status_string(99) == b"unknown status"


def dims(n=1, T=64, hqk=2, hv=4, dk=128, dv=128):
    return gdn.make_dims(n, T, hqk, hv, dk, dv)


def ws_size(lib, d):
    out = ctypes.c_size_t(0)
    st = lib.gdn_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(out))
    return st, out.value


def test_workspace_size_formula(lib):
    st, b = ws_size(lib, dims(n=1, T=4000, hqk=16, hv=32))
    assert st == 0
    slots = 1 + 4000 // 64 + 1
    per_v = 3072 * 2 * 2 + 128 * 4             # per value head: TU, P (fp16), decay vectors (fp32)
    per_qk = 8192 * 2 * 2                        # per q/k head: K^T, Q (fp16)
    need = slots * (32 * per_v + 16 * per_qk) + 1024  # + the sink of masked-off stores
    assert need <= b < need + 7 * 256


@pytest.mark.parametrize("d,code", [
    (dims(dk=64, dv=64), gdn.GDN_ERR_NOT_SUPPORTED),
    (dims(dk=128, dv=64), gdn.GDN_ERR_NOT_SUPPORTED),
    (dims(hqk=3, hv=4), gdn.GDN_ERR_INVALID_VALUE),
    (dims(hqk=0), gdn.GDN_ERR_INVALID_VALUE),
    (dims(n=-1), gdn.GDN_ERR_INVALID_VALUE),
    (dims(T=-5), gdn.GDN_ERR_INVALID_VALUE),
    (dims(n=0, T=10), gdn.GDN_ERR_INVALID_VALUE),
    (dims(T=2**31), gdn.GDN_ERR_INVALID_VALUE),
    (dims(T=2**30), gdn.GDN_ERR_INVALID_VALUE),            # more than 2^24 chunk slots
    (dims(n=2**16, hqk=32, hv=64), gdn.GDN_ERR_INVALID_VALUE),  # more than 2^21 (sequence, head) pairs
    (dims(hqk=1, hv=70000), gdn.GDN_ERR_INVALID_VALUE),     # more value heads than a grid dimension holds
    (dims(dk=0), gdn.GDN_ERR_INVALID_VALUE),
])
def test_workspace_size_rejects_bad_dims(lib, d, code):
    st, _ = ws_size(lib, d)
    assert st == code
    assert lib.gdn_get_last_error()


def min_ws_size(lib, d):
    out = ctypes.c_size_t(0)
    st = lib.gdn_chunk_fwd_min_workspace_size(ctypes.byref(d), ctypes.byref(out))
    return st, out.value


def test_min_workspace_size_for_one_long_sequence(lib):
    """One sequence whose intermediates exceed 160 MiB runs range by range and
    needs one range's intermediates (64 chunk slots at 32 value / 16 q/k
    heads) plus the carried fp32 state; anything else needs the full
    workspace."""
    d = dims(n=1, T=131072, hqk=16, hv=32)
    st, full = ws_size(lib, d)
    st2, small = min_ws_size(lib, d)
    assert st == 0 and st2 == 0
    per_v = 3072 * 2 * 2 + 128 * 4
    per_qk = 8192 * 2 * 2
    expect = 64 * (32 * per_v + 16 * per_qk) + 1024 + 32 * 128 * 128 * 4
    assert expect <= small < expect + 8 * 256
    assert full > 1800e6 and small < 64e6
    assert small <= gdn.GDN_NOALLOC_SCRATCH_BYTES          # the no-allocation entry point takes it
    # 16 value / 8 q/k heads: ranges of 128 slots
    st, small16 = min_ws_size(lib, dims(n=1, T=131072, hqk=8, hv=16))
    per16 = 16 * per_v + 8 * per_qk
    assert st == 0 and 128 * per16 <= small16 < 128 * per16 + 16 * 128 * 128 * 4 + 8 * 256 + 1024
    # below 160 MiB of intermediates, or several sequences: the full workspace
    for dd in (dims(n=1, T=4000, hqk=16, hv=32), dims(n=2, T=131072, hqk=16, hv=32),
               dims(n=1, T=9400, hqk=16, hv=32)):
        assert min_ws_size(lib, dd) == ws_size(lib, dd)
    # very many heads over few chunks: one range would be the whole sequence
    # and take more room than the single pass, so the single pass stays
    dd = dims(n=1, T=128, hqk=1024, hv=2048)
    assert min_ws_size(lib, dd) == ws_size(lib, dd)


def test_min_workspace_size_is_what_gdn_chunk_fwd_checks(lib):
    """gdn_chunk_fwd takes a range-sized workspace for one long sequence (and
    refuses one byte less); the stage-by-stage call, which runs the single
    pass, still needs the full size."""
    d = dims(n=1, T=131072, hqk=16, hv=32)
    small = min_ws_size(lib, d)[1]
    assert chunk_call(lib, d, wsb=small - 1) == gdn.GDN_ERR_WORKSPACE
    assert str(small) in lib.gdn_get_last_error().decode()
    st = lib.gdn_chunk_fwd_stages(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, ctypes.byref(d),
                                  FAKE, small, 1, None)
    assert st == gdn.GDN_ERR_WORKSPACE
    msg = lib.gdn_get_last_error().decode()
    assert str(ws_size(lib, d)[1]) in msg
    out = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_min_workspace_size(None, ctypes.byref(out)) == gdn.GDN_ERR_INVALID_VALUE
    assert lib.gdn_chunk_fwd_min_workspace_size(ctypes.byref(d), None) == gdn.GDN_ERR_INVALID_VALUE
    assert min_ws_size(lib, dims(dk=64, dv=64))[0] == gdn.GDN_ERR_NOT_SUPPORTED


def test_workspace_size_null_args(lib):
    out = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(None, ctypes.byref(out)) == gdn.GDN_ERR_INVALID_VALUE
    d = dims()
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(d), None) == gdn.GDN_ERR_INVALID_VALUE


def chunk_call(lib, d, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, s0=None, out=FAKE, fin=None,
                ws=FAKE, wsb=None)
    args.update(over)
    if args["wsb"] is None:
        args["wsb"] = ws_size(lib, d)[1]
    return lib.gdn_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"], args["cu"],
                             args["s0"], args["out"], args["fin"], ctypes.byref(d), args["ws"],
                             args["wsb"], None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "cu", "out"])
def test_chunk_fwd_rejects_null(lib, name):
    assert chunk_call(lib, dims(), **{name: None}) == gdn.GDN_ERR_INVALID_VALUE
    assert name.replace("cu", "cu_seqlens") in lib.gdn_get_last_error().decode()


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "cu", "out", "s0", "fin"])
def test_chunk_fwd_rejects_misaligned(lib, name):
    assert chunk_call(lib, dims(), **{name: MIS}) == gdn.GDN_ERR_MISALIGNED


def test_chunk_fwd_workspace_checks(lib):
    d = dims()
    assert chunk_call(lib, d, ws=None) == gdn.GDN_ERR_WORKSPACE
    need = ws_size(lib, d)[1]
    assert chunk_call(lib, d, wsb=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert chunk_call(lib, d, ws=FAKE + 16) == gdn.GDN_ERR_MISALIGNED


def test_chunk_fwd_rejects_unsupported_dims(lib):
    assert chunk_call(lib, dims(dk=64, dv=64), wsb=1 << 30) == gdn.GDN_ERR_NOT_SUPPORTED
    assert chunk_call(lib, dims(hqk=3, hv=4), wsb=1 << 30) == gdn.GDN_ERR_INVALID_VALUE


def test_chunk_fwd_zero_sequences_is_a_noop(lib):
    d = dims(n=0, T=0)
    assert chunk_call(lib, d, q=None, k=None, v=None, g=None, beta=None, cu=None, out=None,
                      ws=None, wsb=0) == gdn.GDN_SUCCESS
    assert lib.gdn_get_last_error() == b""


def step_call(lib, d, R=2, n=3, save=1, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s_in=FAKE, s_out=FAKE, out=FAKE,
                inter=FAKE if save else None)
    args.update(over)
    return lib.gdn_recurrent_step(args["q"], args["k"], args["v"], args["g"], args["beta"], R, n,
                                  args["s_in"], args["s_out"], args["out"], args["inter"], save,
                                  ctypes.byref(d), None)


def sdims(R=2, n=3, **kw):
    return dims(n=R, T=R * n, **kw)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "s_in", "out"])
def test_recurrent_step_rejects_null(lib, name):
    assert step_call(lib, sdims(), **{name: None}) == gdn.GDN_ERR_INVALID_VALUE


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "s_in", "s_out", "out", "inter"])
def test_recurrent_step_rejects_misaligned(lib, name):
    assert step_call(lib, sdims(), **{name: MIS}) == gdn.GDN_ERR_MISALIGNED


def test_recurrent_step_save_flag_consistency(lib):
    assert step_call(lib, sdims(), save=1, inter=None) == gdn.GDN_ERR_INVALID_VALUE
    assert step_call(lib, sdims(), save=0, inter=FAKE) == gdn.GDN_ERR_INVALID_VALUE
    assert step_call(lib, sdims(), save=0, s_out=None) == gdn.GDN_ERR_INVALID_VALUE


def test_recurrent_step_dims_must_match_counts(lib):
    assert step_call(lib, dims(n=3, T=6)) == gdn.GDN_ERR_INVALID_VALUE
    assert step_call(lib, dims(n=2, T=7)) == gdn.GDN_ERR_INVALID_VALUE
    assert lib.gdn_recurrent_step(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 3, FAKE, FAKE, FAKE, FAKE, 1,
                                  ctypes.byref(dims(n=-1, T=0)), None) == gdn.GDN_ERR_INVALID_VALUE
    assert step_call(lib, sdims(dk=64, dv=64)) == gdn.GDN_ERR_NOT_SUPPORTED


def test_recurrent_step_zero_requests_is_a_noop(lib):
    assert lib.gdn_recurrent_step(None, None, None, None, None, 0, 6, None, None, None, None, 0,
                                  ctypes.byref(dims(n=0, T=0)), None) == gdn.GDN_SUCCESS


def test_binding_raises_with_detail(lib):
    with pytest.raises(gdn.GDNError) as e:
        gdn.gdn_chunk_fwd_workspace_size(1, 64, 2, 4, 64, 64)
    assert e.value.status == gdn.GDN_ERR_NOT_SUPPORTED
    assert "128" in str(e.value)


def test_last_error_is_thread_local(lib):
    import threading
    assert ws_size(lib, dims(dk=64, dv=64))[0] == gdn.GDN_ERR_NOT_SUPPORTED
    seen = {}

    def other():
        seen["msg"] = lib.gdn_get_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == b""
    assert lib.gdn_get_last_error() != b""


def test_stages_rejects_bad_mask(lib):
    d = dims()
    need = ws_size(lib, d)[1]
    for mask in (0, 4, 7, 8, -1):
        assert lib.gdn_chunk_fwd_stages(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                        ctypes.byref(d), FAKE, need, mask, None) == gdn.GDN_ERR_INVALID_VALUE


def slots_call(lib, d, R=2, M=6, dtype=gdn.GDN_STATE_F16, pool_slots=14, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, pool=FAKE, table=FAKE,
                acc=None, out=FAKE)
    args.update(over)
    return lib.gdn_recurrent_step_slots(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                        args["cu"], R, M, args["pool"], dtype, pool_slots,
                                        args["table"], args["acc"], args["out"], ctypes.byref(d), None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "cu", "pool", "table", "out"])
def test_slots_step_rejects_null(lib, name):
    assert slots_call(lib, dims(n=2, T=9), **{name: None}) == gdn.GDN_ERR_INVALID_VALUE


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "pool", "out"])
def test_slots_step_rejects_misaligned(lib, name):
    assert slots_call(lib, dims(n=2, T=9), **{name: MIS}) == gdn.GDN_ERR_MISALIGNED


@pytest.mark.parametrize("name", ["cu", "table", "acc"])
def test_slots_step_rejects_misaligned_index_arrays(lib, name):
    assert slots_call(lib, dims(n=2, T=9), **{name: FAKE + 2}) == gdn.GDN_ERR_MISALIGNED


def test_slots_step_argument_checks(lib):
    d = dims(n=2, T=9)
    assert slots_call(lib, d, dtype=2) == gdn.GDN_ERR_INVALID_VALUE
    assert slots_call(lib, d, dtype=-1) == gdn.GDN_ERR_INVALID_VALUE
    assert slots_call(lib, d, pool_slots=0) == gdn.GDN_ERR_INVALID_VALUE
    assert slots_call(lib, d, R=3) == gdn.GDN_ERR_INVALID_VALUE          # dims->n_seqs differs
    assert slots_call(lib, d, M=-1) == gdn.GDN_ERR_INVALID_VALUE
    assert slots_call(lib, dims(n=2, T=9, dk=64, dv=64)) == gdn.GDN_ERR_NOT_SUPPORTED
    assert b"state_dtype" in (slots_call(lib, d, dtype=5), lib.gdn_get_last_error())[1]


def test_slots_step_zero_requests_is_a_noop(lib):
    assert slots_call(lib, dims(n=0, T=0), R=0, q=None, k=None, v=None, g=None, beta=None, cu=None,
                      pool=None, table=None, out=None) == gdn.GDN_SUCCESS


def test_chunk_state_slots(lib):
    n = ctypes.c_int64(-1)
    assert lib.gdn_chunk_state_slots(ctypes.byref(dims(n=3, T=200)), ctypes.byref(n)) == gdn.GDN_SUCCESS
    assert n.value == 3 + 200 // 64 + 1
    assert lib.gdn_chunk_state_slots(ctypes.byref(dims(n=3, T=200)), None) == gdn.GDN_ERR_INVALID_VALUE
    assert lib.gdn_chunk_state_slots(ctypes.byref(dims(dk=64, dv=64)), ctypes.byref(n)) == gdn.GDN_ERR_NOT_SUPPORTED
    assert gdn.gdn_chunk_state_slots(1, 4000, 16, 32) == 64


def snap_call(lib, d, **over):
    need = ws_size(lib, d)[1]
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, s0=None, out=FAKE, fin=None,
                cs=FAKE, ws=FAKE, wsb=need)
    args.update(over)
    return lib.gdn_chunk_fwd_snapshots(args["q"], args["k"], args["v"], args["g"], args["beta"], args["cu"],
                                       args["s0"], args["out"], args["fin"], args["cs"], ctypes.byref(d),
                                       args["ws"], args["wsb"], None)


def test_snapshots_rejects_bad_arguments(lib):
    d = dims(n=2, T=130)
    assert snap_call(lib, d, cs=None) == gdn.GDN_ERR_INVALID_VALUE
    assert snap_call(lib, d, cs=MIS) == gdn.GDN_ERR_MISALIGNED
    assert snap_call(lib, d, q=None) == gdn.GDN_ERR_INVALID_VALUE
    assert snap_call(lib, d, ws=None) == gdn.GDN_ERR_WORKSPACE
    assert snap_call(lib, d, wsb=ws_size(lib, d)[1] - 1) == gdn.GDN_ERR_WORKSPACE
    assert snap_call(lib, dims(n=2, T=130, dk=64, dv=64)) == gdn.GDN_ERR_NOT_SUPPORTED
    assert snap_call(lib, dims(n=0, T=0), cs=None, q=None, k=None, v=None, g=None, beta=None, cu=None,
                     out=None, ws=None, wsb=0) == gdn.GDN_SUCCESS


def test_segmented_workspace_and_arguments(lib):
    d = dims(n=2, T=1000, hqk=16, hv=32)
    base = ws_size(lib, d)[1]
    for sc in (1, 4, 64):
        b = ctypes.c_size_t(0)
        assert lib.gdn_chunk_fwd_segmented_workspace_size(ctypes.byref(d), sc, ctypes.byref(b)) == gdn.GDN_SUCCESS
        segslots = 2 + (2 + 1000 // 64 + 1) // sc + 1
        per = segslots * 32 * 128 * 128 * 4
        assert base + 3 * per <= b.value < base + 3 * per + 3 * 256
    b = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_segmented_workspace_size(ctypes.byref(d), 0, ctypes.byref(b)) == gdn.GDN_ERR_INVALID_VALUE
    assert lib.gdn_chunk_fwd_segmented_workspace_size(ctypes.byref(d), 4, None) == gdn.GDN_ERR_INVALID_VALUE
    need = ctypes.c_size_t(0)
    lib.gdn_chunk_fwd_segmented_workspace_size(ctypes.byref(d), 4, ctypes.byref(need))
    call = lambda sc, wsb, **o: lib.gdn_chunk_fwd_segmented(
        o.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, sc, ctypes.byref(d), FAKE, wsb, None)
    assert call(0, need.value) == gdn.GDN_ERR_INVALID_VALUE
    assert call(-3, need.value) == gdn.GDN_ERR_INVALID_VALUE
    assert call(4, need.value - 1) == gdn.GDN_ERR_WORKSPACE
    assert call(4, need.value, q=None) == gdn.GDN_ERR_INVALID_VALUE
    assert call(4, need.value, q=MIS) == gdn.GDN_ERR_MISALIGNED


def test_noalloc_rejects_batches_beyond_its_scratch(lib):
    """The fixed scratch holds GDN_NOALLOC_SCRATCH_BYTES; a batch that needs more
    is refused on the host, before any device call, with the sizes named."""
    import ctypes as ct
    d = dims(1, 9400, 16, 32)
    need = ct.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(ct.byref(d), ct.byref(need)) == 0
    assert need.value > gdn.GDN_NOALLOC_SCRATCH_BYTES
    st = lib.gdn_chunk_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, ct.byref(d), None)
    assert st == gdn.GDN_ERR_WORKSPACE
    msg = lib.gdn_get_last_error().decode()
    assert str(need.value) in msg and str(gdn.GDN_NOALLOC_SCRATCH_BYTES) in msg
    bad = dims(1, 64, 3, 4)
    assert lib.gdn_chunk_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                     ct.byref(bad), None) == gdn.GDN_ERR_INVALID_VALUE
    zero = dims(0, 0, 16, 32)
    assert lib.gdn_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, None,
                                     ct.byref(zero), None) == gdn.GDN_SUCCESS


def test_noalloc_header_size_matches_binding():
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.GDN_NOALLOC_SCRATCH_BYTES
