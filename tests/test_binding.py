"""The Python binding refuses tensors the kernels would misread (CPU-only:
every case fails before the library is called)."""
import pytest
import torch

import hybrid_linear_attention_gdn_amd as gdn

T, HQK, HV, D = 70, 2, 4, 128
ADDR = 1 << 20          # a stand-in device address: the binding does not check int addresses


def prefill_args(**over):
    # every argument but the one under test is an address, so that the check of
    # that one is reached (a well-formed CPU tensor is refused as such)
    a = dict(q=ADDR, k=ADDR, v=ADDR, g=ADDR, beta=ADDR, cu_seqlens=ADDR, initial_state=None, out=ADDR,
             final_state=None, workspace=ADDR)
    a.update(over)
    return a


def call_prefill(**over):
    a = prefill_args(**over)
    gdn.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"], a["initial_state"], a["out"],
                      a["final_state"], a["workspace"], dims=gdn.make_dims(2, T, HQK, HV), workspace_bytes=1 << 30)


@pytest.mark.parametrize("over,needle", [
    (dict(k=torch.zeros(T - 1, HQK, D, dtype=torch.bfloat16)), "k has shape"),
    (dict(k=torch.zeros(T, HQK, D, dtype=torch.float16)), "k has dtype"),
    (dict(v=torch.zeros(T, D, HV, dtype=torch.bfloat16).transpose(1, 2)), "v is not contiguous"),
    (dict(g=torch.zeros(T, HV, dtype=torch.float64)), "g has dtype"),
    (dict(beta=torch.zeros(T)), "beta has shape"),
    (dict(out=torch.zeros(T, HV, D, dtype=torch.bfloat16)), "out has dtype"),
    (dict(cu_seqlens=torch.tensor([0, 30, T], dtype=torch.int64)), "cu_seqlens has dtype"),
    (dict(cu_seqlens=torch.tensor([0, T], dtype=torch.int32)), "cu_seqlens has shape"),
    (dict(initial_state=torch.zeros(1, HV, D, D)), "initial_state has shape"),
    (dict(final_state=torch.zeros(2, HV, D, D, dtype=torch.float16)), "final_state has dtype"),
    (dict(out=torch.zeros(T, HV, D)), "out is not a GPU tensor"),
])
def test_prefill_rejects_bad_tensors(over, needle):
    with pytest.raises(gdn.GDNError, match=needle):
        call_prefill(**over)


def test_shapes_are_derived_from_q_v_and_cu_seqlens():
    # without dims the sizes come from q, v and cu_seqlens, and every other
    # tensor must match them; a CPU tensor is refused (there is no CPU path)
    q = torch.zeros(T, HQK, D, dtype=torch.bfloat16)
    v = torch.zeros(T, HV, D, dtype=torch.bfloat16)
    cu = torch.tensor([0, 30, T], dtype=torch.int32)
    dims = gdn._prefill_dims(q, v, cu)
    assert (dims.n_seqs, dims.total_tokens, dims.n_heads_qk, dims.n_heads_v) == (2, T, HQK, HV)
    with pytest.raises(gdn.GDNError, match="k has shape"):
        gdn._check_prefill(ADDR, q[1:], ADDR, ADDR, ADDR, ADDR, None, ADDR, None, ADDR, dims, "prefill")
    with pytest.raises(gdn.GDNError, match="q is not a GPU tensor"):
        gdn.gdn_chunk_fwd(q, q, v, ADDR, ADDR, cu, None, ADDR, None, torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(gdn.GDNError, match="cu_seqlens must be a 1-D tensor"):
        gdn.gdn_chunk_fwd(q, q, v, ADDR, ADDR, ADDR, None, ADDR, None, None)


def test_workspace_address_needs_its_size():
    with pytest.raises(gdn.GDNError, match="workspace_bytes is required"):
        gdn.gdn_chunk_fwd(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, None, ADDR, None, ADDR, dims=gdn.make_dims(2, T, HQK, HV))


def test_snapshot_buffer_must_hold_every_chunk_slot():
    slots = gdn.gdn_chunk_state_slots(2, T, HQK, HV)
    with pytest.raises(gdn.GDNError, match="chunk_states has shape"):
        gdn.gdn_chunk_fwd_snapshots(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, None, ADDR, None,
                                    torch.zeros(slots - 1, HV, D, D), ADDR,
                                    dims=gdn.make_dims(2, T, HQK, HV), workspace_bytes=1 << 30)


def test_recurrent_step_checks_the_intermediate_states():
    R, n = 3, 6
    with pytest.raises(gdn.GDNError, match="intermediate_states has shape"):
        gdn.gdn_recurrent_step(ADDR, ADDR, ADDR, ADDR, ADDR, R, n, ADDR, None, ADDR,
                               torch.zeros(R, n - 1, HV, D, D), True, dims=gdn.make_dims(R, R * n, HQK, HV))
    with pytest.raises(gdn.GDNError, match="state_in has dtype"):
        gdn.gdn_recurrent_step(ADDR, ADDR, ADDR, ADDR, ADDR, R, n, torch.zeros(R, HV, D, D, dtype=torch.float16),
                               ADDR, ADDR, None, False, dims=gdn.make_dims(R, R * n, HQK, HV))


def test_slot_step_checks_its_index_arrays():
    R, mt, Tt = 2, 5, 7
    dims = gdn.make_dims(R, Tt, HQK, HV)
    pool = torch.zeros(9, HV, D, D, dtype=torch.float16)
    kw = dict(dims=dims, state_dtype=gdn.GDN_STATE_F16, pool_slots=9)
    with pytest.raises(gdn.GDNError, match="slot_table has shape"):
        gdn.gdn_recurrent_step_slots(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, R, mt, ADDR,
                                     torch.zeros(R, mt, dtype=torch.int32), None, ADDR, **kw)
    with pytest.raises(gdn.GDNError, match="num_accepted has dtype"):
        gdn.gdn_recurrent_step_slots(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, R, mt, ADDR,
                                     ADDR, torch.zeros(R, dtype=torch.int64), ADDR, **kw)
    with pytest.raises(gdn.GDNError, match="state_pool has shape"):
        gdn.gdn_recurrent_step_slots(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, R, mt, pool[1:], ADDR, None, ADDR, **kw)
    with pytest.raises(gdn.GDNError, match="state_pool is not a GPU tensor"):
        gdn.gdn_recurrent_step_slots(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, R, mt, pool, ADDR, None, ADDR, dims=dims)


def test_prepared_calls_check_their_arguments_once_like_the_plain_calls():
    R, n = 3, 6
    dims = gdn.make_dims(R, R * n, HQK, HV)
    with pytest.raises(gdn.GDNError, match="intermediate_states has shape"):
        gdn.prepare_recurrent_step(ADDR, ADDR, ADDR, ADDR, ADDR, R, n, ADDR, None, ADDR,
                                   torch.zeros(R, n - 1, HV, D, D), True, dims=dims)
    pool = torch.zeros(9, HV, D, D, dtype=torch.float16)
    with pytest.raises(gdn.GDNError, match="state_pool is not a GPU tensor"):
        gdn.prepare_recurrent_step_slots(ADDR, ADDR, ADDR, ADDR, ADDR, ADDR, R, 5, pool, ADDR, None, ADDR,
                                         dims=gdn.make_dims(R, 7, HQK, HV))
    # raw addresses carry no device, so a call needs an explicit stream
    step = gdn.prepare_recurrent_step(ADDR, ADDR, ADDR, ADDR, ADDR, R, n, ADDR, ADDR, ADDR, None, False, dims=dims)
    with pytest.raises(gdn.GDNError, match="need an explicit stream"):
        step()
