"""Gated DeltaNet layer on MI355X (gfx950): Python binding of libgdn.so.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI (``include/gdn.h``).  PyTorch provides device memory and the
current stream.  The names mirror the C entry points:

* ``gdn_chunk_fwd_workspace_size(n_seqs, total_tokens, h_qk, h_v)``
* ``gdn_chunk_fwd_min_workspace_size(n_seqs, total_tokens, h_qk, h_v)`` (what
  ``gdn_chunk_fwd`` accepts: one range's worth for one long sequence)
* ``gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace)``
* ``gdn_chunk_fwd_stages(..., stage_mask)`` (prep = 1, state with output = 2)
* ``gdn_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state)``
  (the library's fixed per-GPU scratch as workspace, for callers that cannot allocate)
* ``gdn_chunk_state_slots(n_seqs, total_tokens, h_qk, h_v)``
* ``gdn_chunk_fwd_segmented_workspace_size(n_seqs, total_tokens, h_qk, h_v, segment_chunks)``
* ``gdn_chunk_fwd_segmented(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
  segment_chunks, workspace)``
* ``gdn_chunk_fwd_snapshots(q, k, v, g, beta, cu_seqlens, initial_state, out,
  final_state, chunk_states, workspace)``
* ``gdn_recurrent_step(q, k, v, g, beta, n_requests, tokens_per_request, state_in,
  state_out, out, intermediate_states, save_intermediate_states)``
* ``gdn_recurrent_step_slots(q, k, v, g, beta, cu_tokens, n_requests, max_tokens,
  state_pool, slot_table, num_accepted, out)`` (pool dtype float32 or float16)
* ``gdn_check_chunk_inputs_host(...)`` / ``gdn_check_step_inputs_host(...)``: the
  device-content preconditions on host (numpy) arrays, the checks that
  ``GDN_DEBUG_CHECKS=1`` runs inside every entry point

There is no fallback: if ``libgdn.so`` is missing or a call fails, a
``GDNError`` is raised.  Build the library with
``python -m hybrid_linear_attention_gdn_amd.build``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_SUCCESS = 0
GDN_ERR_INVALID_VALUE = 1
GDN_ERR_NOT_SUPPORTED = 2
GDN_ERR_MISALIGNED = 3
GDN_ERR_WORKSPACE = 4
GDN_ERR_LAUNCH = 5

GDN_NOALLOC_SCRATCH_BYTES = 128 << 20   # fixed workspace of gdn_chunk_fwd_noalloc, per GPU

GDN_STATE_F32 = 0
GDN_STATE_F16 = 1

EXPORTED_SYMBOLS = (
    "gdn_chunk_fwd_workspace_size",
    "gdn_chunk_fwd_min_workspace_size",
    "gdn_chunk_fwd",
    "gdn_chunk_fwd_stages",
    "gdn_chunk_state_slots",
    "gdn_chunk_fwd_snapshots",
    "gdn_chunk_fwd_segmented_workspace_size",
    "gdn_chunk_fwd_segmented",
    "gdn_recurrent_step",
    "gdn_recurrent_step_slots",
    "gdn_chunk_fwd_noalloc",
    "gdn_check_chunk_inputs_host",
    "gdn_check_step_inputs_host",
    "gdn_status_string",
    "gdn_get_last_error",
)


class GDNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class gdn_dims(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64),
                ("n_heads_qk", ctypes.c_int32),
                ("n_heads_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise GDNError(-1, f"{path} not found: build it with `python -m hybrid_linear_attention_gdn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, c32, c64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dims_p = ctypes.POINTER(gdn_dims)
    lib.gdn_chunk_fwd_workspace_size.argtypes = [dims_p, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.gdn_chunk_fwd_min_workspace_size.argtypes = [dims_p, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_min_workspace_size.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, dims_p, vp, sz, vp]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_stages.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, dims_p, vp, sz, ctypes.c_int, vp]
    lib.gdn_chunk_fwd_stages.restype = ctypes.c_int
    lib.gdn_chunk_state_slots.argtypes = [dims_p, ctypes.POINTER(c64)]
    lib.gdn_chunk_state_slots.restype = ctypes.c_int
    lib.gdn_chunk_fwd_snapshots.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, dims_p, vp, sz, vp]
    lib.gdn_chunk_fwd_snapshots.restype = ctypes.c_int
    lib.gdn_chunk_fwd_segmented_workspace_size.argtypes = [dims_p, c32, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_segmented_workspace_size.restype = ctypes.c_int
    lib.gdn_chunk_fwd_segmented.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, c32, dims_p, vp, sz, vp]
    lib.gdn_chunk_fwd_segmented.restype = ctypes.c_int
    lib.gdn_recurrent_step.argtypes = [vp, vp, vp, vp, vp, c32, c32, vp, vp, vp, vp, ctypes.c_int, dims_p, vp]
    lib.gdn_recurrent_step.restype = ctypes.c_int
    lib.gdn_recurrent_step_slots.argtypes = [vp, vp, vp, vp, vp, vp, c32, c32, vp, c32, c64, vp, vp, vp,
                                             dims_p, vp]
    lib.gdn_recurrent_step_slots.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, dims_p, vp]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_check_chunk_inputs_host.argtypes = [vp, vp, vp, vp, vp, vp, vp, dims_p]
    lib.gdn_check_chunk_inputs_host.restype = ctypes.c_int
    lib.gdn_check_step_inputs_host.argtypes = [vp, vp, vp, vp, vp, vp, c64, dims_p]
    lib.gdn_check_step_inputs_host.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_get_last_error.argtypes = []
    lib.gdn_get_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(lib, status: int, what: str) -> None:
    if status != GDN_SUCCESS:
        name = lib.gdn_status_string(status).decode()
        detail = lib.gdn_get_last_error().decode()
        raise GDNError(status, f"{what}: {name}: {detail}")


def _ptr(x) -> Optional[int]:
    """Device address of a tensor, an int address as is, None for NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return _current_stream(t.get_device())
    return None


def make_dims(n_seqs: int, total_tokens: int, h_qk: int, h_v: int, d_k: int = 128, d_v: int = 128) -> gdn_dims:
    return gdn_dims(int(n_seqs), int(total_tokens), int(h_qk), int(h_v), int(d_k), int(d_v))


def _check_arg(x, what: str, name: str, dtypes, shape=None) -> None:
    """Refuse a tensor argument whose dtype, shape or layout the kernels would
    misread.  The C ABI sees bare addresses, so this is the only place where a
    short or strided buffer can be caught before a kernel reads past it.  None
    and int addresses pass unchecked (the caller then vouches for them)."""
    if x is None or isinstance(x, int):
        return
    import torch
    if not isinstance(x, torch.Tensor):
        raise GDNError(GDN_ERR_INVALID_VALUE, f"{what}: {name} must be a tensor, a device address or None")
    if dtypes is not None and x.dtype not in dtypes:
        raise GDNError(GDN_ERR_INVALID_VALUE, f"{what}: {name} has dtype {x.dtype}, expected one of {list(dtypes)}")
    if shape is not None and x.shape != shape:
        raise GDNError(GDN_ERR_INVALID_VALUE, f"{what}: {name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if not x.is_contiguous():
        raise GDNError(GDN_ERR_INVALID_VALUE, f"{what}: {name} is not contiguous")
    if not x.is_cuda:
        raise GDNError(GDN_ERR_INVALID_VALUE, f"{what}: {name} is not a GPU tensor (there is no CPU path)")


def _check_tokens(q, k, v, g, beta, out, dims: gdn_dims, what: str) -> None:
    import torch
    bf16, f32 = (torch.bfloat16,), (torch.float32,)
    T, hqk, hv, dk, dv = dims.total_tokens, dims.n_heads_qk, dims.n_heads_v, dims.d_k, dims.d_v
    _check_arg(q, what, "q", bf16, (T, hqk, dk))
    _check_arg(k, what, "k", bf16, (T, hqk, dk))
    _check_arg(v, what, "v", bf16, (T, hv, dv))
    _check_arg(g, what, "g", f32, (T, hv))
    _check_arg(beta, what, "beta", f32, (T, hv))
    _check_arg(out, what, "out", f32, (T, hv, dv))


def _check_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace,
                   dims: gdn_dims, what: str) -> None:
    import torch
    _check_tokens(q, k, v, g, beta, out, dims, what)
    state = (dims.n_seqs, dims.n_heads_v, dims.d_k, dims.d_v)
    _check_arg(cu_seqlens, what, "cu_seqlens", (torch.int32,), (dims.n_seqs + 1,))
    _check_arg(initial_state, what, "initial_state", (torch.float32,), state)
    _check_arg(final_state, what, "final_state", (torch.float32,), state)
    _check_arg(workspace, what, "workspace", None)


def _nbytes(workspace, workspace_bytes: Optional[int]) -> int:
    if workspace_bytes is not None:
        return int(workspace_bytes)
    if workspace is None:
        return 0
    if isinstance(workspace, int):
        raise GDNError(GDN_ERR_INVALID_VALUE, "workspace_bytes is required with a workspace address")
    return workspace.numel() * workspace.element_size()


def _dims_from(q, v, n_seqs: int, total_tokens: int) -> gdn_dims:
    import torch
    for name, t in (("q", q), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise GDNError(GDN_ERR_INVALID_VALUE, f"{name} must be a [tokens, heads, dim] tensor unless dims is given")
    return make_dims(n_seqs, total_tokens, q.shape[1], v.shape[1], q.shape[2], v.shape[2])


def _prefill_dims(q, v, cu_seqlens) -> gdn_dims:
    import torch
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1:
        raise GDNError(GDN_ERR_INVALID_VALUE, "cu_seqlens must be a 1-D tensor unless dims is given")
    return _dims_from(q, v, cu_seqlens.shape[0] - 1, q.shape[0] if hasattr(q, "shape") else 0)


def gdn_chunk_fwd_workspace_size(n_seqs: int, total_tokens: int, h_qk: int, h_v: int,
                                 d_k: int = 128, d_v: int = 128) -> int:
    lib = load_library()
    dims = make_dims(n_seqs, total_tokens, h_qk, h_v, d_k, d_v)
    out = ctypes.c_size_t(0)
    _check(lib, lib.gdn_chunk_fwd_workspace_size(ctypes.byref(dims), ctypes.byref(out)),
           "gdn_chunk_fwd_workspace_size")
    return int(out.value)


def gdn_chunk_fwd_min_workspace_size(n_seqs: int, total_tokens: int, h_qk: int, h_v: int,
                                     d_k: int = 128, d_v: int = 128) -> int:
    lib = load_library()
    dims = make_dims(n_seqs, total_tokens, h_qk, h_v, d_k, d_v)
    out = ctypes.c_size_t(0)
    _check(lib, lib.gdn_chunk_fwd_min_workspace_size(ctypes.byref(dims), ctypes.byref(out)),
           "gdn_chunk_fwd_min_workspace_size")
    return int(out.value)


def gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace,
                  *, dims: Optional[gdn_dims] = None, workspace_bytes: Optional[int] = None,
                  stream=None) -> None:
    """Chunked prefill.  Tensors are device tensors (or raw int addresses with ``dims``)."""
    lib = load_library()
    if dims is None:
        dims = _prefill_dims(q, v, cu_seqlens)
    _check_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace, dims, "gdn_chunk_fwd")
    workspace_bytes = _nbytes(workspace, workspace_bytes)
    st = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                           _ptr(initial_state), _ptr(out), _ptr(final_state), ctypes.byref(dims),
                           _ptr(workspace), int(workspace_bytes),
                           _stream(stream, q, out, cu_seqlens))
    _check(lib, st, "gdn_chunk_fwd")


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                          *, dims: Optional[gdn_dims] = None, stream=None) -> None:
    """Chunked prefill with the library's fixed per-GPU scratch as its workspace
    (allocates nothing; batches up to GDN_NOALLOC_SCRATCH_BYTES of workspace;
    overlapping calls on one GPU race).  See include/gdn.h."""
    lib = load_library()
    if dims is None:
        dims = _prefill_dims(q, v, cu_seqlens)
    _check_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, None, dims,
                   "gdn_chunk_fwd_noalloc")
    st = lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                   _ptr(initial_state), _ptr(out), _ptr(final_state), ctypes.byref(dims),
                                   _stream(stream, q, out, cu_seqlens))
    _check(lib, st, "gdn_chunk_fwd_noalloc")


def gdn_chunk_fwd_stages(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace,
                         stage_mask: int, *, dims: Optional[gdn_dims] = None,
                         workspace_bytes: Optional[int] = None, stream=None) -> None:
    """Selected stages of the chunked prefill (1 = prep, 2 = state with output)."""
    lib = load_library()
    if dims is None:
        dims = _prefill_dims(q, v, cu_seqlens)
    _check_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace, dims, "gdn_chunk_fwd_stages")
    workspace_bytes = _nbytes(workspace, workspace_bytes)
    st = lib.gdn_chunk_fwd_stages(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                  _ptr(initial_state), _ptr(out), _ptr(final_state), ctypes.byref(dims),
                                  _ptr(workspace), int(workspace_bytes), int(stage_mask),
                                  _stream(stream, q, out, cu_seqlens))
    _check(lib, st, "gdn_chunk_fwd_stages")


def gdn_chunk_state_slots(n_seqs: int, total_tokens: int, h_qk: int, h_v: int,
                          d_k: int = 128, d_v: int = 128) -> int:
    lib = load_library()
    dims = make_dims(n_seqs, total_tokens, h_qk, h_v, d_k, d_v)
    out = ctypes.c_int64(0)
    _check(lib, lib.gdn_chunk_state_slots(ctypes.byref(dims), ctypes.byref(out)), "gdn_chunk_state_slots")
    return int(out.value)


def gdn_chunk_fwd_snapshots(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, chunk_states,
                            workspace, *, dims: Optional[gdn_dims] = None,
                            workspace_bytes: Optional[int] = None, stream=None) -> None:
    """Chunked prefill that also writes the state after every chunk (see include/gdn.h)."""
    lib = load_library()
    if dims is None:
        dims = _prefill_dims(q, v, cu_seqlens)
    _check_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace, dims, "gdn_chunk_fwd_snapshots")
    if not isinstance(chunk_states, int):
        import torch
        slots = gdn_chunk_state_slots(dims.n_seqs, dims.total_tokens, dims.n_heads_qk, dims.n_heads_v,
                                      dims.d_k, dims.d_v)
        _check_arg(chunk_states, "gdn_chunk_fwd_snapshots", "chunk_states", (torch.float32,),
                   (slots, dims.n_heads_v, dims.d_k, dims.d_v))
    workspace_bytes = _nbytes(workspace, workspace_bytes)
    st = lib.gdn_chunk_fwd_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                     _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(chunk_states),
                                     ctypes.byref(dims), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream, q, out, cu_seqlens))
    _check(lib, st, "gdn_chunk_fwd_snapshots")


def gdn_chunk_fwd_segmented_workspace_size(n_seqs: int, total_tokens: int, h_qk: int, h_v: int,
                                           segment_chunks: int, d_k: int = 128, d_v: int = 128) -> int:
    lib = load_library()
    dims = make_dims(n_seqs, total_tokens, h_qk, h_v, d_k, d_v)
    out = ctypes.c_size_t(0)
    _check(lib, lib.gdn_chunk_fwd_segmented_workspace_size(ctypes.byref(dims), int(segment_chunks),
                                                          ctypes.byref(out)),
           "gdn_chunk_fwd_segmented_workspace_size")
    return int(out.value)


def gdn_chunk_fwd_segmented(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, segment_chunks: int,
                            workspace, *, dims: Optional[gdn_dims] = None,
                            workspace_bytes: Optional[int] = None, stream=None) -> None:
    """Chunked prefill with the recurrence parallel over segments (see include/gdn.h)."""
    lib = load_library()
    if dims is None:
        dims = _prefill_dims(q, v, cu_seqlens)
    _check_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace, dims, "gdn_chunk_fwd_segmented")
    workspace_bytes = _nbytes(workspace, workspace_bytes)
    st = lib.gdn_chunk_fwd_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                     _ptr(initial_state), _ptr(out), _ptr(final_state), int(segment_chunks),
                                     ctypes.byref(dims), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream, q, out, cu_seqlens))
    _check(lib, st, "gdn_chunk_fwd_segmented")


def _recurrent_step_args(q, k, v, g, beta, n_requests, tokens_per_request, state_in, state_out, out,
                         intermediate_states, save_intermediate_states, dims):
    if dims is None:
        dims = _dims_from(q, v, n_requests, n_requests * tokens_per_request)
    import torch
    _check_tokens(q, k, v, g, beta, out, dims, "gdn_recurrent_step")
    state = (dims.n_seqs, dims.n_heads_v, dims.d_k, dims.d_v)
    _check_arg(state_in, "gdn_recurrent_step", "state_in", (torch.float32,), state)
    _check_arg(state_out, "gdn_recurrent_step", "state_out", (torch.float32,), state)
    _check_arg(intermediate_states, "gdn_recurrent_step", "intermediate_states", (torch.float32,),
               (dims.n_seqs, tokens_per_request) + state[1:])
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), int(n_requests), int(tokens_per_request),
            _ptr(state_in), _ptr(state_out), _ptr(out), _ptr(intermediate_states),
            1 if save_intermediate_states else 0, ctypes.byref(dims))
    return args, dims


def gdn_recurrent_step(q, k, v, g, beta, n_requests: int, tokens_per_request: int,
                       state_in, state_out, out, intermediate_states, save_intermediate_states: bool,
                       *, dims: Optional[gdn_dims] = None, stream=None) -> None:
    """Per-token update for decode / speculative verify (see include/gdn.h)."""
    lib = load_library()
    args, _ = _recurrent_step_args(q, k, v, g, beta, n_requests, tokens_per_request, state_in, state_out, out,
                                   intermediate_states, save_intermediate_states, dims)
    st = lib.gdn_recurrent_step(*args, _stream(stream, q, state_in, out))
    _check(lib, st, "gdn_recurrent_step")


class Prepared:
    """One entry point's call with its arguments checked and marshalled once.

    For a serving loop that reuses the same buffers, writing each step's
    token inputs into them in place: calling the object enqueues the step on
    `stream` (a torch stream or a raw handle), or on the current stream of
    the buffers' device, with no tensor checks, so that the host cost of an
    eager step is the library call alone.  The buffers must stay alive, on
    their device, with their shapes; the object keeps references to them."""

    __slots__ = ("_lib", "_fn", "_args", "_device", "_what", "_keep")

    def __init__(self, lib, fn, args, device, what, keep):
        self._lib, self._fn, self._args, self._device, self._what, self._keep = lib, fn, args, device, what, keep

    def __call__(self, stream=None) -> None:
        if stream is None:
            if self._device is None:
                raise GDNError(GDN_ERR_INVALID_VALUE, f"{self._what}: raw addresses need an explicit stream")
            handle = _current_stream(self._device)
        else:
            handle = stream if isinstance(stream, int) else stream.cuda_stream
        st = self._fn(*self._args, handle)
        if st != GDN_SUCCESS:
            _check(self._lib, st, self._what)


def _current_stream(device: int) -> int:
    """The current stream's handle without building a Stream object (0.1
    instead of 2 us per call; the same handle, also inside
    torch.cuda.stream(...) and graph capture)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device)
    return torch.cuda.current_stream(device).cuda_stream


def _device_of(*tensors) -> Optional[int]:
    for t in tensors:
        if t is not None and not isinstance(t, int):
            return t.get_device()
    return None


def prepare_recurrent_step(q, k, v, g, beta, n_requests: int, tokens_per_request: int,
                           state_in, state_out, out, intermediate_states, save_intermediate_states: bool,
                           *, dims: Optional[gdn_dims] = None) -> Prepared:
    """gdn_recurrent_step with its arguments checked once (see Prepared)."""
    lib = load_library()
    args, dims = _recurrent_step_args(q, k, v, g, beta, n_requests, tokens_per_request, state_in, state_out, out,
                                      intermediate_states, save_intermediate_states, dims)
    keep = (q, k, v, g, beta, state_in, state_out, out, intermediate_states, dims)
    return Prepared(lib, lib.gdn_recurrent_step, args, _device_of(q, state_in, out), "gdn_recurrent_step", keep)


def _state_dtype(pool) -> int:
    import torch
    if pool.dtype == torch.float32:
        return GDN_STATE_F32
    if pool.dtype == torch.float16:
        return GDN_STATE_F16
    raise GDNError(GDN_ERR_INVALID_VALUE, f"state pool dtype {pool.dtype} is neither float32 nor float16")


def _recurrent_step_slots_args(q, k, v, g, beta, cu_tokens, n_requests, max_tokens, state_pool, slot_table,
                               num_accepted, out, state_dtype, pool_slots, dims):
    if dims is None:
        dims = _dims_from(q, v, n_requests, q.shape[0])
    if state_dtype is None:
        state_dtype = _state_dtype(state_pool)
    if pool_slots is None:
        pool_slots = state_pool.shape[0]
    import torch
    _check_tokens(q, k, v, g, beta, out, dims, "gdn_recurrent_step_slots")
    i32 = (torch.int32,)
    _check_arg(cu_tokens, "gdn_recurrent_step_slots", "cu_tokens", i32, (dims.n_seqs + 1,))
    _check_arg(state_pool, "gdn_recurrent_step_slots", "state_pool",
               (torch.float16,) if state_dtype == GDN_STATE_F16 else (torch.float32,),
               (pool_slots, dims.n_heads_v, dims.d_k, dims.d_v))
    _check_arg(slot_table, "gdn_recurrent_step_slots", "slot_table", i32, (dims.n_seqs, int(max_tokens) + 1))
    _check_arg(num_accepted, "gdn_recurrent_step_slots", "num_accepted", i32, (dims.n_seqs,))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_tokens),
            int(n_requests), int(max_tokens), _ptr(state_pool), int(state_dtype),
            int(pool_slots), _ptr(slot_table), _ptr(num_accepted), _ptr(out), ctypes.byref(dims))
    return args, dims


def gdn_recurrent_step_slots(q, k, v, g, beta, cu_tokens, n_requests: int, max_tokens: int,
                             state_pool, slot_table, num_accepted, out, *,
                             state_dtype: Optional[int] = None, pool_slots: Optional[int] = None,
                             dims: Optional[gdn_dims] = None, stream=None) -> None:
    """Per-token update over a pool of state slots (see include/gdn.h).

    ``state_pool`` is a float32 or float16 tensor [pool_slots, H_v, d_k, d_v];
    ``slot_table`` int32 [R, max_tokens + 1]; ``num_accepted`` int32 [R] or None.
    """
    lib = load_library()
    args, _ = _recurrent_step_slots_args(q, k, v, g, beta, cu_tokens, n_requests, max_tokens, state_pool,
                                         slot_table, num_accepted, out, state_dtype, pool_slots, dims)
    st = lib.gdn_recurrent_step_slots(*args, _stream(stream, q, state_pool, out))
    _check(lib, st, "gdn_recurrent_step_slots")


def prepare_recurrent_step_slots(q, k, v, g, beta, cu_tokens, n_requests: int, max_tokens: int,
                                 state_pool, slot_table, num_accepted, out, *,
                                 state_dtype: Optional[int] = None, pool_slots: Optional[int] = None,
                                 dims: Optional[gdn_dims] = None) -> Prepared:
    """gdn_recurrent_step_slots with its arguments checked once (see Prepared)."""
    lib = load_library()
    args, dims = _recurrent_step_slots_args(q, k, v, g, beta, cu_tokens, n_requests, max_tokens, state_pool,
                                            slot_table, num_accepted, out, state_dtype, pool_slots, dims)
    keep = (q, k, v, g, beta, cu_tokens, state_pool, slot_table, num_accepted, out, dims)
    return Prepared(lib, lib.gdn_recurrent_step_slots, args, _device_of(q, state_pool, out),
                    "gdn_recurrent_step_slots", keep)


def _host_ptr(a):
    """Address of a C-contiguous numpy array (None stays NULL)."""
    if a is None:
        return None
    import numpy as np
    if not isinstance(a, np.ndarray) or not a.flags.c_contiguous:
        raise GDNError(GDN_ERR_INVALID_VALUE, "host checks take C-contiguous numpy arrays")
    return a.ctypes.data


def _host_bits(x):
    """bf16 operands as their uint16 bit patterns (numpy uint16, or float32 holding bf16 values)."""
    import numpy as np
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x
    if x.dtype == np.float32:
        return np.ascontiguousarray((x.view(np.uint32) >> 16).astype(np.uint16))
    raise GDNError(GDN_ERR_INVALID_VALUE, f"bf16 operand dtype {x.dtype} is neither uint16 bits nor float32")


def gdn_check_chunk_inputs_host(q, k, v, g, beta, cu_seqlens, initial_state, *, h_qk: int, h_v: int,
                                d_k: int = 128, d_v: int = 128) -> None:
    """Device-content preconditions of the prefill on host arrays (raises GDNError).
    q, k, v: uint16 bf16 bits or float32 bf16 values; g, beta float32; cu_seqlens int32."""
    import numpy as np
    lib = load_library()
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    dims = make_dims(cu.shape[0] - 1, int(cu[-1]) if cu.size else 0, h_qk, h_v, d_k, d_v)
    bq, bk, bv = _host_bits(q), _host_bits(k), _host_bits(v)
    g = None if g is None else np.ascontiguousarray(g, np.float32)
    beta = None if beta is None else np.ascontiguousarray(beta, np.float32)
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, np.float32)
    st = lib.gdn_check_chunk_inputs_host(_host_ptr(bq), _host_ptr(bk), _host_ptr(bv), _host_ptr(g),
                                         _host_ptr(beta), _host_ptr(cu), _host_ptr(s0), ctypes.byref(dims))
    _check(lib, st, "gdn_check_chunk_inputs_host")


def gdn_check_step_inputs_host(q, k, v, g, beta, state_in, *, n_requests: int, h_qk: int, h_v: int,
                               d_k: int = 128, d_v: int = 128) -> None:
    """Device-content preconditions of the recurrent steps on host arrays (raises GDNError)."""
    import numpy as np
    lib = load_library()
    bq, bk, bv = _host_bits(q), _host_bits(k), _host_bits(v)
    T = 0 if bq is None else bq.shape[0]
    dims = make_dims(n_requests, T, h_qk, h_v, d_k, d_v)
    g = None if g is None else np.ascontiguousarray(g, np.float32)
    beta = None if beta is None else np.ascontiguousarray(beta, np.float32)
    s = None if state_in is None else np.ascontiguousarray(state_in, np.float32)
    n_states = 0 if s is None else s.shape[0]
    st = lib.gdn_check_step_inputs_host(_host_ptr(bq), _host_ptr(bk), _host_ptr(bv), _host_ptr(g),
                                        _host_ptr(beta), _host_ptr(s), int(n_states), ctypes.byref(dims))
    _check(lib, st, "gdn_check_step_inputs_host")
