"""Helpers for GPU tests: move seeded inputs to the device and call the C ABI."""

import numpy as np
import torch

import hybrid_linear_attention_gdn_amd as gdn

OUT_TOL = 2e-3     # relative L2 on outputs (bf16 inputs, fp32 accumulation)
STATE_TOL = 1e-3   # relative L2 on states


ROW_TOL = 1e-2     # relative L2 of one boundary row (token, value head) over d_v


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


class DevInputs:
    def __init__(self, x, device="cuda"):
        self.x = x
        bf = torch.bfloat16
        self.q = torch.from_numpy(np.ascontiguousarray(x.q)).to(device=device, dtype=bf)
        self.k = torch.from_numpy(np.ascontiguousarray(x.k)).to(device=device, dtype=bf)
        self.v = torch.from_numpy(np.ascontiguousarray(x.v)).to(device=device, dtype=bf)
        self.g = torch.from_numpy(np.ascontiguousarray(x.g)).to(device)
        self.beta = torch.from_numpy(np.ascontiguousarray(x.beta)).to(device)
        self.cu = torch.from_numpy(np.ascontiguousarray(x.cu_seqlens)).to(device)
        self.s0 = None if x.initial_state is None else torch.from_numpy(x.initial_state).to(device)
        self.device = device


def workspace_for(x, device="cuda"):
    nbytes = gdn.gdn_chunk_fwd_workspace_size(x.n_seqs, x.total_tokens, x.h_qk, x.h_v)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def chunk_fwd(d: DevInputs, initial_state="default", want_final=True, workspace=None, poison=False):
    x = d.x
    s0 = d.s0 if isinstance(initial_state, str) else initial_state
    out = torch.empty((x.total_tokens, x.h_v, x.d_v), dtype=torch.float32, device=d.device)
    fin = (torch.empty((x.n_seqs, x.h_v, x.d_k, x.d_v), dtype=torch.float32, device=d.device)
           if want_final else None)
    ws = workspace if workspace is not None else workspace_for(x, d.device)
    if poison:
        out.fill_(float("nan"))
        if fin is not None:
            fin.fill_(float("nan"))
        ws.fill_(0xFF)   # fp16 NaN pattern
    gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.cu, s0, out, fin, ws)
    torch.cuda.synchronize()
    return out, fin


def recurrent_step(d: DevInputs, n_req, n_tok, save=True, state_out=True):
    x = d.x
    out = torch.empty((n_req * n_tok, x.h_v, x.d_v), dtype=torch.float32, device=d.device)
    inter = (torch.empty((n_req, n_tok, x.h_v, x.d_k, x.d_v), dtype=torch.float32, device=d.device)
             if save else None)
    s_out = (torch.empty((n_req, x.h_v, x.d_k, x.d_v), dtype=torch.float32, device=d.device)
             if state_out else None)
    gdn.gdn_recurrent_step(d.q, d.k, d.v, d.g, d.beta, n_req, n_tok, d.s0, s_out, out, inter, save)
    torch.cuda.synchronize()
    return out, s_out, inter


def head_errors(o, ro, cu):
    """Relative L2 per (sequence, value head) of outputs [T, H_v, d_v]; NaN for empty sequences."""
    cu = np.asarray(cu, np.int64)
    n, hv = len(cu) - 1, o.shape[1]
    err = np.full((n, hv), np.nan)
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        d = np.asarray(o[a:b], np.float64) - ro[a:b]
        num = np.sqrt((d * d).sum(axis=(0, 2)))
        den = np.sqrt((np.asarray(ro[a:b], np.float64) ** 2).sum(axis=(0, 2)))
        err[s] = num / np.where(den > 0, den, 1.0)
    return err


def boundary_rows(cu, chunk=64, head=16):
    """Token rows where sequence-boundary bugs live: each sequence's first
    `head` rows and every row of its last (possibly short) chunk."""
    rows = []
    cu = np.asarray(cu, np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        last = a + chunk * ((b - a - 1) // chunk)
        rows.append(np.arange(a, min(b, a + head)))
        rows.append(np.arange(last, b))
    return np.unique(np.concatenate(rows)) if rows else np.zeros(0, np.int64)


def row_errors(o, ro, rows):
    """Relative L2 of each (row, value head) over d_v, the denominator floored
    at a tenth of that head's RMS row norm over the rows checked (so rows with
    almost no signal cannot divide by ~0)."""
    a = np.asarray(o[rows], np.float64)
    b = np.asarray(ro[rows], np.float64)
    num = np.sqrt(((a - b) ** 2).sum(axis=2))
    nb = np.sqrt((b * b).sum(axis=2))
    floor = 0.1 * np.sqrt((nb * nb).mean(axis=0, keepdims=True))
    return num / np.maximum(nb, np.maximum(floor, 1e-30))


def check_detail(name, o, ro, f, rf, cu):
    """Gates finer than the whole-tensor one: every (sequence, value head) output
    and final state, and every boundary row (first rows and last chunk of
    each sequence), so that one wrong head or short chunk cannot hide in the
    bulk of a large tensor."""
    he = head_errors(o, ro, cu)
    worst = float(np.nanmax(he)) if np.isfinite(he).any() else 0.0
    n = len(cu) - 1
    fe = 0.0
    if f is not None:
        d = np.asarray(f, np.float64) - rf
        num = np.sqrt((d * d).reshape(n, f.shape[1], -1).sum(axis=2))
        den = np.sqrt((np.asarray(rf, np.float64) ** 2).reshape(n, f.shape[1], -1).sum(axis=2))
        fe = float((num / np.where(den > 0, den, 1.0)).max()) if n else 0.0
    rows = boundary_rows(cu)
    re = float(row_errors(o, ro, rows).max()) if len(rows) else 0.0
    print(f"[detail] {name}: worst (seq, head) out {worst:.3e} state {fe:.3e}; "
          f"worst boundary row {re:.3e} over {len(rows)} rows", flush=True)
    assert worst <= OUT_TOL, (name, "per-head output", worst)
    assert fe <= STATE_TOL, (name, "per-head state", fe)
    assert re <= ROW_TOL, (name, "boundary row", re)
