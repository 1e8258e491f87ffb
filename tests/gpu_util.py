"""Helpers for GPU tests: move seeded inputs to the device and call the C ABI."""

import numpy as np
import torch

import hybrid_linear_attention_gdn_amd as gdn

OUT_TOL = 2e-3     # relative L2 on outputs (bf16 inputs, fp32 accumulation)
STATE_TOL = 1e-3   # relative L2 on states


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
