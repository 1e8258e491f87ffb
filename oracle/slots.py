"""Slot-pool semantics of the per-token update -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.

The "Qwen3.8-27B on one RTX 3090" page keeps a fixed-size recurrent state per
request, stored in fp16 (section "Exploiter l'architecture hybride"), plus
eight speculative state slots per request (section on the 131,072-token
limit) so that a verify pass can roll back to the state after the last
accepted draft token.  The "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page
verifies 1 + K query tokens per request.

``slots_step`` states that bookkeeping plainly: for each request, gather its
incoming state from the pool, run the token recurrence of ``oracle.forward``
over its tokens, and scatter the state after every token to the slot the
table names, rounded to the pool's storage type.  All reads see the pool as
it was before the call.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from . import forward


def slots_step(q, k, v, g, beta, cu_tokens, pool: np.ndarray, slot_table, num_accepted=None, *,
               precision: str = "f64") -> Tuple[np.ndarray, np.ndarray]:
    """One verify / decode call over a pool of state slots.

    q, k [T, H_qk, d_k]; v [T, H_v, d_v]; g, beta [T, H_v]; cu_tokens [R + 1];
    pool [P, H_v, d_k, d_v] (float32 or float16: the stored values);
    slot_table [R, max_tokens + 1]: column 0 (or column num_accepted[r]) is the
    incoming slot, column 1 + t receives the state after token t (negative:
    not stored).  Returns (out [T, H_v, d_v] float64, new pool of pool's dtype).

    Index handling follows the library's documented contract: a request whose
    token range is outside [0, T) or longer than max_tokens is skipped; one
    whose incoming column or slot, or any write slot, is outside the table or
    pool gets NaN outputs and no state change.
    """
    cu = np.asarray(cu_tokens, np.int64)
    table = np.asarray(slot_table, np.int64)
    n_req = cu.shape[0] - 1
    T, h_v, d_v = v.shape
    max_tok = table.shape[1] - 1
    n_pool = pool.shape[0]
    out = np.zeros((T, h_v, d_v), np.float64)
    new_pool = pool.copy()
    for r in range(n_req):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        if t0 < 0 or t1 < t0 or t1 > T or t1 - t0 > max_tok:
            continue
        n = t1 - t0
        col = 0 if num_accepted is None else int(num_accepted[r])
        src = int(table[r, col]) if 0 <= col <= max_tok else -1
        dst = [int(table[r, 1 + t]) for t in range(n)]
        if not (0 <= src < n_pool) or any(s >= n_pool for s in dst):
            out[t0:t1] = np.nan
            continue
        s_in = pool[src].astype(np.float64)[None]
        o, _, states = forward(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1],
                               np.array([0, n], np.int32), s_in, precision=precision,
                               record_states=True)
        out[t0:t1] = o
        for t, s in enumerate(dst):
            if s >= 0:
                new_pool[s] = states[t].astype(pool.dtype)   # fp16: one rounding, to nearest even
    return out, new_pool

