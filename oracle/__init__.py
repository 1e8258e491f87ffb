"""CPU oracle for the Gated DeltaNet layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and it
never imports the HIP library: the two share no code.

* ``forward`` -- the plain token-by-token gated delta rule (C, ``gdn_oracle.c``),
  in fp64 or fp32, threaded over (sequence, value head).
* ``chunked.chunked_forward`` -- a naive chunkwise form in numpy fp64, a
  second, independently derived formulation used to pin the first.

Both take plain numpy arrays; see ``gdn_oracle.c`` for layouts.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gdn.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (host only)."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    global _lib
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    for suffix in ("f64", "f32"):
        fn = getattr(lib, f"gdn_oracle_forward_{suffix}")
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_int32]
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, g, beta, cu_seqlens, initial_state=None, *, precision: str = "f64",
            record_states: bool = False, n_threads: Optional[int] = None
            ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Run the token recurrence.

    Returns (out [T,H_v,d_v], final_state [N,H_v,d_k,d_v], token_states or None),
    where token_states[t] is the state right after token t ([T,H_v,d_k,d_v]).
    """
    real = {"f64": np.float64, "f32": np.float32}[precision]
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    g = np.ascontiguousarray(g, np.float32)
    beta = np.ascontiguousarray(beta, np.float32)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n = cu.shape[0] - 1
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, h_v) or beta.shape != (T, h_v):
        raise ValueError("inconsistent input shapes")
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, real)
        if s0.shape != (n, h_v, d_k, d_v):
            raise ValueError("initial_state shape")
    out = np.zeros((T, h_v, d_v), real)
    fin = np.zeros((n, h_v, d_k, d_v), real)
    states = np.zeros((T, h_v, d_k, d_v), real) if record_states else None
    if n_threads is None:
        n_threads = min(os.cpu_count() or 1, max(1, n * h_v))
    fn = getattr(_load(), f"gdn_oracle_forward_{precision}")
    rc = fn(T, n, _ptr(cu), h_qk, h_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(s0), _ptr(out), _ptr(fin), _ptr(states), int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, fin, states


def forward_inputs(x, **kw):
    """``forward`` on an object with q, k, v, g, beta, cu_seqlens, initial_state fields."""
    return forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, **kw)
