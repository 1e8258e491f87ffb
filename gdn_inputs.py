"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module only draws random tensors and rounds them to the storage
precision; it holds none of the layer's arithmetic, so both the CPU oracle
and the HIP path can be fed from it without sharing any computation.

Recipe (every tensor comes from its own child stream of
``numpy.random.SeedSequence(seed)``, so changing one size never shifts the
draws of another):

* q, k ~ N(0, 1), L2-normalised per token and head.  q is then multiplied by
  1/sqrt(d_k); k keeps unit norm so that (I - beta k k^T) is a contraction.
  With ``k_scale=True`` k is scaled by 1/sqrt(d_k) as well (the alternative
  reading of "q,k scaled"), kept as an option for robustness tests.
* v ~ N(0, 1).
* beta = sigmoid(N(0, 1)).
* g = -softplus(N(mu_g, 1)) (natural-log decay, alpha = exp(g) in (0, 1)).
  mu_g = 0 for the standard workloads, -2 for the long-context one.
* initial states ~ N(0, state_std^2) in fp32, or None.
* q, k, v are rounded to bfloat16 (round to nearest even) unless the
  workload is fp32; the rounded values are what both sides consume.

The pages that describe the layer (the "2080 Ti runs Qwen3.8-27B: a vLLM
plugin" page, section 2 on the GDN prefill) give one workload: one layer at
4000 tokens.  The sizes below restate the workloads this library is measured
on; nothing here comes from a public dataset.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CHUNK = 64


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16-exact; call bf16_round first")
    return (u >> 16).astype(np.uint16)


@dataclasses.dataclass
class GDNInputs:
    """One packed batch.  Token-major layouts, d_v contiguous in states."""

    name: str
    q: np.ndarray            # [T, H_qk, d_k] float32 (bf16-exact unless fp32 workload)
    k: np.ndarray            # [T, H_qk, d_k]
    v: np.ndarray            # [T, H_v, d_v]
    g: np.ndarray            # [T, H_v] float32, natural-log decay (<= 0)
    beta: np.ndarray         # [T, H_v] float32
    cu_seqlens: np.ndarray   # [N + 1] int32
    initial_state: Optional[np.ndarray]  # [N, H_v, d_k, d_v] float32 or None
    bf16: bool               # q, k, v are bfloat16-exact

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def h_qk(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_v(self) -> int:
        return int(self.v.shape[1])

    @property
    def d_k(self) -> int:
        return int(self.q.shape[2])

    @property
    def d_v(self) -> int:
        return int(self.v.shape[2])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    def slice_seq(self, n: int) -> "GDNInputs":
        """The n-th sequence as a batch of its own."""
        a, b = int(self.cu_seqlens[n]), int(self.cu_seqlens[n + 1])
        s0 = None if self.initial_state is None else self.initial_state[n:n + 1].copy()
        return GDNInputs(f"{self.name}[{n}]", self.q[a:b].copy(), self.k[a:b].copy(),
                         self.v[a:b].copy(), self.g[a:b].copy(), self.beta[a:b].copy(),
                         np.array([0, b - a], np.int32), s0, self.bf16)


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def make_inputs(lengths, h_qk: int, h_v: int, d_k: int, d_v: int, *, seed: int = 0,
                bf16: bool = True, g_mean: float = 0.0, state_std: Optional[float] = None,
                k_scale: bool = False, name: str = "custom") -> GDNInputs:
    """Draw one packed batch with the recipe in the module docstring."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if np.any(lengths < 0):
        raise ValueError("negative sequence length")
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    if cu[-1] >= 2**31:
        raise ValueError("too many tokens for int32 cu_seqlens")
    T = int(cu[-1])
    n = len(lengths)
    rq, rk, rv, rb, rg, rs = _streams(seed, 6)
    q = rq.standard_normal((T, h_qk, d_k), dtype=np.float32)
    k = rk.standard_normal((T, h_qk, d_k), dtype=np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q *= np.float32(1.0 / np.sqrt(d_k))
    if k_scale:
        k *= np.float32(1.0 / np.sqrt(d_k))
    v = rv.standard_normal((T, h_v, d_v), dtype=np.float32)
    beta = _sigmoid(rb.standard_normal((T, h_v), dtype=np.float32)).astype(np.float32)
    g = (-_softplus(rg.standard_normal((T, h_v), dtype=np.float32) + np.float32(g_mean))).astype(np.float32)
    s0 = None
    if state_std is not None:
        s0 = (rs.standard_normal((n, h_v, d_k, d_v), dtype=np.float32) * np.float32(state_std)).astype(np.float32)
    if bf16:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return GDNInputs(name, q, k, v, g, beta, cu.astype(np.int32), s0, bf16)


# ---------------------------------------------------------------------------
# Named workloads.
# ---------------------------------------------------------------------------

def tiny(seed: int = 0) -> GDNInputs:
    """1 sequence, T=128, 1 head, d_k=d_v=32, fp32 inputs, zero initial state (2 chunks)."""
    return make_inputs([128], 1, 1, 32, 32, seed=seed, bf16=False, name="tiny_T128_d32")


def prefill_4000(seed: int = 0) -> GDNInputs:
    """One layer prefill: 1 sequence, T=4000, 32 value heads / 16 q-k heads, d=128, bf16."""
    return make_inputs([4000], 16, 32, 128, 128, seed=seed, name="prefill_T4000_hv32_hqk16_d128")


def varlen_lengths(seed: int = 0, n: int = 8, lo: int = 512, hi: int = 4096) -> np.ndarray:
    """Sequence lengths uniform on the integers [lo, hi], inclusive."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 8]))
    return rng.integers(lo, hi, size=n, endpoint=True)


def varlen_8(seed: int = 0) -> GDNInputs:
    """8 packed sequences, lengths U{512..4096}, nonzero initial states N(0, 0.02^2)."""
    return make_inputs(varlen_lengths(seed), 16, 32, 128, 128, seed=seed, state_std=0.02,
                       name="varlen_8seq_512to4096_hv32_hqk16_d128")


def long_131072(seed: int = 0) -> GDNInputs:
    """1 sequence, T=131072, slow decay g = -softplus(N(-2, 1))."""
    return make_inputs([131072], 16, 32, 128, 128, seed=seed, g_mean=-2.0,
                       name="long_T131072_hv32_hqk16_d128")


def verify_8x6(seed: int = 0) -> GDNInputs:
    """Speculative verify: 8 requests x (1+5) tokens, states N(0, 0.02^2)."""
    return make_inputs([6] * 8, 16, 32, 128, 128, seed=seed, state_std=0.02,
                       name="verify_8req_6tok_hv32_hqk16_d128")


def slow_decay(T: int = 4000, seed: int = 0) -> GDNInputs:
    """Stress set for the inter-chunk path: alpha ~ 0.993 (g = -softplus(N(-5, 1)))."""
    return make_inputs([T], 16, 32, 128, 128, seed=seed, g_mean=-5.0, state_std=0.02,
                       name=f"slow_decay_T{T}")


def no_decay_small_beta(T: int = 4000, seed: int = 0) -> GDNInputs:
    """Stress set: alpha == 1 (g == 0) and beta ~ U(0, 0.1)."""
    x = make_inputs([T], 16, 32, 128, 128, seed=seed, state_std=0.02, name=f"nodecay_T{T}")
    rb = np.random.default_rng(np.random.SeedSequence([seed, 99]))
    x.g[:] = 0.0
    x.beta[:] = rb.uniform(0.0, 0.1, size=x.beta.shape).astype(np.float32)
    return x


def slot_table_contiguous(n_requests: int, max_tokens: int, first_write_slot: int,
                          read_slots=None) -> np.ndarray:
    """Slot table [R, max_tokens + 1] (int32): request r reads slot read_slots[r]
    (default r) and stores the state after token t in slot
    first_write_slot + r * max_tokens + t."""
    table = np.empty((n_requests, max_tokens + 1), np.int32)
    table[:, 0] = np.arange(n_requests) if read_slots is None else read_slots
    for r in range(n_requests):
        table[r, 1:] = first_write_slot + r * max_tokens + np.arange(max_tokens)
    return table


def state_pool(x: GDNInputs, extra_slots: int, *, f16: bool = False, seed: int = 0) -> np.ndarray:
    """Pool [N + extra_slots, H_v, d_k, d_v]: slots 0..N-1 hold x.initial_state,
    the rest distinct N(0, 0.02^2) fill (so a wrong read shows).  float16 pools
    hold the fp16 rounding of those values."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    fill = rng.normal(0.0, 0.02, size=(extra_slots,) + x.initial_state.shape[1:]).astype(np.float32)
    pool = np.concatenate([x.initial_state, fill], axis=0)
    return pool.astype(np.float16) if f16 else pool


def verify_variable(lengths, seed: int = 0) -> GDNInputs:
    """Verify tokens with a variable count per request (accepted length varies)."""
    return make_inputs(list(lengths), 16, 32, 128, 128, seed=seed, state_std=0.02,
                       name="verify_var_" + "_".join(str(int(n)) for n in lengths))


WORKLOADS = {
    "tiny": tiny,
    "prefill_4000": prefill_4000,
    "varlen_8": varlen_8,
    "long_131072": long_131072,
    "verify_8x6": verify_8x6,
}
