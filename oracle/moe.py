"""Routed MoE layer, written out plainly -- TEST INFRASTRUCTURE ONLY.

What the layer computes (bloomery issue #967, section 2 "Checkpoint facts":
top-6 routing over 128 experts, ungated ReLU^2 experts, width 2688, expert
width 1856; section 3: experts have only up and down parts; audio.cpp port
notes, section "CPU weight offload": router, expert activation and routing
weights are separate fixed formulas):

  l_t   = x_t . W_r^T + b                         (x bf16, W_r and b fp32)
  S_t   = the 6 largest l_t,e (ties -> lower expert index)
  g_t,e = exp(l_t,e) / sum_{e' in S_t} exp(l_t,e')   (softmax renormalised
                                                   over the selected experts)
  h     = W_up,e . x~_t                           (2688 -> 1856)
  a     = bf16(relu(h)^2)
  y_t   = sum_{j=0..5} g_t,j * (W_down,e_j . a~_t,j)   (1856 -> 2688)

x~ and a~ are the activations as the weight format quantises them (identity
for BF16; per-tensor E4M3 for FP8 W8A8; NVFP4 blocks for W4A4, see
oracle.codecs), W the dequantised stored weights.  Sums are float64.

Parity status:
  route            pinned: brute-force subset enumeration, W_r = 0 closed form,
                   gate sum and shift invariance (tests/test_oracle.py)
  forward          pinned: identity experts (bit-exact closed form), scaled
                   identity per expert (gate/index placement), textbook
                   single-expert FFN by per-token loops, dense masked sum over
                   all experts, linearity in the gates, expert relabelling
  quantised paths  pinned through the codec pins, and by a per-token, per-slot
                   loop over hand-dequantised operands for both halves: x
                   quantised as one tensor, each expert projection on its own,
                   the stacked intermediate [T*k, F] as one tensor (a loop that
                   quantised it per expert, or not at all, fails the pin)
  shared_expert    pinned: per-token textbook loop (bf16) and hand-dequantised
                   loop with its own intermediate tensor scale (fp8, nvfp4);
                   identity weights bit-exact; block = routed + shared
  prenorm/stack    prenorm pinned by closed form on constant rows; the stack
                   is composition only (the pre-norm is a reading: the literal residual
                   stack without normalisation diverges within a few layers)
"""
from __future__ import annotations

import numpy as np

from . import codecs

NEAR_TIE = 1e-5


# --------------------------------------------------------------------------- router
def route(x, w_r, bias, k: int):
    """Top-k routing.  Returns (ids int32 [T,k], gates float64 [T,k],
    gap float64 [T] = l_(k) - l_(k+1), logits float64 [T,E]).

    Ids are ordered by (logit descending, index ascending)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_r, dtype=np.float64)
    logits = x @ w.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("route: need 1 <= k <= E")
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k]
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel[:, :1])
    gates = z / z.sum(axis=1, keepdims=True)
    if k < E:
        kth = sel[:, k - 1]
        nxt = np.take_along_axis(logits, order[:, k:k + 1], axis=1)[:, 0]
        gap = kth - nxt
    else:
        gap = np.full(T, np.inf)
    return ids.astype(np.int32), gates, gap, logits


# --------------------------------------------------------------------------- experts
class ExpertBank:
    """Dequantised expert weights of one layer, produced one expert at a time.

    `up_bf16` [E, F, H] and `down_bf16` [E, H, F] are torch bf16 CPU tensors
    (or float arrays holding bf16 values).  For "fp8" and "nvfp4" the oracle
    quantises each expert projection itself (oracle.codecs recipes)."""

    def __init__(self, up_bf16, down_bf16, fmt: str = "bf16"):
        if fmt not in ("bf16", "fp8", "nvfp4"):
            raise ValueError(fmt)
        self.fmt = fmt
        self._up = up_bf16
        self._down = down_bf16
        self._pre = {}

    @staticmethod
    def _f64(t):
        if hasattr(t, "float"):
            return t.float().numpy().astype(np.float64)
        return np.asarray(t, dtype=np.float64)

    def _deq(self, w):
        w = self._f64(w)
        if self.fmt == "bf16":
            return w
        if self.fmt == "fp8":
            q, s = codecs.fp8_quantize(w)
            return codecs.fp8_dequantize(q, s)
        q, sb, S = codecs.nvfp4_quantize(w)
        return codecs.nvfp4_dequantize(q, sb, S)

    def up(self, e: int) -> np.ndarray:
        """Dequantised W_up of expert e, float64 [F, H]."""
        if ("up", e) in self._pre:
            return self._pre[("up", e)]
        return self._deq(self._up[e])

    def down(self, e: int) -> np.ndarray:
        """Dequantised W_down of expert e, float64 [H, F]."""
        if ("down", e) in self._pre:
            return self._pre[("down", e)]
        return self._deq(self._down[e])

    def preload(self, experts, threads: int = 8):
        """Dequantise the given experts up front on a thread pool (the same
        arithmetic as up()/down(); used by tests to save wall time)."""
        from concurrent.futures import ThreadPoolExecutor
        jobs = [(kind, int(e)) for e in experts for kind in ("up", "down")]

        def one(job):
            kind, e = job
            src = self._up if kind == "up" else self._down
            return job, self._deq(src[e])

        with ThreadPoolExecutor(max(1, threads)) as ex:
            for job, arr in ex.map(one, jobs):
                self._pre[job] = arr
        return self


def quantise_activation(v, fmt: str) -> np.ndarray:
    """The activation a projection consumes: identity for bf16, per-tensor
    fake quantisation (quantise then dequantise) for fp8 / nvfp4."""
    v = np.asarray(v, dtype=np.float64)
    if fmt == "bf16":
        return v
    if fmt == "fp8":
        q, s = codecs.fp8_quantize(v)
        return codecs.fp8_dequantize(q, s)
    if fmt == "nvfp4":
        q, sb, S = codecs.nvfp4_quantize(v)
        return codecs.nvfp4_dequantize(q, sb, S)
    raise ValueError(fmt)


def forward(x, ids, gates, bank: ExpertBank, return_a: bool = False):
    """Expert part of the layer for given routing.  Returns y float64 [T, H]
    (and the bf16 intermediate a [T*k, F] in flat (token, slot) order)."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    gates = np.asarray(gates, dtype=np.float64)
    T, H = x.shape
    k = ids.shape[1] if ids.ndim == 2 else 0
    if T == 0:
        return (np.zeros((0, H)), None) if return_a else np.zeros((0, H))
    xq = quantise_activation(x, bank.fmt)
    flat_e = ids.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    experts = np.unique(flat_e)

    F = None
    a = None
    for e in experts:
        rows = np.nonzero(flat_e == e)[0]
        w_up = bank.up(int(e))
        if a is None:
            F = w_up.shape[0]
            a = np.zeros((T * k, F))
        h = xq[flat_t[rows]] @ w_up.T
        a[rows] = codecs.bf16_rne(np.maximum(h, 0.0) ** 2)
    aq = quantise_activation(a, bank.fmt)

    o = np.zeros((T * k, H))
    for e in experts:
        rows = np.nonzero(flat_e == e)[0]
        o[rows] = aq[rows] @ bank.down(int(e)).T
    y = np.zeros((T, H))
    og = o.reshape(T, k, H)
    for j in range(k):
        y += gates[:, j:j + 1] * og[:, j, :]
    return (y, a) if return_a else y


def layer(x, w_r, bias, bank: ExpertBank, k: int):
    """Route then run the experts: y float64 [T, H], plus the routing."""
    ids, gates, gap, _ = route(x, w_r, bias, k)
    return forward(x, ids, gates, bank), ids, gates, gap


# --------------------------------------------------------------------------- shared expert
def shared_expert(x, up, down, fmt: str = "bf16"):
    """Shared expert beside the routed ones: one ungated ReLU^2 FFN applied
    to every token with weight 1, y_s,t = W_down,s . a~_t with
    a = bf16(relu(W_up,s . x~_t)^2).  In the quantised formats its activations
    are quantised like a routed expert's: x~ per tensor over all of x, a~ per
    tensor over its own intermediate [T, F_s] (a tensor of its own, apart
    from the routed intermediate).  up bf16 [F_s, H], down bf16 [H, F_s].
    The pages keep shared experts on the card beside the routed ones and give
    no width for them (bloomery issue #967, section 4 "Placement on card,
    host RAM and NVMe"); the width is the caller's."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    ids = np.zeros((T, 1), np.int32)
    return forward(x, ids, np.ones((T, 1)), ExpertBank(up[None], down[None], fmt))


def block(x, w_r, bias, bank: ExpertBank, shared_up, shared_down, k: int):
    """The MoE block: routed layer plus the shared expert, y = y_routed + y_s."""
    y, ids, gates, gap = layer(x, w_r, bias, bank, k)
    return y + shared_expert(x, shared_up, shared_down, bank.fmt), ids, gates, gap


# --------------------------------------------------------------------------- stacked path
def prenorm(x, eps: float = 1e-6) -> np.ndarray:
    """Weightless RMS pre-norm of each row, rounded to bf16 (stacked-path reading)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return codecs.bf16_rne(x / r)


def residual_add(x, y) -> np.ndarray:
    """x <- bf16(x + y)."""
    return codecs.bf16_rne(np.asarray(x, dtype=np.float64) + np.asarray(y, dtype=np.float64))
