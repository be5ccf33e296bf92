"""Float64 CPU oracle of the true-sequential block driver.

TEST INFRASTRUCTURE. Only the test suite may import this module; the product path never imports,
links or runs anything here, and this module imports nothing from the product.

What it follows:

* GPTQ tools page (ozercemkelahmet.com/tools/gptq), "How it works", Step 9: the layers of a block
  are solved one after another, and with true-sequential ordering the attention projections go
  first and the inputs of the later layers are recomputed through the layers already quantized.
* "GPTQ Quantization: Complete Technical Guide", the quantize-config listing (true_sequential) and
  the section "True Sequential": a setting that trades time for accuracy by quantizing layers in
  order. (Its cost comparison is garbled and is not used.)

Readings (the pages name the order, not the block):

* The block is a pre-norm decoder block with the layer names the pages use (q/k/v/o, gate/up/down):
  x_a = RMSNorm(X); attention o_in = softmax_causal(Q K^T / sqrt(dh)) V per head with
  Q = x_a Wq^T, K = x_a Wk^T, V = x_a Wv^T; h1 = X + o_in Wo^T; x_m = RMSNorm(h1);
  down_in = silu(x_m Wg^T) * (x_m Wu^T); out = h1 + down_in Wd^T. RMSNorm has no learned weight
  (y = x / sqrt(mean(x^2) + eps)); there is no positional rotation.
* The stages are (q, k, v) <- x_a, (o) <- o_in, (gate, up) <- x_m, (down) <- down_in. Layers of a
  stage share the stage's Hessian, damping and processing order.
* true_sequential=False takes every stage input from one forward pass with the original weights.
  Either way the block output is recomputed through the quantized weights.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from . import gptq_ref as ref

LAYERS = ("q", "k", "v", "o", "gate", "up", "down")
STAGES = ((0, 1, 2), (3,), (4, 5), (6,))


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """Each row divided by the root of its mean square plus eps."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seqs: int, seq_len: int, heads: int) -> np.ndarray:
    """Per sequence and head: P = softmax over j <= i of (q_i . k_j) / sqrt(dh), output P V."""
    n, hidden = q.shape
    dh = hidden // heads
    out = np.zeros((n, hidden))
    mask = np.triu(np.ones((seq_len, seq_len), dtype=bool), 1)     # True where j > i
    for s in range(seqs):
        r = slice(s * seq_len, (s + 1) * seq_len)
        for h in range(heads):
            c = slice(h * dh, (h + 1) * dh)
            S = q[r, c] @ k[r, c].T / np.sqrt(dh)
            S[mask] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[r, c] = P @ v[r, c]
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


@dataclass
class BlockShape:
    hidden: int
    heads: int
    inter: int
    seqs: int
    seq_len: int
    eps: float = 1e-6


def forward(X: np.ndarray, W: Sequence[np.ndarray], sh: BlockShape) -> dict:
    """The block's forward pass; returns the four stage inputs and the output."""
    X = np.asarray(X, dtype=np.float64)
    xa = rmsnorm(X, sh.eps)
    q, k, v = (xa @ W[i].T for i in range(3))
    o_in = causal_attention(q, k, v, sh.seqs, sh.seq_len, sh.heads)
    h1 = X + o_in @ W[3].T
    xm = rmsnorm(h1, sh.eps)
    down_in = silu(xm @ W[4].T) * (xm @ W[5].T)
    out = h1 + down_in @ W[6].T
    return dict(inputs=[xa, o_in, xm, down_in], out=out)


@dataclass
class BlockResult:
    layers: List[ref.LayerResult]
    hessians: List[np.ndarray]
    out: np.ndarray


def quantize_block(X: np.ndarray, W: Sequence[np.ndarray], sh: BlockShape, bits: int, group_size: int,
                   block_size: int, act_order: bool = False, damp: float = 0.01, true_sequential: bool = True,
                   **kw) -> BlockResult:
    """Solves the block's layers stage by stage (tools page, Step 9). kw goes to gptq_ref.gptq."""
    W = [np.asarray(w, dtype=np.float64) for w in W]
    cur = list(W)                       # weights the stage inputs are computed with
    layers: List[Optional[ref.LayerResult]] = [None] * 7
    hessians = []
    base = None if true_sequential else forward(X, W, sh)["inputs"]
    for si, members in enumerate(STAGES):
        A = forward(X, cur, sh)["inputs"][si] if true_sequential else base[si]
        H, n = ref.hessian([A])
        hessians.append(H)
        for i in members:
            layers[i] = ref.gptq(W[i], None, bits, group_size, block_size, act_order=act_order, damp=damp, H=H, n=n,
                                 **kw)
            cur[i] = layers[i].quant.Q
    Wq = [lr.quant.Q for lr in layers]
    return BlockResult(layers=layers, hessians=hessians, out=forward(X, Wq, sh)["out"])
