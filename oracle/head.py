"""The attentive-pool classifier head, written as its plain definition in float64.

TEST INFRASTRUCTURE (see the package docstring).  numpy's matmul is the only
library primitive; the encoder's own oracle functions supply the blocks.

The V-JEPA 2 SSv2 card (opening paragraph) and the benchmarks page
("Attentive-pool head" table and its note) describe the head only as three
self-attention blocks over the tokens, one cross-attention query, an MLP and
a linear layer giving the 174 class scores.  Readings (R13):
  * The head reads the encoder's final-LayerNorm token map (every token,
    CLS included when the model has one).
  * Its self-attention blocks are the encoder's pre-LN block (tensors
    head.blk.{i}.*), bidirectional, without position terms.
  * The cross-attention block holds one learned query token q0.  The tokens
    are layer-normalised (head.xattn.ln1) and projected to keys and values;
    q0 itself is projected to the query without a LayerNorm.  Attention is
    multi-head with the encoder's heads, scale 1/sqrt(head_dim).  Then
    x = q0 + out_proj(attention), and x += MLP(LN2 x) with the erf GELU.
  * The classifier is a linear layer on x, with no LayerNorm before it.
"""
from __future__ import annotations

import numpy as np

from oracle.encoder import attention_head, block, gelu, layer_norm, linear


def cross_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, heads: int) -> np.ndarray:
    """One query row q [D] against the keys k and values v [N, D] of one item,
    head by head (each the plain softmax(q_h k_h^T / sqrt(dh)) v_h)."""
    D = q.shape[0]
    dh = D // heads
    out = np.empty(D)
    for a in range(heads):
        sl = slice(a * dh, (a + 1) * dh)
        out[sl] = attention_head(q[None, sl], k[:, sl], v[:, sl], None)[0]
    return out


def classify(dims: dict, w: dict, y: np.ndarray) -> np.ndarray:
    """Final token map y [B, N, D] -> class scores [B, C] (R13)."""
    eps = dims["ln_eps"]
    x = y
    for i in range(dims["head_blocks"]):
        x = block(dims, w, i, x, None, prefix="head.blk.", rotary=False)
    p = "head.xattn."
    h = layer_norm(x, w[p + "ln1.weight"], w[p + "ln1.bias"], eps)
    k = linear(h, w[p + "attn_k.weight"], w[p + "attn_k.bias"])
    v = linear(h, w[p + "attn_v.weight"], w[p + "attn_v.bias"])
    q0 = w["head.query_token"]
    q = linear(q0[None], w[p + "attn_q.weight"], w[p + "attn_q.bias"])[0]
    o = np.stack([cross_attention(q, k[b], v[b], dims["heads"]) for b in range(y.shape[0])])
    xq = q0[None] + linear(o, w[p + "attn_out.weight"], w[p + "attn_out.bias"])
    u = gelu(linear(layer_norm(xq, w[p + "ln2.weight"], w[p + "ln2.bias"], eps),
                    w[p + "ffn_up.weight"], w[p + "ffn_up.bias"]))
    xq = xq + linear(u, w[p + "ffn_down.weight"], w[p + "ffn_down.bias"])
    return linear(xq, w["head.classifier.weight"], w["head.classifier.bias"])
