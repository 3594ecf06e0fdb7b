"""Calibration capture: the inputs X and output gradients G of a decoder block's linear layers.

The KronQ pages accumulate H_X from the calibration activations, as GPTQ does, and H_G from
the gradients of the layer outputs, which one backward pass supplies (the wmrh.cn KronQ
article, sections 二 and 三; the gptget.net summaries, Methodology and 方法论). This module
produces both for a LLaMA-shaped decoder block with seeded random weights (no trained
weights, no dataset): the
block runs forward on seeded token states and back once from a seeded linear loss, and every
linear layer's input rows and output-gradient rows are kept in bfloat16, ready for
kq_accumulate_cov. Layers that read the same tensor share one X (q, k and v read the
attention input; gate and up read the MLP input), which is why the input side of BiIP is keyed
by input group.

The block is float32 torch, causal attention without rotary embeddings, RMSNorm with unit
weights, SwiGLU MLP: it is the step before the quantization path, not part of it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

# input group of each linear layer, and the layers in block order
GROUP_OF = {"q_proj": "attn_in", "k_proj": "attn_in", "v_proj": "attn_in", "o_proj": "o_in",
            "gate_proj": "mlp_in", "up_proj": "mlp_in", "down_proj": "down_in"}
LAYERS = list(GROUP_OF)


@dataclass
class BlockShape:
    d: int          # model width
    heads: int
    d_ff: int       # MLP width

    @property
    def dims(self) -> Dict[str, tuple]:
        """(dout, din) of every linear layer."""
        d, f = self.d, self.d_ff
        return {"q_proj": (d, d), "k_proj": (d, d), "v_proj": (d, d), "o_proj": (d, d),
                "gate_proj": (f, d), "up_proj": (f, d), "down_proj": (d, f)}


LLAMA2_7B = BlockShape(d=4096, heads=32, d_ff=11008)


@dataclass
class Captured:
    """X[group] [N, din] and G[layer] [N, dout], bfloat16, on the block's device."""
    x: Dict[str, object] = field(default_factory=dict)
    g: Dict[str, object] = field(default_factory=dict)
    tokens: int = 0


def block_weights(shape: BlockShape, seed: int, device, dtype):
    """Seeded N(0, 0.02²) weights [dout, din] of every linear layer."""
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    w = {}
    for name in LAYERS:
        dout, din = shape.dims[name]
        w[name] = (torch.randn((dout, din), generator=gen, dtype=torch.float32) * 0.02).to(device=device, dtype=dtype)
    return w


def _rmsnorm(h, eps: float = 1e-5):
    import torch
    return h * torch.rsqrt(h.pow(2).mean(-1, keepdim=True) + eps)


def block_forward(h, w, shape: BlockShape, hook=None):
    """One decoder block on h [b, s, d]; hook(name, input, output) sees every linear layer."""
    import torch
    import torch.nn.functional as F

    def lin(name, x):
        y = x @ w[name].t()
        if hook is not None:
            hook(name, x, y)
        return y

    b, s, d = h.shape
    dh = d // shape.heads
    a = _rmsnorm(h)
    q = lin("q_proj", a).view(b, s, shape.heads, dh).transpose(1, 2)
    k = lin("k_proj", a).view(b, s, shape.heads, dh).transpose(1, 2)
    v = lin("v_proj", a).view(b, s, shape.heads, dh).transpose(1, 2)
    att = (q @ k.transpose(-1, -2).contiguous()) / (dh ** 0.5)
    mask = torch.ones((s, s), dtype=torch.bool, device=h.device).triu(1)
    att = att.masked_fill(mask, float("-inf")).softmax(-1)
    ctx = (att @ v.contiguous()).transpose(1, 2).reshape(b, s, d)
    h2 = h + lin("o_proj", ctx)
    m = _rmsnorm(h2)
    return h2 + lin("down_proj", F.silu(lin("gate_proj", m)) * lin("up_proj", m))


def token_states(n_seq: int, seq: int, d: int, seed: int, device, dtype):
    """Seeded block inputs: N(0, 1) entries times a lognormal(0, 1.5) scale per channel."""
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    scale = torch.exp(torch.randn(d, generator=gen) * 1.5)
    h = torch.randn((n_seq, seq, d), generator=gen) * scale
    return h.to(device=device, dtype=dtype)


def loss_direction(n_seq: int, seq: int, d: int, seed: int, device, dtype):
    """R of the loss L = sum(out * R) / N, seeded N(0, 1)."""
    import torch
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed + 1)
    return torch.randn((n_seq, seq, d), generator=gen).to(device=device, dtype=dtype)


def block_inputs(shape: BlockShape, n_seq: int, seq: int, seed: int, device, dtype=None):
    """(token states, loss direction R) [n_seq, seq, d] for ``capture``, drawn on the host."""
    import torch
    dtype = torch.float32 if dtype is None else dtype
    return (token_states(n_seq, seq, shape.d, seed, device, dtype),
            loss_direction(n_seq, seq, shape.d, seed, device, dtype))


def capture(shape: BlockShape, n_seq: int, seq: int, *, seed: int = 0, device="cpu", dtype=None,
            micro_batch: Optional[int] = None, weights=None, inputs=None) -> Captured:
    """Forward and one backward pass of the block over n_seq sequences of `seq` tokens, in
    micro-batches of sequences; returns X and G of every linear layer as bfloat16 [N, .].
    ``weights`` and ``inputs`` (from ``block_weights`` / ``block_inputs``) default to the
    seeded draws of ``seed``."""
    import torch
    dtype = torch.float32 if dtype is None else dtype
    w = block_weights(shape, seed, device, dtype) if weights is None else weights
    n = n_seq * seq
    out = Captured(tokens=n)
    for name in LAYERS:
        dout, din = shape.dims[name]
        grp = GROUP_OF[name]
        if grp not in out.x:
            out.x[grp] = torch.empty((n, din), dtype=torch.bfloat16, device=device)
        out.g[name] = torch.empty((n, dout), dtype=torch.bfloat16, device=device)
    mb = n_seq if micro_batch is None else micro_batch
    h_all, r_all = block_inputs(shape, n_seq, seq, seed, device, dtype) if inputs is None else inputs
    for s0 in range(0, n_seq, mb):
        s1 = min(n_seq, s0 + mb)
        rows = slice(s0 * seq, s1 * seq)

        def hook(name, x, y, rows=rows):
            grp = GROUP_OF[name]
            if name in ("q_proj", "gate_proj") or GROUP_OF[name] in ("o_in", "down_in"):
                out.x[grp][rows] = x.detach().reshape(-1, x.shape[-1]).to(torch.bfloat16)

            def keep_grad(gy, name=name):
                out.g[name][rows] = gy.reshape(-1, gy.shape[-1]).to(torch.bfloat16)
            y.register_hook(keep_grad)

        h = h_all[s0:s1].detach().requires_grad_(True)  # gradients flow back through every layer
        y = block_forward(h, w, shape, hook)
        loss = (y * r_all[s0:s1]).sum() / n
        loss.backward()
    return out
