"""A decoder block with QLoRA adapters on every linear layer (oracle side).
Test infrastructure only; see the package docstring.

Sources on the page "QLoRA: Efficient Finetuning of Quantized LLMs":
  the introduction: QLoRA puts adapters on every network layer (the seven
      linear layers of a LLaMA block: the attention projections q, k, v, o
      and the MLP projections gate, up, down);
  section 2 "Memory Requirement of Parameter-Efficient Finetuning": most of
      the memory goes to activation gradients, not to the LoRA parameters,
      and gradient checkpointing shrinks them;
  Appendix G "Memory Footprint" (Figure 6): batch 1, sequence length 512,
      gradient checkpointing.

Reading G18: the page fine-tunes LLaMA but does not spell out its block.
The block is the usual pre-norm LLaMA layer without the rotary position
encoding (which touches neither the weights nor the adapters):
    n1 = rmsnorm(x) * g1
    a  = softmax_causal(q k^T / sqrt(d)) v      per sequence and head,
         q = L_q(n1), k = L_k(n1), v = L_v(n1)
    h  = x + L_o(a)
    n2 = rmsnorm(h) * g2
    y  = h + L_down(silu(L_gate(n2)) * L_up(n2))
with rmsnorm(z) = z / sqrt(mean(z^2) + eps) over the hidden dimension and
every L a QLoRA linear of Eq. (5), L(X) = X W^T + s (X A) B with W the BF16
dequantised weight (Eq. 6).  Only the adapters A, B and the block input x
get gradients (the norm gains and W are frozen).  Everything is fp64; the
backward is torch.autograd over this forward, pinned by finite differences.
"""

import math

import numpy as np
import torch

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
EPS = 1e-6


def shapes(hidden, mlp):
    """[out, in] shape of each linear's weight (reading G11)."""
    return {"q": (hidden, hidden), "k": (hidden, hidden), "v": (hidden, hidden), "o": (hidden, hidden),
            "gate": (mlp, hidden), "up": (mlp, hidden), "down": (hidden, mlp)}


def rms_norm(z, g):
    return z / torch.sqrt(torch.mean(z * z, dim=-1, keepdim=True) + EPS) * g


def causal_attention(q, k, v, heads):
    """softmax(q k^T / sqrt(d)) v over each sequence and head, position t
    attending to positions <= t.  q, k, v: [batch, seq, hidden]."""
    b, t, hd = q.shape
    d = hd // heads

    def split(z):
        return z.reshape(b, t, heads, d).permute(0, 2, 1, 3)  # [b, heads, t, d]

    qh, kh, vh = split(q), split(k), split(v)
    scores = qh @ kh.transpose(-1, -2) / math.sqrt(d)
    future = torch.triu(torch.ones(t, t, dtype=torch.bool), diagonal=1)
    scores = scores.masked_fill(future, float("-inf"))
    p = torch.softmax(scores, dim=-1)
    return (p @ vh).permute(0, 2, 1, 3).reshape(b, t, hd)


def qlora_linear(X, W, A, B, s):
    """Eq. (5) on fp64 tensors: X [..., K], W [N, K], A [K, r], B [r, N]."""
    return X @ W.T + s * ((X @ A) @ B)


def forward(x, W, A, B, g1, g2, s, heads):
    """The block of reading G18.  x [batch, seq, hidden]; W, A, B: dicts by
    linear name (W the BF16 dequantised weights as values).  Returns y."""
    def L(name, X):
        return qlora_linear(X, W[name], A[name], B[name], s)

    n1 = rms_norm(x, g1)
    a = causal_attention(L("q", n1), L("k", n1), L("v", n1), heads)
    h = x + L("o", a)
    n2 = rms_norm(h, g2)
    return h + L("down", torch.nn.functional.silu(L("gate", n2)) * L("up", n2))


def forward_backward(x, W, A, B, g1, g2, s, heads, dy):
    """y and the gradients of sum(dy * y) for x and every A, B (fp64).
    Inputs are numpy arrays or tensors; returns numpy arrays:
    (y, dx, {name: dA}, {name: dB})."""
    t = lambda a, grad=False: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=grad)  # noqa: E731
    xt = t(x, True)
    At = {n: t(A[n], True) for n in LINEARS}
    Bt = {n: t(B[n], True) for n in LINEARS}
    Wt = {n: t(W[n]) for n in LINEARS}
    y = forward(xt, Wt, At, Bt, t(g1), t(g2), s, heads)
    (y * t(dy)).sum().backward()
    return (y.detach().numpy(), xt.grad.numpy(), {n: At[n].grad.numpy() for n in LINEARS},
            {n: Bt[n].grad.numpy() for n in LINEARS})
