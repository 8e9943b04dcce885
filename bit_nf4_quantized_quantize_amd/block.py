"""A LLaMA-shaped decoder block with QLoRA adapters on all seven linear
layers, for measuring what a whole layer costs in memory and time.

QLoRA (Dettmers et al., arXiv 2305.14314) puts adapters on every network
layer (introduction). Section 2 "Memory Requirement of Parameter-Efficient
Finetuning" finds that activation gradients, not LoRA parameters, dominate
training memory, and that gradient checkpointing shrinks them. Appendix G
"Memory Footprint" (Figure 6) measures with batch 1, sequence length 512 and
checkpointing.

The block is the pre-norm LLaMA layer without rotary encoding:
    n1 = rmsnorm(x) g1;  h = x + L_o(attn(L_q(n1), L_k(n1), L_v(n1)))
    n2 = rmsnorm(h) g2;  y = h + L_down(silu(L_gate(n2)) * L_up(n2))
Every L is the library's frozen-NF4 linear with a LoRA adapter, run through
qlora_linear_fwd / qlora_linear_bwd on bf16 operands. The glue around them
(rmsnorm, causal attention, SiLU, residuals) is the surrounding model, not
part of the layer, and runs as plain fp32 torch ops. Only the adapters and
the block input receive gradients. With checkpoint=True the forward keeps
only the block input for the backward and runs again inside it.
"""

import math

import torch
import torch.utils.checkpoint

from . import binding as B

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
EPS = 1e-6


def linear_shapes(hidden, mlp):
    """[out, in] weight shape of each linear."""
    return {"q": (hidden, hidden), "k": (hidden, hidden), "v": (hidden, hidden), "o": (hidden, hidden),
            "gate": (mlp, hidden), "up": (mlp, hidden), "down": (hidden, mlp)}


class _QLoraLinearFn(torch.autograd.Function):
    """Y = X W_bf16^T + s (X A) B on the library's kernels; the backward
    returns dX, dA, dB (no dW)."""

    @staticmethod
    def forward(ctx, X, A, Bm, lin):
        Y, XA = B.qlora_linear_fwd(X, lin.qw, A, Bm, lin.s)
        ctx.save_for_backward(X, XA, A, Bm)
        ctx.lin = lin
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, XA, A, Bm = ctx.saved_tensors
        lin = ctx.lin
        dX, dA, dB = B.qlora_linear_bwd(dY.contiguous(), X, XA, lin.qw, A, Bm, lin.s)
        return dX, dA, dB, None


class QLoraLinear:
    """One frozen NF4 (+ double quantisation) weight with a bf16 LoRA adapter
    (A [in, r], B [r, out], both leaves with requires_grad)."""

    def __init__(self, W, A, Bm, s):
        self.qw = B.qlora_nf4_quantize(W.contiguous(), double_quant=True)
        self.out_features, self.in_features = W.shape
        self.A = A.to(torch.bfloat16).contiguous().requires_grad_(True)
        self.B = Bm.to(torch.bfloat16).contiguous().requires_grad_(True)
        self.s = float(s)

    def __call__(self, z):
        """z: fp32 [..., in] -> fp32 [..., out] (bf16 at the layer boundary)."""
        lead = z.shape[:-1]
        X = z.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        Y = _QLoraLinearFn.apply(X, self.A, self.B, self)
        return Y.float().reshape(*lead, self.out_features)

    def storage_bytes(self):
        return sum(self.qw.sizes.values())


def rms_norm(z, g):
    return z * torch.rsqrt(torch.mean(z * z, dim=-1, keepdim=True) + EPS) * g


def causal_attention(q, k, v, heads):
    """softmax(q k^T / sqrt(d)) v per sequence and head, causal; fp32.
    q, k, v: [batch, seq, hidden]."""
    b, t, hd = q.shape
    d = hd // heads

    def split(z):
        return z.reshape(b, t, heads, d).permute(0, 2, 1, 3).contiguous()

    qh, kh, vh = split(q), split(k), split(v)
    scores = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) / math.sqrt(d)
    future = torch.triu(torch.ones(t, t, dtype=torch.bool, device=q.device), diagonal=1)
    p = torch.softmax(scores.masked_fill(future, float("-inf")), dim=-1)
    return torch.matmul(p, vh).permute(0, 2, 1, 3).reshape(b, t, hd)


class QLoraBlock:
    """The decoder block above.  `W`, `A`, `Bm`: dicts by linear name of fp32
    device tensors (W [out, in]); g1, g2: fp32 [hidden] norm gains; s =
    alpha / r."""

    def __init__(self, W, A, Bm, g1, g2, s, heads):
        self.lin = {n: QLoraLinear(W[n], A[n], Bm[n], s) for n in LINEARS}
        self.g1, self.g2 = g1.float(), g2.float()
        self.heads = int(heads)
        self.hidden = W["q"].shape[1]

    def parameters(self):
        """The trainable tensors: every adapter's A and B."""
        out = []
        for n in LINEARS:
            out += [self.lin[n].A, self.lin[n].B]
        return out

    def _forward(self, x):
        L = self.lin
        n1 = rms_norm(x, self.g1)
        a = causal_attention(L["q"](n1), L["k"](n1), L["v"](n1), self.heads)
        h = x + L["o"](a)
        n2 = rms_norm(h, self.g2)
        return h + L["down"](torch.nn.functional.silu(L["gate"](n2)) * L["up"](n2))

    def __call__(self, x, checkpoint=False):
        """x: fp32 [batch, seq, hidden] -> y (same shape)."""
        if x.shape[-1] != self.hidden:
            raise ValueError(f"x must end in the hidden size {self.hidden}")
        if checkpoint:
            return torch.utils.checkpoint.checkpoint(self._forward, x, use_reentrant=False)
        return self._forward(x)

    def weight_bytes(self):
        """HBM bytes of the seven quantised weights (codes and constants)."""
        return sum(self.lin[n].storage_bytes() for n in LINEARS)

    def adapter_bytes(self):
        """HBM bytes of the bf16 adapters."""
        return sum(p.numel() * p.element_size() for p in self.parameters())
