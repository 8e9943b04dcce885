"""QLoRA linear layer forward and backward (oracle side).  Test
infrastructure only; see the package docstring.

Sources on the page "QLoRA: Efficient Finetuning of Quantized LLMs":
  section 2 "Low-rank Adapters", Eq. (3): Y = XW + s X L1 L2 with
      L1 in R^{h x r}, L2 in R^{r x o}, s a scalar;
  section 3 "QLoRA", Eq. (5): the same with W replaced by
      doubleDequant(c1, c2, W^NF4) = W^BF16 (Eq. 6), every operand in BF16;
  section 3 "QLoRA", the paragraph after Eq. (6): only dE/dL_i is needed,
      not dE/dW, but the input gradient still flows through W dequantised to
      BF16.

Notation: the weight is stored [out, in] = [N, K] (reading G11), so with
X [M, K], L1 = A [K, r], L2 = B [r, N]:
    Y  = X W^T + s (X A) B                           [M, N]
and for an upstream gradient dY [M, N]:
    T  = dY B^T                                      [M, r]
    dX = dY W + s T A^T                              [M, K]
    dA = s X^T T                                     [K, r]
    dB = s (X A)^T dY                                [r, N]
There is no dW.

Reading G3: s = alpha / r (the page's LoRA reference; Eq. (5) drops s).
Reading G10: every product here is taken in fp64 from the exact BF16 input
values and the BF16 dequantised weight; the GPU side is held to a tolerance
against these.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(X, W_bf16, A, B, s):
    """Eq. (5).  X [M,K], W_bf16 [N,K] (the BF16 weight of Eq. 6, as values),
    A [K,r], B [r,N].  Returns (Y [M,N], XA [M,r]) in fp64."""
    X, W, A, B = _f64(X), _f64(W_bf16), _f64(A), _f64(B)
    XA = X @ A
    Y = X @ W.T + s * (XA @ B)
    return Y, XA


def backward(dY, X, W_bf16, A, B, s):
    """Gradients of Eq. (5) for the adapters and the input; no dW.
    Returns (dX [M,K], dA [K,r], dB [r,N]) in fp64."""
    dY, X, W, A, B = _f64(dY), _f64(X), _f64(W_bf16), _f64(A), _f64(B)
    T = dY @ B.T
    dX = dY @ W + s * (T @ A.T)
    dA = s * (X.T @ T)
    dB = s * ((X @ A).T @ dY)
    return dX, dA, dB


# ------------------------------------------------------------ LoRA dropout
# Appendix B.2 ("Hyperparameters") trains with LoRA dropout 0.1 (models up to
# 13B) or 0.05 (33B, 65B) but does not say where it acts.  Reading G15: the
# usual LoRA dropout on the adapter's input, with the inverted scaling that
# keeps its expectation,
#     Y  = X W^T + s (drop(X) A) B,   drop(X) = X * keep / (1 - p),
# where keep [M, K] is a Bernoulli(1 - p) mask drawn by the caller (an input
# here, so both sides see the same draws).  Its gradients:
#     T  = dY B^T
#     dX = dY W + s (T A^T) * keep / (1 - p)
#     dA = s drop(X)^T T
#     dB = s (drop(X) A)^T dY
# and the saved XA is drop(X) A.

def forward_dropout(X, W_bf16, A, B, s, keep, p):
    """Eq. (5) with LoRA dropout on the adapter input (G15).  keep: bool or
    0/1 array [M, K]; p: drop probability in [0, 1).  Returns (Y, XA)."""
    X, W, A, B = _f64(X), _f64(W_bf16), _f64(A), _f64(B)
    Xd = X * _f64(keep) / (1.0 - p)
    XA = Xd @ A
    Y = X @ W.T + s * (XA @ B)
    return Y, XA


def backward_dropout(dY, X, W_bf16, A, B, s, keep, p):
    """Gradients of forward_dropout for the adapters and the input (G15).
    Returns (dX, dA, dB) in fp64."""
    dY, X, W, A, B = _f64(dY), _f64(X), _f64(W_bf16), _f64(A), _f64(B)
    kp = _f64(keep) / (1.0 - p)
    Xd = X * kp
    T = dY @ B.T
    dX = dY @ W + s * (T @ A.T) * kp
    dA = s * (Xd.T @ T)
    dB = s * ((Xd @ A).T @ dY)
    return dX, dA, dB


def flops(M, N, K, r):
    """Algorithmic flops of one forward plus one backward (no dW)."""
    return 4 * M * N * K + 6 * M * r * (K + N)


def rel_l2(out, ref):
    """||out - ref||_2 / ||ref||_2 in fp64 (0 when both are zero)."""
    out, ref = _f64(out), _f64(ref)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(out - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
