"""The LoRA-only optimizer step (oracle side).  Test infrastructure only; see
the package docstring.

Sources on the page "QLoRA: Efficient Finetuning of Quantized LLMs":
  section 3 "Paged Optimizers": the optimizer states live in memory that can
      be evicted to CPU RAM and paged back for the update step;
  Appendix B.2 "Hyperparameters": Adam beta2 = 0.999, maximum gradient norm
      0.3 and a constant learning rate; only the LoRA parameters are trained
      (section 3 "QLoRA", the paragraph after Eq. (6)).

Reading G16: "Adam" with decoupled weight decay (AdamW, the usual optimizer
for this fine-tuning) and global gradient-norm clipping over all LoRA
gradients:
    scale = min(1, max_norm / (||g||_2 + 1e-6))
    g'    = scale * g
    m     = beta1 m + (1 - beta1) g'
    v     = beta2 v + (1 - beta2) g'^2
    p     = p * (1 - lr * wd)                      (decoupled weight decay)
    p     = p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
at step t = 1, 2, ...  Every operation here is fp64.  Where the states live
(device memory or host memory) does not change the arithmetic.
"""

import numpy as np


def clip_scale(grads, max_norm):
    """min(1, max_norm / (||g||_2 + 1e-6)) over the concatenation of all
    gradient arrays, in fp64."""
    total = np.sqrt(sum(float(np.sum(np.asarray(g, dtype=np.float64) ** 2)) for g in grads))
    return min(1.0, max_norm / (total + 1e-6))


def adamw_step(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay, scale=1.0):
    """One AdamW update (G16) of parameters p with gradient g (times the clip
    scale) and states m, v; step counts from 1.  Returns new (p, m, v) in
    fp64 and leaves the inputs untouched."""
    p, g, m, v = (np.asarray(a, dtype=np.float64) for a in (p, g, m, v))
    g = g * scale
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    p = p * (1.0 - lr * weight_decay)
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    p = p - lr * mh / (np.sqrt(vh) + eps)
    return p, m, v
