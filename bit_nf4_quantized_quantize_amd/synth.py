"""Seeded synthetic inputs for the QLoRA NF4 linear workloads.

This module only draws random tensors; it holds none of the method's
arithmetic.  Tests feed the same tensors to the HIP library and (as host
copies) to the CPU oracle, and the benchmark draws its inputs here.

Distributions follow the workloads: weights ~ N(0, 0.02^2) (QLoRA Appendix F
on the near-normality of pretrained weights) or Student-t with nu = 5 scaled
to std 0.02 (outlier-heavy blocks); activations and upstream gradients
~ N(0, 1); LoRA factors ~ N(0, 0.01^2).  BF16 tensors are nearest-even casts
of fp32 draws.

Seeds: seed = (workload << 16) | (layer << 8) | tensor_id, with tensor ids
W 0, X 1, A 2, B 3, dY 4, H 5.
"""

import math

import torch

TENSOR_ID = {"W": 0, "X": 1, "A": 2, "B": 3, "dY": 4, "H": 5}


def seed_of(workload, layer, tensor):
    return (int(workload) << 16) | (int(layer) << 8) | TENSOR_ID[tensor]


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, device="cpu", dtype=torch.float32):
    """N(0, std^2) draw in fp32, then cast to `dtype`."""
    g = _gen(seed, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x if dtype == torch.float32 else x.to(dtype)


def student_t(shape, nu, std, seed, device="cpu", dtype=torch.float32):
    """Student-t(nu) draw scaled to standard deviation `std` (nu > 2):
    Z / sqrt(V / nu) with V the sum of nu squared standard normals."""
    nu = int(nu)
    g = _gen(seed, device)
    shape = tuple(shape)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(nu):
        e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v.addcmul_(e, e)
        del e
    v.div_(nu).sqrt_()
    z.div_(v)
    del v
    z.mul_(std / math.sqrt(nu / (nu - 2.0)))
    return z if dtype == torch.float32 else z.to(dtype)


def weight(shape, dist, seed, device="cpu"):
    """fp32 weight [out, in] for dist 'normal' or 't5'."""
    if dist == "normal":
        return normal(shape, 0.02, seed, device)
    if dist == "t5":
        return student_t(shape, 5, 0.02, seed, device)
    raise ValueError(dist)


class Linear:
    """Shapes and distributions of one QLoRA linear of a workload."""

    def __init__(self, workload, layer, M, N, K, r, alpha, dist, name):
        self.workload, self.layer = workload, layer
        self.M, self.N, self.K, self.r = M, N, K, r
        self.alpha, self.s = alpha, alpha / r
        self.dist, self.name = dist, name

    def draw(self, device="cpu", M=None, with_grad=True):
        """Draw W (fp32), X, A, B, dY (bf16) for this linear."""
        M = self.M if M is None else M
        w, l = self.workload, self.layer
        bf = torch.bfloat16
        out = {
            "W": weight((self.N, self.K), self.dist, seed_of(w, l, "W"), device),
            "X": normal((M, self.K), 1.0, seed_of(w, l, "X" if self.name != "down" else "H"), device, bf),
            "A": normal((self.K, self.r), 0.01, seed_of(w, l, "A"), device, bf),
            "B": normal((self.r, self.N), 0.01, seed_of(w, l, "B"), device, bf),
        }
        if with_grad:
            out["dY"] = normal((M, self.N), 1.0, seed_of(w, l, "dY"), device, bf)
        return out


def workload(index):
    """The linears of synthetic workload 1..5 (sizes as [out, in])."""
    if index == 1:   # tiny: 256x256, 16 tokens, rank 8, alpha 16
        return [Linear(1, 0, 16, 256, 256, 8, 16.0, "normal", "tiny")]
    if index == 2:   # 7B attention projection: 4096 tokens (4 x 1024)
        return [Linear(2, 0, 4096, 4096, 4096, 64, 16.0, "normal", "attn")]
    if index == 3:   # 7B MLP block: gate, up [11008, 4096], down [4096, 11008]; 2048 tokens
        return [Linear(3, 0, 2048, 11008, 4096, 64, 16.0, "normal", "gate"),
                Linear(3, 1, 2048, 11008, 4096, 64, 16.0, "normal", "up"),
                Linear(3, 2, 2048, 4096, 11008, 64, 16.0, "normal", "down")]
    if index == 4:   # 65B-shaped MLP, Student-t weights; 8192 tokens
        return [Linear(4, 0, 8192, 22016, 8192, 64, 16.0, "t5", "gate"),
                Linear(4, 1, 8192, 22016, 8192, 64, 16.0, "t5", "up"),
                Linear(4, 2, 8192, 8192, 22016, 64, 16.0, "t5", "down")]
    if index == 5:   # small-batch forward against the 65B-shaped down weight
        return [Linear(5, 0, m, 8192, 22016, 64, 16.0, "t5", "gemv") for m in (1, 4, 16)]
    raise ValueError(index)


def sweep_7b_shapes():
    """[out, in] shapes of the 32-layer 7B-shaped quantise/dequantise sweep:
    per layer four 4096x4096 attention projections, gate and up 11008x4096
    and down 4096x11008."""
    layer = [(4096, 4096)] * 4 + [(11008, 4096), (11008, 4096), (4096, 11008)]
    return [shape for _ in range(32) for shape in layer]


def sweep_weight(i, device="cpu"):
    """fp32 weight i (0..223) of the sweep, N(0, 0.02^2), seed of workload 5
    with layer slot 1 + i (slot 0 is the small-batch weight)."""
    return weight(sweep_7b_shapes()[i], "normal", seed_of(5, 1 + i, "W"), device)
