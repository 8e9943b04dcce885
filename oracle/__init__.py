"""Plain CPU oracle for the QLoRA frozen-NF4 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, table or helper
with the HIP library; the two meet only at the seeded inputs the tests feed to
both.

Every function follows a passage of the page "QLoRA: Efficient Finetuning of
Quantized LLMs" (Dettmers, Pagnoni, Holtzman, Zettlemoyer; arXiv 2305.14314),
read in its Chinese translation at aiingo.vercel.app/paper/paper-2305-14314.
Citations below name that page's section, equation or appendix.  Where the
page leaves a step open, the reading taken is stated in the docstring and
tagged G<n>; the same tags are listed with their justification in the
project's design notes.

Precision: floating-point steps that decide a stored integer (an NF4 code, an
FP8 byte) are taken in IEEE fp32 with round-to-nearest-even, one rounding per
operation and no fused multiply-add, because that is the precision the stored
format fixes.  Matrix products are taken in fp64.

Parity status of each function (what pins it to something other than itself
is in tests/test_oracle_pins.py):
  codebook.NF4                 pinned (Appendix E values, quantile derivation)
  fp8_e4m3.*                   pinned (format definition, torch float8_e4m3fn)
  blockwise.nearest_code       pinned (brute force, Eq. 1 Int8 special case)
  blockwise.quantize_nf4       pinned (round trips, brute force, closed forms)
  blockwise.exact_mean_f32     pinned (rational arithmetic, closed forms)
  blockwise.double_quantize    bit layout "parity unpinned" by the pages (the
                               FP8 variant and where the mean lives are not
                               printed); its size is pinned by the bits/param
                               closed form of section 3 and its arithmetic by
                               the round-trip special cases
  blockwise.dequantize         pinned (round trips)
  codebook.FP4_E2M1 / FP4_E3M0 pinned (format tables), INT4 pinned (two's
                               complement over 7), INT8 pinned (each value the
                               exact-rational nearest fp32 to k / 127)
  blockwise.nearest_level,
  blockwise.quantize_4bit      pinned (brute force at every decision point,
                               Eq. 1 rounding for Int4 and Int8, round trips,
                               equality with the NF4 quantiser, NF4 lowest
                               error on normal weights)
  linear.forward / backward    pinned (brute force, finite differences,
                               special cases, torch.autograd in fp64)
  optim.clip_scale /
  optim.adamw_step             pinned (torch.optim.AdamW and clip_grad_norm_
                               in fp64 over five steps, closed forms)
  block.forward /
  block.forward_backward       pinned (attention against torch's causal
                               scaled-dot-product attention and causality,
                               rmsnorm scale invariance, identity with W = B
                               = 0, Eq. 5 linears, finite differences of dx,
                               dA, dB)
  linear.forward_dropout /
  linear.backward_dropout      pinned (reduction to the plain layer, brute
                               force, finite differences, torch.autograd in
                               fp64 with the mask as a tensor)
  dropout_rng.*                pinned (numpy.random.Philox, the bit
                               generator numpy ships for Philox4x64-10;
                               per-element evaluation of the mask layout;
                               exact threshold; binomial keep rate)
"""

from . import codebook, fp8_e4m3, blockwise, linear, optim, dropout_rng  # noqa: F401
