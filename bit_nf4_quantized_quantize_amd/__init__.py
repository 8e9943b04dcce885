"""MI355X (gfx950) QLoRA frozen-NF4 linear layer.

NF4 blockwise quantisation with double quantisation, dequantisation, and the
forward/backward of a linear layer with a LoRA adapter over the frozen NF4
weight, as hand-written HIP kernels behind the C ABI of include/qlora_nf4.h.
`binding` is the ctypes layer over that ABI; `build` compiles the library.
"""

from .binding import (  # noqa: F401
    NF4Weight,
    QLoraError,
    QLoraLibraryError,
    Workspace,
    qlora_linear_bwd,
    qlora_linear_fwd,
    qlora_linear_workspace,
    qlora_nf4_codebook,
    qlora_nf4_dequantize,
    qlora_nf4_quantize,
    qlora_nf4_quantize_workspace,
    qlora_nf4_storage_bytes,
)
