"""Oracle of the low-rank adapter (LoRA) side path on the quantized linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: the "FLUX 3 Image Klein vs Qwen-Image-2.1" page (overview of the two
models, the paragraph after the comparison table) and the FLUX 3 Image Klein
open-source release page (section three, the speed figures) both report that
running the quantized model with a LoRA attached costs about 5 % more
generation time. Neither page gives the adapter's arithmetic.

Reading taken (the plain one): the standard low-rank adapter on a linear layer,

    y = base(x) + s * B (A x),

with the down projection A [r][K] and the up projection B [N][r] stored in
bf16, the scale s (the adapter's alpha / r times its strength) an fp32 host
number, and the adapter fed the layer's unquantized bf16 activations. ``base``
is whatever the layer computes without the adapter (the fp8r or nvfp4 product,
or the bf16 fallback). Everything here is fp64 from exact bf16 values.

Pins (``tests/test_oracle_lora.py``): exact rational arithmetic on tiny shapes,
the merged-weight identity W x + s B (A x) = (W + s B A) x, a one-hot rank-1
case in closed form and the zero adapter.
"""

import numpy as np

from .codec import bf16_to_f64


def scale_f32(scale):
    """The adapter scale as the fp32 number the layer receives."""
    return np.float64(np.float32(scale))


def lora_down(x_bits, a_bits, scale):
    """Scaled rank-r projection T = s * X A^T [M][r] (fp64; X [M][K], A [r][K] as bf16 bits)."""
    x = bf16_to_f64(x_bits)
    a = bf16_to_f64(a_bits)
    return scale_f32(scale) * (x @ a.T)


def lora_delta(x_bits, a_bits, b_bits, scale):
    """The adapter's contribution s * (X A^T) B^T to Y [M][N] (B [N][r] as bf16 bits)."""
    return lora_down(x_bits, a_bits, scale) @ bf16_to_f64(b_bits).T


def lora_linear(base, x_bits, a_bits, b_bits, scale):
    """Y = base + s * (X A^T) B^T, with ``base`` the layer's fp64 output without the adapter."""
    return np.asarray(base, np.float64) + lora_delta(x_bits, a_bits, b_bits, scale)
