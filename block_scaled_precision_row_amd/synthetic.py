"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random tensors; it holds none of the quantization
arithmetic. Every tensor comes from its own NumPy generator seeded with
``[0, workload, tensor_id, block]``, so a tensor does not depend on what else
was drawn or in which order. Values are float32 standard normals scaled by
``sigma`` (a standard deviation), optionally with a set of outlier input
channels multiplied by ``outlier_gain``, and rounded once to bf16
(round-to-nearest-even) by PyTorch. Tensors are returned as uint16 bf16 bit
patterns.

Shapes follow the transformer the pages describe: a flow-matching image
generator whose joint blocks run qkv (N = 3 * 3072), attention-out
projection (3072), MLP-up (4 * 3072) and MLP-down (K = 12288) linears over
image tokens; a 1 MP image is 4096 tokens and a 4 MP image 16384 tokens
(16-pixel token grid), and text adds a few hundred tokens.
"""

import numpy as np
import torch

# workload ids (the second word of every seed)
TINY = 1          # X [64, 256], W [128, 256]: nvfp4 weight-only smoke shape
FP8R_4096 = 2     # X [4096, 3072] with 1 % outlier channels, W [3072, 3072]
NVFP4_UP = 3      # X [4096, 3072], W [12288, 3072]
SMALL_M = 4       # X [512, 3072], W [3072, 3072] and [12288, 3072]
JOINT_4MP = 5     # M = 16384, 28 joint blocks x {qkv, proj, up, down}

X_ID, W_ID, W2_ID = 0, 1, 2
WEIGHT_SIGMA = 0.02


def rng_for(workload, tensor_id, block=0):
    return np.random.default_rng([0, workload, tensor_id, block])


def _to_bf16_bits(z):
    t = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, workload, tensor_id, block=0, sigma=1.0, outlier_frac=0.0, outlier_gain=20.0):
    """bf16 bit patterns of N(0, sigma^2) float32 draws, with round(outlier_frac * K) columns x gain."""
    rng = rng_for(workload, tensor_id, block)
    z = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    n_out = int(round(outlier_frac * shape[-1]))
    if n_out:
        cols = rng.choice(shape[-1], n_out, replace=False)
        z[..., cols] *= np.float32(outlier_gain)
    return _to_bf16_bits(z)


def activations(workload, M, K, block=0):
    frac = 0.01 if workload == FP8R_4096 else 0.0
    return normal_bf16((M, K), workload, X_ID, block, 1.0, frac)


def weights(workload, N, K, block=0, tensor_id=W_ID):
    return normal_bf16((N, K), workload, tensor_id, block, WEIGHT_SIGMA)


# the joint block's four linears: (name, N, K)
JOINT_GEMMS = (("qkv", 9216, 3072), ("proj", 3072, 3072), ("up", 12288, 3072), ("down", 3072, 12288))
JOINT_BLOCKS = 28
JOINT_TOKENS = 16384


def joint_scheme(block):
    """Even joint blocks carry nvfp4 weights, odd ones fp8r."""
    return "nvfp4" if block % 2 == 0 else "fp8r"


# low-rank adapters (LoRA) on a linear of any workload: A [rank, K] ~ N(0, 1 / K) (unit-variance
# X A^T for unit-variance X), B [N, rank] ~ N(0, 0.02^2); their tensor ids follow the layer's
LORA_A_ID, LORA_B_ID = 3, 4
LORA_B_SIGMA = 0.02


def lora_adapter(workload, rank, N, K, block=0):
    """(A bits [rank, K], B bits [N, rank]) of a synthetic adapter on an N x K linear."""
    a = normal_bf16((rank, K), workload, LORA_A_ID, block, float(1.0 / np.sqrt(K)))
    b = normal_bf16((N, rank), workload, LORA_B_ID, block, LORA_B_SIGMA)
    return a, b
