"""CPU oracle for the block-scaled quantized linear layer (fp8r / nvfp4).

This package is TEST INFRASTRUCTURE ONLY. It is a plain, slow, obviously
correct fp64 NumPy statement of what the HIP path computes. Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product path never does, and the oracle imports nothing from the
product package (it shares no code, tables or helpers with the HIP kernels).

Sources, cited by page title and section:

* "BFL (fp8r / nvfp4)" (diffusers quantization docs), opening list of the two
  schemes: fp8r stores an E4M3 ``weight`` with one fp32 ``weight_scale`` per
  row and quantizes activations to E4M3 per row at run time; nvfp4 stores a
  packed E2M1 ``weight`` (two values per byte), E4M3 block scales over 16
  elements (``weight_scale``), an fp32 global ``weight_scale_2`` and a
  calibrated fp32 ``input_scale``.
* Same page, "Kernels" section: per-row scales applied around an fp8 GEMM,
  runtime nvfp4 quantization of the activations before an fp4 GEMM, and the
  fallback that dequantizes weights to the compute dtype and runs a plain
  linear with unquantized activations.
* "NVFP4 vs FP8 vs BF16" (FLUX.2-klein-4b-nvfp4 comparison), format overview
  and usage sections: a per-block scale factor is what separates NVFP4 from a
  plain 4-bit integer; PyTorch's packed dtype is ``float4_e2m1fn_x2``.
* "FLUX 3 Image Klein vs Qwen-Image-2.1" (model overview) and the FLUX 3 Image
  Klein open-source release page (section three, speed figures): a LoRA can
  be attached to the quantized model at about 5 % extra generation time.

Modules:
  codec   -- E2M1 / E4M3 value sets, round-to-nearest-even encoders, bf16, packing
  quant   -- fp8r and nvfp4 quantizers, global-scale calibration
  dequant -- dequantized values (exact) and the bf16 fallback weights
  gemm    -- fp64 reference products and an exact rational dot product
  lora    -- the low-rank adapter side path, y = base + s (X A^T) B^T

Pinned functions: every public function here is checked by ``tests/`` against
value sets, brute-force searches, closed forms, invariants or exact rational
arithmetic (see ``tests/test_oracle_*.py``). No function is "parity unpinned".
"""

from . import codec, quant, dequant, gemm, lora  # noqa: F401
