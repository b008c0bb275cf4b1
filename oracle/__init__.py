"""Plain, slow CPU oracle for NVFP4 MLA attention.

TEST INFRASTRUCTURE ONLY.  This package is the independent statement of what the
GPU path computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library never
does, and this package imports nothing from the product (``include/``,
``mla_attention_nvfp4_amd``).  The two share no code.

Arithmetic conventions
----------------------
* Quantization steps use IEEE binary32 NumPy arithmetic, one correctly rounded
  operation per step, so every quantized code has one defined value.
* Attention arithmetic (scores, softmax, weighted sums, log-sum-exp) is float64.

The pages this follows (cited by title and section throughout):

* [FUSED-OUT]  vLLM pull request "feat: MLA prefill NVFP4 fused output"
  (carlyou/vllm #8): the prefill writes packed e2m1 output, a 128x4-swizzled
  e4m3 block-scale buffer and uses an fp32 global scale.
* [MO-MLA]     Model-Optimizer pull request "Add NVFP4/FP8 Q/K/P/V + 2:4
  attention quantization for MLA (vLLM TRITON_MLA)" (NVIDIA/Model-Optimizer
  #2244): split-K absorbed decode over the paged latent, natural-log LSE, varlen
  prefill with Q/K/P/V NVFP4 fake quantization along each contraction axis.
* [B12X]       b12x pull request "nvfp4 MLA KV cache + per-layer outer-scale +
  fp8-RoPE KV-cell (sm120)" (local-inference-lab/b12x #33): NVFP4 latent cache
  record of 432 or 368 bytes, per-layer outer scale restored on read, top-k
  sparse decode.

Modules
-------
formats  e2m1 / e4m3 codecs, NVFP4 two-level block quantizer   (pinned)
record   latent cache record pack/unpack and cache write         (pinned)
decode   dense and sparse paged decode, split-K LSE merge         (pinned)
prefill  varlen causal prefill with Q/K/P/V fake quantization      (pinned;
         the P-quantization schedule is a convention, see prefill.py)
swizzle  128x4 block-scale layout and the NVFP4 output quantizer  (pinned)
"""

from . import formats, record, decode, prefill, swizzle  # noqa: F401
