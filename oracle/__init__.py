"""CPU oracle for the hybrid-precision W4A16 fused MoE layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the CPU-baseline leg of ``bench.py`` may import
anything from this package. The product path (the HIP library and its Python
binding) never imports it and fails loudly when its native library is missing.

What it computes, and where that is defined:

* the hybrid layer itself (pages: local-inference-lab/vllm PR #92 "quant:
  nvfp4_nf3_hybrid", "How it works", and PR #104 description): per-expert tier
  selection by a bit map (4 = kept tier, 3 = NF3 tail), the kept tier in NVFP4 or,
  when the kept format says so, MXFP4; both tiers share one routing result and add
  into one top-k weighted sum; layers absent from the map run uniform NVFP4;
* W4A16 semantics (page: vllm-project/vllm PR #42428, "What's in this PR", item
  1): 4-bit weights, activations left in 16-bit, no activation scales;
* the number formats, which the pages only name: E2M1 / E8M0 / the MXFP4 block
  of 32 from the OCP Microscaling Formats v1.0 specification, E4M3 ("fn") from
  the OCP 8-bit floating point specification, NVFP4 as E2M1 values with one
  E4M3 scale per 16 and one fp32 per-tensor scale, and NF3 as the QLoRA
  NormalFloat construction (Dettmers et al. 2023, section 3) carried out at 3 bits
  with an fp16 absmax scale per 64 elements along K.

Precision: dequantised weights are defined in fp32 (they are the bit-exact
targets); routing weights and the expert MLP are computed in fp64.

Parity pins live in tests/test_oracle_*.py. Two functions are parity unpinned
in the sense that nothing outside this package fixes their choice: the NVFP4
per-tensor scale rule g = amax / (6 * 448) and the MXFP4 zero-block scale byte
(127). Both only shape the synthetic inputs; the HIP path consumes the codes
the quantiser emits and never quantises.
"""
from . import formats, layer  # noqa: F401
