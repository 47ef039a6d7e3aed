"""Plain fp64 CPU oracle of the latent mixture-of-experts layer.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package. The HIP library never links it, and
the two share no code: no kernels, helpers, tables or constant generators.

What it follows (cited by page title, then section / equation / table):

* LAYER = "Edge0 145B and Edge0 120B" model page: "Model profile" table and
  the "Edge0-145B architecture" / "Edge0-120B architecture" text.
* TEARDOWN = "Edge0-145B: a Qwen MoE with its experts squeezed, and a 51B
  table left on the SSD": section "A latent in front of the experts" (the
  layer equation and the statement that D runs over all groups while U runs
  once per routed group), "What is 4-bit" (record sizes and formats), "The
  base, byte for byte" (bf16 router, 2,621,440 B per layer).
* README = the Edge0 README ("Architecture": 10 of 512 experts plus one
  shared expert).
* Q3_K builds = TEARDOWN "What is 4-bit" (Q3_K gate/up, IQ4_NL down, the
  record sizes), module ``kquants`` (block layouts restated from GGML's
  published definitions; the quantizer is ours).
* PLE = TEARDOWN, section "The 51.2B the GPU never holds" (the n-gram
  embedding gather, module ``ple``; its hash is a reading, see there).

Where the pages leave a step open, the reading taken is stated at the
function that takes it. Numeric parity of the layer output has no printed
worked example on the pages ("parity unpinned" externally); the oracle is
pinned by exhaustive codec tables, library conversions, round-trip bounds,
the printed byte sizes, brute-force evaluation on tiny shapes, the linearity
identity and special cases (see ``tests/test_oracle_*.py``).
"""

from .formats import (  # noqa: F401
    e2m1_decode, e4m3_decode, e4m3_encode, e2m1_encode, round_pos,
    f32_to_bf16_bits, bf16_bits_to_f64, f64_to_f16_bits, f16_bits_to_f64,
    quantize_nvfp4, dequantize_nvfp4, quantize_blocks, dequantize_blocks,
    pack_expert_record, unpack_expert_record, expert_record_bytes,
    du_group_bytes,
)
from .layer import (  # noqa: F401
    LayerDims, pack_layer, decode_layer, router_logits, select_topk,
    permute, expert_offsets, layer_forward, rmsnorm, stack_forward,
)
