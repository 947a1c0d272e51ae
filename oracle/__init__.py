"""CPU oracle for the NVFP4 sparse-MLA decode path.

TEST INFRASTRUCTURE ONLY. Nothing in the product library (the HIP kernels,
the C-ABI or its Python binding) may import, call or link anything here: only
the test suite, the smoke check and the CPU-baseline leg of the benchmark do.

The oracle is a plain, slow, obviously-correct restatement of what the pages
define, in float64 (exact rational arithmetic where a rounding decision must be
exact).  It shares no code, table or constant generator with the GPU path.

Sources (cited by page title and section):
  [FlashMLA-18]  "W4A16 DSA: NVFP4 KV cache format for SM100 sparse decode",
                 PR description (record layout, permuted scales, A16 dequant).
  [vLLM-82]      "kv: nvfp4_ds_mla -- 4-bit NVFP4 KV cache for B12X sparse MLA
                 (SM120)", Fix and Tests sections and the test commit message
                 (scale = E4M3(group_amax/6), error bound, slot_mapping).
  [sglang-38646] "[SM120] Add opt-in NVFP4 sparse-MLA KV cache format for
                 DeepSeek-V4", Modifications (slot ids shared by writers and
                 readers) and Limitations (the fused norm + rope + quantize +
                 store kernel).

Modules:
  formats    -- element encodings: E2M1, E4M3 decode/encode, record layout.
  codec      -- quantize-append (write path) and record dequantization.
  attention  -- sparse MLA decode (O, LSE) and the split-KV combine.
  norm_rope  -- the fused write path: RMSNorm + rotary embedding, rounded to
                bf16, then the write rule.
"""

from . import formats, codec, attention, norm_rope  # noqa: F401
