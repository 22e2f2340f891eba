"""fp64 CPU oracle for the paged decoder-attention core.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do. It shares no code with the HIP library (not even the
bf16 codec) and imports nothing from it.

It is the plain definition of what the path computes, written from the model
pages ("Phi-3 Mini 4K Instruct" files: src/attention.linnet and
src/rope.linnet; "Mistral 7B Instruct v0.3": Entries; "Qwen3-4B": QK-norm;
"Llama 3.1 8B Instruct": rope scaling), in float64, with no blocking, tiling,
online softmax or split-K:

  rope.inv_freq          frequency table, optional llama3 bands
  norm.rms_norm_heads    per-head QK-RMSNorm
  rope.rotate            rotary positions (rotate-half pairing)
  pages.*                page addressing, pool layout, the K/V write
  attention.*            causal (optionally windowed) GQA softmax attention
                         read through page tables, and its contiguous twin

Every function is pinned by tests under tests/ (marked "not gpu") against
closed forms, library routines, invariants and brute force on tiny inputs.
"""
from . import bf16, rope, norm, pages, attention  # noqa: F401
from .core import prepare_tokens, write_tokens  # noqa: F401
