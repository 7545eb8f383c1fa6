"""CPU oracle for exact layer-streamed NF4 LoRA.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct restatement of
what the hot path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product package
(``layer_streamed_nf4_dequant_amd``) never imports, calls or links anything here, and this
package imports nothing from the product package: the two share no code, tables or
constants. Inputs reach both sides from the seeded generators in
``layer_streamed_nf4_dequant_amd.inputs``, which hold none of the method's arithmetic.

Modules
-------
nf4
    The NF4 storage format with double-quantised absmax (codebook, pack, absmax decode,
    dequantise, bf16 round-to-nearest-even).  Sources: "Can You Fine-Tune a 27B Model on
    a Laptop? (I Did the Math)", transcript @2:19-2:29 (a 4-bit format for bell-curve
    weights, then a second quantisation pass over the first pass's constants), and the
    QLoRA paper (arXiv 2305.14314) that "An 8B Fine-Tune Now Fits in 4 GB of VRAM" links.
lora
    The LoRA linear on a frozen base, forward and analytic backward, in float64.
    Source: "Can You Fine-Tune a 27B Model on a Laptop?", transcript @1:25-1:58 (frozen base,
    a thin pair of trainable matrices per layer); the formulas are the standard LoRA ones.
glue
    The decoder-layer glue around the projections: RMSNorm, rotary position embedding and the
    SwiGLU gate, forward and backward, in float64 (the published definitions of the Llama and Qwen
    layers the pages train; the pages print none of them).
attention
    Causal multi-head attention with grouped key/value heads on packed equal-length sequences,
    forward (output and row log-sum-exp) and backward, in float64 (the published definition of
    the Llama and Qwen attention the pages' models use; the pages print none of it).
ce
    The frozen embedding lookup and token-level cross-entropy through the frozen LM head
    (loss, logit gradient, hidden-state gradient), in float64.  Source: "Can You Fine-Tune a
    27B Model on a Laptop?", transcript @7:42-7:55 (resident, unquantised embedding and output
    head); the formulas are the standard cross-entropy ones.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms, invariants,
brute force and finite differences. Parity with the pages themselves is unpinned where
the pages print no values (they print no codebook, tensor or checksum).
"""

from . import attention, ce, glue, nf4, lora  # noqa: F401
