"""Plain, slow fp64 CPU oracle for the P-EAGLE parallel-drafting hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) may import, call or execute this package.  It is used by
``tests/``, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``.  It shares no code with the HIP path: it imports only numpy
(and, for bf16 storage, decodes the bit patterns itself).

Sources cited in this package, by title:

* [PD]  "P-EAGLE: parallel speculative decoding in vLLM" (agentlenshq.com
        blog, Traditional-Chinese and Korean versions): "Step 2: parallel
        drafting"; "Training on long sequences"; "vLLM implementation
        details" (fused Triton kernel, hidden-state management, KV cache and
        CUDA graphs).
* [RFC] vllm-project/speculators issue #567, "[RFC]: Add random anchor for
        p-eagle first position": "Motivation", "Proposed Change", the
        "Random Anchor Subsampling" note (every original position is a
        depth-0 row), and the "Experiment Setup" table.
* [AD]  "Attention Drift: what autoregressive speculative-decoding models
        learn" (arXiv 2605.09992): section 2 (EAGLE-3 drafter: fc fusion into
        one pre-norm decoder layer), section 4.1 (RMS = ||x||_2 / sqrt(d)) and
        its Observation 2 (RMSNorm on each captured target stream before fc).

Every step is the plain definition of what the path computes; the GPU path
reaches the same results by tiling, online softmax, index-based tile skipping,
chunking and a fused argmax, so agreement is exact up to rounding.

Pins (tests/test_oracle_*.py): a hand-worked batch-build example and the
batch invariants; RMSNorm against its closed form and torch.nn.functional;
the COD visibility predicate against brute-force enumeration on tiny
layouts; single-depth COD against torch causal SDPA; decode attention
against SDPA with an explicit boolean mask; the position-count closed forms;
softmax invariants; argmax against numpy.

Parity unpinned: the drafter's internal composition (embedding added to the
fc output, where h_shared enters, the final norm, bias-free linears, no
positional encoding, SwiGLU form).  The pages print no value that fixes it;
both sides follow the same reading.
"""
from . import batch, cod, drafter, metrics  # noqa: F401
