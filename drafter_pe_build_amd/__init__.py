"""P-EAGLE parallel-drafting hot path on AMD MI355X (gfx950).

The compute lives in libpe.so (HIP kernels behind the C ABI of include/pe.h);
this package holds its sources (csrc/), the build script, the ctypes binding
(_lib) and a step runner that chains the stage calls on device buffers.
"""
from ._lib import (PE_BF16, PE_F32, PE_PADDING_SLOT_ID, PeError, attn_args, dims_struct,  # noqa: F401
                   pe_build_draft_batch, pe_draft_attention, pe_draft_attention_workspace, pe_draft_layer,
                   pe_draft_layer_workspace, pe_fuse_hidden, pe_fuse_hidden_workspace, pe_lm_head_argmax,
                   pe_lm_head_argmax_workspace, pe_version)
