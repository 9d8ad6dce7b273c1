"""CPU oracle for the DFlash draft-verify hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, float64 reference that the HIP kernels are
checked against.  It is not part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run it.  It shares no code with the HIP path (``csrc/``) and never
imports the ``block_speculative_decoding_amd`` package.

Every function states which passage of the source pages it follows.  The
pages are:

* "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash"
  (flozi.net, English edition; a German edition carries the same text) --
  cited below as [E4B] with its section titles.
* "DFlash & DFlash2: Block-Diffusion LLM-Speedup" (xencorenexus.com, German)
  -- cited below as [DF2] with its numbered section titles.

Modules:

* ``philox``      -- Philox4x64-10 counter-based generator and the uniform /
                     Gumbel layout shared (by definition, not by code) with
                     the GPU.
* ``common``      -- RMSNorm, rotate-half RoPE, bf16 round-to-nearest-even.
* ``ctx_fuse``    -- context fusion + K/V injection.
* ``block_attn``  -- non-causal block attention over cached context + block.
* ``spec_verify`` -- exact speculative verification (greedy and sampled).
* ``draft_layer`` -- the rest of a draft layer around block attention: block
                     embedding, input norm + fused Q/K/V projection, output
                     projection + residual, SwiGLU MLP, final norm.
* ``window_cache`` -- the sliding-window draft cache as a ring of pages:
                     capacity, append slots, wrapped block table.
* ``draft_head``  -- the shared LM head over the block rows and the draft
                     proposals (argmax, or Gumbel-max on stream 2).
* ``dflash2``     -- DFlash2's depthwise block convolution (a residual branch
                     between attention and the feed-forward half) and the
                     top-m path selector (per-position candidates, entropy,
                     top-P paths).

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against values printed on the pages, closed forms, invariants, brute force
or an independent library routine; none is "parity unpinned".
"""

from .common import bf16_round, rms_norm, rope_rotate_half, rope_angles
from .philox import philox4x64_10, uniforms, gumbel
from .ctx_fuse import ctx_fuse_ref, concat_capture
from .block_attn import block_attn_ref, attend, prep_block
from .spec_verify import spec_verify_ref, VerifyTrace
from .draft_layer import embed_block, qkv_ref, mlp_ref, o_proj_residual_ref, ffn_ref, silu, layer_weight_shapes
from .window_cache import ring_pages, ring_append, ring_block_table
from .draft_head import head_logits_ref, draft_keys, draft_sample_ref, draft_stats_ref
from .dflash2 import depthwise_conv_ref, conv_mlp_ref, row_stats_ref, top_paths_ref, path_select_ref

__all__ = [
    "bf16_round", "rms_norm", "rope_rotate_half", "rope_angles",
    "philox4x64_10", "uniforms", "gumbel",
    "ctx_fuse_ref", "concat_capture",
    "block_attn_ref", "attend", "prep_block",
    "spec_verify_ref", "VerifyTrace",
    "embed_block", "qkv_ref", "mlp_ref", "o_proj_residual_ref", "ffn_ref", "silu", "layer_weight_shapes",
    "ring_pages", "ring_append", "ring_block_table",
    "head_logits_ref", "draft_keys", "draft_sample_ref", "draft_stats_ref",
    "depthwise_conv_ref", "conv_mlp_ref", "row_stats_ref", "top_paths_ref", "path_select_ref",
]
