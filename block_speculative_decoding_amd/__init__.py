"""DFlash draft-verify hot path on AMD MI355X (gfx950).

Python surface of libdflash.so; see include/dflash.h for the contract of each
call.  Importing does not load the library; the first call does, and raises
DFlashError if it has not been built.
"""

from ._lib import (DFlashError, load, ctx_fuse, block_attn, spec_verify,
                   prepare_ctx_fuse, prepare_block_attn, prepare_spec_verify,
                   spec_verify_noalloc, prepare_spec_verify_noalloc, verify_scratch_bytes,
                   draft_embed, draft_qkv, draft_mlp,
                   prepare_draft_embed, prepare_draft_qkv, prepare_draft_mlp,
                   ring_append, prepare_ring_append, draft_head, prepare_draft_head,
                   draft_paths, prepare_draft_paths, calib_sink, calib_stream, calib_gather, calib_mfma, EXPORTS)

__all__ = ["DFlashError", "load", "ctx_fuse", "block_attn", "spec_verify",
           "prepare_ctx_fuse", "prepare_block_attn", "prepare_spec_verify",
           "spec_verify_noalloc", "prepare_spec_verify_noalloc", "verify_scratch_bytes",
           "draft_embed", "draft_qkv", "draft_mlp",
           "prepare_draft_embed", "prepare_draft_qkv", "prepare_draft_mlp",
           "ring_append", "prepare_ring_append", "draft_head", "prepare_draft_head",
           "draft_paths", "prepare_draft_paths", "calib_sink", "calib_stream", "calib_gather", "calib_mfma", "EXPORTS"]
