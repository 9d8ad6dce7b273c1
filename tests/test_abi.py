"""CPU tests of the C ABI: the library loads, exports every function the
header declares, its struct sizes match the binding, and invalid calls are
rejected before anything reaches the GPU.  Also checks the page-layout
formulas of the header are permutations (every slot used once)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from tests.layout import k_offsets, v_offsets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


@pytest.fixture(scope="module")
def lib():
    from block_speculative_decoding_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from block_speculative_decoding_amd.build import build_library
        build_library(verbose=False)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dflash_\w+)\s*\(", text, re.M)))


def test_header_declares_every_operation():
    fns = declared_functions()
    for f in ("dflash_ctx_fuse", "dflash_block_attn", "dflash_spec_verify",
              "dflash_fuse_workspace_size", "dflash_attn_workspace_size",
              "dflash_verify_workspace_size", "dflash_last_error", "dflash_version",
              "dflash_args_size", "dflash_draft_embed", "dflash_draft_qkv", "dflash_draft_mlp",
              "dflash_draft_qkv_workspace_size", "dflash_draft_mlp_workspace_size", "dflash_ring_append",
              "dflash_draft_head", "dflash_draft_head_workspace_size", "dflash_draft_paths",
              "dflash_draft_paths_workspace_size", "dflash_spec_verify_noalloc", "dflash_verify_scratch_bytes"):
        assert f in fns


def test_library_exports_every_declared_symbol(lib):
    from block_speculative_decoding_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, re.M))
    for f in declared_functions():
        assert f in exported, f
        assert hasattr(lib, f)
    assert sorted(declared_functions()) == sorted(_lib.EXPORTS)


def test_struct_sizes_and_version(lib):
    from block_speculative_decoding_amd import _lib
    assert lib.dflash_version() == 10501
    for kind, st in enumerate(_lib.ARG_STRUCTS):
        assert lib.dflash_args_size(kind) == ctypes.sizeof(st)
    assert lib.dflash_args_size(len(_lib.ARG_STRUCTS)) == 0


def test_page_layouts_are_permutations():
    for off in (k_offsets(), v_offsets()):
        assert sorted(off.reshape(-1).tolist()) == list(range(2048))


# ---------------------------------------------------------------- validation
FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced


def _verify_args(**kw):
    from block_speculative_decoding_amd import _lib
    a = _lib.VerifyArgs()
    a.dtype, a.B, a.V = 0, 4, 4096
    a.target_logits, a.t_batch_stride, a.t_row_stride = FAKE, 8 * 4096, 4096
    a.draft_logits, a.d_batch_stride, a.d_row_stride = FAKE, 7 * 4096, 4096
    a.draft_tokens = a.temperature = a.out_tokens = a.out_len = a.near_ties = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _attn_args(**kw):
    from block_speculative_decoding_amd import _lib
    a = _lib.AttnArgs()
    a.dtype, a.B = 0, 2
    a.q = a.k_blk = a.v_blk = a.gq = a.gk = a.k_cache = a.v_cache = FAKE
    a.block_table = a.ctx_len = a.out = FAKE
    a.eps, a.rope_theta = 1e-6, 1e6
    a.num_pages, a.max_pages = 10, 5
    a.page_size, a.block_len, a.window, a.split_tokens = 16, 8, 0, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _fuse_args(**kw):
    from block_speculative_decoding_amd import _lib
    a = _lib.FuseArgs()
    a.dtype, a.num_layers, a.M = 0, 2, 64
    for i in range(5):
        a.hs[i] = FAKE
        a.k_cache[i] = a.v_cache[i] = FAKE
    a.hs_stride = 2560
    a.wc = a.gc = a.wkv = a.gk = a.pos = a.slot = FAKE
    a.eps, a.rope_theta, a.num_pages = 1e-6, 1e6, 16
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _ws(lib, kind, a):
    n = ctypes.c_size_t()
    rc = getattr(lib, f"dflash_{kind}_workspace_size")(ctypes.byref(a), ctypes.byref(n))
    return rc, n.value


def _call(lib, fn, a, ws=None, nbytes=0):
    return getattr(lib, fn)(ctypes.byref(a), ws, nbytes, None)


def test_verify_validation(lib):
    rc, n = _ws(lib, "verify", _verify_args())
    assert rc == 0 and n > 0
    assert _ws(lib, "verify", _verify_args(V=4100))[0] == -1          # not a multiple of 8
    assert _ws(lib, "verify", _verify_args(dtype=7))[0] == -2
    assert _ws(lib, "verify", _verify_args(B=0))[0] == -1
    assert _call(lib, "dflash_spec_verify", _verify_args(target_logits=None), FAKE, n) == -1
    assert _call(lib, "dflash_spec_verify", _verify_args(draft_tokens=FAKE + 4), FAKE, n) == -1  # misaligned
    assert _call(lib, "dflash_spec_verify", _verify_args(t_row_stride=4000), FAKE, n) == -1
    assert _call(lib, "dflash_spec_verify", _verify_args(d_batch_stride=7 * 4096 + 4), FAKE, n) == -1
    assert _call(lib, "dflash_spec_verify", _verify_args(), None, 0) == -4
    assert _call(lib, "dflash_spec_verify", _verify_args(), FAKE, n - 1) == -4
    assert b"workspace" in lib.dflash_last_error()
    # workspace grows with B and V
    assert _ws(lib, "verify", _verify_args(B=8))[1] > n
    assert _ws(lib, "verify", _verify_args(V=262144))[1] > n


def test_verify_noalloc_validation(lib):
    # The allocation-free entry point validates like dflash_spec_verify and
    # rejects calls whose workspace would exceed its fixed device scratch;
    # none of these calls reaches the GPU.
    n = ctypes.c_size_t()
    assert lib.dflash_verify_scratch_bytes(ctypes.byref(n)) == 0 and n.value == 4 << 20
    cap = n.value
    assert _ws(lib, "verify", _verify_args(B=1409, V=262144))[1] <= cap
    assert _ws(lib, "verify", _verify_args(B=1410, V=262144))[1] > cap

    def call(a):
        return lib.dflash_spec_verify_noalloc(ctypes.byref(a), None)

    def big(B, V):
        return _verify_args(B=B, V=V, t_batch_stride=8 * V, t_row_stride=V, d_batch_stride=7 * V, d_row_stride=V)
    assert call(big(1410, 262144)) == -4
    msg = lib.dflash_last_error().decode()
    assert "dflash_spec_verify_noalloc" in msg and str(cap) in msg and "B = 1410" in msg
    assert call(big(4096, 1 << 20)) == -4
    assert call(_verify_args(target_logits=None)) == -1
    assert call(_verify_args(V=4100)) == -1
    assert call(_verify_args(dtype=7)) == -2
    assert lib.dflash_spec_verify_noalloc(None, None) == -1
    assert lib.dflash_verify_scratch_bytes(None) == -1


def test_attn_validation(lib):
    assert _ws(lib, "attn", _attn_args())[0] == 0
    assert _ws(lib, "attn", _attn_args(block_len=7))[0] == -1
    assert _ws(lib, "attn", _attn_args(page_size=32))[0] == -1
    assert _ws(lib, "attn", _attn_args(split_tokens=100))[0] == -1
    assert _ws(lib, "attn", _attn_args(window=-1))[0] == -1
    assert _ws(lib, "attn", _attn_args(B=0))[0] == -1
    assert _ws(lib, "attn", _attn_args(dtype=3))[0] == -2
    assert _call(lib, "dflash_block_attn", _attn_args(q=None)) == -1
    assert _call(lib, "dflash_block_attn", _attn_args(eps=0.0)) == -1
    assert _call(lib, "dflash_block_attn", _attn_args(block_len=16)) == -1
    assert b"block_len" in lib.dflash_last_error()
    # A split count above one needs a workspace; a single split does not.
    rc, n = _ws(lib, "attn", _attn_args(max_pages=1000, split_tokens=128))
    assert rc == 0 and n > 0
    assert _call(lib, "dflash_block_attn", _attn_args(max_pages=1000, split_tokens=128)) == -4
    rc, n1 = _ws(lib, "attn", _attn_args(max_pages=8, split_tokens=1024))
    assert rc == 0 and n1 == 0
    # workspace is monotone in the context capacity
    sizes = [_ws(lib, "attn", _attn_args(max_pages=p, split_tokens=128))[1] for p in (8, 64, 512)]
    assert sizes == sorted(sizes)
    # fp32 path needs no workspace
    assert _ws(lib, "attn", _attn_args(dtype=1, max_pages=1000))[1] == 0
    # Balanced pieces (split_tokens = -1): 64 pieces x 2 slots x 8 KV heads of
    # (m[32], l[32], acc[32][128]) fp32 partials, then B + 1 ints of merge
    # table; -2 is not a mode.
    kpart = (64 + 32 * 128) * 4
    assert _ws(lib, "attn", _attn_args(B=64, max_pages=513, split_tokens=-1)) == (0, 64 * 2 * 8 * kpart + 65 * 4)
    assert _ws(lib, "attn", _attn_args(split_tokens=-2))[0] == -1
    # Beyond 1024 sequences, or where a piece could pass 32768 tokens, the
    # automatic split takes over (one split per sequence here: no workspace).
    assert _ws(lib, "attn", _attn_args(B=1025, max_pages=8, split_tokens=-1)) == (0, 0)
    assert _ws(lib, "attn", _attn_args(B=1024, max_pages=8192, split_tokens=-1)) == \
        _ws(lib, "attn", _attn_args(B=1024, max_pages=8192, split_tokens=0))


def test_fuse_validation(lib):
    rc, n = _ws(lib, "fuse", _fuse_args())
    assert rc == 0 and n > 0
    assert _ws(lib, "fuse", _fuse_args(M=0))[1] == 0
    assert _call(lib, "dflash_ctx_fuse", _fuse_args(M=0)) == 0   # valid no-op
    assert _ws(lib, "fuse", _fuse_args(num_layers=0))[0] == -1
    assert _ws(lib, "fuse", _fuse_args(num_layers=6))[0] == -1
    assert _ws(lib, "fuse", _fuse_args(M=-1))[0] == -1
    assert _call(lib, "dflash_ctx_fuse", _fuse_args(hs_stride=2500), FAKE, n) == -1
    assert _call(lib, "dflash_ctx_fuse", _fuse_args(hs_stride=(1 << 22) + 8), FAKE, n) == -1
    assert _call(lib, "dflash_ctx_fuse", _fuse_args(wc=None), FAKE, n) == -1
    a = _fuse_args()
    a.k_cache[1] = None
    assert _call(lib, "dflash_ctx_fuse", a, FAKE, n) == -1
    a = _fuse_args(num_layers=1)
    a.k_cache[1] = None  # ignored beyond num_layers
    assert _call(lib, "dflash_ctx_fuse", a, None, 0) == -4
    assert _call(lib, "dflash_ctx_fuse", _fuse_args(num_pages=0), FAKE, n) == -1
    assert _ws(lib, "fuse", _fuse_args(M=4096))[1] > n


def test_binding_refuses_host_tensors(lib):
    import torch
    import block_speculative_decoding_amd as dfl
    z = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(dfl.DFlashError):
        dfl.spec_verify(z, z[:, :7], torch.zeros((2, 7), dtype=torch.int32), torch.zeros(2))


def _qkv_args(**kw):
    from block_speculative_decoding_amd import _lib
    a = _lib.QkvArgs()
    a.dtype, a.B, a.eps = 0, 64, 1e-6
    a.x = a.g_in = a.w_qkv = a.q = a.k_blk = a.v_blk = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _mlp_args(**kw):
    from block_speculative_decoding_amd import _lib
    a = _lib.MlpArgs()
    a.dtype, a.B, a.eps = 0, 64, 1e-6
    a.x = a.o = a.w_o = a.g_post = a.w_gu = a.w_d = a.x_out = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _embed_args(**kw):
    from block_speculative_decoding_amd import _lib
    a = _lib.EmbedArgs()
    a.dtype, a.B, a.V, a.mask_id = 0, 4, 1000, 999
    a.emb = a.anchor = a.x = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_draft_layer_validation(lib):
    # Only calls that fail validation are made: nothing reaches the GPU.
    rc, n = _ws(lib, "draft_qkv", _qkv_args())
    assert rc == 0 and n > 0
    assert _ws(lib, "draft_qkv", _qkv_args(B=0))[0] == -1
    assert _ws(lib, "draft_qkv", _qkv_args(B=8193))[0] == -1
    assert _ws(lib, "draft_qkv", _qkv_args(dtype=5))[0] == -2
    assert _ws(lib, "draft_qkv", _qkv_args(B=128))[1] > n
    assert _call(lib, "dflash_draft_qkv", _qkv_args(x=None), FAKE, n) == -1
    assert _call(lib, "dflash_draft_qkv", _qkv_args(w_qkv=FAKE + 8), FAKE, n) == -1
    assert _call(lib, "dflash_draft_qkv", _qkv_args(eps=0.0), FAKE, n) == -1
    assert _call(lib, "dflash_draft_qkv", _qkv_args(), FAKE, n - 1) == -4

    rc, m = _ws(lib, "draft_mlp", _mlp_args())
    assert rc == 0 and m > 0
    assert _ws(lib, "draft_mlp", _mlp_args(B=0))[0] == -1
    assert _call(lib, "dflash_draft_mlp", _mlp_args(w_d=None), FAKE, m) == -1
    assert _call(lib, "dflash_draft_mlp", _mlp_args(g_final=FAKE), FAKE, m) == -1  # y_out missing
    assert b"y_out" in lib.dflash_last_error()
    assert _call(lib, "dflash_draft_mlp", _mlp_args(), None, 0) == -4
    assert _ws(lib, "draft_mlp", _mlp_args(dtype=1))[1] > 0

    emb = lib.dflash_draft_embed
    assert emb(ctypes.byref(_embed_args(mask_id=1000)), None) == -1
    assert emb(ctypes.byref(_embed_args(mask_id=-1)), None) == -1
    assert emb(ctypes.byref(_embed_args(V=0, mask_id=0)), None) == -1
    assert emb(ctypes.byref(_embed_args(anchor=None)), None) == -1
    assert emb(ctypes.byref(_embed_args(B=0)), None) == -1
    assert emb(ctypes.byref(_embed_args(dtype=9)), None) == -2


def test_ring_append_validation(lib):
    from block_speculative_decoding_amd import _lib

    def args(**kw):
        a = _lib.RingArgs()
        a.B, a.ring_pages, a.rows_per_seq = 4, 64, 8
        a.ring = a.ctx_len = a.n_new = a.slot = a.pos = FAKE
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    f = lib.dflash_ring_append
    assert f(ctypes.byref(args(B=0)), None) == -1
    assert f(ctypes.byref(args(ring_pages=0)), None) == -1
    assert f(ctypes.byref(args(rows_per_seq=0)), None) == -1
    assert f(ctypes.byref(args(rows_per_seq=65)), None) == -1
    assert f(ctypes.byref(args(n_new=None)), None) == -1
    assert b"null" in lib.dflash_last_error()



def test_draft_head_validation(lib):
    from block_speculative_decoding_amd import _lib

    def args(**kw):
        a = _lib.HeadArgs()
        a.dtype, a.B, a.V = 0, 64, 262144
        a.y = a.w_head = a.temperature = a.logits = a.draft_tokens = FAKE
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    rc, n = _ws(lib, "draft_head", args())
    # one (key, index) partial and one (max, sum) partial per 256-column
    # tile of each proposal row
    assert rc == 0 and n == 2 * 64 * 7 * 1024 * 8
    assert _ws(lib, "draft_head", args(V=262144 + 64))[0] == -1      # not a multiple of 128
    assert _ws(lib, "draft_head", args(V=0))[0] == -1
    assert _ws(lib, "draft_head", args(V=(1 << 21) + 128))[0] == -1
    assert _ws(lib, "draft_head", args(B=0))[0] == -1
    assert _ws(lib, "draft_head", args(B=8193))[0] == -1
    assert _ws(lib, "draft_head", args(dtype=3))[0] == -2
    assert _ws(lib, "draft_head", args(V=128, B=1))[1] == 512        # one chunk of each, rounded to 256 bytes
    assert _call(lib, "dflash_draft_head", args(draft_stats=FAKE + 8), FAKE, n) == -1   # misaligned
    assert _call(lib, "dflash_draft_head", args(w_head=None), FAKE, n) == -1
    assert _call(lib, "dflash_draft_head", args(logits=FAKE + 4), FAKE, n) == -1
    assert _call(lib, "dflash_draft_head", args(temperature=None), FAKE, n) == -1
    assert _call(lib, "dflash_draft_head", args(), FAKE, n - 1) == -4
    assert _call(lib, "dflash_draft_head", args(), None, 0) == -4


def test_draft_paths_validation(lib):
    from block_speculative_decoding_amd import _lib

    def args(**kw):
        a = _lib.PathsArgs()
        a.dtype, a.B, a.V, a.m, a.P = 0, 64, 262144, 4, 16
        a.batch_stride, a.row_stride = 8 * 262144, 262144
        a.logits = a.cand_ids = a.cand_logp = a.entropy = a.paths = a.scores = FAKE
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    rc, n = _ws(lib, "draft_paths", args())
    assert rc == 0 and n == 64 * 7 * 32 * 80          # one 80-byte partial per 8192 entries of a row (one per wave)
    assert _ws(lib, "draft_paths", args(m=0))[0] == -1
    assert _ws(lib, "draft_paths", args(m=9))[0] == -1
    assert _ws(lib, "draft_paths", args(P=65))[0] == -1
    assert _ws(lib, "draft_paths", args(m=1, P=2))[0] == -1      # only one path exists
    assert _ws(lib, "draft_paths", args(m=2, P=64))[0] == 0      # 128 paths exist
    assert _ws(lib, "draft_paths", args(V=262140))[0] == -1
    assert _ws(lib, "draft_paths", args(V=3, row_stride=8, batch_stride=64))[0] == -1  # V < m
    assert _ws(lib, "draft_paths", args(row_stride=262136))[0] == -1
    assert _ws(lib, "draft_paths", args(batch_stride=7 * 262144))[0] == -1
    assert _ws(lib, "draft_paths", args(dtype=4))[0] == -2
    assert _call(lib, "dflash_draft_paths", args(paths=None), FAKE, n) == -1
    assert _call(lib, "dflash_draft_paths", args(logits=FAKE + 2), FAKE, n) == -1
    assert _call(lib, "dflash_draft_paths", args(), FAKE, n - 1) == -4


def test_draft_mlp_conv_validation(lib):
    rc, m = _ws(lib, "draft_mlp", _mlp_args())
    assert _call(lib, "dflash_draft_mlp", _mlp_args(conv_k=9, w_conv=FAKE, b_conv=FAKE), FAKE, m) == -1
    assert _call(lib, "dflash_draft_mlp", _mlp_args(conv_k=-1), FAKE, m) == -1
    assert _call(lib, "dflash_draft_mlp", _mlp_args(conv_k=3, w_conv=FAKE), FAKE, m) == -1   # b_conv missing
    assert b"b_conv" in lib.dflash_last_error()
    assert _call(lib, "dflash_draft_mlp", _mlp_args(conv_k=3, b_conv=FAKE, w_conv=FAKE + 8), FAKE, m) == -1


def test_calibration_validation(lib):
    n = ctypes.c_size_t()
    assert lib.dflash_calib_sink_bytes(ctypes.byref(n)) == 0 and n.value >= 65536 * 16
    assert lib.dflash_calib_stream(None, None, 1024, 0, FAKE, None) == -1
    assert lib.dflash_calib_stream(FAKE, None, 1000, 0, FAKE, None) == -1          # not a multiple of 16
    assert lib.dflash_calib_stream(FAKE, FAKE + 8, 1024, 0, FAKE, None) == -1      # misaligned copy target
    assert lib.dflash_calib_stream(FAKE, None, 1024, 0, None, None) == -1
    assert lib.dflash_calib_stream(FAKE, None, 1024, 65537, FAKE, None) == -1
    g = lib.dflash_calib_gather
    g.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert g(None, 1 << 20, FAKE, 4, 8192, 0, FAKE, None) == -1
    assert g(FAKE, 1 << 20, None, 4, 8192, 0, FAKE, None) == -1
    assert g(FAKE, 1 << 20, FAKE, 4, 8192, 0, None, None) == -1
    assert g(FAKE + 8, 1 << 20, FAKE, 4, 8192, 0, FAKE, None) == -1                 # misaligned source
    assert g(FAKE, 1000, FAKE, 4, 8192, 0, FAKE, None) == -1                        # not a multiple of 16
    assert g(FAKE, 1 << 20, FAKE, 4, 6000, 0, FAKE, None) == -1                     # chunk not 4 KiB pieces
    assert g(FAKE, 1 << 20, FAKE, 4, 2 << 20, 0, FAKE, None) == -1                  # chunk above 1 MiB
    assert g(FAKE, 1 << 20, FAKE, 0, 8192, 0, FAKE, None) == -1
    assert g(FAKE, 1 << 20, FAKE, (1 << 30) + 1, 8192, 0, FAKE, None) == -1         # over 2^31 pieces
    assert g(FAKE, 1 << 20, FAKE, 4, 8192, 65537, FAKE, None) == -1
    assert b"dflash_calib_gather" in lib.dflash_last_error()
    f = ctypes.c_double()
    assert lib.dflash_calib_mfma(0, FAKE, ctypes.byref(f), None) == -1
    assert lib.dflash_calib_mfma(5, None, ctypes.byref(f), None) == -1


def test_sanitizer_runtime_present_when_expected(lib):
    """Run under the host-sanitized library (test_abi_sanitized.py), this
    process must have the AddressSanitizer and UBSan runtimes mapped and must
    have loaded that library, not the default one."""
    if os.environ.get("DFLASH_EXPECT_SANITIZERS") != "1":
        return
    from block_speculative_decoding_amd import _lib
    maps = open("/proc/self/maps").read()
    assert "libasan" in maps and "libubsan" in maps
    assert _lib.LIB_PATH == os.environ["DFLASH_LIBRARY"] and _lib.LIB_PATH in maps
