"""ctypes binding of libdflash.so (include/dflash.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of the library.  PyTorch provides device memory and the stream.
The library must be built (``__graft_entry__.build()``); importing works
without it, but every call raises DFlashError if it is missing.
"""

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIBRARY names another build of the same library (the host-sanitized
# build the ABI tests run against); by default the in-tree libdflash.so.
LIB_PATH = os.environ.get("DFLASH_LIBRARY") or os.path.join(PKG, "libdflash.so")

DFLASH_BF16, DFLASH_F32 = 0, 1
SPLIT_BALANCED = -1   # dflash_attn_args.split_tokens: equal pieces of all sequences' tiles
D, NCAPTURE, HQ, HKV, HEAD_DIM, BLOCK, PAGE, INTER = 2560, 5, 32, 8, 128, 8, 16, 5120

_P = ctypes.c_void_p
_I32, _I64, _U64, _F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


class DFlashError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"dflash error {code}: {msg}")
        self.code = code


class FuseArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("num_layers", _I32), ("M", _I64),
                ("hs", _P * 5), ("hs_stride", _I64),
                ("wc", _P), ("gc", _P), ("wkv", _P), ("gk", _P),
                ("eps", _F32), ("rope_theta", _F32),
                ("pos", _P), ("slot", _P),
                ("k_cache", _P * 5), ("v_cache", _P * 5), ("num_pages", _I64),
                ("ht_out", _P)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32),
                ("q", _P), ("k_blk", _P), ("v_blk", _P), ("gq", _P), ("gk", _P),
                ("eps", _F32), ("rope_theta", _F32),
                ("k_cache", _P), ("v_cache", _P), ("num_pages", _I64),
                ("block_table", _P), ("max_pages", _I32), ("ctx_len", _P),
                ("page_size", _I32), ("block_len", _I32), ("window", _I32), ("split_tokens", _I32),
                ("out", _P), ("lse_out", _P)]


class VerifyArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32), ("V", _I64),
                ("target_logits", _P), ("t_batch_stride", _I64), ("t_row_stride", _I64),
                ("draft_logits", _P), ("d_batch_stride", _I64), ("d_row_stride", _I64),
                ("draft_tokens", _P), ("temperature", _P),
                ("seed", _U64), ("offset", _U64),
                ("out_tokens", _P), ("out_len", _P), ("near_ties", _P), ("draft_stats", _P)]


class EmbedArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32), ("V", _I64),
                ("emb", _P), ("anchor", _P), ("mask_id", _I32), ("x", _P)]


class QkvArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32),
                ("x", _P), ("g_in", _P), ("w_qkv", _P), ("eps", _F32),
                ("q", _P), ("k_blk", _P), ("v_blk", _P)]


class MlpArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32),
                ("x", _P), ("o", _P), ("w_o", _P), ("g_post", _P), ("w_gu", _P), ("w_d", _P),
                ("g_final", _P), ("eps", _F32), ("x_out", _P), ("y_out", _P), ("h_out", _P),
                ("conv_k", _I32), ("w_conv", _P), ("b_conv", _P)]


class RingArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("ring_pages", _I32), ("ring", _P), ("ctx_len", _P), ("n_new", _P),
                ("rows_per_seq", _I32), ("slot", _P), ("pos", _P)]


class HeadArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32), ("V", _I64), ("y", _P), ("w_head", _P), ("temperature", _P),
                ("seed", _U64), ("offset", _U64), ("logits", _P), ("draft_tokens", _P), ("draft_stats", _P)]


class PathsArgs(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("B", _I32), ("V", _I64), ("logits", _P), ("batch_stride", _I64),
                ("row_stride", _I64), ("m", _I32), ("P", _I32), ("lam", _F32), ("cand_ids", _P),
                ("cand_logp", _P), ("entropy", _P), ("paths", _P), ("scores", _P)]


ARG_STRUCTS = (FuseArgs, AttnArgs, VerifyArgs, EmbedArgs, QkvArgs, MlpArgs, RingArgs, HeadArgs, PathsArgs)

EXPORTS = ["dflash_version", "dflash_last_error", "dflash_args_size",
           "dflash_fuse_workspace_size", "dflash_attn_workspace_size", "dflash_verify_workspace_size",
           "dflash_draft_qkv_workspace_size", "dflash_draft_mlp_workspace_size",
           "dflash_draft_head_workspace_size", "dflash_draft_paths_workspace_size",
           "dflash_ctx_fuse", "dflash_block_attn", "dflash_spec_verify",
           "dflash_spec_verify_noalloc", "dflash_verify_scratch_bytes",
           "dflash_draft_embed", "dflash_draft_qkv", "dflash_draft_mlp", "dflash_ring_append",
           "dflash_draft_head", "dflash_draft_paths",
           "dflash_calib_sink_bytes", "dflash_calib_stream", "dflash_calib_gather", "dflash_calib_mfma"]

_lib = None


def load():
    """Load libdflash.so once; raise DFlashError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise DFlashError(-100, f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dflash_version.restype = ctypes.c_int
    lib.dflash_last_error.restype = ctypes.c_char_p
    lib.dflash_args_size.restype = ctypes.c_size_t
    lib.dflash_args_size.argtypes = [ctypes.c_int]
    for name, st in (("fuse", FuseArgs), ("attn", AttnArgs), ("verify", VerifyArgs),
                     ("draft_qkv", QkvArgs), ("draft_mlp", MlpArgs), ("draft_head", HeadArgs),
                     ("draft_paths", PathsArgs)):
        f = getattr(lib, f"dflash_{name}_workspace_size")
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(st), ctypes.POINTER(ctypes.c_size_t)]
    for name, st in (("dflash_ctx_fuse", FuseArgs), ("dflash_block_attn", AttnArgs),
                     ("dflash_spec_verify", VerifyArgs), ("dflash_draft_qkv", QkvArgs),
                     ("dflash_draft_mlp", MlpArgs), ("dflash_draft_head", HeadArgs),
                     ("dflash_draft_paths", PathsArgs)):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(st), _P, ctypes.c_size_t, _P]
    lib.dflash_spec_verify_noalloc.restype = ctypes.c_int
    lib.dflash_spec_verify_noalloc.argtypes = [ctypes.POINTER(VerifyArgs), _P]
    lib.dflash_verify_scratch_bytes.restype = ctypes.c_int
    lib.dflash_verify_scratch_bytes.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.dflash_calib_sink_bytes.restype = ctypes.c_int
    lib.dflash_calib_sink_bytes.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.dflash_calib_stream.restype = ctypes.c_int
    lib.dflash_calib_stream.argtypes = [_P, _P, ctypes.c_size_t, ctypes.c_int, _P, _P]
    lib.dflash_calib_gather.restype = ctypes.c_int
    lib.dflash_calib_gather.argtypes = [_P, ctypes.c_size_t, _P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P, _P]
    lib.dflash_calib_mfma.restype = ctypes.c_int
    lib.dflash_calib_mfma.argtypes = [ctypes.c_int, _P, ctypes.POINTER(ctypes.c_double), _P]
    lib.dflash_draft_embed.restype = ctypes.c_int
    lib.dflash_draft_embed.argtypes = [ctypes.POINTER(EmbedArgs), _P]
    lib.dflash_ring_append.restype = ctypes.c_int
    lib.dflash_ring_append.argtypes = [ctypes.POINTER(RingArgs), _P]
    for kind, st in enumerate(ARG_STRUCTS):
        got = lib.dflash_args_size(kind)
        if got != ctypes.sizeof(st):
            raise DFlashError(-101, f"struct mirror {st.__name__} is {ctypes.sizeof(st)} bytes, library has {got}")
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise DFlashError(rc, load().dflash_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return DFLASH_BF16
    if t.dtype == torch.float32:
        return DFLASH_F32
    raise DFlashError(-2, f"unsupported tensor dtype {t.dtype}")


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise DFlashError(-1, f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise DFlashError(-1, f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise DFlashError(-1, f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise DFlashError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise DFlashError(-1, f"{name} must be contiguous")
    return t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_NO_WORKSPACE = object()   # sizes the call but allocates no workspace (allocation-free entry point)


def _workspace(nbytes, workspace, device):
    if nbytes == 0 or workspace is _NO_WORKSPACE:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise DFlashError(-4, f"workspace holds {workspace.numel() * workspace.element_size()} bytes, {nbytes} needed")
    return workspace, workspace.numel() * workspace.element_size()


def _record(stream, objs):
    """Tell torch's caching allocator that every tensor the call reads or
    writes is in use on `stream` when that is not the current stream: the
    workspace and outputs allocated here live on the current stream, and the
    one-shot wrappers drop them as soon as the call is enqueued, so without
    this their memory could be handed out again while the kernels still run."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for o in objs:
        if isinstance(o, (list, tuple)):
            _record(stream, o)
        elif isinstance(o, torch.Tensor):
            o.record_stream(stream)


class Prepared:
    """A validated argument struct plus its workspace: call it to enqueue."""

    def __init__(self, fn, args, workspace, ws_bytes, keep):
        self._fn, self.args, self.workspace, self.ws_bytes = fn, args, workspace, ws_bytes
        self._keep = keep  # tensors the struct points into

    def __call__(self, stream=None):
        _check(self._fn(ctypes.byref(self.args), _ptr(self.workspace), self.ws_bytes, _stream(stream)))
        _record(stream, (self.workspace, self._keep))


# ---------------------------------------------------------------- ctx_fuse
def prepare_ctx_fuse(hs, wc, gc, wkv, gk, pos, slot, k_caches, v_caches, eps=1e-6, rope_theta=1e6,
                     ht_out=None, workspace=None):
    """Context fusion + K/V injection (include/dflash.h, dflash_ctx_fuse).

    hs: 5 tensors [M, >=2560] (row stride from the tensor); wc [2560, 12800];
    gc [2560]; wkv [L*2048, 2560]; gk [L, 128]; pos int32 [M]; slot int64 [M];
    k_caches / v_caches: L tensors [num_pages, 8, 2048] in the page layout.
    """
    lib = load()
    if len(hs) != NCAPTURE:
        raise DFlashError(-1, "hs must hold five tensors")
    dt = hs[0].dtype
    M = hs[0].shape[0]
    for i, h in enumerate(hs):
        if not h.is_cuda or h.dtype != dt or h.dim() != 2 or h.shape[0] != M or h.stride(1) != 1 \
                or h.stride(0) != hs[0].stride(0) or h.shape[1] < D:
            raise DFlashError(-1, f"hs[{i}] must be a device [M, >=2560] tensor with unit column stride, "
                                  "dtype and row stride equal to hs[0]")
    L = len(k_caches)
    if len(v_caches) != L or not 1 <= L <= 5:
        raise DFlashError(-1, "k_caches and v_caches need the same length in 1..5")
    _need(wc, "wc", dt, (D, NCAPTURE * D))
    _need(gc, "gc", dt, (D,))
    _need(wkv, "wkv", dt, (L * 2048, D))
    _need(gk, "gk", dt, (L, HEAD_DIM))
    _need(pos, "pos", torch.int32, (M,))
    _need(slot, "slot", torch.int64, (M,))
    npages = k_caches[0].shape[0]
    for i in range(L):
        _need(k_caches[i], f"k_caches[{i}]", dt, (npages, HKV, 2048))
        _need(v_caches[i], f"v_caches[{i}]", dt, (npages, HKV, 2048))
    if ht_out is not None:
        _need(ht_out, "ht_out", dt, (M, D))
    a = FuseArgs()
    a.dtype = _dtype_code(hs[0])
    a.num_layers = L
    a.M = M
    for i in range(5):
        a.hs[i] = hs[i].data_ptr()
    a.hs_stride = hs[0].stride(0)
    a.wc, a.gc, a.wkv, a.gk = wc.data_ptr(), gc.data_ptr(), wkv.data_ptr(), gk.data_ptr()
    a.eps, a.rope_theta = eps, rope_theta
    a.pos, a.slot = pos.data_ptr(), slot.data_ptr()
    for i in range(L):
        a.k_cache[i] = k_caches[i].data_ptr()
        a.v_cache[i] = v_caches[i].data_ptr()
    a.num_pages = npages
    a.ht_out = None if ht_out is None else ht_out.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_fuse_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, hs[0].device)
    return Prepared(lib.dflash_ctx_fuse, a, ws, wsb,
                    (list(hs), wc, gc, wkv, gk, pos, slot, list(k_caches), list(v_caches), ht_out))


def ctx_fuse(*args, stream=None, **kw):
    prepare_ctx_fuse(*args, **kw)(stream)


# ---------------------------------------------------------------- block_attn
def prepare_block_attn(q, k_blk, v_blk, gq, gk, k_cache, v_cache, block_table, ctx_len, out=None,
                       lse_out=None, eps=1e-6, rope_theta=1e6, window=0, split_tokens=0, workspace=None):
    """One draft layer's block attention (include/dflash.h, dflash_block_attn).

    q [B,32,8,128]; k_blk, v_blk [B,8,8,128]; gq, gk [128]; caches
    [num_pages, 8, 2048] in the page layout; block_table int32 [B, max_pages];
    ctx_len int32 [B]; out [B,32,8,128] (allocated if None); lse_out float32
    [B,32,8] or None.
    """
    lib = load()
    dt = q.dtype
    B = q.shape[0]
    _need(q, "q", dt, (B, HQ, BLOCK, HEAD_DIM))
    _need(k_blk, "k_blk", dt, (B, HKV, BLOCK, HEAD_DIM))
    _need(v_blk, "v_blk", dt, (B, HKV, BLOCK, HEAD_DIM))
    _need(gq, "gq", dt, (HEAD_DIM,))
    _need(gk, "gk", dt, (HEAD_DIM,))
    npages = k_cache.shape[0]
    _need(k_cache, "k_cache", dt, (npages, HKV, 2048))
    _need(v_cache, "v_cache", dt, (npages, HKV, 2048))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise DFlashError(-1, "block_table must be [B, max_pages]")
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, HQ, BLOCK, HEAD_DIM), dtype=dt, device=q.device)
    _need(out, "out", dt, (B, HQ, BLOCK, HEAD_DIM))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (B, HQ, BLOCK))
    a = AttnArgs()
    a.dtype = _dtype_code(q)
    a.B = B
    a.q, a.k_blk, a.v_blk = q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr()
    a.gq, a.gk = gq.data_ptr(), gk.data_ptr()
    a.eps, a.rope_theta = eps, rope_theta
    a.k_cache, a.v_cache, a.num_pages = k_cache.data_ptr(), v_cache.data_ptr(), npages
    a.block_table, a.max_pages, a.ctx_len = block_table.data_ptr(), block_table.shape[1], ctx_len.data_ptr()
    a.page_size, a.block_len, a.window, a.split_tokens = PAGE, BLOCK, window, split_tokens
    a.out = out.data_ptr()
    a.lse_out = None if lse_out is None else lse_out.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_attn_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, q.device)
    prep = Prepared(lib.dflash_block_attn, a, ws, wsb,
                    (q, k_blk, v_blk, gq, gk, k_cache, v_cache, block_table, ctx_len, out, lse_out))
    prep.out = out
    return prep


def block_attn(*args, stream=None, **kw):
    prep = prepare_block_attn(*args, **kw)
    prep(stream)
    return prep.out


# ---------------------------------------------------------------- spec_verify
def prepare_spec_verify(target_logits, draft_logits, draft_tokens, temperature, seed=0, offset=0,
                        out_tokens=None, out_len=None, near_ties=None, workspace=None, draft_stats=None):
    """Exact speculative verification (include/dflash.h, dflash_spec_verify).

    target_logits [B, 8, V] and draft_logits [B, 7, V] (last dim contiguous;
    any 16-byte-aligned row/batch strides); draft_tokens int32 [B, 7];
    temperature float32 [B] (<= 0: greedy).  Outputs int32 [B, 8], int32 [B]
    and a uint64-sized int64 [1] near-tie counter (allocated if None).
    draft_stats: optional float32 [B, 7, 2] from draft_head (the draft rows'
    softmax statistics; their rows are then not read for statistics).
    """
    lib = load()
    dt = target_logits.dtype
    B, R, V = target_logits.shape
    if R != 8 or tuple(draft_logits.shape) != (B, 7, V) or draft_logits.dtype != dt:
        raise DFlashError(-1, "target_logits must be [B, 8, V] and draft_logits [B, 7, V] of one dtype")
    for n, t in (("target_logits", target_logits), ("draft_logits", draft_logits)):
        if not t.is_cuda or t.stride(2) != 1:
            raise DFlashError(-1, f"{n} must be a device tensor with a contiguous last dim")
    _need(draft_tokens, "draft_tokens", torch.int32, (B, 7))
    _need(temperature, "temperature", torch.float32, (B,))
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, 8), dtype=torch.int32, device=dev)
    if out_len is None:
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if near_ties is None:
        near_ties = torch.zeros((1,), dtype=torch.int64, device=dev)
    _need(out_tokens, "out_tokens", torch.int32, (B, 8))
    _need(out_len, "out_len", torch.int32, (B,))
    _need(near_ties, "near_ties", torch.int64, (1,))
    if draft_stats is not None:
        _need(draft_stats, "draft_stats", torch.float32, (B, 7, 2))
    a = VerifyArgs()
    a.dtype = _dtype_code(target_logits)
    a.B, a.V = B, V
    a.target_logits = target_logits.data_ptr()
    a.t_batch_stride, a.t_row_stride = target_logits.stride(0), target_logits.stride(1)
    a.draft_logits = draft_logits.data_ptr()
    a.d_batch_stride, a.d_row_stride = draft_logits.stride(0), draft_logits.stride(1)
    a.draft_tokens, a.temperature = draft_tokens.data_ptr(), temperature.data_ptr()
    a.seed, a.offset = int(seed), int(offset)
    a.out_tokens, a.out_len, a.near_ties = out_tokens.data_ptr(), out_len.data_ptr(), near_ties.data_ptr()
    a.draft_stats = None if draft_stats is None else draft_stats.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_verify_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, dev)
    prep = Prepared(lib.dflash_spec_verify, a, ws, wsb,
                    (target_logits, draft_logits, draft_tokens, temperature, out_tokens, out_len, near_ties,
                     draft_stats))
    prep.outputs = (out_tokens, out_len, near_ties)
    return prep


def spec_verify(*args, stream=None, **kw):
    prep = prepare_spec_verify(*args, **kw)
    prep(stream)
    return prep.outputs


class PreparedNoAlloc:
    """dflash_spec_verify_noalloc: the library's fixed device scratch, no workspace."""

    def __init__(self, args, keep):
        self.args, self._keep = args, keep

    def __call__(self, stream=None):
        _check(load().dflash_spec_verify_noalloc(ctypes.byref(self.args), _stream(stream)))
        _record(stream, self._keep)


def verify_scratch_bytes():
    """Size of the allocation-free verification's device scratch."""
    n = ctypes.c_size_t()
    _check(load().dflash_verify_scratch_bytes(ctypes.byref(n)))
    return n.value


def prepare_spec_verify_noalloc(target_logits, draft_logits, draft_tokens, temperature, out_tokens, out_len,
                                near_ties, seed=0, offset=0, draft_stats=None):
    """Allocation-free verification (include/dflash.h, dflash_spec_verify_noalloc):
    the arguments of prepare_spec_verify, with every output supplied by the
    caller; nothing is allocated here or in the library."""
    for n, t in (("out_tokens", out_tokens), ("out_len", out_len), ("near_ties", near_ties)):
        if t is None:
            raise DFlashError(-1, f"{n} must be supplied: this entry point allocates nothing")
    prep = prepare_spec_verify(target_logits, draft_logits, draft_tokens, temperature, seed, offset,
                               out_tokens, out_len, near_ties, workspace=_NO_WORKSPACE, draft_stats=draft_stats)
    out = PreparedNoAlloc(prep.args, prep._keep)
    out.outputs = prep.outputs
    return out


def spec_verify_noalloc(*args, stream=None, **kw):
    prep = prepare_spec_verify_noalloc(*args, **kw)
    prep(stream)
    return prep.outputs


# ---------------------------------------------------------------- draft layer
class PreparedEmbed:
    """dflash_draft_embed has no workspace."""

    def __init__(self, args, keep):
        self.args, self._keep = args, keep

    def __call__(self, stream=None):
        _check(load().dflash_draft_embed(ctypes.byref(self.args), _stream(stream)))
        _record(stream, self._keep)


def prepare_draft_embed(emb, anchor, mask_id, x=None):
    """Block input of the first draft layer (include/dflash.h, dflash_draft_embed).

    emb [V, 2560]; anchor int32 [B]; x [B, 8, 2560] (allocated if None).
    """
    load()
    dt = emb.dtype
    _need(emb, "emb", dt)
    if emb.dim() != 2 or emb.shape[1] != D:
        raise DFlashError(-1, "emb must be [V, 2560]")
    B = anchor.shape[0]
    _need(anchor, "anchor", torch.int32, (B,))
    if x is None:
        x = torch.empty((B, BLOCK, D), dtype=dt, device=emb.device)
    _need(x, "x", dt, (B, BLOCK, D))
    a = EmbedArgs()
    a.dtype, a.B, a.V = _dtype_code(emb), B, emb.shape[0]
    a.emb, a.anchor, a.mask_id, a.x = emb.data_ptr(), anchor.data_ptr(), int(mask_id), x.data_ptr()
    prep = PreparedEmbed(a, (emb, anchor, x))
    prep.out = x
    return prep


def draft_embed(*args, stream=None, **kw):
    prep = prepare_draft_embed(*args, **kw)
    prep(stream)
    return prep.out


def prepare_draft_qkv(x, g_in, w_qkv, q=None, k_blk=None, v_blk=None, eps=1e-6, workspace=None):
    """Input RMSNorm + fused Q/K/V projection (include/dflash.h, dflash_draft_qkv).

    x [B, 8, 2560]; g_in [2560]; w_qkv [6144, 2560].  Outputs q [B,32,8,128],
    k_blk and v_blk [B,8,8,128] (allocated if None), the inputs of block_attn.
    """
    lib = load()
    dt = x.dtype
    B = x.shape[0]
    _need(x, "x", dt, (B, BLOCK, D))
    _need(g_in, "g_in", dt, (D,))
    _need(w_qkv, "w_qkv", dt, ((HQ + 2 * HKV) * HEAD_DIM, D))
    dev = x.device
    if q is None:
        q = torch.empty((B, HQ, BLOCK, HEAD_DIM), dtype=dt, device=dev)
    if k_blk is None:
        k_blk = torch.empty((B, HKV, BLOCK, HEAD_DIM), dtype=dt, device=dev)
    if v_blk is None:
        v_blk = torch.empty((B, HKV, BLOCK, HEAD_DIM), dtype=dt, device=dev)
    _need(q, "q", dt, (B, HQ, BLOCK, HEAD_DIM))
    _need(k_blk, "k_blk", dt, (B, HKV, BLOCK, HEAD_DIM))
    _need(v_blk, "v_blk", dt, (B, HKV, BLOCK, HEAD_DIM))
    a = QkvArgs()
    a.dtype, a.B = _dtype_code(x), B
    a.x, a.g_in, a.w_qkv, a.eps = x.data_ptr(), g_in.data_ptr(), w_qkv.data_ptr(), eps
    a.q, a.k_blk, a.v_blk = q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_draft_qkv_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, dev)
    prep = Prepared(lib.dflash_draft_qkv, a, ws, wsb, (x, g_in, w_qkv, q, k_blk, v_blk))
    prep.outputs = (q, k_blk, v_blk)
    return prep


def draft_qkv(*args, stream=None, **kw):
    prep = prepare_draft_qkv(*args, **kw)
    prep(stream)
    return prep.outputs


def prepare_draft_mlp(x, o, w_o, g_post, w_gu, w_d, g_final=None, x_out=None, y_out=None, h_out=None, eps=1e-6,
                      workspace=None, w_conv=None, b_conv=None):
    """Output projection + residual, RMSNorm, SwiGLU MLP + residual and the
    optional final RMSNorm (include/dflash.h, dflash_draft_mlp).

    x [B, 8, 2560] layer input; o [B, 32, 8, 128] attention output;
    w_o [2560, 4096]; g_post [2560]; w_gu [10240, 2560]; w_d [2560, 5120];
    g_final [2560] or None.  Outputs x_out (may be x), with g_final y_out,
    and the stored residual h in h_out when that is given.  With w_conv
    [k, 2560] and b_conv [2560], DFlash2's block convolution h' = h +
    conv(h) runs between the two halves (h_out then holds h').
    """
    lib = load()
    dt = x.dtype
    B = x.shape[0]
    _need(x, "x", dt, (B, BLOCK, D))
    _need(o, "o", dt, (B, HQ, BLOCK, HEAD_DIM))
    _need(w_o, "w_o", dt, (D, HQ * HEAD_DIM))
    _need(g_post, "g_post", dt, (D,))
    _need(w_gu, "w_gu", dt, (2 * INTER, D))
    _need(w_d, "w_d", dt, (D, INTER))
    dev = x.device
    if x_out is None:
        x_out = torch.empty((B, BLOCK, D), dtype=dt, device=dev)
    _need(x_out, "x_out", dt, (B, BLOCK, D))
    if g_final is not None:
        _need(g_final, "g_final", dt, (D,))
        if y_out is None:
            y_out = torch.empty((B, BLOCK, D), dtype=dt, device=dev)
        _need(y_out, "y_out", dt, (B, BLOCK, D))
    if h_out is not None:
        _need(h_out, "h_out", dt, (B, BLOCK, D))
    if (w_conv is None) != (b_conv is None):
        raise DFlashError(-1, "w_conv and b_conv go together")
    if w_conv is not None:
        _need(w_conv, "w_conv", dt, (w_conv.shape[0], D))
        _need(b_conv, "b_conv", dt, (D,))
    a = MlpArgs()
    a.dtype, a.B = _dtype_code(x), B
    a.x, a.o, a.w_o, a.g_post = x.data_ptr(), o.data_ptr(), w_o.data_ptr(), g_post.data_ptr()
    a.w_gu, a.w_d = w_gu.data_ptr(), w_d.data_ptr()
    a.g_final = None if g_final is None else g_final.data_ptr()
    a.eps = eps
    a.x_out = x_out.data_ptr()
    a.y_out = None if y_out is None else y_out.data_ptr()
    a.h_out = None if h_out is None else h_out.data_ptr()
    if w_conv is not None:
        a.conv_k, a.w_conv, a.b_conv = w_conv.shape[0], w_conv.data_ptr(), b_conv.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_draft_mlp_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, dev)
    prep = Prepared(lib.dflash_draft_mlp, a, ws, wsb,
                    (x, o, w_o, g_post, w_gu, w_d, g_final, x_out, y_out, h_out, w_conv, b_conv))
    prep.outputs = (x_out, y_out, h_out)
    return prep


def draft_mlp(*args, stream=None, **kw):
    prep = prepare_draft_mlp(*args, **kw)
    prep(stream)
    return prep.outputs


# ---------------------------------------------------------------- window cache
class PreparedRing:
    """dflash_ring_append has no workspace."""

    def __init__(self, args, keep):
        self.args, self._keep = args, keep

    def __call__(self, stream=None):
        _check(load().dflash_ring_append(ctypes.byref(self.args), _stream(stream)))
        _record(stream, self._keep)


def prepare_ring_append(ring, ctx_len, n_new, rows_per_seq=8, slot=None, pos=None):
    """Slots and positions of a cycle's verified rows in a sliding-window
    cache kept as a ring of pages (include/dflash.h, dflash_ring_append).

    ring int32 [B, R]; ctx_len int32 [B] (advanced in place); n_new int32
    [B].  Outputs slot int64 and pos int32 [B * rows_per_seq] (allocated if
    None), the slot / pos inputs of ctx_fuse.
    """
    load()
    B, R = ring.shape
    _need(ring, "ring", torch.int32, (B, R))
    _need(ctx_len, "ctx_len", torch.int32, (B,))
    _need(n_new, "n_new", torch.int32, (B,))
    dev = ring.device
    if slot is None:
        slot = torch.empty((B * rows_per_seq,), dtype=torch.int64, device=dev)
    if pos is None:
        pos = torch.empty((B * rows_per_seq,), dtype=torch.int32, device=dev)
    _need(slot, "slot", torch.int64, (B * rows_per_seq,))
    _need(pos, "pos", torch.int32, (B * rows_per_seq,))
    a = RingArgs()
    a.B, a.ring_pages, a.rows_per_seq = B, R, rows_per_seq
    a.ring, a.ctx_len, a.n_new = ring.data_ptr(), ctx_len.data_ptr(), n_new.data_ptr()
    a.slot, a.pos = slot.data_ptr(), pos.data_ptr()
    prep = PreparedRing(a, (ring, ctx_len, n_new, slot, pos))
    prep.outputs = (slot, pos)
    return prep


def ring_append(*args, stream=None, **kw):
    prep = prepare_ring_append(*args, **kw)
    prep(stream)
    return prep.outputs



# ---------------------------------------------------------------- LM head
def prepare_draft_head(y, w_head, temperature, seed=0, offset=0, logits=None, draft_tokens=None, workspace=None,
                       draft_stats=None):
    """Shared LM head over the block rows and the seven draft proposals
    (include/dflash.h, dflash_draft_head).

    y [B, 8, 2560] final-norm output; w_head [V, 2560]; temperature float32
    [B] (<= 0: greedy).  Outputs logits [B, 8, V] (dtype of y) and
    draft_tokens int32 [B, 7] (allocated if None); logits[:, 1:] is the
    draft_logits input of spec_verify.  draft_stats: None (not computed),
    True (allocated) or a float32 [B, 7, 2] tensor; it is the draft_stats
    input of spec_verify and is returned as a third output when requested.
    """
    lib = load()
    dt = y.dtype
    B = y.shape[0]
    V = w_head.shape[0]
    _need(y, "y", dt, (B, BLOCK, D))
    _need(w_head, "w_head", dt, (V, D))
    _need(temperature, "temperature", torch.float32, (B,))
    dev = y.device
    if logits is None:
        logits = torch.empty((B, BLOCK, V), dtype=dt, device=dev)
    if draft_tokens is None:
        draft_tokens = torch.empty((B, BLOCK - 1), dtype=torch.int32, device=dev)
    _need(logits, "logits", dt, (B, BLOCK, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, BLOCK - 1))
    if draft_stats is True:
        draft_stats = torch.empty((B, BLOCK - 1, 2), dtype=torch.float32, device=dev)
    if draft_stats is not None:
        _need(draft_stats, "draft_stats", torch.float32, (B, BLOCK - 1, 2))
    a = HeadArgs()
    a.dtype, a.B, a.V = _dtype_code(y), B, V
    a.y, a.w_head, a.temperature = y.data_ptr(), w_head.data_ptr(), temperature.data_ptr()
    a.seed, a.offset = int(seed), int(offset)
    a.logits, a.draft_tokens = logits.data_ptr(), draft_tokens.data_ptr()
    a.draft_stats = None if draft_stats is None else draft_stats.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_draft_head_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, dev)
    prep = Prepared(lib.dflash_draft_head, a, ws, wsb, (y, w_head, temperature, logits, draft_tokens, draft_stats))
    prep.outputs = (logits, draft_tokens) if draft_stats is None else (logits, draft_tokens, draft_stats)
    return prep


def draft_head(*args, stream=None, **kw):
    prep = prepare_draft_head(*args, **kw)
    prep(stream)
    return prep.outputs


# ---------------------------------------------------------------- DFlash2 paths
def prepare_draft_paths(logits, m, P, lam=0.0, cand_ids=None, cand_logp=None, entropy=None, paths=None,
                        scores=None, workspace=None):
    """DFlash2's top-m candidate path selector (include/dflash.h,
    dflash_draft_paths).

    logits [B, 8, V] (rows 1..7 read; last dim contiguous, any 16-byte
    aligned row / batch strides).  Outputs cand_ids int32 [B, 7, m],
    cand_logp float32 [B, 7, m], entropy float32 [B, 7], paths int32
    [B, P, 7] and scores float32 [B, P] (allocated if None).
    """
    lib = load()
    B, R, V = logits.shape
    if R != BLOCK or not logits.is_cuda or logits.stride(2) != 1:
        raise DFlashError(-1, "logits must be a device tensor [B, 8, V] with a contiguous last dim")
    dev = logits.device
    J = BLOCK - 1
    outs = {"cand_ids": (cand_ids, torch.int32, (B, J, m)), "cand_logp": (cand_logp, torch.float32, (B, J, m)),
            "entropy": (entropy, torch.float32, (B, J)), "paths": (paths, torch.int32, (B, P, J)),
            "scores": (scores, torch.float32, (B, P))}
    t = {}
    for name, (x, dt, shape) in outs.items():
        t[name] = torch.empty(shape, dtype=dt, device=dev) if x is None else x
        _need(t[name], name, dt, shape)
    a = PathsArgs()
    a.dtype, a.B, a.V = _dtype_code(logits), B, V
    a.logits, a.batch_stride, a.row_stride = logits.data_ptr(), logits.stride(0), logits.stride(1)
    a.m, a.P, a.lam = m, P, lam
    for name in outs:
        setattr(a, name, t[name].data_ptr())
    nbytes = ctypes.c_size_t()
    _check(lib.dflash_draft_paths_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws, wsb = _workspace(nbytes.value, workspace, dev)
    prep = Prepared(lib.dflash_draft_paths, a, ws, wsb, (logits,) + tuple(t.values()))
    prep.outputs = tuple(t[n] for n in outs)
    return prep


def draft_paths(*args, stream=None, **kw):
    prep = prepare_draft_paths(*args, **kw)
    prep(stream)
    return prep.outputs


# ---------------------------------------------------------------- calibration
def calib_sink(device="cuda"):
    n = ctypes.c_size_t()
    _check(load().dflash_calib_sink_bytes(ctypes.byref(n)))
    return torch.empty(n.value, dtype=torch.uint8, device=device)


def calib_stream(src, sink, dst=None, grid=0, stream=None):
    """Read (dst None) or copy (dst given) every byte of src once over `grid`
    workgroups (0: the default)."""
    nbytes = src.numel() * src.element_size()
    _check(load().dflash_calib_stream(_ptr(src), _ptr(dst), nbytes, int(grid), _ptr(sink), _stream(stream)))
    return nbytes


def calib_gather(src, chunk_ids, chunk_bytes, sink, grid=0, stream=None):
    """Read the chunk_bytes-sized chunks of src listed in chunk_ids (device
    int32) in that order over `grid` workgroups (0: the default); returns
    nchunks x chunk_bytes."""
    nbytes = src.numel() * src.element_size()
    if chunk_ids.dtype != torch.int32 or not chunk_ids.is_contiguous():
        raise DFlashError("calib_gather: chunk_ids must be contiguous int32")
    _check(load().dflash_calib_gather(_ptr(src), nbytes, _ptr(chunk_ids), chunk_ids.numel(), int(chunk_bytes),
                                      int(grid), _ptr(sink), _stream(stream)))
    return chunk_ids.numel() * int(chunk_bytes)


def calib_mfma(iters, sink, stream=None):
    """Register-only bf16 MFMA loop; returns the launch's FLOPs."""
    f = ctypes.c_double()
    _check(load().dflash_calib_mfma(int(iters), _ptr(sink), ctypes.byref(f), _stream(stream)))
    return f.value
