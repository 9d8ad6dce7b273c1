"""Draft-verify cycle benchmark on one MI355X.

One step = one DFlash draft-verify cycle's hot path on the serving batch:
  ctx_fuse  of the newly verified rows (1..8 per sequence) into 5 layer caches
  5 x block_attn (one per draft layer, over ctx_len + new rows)
  spec_verify over [64, 8, 262144] target and [64, 7, 262144] draft logits
Inputs are synthetic and already resident in HBM when timing starts.  The K
timed steps are first run eagerly (per-kernel HIP events; "eager_ms_per_step")
and then replayed from one HIP graph per step, captured with the same Philox
offsets (the reported "ms_per_step" and value): the same kernels and work,
without the per-launch gaps of 13 back-to-back launches.  Prints one JSON line
(rank 0) with cycles/s, the attention roofline and an oracle CPU baseline on a
bounded sample.

After the timed cycles (outside the timed region) it also times the prefill
workload's context fusion (one 32768-token prompt: the [32768,12800]x[12800,2560]
fusion GEMM, the five layers' K/V projection with k_norm + RoPE + cache write)
and its verify-only step over [256,8,262144] logits at T = 0.7, reported under
"kernels" as the fusion's MFMA fraction and the verification's HBM fraction,
and one layer's block attention over the long-context workload (B = 4
sequences of 131072 cached tokens on shuffled pages: 16 splits of each
sequence and the log-sum-exp merge launch), and the serving batch's draft
forward around block attention (block embedding, 5 x [input norm + Q/K/V
projection, block attention, output projection + SwiGLU MLP], final norm),
whole and its dense part alone, and one layer's attention restricted to the
drafter's 1024-token window.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill] [--eager]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FP32_VECTOR_PEAK_TFLOPS = 157.3 # MI355X fp32 vector
B, S_CTX, V, LAYERS = 64, 8192, 262144, 5
SEED = 2
ATTN_SRC = os.path.join(ROOT, "block_speculative_decoding_amd", "csrc", "attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_attn_serving_b64_s8192_traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the timings outside the serving cycle (prefill fusion, B=256 verify, "
                         "long-context and windowed attention, draft forward)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (default: also replay each step from a HIP graph)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (5 times), the known-size "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only run the prefill fusion at M=32768 (2 warm-up + 5 timed calls) and, as a "
                         "reference on the same two GEMM shapes, torch's bf16 matmul (2 + 5 each): the "
                         "run behind the GEMM counter passes")
    ap.add_argument("--gemm-probe-rows", type=int, default=32768,
                    help="rows M of the --gemm-probe fusion (default 32768, the prefill; 4096 is the "
                         "single-stream context)")
    ap.add_argument("--serving-gemm-probe", action="store_true",
                    help="only time ctx_fuse on the serving batch's new rows in its place in the cycle, "
                         "back to back (weights left in the MALL) and cold (MALL flushed before each "
                         "call), and torch's bf16 matmul on the same two GEMM shapes warm and cold")
    ap.add_argument("--head-gemm-probe", action="store_true",
                    help="only time torch's bf16 matmul (hipBLASLt) on the shared head's shape at the serving "
                         "batch, [512,2560] x [262144,2560]^T with bf16 out, for comparison with the head's "
                         "greedy call")
    return ap.parse_args()


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "repeats": 5}))


def gemm_probe(M=32768):
    """The context fusion at M rows (first GEMM [M,12800] x [12800,2560], the
    K/V GEMM [M,2560] x [2560,10240] with its epilogue; M = 32768 is the
    prefill) and torch's bf16 matmul on the same two shapes, for counter
    passes that compare the matrix pipes' busy fraction, the shader clock and
    the L2 traffic."""
    import torch
    import block_speculative_decoding_amd as dfl
    from block_speculative_decoding_amd import synth
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(SEED + 1)
    hs = [torch.randn((M, 2560), generator=g, device=dev, dtype=torch.float32).to(bf) for _ in range(5)]
    w = {k: torch.from_numpy(np.ascontiguousarray(v)).to(bf).to(dev) for k, v in synth.fuse_weights(SEED, LAYERS).items()}
    npages = M // 16
    kc = [torch.zeros((npages, 8, 2048), dtype=bf, device=dev) for _ in range(LAYERS)]
    vc = [torch.zeros((npages, 8, 2048), dtype=bf, device=dev) for _ in range(LAYERS)]
    pos = torch.arange(M, dtype=torch.int32, device=dev)
    slot = torch.arange(M, dtype=torch.int64, device=dev)
    fuse = dfl.prepare_ctx_fuse(hs, w["wc"], w["gc"], w["wkv"], w["gk"], pos, slot, kc, vc)
    f_ms = timed(torch, fuse)
    flops, _ = fuse_flops_bytes(M)
    del hs, kc, vc, fuse
    torch.cuda.empty_cache()
    a1 = torch.randn((M, 12800), generator=g, device=dev, dtype=torch.float32).to(bf)
    h = torch.randn((M, 2560), generator=g, device=dev, dtype=torch.float32).to(bf)
    wc_t = w["wc"].t().contiguous()
    wkv_t = w["wkv"].t().contiguous()
    t1 = timed(torch, lambda: torch.matmul(a1, wc_t))
    t2 = timed(torch, lambda: torch.matmul(h, wkv_t))
    f1, f2 = 2 * M * 12800 * 2560, 2 * M * 2560 * LAYERS * 2048
    print(json.dumps({"gemm_probe": {
        "M": M, "ctx_fuse_ms": round(f_ms, 4), "ctx_fuse_TFLOP/s": round(flops / (f_ms * 1e-3) / 1e12, 1),
        "torch_matmul_fuse_gemm_ms": round(t1, 4), "torch_matmul_fuse_gemm_TFLOP/s": round(f1 / (t1 * 1e-3) / 1e12, 1),
        "torch_matmul_kv_gemm_ms": round(t2, 4), "torch_matmul_kv_gemm_TFLOP/s": round(f2 / (t2 * 1e-3) / 1e12, 1)}}))


def serving_gemm_probe():
    """ctx_fuse at the serving batch's new rows (302 at the default seed)
    under three cache states, and torch's bf16 matmul (hipBLASLt) on its two
    GEMM shapes: [M,12800] x [2560,12800]^T and [M,2560] x [10240,2560]^T,
    bf16 out, with no reduction, norm or K/V epilogue."""
    import torch
    import block_speculative_decoding_amd as dfl
    from block_speculative_decoding_amd import synth
    dfl.load()
    wl = Workload(torch, dfl, synth)
    for i in range(3):
        wl.step(i)
    torch.cuda.synchronize()
    # In its place: the previous cycle's attention and verification are
    # queued ahead of it, as in the timed steps.
    ts = []
    for i in range(20):
        for a in wl.attn:
            a()
        wl.verify()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wl.fuse()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    r = {"M": int(wl.M), "ctx_fuse_in_cycle_ms": round(float(np.median(ts)), 4),
         "ctx_fuse_back_to_back_ms": round(timed(torch, wl.fuse, reps=20), 4),
         "ctx_fuse_cold_ms": round(timed_cold(torch, wl.fuse, reps=20), 4)}
    # Which traffic evicts the weights: 2 GiB read with nontemporal loads (as
    # attention and verification read) or with plain loads, before each call.
    big = torch.zeros(1 << 31, dtype=torch.uint8, device="cuda")
    sink = dfl.calib_sink()
    for name, before in (("after_2GiB_nontemporal_read", lambda: dfl.calib_stream(big, sink)),
                         ("after_2GiB_plain_read", lambda: big.view(torch.int32).max())):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in ev:
            before()
            e0.record()
            wl.fuse()
            e1.record()
        torch.cuda.synchronize()
        r["ctx_fuse_" + name + "_ms"] = round(sum(a.elapsed_time(b) for a, b in ev) / len(ev), 4)
    del big
    bf = torch.bfloat16
    a1 = torch.cat(list(wl.hs), dim=1).contiguous()
    w = {k: torch.from_numpy(np.ascontiguousarray(v)).to(bf).cuda() for k, v in wl.w_np.items()}
    h = torch.randn((wl.M, 2560), device="cuda").to(bf)
    lin = torch.nn.functional.linear
    for name, fn in (("torch_fuse_gemm", lambda: lin(a1, w["wc"])), ("torch_kv_gemm", lambda: lin(h, w["wkv"]))):
        r[name + "_back_to_back_ms"] = round(timed(torch, fn, reps=20), 4)
        r[name + "_cold_ms"] = round(timed_cold(torch, fn, reps=20), 4)
    print(json.dumps({"serving_gemm_probe": r}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Workload:
    """Serving-batch inputs on the device."""

    def __init__(self, torch, dfl, synth, ctx=None, split_tokens=0):
        self.torch = torch
        dev = torch.device("cuda:0")
        bf = torch.bfloat16
        t0 = time.time()

        def d(x, dt=bf):
            return torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev)

        # Paged caches: ctx 8192 (or the given lengths) + up to 8 new rows per
        # sequence, shuffled pages.
        self.n_new = synth.new_rows(SEED, B)
        self.ctx = np.full(B, S_CTX, dtype=np.int32) if ctx is None else np.asarray(ctx, dtype=np.int32)
        self.lens = (self.ctx + self.n_new).astype(np.int32)
        table, npages = synth.page_table(SEED, self.ctx + 8)
        self.table_np = table
        self.block_table = d(table, torch.int32)
        self.ctx_len = d(self.lens, torch.int32)
        gen = torch.Generator(device=dev).manual_seed(SEED)
        self.kc, self.vc = [], []
        for _ in range(LAYERS):
            self.kc.append(torch.randn((npages, 8, 2048), generator=gen, device=dev, dtype=torch.float32).to(bf))
            self.vc.append(torch.randn((npages, 8, 2048), generator=gen, device=dev, dtype=torch.float32).to(bf))
        # New rows: slots and positions right after each context.
        slots, pos = [], []
        for b in range(B):
            for r in range(self.n_new[b]):
                t = self.ctx[b] + r
                slots.append(table[b, t // 16] * 16 + t % 16)
                pos.append(t)
        self.M = len(slots)
        self.hs_np = synth.capture_states(SEED, self.M)
        self.w_np = synth.fuse_weights(SEED, LAYERS)
        self.hs = [d(h) for h in self.hs_np]
        w = {k: d(v) for k, v in self.w_np.items()}
        self.pos_np = np.array(pos, dtype=np.int32)
        self.fuse = dfl.prepare_ctx_fuse(self.hs, w["wc"], w["gc"], w["wkv"], w["gk"], d(self.pos_np, torch.int32),
                                         d(np.array(slots, dtype=np.int64), torch.int64), self.kc, self.vc)
        # Per-layer block inputs.
        self.blk_np = [synth.attn_block(SEED, B, layer=l) for l in range(LAYERS)]
        self.attn = []
        ws = None
        for l in range(LAYERS):
            bl = {k: d(v) for k, v in self.blk_np[l].items()}
            p = dfl.prepare_block_attn(bl["q"], bl["k_blk"], bl["v_blk"], bl["gq"], bl["gk"], self.kc[l],
                                       self.vc[l], self.block_table, self.ctx_len, split_tokens=split_tokens,
                                       workspace=ws)
            ws = p.workspace  # one workspace shared by the five layers (same stream)
            self.attn.append(p)
        # Logits: N(0, 4^2) target, draft = target + N(0, 1); half greedy, half T = 0.7.
        zt, zd = synth.logits(SEED, B, V, 4.0, 1.0)
        self.temp_np = np.where(np.arange(B) < B // 2, 0.0, 0.7).astype(np.float32)
        self.zt, self.zd = d(zt), d(zd)
        del zt, zd
        self.d_np = synth.sample_drafts(SEED, self.zd.float().cpu().numpy(), self.temp_np)
        self.verify = dfl.prepare_spec_verify(self.zt, self.zd, d(self.d_np, torch.int32),
                                              d(self.temp_np, torch.float32), seed=SEED, offset=0)
        torch.cuda.synchronize()
        log(f"[bench] inputs ready in {time.time() - t0:.1f}s: M={self.M} new rows, "
            f"{npages} pages/layer, cache {LAYERS * 2 * self.kc[0].numel() * 2 / 1e9:.2f} GB")

    def step(self, offset, ev=None):
        self.verify.args.offset = offset
        if ev is None:
            self.fuse()
            for a in self.attn:
                a()
            self.verify()
            return
        ev["fuse"][0].record()
        self.fuse()
        ev["fuse"][1].record()
        for a in self.attn:
            e0, e1 = ev["attn"].pop()
            e0.record()
            a()
            e1.record()
            ev["attn_done"].append((e0, e1))
        ev["verify"][0].record()
        self.verify()
        ev["verify"][1].record()


def attn_bytes(lens):
    """Algorithmic bytes of one block_attn launch: K and V of every cached
    token (8 heads x 128 x bf16 x 2) plus q, block K/V and out per sequence."""
    per_seq = 32 * 8 * 128 * 2 * 2 + 2 * 8 * 8 * 128 * 2
    return int(np.sum(lens.astype(np.int64) * 4096) + len(lens) * per_seq)


def verify_bytes(temp):
    # One pass over the rows the decisions need: 8 target rows of a greedy
    # sequence; target rows 0..6 and draft rows 0..6 of a sampled one (its
    # bonus draw at row 7 needs no normaliser).
    rows = np.where(temp > 0, 14, 8)
    return int(rows.sum() * V * 2)


def fuse_flops_bytes(M):
    flops = 2 * M * (12800 * 2560 + LAYERS * 2048 * 2560)
    bytes_ = (12800 * 2560 + LAYERS * 2048 * 2560) * 2 + M * (5 * 2560 * 2 + LAYERS * 2048 * 2)
    return flops, bytes_


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_per_launch():
    """HBM bytes per block_attn launch from the committed rocprofv3 counter
    summary (lines "key: value"), if it was taken on the current kernel
    source; else None."""
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_FILE).read().splitlines() if ":" in l)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("attn_src_sha256_16") != src_hash(ATTN_SRC):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload and scaled to one full cycle: the fusion of all new rows,
    block attention of 32 of the 64 sequences in each of the 5 layers (x2) and
    verification of all 64 sequences (32 greedy + 32 sampled)."""
    import oracle
    from threadpoolctl import threadpool_info
    from tests.layout import k_offsets, v_offsets, unpack
    torch = wl.torch
    t0 = time.perf_counter()
    oracle.ctx_fuse_ref([h.astype(np.float64) for h in wl.hs_np], wl.w_np["wc"], wl.w_np["gc"], wl.w_np["wkv"],
                        wl.w_np["gk"], wl.pos_np)
    t_fuse = time.perf_counter() - t0
    sample_b = list(range(0, B, 2))
    t_attn = 0.0
    for l in range(LAYERS):
        for b in sample_b:
            pages = torch.from_numpy(wl.table_np[b][wl.table_np[b] >= 0].astype(np.int64)).cuda()
            kb = wl.kc[l].index_select(0, pages).float().cpu().numpy()
            vb = wl.vc[l].index_select(0, pages).float().cpu().numpy()
            loc = np.arange(len(pages))
            kctx = unpack(kb, loc, int(wl.lens[b]), k_offsets()).astype(np.float64)
            vctx = unpack(vb, loc, int(wl.lens[b]), v_offsets()).astype(np.float64)
            blk = wl.blk_np[l]
            t1 = time.perf_counter()
            oracle.block_attn_ref(blk["q"][b:b + 1], blk["k_blk"][b:b + 1], blk["v_blk"][b:b + 1], blk["gq"],
                                  blk["gk"], [kctx], [vctx], wl.lens[b:b + 1])
            t_attn += time.perf_counter() - t1
    vb_sel = list(range(B))
    t_ver = 0.0
    traces = []
    for b in vb_sel:
        zt = wl.zt[b:b + 1].float().cpu().numpy()
        zd = wl.zd[b:b + 1].float().cpu().numpy()
        t1 = time.perf_counter()
        traces.append(oracle.spec_verify_ref(zt, zd, wl.d_np[b:b + 1], wl.temp_np[b:b + 1], SEED, 0,
                                             batch_offset=b))
        t_ver += time.perf_counter() - t1
    wl.verify_traces = traces
    cycle = t_fuse + t_attn * (B / len(sample_b)) + t_ver * (B / len(vb_sel))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": round(1.0 / cycle, 6), "unit": "cycles/s", "cores": int(threads), "kind": "oracle",
        "host": {"cpu_count": os.cpu_count(), "model": host_cpu_model()},
        "sample": (f"float64 numpy oracle: fusion of all {wl.M} new rows ({t_fuse:.2f}s), block attention of "
                   f"32 of 64 sequences x 5 layers ({t_attn:.2f}s, scaled x2), verification of all 64 "
                   f"sequences, 32 greedy + 32 sampled ({t_ver:.2f}s); "
                   f"{t_fuse + t_attn + t_ver:.1f}s measured, {cycle:.1f}s per scaled cycle"),
    }


def head_gemm_probe():
    """torch's bf16 matmul (hipBLASLt) on the shared LM head's product at the
    serving batch: 64 sequences x 8 block rows against a 262144-row head of
    width 2560, bf16 out (268 MB), with no sampling fold."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(SEED)
    a = torch.randn(512, 2560, device=dev, generator=g).to(torch.bfloat16)
    w = (torch.randn(262144, 2560, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    out = torch.empty(512, 262144, device=dev, dtype=torch.bfloat16)
    ms = timed(torch, lambda: torch.matmul(a, w.t(), out=out), warmup=3, reps=20)
    fl = 2 * 512 * 262144 * 2560
    print(json.dumps({"head_gemm_probe": {"shape": "[512,2560] x [262144,2560]^T -> bf16", "torch_matmul_ms": round(ms, 4),
                                          "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1)}}), flush=True)


def timed(torch, fn, warmup=2, reps=5):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def timed_cold(torch, fn, reps=10):
    """Average time of fn with the MALL (256 MB) flushed before every rep by
    writing a 512 MiB buffer; only fn is inside the events."""
    flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda:0")
    fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        flush.fill_(reps)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    del flush
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps


def prefill_measurements(torch, dfl, synth):
    """Prefill workload: ctx_fuse of a 32768-token prompt into 5 layer caches
    (slots 0..32767 in order), then one verify-only step over B = 256."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(SEED + 1)
    M = 32768
    hs = [torch.randn((M, 2560), generator=g, device=dev, dtype=torch.float32).to(bf) for _ in range(5)]
    w = {k: torch.from_numpy(np.ascontiguousarray(v)).to(bf).to(dev) for k, v in synth.fuse_weights(SEED, LAYERS).items()}
    npages = M // 16
    kc = [torch.zeros((npages, 8, 2048), dtype=bf, device=dev) for _ in range(LAYERS)]
    vc = [torch.zeros((npages, 8, 2048), dtype=bf, device=dev) for _ in range(LAYERS)]
    pos = torch.arange(M, dtype=torch.int32, device=dev)
    slot = torch.arange(M, dtype=torch.int64, device=dev)
    fuse = dfl.prepare_ctx_fuse(hs, w["wc"], w["gc"], w["wkv"], w["gk"], pos, slot, kc, vc)
    f_ms = timed(torch, fuse)
    flops, _ = fuse_flops_bytes(M)
    del hs, kc, vc, fuse
    # Verify-only step: B = 256, N(0, 4^2) target, draft = target + N(0, 1), T = 0.7.
    Bv = 256
    zt = (4.0 * torch.randn((Bv, 8, V), generator=g, device=dev, dtype=torch.float32)).to(bf)
    zd = (zt[:, :7].float() + torch.randn((Bv, 7, V), generator=g, device=dev, dtype=torch.float32)).to(bf)
    temp = torch.full((Bv,), 0.7, dtype=torch.float32, device=dev)
    u = torch.rand((Bv, 7, V), generator=g, device=dev).clamp_(1e-7, 1 - 1e-7)
    d = (zd.float() / 0.7 - torch.log(-torch.log(u))).argmax(-1).to(torch.int32)
    del u
    ver = dfl.prepare_spec_verify(zt, zd, d, temp, seed=SEED, offset=0)
    v_ms = timed(torch, ver)
    v_bytes = verify_bytes(temp.cpu().numpy())
    out = {"prefill_ctx_fuse_m32768": {"ms": round(f_ms, 4), "M": M,
                                       "TFLOP/s": round(flops / (f_ms * 1e-3) / 1e12, 1),
                                       "mfma_frac": round(flops / (f_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
           "prefill_verify_b256": {"ms": round(v_ms, 4), "GB/s": round(v_bytes / (v_ms * 1e-3) / 1e9, 1),
                                   "hbm_frac": round(v_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "algorithmic_bytes": v_bytes}}
    del zt, zd, ver
    torch.cuda.empty_cache()
    return out


def config_measurements(torch, dfl, synth):
    """The smaller configurations, each as its own cycle (eager, 20 reps after
    warm-up; per-kernel times from the same kind of loop):
    tiny fp32  -- B = 1, S = 128: ctx_fuse of the 128 context rows (one layer),
                  block attention over them, verify over V = 4096 (target and
                  draft N(0, 3^2), independent) at T = 1 and greedy;
    single     -- B = 1, S = 4096 bf16: ctx_fuse of the 4096 context rows into
                  5 layers ([4096,12800]x[12800,2560] + K/V of 5 layers), 5 x
                  block attention over 4096 cached tokens, verify over
                  V = 262144 at T = 1 (draft = target + N(0, 1));
    long-context verify -- B = 4, V = 262144, T = 1 (draft = target + N(0, 1)).
    Launch-bound at these sizes: reported as latency, with the fusion's MFMA
    fraction where it is a real contraction (M = 4096)."""
    dev = torch.device("cuda:0")
    out = {}

    def cycle_of(fuse, attns, ver):
        def run():
            fuse()
            for a in attns:
                a()
            ver()
        return run

    for name, dt, M, L, Vc, sig, T in (("tiny_fp32_cycle_b1_s128", torch.float32, 128, 1, 4096, 3.0, 1.0),
                                        ("single_stream_cycle_b1_s4096", torch.bfloat16, 4096, LAYERS, V, 4.0, 1.0)):
        d = lambda x, t=dt: torch.from_numpy(np.ascontiguousarray(x)).to(t).to(dev)
        seed = SEED + 10 + M
        hs = [d(h) for h in synth.capture_states(seed, M)]
        w = {k: d(v) for k, v in synth.fuse_weights(seed, L).items()}
        table, npages = synth.page_table(seed, [M + 8])
        kc = [torch.zeros((npages, 8, 2048), dtype=dt, device=dev) for _ in range(L)]
        vc = [torch.zeros((npages, 8, 2048), dtype=dt, device=dev) for _ in range(L)]
        slot = np.array([table[0, t // 16] * 16 + t % 16 for t in range(M)], dtype=np.int64)
        fuse = dfl.prepare_ctx_fuse(hs, w["wc"], w["gc"], w["wkv"], w["gk"],
                                    torch.arange(M, dtype=torch.int32, device=dev), d(slot, torch.int64), kc, vc)
        bt = d(table, torch.int32)
        cl = torch.tensor([M], dtype=torch.int32, device=dev)
        attns = []
        for l in range(L):
            blk = {k: d(v) for k, v in synth.attn_block(seed, 1, layer=l).items()}
            attns.append(dfl.prepare_block_attn(blk["q"], blk["k_blk"], blk["v_blk"], blk["gq"], blk["gk"],
                                                kc[l], vc[l], bt, cl))
        if dt == torch.float32:
            zt = synth.normal(seed, "zt_tiny", (1, 8, Vc), std=sig)
            zd = synth.normal(seed, "zd_tiny", (1, 7, Vc), std=sig)
        else:
            zt, zd = synth.logits(seed, 1, Vc, sig, 1.0)
        zt_d, zd_d = d(zt), d(zd)
        temp = np.array([T], dtype=np.float32)
        dr = d(synth.sample_drafts(seed, zd_d.float().cpu().numpy(), temp), torch.int32)
        ver = dfl.prepare_spec_verify(zt_d, zd_d, dr, d(temp, torch.float32), seed=SEED, offset=0)
        ver_g = dfl.prepare_spec_verify(zt_d, zd_d, dr, torch.zeros(1, device=dev), seed=SEED, offset=0)
        fuse()
        torch.cuda.synchronize()
        c_ms = timed(torch, cycle_of(fuse, attns, ver), warmup=5, reps=20)
        f_ms = timed(torch, fuse, warmup=5, reps=20)
        a_ms = timed(torch, attns[0], warmup=5, reps=20)
        v_ms = timed(torch, ver, warmup=5, reps=20)
        vg_ms = timed(torch, ver_g, warmup=5, reps=20)
        flops, _ = fuse_flops_bytes(M) if L == LAYERS else (2 * M * (12800 * 2560 + L * 2048 * 2560), 0)
        a_bytes = attn_bytes(np.array([M]))
        ent = {"cycle_ms": round(c_ms, 4), "layers": L, "dtype": "f32" if dt == torch.float32 else "bf16",
               "ctx_fuse_ms": round(f_ms, 4), "ctx_fuse_rows": M,
               "ctx_fuse_TFLOP/s": round(flops / (f_ms * 1e-3) / 1e12, 2),
               "block_attn_ms": round(a_ms, 4), "block_attn_GB/s": round(a_bytes / (a_ms * 1e-3) / 1e9, 1),
               "verify_ms": round(v_ms, 4), "verify_greedy_ms": round(vg_ms, 4), "V": Vc,
               "timing": "eager, warm (the working set fits the 256 MB MALL)"}
        if dt == torch.bfloat16:
            ent["ctx_fuse_mfma_frac"] = round(flops / (f_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        else:
            ent["ctx_fuse_fp32_vector_frac"] = round(flops / (f_ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS, 4)
        out[name] = ent
        del hs, w, kc, vc, fuse, attns, ver, ver_g, zt_d, zd_d
        torch.cuda.empty_cache()

    # Long-context workload's verify: B = 4, V = 262144, T = 1.
    Bv = 4
    zt, zd = synth.logits(SEED + 3, Bv, V, 4.0, 1.0)
    d = lambda x, t=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(x)).to(t).to(dev)
    zt_d, zd_d = d(zt), d(zd)
    temp = np.ones(Bv, dtype=np.float32)
    dr = d(synth.sample_drafts(SEED + 3, zd_d.float().cpu().numpy(), temp), torch.int32)
    ver = dfl.prepare_spec_verify(zt_d, zd_d, dr, d(temp, torch.float32), seed=SEED, offset=0)
    v_ms = timed(torch, ver, warmup=5, reps=20)
    vb = verify_bytes(temp)
    out["long_context_verify_b4"] = {"ms": round(v_ms, 4), "GB/s": round(vb / (v_ms * 1e-3) / 1e9, 1),
                                     "hbm_frac": round(vb / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": vb,
                                     "timing": "eager, warm (29 MB: MALL-resident, latency-bound)"}
    return out


def measured_peaks(torch, dfl):
    """Practical ceilings of the part measured in the same run with the
    library's calibration kernels (dflash_calib_*): a streaming read of
    4 GiB with 16-byte loads, the same 4 GiB gathered as randomly ordered
    8-KiB or 32-KiB chunks, a 2 GiB copy (read + write bytes), and a
    register-only bf16 MFMA loop; for reference also torch's bf16 matmul
    8192^3 (hipBLASLt, N(0, 1) operands).  The roofline fractions stay
    against the datasheet peaks; these say how much of them the part
    delivers to any kernel."""
    dev = torch.device("cuda:0")
    sink = dfl.calib_sink(dev)
    x = torch.empty(1 << 32, dtype=torch.uint8, device=dev).random_()
    grids = (256, 512, 1024, 2048, 4096, 8192, 16384)
    r_all = {gd: timed(torch, lambda: dfl.calib_stream(x, sink, grid=gd), warmup=2, reps=5) for gd in grids}
    r_grid = min(r_all, key=r_all.get)
    r_ms = r_all[r_grid]
    # The same 4 GiB read as chunks in a random order: the access pattern of
    # shuffled cache pages (attention reads 8-KiB runs of 32-KiB pages).
    gen = torch.Generator(device=dev).manual_seed(SEED)
    gather = {}
    for cb in (8192, 32768):
        ids = torch.randperm((1 << 32) // cb, generator=gen, device=dev).to(torch.int32)
        best = min(timed(torch, lambda: dfl.calib_gather(x, ids, cb, sink, grid=gd), warmup=2, reps=5)
                   for gd in (256, 1024, 2048, 4096))
        gather[f"{cb // 1024}KiB"] = round((1 << 32) / (best * 1e-3) / 1e9, 1)
        del ids
    src = x[: 1 << 31]
    dst = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    c_ms = timed(torch, lambda: dfl.calib_stream(src, sink, dst=dst, grid=r_grid), warmup=3, reps=10)
    del x, src, dst
    iters = 20000
    flops = dfl.calib_mfma(iters, sink)
    f_ms = timed(torch, lambda: dfl.calib_mfma(iters, sink), warmup=2, reps=5)
    a = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
    m_ms = timed(torch, lambda: torch.matmul(a, b), warmup=3, reps=10)
    del a, b
    torch.cuda.empty_cache()
    read = (1 << 32) / (r_ms * 1e-3) / 1e9
    mfma = flops / (f_ms * 1e-3) / 1e12
    return {"read_GB/s": round(read, 1), "read_frac_of_datasheet": round(read / HBM_PEAK_GBS, 4),
            "read_grid_sweep_GB/s": {str(gd): round((1 << 32) / (ms * 1e-3) / 1e9, 1) for gd, ms in r_all.items()},
            "gather_random_chunks_GB/s": gather,
            "copy_GB/s": round(2 * (1 << 31) / (c_ms * 1e-3) / 1e9, 1),
            "mfma_loop_TFLOP/s": round(mfma, 1), "mfma_loop_frac_of_datasheet": round(mfma / MFMA_BF16_PEAK_TFLOPS, 4),
            "torch_matmul_bf16_TFLOP/s": round(2 * 8192 ** 3 / (m_ms * 1e-3) / 1e12, 1),
            "how": ("dflash_calib_stream over 4 GiB (read; best of a grid sweep) and 2 GiB (copy, read+write "
                    "bytes); dflash_calib_gather over the same 4 GiB as 8-KiB or 32-KiB chunks in a random order "
                    "(best of 256-4096 workgroups); dflash_calib_mfma "
                    f"({iters} rounds of 8 bf16 32x32x16 MFMAs per wave, 2 waves per SIMD); torch.matmul bf16 "
                    "8192^3")}


def long_context_measurement(torch, dfl, synth):
    """One layer's block attention over 4 sequences of 131072 cached tokens
    (shuffled 16-token pages, 2.15 GB of K and V): split-K over each sequence,
    then the log-sum-exp merge."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    Bl, Sl = 4, 131072
    lens = np.full(Bl, Sl, dtype=np.int32)
    table, npages = synth.page_table(SEED + 2, lens)
    g = torch.Generator(device=dev).manual_seed(SEED + 2)
    kc = torch.randn((npages, 8, 2048), generator=g, device=dev, dtype=torch.float32).to(bf)
    vc = torch.randn((npages, 8, 2048), generator=g, device=dev, dtype=torch.float32).to(bf)
    blk = {k: torch.from_numpy(np.ascontiguousarray(v)).to(bf).to(dev) for k, v in synth.attn_block(SEED + 2, Bl).items()}
    att = dfl.prepare_block_attn(blk["q"], blk["k_blk"], blk["v_blk"], blk["gq"], blk["gk"], kc, vc,
                                 torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev))
    ms = timed(torch, att, warmup=2, reps=10)
    nbytes = attn_bytes(lens)
    out = {"long_context_attn_b4_s131072": {
        "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
        "merge_launch": bool(att.ws_bytes)}}
    del kc, vc, att
    torch.cuda.empty_cache()
    return out


def window_measurement(torch, dfl, wl):
    """One layer's block attention at the serving batch restricted to the
    latest 1024 cached tokens (the drafter's window)."""
    W = 1024
    blk = wl.blk_np[0]
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to("cuda:0")
    att = dfl.prepare_block_attn(d(blk["q"]), d(blk["k_blk"]), d(blk["v_blk"]), d(blk["gq"]), d(blk["gk"]),
                                 wl.kc[0], wl.vc[0], wl.block_table, wl.ctx_len, window=W)
    ms = timed(torch, att, warmup=3, reps=20)
    cold = timed_cold(torch, att)
    nbytes = attn_bytes(np.minimum(wl.lens, W))
    return {"window_attn_b64_w1024": {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                      "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      "cold_ms": round(cold, 4),
                                      "cold_hbm_frac": round(nbytes / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      "algorithmic_bytes": nbytes,
                                      "timing": "ms: warm (repeated; the 279 MB working set is about the "
                                                "MALL's size); cold_ms: MALL flushed before each launch"}}


def draft_measurement(torch, dfl, synth, wl):
    """The serving batch's draft forward around block attention: the block
    embedding, then per layer the input norm + Q/K/V projection, block
    attention over the workload's caches and the output projection + MLP
    (final norm after the last layer).  Reports the whole forward and its
    dense part (embedding, projections, norms, MLP) on its own."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(SEED + 3)
    emb = torch.randn((V, 2560), generator=g, device=dev, dtype=torch.float32).to(bf)
    anchors = torch.from_numpy(synth.anchors(SEED, B, V)).to(dev)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
    embed = dfl.prepare_draft_embed(emb, anchors, 3)
    x = embed.out
    dense, layers = [embed], []
    y = torch.empty_like(x)
    for l in range(LAYERS):
        w = {k: d(v) for k, v in synth.draft_layer_weights(SEED, l).items()}
        blk = wl.blk_np[l]
        qkv = dfl.prepare_draft_qkv(x, w["g_in"], w["w_qkv"])
        q, kb, vb = qkv.outputs
        att = dfl.prepare_block_attn(q, kb, vb, d(blk["gq"]), d(blk["gk"]), wl.kc[l], wl.vc[l],
                                     wl.block_table, wl.ctx_len)
        last = l == LAYERS - 1
        mlp = dfl.prepare_draft_mlp(x, att.out, w["w_o"], w["g_post"], w["w_gu"], w["w_d"],
                                    g_final=d(synth.final_norm(SEED)) if last else None, x_out=x,
                                    y_out=y if last else None)
        layers.append((qkv, att, mlp))
        dense += [qkv, mlp]

    def forward():
        embed()
        for qkv, att, mlp in layers:
            qkv()
            att()
            mlp()

    def dense_only():
        for p in dense:
            p()

    f_ms = timed(torch, forward, warmup=2, reps=10)
    d_ms = timed(torch, dense_only, warmup=2, reps=10)
    # One layer's output projection + MLP with DFlash2's block convolution
    # (k = 5) between the halves, against the same call without it.
    w0 = {k: d(v) for k, v in synth.draft_layer_weights(SEED, 0).items()}
    wc, bc = (d(v) for v in synth.conv_weights(SEED, 5))
    o0 = layers[0][1].out
    xs = torch.empty_like(x)
    plain = dfl.prepare_draft_mlp(x, o0, w0["w_o"], w0["g_post"], w0["w_gu"], w0["w_d"], x_out=xs)
    conv = dfl.prepare_draft_mlp(x, o0, w0["w_o"], w0["g_post"], w0["w_gu"], w0["w_d"], x_out=xs, w_conv=wc,
                                 b_conv=bc, workspace=plain.workspace)
    pl_ms = timed(torch, plain, warmup=2, reps=10)
    cv_ms = timed(torch, conv, warmup=2, reps=10)
    per_layer = (6144 * 2560 + 2560 * 4096 + 10240 * 2560 + 2560 * 5120)
    M = 8 * B
    flops = 2 * M * per_layer * LAYERS
    # Algorithmic bytes: every weight once, plus per layer and block row the
    # layer input (read twice: projection and residual), Q/K/V out, the
    # attention output in and the layer output; the embedding writes M rows.
    nbytes = per_layer * 2 * LAYERS + LAYERS * M * 2 * (2 * 2560 + 6144 + 4096 + 2560) + M * 2560 * 2
    del emb, embed, dense, layers, plain, conv
    torch.cuda.empty_cache()
    return {"draft_forward_b64": {"ms": round(f_ms, 4), "layers": LAYERS, "block_rows": M},
            "draft_mlp_block_conv_b64": {"ms": round(cv_ms, 4), "without_conv_ms": round(pl_ms, 4), "k": 5},
            "draft_dense_b64": {"ms": round(d_ms, 4), "TFLOP/s": round(flops / (d_ms * 1e-3) / 1e12, 1),
                                "mfma_frac": round(flops / (d_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                "GB/s": round(nbytes / (d_ms * 1e-3) / 1e9, 1),
                                "hbm_frac": round(nbytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "weight_bytes": per_layer * 2 * LAYERS}}


def ragged_measurement(torch, dfl, synth):
    """The serving batch with ragged cached contexts, uniform on [1024, 8192]
    (mean ~4.6k) on shuffled pages: whole cycles (fusion of the new rows, 5
    attention layers, verification) eagerly, and attention per layer; once
    with the automatic split (one split per sequence: the batch alone fills
    the chip, and the host does not see the lengths) and once with balanced
    pieces (split_tokens = -1, for a caller whose batch mixes lengths: equal
    shares of all sequences' tiles per workgroup, cut sequences merged)."""
    ctx = synth.ragged_lengths(SEED + 5, B, 1024, 8192)
    out = {}
    for split in (0, -1):
        wl = Workload(torch, dfl, synth, ctx=ctx, split_tokens=split)
        step_ms = timed(torch, lambda: wl.step(0), warmup=2, reps=10)
        a_ms = timed(torch, lambda: [a() for a in wl.attn], warmup=2, reps=10) / LAYERS
        a_bytes = attn_bytes(wl.lens)
        out["serving_ragged_b64" + ("_balanced" if split else "")] = {
            "cycles/s_eager": round(1000.0 / step_ms, 1), "ms_per_step_eager": round(step_ms, 4),
            "mean_ctx": round(float(np.mean(wl.lens)), 1), "attn_ms": round(a_ms, 4),
            "attn_GB/s": round(a_bytes / (a_ms * 1e-3) / 1e9, 1),
            "attn_hbm_frac": round(a_bytes / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "split_tokens": "balanced pieces" if split else "auto (one split per sequence)"}
        del wl
        torch.cuda.empty_cache()
    return out


def head_measurement(torch, dfl, synth):
    """The shared LM head over the serving batch's block rows (B = 64, 8 rows
    each, V = 262144) and the seven proposals per sequence, once with the
    batch's temperature mix (a quarter greedy) and once all greedy; the
    difference is the cost of the Gumbel draws."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(SEED + 4)
    y = torch.randn((B, 8, 2560), generator=g, device=dev, dtype=torch.float32).to(bf)
    w = (torch.randn((V, 2560), generator=g, device=dev, dtype=torch.float32) * 0.05).to(bf)
    temp = torch.from_numpy(synth.head_temperatures(SEED, B)).to(dev)
    mixed = dfl.prepare_draft_head(y, w, temp, seed=SEED, offset=0)
    logits, d = mixed.outputs
    greedy = dfl.prepare_draft_head(y, w, torch.zeros_like(temp), seed=SEED, offset=0, logits=logits,
                                    draft_tokens=d, workspace=mixed.workspace)
    m_ms = timed(torch, mixed, warmup=2, reps=10)
    g_ms = timed(torch, greedy, warmup=2, reps=10)
    # NEXT-2's statistics half: the head also folds the sampled proposal rows'
    # softmax statistics, and verification takes them instead of reading the
    # draft rows.  Timed as head + verify over the same logits, against head
    # + verify that computes them itself (target N(0, 4^2); the head's mix).
    stats = torch.empty((B, 7, 2), dtype=torch.float32, device=dev)
    with_stats = dfl.prepare_draft_head(y, w, temp, seed=SEED, offset=0, logits=logits, draft_tokens=d,
                                        workspace=mixed.workspace, draft_stats=stats)
    s_ms = timed(torch, with_stats, warmup=2, reps=10)
    zt = (4.0 * torch.randn((B, 8, V), generator=g, device=dev, dtype=torch.float32)).to(bf)
    ver_plain = dfl.prepare_spec_verify(zt, logits[:, 1:], d, temp, seed=SEED, offset=0)
    ver_stats = dfl.prepare_spec_verify(zt, logits[:, 1:], d, temp, seed=SEED, offset=0,
                                        workspace=ver_plain.workspace, draft_stats=stats)
    vp_ms = timed(torch, ver_plain, warmup=2, reps=10)
    vs_ms = timed(torch, ver_stats, warmup=2, reps=10)

    def pair(head, ver):
        def run():
            head()
            ver()
        return run
    pp_ms = timed(torch, pair(mixed, ver_plain), warmup=2, reps=10)
    ps_ms = timed(torch, pair(with_stats, ver_stats), warmup=2, reps=10)
    n_samp = int((temp > 0).sum().item())
    v_read_plain = (8 * (B - n_samp) + 14 * n_samp) * V * 2
    v_read_stats = (8 * (B - n_samp) + 7 * n_samp) * V * 2
    # DFlash2's path selector on the head's own logits (rows 1..7): top-4
    # candidates per position, 16 paths.
    paths = dfl.prepare_draft_paths(logits, 4, 16, 0.2)
    p_ms = timed(torch, paths, warmup=2, reps=10)
    p_bytes = 7 * B * V * 2
    M = 8 * B
    flops = 2 * M * V * 2560
    # Algorithmic bytes: the head once, the block rows in, the logits out,
    # the seven proposal rows read back by the sampling pass.
    nbytes = V * 2560 * 2 + M * 2560 * 2 + M * V * 2 + 7 * B * V * 2
    n_sampled = int((temp > 0).sum().item())
    del w, logits, mixed, greedy, paths, with_stats, ver_plain, ver_stats, zt
    torch.cuda.empty_cache()
    return {"head_stats_into_verify_b64": {
                "head_ms": round(m_ms, 4), "head_with_stats_ms": round(s_ms, 4),
                "verify_ms": round(vp_ms, 4), "verify_with_stats_ms": round(vs_ms, 4),
                "head_then_verify_ms": round(pp_ms, 4), "head_with_stats_then_verify_ms": round(ps_ms, 4),
                "sampled_sequences": n_samp,
                "verify_read_bytes": v_read_plain, "verify_with_stats_read_bytes": v_read_stats,
                "verify_with_stats_GB/s": round(v_read_stats / (vs_ms * 1e-3) / 1e9, 1),
                "verify_with_stats_hbm_frac": round(v_read_stats / (vs_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "draft_paths_b64": {"ms": round(p_ms, 4), "m": 4, "P": 16, "V": V,
                                "GB/s": round(p_bytes / (p_ms * 1e-3) / 1e9, 1),
                                "hbm_frac": round(p_bytes / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "algorithmic_bytes": p_bytes},
            "draft_head_b64": {"ms": round(m_ms, 4), "greedy_ms": round(g_ms, 4), "V": V, "block_rows": M,
                               "sampled_sequences": n_sampled,
                               "TFLOP/s": round(flops / (m_ms * 1e-3) / 1e12, 1),
                               "mfma_frac": round(flops / (m_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "GB/s": round(nbytes / (m_ms * 1e-3) / 1e9, 1),
                               "hbm_frac": round(nbytes / (m_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gemm_probe:
        gemm_probe(args.gemm_probe_rows)
        return
    if args.serving_gemm_probe:
        serving_gemm_probe()
        return
    if args.head_gemm_probe:
        head_gemm_probe()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import block_speculative_decoding_amd as dfl
    from block_speculative_decoding_amd import synth
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    dfl.load()
    wl = Workload(torch, dfl, synth)

    for i in range(args.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    K = args.steps
    ev = {"fuse": None, "verify": None, "attn": [], "attn_done": []}
    fuse_ms, attn_ms, ver_ms = [], [], []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_step = []
    for i in range(K):
        per_step.append({"fuse": (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)),
                         "verify": (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)),
                         "attn": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                                  for _ in range(LAYERS)],
                         "attn_done": []})
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        wl.step(args.warmup + i, per_step[i])
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end)
    for e in per_step:
        fuse_ms.append(e["fuse"][0].elapsed_time(e["fuse"][1]))
        ver_ms.append(e["verify"][0].elapsed_time(e["verify"][1]))
        attn_ms.extend(a.elapsed_time(b) for a, b in e["attn_done"])
    eager_step = eager_ms / K
    log(f"[bench] {K} eager steps: {eager_step:.3f} ms/step")
    ms_step = eager_step
    launch = "eager"
    if not args.eager:
        # The same K steps (same Philox offsets) captured as one HIP graph each:
        # identical kernels and work, without per-launch gaps on the stream.
        graphs = []
        for i in range(K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                wl.step(args.warmup + i)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for g in graphs:
            g.replay()
        end.record()
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / K
        launch = "hip graph per step"
        log(f"[bench] {K} graph-replayed steps: {ms_step:.3f} ms/step")

    a_bytes = attn_bytes(wl.lens)
    a_ms = float(np.mean(attn_ms))
    a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
    v_bytes = verify_bytes(wl.temp_np)
    v_ms = float(np.mean(ver_ms))
    f_flops, f_bytes = fuse_flops_bytes(wl.M)
    f_ms = float(np.mean(fuse_ms))
    traffic = traffic_per_launch()
    out_len = wl.verify.outputs[1].float().mean().item()
    f_cold = timed_cold(torch, wl.fuse, reps=20)

    res = {
        "metric": "draft-verify cycles/s @B=64,S=8192; attn/verify HBM GB/s; fuse GEMM MFMA %",
        "value": round(1000.0 / ms_step, 3),
        "unit": "cycles/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "eager_ms_per_step": round(eager_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "serving batch: B=64, cached context 8192 + 1..8 newly verified rows per "
                               "sequence (shuffled 16-token pages), 5 draft layers, ctx-fuse of the new rows, "
                               "block attention per layer, spec-verify over V=262144 (32 greedy, 32 at T=0.7)",
                   "B": B, "S": S_CTX, "new_rows": int(wl.M), "layers": LAYERS, "V": V, "parallelism": "none",
                   "launch": launch},
        "roofline": {"kernel": "block_attn (attn_bf16_kernel" + (" + attn_merge_kernel)" if wl.attn[0].ws_bytes else
                                                                  ", one split per sequence: no merge launch)"),
                     "bound": "hbm",
                     "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(a_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic / (a_ms * 1e-3) / 1e9, 1),
                     "algorithmic_bytes_per_launch": a_bytes, "avg_launch_ms": round(a_ms, 4)},
        "kernels": {
            "timing": ("cycle kernels: per-launch events inside the eager timed steps.  Attention (2.16 GB "
                       "per launch) and verify (369 MB of logits) read with nontemporal loads, which do not "
                       "allocate in the 256 MB MALL, so both read HBM (cold).  For the same reason ctx_fuse's "
                       "weights (118 MB) stay in the MALL from one cycle to the next (warm); its cold time, "
                       "with the MALL flushed before each call, is ctx_fuse.cold_ms"),
            "block_attn": {"ms": round(a_ms, 4), "GB/s": round(a_gbs, 1), "hbm_frac": round(a_gbs / HBM_PEAK_GBS, 4)},
            "spec_verify": {"ms": round(v_ms, 4), "GB/s": round(v_bytes / (v_ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(v_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "algorithmic_bytes": v_bytes, "mean_out_len": round(out_len, 3)},
            "ctx_fuse": {"ms": round(f_ms, 4), "M": int(wl.M), "TFLOP/s": round(f_flops / (f_ms * 1e-3) / 1e12, 1),
                         "mfma_frac": round(f_flops / (f_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "GB/s": round(f_bytes / (f_ms * 1e-3) / 1e9, 1),
                         "cold_ms": round(f_cold, 4),
                         "cold_mfma_frac": round(f_flops / (f_cold * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        },
    }
    calls = args.warmup + K * (1 if args.eager else 3)
    res["kernels"]["spec_verify"]["near_ties"] = {
        "count": int(wl.verify.outputs[2].item()), "verify_calls": calls,
        "rule": "acceptance decisions with |u - p/q| < 1e-6, counted by the kernel"}
    if not args.no_prefill:
        log("[bench] prefill workload: ctx_fuse M=32768, verify B=256")
        res["kernels"].update(prefill_measurements(torch, dfl, synth))
        log("[bench] long-context workload: block_attn B=4, S=131072")
        res["kernels"].update(long_context_measurement(torch, dfl, synth))
        log("[bench] windowed attention: B=64, latest 1024 tokens")
        res["kernels"].update(window_measurement(torch, dfl, wl))
        log("[bench] draft forward around attention: B=64, 5 layers")
        res["kernels"].update(draft_measurement(torch, dfl, synth, wl))
        log("[bench] serving batch with ragged contexts in [1024, 8192]")
        res["kernels"].update(ragged_measurement(torch, dfl, synth))
        log("[bench] shared LM head and draft proposals: B=64, V=262144")
        res["kernels"].update(head_measurement(torch, dfl, synth))
        log("[bench] tiny fp32 and single-stream cycles, long-context verify")
        res["kernels"].update(config_measurements(torch, dfl, synth))
        log("[bench] measured copy / read / matmul ceilings")
        res["measured_peaks"] = measured_peaks(torch, dfl)
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl)
        res["kernels"]["spec_verify"]["parity_vs_oracle"] = verify_parity(wl)
    print(json.dumps(res), flush=True)


def verify_parity(wl):
    """The serving batch's verification at offset 0 on the GPU against the
    oracle's traces of the CPU baseline, sequence by sequence, under the
    parity rule of the tests (bit-exact; an acceptance decision within 1e-6
    of its uniform, or a final draw inside its fp32 key bound, is excluded
    and counted)."""
    from tests.gpu_util import compare_verify
    torch = wl.torch
    wl.verify.args.offset = 0
    wl.verify()
    torch.cuda.synchronize()
    toks = wl.verify.outputs[0].cpu().numpy()
    lens = wl.verify.outputs[1].cpu().numpy()
    excluded = sum(compare_verify(toks[b:b + 1], lens[b:b + 1], tr) for b, tr in enumerate(wl.verify_traces))
    return {"sequences": len(wl.verify_traces), "bit_exact": len(wl.verify_traces) - excluded,
            "excluded": excluded, "oracle_near_ties": int(sum(tr.near_ties for tr in wl.verify_traces))}


if __name__ == "__main__":
    main()
