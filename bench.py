"""Benchmark of the block-diffusion hot path on one MI355X.

Default workload: the 30-layer stack (hidden 2048, 16/8 heads of 128, 128
experts top-8 of width 768, vocab 262144, bf16), batch 1, 4096 cached prefix
tokens, blocks of 256 positions decoded with the entropy-bounded sampler
(gamma 1.0, step cap 64) and committed to the KV cache.  One bench step is
one block: denoise step + EB selection repeated until every position is
committed (adaptive stopping; the step cap binds with random weights), then
the causal encode-and-append of the block.  Timed steps decode consecutive
blocks, so the cache grows by 256 rows per step, as in a generation of
K x 256 tokens after the prompt.  All inputs are seeded synthetic data
resident in HBM before the timed region.

Printed: one JSON line.  value = canvas tokens/s over the timed region
(256 x denoise steps / time, EB selections, host stopping checks and
commits included); committed tokens/s; the median and p90 of the per-step
times (hipEvents around each denoise step and each EB selection); the same
block decoded with the final-norm gain scaled so that EB commits ~19.74
positions per step (the pages' tokens per forward) as a labelled variant;
per-kernel times with their roofline fractions and the dominant kernel's
roofline; labelled extras: AR decoding (greedy, one position per step) and
token-mode prompt prefill on request 0, the step replayed from a HIP graph
against the same steps launched eagerly, and the same decoding in W8A8
(E4M3 projections, experts and LM head; after the bf16 engine is freed); the
CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
  python bench.py --denoise-only 3     # a few plain denoise steps, for profilers
  python bench.py --prefill-only 32768 # token-mode prefill of a long prompt
  python bench.py --copy-calibration   # one plain copy of 1 GiB, for counters
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOAD = "stack30_h2048_p4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
TPF_TARGET = 19.74             # tokens per forward, write-up Table 3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(kind, s, wl, mean_rows, prefix):
    """(bytes, flops) the method must move / compute per launch of a kernel
    kind: weights read once, activations in and out.  mean_rows: mean
    uncommitted rows per LM-head launch; prefix: cached keys per canvas."""
    T = wl.batch * 256
    H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
    E, k, F, V = s.n_experts, s.top_k, s.expert_ffn, s.vocab
    wb = 1 if s.expert_dtype == "fp8_e4m3" else 2     # expert weight bytes
    # expert GEMM token rows: E4M3 codes plus one fp32 scale per row
    ab = H + 4 if s.act_dtype == "fp8_e4m3" else 2 * H
    fb = F + 4 if s.act_dtype == "fp8_e4m3" else 2 * F
    # cached K / V rows: E4M3 codes plus one fp32 scale per row
    kvb = D + 4 if s.kv_dtype == "fp8_e4m3" else 2 * D
    # E4M3 projections / LM head: 1-byte weights plus a scale per row, input
    # rows as codes plus a scale
    p8 = s.proj_dtype == "fp8_e4m3"
    l8 = s.lm_dtype == "fp8_e4m3"
    pairs = T * k
    touched = E * (1.0 - (1.0 - k / E) ** T)   # experts receiving a token
    qkvN = (Hq + 2 * Hkv) * D
    P = prefix
    if kind == "lm_head":
        if l8:
            return (V * H + V * 4 + mean_rows * (H + 4) + mean_rows * 16,
                    2.0 * mean_rows * H * V)
        return (V * H * 2 + mean_rows * H * 2 + mean_rows * 16,
                2.0 * mean_rows * H * V)
    if kind == "moe_gate_up":
        return (touched * 2 * F * H * wb + pairs * ab + pairs * F * 2,
                2.0 * pairs * H * 2 * F)
    if kind == "moe_down":
        return (touched * H * F * wb + pairs * fb + pairs * H * 4,
                2.0 * pairs * F * H)
    if kind == "attention":
        return (wl.batch * P * Hkv * kvb * 2 + wl.batch * 256 * Hkv * D * 2 * 2
                + T * Hq * D * 2 * 2 + T * 2 * Hkv * D * 2,
                4.0 * T * Hq * D * (P + 256))
    if kind == "qkv_proj":
        if p8:
            return (qkvN * (H + 4) + T * (H + 4) + T * qkvN * 2,
                    2.0 * T * H * qkvN)
        return (qkvN * H * 2 + T * H * 2 + T * qkvN * 2, 2.0 * T * H * qkvN)
    if kind == "o_proj":
        if p8:
            return (H * (Hq * D + 4) + T * (Hq * D + 4) + T * H * 8,
                    2.0 * T * Hq * D * H)
        return (H * Hq * D * 2 + T * Hq * D * 2 + T * H * 8,
                2.0 * T * Hq * D * H)
    if kind == "router":
        return (E * H * 2 + T * H * 2 + T * E * 4, 2.0 * T * H * E)
    return None


def mfma_peak(kind, s, rows=None):
    """Dense MFMA peak (TFLOP/s) of the type a kernel kind computes in:
    the expert GEMMs run the fp8 MFMA when token rows are E4M3; E4M3
    projections from 1024 rows and an E4M3 LM head above 128 rows take the
    large-tile kernel's fp8 MFMA (fewer rows: E4M3 codes widened to bf16).
    rows: token rows of a projection launch or mean LM-head rows."""
    if kind in ("moe_gate_up", "moe_down") and s.act_dtype == "fp8_e4m3":
        return FP8_PEAK_TFLOPS
    if kind in ("qkv_proj", "o_proj") and s.proj_dtype == "fp8_e4m3" and \
            rows is not None and rows >= 1024:
        return FP8_PEAK_TFLOPS
    if kind == "lm_head" and s.lm_dtype == "fp8_e4m3" and rows is not None \
            and rows > 128:
        return FP8_PEAK_TFLOPS
    return BF16_PEAK_TFLOPS


def roofline_of(kind, alg, t_avg_s, peak_tflops=BF16_PEAK_TFLOPS):
    nbytes, flops = alg
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (peak_tflops * 1e12)
    if t_hbm >= t_mfma:
        ach = nbytes / t_avg_s / 1e9
        return {"kernel": kind, "bound": "hbm", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": int(nbytes),
                "avg_launch_us": round(t_avg_s * 1e6, 2)}
    ach = flops / t_avg_s / 1e12
    return {"kernel": kind, "bound": "mfma", "achieved": round(ach, 2),
            "peak": peak_tflops, "unit": "TFLOP/s",
            "frac": round(ach / peak_tflops, 4),
            "algorithmic_flops_per_launch": int(flops),
            "avg_launch_us": round(t_avg_s * 1e6, 2)}


def traffic_profile_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.md")


def kernel_source_hash():
    """sha256 over the HIP sources and headers the kernels are built from;
    traffic figures measured on other sources are not reported."""
    import hashlib
    h = hashlib.sha256()
    dirs = [os.path.join(ROOT, "block_discrete_diffusion_tok_amd", "csrc"),
            os.path.join(ROOT, "include")]
    for d in dirs:
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h")):
                h.update(f.encode())
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kind):
    """HBM bytes per launch of a kernel kind from the committed counter
    summary of the workload (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when there is none or it was taken on other kernel sources."""
    try:
        with open(traffic_profile_path(workload)) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    vals = {}
    for ln in lines:
        if ln.startswith("    ") and ":" in ln:
            k, v = ln.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    v = vals.get(f"traffic_bytes_per_launch[{kind}]")
    return int(v) if v else None


def copy_calibration():
    import torch
    n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4,
                      "copy_calibration_bytes_written": n * 4}))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class Bench:
    """One engine over the workload's requests; decodes blocks."""

    def __init__(self, wl, seed=0, max_blocks=None):
        import torch
        from block_discrete_diffusion_tok_amd import dg, synth
        self.torch, self.dg, self.synth = torch, dg, synth
        self.wl = wl
        s = wl.shape
        dev = "cuda"
        n = wl.batch
        self.n = n
        self.req = list(range(n))
        blocks = max(wl.blocks, max_blocks or 1)
        t0 = time.time()
        self.w = synth.make_weights(s, seed=seed, device=dev)
        self.eng = dg.Engine(s, self.w, max_requests=n,
                             max_kv_len=wl.prefix_len + 256 * blocks,
                             max_canvases=n)
        self.prefix = []
        for r in range(n):
            k, v = synth.make_prefix_kv(s, wl.prefix_len, r, seed=seed,
                                        device=dev)
            self.eng.prefill_kv(r, k.contiguous(), v.contiguous())
            # host copies for the oracle baseline: the first two requests
            self.prefix.append((k, v) if r < 2 else None)
            del k, v
        self.init = []
        for blk in range(blocks):
            cv = synth.make_canvas(s, n, wl.uncommitted, seed=seed, block=blk)
            self.init.append((cv, {kk: t.to(dev) for kk, t in cv.items()}))
        self.cv = self.init[0][0]
        self.st = {kk: t.clone() for kk, t in self.init[0][1].items()}
        self.ent = torch.zeros((n, 256), dtype=torch.float32, device=dev)
        self.lse = torch.zeros_like(self.ent)
        self.am = torch.zeros((n, 256), dtype=torch.int32, device=dev)
        self.gamma = torch.full((n,), wl.gamma, dtype=torch.float32, device=dev)
        self.n_new = torch.zeros(n, dtype=torch.int32, device=dev)
        # stopping flags in pinned host memory: the EB kernel writes them
        # there, the loop reads them after an event sync (no copy launched).
        # Two flag sets and two events: step n + 1 is queued before step n's
        # flags are read.
        self.done = torch.zeros((2, n), dtype=torch.uint8, pin_memory=True)
        self.ev = [torch.cuda.Event(), torch.cuda.Event()]
        self.timing = None      # list of per-step event triples when timing
        torch.cuda.synchronize()
        log(f"[bench] inputs ready in {time.time() - t0:.1f} s")

    def denoise(self):
        st = self.st
        self.eng.denoise_step(self.req, st["tokens"], st["committed"],
                              st["step"], self.ent, self.lse, self.am)

    def _launch_step(self, i):
        torch = self.torch
        st = self.st
        if self.timing is not None:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            evs[0].record()
        self.denoise()
        if self.timing is not None:
            evs[1].record()
        self.eng.eb_select(self.req, st["tokens"], st["committed"], st["step"],
                           self.ent, self.am, self.gamma, self.wl.step_cap,
                           True, self.n_new, self.done[i % 2])
        if self.timing is not None:
            evs[2].record()
            self.timing.append(evs)
        self.ev[i % 2].record()

    def block(self, lookahead=True, blk=0, kv_start=None):
        """Decode one block from block blk's initial canvas, starting from
        cache length kv_start (default: the prefix); returns the number of
        denoise steps.  With a fixed step count (wl.steps > 0) the block runs
        exactly that many steps and is not committed.

        Adaptive stopping reads each step's done flags on the host.  With
        lookahead the next step is queued first, so the GPU does not idle
        while the host reads them; a step queued after the last is a denoise
        step and EB selection of canvases with nothing left to unmask, which
        changes neither tokens, mask nor step counters (its time is spent,
        its step is not counted).  None is queued past the step cap."""
        st = self.st
        init = self.init[blk % len(self.init)][1]
        for kk in st:
            st[kk].copy_(init[kk])
        for r in self.req:
            self.eng.set_kv_len(r, self.wl.prefix_len if kv_start is None
                                else kv_start)
        fixed = self.wl.steps
        # the block cannot run past the fixed step count or the step cap (the
        # cap step commits every remaining position), so no step is queued
        # ahead beyond it
        last = fixed if fixed else self.wl.step_cap
        n = 0
        launched = 1
        self._launch_step(0)
        while True:
            if lookahead and n + 1 < last:
                self._launch_step(n + 1)
                launched += 1
            self.ev[n % 2].synchronize()
            done = bool(self.done[n % 2].all())
            n += 1
            if (fixed and n >= fixed) or (not fixed and done):
                break
            if not lookahead:
                self._launch_step(n)
                launched += 1
        if self.timing is not None and launched > n:
            self.timing.pop()   # the step queued after the last is not timed
        if not fixed:
            self.eng.commit_block(self.req, st["tokens"], st["committed"],
                                  st["step"])
        return n


def cpu_baseline(b, prof_layers=2):
    """The oracle, as it stands, on a bounded sample of the workload: the
    first prof_layers layers of one denoise step of the first canvas (two
    for the 32-canvas workload), the final norm + LM head statistics + EB
    selection of those canvases, and the first prof_layers layers of their
    causal commit; the full step and block times are extrapolated linearly
    in layers (and canvases)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    wl, synth = b.wl, b.synth
    s = wl.shape
    L = s.n_layers
    nl = min(prof_layers, L)
    nb = min(b.n, 2)
    osh = oracle.Shapes(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads,
                        s.head_dim, s.n_experts, s.top_k, s.expert_ffn,
                        s.vocab, s.rms_eps)
    wn = synth.to_numpy_weights({"embed": b.w["embed"],
                                 "final_norm": b.w["final_norm"],
                                 "layers": b.w["layers"][:nl]})
    pre = []
    for r in range(nb):
        k, v = b.prefix[r]
        pre.append((k[:nl].float().cpu().numpy(), v[:nl].float().cpu().numpy()))
    tok = b.cv["tokens"].numpy()[:nb].astype(np.int64)
    com = b.cv["committed"].numpy()[:nb]
    step = b.cv["step"].numpy()[:nb].astype(np.int64)
    osh_l = oracle.Shapes(nl, *[getattr(osh, f) for f in (
        "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "expert_ffn", "vocab", "rms_eps")])
    t0 = time.time()
    x = oracle.model._layers_forward(osh_l, wn, tok, pre, True, False, None)
    t_layers = time.time() - t0
    t0 = time.time()
    rows = np.nonzero(com.reshape(-1) == 0)[0]
    xf = oracle.round_bf16(oracle.rmsnorm(x[rows], wn["final_norm"], s.rms_eps))
    st = oracle.lm_head_stats(xf, wn["embed"])
    ent = np.full(com.size, np.nan)
    am = np.full(com.size, -1, dtype=np.int64)
    ent[rows] = st["entropy"]
    am[rows] = st["argmax"]
    oracle.eb_select(ent.reshape(com.shape).astype(np.float32),
                     am.reshape(com.shape), com, tok, step,
                     np.full(nb, wl.gamma, np.float32), wl.step_cap)
    t_head = time.time() - t0
    t_commit = 0.0
    if not wl.steps:
        t0 = time.time()
        oracle.commit_block(osh_l, wn, tok, pre, mirror=True)
        t_commit = time.time() - t0
    scale_b = b.n / nb
    t_step = (t_layers * L / nl + t_head) * scale_b
    t_commit_full = t_commit * L / nl * scale_b
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    out = {"value": round(256.0 * b.n / t_step, 3), "unit": "canvas tokens/s",
           "cores": int(threads), "host_cores": os.cpu_count(),
           "cpu_model": cpu_model(), "kind": "oracle",
           "sample": f"{nl} of {L} layers of one denoise step of {nb} of "
                     f"{b.n} canvas(es) ({t_layers:.1f} s), their final norm + "
                     f"LM head statistics + EB ({t_head:.1f} s)"
                     + (f", {nl} layers of their causal commit "
                        f"({t_commit:.1f} s)" if t_commit else "")
                     + f"; fp64 numpy; step time extrapolated as "
                     f"(t_layers x {L}/{nl} + t_head)"
                     + (f" x {scale_b:g} canvases" if scale_b != 1 else "")
                     + f" = {t_step:.1f} s"}
    if not wl.steps:
        dns = wl.step_cap if wl.uncommitted > wl.step_cap else wl.uncommitted
        t_block = dns * t_step + t_commit_full
        out["committed_tok_s"] = round(256.0 * b.n / t_block, 4)
        out["block_formula"] = (f"DNS x t_step + t_commit = {dns} x "
                                f"{t_step:.1f} s + {t_commit_full:.1f} s")
    return out


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    i = min(len(xs) - 1, max(0, int(round(q / 100.0 * (len(xs) - 1)))))
    return xs[i]


def tpf_matched(b, blocks):
    """The same workload with the final-norm gain scaled so that EB commits
    about TPF_TARGET positions per denoise step (a labelled synthetic
    variant: with random weights every entropy is near ln V and EB commits
    one position per step).  The gain scale is found by bisection on the
    first block's step count; the blocks are then timed from the prefix."""
    torch = b.torch
    wl = b.wl
    target_steps = max(1, round(wl.uncommitted / TPF_TARGET))
    g0 = b.w["final_norm"].clone()
    lo, hi = 0.0, 6.0     # log2 of the gain scale

    def steps_at(lg):
        b.w["final_norm"].copy_(g0 * (2.0 ** lg))
        n = b.block(lookahead=False, blk=0)
        torch.cuda.synchronize()
        return n
    best = None
    for _ in range(10):
        mid = 0.5 * (lo + hi)
        n = steps_at(mid)
        if best is None or abs(n - target_steps) < abs(best[1] - target_steps):
            best = (mid, n)
        if n > target_steps:
            lo = mid
        elif n < target_steps:
            hi = mid
        else:
            break
    lg = best[0]
    b.w["final_norm"].copy_(g0 * (2.0 ** lg))
    b.block(lookahead=False, blk=0)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    steps = []
    for i in range(blocks):
        steps.append(b.block(lookahead=False, blk=i,
                             kv_start=wl.prefix_len + 256 * i))
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    b.w["final_norm"].copy_(g0)
    for r in b.req:
        b.eng.set_kv_len(r, wl.prefix_len)
    total = sum(steps)
    return {"final_norm_gain_scale": round(2.0 ** lg, 4),
            "denoise_steps_per_block": round(total / blocks, 2),
            "tokens_per_forward": round(wl.uncommitted * blocks / total, 2),
            "committed_tok_s": round(wl.uncommitted * b.n * blocks
                                     / (ms / 1000.0), 1),
            "canvas_tok_s": round(256.0 * b.n * total / (ms / 1000.0), 1),
            "ms_per_block": round(ms / blocks, 3),
            "note": f"labelled synthetic variant: final-norm gain x "
                    f"{2.0 ** lg:.3g}, bisected on the first block so that EB "
                    f"commits ~{TPF_TARGET} positions per step (write-up "
                    f"Table 3 tokens per forward); no step queued ahead"}


def ar_and_prefill(b, n_tokens=64):
    """Labelled extras on request 0: AR decoding (n_tokens greedy steps of
    one position, each fed the previous step's argmax, from the workload's
    prefix) and token-mode prefill of a prompt of the prefix length; both
    timed with hipEvents.  They overwrite request 0's cache."""
    torch, wl = b.torch, b.wl
    dev = "cuda"
    ent = torch.zeros(1, dtype=torch.float32, device=dev)
    lse = torch.zeros_like(ent)
    am = torch.zeros(1, dtype=torch.int32, device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    b.eng.set_kv_len(0, wl.prefix_len)
    b.eng.ar_step([0], tok, ent, lse, am)          # warm-up
    b.eng.set_kv_len(0, wl.prefix_len)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_tokens):
        b.eng.ar_step([0], tok, ent, lse, am)
        tok.copy_(am)
    e1.record()
    torch.cuda.synchronize()
    ar_ms = e0.elapsed_time(e1)
    P = min(wl.prefix_len, 8192)
    g = torch.Generator(device="cpu").manual_seed(11)
    prompt = torch.randint(0, wl.shape.vocab, (P,), generator=g,
                           dtype=torch.int32).to(dev)
    b.eng.prefill_tokens(0, prompt)               # warm-up
    torch.cuda.synchronize()
    e0.record()
    b.eng.prefill_tokens(0, prompt)
    e1.record()
    torch.cuda.synchronize()
    pf_ms = e0.elapsed_time(e1)
    b.eng.set_kv_len(0, wl.prefix_len)
    return {"ar_decode": {"tokens": n_tokens, "prefix": wl.prefix_len,
                          "ms_per_token": round(ar_ms / n_tokens, 4),
                          "tok_s": round(n_tokens / (ar_ms / 1000.0), 1),
                          "note": "labelled extra: batch 1, greedy, one "
                                  "position per dg_ar_step"},
            "prefill_tokens": {"tokens": P, "ms": round(pf_ms, 3),
                               "tok_s": round(P / (pf_ms / 1000.0), 1),
                               "note": "labelled extra: token-mode "
                                       "dg_prefill_kv, causal encode in "
                                       "chunks of 256"}}


def graph_variant(b, steps=32):
    """Labelled extra: one denoise step + EB selection captured into a HIP
    graph on a side stream (dg_set_stream) and replayed `steps` times from
    the first block's initial canvas, against the same steps launched
    eagerly on that stream; hipEvents around each run of steps."""
    torch = b.torch
    st = b.st
    init = b.init[0][1]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    b.eng.set_stream(s)

    def restore():
        for kk in st:
            st[kk].copy_(init[kk])
        for r in b.req:
            b.eng.set_kv_len(r, b.wl.prefix_len)

    def one():
        b.eng.denoise_step(b.req, st["tokens"], st["committed"], st["step"],
                           b.ent, b.lse, b.am)
        b.eng.eb_select(b.req, st["tokens"], st["committed"], st["step"],
                        b.ent, b.am, b.gamma, b.wl.step_cap, True, b.n_new,
                        b.done[0])

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        restore()
        one()                                   # warm-up on the stream
        restore()
        e0.record()
        for _ in range(steps):
            one()
        e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        one()
    with torch.cuda.stream(s):
        restore()
        g.replay()                              # warm-up replay
        restore()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    graph = e0.elapsed_time(e1) / steps
    del g
    b.eng.set_stream(None)
    restore()
    torch.cuda.synchronize()
    return {"steps": steps, "eager_step_ms": round(eager, 4),
            "graph_step_ms": round(graph, 4),
            "note": "labelled extra: denoise step + EB selection replayed "
                    "from a HIP graph vs launched eagerly, same stream"}


def w8a8_variant(name, steps=2):
    """Labelled extra: the same batch-1 decoding in W8A8 (E4M3 weights and
    rows in the projections, the experts and the LM head), one warm-up
    block and `steps` consecutive timed blocks, hipEvents around each
    denoise step."""
    import torch
    from block_discrete_diffusion_tok_amd import synth
    wl = synth.WORKLOADS[name]
    b = Bench(wl, seed=0, max_blocks=steps)
    b.block(blk=0)
    torch.cuda.synchronize()
    b.timing = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    n = 0
    for i in range(steps):
        n += b.block(blk=i, kv_start=wl.prefix_len + 256 * i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    step_ms = [e[0].elapsed_time(e[1]) for e in b.timing]
    med = percentile(step_ms, 50)
    b.eng.close()
    del b
    torch.cuda.empty_cache()
    return {"workload": name, "blocks": steps, "denoise_steps": n,
            "canvas_tok_s": round(256.0 * n / (ms / 1000.0), 1),
            "committed_tok_s": round(wl.uncommitted * steps / (ms / 1000.0), 1),
            "denoise_step_ms_median": round(med, 4),
            "note": "labelled extra: W8A8 -- E4M3 weights (per-row scales) "
                    "and E4M3 rows in the Q/K/V and output projections, the "
                    "experts and the LM head; attention, router and norms "
                    "in bf16 / fp32, bf16 KV cache"}


def prefill_only(wl, n_tokens):
    """Token-mode prefill (dg_prefill_kv from tokens: the causal encode in
    chunks of 256 through every layer, K/V written to the cache) of one
    seeded prompt of n_tokens on the workload's model; a 512-token warm-up
    first, then one timed prefill with hipEvents."""
    import torch
    from block_discrete_diffusion_tok_amd import dg, synth
    s = wl.shape
    w = synth.make_weights(s, seed=0, device="cuda")
    eng = dg.Engine(s, w, max_requests=1, max_kv_len=n_tokens + 256,
                    max_canvases=1)
    g = torch.Generator(device="cpu").manual_seed(13)
    prompt = torch.randint(0, s.vocab, (n_tokens,), generator=g,
                           dtype=torch.int32).to("cuda")
    eng.prefill_tokens(0, prompt[:512].contiguous())
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    eng.prefill_tokens(0, prompt)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert eng.kv_len(0) == n_tokens
    eng.close()
    return {"metric": "token-mode prefill tokens/s", "value": round(
        n_tokens / (ms / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
            "ms": round(ms, 2), "tokens": n_tokens, "higher_is_better": True,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": wl.name, "layers": s.n_layers,
                       "step": "causal encode in chunks of 256"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4,
                    help="timed bench steps (blocks); default: the 4 blocks "
                         "of the workload")
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tpf-variant", action="store_true")
    ap.add_argument("--no-ar", action="store_true",
                    help="skip the AR-decoding and token-prefill extras")
    ap.add_argument("--no-w8a8", action="store_true",
                    help="skip the W8A8 batch-1 extra")
    ap.add_argument("--denoise-only", type=int, default=0)
    ap.add_argument("--prefill-only", type=int, default=0,
                    help="time token-mode prefill of a prompt of this many "
                         "tokens on the workload's model (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: libdg has no multi-GPU "
              "path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    from block_discrete_diffusion_tok_amd import synth
    wl = synth.WORKLOADS[args.workload]
    s = wl.shape
    if args.prefill_only:
        print(json.dumps(prefill_only(wl, args.prefill_only)), flush=True)
        return
    b = Bench(wl, max_blocks=max(args.steps, args.warmup))

    if args.denoise_only:
        for i in range(args.denoise_only):
            b.denoise()
            torch.cuda.synchronize()
            log(f"[bench] denoise step {i} done")
        return

    for i in range(args.warmup):
        n = b.block(blk=i)
        log(f"[bench] warmup block {i}: {n} denoise steps")
    torch.cuda.synchronize()
    # timed region: K consecutive blocks (the cache grows by 256 rows each),
    # per-step hipEvents around every denoise step and EB selection
    b.timing = []
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    t0 = time.time()
    steps = []
    commits = not wl.steps
    for i in range(args.steps):
        kv0 = wl.prefix_len + (256 * i if commits else 0)
        steps.append(b.block(blk=i, kv_start=kv0))
        log(f"[bench] block {i}: {steps[-1]} denoise steps")
    ev1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = ev0.elapsed_time(ev1)
    step_ms = [e[0].elapsed_time(e[1]) for e in b.timing]
    eb_ms = [e[1].elapsed_time(e[2]) for e in b.timing]
    b.timing = None
    total_denoise = sum(steps)
    n_canvas = b.n
    value = 256.0 * n_canvas * total_denoise / (ms / 1000.0)
    committed = (wl.uncommitted * b.n * args.steps / (ms / 1000.0)
                 if commits else None)
    med = percentile(step_ms, 50)
    p90 = percentile(step_ms, 90)
    med_eb = percentile([a + c for a, c in zip(step_ms, eb_ms)], 50)

    # per-kernel times of one block from the prefix, hipEvents around every
    # launch (no lookahead: every profiled launch belongs to a step that
    # unmasks); the mean live LM-head rows of the same block
    b.eng.profile_enable(True)
    rows_seen = []
    st = b.st
    init = b.init[0][1]
    for kk in st:
        st[kk].copy_(init[kk])
    for r in b.req:
        b.eng.set_kv_len(r, wl.prefix_len)
    n_prof = 0
    while True:
        rows_seen.append(int((st["committed"] == 0).sum().item()))
        b._launch_step(0)
        torch.cuda.synchronize()
        n_prof += 1
        if (wl.steps and n_prof >= wl.steps) or \
                (not wl.steps and bool(b.done[0].all())):
            break
    if commits:
        b.eng.commit_block(b.req, st["tokens"], st["committed"], st["step"])
    prof = b.eng.profile_read()
    b.eng.profile_enable(False)
    mean_rows = sum(rows_seen) / len(rows_seen)

    def launch_rows(kind):
        return mean_rows if kind == "lm_head" else wl.batch * 256

    kernels = {}
    for name, (t, n) in sorted(prof.items(), key=lambda x: -x[1][0]):
        ent = {"total_ms": round(t, 4), "launches": n,
               "avg_us": round(1000.0 * t / n, 2)}
        alg = algorithmic(name, s, wl, mean_rows, wl.prefix_len)
        if alg is not None:
            rf = roofline_of(name, alg, t / n / 1000.0,
                             mfma_peak(name, s, launch_rows(name)))
            ent["bound"] = rf["bound"]
            ent["frac"] = rf["frac"]
        kernels[name] = ent
    dom = max((k for k in prof if algorithmic(k, s, wl, mean_rows,
                                              wl.prefix_len) is not None),
              key=lambda k: prof[k][0])
    roofline = roofline_of(dom, algorithmic(dom, s, wl, mean_rows,
                                            wl.prefix_len),
                           prof[dom][0] / prof[dom][1] / 1000.0,
                           mfma_peak(dom, s, launch_rows(dom)))
    roofline["traffic"] = measured_traffic(args.workload, dom)

    tpf = None
    if commits and not args.no_tpf_variant:
        log("[bench] TPF-matched variant")
        tpf = tpf_matched(b, args.steps)

    extras = {}
    log("[bench] HIP-graph replay of the step")
    extras["hip_graph"] = graph_variant(b)
    if not args.no_ar:
        log("[bench] AR decoding and token-mode prefill")
        extras.update(ar_and_prefill(b))
        # the write-up's Figure 11 ratio: a 256-position denoise step against
        # a one-position AR step, both at batch 1
        extras["denoise_step_over_ar_step"] = round(
            med / extras["ar_decode"]["ms_per_token"], 3)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(b)

    if not args.no_w8a8 and args.workload == WORKLOAD:
        log("[bench] W8A8 variant of the batch-1 stack")
        b.eng.close()
        del b
        torch.cuda.empty_cache()
        extras["w8a8"] = w8a8_variant("stack30_w8a8_h2048_p4096")

    out = {
        "metric": "canvas tokens/s per denoise step; committed output tok/s "
                  "at batch 1",
        "value": round(value, 1),
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16+e4m3 (w8a8)" if s.proj_dtype == "fp8_e4m3" else
                  "bf16" if s.expert_dtype == "bf16" else "bf16+e4m3 experts"),
        "data": "synthetic: seeded N(0,0.02) bf16 weights, N(0,1) prefix K/V, "
                "uniform canvas tokens",
        "config": {"workload": args.workload, "layers": s.n_layers,
                   "hidden": s.hidden, "q_heads": s.n_q_heads,
                   "kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                   "experts": s.n_experts, "top_k": s.top_k,
                   "expert_ffn": s.expert_ffn, "vocab": s.vocab,
                   "expert_dtype": s.expert_dtype, "act_dtype": s.act_dtype,
                   "proj_dtype": s.proj_dtype, "lm_dtype": s.lm_dtype,
                   "kv_dtype": s.kv_dtype,
                   "prefix_len": wl.prefix_len, "batch": wl.batch,
                   "masked": wl.uncommitted, "gamma": wl.gamma,
                   "step_cap": wl.step_cap,
                   "step": ("one block: denoise + EB until done, then commit; "
                            "consecutive blocks") if commits else
                           f"{wl.steps} denoise steps + EB selections"},
        "committed_tok_s": None if committed is None else round(committed, 1),
        "denoise_steps_per_block": round(total_denoise / args.steps, 2),
        "denoise_step_ms": {"median": round(med, 4), "p90": round(p90, 4),
                            "n": len(step_ms)},
        "denoise_plus_eb_ms_median": round(med_eb, 4),
        "canvas_tok_s_median_step": round(256.0 * n_canvas / (med / 1000.0),
                                          1),
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "lm_head_mean_rows": round(mean_rows, 2),
        "tpf_matched": tpf,
        **extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
