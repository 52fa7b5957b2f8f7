"""Benchmark of the block-diffusion hot path on one MI355X.

One bench step decodes one 256-position block of the one-layer workload
(hidden 2048, 16/8 heads of 128, 128 experts top-8 of width 768, vocab
262144, 2048 cached prefix tokens, batch 1, 128 of 256 positions masked):
denoise step + entropy-bounded selection (gamma 1.0) repeated until every
position is committed, then the causal encode-and-append of the block.  The
block restarts from the same canvas and prefix length each step, so every
step does the same work.  All inputs are seeded synthetic data resident in
HBM before the timed region.

Printed: one JSON line with canvas tokens/s (256 x denoise steps / time) as
the value, committed tokens/s, the roofline of the dominant kernel measured
with hipEvents around its launches, and the CPU oracle timed on a bounded
sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --denoise-only 3     # a few plain denoise steps, for profilers
  python bench.py --copy-calibration   # one plain copy of 1 GiB, for counters
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOAD = "moe_layer_h2048_v262k_p2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(kind, s, wl, mean_rows):
    """(bytes, flops) the method must move / compute per launch of a kernel
    kind at this workload: weights read once, activations in and out.
    mean_rows: mean number of uncommitted rows per LM-head launch."""
    T = wl.batch * 256
    H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
    E, k, F, V = s.n_experts, s.top_k, s.expert_ffn, s.vocab
    pairs = T * k
    touched = E * (1.0 - (1.0 - k / E) ** T)   # experts receiving a token
    qkvN = (Hq + 2 * Hkv) * D
    P = wl.prefix_len
    if kind == "lm_head":
        return (V * H * 2 + mean_rows * H * 2 + mean_rows * 16,
                2.0 * mean_rows * H * V)
    if kind == "moe_gate_up":
        return (touched * 2 * F * H * 2 + pairs * H * 2 + pairs * F * 2,
                2.0 * pairs * H * 2 * F)
    if kind == "moe_down":
        return (touched * H * F * 2 + pairs * F * 2 + pairs * H * 4,
                2.0 * pairs * F * H)
    if kind == "attention":
        return ((P + 256) * Hkv * D * 2 * 2 + T * Hq * D * 2 * 2
                + T * 2 * Hkv * D * 2, 4.0 * T * Hq * D * (P + 256))
    if kind == "qkv_proj":
        return (qkvN * H * 2 + T * H * 2 + T * qkvN * 2, 2.0 * T * H * qkvN)
    if kind == "o_proj":
        return (H * Hq * D * 2 + T * Hq * D * 2 + T * H * 8,
                2.0 * T * Hq * D * H)
    if kind == "router":
        return (E * H * 2 + T * H * 2 + T * E * 4, 2.0 * T * H * E)
    return None


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                               "traffic_moe_layer_h2048_v262k_p2048.md")


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


def measured_traffic(kind):
    """HBM bytes per launch of a kernel kind from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is
    none or it was taken on other kernel sources."""
    try:
        with open(TRAFFIC_PROFILE) as f:
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


class Bench:
    def __init__(self, wl, seed=0):
        import torch
        from block_discrete_diffusion_tok_amd import dg, synth
        self.torch, self.dg, self.synth = torch, dg, synth
        self.wl = wl
        s = wl.shape
        dev = "cuda"
        t0 = time.time()
        self.w = synth.make_weights(s, seed=seed, device=dev)
        k, v = synth.make_prefix_kv(s, wl.prefix_len, 0, seed=seed, device=dev)
        self.prefix = (k, v)
        self.eng = dg.Engine(s, self.w, max_requests=1,
                             max_kv_len=wl.prefix_len + 256, max_canvases=1)
        self.eng.prefill_kv(0, k.contiguous(), v.contiguous())
        cv = synth.make_canvas(s, wl.batch, wl.uncommitted, seed=seed)
        self.cv = cv
        self.init = {kk: t.to(dev) for kk, t in cv.items()}
        self.st = {kk: t.clone() for kk, t in self.init.items()}
        self.ent = torch.zeros((1, 256), dtype=torch.float32, device=dev)
        self.lse = torch.zeros_like(self.ent)
        self.am = torch.zeros((1, 256), dtype=torch.int32, device=dev)
        self.gamma = torch.full((1,), wl.gamma, dtype=torch.float32, device=dev)
        self.n_new = torch.zeros(1, dtype=torch.int32, device=dev)
        # the stopping flags live in pinned host memory: the EB kernel writes
        # them there directly, so the loop reads them after an event sync with
        # no device-to-host copy launched per step.  Two flags and two events:
        # step n + 1 is queued before step n's flag is read.
        self.done = torch.zeros(2, dtype=torch.uint8, pin_memory=True)
        self.ev = [torch.cuda.Event(), torch.cuda.Event()]
        torch.cuda.synchronize()
        log(f"[bench] inputs ready in {time.time() - t0:.1f} s")

    def denoise(self):
        st = self.st
        self.eng.denoise_step([0], st["tokens"], st["committed"], st["step"],
                              self.ent, self.lse, self.am)

    def _launch_step(self, i):
        st = self.st
        self.denoise()
        self.eng.eb_select([0], st["tokens"], st["committed"], st["step"],
                           self.ent, self.am, self.gamma, self.wl.step_cap, True,
                           self.n_new, self.done[i % 2:i % 2 + 1])
        self.ev[i % 2].record()

    def block(self, lookahead=True):
        """Decode one block from the initial canvas; returns denoise steps.

        Adaptive stopping reads each step's done flag on the host.  With
        lookahead the next step is queued first, so the GPU does not idle
        while the host reads the flag; the one step queued after the last is
        a denoise step and EB selection of a canvas with nothing left to
        unmask, which changes neither tokens, mask nor step counter."""
        st, init = self.st, self.init
        for kk in st:
            st[kk].copy_(init[kk])
        self.eng.set_kv_len(0, self.wl.prefix_len)
        n = 0
        self._launch_step(0)
        while True:
            if lookahead:
                self._launch_step(n + 1)
            self.ev[n % 2].synchronize()
            done = int(self.done[n % 2])
            n += 1
            if done:
                break
            if not lookahead:
                self._launch_step(n)
        self.eng.commit_block([0], st["tokens"], st["committed"], st["step"])
        return n


def cpu_baseline(b, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    repeated denoise steps + EB selections from the initial canvas until
    budget_s has elapsed (at least one)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    wl, synth = b.wl, b.synth
    s = wl.shape
    wn = synth.to_numpy_weights(b.w)
    k, v = b.prefix
    pre = [(k.float().cpu().numpy(), v.float().cpu().numpy())]
    osh = oracle.Shapes(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads,
                        s.head_dim, s.n_experts, s.top_k, s.expert_ffn,
                        s.vocab, s.rms_eps)
    tok = b.cv["tokens"].numpy().astype(np.int64)
    com = b.cv["committed"].numpy()
    step = b.cv["step"].numpy().astype(np.int64)
    gamma = np.array([wl.gamma], np.float32)
    t0 = time.time()
    n = 0
    while True:
        out = oracle.denoise_step(osh, wn, tok, com, pre, mirror=True)
        com, tok, step, _, _ = oracle.eb_select(
            out["entropy"].astype(np.float32), out["argmax"], com, tok, step,
            gamma, wl.step_cap)
        n += 1
        if time.time() - t0 >= budget_s:
            break
    dt = time.time() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": 256.0 * n / dt, "unit": "canvas tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{n} denoise step(s) + EB selection(s) of the same "
                      f"workload from its initial canvas, fp64 numpy, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--denoise-only", type=int, default=0)
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
    wl = synth.WORKLOADS[WORKLOAD]
    s = wl.shape
    b = Bench(wl)

    if args.denoise_only:
        for i in range(args.denoise_only):
            b.denoise()
            torch.cuda.synchronize()
            log(f"[bench] denoise step {i} done")
        return

    for i in range(args.warmup):
        n = b.block()
        log(f"[bench] warmup block {i}: {n} denoise steps")
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    t0 = time.time()
    steps = []
    for i in range(args.steps):
        steps.append(b.block())
        log(f"[bench] block {i}: {steps[-1]} denoise steps")
    ev1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = ev0.elapsed_time(ev1)
    total_denoise = sum(steps)
    value = 256.0 * total_denoise / (ms / 1000.0)
    committed = wl.uncommitted * args.steps / (ms / 1000.0)

    # per-kernel times of one block, hipEvents around every launch (no
    # lookahead: every profiled launch belongs to a step that unmasks)
    b.eng.profile_enable(True)
    n_prof = b.block(lookahead=False)
    prof = b.eng.profile_read()
    b.eng.profile_enable(False)
    # plain denoise-step time (no per-step host sync) on the initial canvas:
    # 128 masked rows reach the LM head every step
    for kk in b.st:
        b.st[kk].copy_(b.init[kk])
    reps = 20
    b.denoise()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.denoise()
    e1.record()
    torch.cuda.synchronize()
    ms_denoise = e0.elapsed_time(e1) / reps

    kernels = {name: {"total_ms": round(t, 4), "launches": n,
                      "avg_us": round(1000.0 * t / n, 2)}
               for name, (t, n) in sorted(prof.items(), key=lambda x: -x[1][0])}
    dom = max(prof.items(), key=lambda x: x[1][0])[0]
    mean_rows = (wl.uncommitted + 1) / 2.0
    roofline = None
    for name in [dom] + [n for n in kernels if n != dom]:
        alg = algorithmic(name, s, wl, mean_rows)
        if alg is None:
            continue
        t_avg = prof[name][0] / prof[name][1] / 1000.0   # seconds per launch
        nbytes, flops = alg
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
        if t_hbm >= t_mfma:
            ach = nbytes / t_avg / 1e9
            roofline = {"kernel": name, "bound": "hbm",
                        "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(name),
                        "algorithmic_bytes_per_launch": int(nbytes),
                        "avg_launch_us": round(t_avg * 1e6, 2)}
        else:
            ach = flops / t_avg / 1e12
            roofline = {"kernel": name, "bound": "mfma",
                        "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic(name),
                        "algorithmic_flops_per_launch": int(flops),
                        "avg_launch_us": round(t_avg * 1e6, 2)}
        break

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(b)

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
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights, N(0,1) prefix K/V, "
                "uniform canvas tokens",
        "config": {"workload": WORKLOAD, "layers": s.n_layers,
                   "hidden": s.hidden, "q_heads": s.n_q_heads,
                   "kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                   "experts": s.n_experts, "top_k": s.top_k,
                   "expert_ffn": s.expert_ffn, "vocab": s.vocab,
                   "prefix_len": wl.prefix_len, "batch": wl.batch,
                   "masked": wl.uncommitted, "gamma": wl.gamma,
                   "step": "one block: denoise + EB until done, then commit"},
        "committed_tok_s": round(committed, 1),
        "denoise_steps_per_block": round(total_denoise / args.steps, 2),
        "ms_per_denoise_step": round(ms_denoise, 4),
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
