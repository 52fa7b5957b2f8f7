"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth

DEV = "cuda"
TOL = 2e-2        # max relative error on continuous outputs (per tensor)
# Decisions (top-k routing, argmax) whose oracle margin, relative to the
# largest magnitude among the values decided on, is below MARGIN are not
# required to agree: the bf16 activations the path stores round differently
# from the oracle's fp64 values whenever the two straddle a rounding boundary,
# which moves router and vocabulary logits by ~1e-3 of their scale.
MARGIN = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oshape(s):
    return oracle.Shapes(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads,
                         s.head_dim, s.n_experts, s.top_k, s.expert_ffn,
                         s.vocab, s.rms_eps)


def to_dev(w, dev=DEV):
    return {"embed": w["embed"].to(dev), "final_norm": w["final_norm"].to(dev),
            "layers": [None if lw is None else
                       {k: (v.to(dev).contiguous() if v is not None else None)
                        for k, v in lw.items()} for lw in w["layers"]]}


def np32(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def rel_err(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    scale = np.max(np.abs(o))
    return float(np.max(np.abs(g - o)) / (scale if scale > 0 else 1.0))


def _relative(gap, vals):
    scale = np.max(np.abs(vals), axis=1)
    return gap / np.where(scale > 0, scale, 1.0)


def top2_margin(z):
    """Gap between the largest and second-largest value of each row, relative
    to the row's largest magnitude (the decision margin of an argmax)."""
    part = np.partition(z, -2, axis=1)
    return _relative(part[:, -1] - part[:, -2], z)


def routing_margin(r, k):
    """Smallest gap between consecutive sorted router logits among the first
    k + 1 ranks of each token (the rank order of the selected experts and the
    cut between selected and not selected), relative to the row's largest
    magnitude."""
    s = -np.sort(-r, axis=1)
    last = min(k, r.shape[1] - 1)
    if last == 0:
        return np.full(r.shape[0], np.inf)
    return _relative(np.min(s[:, :last] - s[:, 1:last + 1], axis=1), r)


def new_canvas_tensors(cv, dev=DEV):
    return (cv["tokens"].to(dev).contiguous(),
            cv["committed"].to(dev).contiguous(),
            cv["step"].to(dev).contiguous())


def step_outputs(n, vocab=None, dev=DEV):
    ent = torch.full((n, 256), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((n, 256), float("nan"), dtype=torch.float32, device=dev)
    am = torch.full((n, 256), -1, dtype=torch.int32, device=dev)
    logits = None
    if vocab is not None:
        logits = torch.zeros((n * 256, vocab), dtype=torch.float32, device=dev)
    return ent, lse, am, logits
