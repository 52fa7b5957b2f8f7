"""Canvas size 128 (write-up Table 7 varies the canvas size: 128 or 256) on
a two-layer model: a denoise step in lockstep with the oracle (every layer's
ops, the LM head and the EB selection fed the oracle's values) and against
the single-op entry points; the EB decode of a whole 128-position block
(gamma 0 commits one position per step, so exactly 128 steps); the commit
of the block (lockstep K/V, the cache rows against the op chain, 128 rows
appended)."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, log, np32, oshape, to_dev
from lockstep import Lockstep, lockstep_eb, lockstep_head
from workload_common import (capture_buffers, check_commit_composition,
                             check_composition)

pytestmark = pytest.mark.gpu

SHAPE = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096, canvas_len=128)
C = 128
P = 200


def _setup():
    w = synth.make_weights(SHAPE, seed=9, gain_std=0.1)
    wd = to_dev(w)
    eng = dg.Engine(SHAPE, wd, max_requests=1, max_kv_len=1024, max_canvases=1)
    k, v = synth.make_prefix_kv(SHAPE, P, 0, seed=9)
    eng.prefill_kv(0, k.to(DEV).contiguous(), v.to(DEV).contiguous())
    return eng, w, wd, [(np32(k), np32(v))]


def _outs():
    ent = torch.full((1, C), float("nan"), device=DEV)
    lse = torch.full((1, C), float("nan"), device=DEV)
    am = torch.full((1, C), -1, dtype=torch.int32, device=DEV)
    return ent, lse, am


def test_canvas128_step_lockstep_composition_and_block_decode():
    eng, w, wd, prefix = _setup()
    cv = synth.make_canvas(SHAPE, 1, 100, seed=2)
    assert cv["tokens"].shape == (1, C)
    tok, com, step = (t.to(DEV).contiguous() for t in
                      (cv["tokens"], cv["committed"], cv["step"]))
    ent, lse, am = _outs()
    cap = capture_buffers(SHAPE, C, SHAPE.n_layers, final=False)
    eng.denoise_step([0], tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    check_composition(eng, SHAPE, wd, tok, [0], [P], cap, "canvas128")
    cap_o = []
    ref = oracle.denoise_step(oshape(SHAPE), synth.to_numpy_weights(w),
                              cv["tokens"].numpy(), cv["committed"].numpy(),
                              prefix, mirror=True, want_logits=True,
                              capture=cap_o)
    ls = Lockstep(SHAPE, eng, eng.weights, 1, [0], [P], [0], cap_o,
                  "canvas128", C=C)
    assert ls.finish() == SHAPE.n_layers
    ls.report()
    lockstep_head(SHAPE, eng, eng.weights, ref, ls.x_last,
                  cv["committed"].numpy(), 1, [0], "canvas128")
    lockstep_eb(ref["entropy"], ref["argmax"], cv["committed"].numpy(),
                cv["tokens"].numpy(), cv["step"].numpy(), 0.5, 256, "canvas128")
    # a whole block: every position uncommitted, gamma 0 -> one per step
    cv = synth.make_canvas(SHAPE, 1, C, seed=3)
    tok, com, step = (t.to(DEV).contiguous() for t in
                      (cv["tokens"], cv["committed"], cv["step"]))
    gamma = torch.zeros(1, device=DEV)
    n_new = torch.zeros(1, dtype=torch.int32, device=DEV)
    done = torch.zeros(1, dtype=torch.uint8, device=DEV)
    steps = 0
    while True:
        eng.denoise_step([0], tok, com, step, ent, lse, am)
        eng.eb_select([0], tok, com, step, ent, am, gamma, 256, True, n_new, done)
        torch.cuda.synchronize()
        steps += 1
        assert int(n_new.item()) == 1
        if int(done.item()):
            break
        assert steps < C
    assert steps == C and int(step.item()) == C
    assert bool(com.all())
    eng.commit_block([0], tok, com, step)
    torch.cuda.synchronize()
    assert eng.kv_len(0) == P + C
    check_commit_composition(eng, SHAPE, wd, tok, [0], [P], "canvas128", C=C)
    kv_o, cap_o = [], []
    ls = Lockstep(SHAPE, eng, eng.weights, 1, [0], [P], [0], cap_o,
                  "canvas128 commit", causal=True, kv_o=kv_o, C=C)
    oracle.model._layers_forward(oshape(SHAPE), synth.to_numpy_weights(w),
                                 tok.cpu().numpy(), prefix, True, True, cap_o,
                                 kv_out=kv_o)
    assert ls.finish() == SHAPE.n_layers
    ls.report()
    eng.close()
