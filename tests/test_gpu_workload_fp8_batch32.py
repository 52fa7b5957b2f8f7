"""The concurrency workload at its full size: the 30-layer stack with E4M3
expert weights (per-output-channel scales) -- and its W8A8 variant, whose
projections, expert GEMMs and LM head take E4M3 weights and E4M3 token rows
(readings R13, R15, R16) --, 32 requests with their own
2048-token prefixes, 32 canvases denoised together (8192 rows per MoE grouped
GEMM and per LM head).

* One denoise step of the 32 all-masked canvases.  Lockstep (see
  tests/lockstep.py): the oracle runs canvases 0 and 31 (the first and the
  last, so both ends of every row and key mapping; canvases are
  independent) through its own 30-layer chain, and every layer's ops, the
  LM head and the EB selection are fed the oracle's values for those
  canvases at their rows of the full 32-canvas batch, so the ops take the
  paths the step takes (tiled MoE and LM head at 8192 rows).  Composition:
  all 32 canvases through all 30 layers of the step against the single-op
  entry points.
* The EB sampler (gamma 1) per request until every canvas is finished, then
  the 32 commits, checked by invariants.

The oracle gets the same seeded weights and prefixes (copied from the device)
and never any value the device computed."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, log, new_canvas_tensors, oshape, step_outputs)
from lockstep import Lockstep, lockstep_eb, lockstep_head
from workload_common import (HostPerLayer, capture_buffers,
                             check_composition, host_model)

pytestmark = pytest.mark.gpu

ORACLE_CANVASES = (0, 31)


@pytest.fixture(scope="module",
                params=["stack30_fp8_b32_p2048", "stack30_w8a8_b32_p2048"])
def batch32(request):
    global WL, SHAPE
    WL = synth.WORKLOADS[request.param]
    SHAPE = WL.shape
    assert SHAPE.expert_dtype == "fp8_e4m3" and WL.batch == 32
    log(f"{WL.name}: generating weights and 32 prefixes on the device")
    w = synth.make_weights(SHAPE, seed=1, device=DEV)
    n = WL.batch
    eng = dg.Engine(SHAPE, w, max_requests=n,
                    max_kv_len=WL.prefix_len + 256, max_canvases=n)
    prefixes = {}
    for r in range(n):
        k, v = synth.make_prefix_kv(SHAPE, WL.prefix_len, r, seed=1, device=DEV)
        eng.prefill_kv(r, k.contiguous(), v.contiguous())
        if r in ORACLE_CANVASES:
            prefixes[r] = (k, v)
        del k, v
    torch.cuda.synchronize()
    log("fp8 batch 32: engine ready")
    yield {"w": w, "eng": eng, "prefixes": prefixes, "wl": WL}
    eng.close()


@pytest.mark.timeout(900)
def test_fp8_batch32_step_lockstep_and_composition(batch32):
    eng, w = batch32["eng"], batch32["w"]
    n = WL.batch
    req = list(range(n))
    plen = [WL.prefix_len] * n
    for r in req:
        eng.set_kv_len(r, WL.prefix_len)
    cv = synth.make_canvas(SHAPE, n, 256, seed=1)
    tok, com, step = new_canvas_tensors(cv)
    ent, lse, am, _ = step_outputs(n)
    cap = capture_buffers(SHAPE, n * 256, SHAPE.n_layers, final=False)
    eng.denoise_step(req, tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    e = ent.cpu().numpy()
    a = am.cpu().numpy()
    assert np.all(np.isfinite(e)) and np.all(e >= 0)
    assert np.all(e <= math.log(SHAPE.vocab) * (1 + 1e-5))
    assert np.all((a >= 0) & (a < SHAPE.vocab))
    log("  composition: all 32 canvases, all layers")
    check_composition(eng, SHAPE, w, tok, req, plen, cap, WL.name)
    del cap
    sel = list(ORACLE_CANVASES)
    log(f"  lockstep: oracle canvases {sel}, all {SHAPE.n_layers} layers")
    pre = [(HostPerLayer(batch32["prefixes"][b][0]),
            HostPerLayer(batch32["prefixes"][b][1])) for b in sel]
    cap_o = []
    ls = Lockstep(SHAPE, eng, w, n, req, plen, sel, cap_o, WL.name, seed=1)
    ref = oracle.denoise_step(oshape(SHAPE), host_model(w, stop=ls),
                              cv["tokens"].numpy()[sel],
                              cv["committed"].numpy()[sel], pre, mirror=True,
                              want_logits=True, capture=cap_o)
    assert ls.finish() == SHAPE.n_layers
    ls.report()
    lm8 = None
    if w.get("lm_head") is not None:
        lm8 = (w["lm_head"].cpu().numpy(), w["lm_head_scale"].cpu().numpy())
    lockstep_head(SHAPE, eng, w, ref, ls.x_last, cv["committed"].numpy(), n,
                  sel, WL.name, seed=1, lm8_host=lm8)
    lockstep_eb(ref["entropy"], ref["argmax"], cv["committed"].numpy()[sel],
                cv["tokens"].numpy()[sel], cv["step"].numpy()[sel], WL.gamma,
                WL.step_cap, WL.name)


def test_fp8_batch32_decode_until_every_block_is_committed(batch32):
    """EB per request (gamma 1, cap 256) over the 32 canvases until all are
    done: an unfinished canvas commits >= 1 position per step (exactly one
    while its smallest uncommitted entropy exceeds gamma), a finished one
    none; every canvas finishes within 256 steps; then the 32 blocks are
    committed and every cache grows by 256 rows."""
    eng = batch32["eng"]
    n = WL.batch
    req = list(range(n))
    for r in req:
        eng.set_kv_len(r, WL.prefix_len)
    cv = synth.make_canvas(SHAPE, n, WL.uncommitted, seed=2)
    tok, com, step = new_canvas_tensors(cv)
    ent, lse, am, _ = step_outputs(n)
    gamma = torch.full((n,), WL.gamma, dtype=torch.float32, device=DEV)
    n_new = torch.zeros(n, dtype=torch.int32, device=DEV)
    done = torch.zeros(n, dtype=torch.uint8, device=DEV)
    finished = np.zeros(n, dtype=bool)
    steps = 0
    while not finished.all():
        com_before = com.cpu().numpy().copy()
        eng.denoise_step(req, tok, com, step, ent, lse, am)
        eng.eb_select(req, tok, com, step, ent, am, gamma, WL.step_cap, True,
                      n_new, done)
        torch.cuda.synchronize()
        steps += 1
        nn = n_new.cpu().numpy()
        e = ent.cpu().numpy()
        dn = done.cpu().numpy().astype(bool)
        for b in range(n):
            unc = com_before[b] == 0
            if finished[b]:
                assert nn[b] == 0 and dn[b]
                continue
            assert nn[b] >= 1
            assert np.all(np.isfinite(e[b, unc])) and np.all(e[b, unc] >= 0)
            if e[b, unc].min() > WL.gamma and unc.sum() > 1 and \
                    steps < WL.step_cap:
                assert nn[b] == 1
        finished |= dn
        assert steps <= WL.step_cap
        if steps % 64 == 0:
            log(f"  step {steps}: {int(finished.sum())} canvases finished")
    assert bool(com.cpu().numpy().all())
    t = tok.cpu().numpy()
    assert np.all((t >= 0) & (t < SHAPE.vocab))
    eng.commit_block(req, tok, com, step)
    torch.cuda.synchronize()
    for r in req:
        assert eng.kv_len(r) == WL.prefix_len + 256
    log(f"  all 32 canvases finished after {steps} steps and were committed")
