"""The 30-layer stack (hidden 2048, 16/8 heads of 128, 128 experts top-8 of
width 768, vocab 262144, bf16) through the context API at its full size.

Parity has two links (see tests/lockstep.py):
  1. lockstep: the oracle runs its own 30-layer chain from the seeded
     inputs; every layer's ops are fed the oracle's own values for that
     layer and compared with its next values, then the final norm, the LM
     head and the EB selection likewise -- all 30 layers, the head and EB;
  2. composition: the step's fused kernels against the single-op entry
     points on the step's own state, layer by layer.

* 4096-token prefix: a denoise step of an all-masked canvas (both links);
  the causal commit of a seeded block (lockstep K/V of all 30 layers, and
  the appended cache rows against the op chain); four blocks decoded with
  the EB sampler (gamma 1, step cap 64) and committed, checked by
  invariants.
* 131072-token prefix: a denoise step (both links, all 30 layers), then
  twelve denoise steps with EB selection checked by invariants.

The oracle gets the same seeded weights and prefixes (copied from the device,
one layer at a time) and never any value the device computed."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, log, new_canvas_tensors, oshape, step_outputs)
from lockstep import Lockstep, lockstep_eb, lockstep_head
from workload_common import (HostPerLayer, capture_buffers,
                             check_commit_composition, check_composition,
                             host_model)

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["stack30_h2048_p4096"]
WL_LONG = synth.WORKLOADS["stack30_h2048_p131072"]
SHAPE = WL.shape


@pytest.fixture(scope="module")
def stack():
    """Weights on the device, one engine with two request slots: slot 0 holds
    the 4096-token prefix, slot 1 the 131072-token one."""
    assert WL_LONG.shape == SHAPE
    log("stack30: generating weights on the device")
    w = synth.make_weights(SHAPE, seed=0, device=DEV)
    eng = dg.Engine(SHAPE, w, max_requests=2,
                    max_kv_len=WL_LONG.prefix_len + 256, max_canvases=1)
    k, v = synth.make_prefix_kv(SHAPE, WL.prefix_len, 0, seed=0, device=DEV)
    eng.prefill_kv(0, k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    log("stack30: engine ready")
    yield {"w": w, "eng": eng, "prefix": (k, v)}
    eng.close()


def _invariant_step(ent, am, com_before, vocab):
    """Entropy in [0, ln V] (within rounding), argmax a vocabulary id, at every
    position uncommitted before the step."""
    unc = com_before == 0
    e = ent[unc]
    a = am[unc]
    assert np.all(np.isfinite(e)) and np.all(e >= 0.0)
    assert np.all(e <= math.log(vocab) * (1 + 1e-5))
    assert np.all((a >= 0) & (a < vocab))


def _step_both_links(stack, req, P, prefix, cv, tag, step_cap):
    eng, w = stack["eng"], stack["w"]
    tok, com, step = new_canvas_tensors(cv)
    ent, lse, am, _ = step_outputs(1)
    cap = capture_buffers(SHAPE, 256, SHAPE.n_layers)
    eng.denoise_step([req], tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    _invariant_step(ent.cpu().numpy()[0], am.cpu().numpy()[0],
                    cv["committed"].numpy()[0], SHAPE.vocab)
    log(f"{tag}: composition (step vs ops on the step's own state)")
    check_composition(eng, SHAPE, w, tok, [req], [P], cap, tag)
    del cap
    log(f"{tag}: lockstep (ops fed the oracle's values, all layers)")
    k, v = prefix
    cap_o = []
    ls = Lockstep(SHAPE, eng, w, 1, [req], [P], [0], cap_o, tag)
    ref = oracle.denoise_step(oshape(SHAPE), host_model(w, stop=ls),
                              cv["tokens"].numpy(), cv["committed"].numpy(),
                              [(HostPerLayer(k), HostPerLayer(v))],
                              mirror=True, want_logits=True, capture=cap_o)
    assert ls.finish() == SHAPE.n_layers
    ls.report()
    lockstep_head(SHAPE, eng, w, ref, ls.x_last, cv["committed"].numpy(), 1,
                  [0], tag)
    lockstep_eb(ref["entropy"], ref["argmax"], cv["committed"].numpy(),
                cv["tokens"].numpy(), cv["step"].numpy(), WL.gamma, step_cap,
                tag)
    # the step's own outputs against the oracle's (a diagnostic: the two
    # chains part at bf16 rounding straddles)
    rows = ref["rows"]
    g_ent = ent.cpu().numpy().reshape(-1)[rows]
    o_ent = ref["entropy"].reshape(-1)[rows]
    agree = np.mean(am.cpu().numpy().reshape(-1)[rows] ==
                    ref["argmax"].reshape(-1)[rows])
    log(f"  {tag} free-running step vs oracle (diagnostic): entropy max abs "
        f"diff {np.max(np.abs(g_ent - o_ent)):.2e}, argmax agreement {agree:.3f}")


def test_stack30_denoise_step_lockstep_and_composition(stack):
    eng = stack["eng"]
    eng.set_kv_len(0, WL.prefix_len)
    cv = synth.make_canvas(SHAPE, 1, 256, seed=0)
    _step_both_links(stack, 0, WL.prefix_len, stack["prefix"], cv, "stack30",
                     WL.step_cap)


def test_stack30_commit_lockstep_and_composition(stack):
    """Causal encode-and-append of a seeded finished block: the appended
    K/V of all 30 layers in lockstep with the oracle, and the cache rows
    dg_commit_block wrote against the op chain on the same tokens."""
    eng, w = stack["eng"], stack["w"]
    P = WL.prefix_len
    eng.set_kv_len(0, P)
    cv = synth.make_canvas(SHAPE, 1, 0, seed=3)
    tok, com, step = new_canvas_tensors(cv)
    eng.commit_block([0], tok, com, step)
    torch.cuda.synchronize()
    assert eng.kv_len(0) == P + 256
    check_commit_composition(eng, SHAPE, w, tok, [0], [P], "stack30")
    k, v = stack["prefix"]
    kv_o, cap_o = [], []
    ls = Lockstep(SHAPE, eng, w, 1, [0], [P], [0], cap_o, "stack30 commit",
                  causal=True, kv_o=kv_o)
    oracle.model._layers_forward(oshape(SHAPE), host_model(w, stop=ls),
                                 cv["tokens"].numpy(),
                                 [(HostPerLayer(k), HostPerLayer(v))],
                                 True, True, cap_o, kv_out=kv_o)
    assert ls.finish() == SHAPE.n_layers
    ls.report()
    # the prefix rows are untouched
    kc, vc = eng.cache_view("k"), eng.cache_view("v")
    for li in (0, SHAPE.n_layers - 1):
        assert torch.equal(kc[li, 0, :, :P], k[li])
        assert torch.equal(vc[li, 0, :, :P], v[li])
    eng.set_kv_len(0, P)


def test_stack30_decode_four_blocks(stack):
    """Four blocks: denoise + EB (gamma 1, cap 64) until done, then commit.
    Every step commits >= 1 position, and exactly one while the smallest
    uncommitted entropy exceeds gamma and the cap is not reached; the cap
    step commits the rest; the cache grows by 256 rows per block and the
    prefix rows stay as they were."""
    eng = stack["eng"]
    P, cap_steps = WL.prefix_len, WL.step_cap
    eng.set_kv_len(0, P)
    gamma = torch.full((1,), WL.gamma, dtype=torch.float32, device=DEV)
    n_new = torch.zeros(1, dtype=torch.int32, device=DEV)
    done = torch.zeros(1, dtype=torch.uint8, device=DEV)
    k, v = stack["prefix"]
    for blk in range(WL.blocks):
        cv = synth.make_canvas(SHAPE, 1, WL.uncommitted, seed=0, block=blk)
        tok, com, step = new_canvas_tensors(cv)
        ent, lse, am, _ = step_outputs(1)
        steps, total = 0, 0
        while True:
            com_before = com.cpu().numpy()[0].copy()
            eng.denoise_step([0], tok, com, step, ent, lse, am)
            eng.eb_select([0], tok, com, step, ent, am, gamma, cap_steps, True,
                          n_new, done)
            torch.cuda.synchronize()
            steps += 1
            e = ent.cpu().numpy()[0]
            _invariant_step(e, am.cpu().numpy()[0], com_before, SHAPE.vocab)
            nn = int(n_new.item())
            unc = int((com_before == 0).sum())
            assert nn >= 1
            if steps == cap_steps:
                assert nn == unc
            elif e[com_before == 0].min() > WL.gamma:
                assert nn == 1
            total += nn
            assert int(step.item()) == steps
            if int(done.item()):
                break
            assert steps < cap_steps
        assert total == WL.uncommitted and bool(com.cpu().numpy().all())
        t = tok.cpu().numpy()
        assert np.all((t >= 0) & (t < SHAPE.vocab))
        eng.commit_block([0], tok, com, step)
        torch.cuda.synchronize()
        assert eng.kv_len(0) == P + 256 * (blk + 1)
        log(f"  block {blk}: {steps} steps")
    kc, vc = eng.cache_view("k"), eng.cache_view("v")
    for li in (0, SHAPE.n_layers - 1):
        assert torch.equal(kc[li, 0, :, :P], k[li])
        new = kc[li, 0, :, P:P + 256 * WL.blocks].float()
        assert torch.isfinite(new).all() and new.abs().amax() > 0
    eng.set_kv_len(0, P)


@pytest.mark.timeout(900)
def test_long_prefix_131k_lockstep_and_twelve_steps(stack):
    eng = stack["eng"]
    P = WL_LONG.prefix_len
    log("131k prefix: generating and installing the cache")
    k, v = synth.make_prefix_kv(SHAPE, P, 1, seed=0, device=DEV)
    eng.prefill_kv(1, k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    cv = synth.make_canvas(SHAPE, 1, WL_LONG.uncommitted, seed=5)
    _step_both_links(stack, 1, P, (k, v), cv, "p131k", WL_LONG.step_cap)
    del k, v
    # twelve steps of the decode loop
    ent, lse, am, _ = step_outputs(1)
    gamma = torch.full((1,), WL_LONG.gamma, dtype=torch.float32, device=DEV)
    n_new = torch.zeros(1, dtype=torch.int32, device=DEV)
    done = torch.zeros(1, dtype=torch.uint8, device=DEV)
    tok, com, step = new_canvas_tensors(cv)
    total = 0
    for s in range(WL_LONG.steps):
        com_before = com.cpu().numpy()[0].copy()
        eng.denoise_step([1], tok, com, step, ent, lse, am)
        eng.eb_select([1], tok, com, step, ent, am, gamma, WL_LONG.step_cap,
                      True, n_new, done)
        torch.cuda.synchronize()
        e = ent.cpu().numpy()[0]
        _invariant_step(e, am.cpu().numpy()[0], com_before, SHAPE.vocab)
        nn = int(n_new.item())
        assert nn >= 1
        if e[com_before == 0].min() > WL_LONG.gamma:
            assert nn == 1
        total += nn
    assert int(step.item()) == WL_LONG.steps
    assert int((com.cpu().numpy() == 1).sum()) == 256 - WL_LONG.uncommitted + total
    assert eng.kv_len(1) == P
    log(f"  twelve steps committed {total} positions")
