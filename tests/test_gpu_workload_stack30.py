"""The 30-layer stack (hidden 2048, 16/8 heads of 128, 128 experts top-8 of
width 768, vocab 262144, bf16) through the context API at its full size.

* 4096-token prefix: one denoise step of an all-masked canvas against the
  oracle, layer by layer up to the first low-margin routing difference
  (after it the two residual streams legitimately part), and the LM head
  too when the stack gets through without one; every layer, the final norm
  and the LM head of the step against the single-op entry points
  (composition); the causal commit of a seeded block against the oracle on
  its first layers; four blocks decoded with the EB sampler (gamma 1, step
  cap 64) and committed, checked by invariants.
* 131072-token prefix: the first layers of a denoise step against the oracle
  (its attention over 131k keys takes seconds per layer), all 30 by
  composition (cache offsets of the deep layers pass 2^31 elements), then
  twelve denoise steps with EB selection checked by invariants.

The oracle gets the same seeded weights and prefixes (copied from the device,
one layer at a time) and never any value the device computed."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, MARGIN, TOL, log, new_canvas_tensors, np32,
                        oshape, rel_err, routing_margin, step_outputs,
                        top2_margin)
from workload_common import (ChainChecker, HostPerLayer, capture_buffers,
                             check_composition, host_model)

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["stack30_h2048_p4096"]
WL_LONG = synth.WORKLOADS["stack30_h2048_p131072"]
SHAPE = WL.shape
ORACLE_LAYERS_LONG = 6   # at most this many layers of the 131k-prefix step
                         # go through the oracle


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


def test_stack30_denoise_step_against_oracle(stack):
    eng, w = stack["eng"], stack["w"]
    P = WL.prefix_len
    eng.set_kv_len(0, P)
    cv = synth.make_canvas(SHAPE, 1, 256, seed=0)
    tok, com, step = new_canvas_tensors(cv)
    ent, lse, am, _ = step_outputs(1)
    cap = capture_buffers(SHAPE, 256, SHAPE.n_layers)
    eng.denoise_step([0], tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    log("stack30 step: device done; oracle layer by layer")
    k, v = stack["prefix"]
    cap_o = []
    chk = ChainChecker(SHAPE, cap, cap_o, np.arange(256), "stack30")
    ref = oracle.denoise_step(oshape(SHAPE), host_model(w, stop=chk),
                              cv["tokens"].numpy(), cv["committed"].numpy(),
                              [(HostPerLayer(k), HostPerLayer(v))],
                              mirror=True, want_logits=True, capture=cap_o)
    n_cmp = chk.finish()
    g_ent = ent.cpu().numpy()[0]
    g_lse = lse.cpu().numpy()[0]
    g_am = am.cpu().numpy()[0]
    if not chk.flipped and n_cmp == SHAPE.n_layers:
        rows = ref["rows"]                  # all 256 positions are masked
        assert np.array_equal(rows, np.arange(256))
        e_x = rel_err(np32(cap["final_xhat"]), ref["final_xhat"])
        e_ent = rel_err(g_ent, ref["entropy"][0])
        e_lse = rel_err(g_lse, ref["lse"][0])
        marg = top2_margin(ref["logits"])
        am_diff = g_am != ref["argmax"][0]
        log(f"  oracle LM head: final norm {e_x:.2e}, entropy {e_ent:.2e}, "
            f"lse {e_lse:.2e}; argmax differences {int(am_diff.sum())}")
        assert e_x < TOL and e_ent < TOL and e_lse < TOL
        assert np.all(marg[am_diff] < MARGIN), "argmax differs at a clear margin"
    else:
        log(f"  oracle compared {n_cmp} layer(s); the LM head is checked by "
            "composition and by the full-vocabulary op tests")
    # every layer, the final norm and the LM head by composition
    x_fin = check_composition(eng, SHAPE, w, tok, [0], [P], cap, "stack30")
    xf = torch.empty((256, SHAPE.hidden), dtype=torch.bfloat16, device=DEV)
    dg.op_rmsnorm(x_fin, w["final_norm"], SHAPE.rms_eps, xf)
    e_x = rel_err(np32(xf), np32(cap["final_xhat"]))
    ent2 = torch.empty(256, dtype=torch.float32, device=DEV)
    lse2 = torch.empty_like(ent2)
    am2 = torch.empty(256, dtype=torch.int32, device=DEV)
    dg.op_lmhead_entropy(cap["final_xhat"].to(torch.bfloat16), w["embed"],
                         ent2, lse2, am2)
    torch.cuda.synchronize()
    e_ent = rel_err(g_ent, ent2.cpu().numpy())
    e_lse = rel_err(g_lse, lse2.cpu().numpy())
    log(f"  composition: final norm {e_x:.2e}; LM head entropy {e_ent:.2e} "
        f"lse {e_lse:.2e}")
    assert e_x < TOL and e_ent < 1e-6 and e_lse < 1e-6
    np.testing.assert_array_equal(g_am, am2.cpu().numpy())
    _invariant_step(g_ent, g_am, cv["committed"].numpy()[0], SHAPE.vocab)


def test_stack30_commit_first_layers_against_oracle(stack):
    """Causal encode-and-append of a seeded finished block: the appended K/V
    of the first layers against the oracle.  The commit has no captures, so
    rows that may carry a different residual are left out: a token whose
    routing in layer l has an oracle margin below MARGIN, from layer l+1 on,
    and through the causal attention every row after it one layer later."""
    eng, w = stack["eng"], stack["w"]
    P = WL.prefix_len
    n_cmp = 4
    eng.set_kv_len(0, P)
    cv = synth.make_canvas(SHAPE, 1, 0, seed=3)
    tok, com, step = new_canvas_tensors(cv)
    eng.commit_block([0], tok, com, step)
    torch.cuda.synchronize()
    assert eng.kv_len(0) == P + 256
    k, v = stack["prefix"]
    kv_o, cap_o = [], []
    oracle.model._layers_forward(oshape(SHAPE), host_model(w, n_cmp),
                                 cv["tokens"].numpy(),
                                 [(HostPerLayer(k), HostPerLayer(v))],
                                 True, True, cap_o, kv_out=kv_o)
    kc, vc = eng.cache_view("k"), eng.cache_view("v")
    bad = np.zeros(256, dtype=bool)   # rows whose K/V may differ
    for li in range(n_cmp):
        if li > 0:
            if bad.any():
                bad[int(np.argmax(bad)):] = True
            bad |= routing_margin(cap_o[li - 1]["router_logits"],
                                  SHAPE.top_k) < MARGIN
        ok = ~bad
        if not ok.any():
            log(f"  commit layer {li}: no row left to compare")
            break
        gk = np32(kc[li, 0, :, P:P + 256])
        gv = np32(vc[li, 0, :, P:P + 256])
        ek = rel_err(gk[:, ok], kv_o[li][0][:, ok])
        ev = rel_err(gv[:, ok], kv_o[li][1][:, ok])
        log(f"  commit layer {li}: K {ek:.2e} V {ev:.2e} on {int(ok.sum())} rows")
        assert ek < TOL and ev < TOL
    # the prefix rows are untouched
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


def test_long_prefix_131k_step_and_twelve_steps(stack):
    eng, w = stack["eng"], stack["w"]
    P = WL_LONG.prefix_len
    log("131k prefix: generating and installing the cache")
    k, v = synth.make_prefix_kv(SHAPE, P, 1, seed=0, device=DEV)
    eng.prefill_kv(1, k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    cv = synth.make_canvas(SHAPE, 1, WL_LONG.uncommitted, seed=5)
    tok, com, step = new_canvas_tensors(cv)
    ent, lse, am, _ = step_outputs(1)
    cap = capture_buffers(SHAPE, 256, SHAPE.n_layers, final=False)
    eng.denoise_step([1], tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    log("  device step done; oracle layer by layer")
    cap_o = []
    chk = ChainChecker(SHAPE, cap, cap_o, np.arange(256), "p131k")
    oracle.model._layers_forward(
        oshape(SHAPE), host_model(w, ORACLE_LAYERS_LONG, stop=chk),
        cv["tokens"].numpy(), [(HostPerLayer(k), HostPerLayer(v))], True,
        False, cap_o)
    chk.finish()
    check_composition(eng, SHAPE, w, tok, [1], [P], cap, "p131k")
    del cap
    # twelve steps of the decode loop
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
