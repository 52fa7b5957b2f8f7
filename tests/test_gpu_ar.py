"""AR mode (write-up "What they did": the same weights decode left to right;
model card "Model Overview") through dg_ar_step against the oracle's
ar_step: next-token statistics and the K/V appended to the cache, step
after step, both sides fed the oracle's greedy token and the same cache
(the oracle reads back the rows the device appended).

A position whose oracle routing has a near tie in some layer (the k-th and
(k+1)-th router logits closer than MARGIN) may be routed differently by the
device: its statistics and the K/V of the layers after that one are
reported, not asserted."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, MARGIN, TOL, log, np32, oshape, rel_err, to_dev

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny_l1_h256_p512"].shape
TWO = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096)
GEMMA = synth.WORKLOADS["moe_layer_h2048_v262k_p2048"].shape


def _setup(shape, plens, max_kv=1024, seed=4):
    w = synth.make_weights(shape, seed=seed, gain_std=0.1)
    eng = dg.Engine(shape, to_dev(w), max_requests=len(plens),
                    max_kv_len=max_kv, max_canvases=1)
    caches = []
    for r, p in enumerate(plens):
        k, v = synth.make_prefix_kv(shape, p, r, seed=seed)
        if p:
            eng.prefill_kv(r, k.to(DEV).contiguous(), v.to(DEV).contiguous())
        else:
            eng.set_kv_len(r, 0)
        caches.append([np32(k), np32(v)])
    return eng, synth.to_numpy_weights(w), caches


def _route_gaps(shape, cap):
    """[n, L]: gap between the k-th and (k+1)-th router logits per layer."""
    gaps = []
    for c in cap:
        srt = -np.sort(-np.asarray(c["router_logits"], np.float64), axis=1)
        gaps.append(srt[:, shape.top_k - 1] - srt[:, shape.top_k]
                    if shape.top_k < srt.shape[1] else np.full(len(srt), np.inf))
    return np.stack(gaps, axis=1)


def _ar_compare(shape, eng, wn, caches, req, tokens, tag):
    """One AR step on both sides; returns the oracle's greedy tokens."""
    n = len(req)
    ent = torch.full((n,), float("nan"), device=DEV)
    lse = torch.full_like(ent, float("nan"))
    am = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    logits = torch.zeros((n, shape.vocab), device=DEV)
    plen = [eng.kv_len(r) for r in req]
    eng.ar_step(req, torch.tensor(tokens, dtype=torch.int32, device=DEV),
                ent, lse, am, logits)
    torch.cuda.synchronize()
    cap = []
    ref = oracle.ar_step(oshape(shape), wn, np.asarray(tokens),
                         [tuple(caches[r]) for r in req], mirror=True,
                         request=req, want_logits=True, capture=cap)
    gaps = _route_gaps(shape, cap)
    tied = gaps < MARGIN                       # [n, L]
    # first layer whose routing may differ (L when none)
    first = np.where(tied.any(1), tied.argmax(1), shape.n_layers)
    ok = first == shape.n_layers
    e_h = rel_err(ent.cpu().numpy()[ok], ref["entropy"][ok])
    e_l = rel_err(lse.cpu().numpy()[ok], ref["lse"][ok])
    e_z = rel_err(logits.cpu().numpy()[ok], ref["logits"][ok])
    srt = np.sort(ref["logits"], axis=1)
    marg = srt[:, -1] - srt[:, -2]
    ga = am.cpu().numpy()
    diff = (ga != ref["argmax"]) & ok
    # K/V appended: position j of a sequence sits at its kv_len before the
    # step plus j; layer l's K/V follow the routing of layers < l only
    e_kv, seen, rows = 0.0, {}, []
    for b, r in enumerate(req):
        j = seen.get(r, 0)
        seen[r] = j + 1
        row = plen[b] + j
        rows.append(row)
        for which, i in (("k", 0), ("v", 1)):
            got = eng.cache_view(which)[:, r, :, row, :].float().cpu().numpy()
            lim = first[b] + 1
            e_kv = max(e_kv, rel_err(got[:lim], ref["kv"][b][i][:lim, :, 0]))
    log(f"  {tag}: entropy {e_h:.2e} lse {e_l:.2e} logits {e_z:.2e} K/V "
        f"{e_kv:.2e}; argmax differs at {int(diff.sum())} of {int(ok.sum())} "
        f"(margins {np.sort(marg[diff]).tolist()}); near-tied routing at "
        f"positions {np.flatnonzero(~ok).tolist()} (gaps "
        f"{[float(gaps[i].min()) for i in np.flatnonzero(~ok)]})")
    assert e_h < TOL and e_l < TOL and e_z < TOL and e_kv < TOL
    assert not (diff & (marg >= MARGIN)).any()
    for b, r in enumerate(req):
        assert eng.kv_len(r) == plen[b] + seen[r]
    # both sides continue from the device's cache: the oracle's prefix grows
    # by the rows the device appended
    for b, r in enumerate(req):
        for which, i in (("k", 0), ("v", 1)):
            got = eng.cache_view(which)[:, r, :, rows[b]:rows[b] + 1, :]
            caches[r][i] = np.concatenate(
                [caches[r][i], got.float().cpu().numpy().astype(np.float64)],
                axis=2)
    return ref["argmax"]


@pytest.mark.parametrize("shape,name", [
    (TINY, "tiny"), (TWO, "two-layer"),
    (synth.ModelShape(**{**TWO.__dict__, "lm_dtype": "fp8_e4m3"}),
     "two-layer, E4M3 head")])
def test_ar_decode_steps_against_oracle(shape, name):
    """Two sequences (prefixes 300 and 77) decode five tokens each."""
    log(f"AR {name}")
    eng, wn, caches = _setup(shape, [300, 77])
    rng = np.random.default_rng(5)
    tok = rng.integers(0, shape.vocab, 2)
    for step in range(5):
        tok = _ar_compare(shape, eng, wn, caches, [0, 1], tok,
                          f"{name} step {step}")
    eng.close()


def test_ar_several_positions_of_one_sequence_and_empty_cache():
    """Sequence 0 takes three positions in one call (causal among them),
    sequence 1 starts from an empty cache."""
    log("AR multi-position")
    eng, wn, caches = _setup(TWO, [120, 0])
    _ar_compare(TWO, eng, wn, caches, [0, 0, 0, 1], [5, 17, 4095, 9],
                "three + one")
    _ar_compare(TWO, eng, wn, caches, [0, 1, 1], [1, 2, 3], "one + two")
    eng.close()


def test_ar_step_full_size_layer():
    """Hidden 2048, 262144-token vocabulary, 128 experts, prefix 2048."""
    log("AR full-size layer")
    eng, wn, caches = _setup(GEMMA, [2048], max_kv=2304)
    tok = np.array([1234])
    for step in range(3):
        tok = _ar_compare(GEMMA, eng, wn, caches, [0], tok,
                          f"full-size step {step}")
    eng.close()


def test_ar_step_validation():
    eng, _, _ = _setup(TINY, [510, 3], max_kv=512)
    ent = torch.zeros(4, device=DEV)
    lse = torch.zeros_like(ent)
    am = torch.zeros(4, dtype=torch.int32, device=DEV)
    tok = torch.zeros(4, dtype=torch.int32, device=DEV)
    for req, code in (([0, 1, 0], 1), ([0, 0, 0], 3), ([2], 1), ([], 3)):
        with pytest.raises(dg.DgError) as e:
            eng.ar_step(req, tok, ent, lse, am)
        assert e.value.status == code, req
    assert eng.kv_len(0) == 510 and eng.kv_len(1) == 3
    eng.ar_step([0, 0], tok, ent, lse, am)   # exactly fills the cache
    torch.cuda.synchronize()
    assert eng.kv_len(0) == 512
    eng.close()
