"""Temperature sampling (write-up Figure 9 and Figure 10, tau_t with
annealing; Gumbel-max draws from Philox4x32-10) on the GPU against the
oracle: the LM-head op on both of its kernels (up to 128 rows, and the
256 x 256 tile kernel above), the distribution of the draws, and the
denoising step's wiring of temperatures and counters."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, MARGIN, log, np32, oshape, rel_err,
                        step_outputs, to_dev)

pytestmark = pytest.mark.gpu

SEED = 0x9E3779B97F4A7C15


def _randn(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _score_margin(z, tau, ctr, seed):
    """Per row: the gap between the two best Gumbel-max scores (the two
    largest logits at temperature 0), in the oracle's fp64."""
    v = np.arange(z.shape[1])
    out = np.empty(z.shape[0])
    for r in range(z.shape[0]):
        if tau[r] > 0:
            s = z[r] / tau[r] + oracle.gumbel(v, int(ctr[r][0]), int(ctr[r][1]),
                                              int(ctr[r][2]), seed)
        else:
            s = z[r]
        top = np.partition(s, -2)[-2:]
        out[r] = top[1] - top[0]
    return out


def _check_rows(tag, st, tau, ctr, ent, lse, am, smp):
    """GPU rows against oracle.lm_head_sample's: lse and entropy to fp32
    accuracy, argmax and the drawn token bit-exact except where the
    oracle's own decision is closer than the absolute margin."""
    g_ent, g_lse = ent.cpu().numpy(), lse.cpu().numpy()
    g_am, g_smp = am.cpu().numpy(), smp.cpu().numpy()
    zero = tau <= 0
    assert np.all(g_ent[zero] == 0.0), "temperature 0 must give entropy 0"
    assert np.all(g_smp[zero] == g_am[zero]), "temperature 0 draws the argmax"
    e_h = rel_err(g_ent, st["entropy"])
    e_l = rel_err(g_lse, st["lse"])
    marg_am = np.diff(np.sort(st["logits"], axis=1)[:, -2:], axis=1)[:, 0]
    marg_s = _score_margin(st["logits"], tau, ctr, SEED)
    d_am = g_am != st["argmax"]
    d_s = g_smp != st["sample"]
    log(f"  {tag}: entropy {e_h:.2e} lse {e_l:.2e}; argmax differs at "
        f"{int(d_am.sum())}, draw at {int(d_s.sum())} rows (margins "
        f"{np.sort(marg_s[d_s]).tolist()[:8]}); draws equal to argmax at "
        f"{int((g_smp == g_am).sum())} of {len(g_smp)} rows")
    assert e_h < 1e-4 and e_l < 1e-5
    assert not (d_am & (marg_am >= MARGIN)).any()
    assert not (d_s & (marg_s >= MARGIN)).any()


@pytest.mark.parametrize("m,h,v", [(5, 256, 1000), (128, 256, 4096),
                                   (300, 256, 3000), (48, 2048, 262144),
                                   (129, 2048, 262144)])
def test_lmhead_sample_matches_oracle(m, h, v):
    tag = f"sample M={m} H={h} V={v}"
    log(tag)
    xh = _randn((m, h), 1.0, 11 + m)
    embed = _randn((v, h), 0.05 if h == 256 else 0.02, 17 + v)
    taus = np.array([0.0, 0.25, 0.7, 1.0, 1.5])
    tau = taus[np.arange(m) % len(taus)]
    r = np.arange(m)
    ctr = np.stack([r % 256, (r * 7) % 19, (r // 3) % 4], axis=1)
    ent = torch.empty(m, dtype=torch.float32, device=DEV)
    lse = torch.empty_like(ent)
    am = torch.empty(m, dtype=torch.int32, device=DEV)
    smp = torch.empty_like(am)
    dg.op_lmhead_sample(xh.to(DEV), embed.to(DEV),
                        torch.tensor(tau, dtype=torch.float32, device=DEV),
                        torch.tensor(ctr, dtype=torch.int32, device=DEV),
                        SEED, ent, lse, am, smp)
    torch.cuda.synchronize()
    st = oracle.lm_head_sample(np32(xh), np32(embed), tau.astype(np.float32),
                               ctr, SEED)
    _check_rows(tag, st, tau, ctr, ent, lse, am, smp)


def test_draws_follow_the_tempered_softmax():
    """One row repeated 8192 times under distinct counters: the draws'
    frequencies match softmax(z / tau) (chi-square well inside its
    spread), every row reports the same entropy, and that entropy is the
    tempered distribution's."""
    m, h, v, tau0 = 8192, 64, 130, 0.8
    x1 = _randn((1, h), 1.0, 3)
    embed = _randn((v, h), 0.25, 5)
    xh = x1.repeat(m, 1)
    r = np.arange(m)
    ctr = np.stack([r % 256, np.full(m, 2), r // 256], axis=1)
    tau = np.full(m, tau0, dtype=np.float32)
    ent = torch.empty(m, dtype=torch.float32, device=DEV)
    lse = torch.empty_like(ent)
    am = torch.empty(m, dtype=torch.int32, device=DEV)
    smp = torch.empty_like(am)
    dg.op_lmhead_sample(xh.to(DEV), embed.to(DEV),
                        torch.tensor(tau, device=DEV),
                        torch.tensor(ctr, dtype=torch.int32, device=DEV),
                        SEED, ent, lse, am, smp)
    torch.cuda.synchronize()
    z = np32(x1).astype(np.float64) @ np32(embed).astype(np.float64).T
    p = np.exp(z[0] / tau0 - np.max(z[0] / tau0))
    p /= p.sum()
    counts = np.bincount(smp.cpu().numpy(), minlength=v)
    assert counts.sum() == m and counts.size == v
    expect = p * m
    keep = expect >= 5          # pool the thin tail into one cell
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(expect[keep], expect[~keep].sum())
    chi2 = float(np.sum((obs - exp) ** 2 / exp))
    df = len(obs) - 1
    h_ref = float(-np.sum(p * np.log(p)))
    g_ent = ent.cpu().numpy()
    log(f"  chi-square {chi2:.1f} over {df} degrees of freedom; entropy "
        f"{g_ent[0]:.6f} vs {h_ref:.6f}")
    assert chi2 < df + 6 * np.sqrt(2 * df)
    assert np.all(g_ent == g_ent[0])
    assert abs(g_ent[0] - h_ref) < 1e-4 * max(1.0, h_ref)


def test_denoise_step_sampling_wiring():
    """dg_denoise_step with temperature sampling over two canvases, one at
    step 3 of a budget of 16 (tau = 0.9 (1 - 3/16)), the other past the
    budget (tau clamped to 0: the argmax).  Each uncommitted row's
    temperature and counter (position, step, canvas) come from the batch:
    the oracle's sampler on the step's own final-norm rows gives the same
    draws and entropies; against the oracle's whole step the draws are
    reported.  EB fed the draws commits them."""
    wl = synth.WORKLOADS["tiny_l1_h256_p512"]
    shape = wl.shape
    w = synth.make_weights(shape, seed=3, gain_std=0.1)
    wd = to_dev(w)
    eng = dg.Engine(shape, wd, max_requests=2, max_kv_len=1024,
                    max_canvases=2)
    prefix = []
    for rq, p in enumerate((512, 300)):
        k, v = synth.make_prefix_kv(shape, p, rq, seed=3)
        eng.prefill_kv(rq, k.to(DEV).contiguous(), v.to(DEV).contiguous())
        prefix.append((np32(k), np32(v)))
    cv = synth.make_canvas(shape, 2, 150, seed=8)
    steps = np.array([3, 17], dtype=np.int32)
    cv["step"] = torch.tensor(steps)
    tok, com, step = (t.to(DEV).contiguous() for t in
                      (cv["tokens"], cv["committed"], cv["step"]))
    ent, lse, am, _ = step_outputs(2)
    smp = torch.full((2, 256), -1, dtype=torch.int32, device=DEV)
    fx = torch.zeros((2 * 256, shape.hidden), dtype=torch.float32, device=DEV)
    tau0, budget = 0.9, 16
    eng.denoise_step([0, 1], tok, com, step, ent, lse, am,
                     capture={"final_xhat": fx},
                     sampling=(tau0, budget, SEED, smp))
    torch.cuda.synchronize()
    committed = cv["committed"].numpy().reshape(-1)
    rows = np.nonzero(committed == 0)[0]
    canvas = rows // 256
    tau = oracle.temperature(tau0, budget, steps[canvas])
    assert np.all(tau[canvas == 1] == 0.0)
    ctr = np.stack([rows % 256, steps[canvas], canvas], axis=1)
    st = oracle.lm_head_sample(fx.cpu().numpy()[:len(rows)],
                               synth.to_numpy_weights(w)["embed"], tau, ctr,
                               SEED)
    flat = lambda t: t.reshape(-1)[torch.as_tensor(rows, device=DEV)]
    _check_rows("step rows", st, tau, ctr, flat(ent), flat(lse), flat(am),
                flat(smp))
    assert np.all(smp.cpu().numpy().reshape(-1)[committed == 1] == -1)
    # the whole step in the oracle, free-running (reported, decisions can
    # part where bf16 rounding moves a near tie)
    wn = synth.to_numpy_weights(w)
    ref = oracle.denoise_step(oshape(shape), wn, cv["tokens"].numpy(),
                              cv["committed"].numpy(), prefix, mirror=True,
                              sampling=(tau0, budget, SEED), step=steps)
    d = smp.cpu().numpy().reshape(-1)[rows] != ref["sample"].reshape(-1)[rows]
    log(f"  free-running: draws differ from the oracle's step at "
        f"{int(d.sum())} of {len(rows)} rows")
    # EB on the draws: every newly committed position holds its draw
    n_new = torch.zeros(2, dtype=torch.int32, device=DEV)
    done = torch.zeros(2, dtype=torch.uint8, device=DEV)
    gamma = torch.full((2,), 0.5, dtype=torch.float32, device=DEV)
    com0 = com.clone()
    eng.eb_select([0, 1], tok, com, step, ent, smp, gamma, 256, False, n_new,
                  done)
    torch.cuda.synchronize()
    new = (com.cpu().numpy() == 1) & (com0.cpu().numpy() == 0)
    assert new.sum() == int(n_new.sum()) and new.sum() >= 2
    assert np.array_equal(tok.cpu().numpy()[new], smp.cpu().numpy()[new])
    eng.close()



def test_denoise_step_sampling_rejects_bad_parameters():
    """Negative, non-finite or overflowing temperatures and a negative
    budget are refused before any launch (DG_ERR_INVALID_ARG)."""
    shape = synth.WORKLOADS["tiny_l1_h256_p512"].shape
    w = to_dev(synth.make_weights(shape, seed=3))
    eng = dg.Engine(shape, w, max_requests=1, max_kv_len=512, max_canvases=1)
    eng.set_kv_len(0, 0)
    cv = synth.make_canvas(shape, 1, 10, seed=1)
    tok, com, step = (t.to(DEV).contiguous() for t in
                      (cv["tokens"], cv["committed"], cv["step"]))
    ent, lse, am, _ = step_outputs(1)
    smp = torch.full((1, 256), -1, dtype=torch.int32, device=DEV)
    for tau0, budget in ((-0.5, 4), (float("nan"), 4), (float("inf"), 4),
                         (1e-9, 4), (1.0, -1)):
        with pytest.raises(dg.DgError) as e:
            eng.denoise_step([0], tok, com, step, ent, lse, am,
                             sampling=(tau0, budget, SEED, smp))
        assert e.value.status == 1, (tau0, budget)
    torch.cuda.synchronize()
    assert (smp == -1).all() and torch.isnan(ent).all()
    # tau0 = 0 is the greedy draw
    eng.denoise_step([0], tok, com, step, ent, lse, am,
                     sampling=(0.0, 0, SEED, smp))
    torch.cuda.synchronize()
    unc = cv["committed"].to(DEV) == 0
    assert torch.equal(smp[unc], am[unc]) and (ent[unc] == 0).all()
    eng.close()
