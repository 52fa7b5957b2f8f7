"""W8A8 Q/K/V and output projections (reading R16: E4M3 weight rows with
per-row scales, the input rows quantised per row as E4M3; write-up Table 3
and Figure 11 captions, FP8 serving) against the oracle: the entry point on
the 64 x 64 tile kernel (the codes' bf16 values) and on the FP8 MFMA tile
kernel (from 1024 rows), every mode; then a two-layer model in FP8
throughout (projections, experts and their rows, the LM head) through a
denoise step in lockstep, a commit and AR steps."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, FP8_SUM_BOUND, log, np32

pytestmark = pytest.mark.gpu

ALL8 = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096,
                        expert_dtype="fp8_e4m3", act_dtype="fp8_e4m3",
                        lm_dtype="fp8_e4m3", proj_dtype="fp8_e4m3")


def _randn(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


@pytest.mark.parametrize("m,k,n,mode", [
    (256, 2048, 4096, 0),     # Q/K/V at one canvas: 64 x 64 tiles
    (77, 256, 192, 2),        # few rows, ragged: 32 x 64 tiles, residual add
    (300, 128, 64, 1),        # fp32 store
    (1024, 2048, 2048, 2),    # FP8 MFMA tile kernel, residual add
    (1100, 256, 320, 0),      # FP8 MFMA, ragged rows and columns
])
def test_linear_e4m3_against_oracle(m, k, n, mode):
    log(f"W8A8 projection M={m} K={k} N={n} mode {mode}")
    seed = m + k + n + mode
    w = _randn((n, k), 0.02, seed)
    codes, scale = synth.quantize_e4m3_rows(w)
    x = _randn((m, k), 1.0, seed + 1)
    dt = torch.bfloat16 if mode == 0 else torch.float32
    base = _randn((m, n), 1.0, seed + 2).float() if mode == 2 else \
        torch.zeros((m, n))
    out = base.to(DEV).to(dt).contiguous()
    dg.op_linear_e4m3(x.to(DEV), codes.to(DEV), scale.to(DEV), out, mode)
    torch.cuda.synchronize()
    c8, s8 = codes.numpy(), scale.numpy()
    y = oracle.linear_w8a8(np32(x), c8, s8)
    got = np32(out).astype(np.float64) - (np32(base) if mode == 2 else 0.0)
    # the FP8 sums' bound (FP8 MFMA; the 64 x 64 tiles sum exact products
    # in fp32, well within), plus the bf16 rounding of the stored value
    qx, sx = oracle.quantize_rows_e4m3(np32(x))
    a = (np.abs(oracle.decode_e4m3(qx)) * sx[:, None]) @ \
        (np.abs(oracle.decode_e4m3(c8)) * s8[:, None]).T
    tol = FP8_SUM_BOUND * a + (2.0 ** -8 if mode == 0 else 2.0 ** -22) * np.abs(y)
    if mode == 2:
        tol += 2.0 ** -23 * np.abs(np32(out))   # the fp32 addition
    worst = float(np.max(np.abs(got - y) / (tol + 1e-30)))
    rel = float(np.max(np.abs(got - y)) / np.max(np.abs(y)))
    log(f"  rel err {rel:.2e}; worst |d| / bound {worst:.2f}")
    assert worst <= 1.0


def test_linear_e4m3_rejects_unsupported_shapes():
    codes = torch.zeros((64, 192), dtype=torch.uint8, device=DEV)
    scale = torch.ones(64, dtype=torch.float32, device=DEV)
    x = torch.zeros((4, 192), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dg.DgError) as e:
        dg.op_linear_e4m3(x, codes, scale, out, 0)
    assert e.value.status == 2


@pytest.mark.parametrize("uncommitted", [200, 60])
def test_denoise_step_all_fp8_lockstep(uncommitted):
    """Two layers in FP8 throughout: the step against the oracle layer by
    layer (lockstep: every op fed the oracle's values), the head and EB."""
    from test_gpu_step import _compare_step, _setup
    from workload_common import capture_buffers
    from gpu_common import step_outputs
    log(f"two layers, FP8 throughout, {uncommitted} uncommitted")
    eng, wn, prefix = _setup(ALL8, [300], 1024, seed=23)
    cv = synth.make_canvas(ALL8, 1, uncommitted, seed=23)
    tok, com, step = (t.to(DEV) for t in (cv["tokens"], cv["committed"],
                                          cv["step"]))
    ent, lse, am, logits = step_outputs(1, ALL8.vocab)
    cap = capture_buffers(ALL8, 256, 2, final=False)
    eng.denoise_step([0], tok, com, step, ent, lse, am, logits, cap)
    torch.cuda.synchronize()
    _compare_step(ALL8, eng, wn, prefix, cv, ent, lse, am, logits, cap, 1,
                  [300])
    eng.close()


def test_commit_all_fp8_lockstep():
    from test_gpu_step import commit_case
    commit_case(ALL8, "two layers, FP8 throughout")


def test_ar_all_fp8_lockstep():
    """AR steps of the FP8 model in lockstep: the device's dg_ar_step runs,
    then its single ops are fed the oracle's values of each layer (a canvas
    of one position in the commit pass, the appended K/V compared), and the
    final norm and E4M3 head the oracle's final rows.  (A free-running
    chain of W8A8 layers quantises slightly different rows on the two
    sides, and one-step code differences compound from layer to layer; the
    lockstep bounds each step.)  Both sides continue from the device's
    cache and the oracle's greedy token."""
    from lockstep import Lockstep
    from gpu_common import lm8_decision_bound, oshape, rel_err, top2_margin, TOL
    from test_gpu_ar import _setup
    log("AR lockstep, two layers, FP8 throughout")
    eng, wn, caches = _setup(ALL8, [300, 77])
    rng = np.random.default_rng(6)
    tok = rng.integers(0, ALL8.vocab, 2)
    req = [0, 1]
    for step in range(3):
        plen = [eng.kv_len(r) for r in req]
        ent = torch.full((2,), float("nan"), device=DEV)
        lse = torch.full_like(ent, float("nan"))
        am = torch.full((2,), -1, dtype=torch.int32, device=DEV)
        eng.ar_step(req, torch.tensor(tok, dtype=torch.int32, device=DEV),
                    ent, lse, am)
        torch.cuda.synchronize()
        cap_o = []
        ref = oracle.ar_step(oshape(ALL8), wn, np.asarray(tok),
                             [tuple(caches[r]) for r in req], mirror=True,
                             request=req, want_logits=True, capture=cap_o)
        kv_o = [(np.concatenate([ref["kv"][b][0][li] for b in range(2)], axis=1),
                 np.concatenate([ref["kv"][b][1][li] for b in range(2)], axis=1))
                for li in range(ALL8.n_layers)]
        ls = Lockstep(ALL8, eng, eng.weights, 2, req, plen, [0, 1], cap_o,
                      f"AR step {step}", causal=True, kv_o=kv_o, C=1)
        assert ls.finish() == ALL8.n_layers
        ls.report()
        # final norm and the E4M3 head on the oracle's rows
        xf = torch.empty((2, ALL8.hidden), dtype=torch.bfloat16, device=DEV)
        dg.op_rmsnorm(torch.as_tensor(ls.x_last, dtype=torch.float32, device=DEV),
                      eng.weights["final_norm"], ALL8.rms_eps, xf)
        e_n = rel_err(np32(xf), ref["final_xhat"])
        xo = torch.as_tensor(ref["final_xhat"], dtype=torch.float32,
                             device=DEV).to(torch.bfloat16)
        h_ent = torch.empty(2, dtype=torch.float32, device=DEV)
        h_lse = torch.empty_like(h_ent)
        h_am = torch.empty(2, dtype=torch.int32, device=DEV)
        dg.op_lmhead_entropy_e4m3(xo, eng.weights["lm_head"],
                                  eng.weights["lm_head_scale"], h_ent, h_lse, h_am)
        torch.cuda.synchronize()
        e_h = rel_err(h_ent.cpu().numpy(), ref["entropy"])
        e_l = rel_err(h_lse.cpu().numpy(), ref["lse"])
        d = h_am.cpu().numpy() != ref["argmax"]
        bound = lm8_decision_bound(ref["final_xhat"], ref["logits"],
                                   wn["lm_head"], wn["lm_head_scale"])
        marg = top2_margin(ref["logits"])
        log(f"  AR step {step} head: final norm {e_n:.2e}, entropy {e_h:.2e}, "
            f"lse {e_l:.2e}, argmax differences {int(d.sum())}; the step's own "
            f"argmax equals the oracle's at {int((am.cpu().numpy() == ref['argmax']).sum())} of 2")
        assert e_n < TOL and e_h < TOL and e_l < TOL
        assert np.all(marg[d] < bound[d])
        # both sides continue from the device's cache
        for b, r in enumerate(req):
            for which, i in (("k", 0), ("v", 1)):
                got = eng.cache_view(which)[:, r, :, plen[b]:plen[b] + 1, :]
                caches[r][i] = np.concatenate(
                    [caches[r][i], got.float().cpu().numpy().astype(np.float64)],
                    axis=2)
        tok = ref["argmax"]
    eng.close()
