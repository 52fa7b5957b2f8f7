"""The E4M3 LM head (reading R15: the tied table as E4M3 codes with one
scale per vocabulary row, the final-normed rows quantised per row as E4M3;
write-up Table 3 and Figure 11 captions, FP8 serving) against the oracle:
the entry point on both of its paths (streaming at <= 128 rows, the FP8
MFMA tile kernel above), and a two-layer step with W8A8 experts and the
E4M3 head in lockstep, with its head checked bit for bit against the entry
point on the step's own final rows."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, FP8_SUM_BOUND, TOL, lm8_abs_sums,
                        lm8_decision_bound, log, np32, top2_margin)

pytestmark = pytest.mark.gpu


def _randn(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _head_case(m, h, v, seed, tag):
    log(f"E4M3 head {tag}: M={m} H={h} V={v}")
    embed = _randn((v, h), 0.02, seed)
    codes, scale = synth.quantize_e4m3_rows(embed)
    xh = _randn((m, h), 1.0, seed + 1)
    ent = torch.empty(m, dtype=torch.float32, device=DEV)
    lse = torch.empty_like(ent)
    am = torch.empty(m, dtype=torch.int32, device=DEV)
    logits = torch.empty((m, v), dtype=torch.float32, device=DEV)
    dg.op_lmhead_entropy_e4m3(xh.to(DEV), codes.to(DEV), scale.to(DEV), ent,
                              lse, am, logits)
    torch.cuda.synchronize()
    c8, s8 = codes.numpy(), scale.numpy()
    st = oracle.lm_head_stats(np32(xh), None, want_logits=True, lm8=(c8, s8))
    z = st["logits"]
    gz = logits.cpu().numpy().astype(np.float64)
    # every logit within the FP8 sums' bound of the exact one (checked on
    # the rows' largest logits and a seeded sample of the rest)
    rng = np.random.default_rng(seed)
    cols = np.concatenate([np.argsort(-z, axis=1)[:, :4],
                           rng.integers(0, v, (m, 12))], axis=1)
    a = lm8_abs_sums(np32(xh), c8, s8, cols)
    dz = np.abs(np.take_along_axis(gz, cols, 1) - np.take_along_axis(z, cols, 1))
    worst = float(np.max(dz / (FP8_SUM_BOUND * a + 1e-6)))
    e_z = float(np.max(np.abs(gz - z)) / np.max(np.abs(z)))
    e_h = float(np.max(np.abs(ent.cpu().numpy() - st["entropy"])) /
                np.max(np.abs(st["entropy"])))
    e_l = float(np.max(np.abs(lse.cpu().numpy() - st["lse"])) /
                np.max(np.abs(st["lse"])))
    ga = am.cpu().numpy()
    marg = top2_margin(z)
    bound = lm8_decision_bound(np32(xh), z, c8, s8)
    diff = ga != st["argmax"]
    log(f"  logits rel err {e_z:.2e} (worst |dz| / bound {worst:.2f}), entropy "
        f"{e_h:.2e}, lse {e_l:.2e}; argmax differs at {int(diff.sum())} rows "
        f"(margins {np.sort(marg[diff]).tolist()}, bounds "
        f"{np.sort(bound[diff]).tolist()})")
    assert worst <= 1.0
    assert e_z < TOL and e_h < TOL and e_l < TOL
    assert np.all(marg[diff] < bound[diff])
    return ent, lse, am


def test_e4m3_head_streaming_path():
    # <= 128 rows: E4M3 weights widened to bf16 in the streaming kernel
    _head_case(1, 128, 130, 1, "one")
    _head_case(37, 256, 4173, 2, "ragged")
    _head_case(128, 256, 4096, 3, "full pass")


def test_e4m3_head_tile_path():
    # > 128 rows: the 256 x 256 tile kernel on the FP8 MFMA, ragged row tile
    _head_case(200, 256, 3000, 4, "tiles")
    _head_case(129, 384, 4100, 5, "129")


def test_e4m3_head_full_vocab():
    _head_case(64, 2048, 262144, 6, "gemma stream")
    _head_case(300, 2048, 262144, 7, "gemma tiles")


def test_e4m3_head_rejects_unsupported_shapes():
    v, h = 256, 192          # hidden not a multiple of 128
    codes = torch.zeros((v, h), dtype=torch.uint8, device=DEV)
    scale = torch.ones(v, dtype=torch.float32, device=DEV)
    x = torch.zeros((4, h), dtype=torch.bfloat16, device=DEV)
    out = torch.empty(4, dtype=torch.float32, device=DEV)
    am = torch.empty(4, dtype=torch.int32, device=DEV)
    with pytest.raises(dg.DgError) as e:
        dg.op_lmhead_entropy_e4m3(x, codes, scale, out, out.clone(), am)
    assert e.value.status == 2


@pytest.mark.parametrize("uncommitted", [200, 90])
def test_denoise_step_e4m3_head_lockstep(uncommitted):
    """Two layers, W8A8 experts and the E4M3 head: the step against the
    oracle layer by layer (lockstep, the head fed the oracle's final rows)
    and its head against the entry point on the step's own final rows, bit
    for bit (90 rows: the streaming path; 200: the FP8 MFMA tile path)."""
    from test_gpu_step import _compare_step, _setup
    from workload_common import capture_buffers
    from gpu_common import step_outputs
    shape = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096,
                             expert_dtype="fp8_e4m3", act_dtype="fp8_e4m3",
                             lm_dtype="fp8_e4m3")
    log(f"two layers, W8A8 experts, E4M3 head, {uncommitted} uncommitted")
    eng, wn, prefix = _setup(shape, [300], 1024, seed=17)
    cv = synth.make_canvas(shape, 1, uncommitted, seed=17)
    tok, com, step = (t.to(DEV) for t in (cv["tokens"], cv["committed"],
                                          cv["step"]))
    ent, lse, am, logits = step_outputs(1, shape.vocab)
    cap = capture_buffers(shape, 256, 2, final=True)
    eng.denoise_step([0], tok, com, step, ent, lse, am, logits, cap)
    torch.cuda.synchronize()
    rows = np.nonzero(cv["committed"].numpy().reshape(-1) == 0)[0]
    m = len(rows)
    fx = cap["final_xhat"][:m].to(torch.bfloat16)
    o_ent = torch.empty(m, dtype=torch.float32, device=DEV)
    o_lse = torch.empty_like(o_ent)
    o_am = torch.empty(m, dtype=torch.int32, device=DEV)
    dg.op_lmhead_entropy_e4m3(fx.contiguous(), eng.weights["lm_head"],
                              eng.weights["lm_head_scale"], o_ent, o_lse, o_am)
    torch.cuda.synchronize()
    sel = torch.as_tensor(rows, device=DEV)
    assert torch.equal(ent.reshape(-1)[sel], o_ent)
    assert torch.equal(lse.reshape(-1)[sel], o_lse)
    assert torch.equal(am.reshape(-1)[sel], o_am)
    log(f"  the step's head equals the entry point on its {m} rows, bit for bit")
    _compare_step(shape, eng, wn, prefix, cv, ent, lse, am, logits, cap, 1,
                  [300])
    eng.close()
