"""The library's debugging aids, each in a child process (they are read once
per process from the environment):
  DG_POISON=1 fills the workspace's value regions with NaN before every
    engine call that runs layers: a prefill from tokens, a denoise step, a
    commit and an AR step return the same outputs and caches bit for bit as
    without it, for a bf16 model and for the E4M3 variants (W8A8 experts
    and projections, E4M3 cache, E4M3 LM head), so no kernel reads scratch
    its call did not write;
  DG_CHECK=1 makes a commit of a canvas with uncommitted positions fail
    with DG_ERR_STATE;
  DG_KV_SPLIT=s changes only the attention's summation order."""
import os
import subprocess
import sys
import tempfile

import pytest
import torch

from gpu_common import TOL, rel_err

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# The child: a two-layer model (bf16, or E4M3 experts and projections with
# E4M3 token rows, an E4M3 cache and an E4M3 LM head) with two requests, one prefilled from K/V and one from
# tokens; a denoise step over a canvas of each, their commit, an AR step.
_CHILD = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
from block_discrete_diffusion_tok_amd import dg, synth
fp8 = sys.argv[3] == "fp8"
kw = dict(expert_dtype="fp8_e4m3", act_dtype="fp8_e4m3", kv_dtype="fp8_e4m3",
          lm_dtype="fp8_e4m3", proj_dtype="fp8_e4m3") if fp8 else {}
shape = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096, **kw)
w = synth.make_weights(shape, seed=31, gain_std=0.1, device="cuda")
eng = dg.Engine(shape, w, max_requests=2, max_kv_len=1024, max_canvases=2)
k, v = synth.make_prefix_kv(shape, 300, 0, seed=31, device="cuda")
eng.prefill_kv(0, k.contiguous(), v.contiguous())
g = torch.Generator().manual_seed(32)
prompt = torch.randint(0, shape.vocab, (77,), generator=g, dtype=torch.int32)
eng.prefill_tokens(1, prompt.cuda())
cv = synth.make_canvas(shape, 2, 200, seed=33)
t = {kk: x.cuda().contiguous() for kk, x in cv.items()}
ent = torch.full((2, 256), float("nan"), device="cuda")
lse = torch.full_like(ent, float("nan"))
am = torch.full((2, 256), -1, dtype=torch.int32, device="cuda")
eng.denoise_step([0, 1], t["tokens"], t["committed"], t["step"], ent, lse, am)
eng.commit_block([0, 1], t["tokens"], t["committed"], t["step"])
a_ent = torch.full((2,), float("nan"), device="cuda")
a_lse = torch.full_like(a_ent, float("nan"))
a_am = torch.full((2,), -1, dtype=torch.int32, device="cuda")
eng.ar_step([0, 1], torch.tensor([5, 4000], dtype=torch.int32, device="cuda"),
            a_ent, a_lse, a_am)
torch.cuda.synchronize()
out = {"ent": ent, "lse": lse, "am": am, "a_ent": a_ent, "a_lse": a_lse,
       "a_am": a_am, "kc": eng.cache_view("k"), "vc": eng.cache_view("v")}
# bytes of the workspace left at 0xFF (the poison where no kernel wrote)
ff = int((eng.workspace == 0xFF).sum())
if fp8:
    out["ks"] = eng.scale_view("k")
    out["vs"] = eng.scale_view("v")
res = {kk: x.cpu() for kk, x in out.items()}
res["ff"] = torch.tensor(ff)
torch.save(res, sys.argv[2])
eng.close()
'''


def _run(env_extra, *args):
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "out.pt")
        env = {**os.environ, **env_extra}
        r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, path, *args],
                           env=env, capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, r.stderr[-3000:]
        return torch.load(path, weights_only=True)


@pytest.mark.parametrize("variant", ["bf16", "fp8"])
def test_poison_mode_gives_the_same_outputs(variant):
    print(f"DG_POISON, {variant} model", flush=True)
    off = _run({"DG_POISON": "0"}, variant)
    on = _run({"DG_POISON": "1"}, variant)
    # the poison was laid (the last call's unwritten value bytes keep it)
    ff_on, ff_off = int(on.pop("ff")), int(off.pop("ff"))
    print(f"  workspace bytes at 0xFF: {ff_on} poisoned, {ff_off} not", flush=True)
    assert ff_on > (1 << 20) and ff_on > 2 * ff_off
    for k in off:
        # committed rows keep the NaN the outputs were filled with
        torch.testing.assert_close(on[k], off[k], rtol=0, atol=0, equal_nan=True,
                                   msg=k)
    # the uncommitted positions' statistics are finite (no NaN leaked in)
    assert torch.isfinite(on["ent"]).sum() == 2 * 200
    assert torch.isfinite(on["a_ent"]).all() and torch.isfinite(on["a_lse"]).all()


def test_kv_split_override_changes_only_the_summation_order():
    print("DG_KV_SPLIT=3", flush=True)
    auto = _run({}, "bf16")
    split = _run({"DG_KV_SPLIT": "3"}, "bf16")
    auto.pop("ff"), split.pop("ff")
    # (a different rounding of the attention output can flip a near-tied
    # routing decision of the next layer: the usual continuous bound)
    fin = torch.isfinite(auto["ent"])
    assert torch.equal(fin, torch.isfinite(split["ent"]))
    for k in ("ent", "lse", "a_ent", "a_lse"):
        a = auto[k][torch.isfinite(auto[k])].numpy()
        b = split[k][torch.isfinite(auto[k])].numpy()
        assert rel_err(b, a) < TOL, k
    # layer 0's cached rows come before any attention: the same bits
    assert torch.equal(split["kc"][0], auto["kc"][0])
    assert torch.equal(split["vc"][0], auto["vc"][0])


_CHECK_CHILD = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
from block_discrete_diffusion_tok_amd import dg, synth
shape = synth.WORKLOADS["tiny_l1_h256_p512"].shape
w = synth.make_weights(shape, seed=0, device="cuda")
eng = dg.Engine(shape, w, max_requests=1, max_kv_len=1024, max_canvases=1)
eng.set_kv_len(0, 0)
cv = synth.make_canvas(shape, 1, 3, seed=5)
t = {kk: x.cuda().contiguous() for kk, x in cv.items()}
try:
    eng.commit_block([0], t["tokens"], t["committed"], t["step"])
    print("unfinished: ok", eng.kv_len(0))
except dg.DgError as e:
    print("unfinished: status", e.status, eng.kv_len(0))
t["committed"].fill_(1)
eng.commit_block([0], t["tokens"], t["committed"], t["step"])
torch.cuda.synchronize()
print("finished: ok", eng.kv_len(0))
eng.close()
'''


def test_check_mode_refuses_a_commit_of_an_unfinished_canvas():
    print("DG_CHECK", flush=True)
    outs = {}
    for flag in ("1", "0"):
        r = subprocess.run([sys.executable, "-c", _CHECK_CHILD, ROOT],
                           env={**os.environ, "DG_CHECK": flag},
                           capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, r.stderr[-3000:]
        outs[flag] = r.stdout.split("\n")
    # DG_ERR_STATE = 4; the refused commit leaves kv_len alone
    assert "unfinished: status 4 0" in outs["1"]
    assert "finished: ok 256" in outs["1"]
    assert "unfinished: ok 256" in outs["0"]
    assert "finished: ok 512" in outs["0"]
