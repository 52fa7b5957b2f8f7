"""The step under HIP-graph capture (dg_set_stream): dg_denoise_step and
dg_eb_select captured on a side stream into a graph (torch's CUDA graph,
a HIP graph on ROCm) and replayed, one step and two steps in a row, with
eager work and synchronisations between the replays; every replay equals
the eager steps bit for bit (statistics, canvas state, EB outputs).  Also
for the W8A8 model with the E4M3 head (row quantisation inside the graph)."""
import pytest
import torch

from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, log, to_dev

pytestmark = pytest.mark.gpu

TWO = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096)
ALL8 = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096,
                        expert_dtype="fp8_e4m3", act_dtype="fp8_e4m3",
                        lm_dtype="fp8_e4m3", proj_dtype="fp8_e4m3")


@pytest.mark.parametrize("shape,tag", [(TWO, "bf16"), (ALL8, "W8A8")])
def test_step_replayed_from_a_hip_graph_equals_the_eager_step(shape, tag):
    log(f"HIP graph of denoise + EB, two layers, {tag}")
    w = synth.make_weights(shape, seed=41, gain_std=0.1)
    eng = dg.Engine(shape, to_dev(w), max_requests=2, max_kv_len=1024,
                    max_canvases=2)
    for r, p in enumerate((300, 77)):
        k, v = synth.make_prefix_kv(shape, p, r, seed=41)
        eng.prefill_kv(r, k.to(DEV).contiguous(), v.to(DEV).contiguous())
    cv = synth.make_canvas(shape, 2, 180, seed=42)
    init = {k: t.to(DEV).contiguous() for k, t in cv.items()}
    st = {k: t.clone() for k, t in init.items()}
    ent = torch.zeros((2, 256), device=DEV)
    lse = torch.zeros_like(ent)
    am = torch.zeros((2, 256), dtype=torch.int32, device=DEV)
    gamma = torch.full((2,), 0.5, device=DEV)
    n_new = torch.zeros(2, dtype=torch.int32, device=DEV)
    done = torch.zeros(2, dtype=torch.uint8, device=DEV)
    outs = (ent, lse, am, st["tokens"], st["committed"], st["step"], n_new, done)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    eng.set_stream(s)

    def step():
        eng.denoise_step([0, 1], st["tokens"], st["committed"], st["step"],
                         ent, lse, am)
        eng.eb_select([0, 1], st["tokens"], st["committed"], st["step"], ent,
                      am, gamma, 64, True, n_new, done)

    def restore():
        for kk in st:
            st[kk].copy_(init[kk])
        for t in (ent, lse, am, n_new, done):
            t.zero_()

    # eager: two consecutive steps from the initial state (also the warm-up
    # on the capture stream)
    ref = []
    with torch.cuda.stream(s):
        restore()
        for _ in range(2):
            step()
            ref.append([t.clone() for t in outs])
    torch.cuda.synchronize()
    assert int(ref[0][6].sum()) >= 2          # the step commits something

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        with torch.cuda.stream(s):
            restore()
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref[0]):
            assert torch.equal(a, b), f"replay {rep}"
        # eager work between replays
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        del junk
    # two replays in a row: the second step of the eager run
    with torch.cuda.stream(s):
        restore()
        g.replay()
        g.replay()
    torch.cuda.synchronize()
    for a, b in zip(outs, ref[1]):
        assert torch.equal(a, b), "second replay in a row"
    log(f"  {tag}: 3 single replays and a double replay equal the eager steps "
        f"bit for bit")
    eng.set_stream(None)
    del g
    eng.close()
