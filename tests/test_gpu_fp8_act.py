"""FP8 activations (reading R13: the expert GEMMs take their token rows as
E4M3 codes with one scale per row, W8A8 with the E4M3 experts; write-up
Table 3 and Figure 11 captions, FP8 serving) against the oracle: the row
quantisation bit for bit, the MoE on the streaming and the large-tile
(FP8 MFMA) paths, and a two-layer step in lockstep and composition."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, log, np32, to_dev
from test_gpu_ops import GEMMA, TINY, _moe_case

pytestmark = pytest.mark.gpu


def _w8a8(shape, **kw):
    return synth.ModelShape(**{**shape.__dict__, "expert_dtype": "fp8_e4m3",
                               "act_dtype": "fp8_e4m3", **kw})


@pytest.mark.parametrize("rows,k", [(300, 2048), (77, 768), (5, 128)])
def test_quantize_rows_bit_exact(rows, k):
    g = torch.Generator().manual_seed(rows + k)
    x = torch.randn((rows, k), generator=g)
    x *= torch.exp(torch.randn((rows, 1), generator=g) * 3)   # row scales
    x[0] = 0.0                                                  # zero row
    if rows > 2:
        # a row of exact E4M3 values whose largest is 448: scale 1, exact
        c = torch.randint(0, 0x7F, (k,), generator=g, dtype=torch.uint8)
        c[0] = 0x7E
        x[1] = c.view(torch.float8_e4m3fn).float()
        # a row with ties: midpoints of E4M3 values times the scale
        x[2] = torch.tensor([1.0625, -1.1875, 3 * 2.0 ** -10, 448.0] * (k // 4))
    x = x.to(torch.bfloat16)
    q8 = torch.empty((rows, k), dtype=torch.uint8, device=DEV)
    q16 = torch.empty((rows, k), dtype=torch.bfloat16, device=DEV)
    sc = torch.empty(rows, dtype=torch.float32, device=DEV)
    dg.op_quantize_rows(x.to(DEV), q8, q16, sc)
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_rows_e4m3(np32(x))
    np.testing.assert_array_equal(sc.cpu().numpy(), scale)
    np.testing.assert_array_equal(q8.cpu().numpy(), codes)
    np.testing.assert_array_equal(np32(q16), oracle.decode_e4m3(codes))
    log(f"  quantise {rows} x {k}: codes, values and scales bit for bit")


def test_moe_w8a8_streaming_path():
    _moe_case(_w8a8(TINY), 256, "tiny_w8a8")
    _moe_case(_w8a8(GEMMA), 256, "gemma_w8a8_stream")


def test_moe_w8a8_large_tile_path():
    # above the streaming range E4M3 activations take the 256-row tile
    # kernel with the FP8 MFMA at every size
    _moe_case(_w8a8(GEMMA), 1024, "gemma_w8a8_1024")
    _moe_case(_w8a8(GEMMA), 4096, "gemma_w8a8_4096")
    _moe_case(_w8a8(GEMMA, n_shared_experts=1), 4096, "gemma_w8a8_shared")
    _moe_case(_w8a8(GEMMA), 160, "gemma_w8a8_same", same_rows=True)


def test_denoise_step_w8a8_lockstep_and_composition():
    """Two layers with E4M3 experts and activations: the step against the
    single-op entry points on its own state (composition) and against the
    oracle layer by layer (lockstep), 200 uncommitted positions."""
    from test_gpu_step import _compare_step, _setup
    from workload_common import capture_buffers, check_composition
    shape = _w8a8(synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096))
    log("two layers, W8A8 experts")
    eng, wn, prefix = _setup(shape, [300], 1024, seed=13)
    cv = synth.make_canvas(shape, 1, 200, seed=13)
    tok, com, step = (t.to(DEV) for t in (cv["tokens"], cv["committed"],
                                          cv["step"]))
    from gpu_common import step_outputs
    ent, lse, am, logits = step_outputs(1, shape.vocab)
    cap = capture_buffers(shape, 256, 2, final=False)
    eng.denoise_step([0], tok, com, step, ent, lse, am, logits, cap)
    torch.cuda.synchronize()
    wd = to_dev(synth.make_weights(shape, seed=13, gain_std=0.1))
    check_composition(eng, shape, wd, tok, [0], [300], cap, "w8a8")
    _compare_step(shape, eng, wn, prefix, cv, ent, lse, am, logits, cap, 1,
                  [300])
    eng.close()
