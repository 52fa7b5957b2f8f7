"""The allocation-free LM-head entry point (dg_op_lmhead_entropy_static)
against the workspace entry point (dg_op_lmhead_entropy) through the C ABI:
two calls in a row, the second with fewer rows, equal bit for bit (same
kernels, same partials); and the size limit rejected on the host."""
import pytest
import torch

from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, log

pytestmark = pytest.mark.gpu


def _outs(m):
    return (torch.full((m,), float("nan"), device=DEV),
            torch.full((m,), float("nan"), device=DEV),
            torch.full((m,), -1, dtype=torch.int32, device=DEV))


def test_static_scratch_lmhead_matches_workspace_entry_point():
    V, H = 262144, 2048
    embed = synth.normal((V, H), 0.02, 7, "embed", DEV)
    packed = dg.pack(embed)
    del embed
    for m in (200, 37):          # the second call smaller than the first
        x = synth.normal((m, H), 1.0, m, "xhat", DEV)
        ent_s, lse_s, am_s = _outs(m)
        dg.op_lmhead_entropy_static(x, packed, ent_s, lse_s, am_s)
        ent_w, lse_w, am_w = _outs(m)
        dg.op_lmhead_entropy(x, packed, ent_w, lse_w, am_w)
        torch.cuda.synchronize()
        log(f"  static scratch, {m} rows: entropy max |diff| "
            f"{(ent_s - ent_w).abs().max().item():.1e}")
        assert torch.equal(ent_s, ent_w)
        assert torch.equal(lse_s, lse_w)
        assert torch.equal(am_s, am_w)


def test_static_scratch_lmhead_rejects_sizes_beyond_the_array():
    V, H = 262144, 64
    embed = synth.normal((V, H), 0.02, 7, "embed_small", DEV)
    packed = dg.pack(embed)
    m = 513      # 513 * 2048 tiles * 16 B > 16 MiB
    x = torch.zeros((m, H), dtype=torch.bfloat16, device=DEV)
    ent, lse, am = _outs(m)
    with pytest.raises(dg.DgError) as ei:
        dg.op_lmhead_entropy_static(x, packed, ent, lse, am)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert torch.isnan(ent).all()
