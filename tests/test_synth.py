"""Host checks of the seeded input generators (no GPU)."""
import torch

from block_discrete_diffusion_tok_amd import synth


def test_float32_masters_round_to_the_default_weights():
    sh = synth.WORKLOADS["tiny_l1_h256_p512"].shape
    a = synth.make_weights(sh, seed=0)
    b = synth.make_weights(sh, seed=0, masters=True)
    assert b["embed"].dtype == torch.float32
    assert torch.equal(a["embed"], b["embed"].to(torch.bfloat16))
    for k in ("w_qkv", "w_o", "w_router", "w_gate_up", "w_down"):
        assert b["layers"][0][k].dtype == torch.float32, k
        assert torch.equal(a["layers"][0][k],
                           b["layers"][0][k].to(torch.bfloat16)), k
    assert torch.equal(a["final_norm"], b["final_norm"])


def test_generators_are_seeded_per_name():
    sh = synth.WORKLOADS["tiny_l1_h256_p512"].shape
    a = synth.make_weights(sh, seed=1)
    b = synth.make_weights(sh, seed=1)
    c = synth.make_weights(sh, seed=2)
    assert torch.equal(a["layers"][0]["w_qkv"], b["layers"][0]["w_qkv"])
    assert not torch.equal(a["layers"][0]["w_qkv"], c["layers"][0]["w_qkv"])
    assert not torch.equal(a["layers"][0]["w_qkv"][:64, :64],
                           a["layers"][0]["w_o"][:64, :64])
