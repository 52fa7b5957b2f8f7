"""The E4M3 KV cache (reading R14: every cached key / value row stored as
E4M3 codes with one scale, read as bf16(code value x scale); write-up Table
3 caption, FP8 serving) against the oracle: rows appended and installed
bit for bit, attention over an E4M3 prefix, and steps of a two-layer model
(prefill, denoise step, commit, AR step) in lockstep and composition."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, TOL, log, np32, rel_err, step_outputs, to_dev

pytestmark = pytest.mark.gpu


def _randn(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _cache(max_req, Hkv, S, D):
    codes = torch.zeros((max_req, Hkv, S, D), dtype=torch.uint8, device=DEV)
    scale = torch.zeros((max_req, Hkv, S), dtype=torch.float32, device=DEV)
    return codes, scale


@pytest.mark.parametrize("D", [128, 64])
def test_kv_append_quantises_rows_bit_exact(D):
    n, C, Hq, Hkv, S = 2, 256, 4, 2, 1024
    qkv = _randn((n * C, (Hq + 2 * Hkv) * D), 1.0, D)
    qkv[3, Hq * D:] = 0.0                       # a zero K row and V row
    kc, ks = _cache(3, Hkv, S, D)
    vc, vs = _cache(3, Hkv, S, D)
    dg.op_kv_append(qkv.to(DEV), n, C, Hq, Hkv, D, kc, vc, 3, S, [2, 0],
                    [300, 512], ks, vs)
    torch.cuda.synchronize()
    q = np32(qkv)
    for b, (r, row0) in enumerate(((2, 300), (0, 512))):
        rows = q[b * C:(b + 1) * C]
        for which, col, codes, scale in (("K", Hq * D, kc, ks),
                                         ("V", (Hq + Hkv) * D, vc, vs)):
            src = rows[:, col:col + Hkv * D].reshape(C, Hkv, D).transpose(1, 0, 2)
            o_codes, o_scale = oracle.quantize_rows_e4m3(src.reshape(-1, D))
            np.testing.assert_array_equal(
                codes[r, :, row0:row0 + C].cpu().numpy().reshape(-1, D), o_codes)
            np.testing.assert_array_equal(
                scale[r, :, row0:row0 + C].cpu().numpy().reshape(-1), o_scale)
    # rows outside the appended ranges are untouched
    assert int(kc[1].abs().sum()) == 0 and int(kc[2, :, :300].sum()) == 0
    log(f"  kv append D={D}: E4M3 codes and scales bit for bit")


@pytest.mark.parametrize("P,causal,splits", [(2048, False, 0), (77, True, 3),
                                             (0, False, 0)])
def test_attention_over_an_e4m3_prefix(P, causal, splits):
    """A prefix installed into an E4M3 cache by the KV append (from bf16
    rows), then canvas attention over it; the oracle reads the same rows
    through reading R14 from the same bf16 values."""
    n, C, Hq, Hkv, D, S = 1, 256, 16, 8, 128, 4096
    log(f"attention over an E4M3 prefix P={P} causal={causal} splits={splits}")
    kp = _randn((Hkv, max(P, 1), D), 1.0, 11 + P)
    vp = _randn((Hkv, max(P, 1), D), 1.0, 13 + P)
    kc, ks = _cache(1, Hkv, S, D)
    vc, vs = _cache(1, Hkv, S, D)
    # the prefix goes in through the append path, 256 rows at a time
    for off in range(0, P, C):
        rows = min(C, P - off)
        qkv = torch.zeros((C, (Hq + 2 * Hkv) * D), dtype=torch.bfloat16)
        qkv[:rows, Hq * D:(Hq + Hkv) * D] = kp[:, off:off + rows].transpose(0, 1).reshape(rows, -1)
        qkv[:rows, (Hq + Hkv) * D:] = vp[:, off:off + rows].transpose(0, 1).reshape(rows, -1)
        dg.op_kv_append(qkv.to(DEV), 1, rows, Hq, Hkv, D, kc, vc, 1, S, [0],
                        [off], ks, vs)
    qkv = _randn((C, (Hq + 2 * Hkv) * D), 1.0, 17 + P)
    out = torch.zeros((C, Hq * D), dtype=torch.bfloat16, device=DEV)
    dg.op_canvas_attention(qkv.to(DEV), n, C, Hq, Hkv, D, kc, vc, 1, S, [0],
                           [P], causal, splits, out, ks, vs)
    torch.cuda.synchronize()
    q_all = np32(qkv)
    q = q_all[:, :Hq * D].reshape(C, Hq, D).transpose(1, 0, 2)
    kcan = q_all[:, Hq * D:(Hq + Hkv) * D].reshape(C, Hkv, D).transpose(1, 0, 2)
    vcan = q_all[:, (Hq + Hkv) * D:].reshape(C, Hkv, D).transpose(1, 0, 2)
    k_pre = oracle.kv_cache_values(np32(kp)[:, :P])
    v_pre = oracle.kv_cache_values(np32(vp)[:, :P])
    ref = oracle.canvas_attention(q, k_pre, v_pre, kcan, vcan, causal=causal)
    ref = ref.transpose(1, 0, 2).reshape(C, Hq * D)
    got = np32(out)
    worst = max(rel_err(got[:, h * D:(h + 1) * D], ref[:, h * D:(h + 1) * D])
                for h in range(Hq))
    # and how far the E4M3 prefix moves the result from the bf16 one
    ref16 = oracle.canvas_attention(q, np32(kp)[:, :P], np32(vp)[:, :P], kcan,
                                    vcan, causal=causal)
    ref16 = ref16.transpose(1, 0, 2).reshape(C, Hq * D)
    log(f"  worst per-head rel err {worst:.2e} (E4M3 against bf16 prefix: "
        f"{rel_err(ref, ref16):.2e})")
    assert worst < TOL


def _kv8_shape():
    return synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096,
                            kv_dtype="fp8_e4m3")


def test_two_layer_steps_with_an_e4m3_cache():
    """Install a 300-token prefix and a token-mode 77-token prompt into an
    E4M3 cache; a denoise step over both requests against the oracle in
    lockstep and composition; the commit in composition (codes bit for
    bit); an AR step against the oracle."""
    from lockstep import Lockstep, lockstep_eb, lockstep_head
    from workload_common import (capture_buffers, check_commit_composition,
                                 check_composition)
    from gpu_common import oshape
    shape = _kv8_shape()
    log("two layers, E4M3 KV cache")
    w = synth.make_weights(shape, seed=21, gain_std=0.1)
    wd = to_dev(w)
    eng = dg.Engine(shape, wd, max_requests=2, max_kv_len=1024, max_canvases=2)
    k, v = synth.make_prefix_kv(shape, 300, 0, seed=21)
    eng.prefill_kv(0, k.to(DEV).contiguous(), v.to(DEV).contiguous())
    # request 1: token-mode prefill; its oracle prefix is the oracle's own
    # causal encode of the prompt (bf16 rows; the oracle quantises them on
    # read, as the cache quantised them on the way in)
    g = torch.Generator().manual_seed(22)
    prompt = torch.randint(0, shape.vocab, (77,), generator=g, dtype=torch.int32)
    eng.prefill_tokens(1, prompt.to(DEV))
    wn = synth.to_numpy_weights(w)
    osh = oshape(shape)
    enc = oracle.commit_block(osh, wn, prompt.numpy()[None], [
        (np.zeros((2, 2, 0, 64)), np.zeros((2, 2, 0, 64)))], mirror=True)
    prefix = [(np32(k), np32(v)), enc[0]]
    # the prompt's cached rows: the oracle's rows quantised equal the cache
    kc8, ks8 = eng.cache_view("k"), eng.scale_view("k")
    codes, scale = oracle.quantize_rows_e4m3(
        oracle.round_bf16(enc[0][0][0].reshape(-1, 64)))
    same = np.mean(kc8[0, 1, :, :77].cpu().numpy().reshape(-1, 64) == codes)
    log(f"  token prefill: {same:.4f} of layer-0 K codes equal the oracle's")
    assert same > 0.99
    cv = synth.make_canvas(shape, 2, 200, seed=21)
    tok, com, step = (t.to(DEV).contiguous() for t in
                      (cv["tokens"], cv["committed"], cv["step"]))
    ent, lse, am, _ = step_outputs(2)
    cap = capture_buffers(shape, 512, 2, final=False)
    eng.denoise_step([0, 1], tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    check_composition(eng, shape, wd, tok, [0, 1], [300, 77], cap, "kv8")
    cap_o = []
    ref = oracle.denoise_step(osh, wn, cv["tokens"].numpy(),
                              cv["committed"].numpy(), prefix, mirror=True,
                              want_logits=True, capture=cap_o)
    ls = Lockstep(shape, eng, eng.weights, 2, [0, 1], [300, 77], [0, 1],
                  cap_o, "kv8")
    assert ls.finish() == shape.n_layers
    ls.report()
    lockstep_head(shape, eng, eng.weights, ref, ls.x_last,
                  cv["committed"].numpy(), 2, [0, 1], "kv8")
    lockstep_eb(ref["entropy"], ref["argmax"], cv["committed"].numpy(),
                cv["tokens"].numpy(), cv["step"].numpy(), 0.5, 256, "kv8")
    # commit both canvases: codes and scales of the ops' K / V bit for bit
    eng.commit_block([0, 1], tok, com, step)
    torch.cuda.synchronize()
    assert eng.kv_len(0) == 556 and eng.kv_len(1) == 333
    check_commit_composition(eng, shape, wd, tok, [0, 1], [300, 77], "kv8")
    eng.close()


def test_thirty_layer_stack_with_an_e4m3_cache():
    """The 30-layer stack (hidden 2048, 16/8 heads of 128, 128 experts, the
    262144-token vocabulary) with its 4096-token prefix in an E4M3 cache: a
    denoise step of an all-masked canvas in composition and in lockstep
    through all 30 layers, the LM head and EB.  Checks the per-layer cache
    and scale offsets at the model's full depth."""
    from lockstep import Lockstep, lockstep_eb, lockstep_head
    from workload_common import (HostPerLayer, capture_buffers,
                                 check_composition, host_model)
    from gpu_common import new_canvas_tensors, oshape
    import dataclasses
    wl = synth.WORKLOADS["stack30_h2048_p4096"]
    shape = dataclasses.replace(wl.shape, kv_dtype="fp8_e4m3")
    P = wl.prefix_len
    log("30 layers, E4M3 cache, 4096-token prefix")
    w = synth.make_weights(shape, seed=0, device=DEV)
    eng = dg.Engine(shape, w, max_requests=1, max_kv_len=P + 256, max_canvases=1)
    k, v = synth.make_prefix_kv(shape, P, 0, seed=0, device=DEV)
    eng.prefill_kv(0, k.contiguous(), v.contiguous())
    cv = synth.make_canvas(shape, 1, 256, seed=7)
    tok, com, step = new_canvas_tensors(cv)
    ent, lse, am, _ = step_outputs(1)
    cap = capture_buffers(shape, 256, shape.n_layers)
    eng.denoise_step([0], tok, com, step, ent, lse, am, None, cap)
    torch.cuda.synchronize()
    check_composition(eng, shape, w, tok, [0], [P], cap, "kv8-30")
    del cap
    cap_o = []
    ls = Lockstep(shape, eng, w, 1, [0], [P], [0], cap_o, "kv8-30")
    ref = oracle.denoise_step(oshape(shape), host_model(w, stop=ls),
                              cv["tokens"].numpy(), cv["committed"].numpy(),
                              [(HostPerLayer(k), HostPerLayer(v))],
                              mirror=True, want_logits=True, capture=cap_o)
    assert ls.finish() == shape.n_layers
    ls.report()
    lockstep_head(shape, eng, w, ref, ls.x_last, cv["committed"].numpy(), 1,
                  [0], "kv8-30")
    lockstep_eb(ref["entropy"], ref["argmax"], cv["committed"].numpy(),
                cv["tokens"].numpy(), cv["step"].numpy(), wl.gamma, 64, "kv8-30")
    eng.close()
