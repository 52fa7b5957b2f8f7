"""Op-level parity: each libdg op (through the C ABI) against the CPU oracle on
seeded inputs, element by element; full-size shapes of the one-layer
2048-hidden / 262k-vocab workload included."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, MARGIN, TOL, TOL_ROW_FP8_ACT, fp8_act, log,
                        np32, oshape, rel_err, routing_margin, row_err, to_dev,
                        top2_margin)

pytestmark = pytest.mark.gpu

GEMMA = synth.WORKLOADS["moe_layer_h2048_v262k_p2048"].shape
TINY = synth.WORKLOADS["tiny_l1_h256_p512"].shape


def _randn(shape, std, name, dtype=torch.bfloat16, seed=7):
    return synth.normal(shape, std, seed, name, "cpu", dtype)


# ------------------------------------------------------------------ linear

# Projection shapes of one 2048-hidden layer (Q/K/V, output, router) at 256
# rows (32 x 64 tiles), plus ragged rows/columns (90 columns: scalar
# stores), K not a multiple of the 4-step pipeline (K = 448, 320), and
# products over >= 1024 rows on the 256 x 256 tiles (a ragged last row tile,
# N not a multiple of 256, K = 448).
@pytest.mark.parametrize("m,k,n", [(300, 256, 200), (1, 128, 64),
                                   (256, 2048, 4096), (256, 2048, 2048),
                                   (256, 2048, 128), (200, 448, 96),
                                   (200, 320, 90), (4096, 256, 512),
                                   (1100, 2048, 4096), (2048, 448, 320)])
def test_linear_three_modes(m, k, n):
    log(f"linear m={m} k={k} n={n}")
    x = _randn((m, k), 1.0, f"lin.x{m}")
    w = _randn((n, k), 0.05, f"lin.w{n}")
    ref = np32(x).astype(np.float64) @ np32(w).astype(np.float64).T
    xd, wd = x.to(DEV), w.to(DEV)
    o_bf = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    dg.op_linear(xd, wd, o_bf, 0)
    o32 = torch.empty((m, n), dtype=torch.float32, device=DEV)
    dg.op_linear(xd, wd, o32, 1)
    base = _randn((m, n), 1.0, f"lin.base{m}", torch.float32)
    acc = base.to(DEV)
    dg.op_linear(xd, wd, acc, 2)
    torch.cuda.synchronize()
    e_bf = rel_err(np32(o_bf), ref)
    e32 = rel_err(np32(o32), ref)
    e_add = rel_err(np32(acc), ref + base.numpy())
    log(f"  rel err bf16 {e_bf:.2e} fp32 {e32:.2e} add {e_add:.2e}")
    assert e_bf < 8e-3 and e32 < 1e-5 and e_add < 1e-5


# ------------------------------------------------------------------ packing

def _pack_reference(a, esz):
    """The packed layout by its definition (include/dg.h): groups x [R, K]
    byte matrices -> 1 KB blocks of 16 rows x 64/esz values, piece r + 16 q
    of block (rb, kb) = row 16 rb + r, values kb * 64/esz + q * 16/esz ..
    +16/esz - 1; block (rb, kb) at ((rb // 4) * 4 * KB + kb * 4 + rb % 4) KB,
    KB = K*esz/64; rows zero-padded to 64."""
    g, r, kbytes = a.shape
    rp = (r + 63) // 64 * 64
    kbn = kbytes // 64
    pad = np.zeros((g, rp, kbytes), np.uint8)
    pad[:, :r] = a
    out = np.zeros((g, rp // 16 * kbn, 64, 16), np.uint8)
    for rb in range(rp // 16):
        for kb in range(kbn):
            at = (rb // 4) * 4 * kbn + kb * 4 + rb % 4
            for q in range(4):
                for rr in range(16):
                    out[:, at, rr + 16 * q] = pad[:, 16 * rb + rr,
                                                  64 * kb + 16 * q:64 * kb + 16 * q + 16]
    return out.reshape(-1)


@pytest.mark.parametrize("groups,rows,cols,e4m3", [(1, 40, 96, False), (1, 200, 64, False),
                                                    (3, 64, 128, True)])
def test_pack_weights_matches_layout_definition(groups, rows, cols, e4m3):
    gen = torch.Generator().manual_seed(11)
    if e4m3:
        t = torch.randint(0, 256, (groups, rows, cols), dtype=torch.uint8, generator=gen)
        a = t.numpy()
    else:
        t = torch.randn(groups, rows, cols, generator=gen).to(torch.bfloat16)
        a = t.view(torch.uint8).numpy().reshape(groups, rows, cols * 2)
    p = dg.pack(t.to(DEV) if groups > 1 else t[0].to(DEV))
    torch.cuda.synchronize()
    got = p.buf.cpu().numpy()
    assert np.array_equal(got, _pack_reference(a, 1 if e4m3 else 2))


# ------------------------------------------------------------------ rmsnorm

@pytest.mark.parametrize("rows,h", [(37, 256), (256, 2048)])
def test_rmsnorm(rows, h):
    x = _randn((rows, h), 3.0, f"rms.x{h}", torch.float32)
    g = 1.0 + _randn((h,), 0.1, f"rms.g{h}", torch.float32)
    out = torch.empty((rows, h), dtype=torch.bfloat16, device=DEV)
    dg.op_rmsnorm(x.to(DEV), g.to(DEV), 1e-6, out)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x.numpy(), g.numpy(), 1e-6)
    # bf16 storage: relative error per element at most 2^-8
    rel = np.abs(np32(out) - ref) / np.maximum(np.abs(ref), 1e-30)
    assert np.max(rel) <= 2.0 ** -8 * 1.01


# ------------------------------------------------------------------ attention

def _attn_case(n, C, Hq, Hkv, D, plens, max_kv, causal, splits, q_scale=1.0,
               tag=""):
    log(f"attention n={n} C={C} Hq={Hq} Hkv={Hkv} D={D} P={plens} "
        f"causal={causal} splits={splits} {tag}")
    qkv_cols = (Hq + 2 * Hkv) * D
    max_req = n + 1
    req = [(b + 1) % max_req for b in range(n)]  # slots 1..n, not 0
    qkv = _randn((n * C, qkv_cols), 1.0, f"attn.qkv{tag}")
    if q_scale != 1.0:
        qkv[:, :Hq * D] = (qkv[:, :Hq * D].float() * q_scale).to(torch.bfloat16)
    kc = _randn((max_req, Hkv, max_kv, D), 1.0, f"attn.kc{tag}")
    vc = _randn((max_req, Hkv, max_kv, D), 1.0, f"attn.vc{tag}")
    out = torch.zeros((n * C, Hq * D), dtype=torch.bfloat16, device=DEV)
    dg.op_canvas_attention(qkv.to(DEV), n, C, Hq, Hkv, D, kc.to(DEV),
                           vc.to(DEV), max_req, max_kv, req, plens, causal,
                           splits, out)
    torch.cuda.synchronize()
    got = np32(out)
    q_all = np32(qkv)
    worst = 0.0
    for b in range(n):
        rows = slice(b * C, (b + 1) * C)
        q = q_all[rows, :Hq * D].reshape(C, Hq, D).transpose(1, 0, 2)
        kcan = q_all[rows, Hq * D:(Hq + Hkv) * D].reshape(C, Hkv, D).transpose(1, 0, 2)
        vcan = q_all[rows, (Hq + Hkv) * D:].reshape(C, Hkv, D).transpose(1, 0, 2)
        P = plens[b]
        kp = np32(kc[req[b], :, :P])
        vp = np32(vc[req[b], :, :P])
        ref = oracle.canvas_attention(q, kp, vp, kcan, vcan, causal=causal)
        ref = ref.transpose(1, 0, 2).reshape(C, Hq * D)
        for h in range(Hq):
            e = rel_err(got[rows, h * D:(h + 1) * D], ref[:, h * D:(h + 1) * D])
            worst = max(worst, e)
    log(f"  worst per-head rel err {worst:.2e}")
    assert worst < TOL
    return worst


def test_attention_tiny_shape_all_splits():
    for s in (0, 1, 3, 7):
        _attn_case(1, 256, 4, 2, 64, [512], 1024, False, s, tag=f"t{s}")


def test_attention_full_size_layer_shape():
    _attn_case(1, 256, 16, 8, 128, [2048], 4096, False, 0, tag="g")


def test_attention_edges_empty_and_ragged_prefix_causal_ragged_canvas():
    _attn_case(1, 256, 4, 2, 64, [0], 512, False, 0, tag="p0")
    _attn_case(1, 256, 16, 8, 128, [77], 512, False, 2, tag="p77")
    _attn_case(1, 256, 4, 2, 64, [100], 512, True, 0, tag="causal")
    _attn_case(1, 256, 4, 2, 64, [0], 512, True, 5, tag="causal0")
    _attn_case(1, 100, 8, 2, 128, [65], 512, False, 3, tag="c100")
    _attn_case(1, 256, 4, 4, 64, [130], 512, False, 0, q_scale=6.0,
               tag="mha_sharp")


def test_attention_batch_of_canvases_with_own_prefixes():
    _attn_case(3, 256, 16, 8, 128, [2048, 5, 700], 2048, False, 0, tag="b3")
    _attn_case(3, 256, 16, 8, 128, [2048, 0, 700], 2048, True, 0, tag="b3c")


def test_attention_two_query_blocks_per_wave():
    """Key ranges long enough for the 256-row workgroups (two 16-row query
    blocks per wave, workgroups of one KV head and split on one XCD):
    causal with two canvases of ragged prefixes, one KV head per query head,
    a ragged canvas whose last workgroup holds invalid rows, head dim 64."""
    _attn_case(2, 256, 16, 8, 128, [20000, 9001], 20480, True, 0, tag="qb2c")
    _attn_case(1, 256, 4, 4, 64, [12000], 12288, False, 0, tag="qb2g1")
    _attn_case(1, 100, 8, 2, 128, [30000], 30208, False, 0, tag="qb2c100")


def test_attention_long_prefix_sampled_rows():
    """131072 cached keys (long-context workload) with the launch the step
    uses; the oracle checks 6 sampled canvas positions of every head."""
    Hq, Hkv, D, C, P = 16, 8, 128, 256, 131072
    log("attention long prefix P=131072")
    qkv = synth.normal((C, (Hq + 2 * Hkv) * D), 1.0, 7, "long.qkv", DEV)
    kc = synth.normal((1, Hkv, P, D), 1.0, 7, "long.k", DEV)
    vc = synth.normal((1, Hkv, P, D), 1.0, 7, "long.v", DEV)
    out = torch.zeros((C, Hq * D), dtype=torch.bfloat16, device=DEV)
    dg.op_canvas_attention(qkv, 1, C, Hq, Hkv, D, kc, vc, 1, P, [0], [P],
                           False, 0, out)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 77, 128, 200, 255])
    q_all = np32(qkv)
    q = q_all[rows, :Hq * D].reshape(len(rows), Hq, D).transpose(1, 0, 2)
    kcan = q_all[:, Hq * D:(Hq + Hkv) * D].reshape(C, Hkv, D).transpose(1, 0, 2)
    vcan = q_all[:, (Hq + Hkv) * D:].reshape(C, Hkv, D).transpose(1, 0, 2)
    ref = oracle.canvas_attention(q, np32(kc[0]), np32(vc[0]), kcan, vcan,
                                  q_pos=rows)
    got = np32(out)[rows].reshape(len(rows), Hq, D).transpose(1, 0, 2)
    e = rel_err(got, ref)
    log(f"  rel err {e:.2e}")
    assert e < TOL


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("t,e,k", [(300, 16, 2), (256, 128, 8), (5, 8, 8)])
def test_router_topk_bit_exact_on_identical_logits(t, e, k):
    lg = torch.round(_randn((t, e), 1.0, f"rt{e}", torch.float32) * 8) / 8
    idx = torch.empty((t, k), dtype=torch.int32, device=DEV)
    w = torch.empty((t, k), dtype=torch.float32, device=DEV)
    dg.op_router_topk(lg.to(DEV), k, idx, w)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.router_topk(lg.numpy().astype(np.float64), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    assert rel_err(w.cpu().numpy(), o_w) < 1e-6


# ------------------------------------------------------------------ MoE

def _moe_case(shape, T, tag, top_k=None, same_rows=False):
    """same_rows: one random row repeated T times, so every token picks the
    same k experts (T tokens in each: several token passes per expert)."""
    if top_k is not None:
        shape = synth.ModelShape(**{**shape.__dict__, "top_k": top_k})
    log(f"moe {tag}: T={T} H={shape.hidden} E={shape.n_experts} "
        f"k={shape.top_k} F={shape.expert_ffn} {shape.expert_dtype}")
    w = synth.make_weights(synth.ModelShape(**{**shape.__dict__,
                                               "n_layers": 1, "vocab": 8}),
                           seed=11)
    lw = w["layers"][0]
    xh = _randn((T, shape.hidden), 1.0, f"moe.x{tag}")
    if same_rows:
        xh = xh[:1].repeat(T, 1)
    lwd = {k: (v.to(DEV).contiguous() if v is not None else None)
           for k, v in lw.items()}
    y = torch.zeros((T, shape.hidden), dtype=torch.float32, device=DEV)
    ridx = torch.empty((T, shape.top_k), dtype=torch.int32, device=DEV)
    rw = torch.empty((T, shape.top_k), dtype=torch.float32, device=DEV)
    counts = torch.empty(shape.n_experts, dtype=torch.int32, device=DEV)
    dg.op_moe(shape, lwd, xh.to(DEV), y, ridx, rw, counts)
    torch.cuda.synchronize()
    lwn = synth.to_numpy_weights({"embed": w["embed"][:1],
                                  "final_norm": w["final_norm"],
                                  "layers": [lw]})["layers"][0]
    x64 = np32(xh).astype(np.float64)
    r, o_idx, o_w, ref = oracle.moe_layer(oshape(shape), lwn, x64, mirror=True)
    g_idx = ridx.cpu().numpy()
    same = np.all(g_idx == o_idx, axis=1)
    marg = routing_margin(r, shape.top_k)
    assert np.all(marg[~same] < MARGIN), "routing differs at a clear margin"
    log(f"  routing: {int((~same).sum())} low-margin tokens differ")
    e = rel_err(np32(y)[same], ref[same])
    er = row_err(np32(y)[same], ref[same])
    log(f"  mixture rel err {e:.2e} (per row {er:.2e})")
    assert e < TOL and er < (TOL_ROW_FP8_ACT if fp8_act(shape) else TOL)
    c = counts.cpu().numpy()
    assert c.sum() == T * shape.top_k
    np.testing.assert_array_equal(c, np.bincount(g_idx.reshape(-1),
                                                 minlength=shape.n_experts))
    assert rel_err(rw.cpu().numpy()[same], o_w[same]) < 1e-4
    return e


def test_moe_tiny_shape():
    _moe_case(TINY, 256, "tiny")
    _moe_case(TINY, 37, "tiny_ragged")
    _moe_case(TINY, 1, "tiny_one")


def test_moe_full_shape_every_token_in_the_same_experts():
    # 160 identical rows at the full layer shape: 8 experts hold 160 tokens
    # each (two gate/up and three down token passes per expert), bf16 and
    # e4m3 experts
    _moe_case(GEMMA, 160, "gemma_same", same_rows=True)
    g8 = synth.ModelShape(**{**GEMMA.__dict__, "expert_dtype": "fp8_e4m3"})
    _moe_case(g8, 160, "gemma_fp8_same", same_rows=True)


def test_moe_all_experts_selected():
    _moe_case(TINY, 64, "all", top_k=16)


def test_moe_full_size_layer_shape():
    _moe_case(GEMMA, 256, "gemma")


def test_moe_tiled_path_full_size_layer_shape():
    # 1024 tokens x top-8 over 128 experts: 64 rows per expert on average,
    # beyond the weight-streaming range (the grouped tiled GEMM runs)
    _moe_case(GEMMA, 1024, "gemma_tiled")
    g8 = synth.ModelShape(**{**GEMMA.__dict__, "expert_dtype": "fp8_e4m3"})
    _moe_case(g8, 1024, "gemma_fp8_tiled")


def test_moe_large_tile_path_full_size_layer_shape():
    # 4096 tokens x top-8 over 128 experts: 256 rows per expert on average,
    # the grouped GEMMs on 256-row tiles (ragged per expert), bf16 and e4m3
    _moe_case(GEMMA, 4096, "gemma_mm")
    g8 = synth.ModelShape(**{**GEMMA.__dict__, "expert_dtype": "fp8_e4m3"})
    _moe_case(g8, 4096, "gemma_fp8_mm")


@pytest.mark.parametrize("t", [1, 8, 15])
@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("shared", [0, 1])
def test_moe_few_tokens_most_experts_empty(t, dtype, shared):
    # fewer (token, rank) pairs than expert groups (one decoded position
    # routes to 8 of 128 experts): the expert kernels read each group's
    # count before any load, and the empty groups leave at once
    g = synth.ModelShape(**{**GEMMA.__dict__, "expert_dtype": dtype,
                            "n_shared_experts": shared})
    _moe_case(g, t, f"few_{dtype}_{t}_{shared}")


@pytest.mark.parametrize("t", [256, 1024, 4096])
@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_moe_with_shared_expert(t, dtype):
    # write-up Table 1 "+ 1 shared": every token's pairs end with the shared
    # expert (weight 1) on each MoE path: weight streaming (256 tokens),
    # 64-row tiles (1024) and 256-row tiles (4096)
    g = synth.ModelShape(**{**GEMMA.__dict__, "expert_dtype": dtype,
                            "n_shared_experts": 1})
    _moe_case(g, t, f"shared_{dtype}_{t}")


def test_moe_e4m3_experts():
    s8 = synth.ModelShape(**{**TINY.__dict__, "expert_dtype": "fp8_e4m3"})
    _moe_case(s8, 256, "tiny_fp8")
    g8 = synth.ModelShape(**{**GEMMA.__dict__, "expert_dtype": "fp8_e4m3"})
    _moe_case(g8, 512, "gemma_fp8")


# ------------------------------------------------------------------ LM head

def _lm_case(m, h, v, tag, embed=None, xh=None):
    log(f"lmhead {tag}: M={m} H={h} V={v}")
    if embed is None:
        embed = _randn((v, h), 0.02, f"lm.E{tag}")
    if xh is None:
        xh = _randn((m, h), 1.0, f"lm.x{tag}")
    ent = torch.empty(m, dtype=torch.float32, device=DEV)
    lse = torch.empty(m, dtype=torch.float32, device=DEV)
    am = torch.empty(m, dtype=torch.int32, device=DEV)
    logits = torch.empty((m, v), dtype=torch.float32, device=DEV)
    dg.op_lmhead_entropy(xh.to(DEV), embed.to(DEV), ent, lse, am, logits)
    torch.cuda.synchronize()
    st = oracle.lm_head_stats(np32(xh), np32(embed), want_logits=True)
    e_z = rel_err(np32(logits), st["logits"])
    e_h = rel_err(ent.cpu().numpy(), st["entropy"])
    e_l = rel_err(lse.cpu().numpy(), st["lse"])
    marg = top2_margin(st["logits"])
    ga = am.cpu().numpy()
    bad = (ga != st["argmax"]) & (marg >= MARGIN)
    log(f"  rel err logits {e_z:.2e} entropy {e_h:.2e} lse {e_l:.2e}; "
        f"argmax differs at {int((ga != st['argmax']).sum())} rows "
        f"({int(bad.sum())} with margin >= {MARGIN})")
    assert e_z < 1e-5 and e_h < 1e-4 and e_l < 1e-5 and not bad.any()
    return ent, am


def test_lmhead_tiny_and_ragged_vocab():
    _lm_case(128, 256, 4096, "tiny")
    _lm_case(5, 256, 1000, "ragged")
    _lm_case(1, 128, 130, "one")


def test_lmhead_full_vocab():
    _lm_case(128, 2048, 262144, "gemma")


def test_lmhead_tile_counts():
    # the streaming LM head runs 2, 4, 6 or 8 token tiles per pass by row
    # count: both sides of each boundary, and two passes of 8 tiles
    for m in (32, 33, 64, 65, 96, 97, 200):
        _lm_case(m, 256, 3000, f"tiles{m}")


def test_lmhead_full_vocab_four_tiles():
    _lm_case(48, 2048, 262144, "gemma48")


def test_lmhead_full_vocab_tiled_path():
    # more than 128 rows: the 256 x 256 tile kernel (two partials per
    # workgroup), with a ragged last row tile
    _lm_case(300, 2048, 262144, "gemma_tiled")
    _lm_case(129, 2048, 262144, "gemma_129")


def test_lmhead_uniform_and_tied_logits():
    v, h = 4096, 256
    embed = torch.full((v, h), 0.03125, dtype=torch.bfloat16)
    ent, am = _lm_case(3, h, v, "uniform", embed=embed)
    np.testing.assert_allclose(ent.cpu().numpy(), math.log(v), rtol=1e-5)
    assert np.all(am.cpu().numpy() == 0)


# ------------------------------------------------------------------ EB

def _eb_gpu(ent, am, com, tok, step, gamma, cap, refine):
    n = ent.shape[0]
    d = {k: t.to(DEV).contiguous() for k, t in
         dict(ent=ent, am=am, com=com, tok=tok, step=step, gamma=gamma).items()}
    n_new = torch.zeros(n, dtype=torch.int32, device=DEV)
    done = torch.zeros(n, dtype=torch.uint8, device=DEV)
    dg.op_eb_select(d["ent"], d["am"], d["com"], d["tok"], d["step"],
                    d["gamma"], cap, refine, n_new, done)
    torch.cuda.synchronize()
    return (d["com"].cpu().numpy(), d["tok"].cpu().numpy(),
            d["step"].cpu().numpy(), n_new.cpu().numpy(), done.cpu().numpy())


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("gamma", [0.0, 0.5, 7.25, float("inf")])
def test_eb_select_bit_exact(ties, gamma):
    n = 6
    ent, am, com = synth.make_entropy_inputs(n, seed=3, ties=ties)
    com[4] = 1  # a finished canvas
    tok = am.clone() + 7
    step = torch.tensor([0, 3, 63, 10, 2, 0], dtype=torch.int32)
    gam = torch.full((n,), gamma, dtype=torch.float32)
    for cap, refine in ((256, True), (64, False)):
        got = _eb_gpu(ent, am, com, tok, step, gam, cap, refine)
        ref = oracle.eb_select(ent.numpy(), am.numpy(), com.numpy(),
                               tok.numpy(), step.numpy(), gam.numpy(), cap,
                               refine=refine)
        for g, o in zip(got, ref):
            np.testing.assert_array_equal(g, o)


def test_eb_worked_example_on_device(golden_dir):
    with open(os.path.join(golden_dir, "eb_worked_example.json")) as f:
        ex = json.load(f)
    for case in ex["cases"]:
        ent = torch.zeros((1, 256), dtype=torch.float32)
        ent[0, :8] = torch.tensor(ex["entropy"])
        com = torch.ones((1, 256), dtype=torch.uint8)
        com[0, :8] = torch.tensor(ex["committed"], dtype=torch.uint8)
        tok = torch.zeros((1, 256), dtype=torch.int32)
        tok[0, :8] = torch.tensor(ex["tokens"], dtype=torch.int32)
        am = torch.zeros((1, 256), dtype=torch.int32)
        am[0, :8] = torch.tensor(ex["argmax"], dtype=torch.int32)
        c, t, s, nn, d = _eb_gpu(ent, am, com, tok,
                                 torch.tensor([case["step"]], dtype=torch.int32),
                                 torch.tensor([case["gamma"]], dtype=torch.float32),
                                 case["cap"], True)
        assert c[0, :8].tolist() == case["committed"], case["why"]
        assert t[0, :8].tolist() == case["tokens_refine"], case["why"]
        assert nn[0] == case["n_new"] and d[0] == case["done"]


# ------------------------------------------------------------------ KV append

def test_kv_append_rows():
    n, C, Hq, Hkv, D, S = 2, 256, 16, 8, 128, 1024
    qkv = _randn((n * C, (Hq + 2 * Hkv) * D), 1.0, "kva.qkv").to(DEV)
    kc = torch.zeros((3, Hkv, S, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    dg.op_kv_append(qkv, n, C, Hq, Hkv, D, kc, vc, 3, S, [2, 0], [300, 768])
    torch.cuda.synchronize()
    q = qkv.cpu()
    for b, (r, row0) in enumerate(((2, 300), (0, 768))):
        rows = q[b * C:(b + 1) * C]
        k_ref = rows[:, Hq * D:(Hq + Hkv) * D].reshape(C, Hkv, D).transpose(0, 1)
        v_ref = rows[:, (Hq + Hkv) * D:].reshape(C, Hkv, D).transpose(0, 1)
        assert torch.equal(kc[r, :, row0:row0 + C].cpu(), k_ref)
        assert torch.equal(vc[r, :, row0:row0 + C].cpu(), v_ref)
    assert float(kc[1].abs().sum()) == 0.0
