"""Pins of the CPU oracle against things other than itself: hand-worked
fixtures, closed forms, invariants, brute force on tiny inputs and library
routines for the number formats.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.model import _layers_forward

RNG = np.random.default_rng(1234)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- numerics

def test_round_bf16_matches_torch_on_float32_values():
    x = RNG.standard_normal(20000).astype(np.float32) * 10.0 ** RNG.integers(
        -6, 6, 20000)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    assert oracle.round_bf16(one + ulp / 2) == one              # tie, even down
    assert oracle.round_bf16(one + 3 * ulp / 2) == one + 2 * ulp  # tie, even up
    assert oracle.round_bf16(one + ulp / 2 + 1e-12) == one + ulp
    assert oracle.round_bf16(-(one + ulp / 2)) == -one


def test_decode_e4m3_matches_torch_and_known_values():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert oracle.decode_e4m3(np.uint8(0x7E)) == 448.0
    assert oracle.decode_e4m3(np.uint8(0x01)) == 2.0 ** -9
    assert oracle.decode_e4m3(np.uint8(0x38)) == 1.0
    assert oracle.decode_e4m3(np.uint8(0xB8)) == -1.0


# ----------------------------------------------------------------- rmsnorm

def test_rmsnorm_closed_form_and_scale_invariance():
    eps = 1e-6
    g = RNG.standard_normal(16)
    c = -3.0
    y = oracle.rmsnorm(np.full(16, c), g, eps)
    np.testing.assert_allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-15)
    x = RNG.standard_normal((4, 16))
    np.testing.assert_allclose(oracle.rmsnorm(1e3 * x, g, 0.0),
                               oracle.rmsnorm(x, g, 0.0), rtol=1e-12)
    # unit gains: root mean square of the output is 1 when eps = 0
    y = oracle.rmsnorm(x, np.ones(16), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0,
                               rtol=1e-13)


# ----------------------------------------------------------------- attention

def test_attention_hand_example(golden_dir):
    ex = _load(golden_dir, "attention_d1_example.json")
    q = np.array([[[ex["q"]]]])
    kp = np.array(ex["k_prefix"]).reshape(1, -1, 1)
    vp = np.array(ex["v_prefix"]).reshape(1, -1, 1)
    kc = np.array(ex["k_canvas"]).reshape(1, -1, 1)
    vc = np.array(ex["v_canvas"]).reshape(1, -1, 1)
    for causal in (False, True):
        o = oracle.canvas_attention(q, kp, vp, kc, vc, causal=causal)
        assert o[0, 0, 0] == pytest.approx(ex["expected"], rel=1e-14)


def _rand_attn(hq=4, hkv=2, p=5, c=7, d=8, scale=1.0):
    q = RNG.standard_normal((hq, c, d)) * scale
    kp = RNG.standard_normal((hkv, p, d))
    vp = RNG.standard_normal((hkv, p, d))
    kc = RNG.standard_normal((hkv, c, d))
    vc = RNG.standard_normal((hkv, c, d))
    return q, kp, vp, kc, vc


def test_attention_single_visible_key_returns_its_value():
    q, _, _, kc, vc = _rand_attn(p=0)
    empty = np.zeros((2, 0, 8))
    o = oracle.canvas_attention(q, empty, empty, kc, vc, causal=True)
    # query 0 of head h sees only canvas key 0 of KV head h // 2
    for h in range(4):
        np.testing.assert_allclose(o[h, 0], vc[h // 2, 0], rtol=1e-14)


def test_attention_identical_keys_average_values():
    q, kp, vp, kc, vc = _rand_attn()
    kp[:] = 0.3
    kc[:] = 0.3
    o = oracle.canvas_attention(q, kp, vp, kc, vc)
    for h in range(4):
        mean = np.concatenate([vp[h // 2], vc[h // 2]]).mean(axis=0)
        np.testing.assert_allclose(o[h], np.broadcast_to(mean, o[h].shape),
                                   rtol=1e-12)


def test_attention_permutation_equivariance_without_positions():
    q, kp, vp, kc, vc = _rand_attn()
    perm = RNG.permutation(q.shape[1])
    o = oracle.canvas_attention(q, kp, vp, kc, vc)
    o_p = oracle.canvas_attention(q[:, perm], kp, vp, kc[:, perm], vc[:, perm])
    np.testing.assert_allclose(o_p, o[:, perm], rtol=1e-12, atol=1e-14)


def test_attention_keys_are_a_set_prefix_canvas_split_irrelevant():
    q, kp, vp, kc, vc = _rand_attn(p=6, c=7)
    o = oracle.canvas_attention(q, kp, vp, kc, vc)
    # move the first 3 canvas keys into the prefix and put the prefix last
    kp2 = np.concatenate([kc[:, :3], kp], axis=1)
    vp2 = np.concatenate([vc[:, :3], vp], axis=1)
    o2 = oracle.canvas_attention(q, kp2, vp2, kc[:, 3:], vc[:, 3:])
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)


def test_attention_gqa_equals_mha_with_repeated_kv_heads():
    q, kp, vp, kc, vc = _rand_attn(hq=6, hkv=2)
    o = oracle.canvas_attention(q, kp, vp, kc, vc)
    rep = lambda a: np.repeat(a, 3, axis=0)  # noqa: E731
    o_mha = oracle.canvas_attention(q, rep(kp), rep(vp), rep(kc), rep(vc))
    np.testing.assert_allclose(o_mha, o, rtol=1e-13)


def test_attention_causal_equals_truncated_key_set():
    q, kp, vp, kc, vc = _rand_attn(c=9)
    o = oracle.canvas_attention(q, kp, vp, kc, vc, causal=True)
    for i in range(9):
        oi = oracle.canvas_attention(q[:, i:i + 1], kp, vp, kc[:, :i + 1],
                                     vc[:, :i + 1])
        np.testing.assert_allclose(o[:, i], oi[:, 0], rtol=1e-12, atol=1e-14)


def test_attention_output_in_convex_hull_of_values():
    q, kp, vp, kc, vc = _rand_attn(scale=5.0)
    o = oracle.canvas_attention(q, kp, vp, kc, vc)
    for h in range(4):
        vals = np.concatenate([vp[h // 2], vc[h // 2]])
        assert np.all(o[h] <= vals.max(axis=0) + 1e-12)
        assert np.all(o[h] >= vals.min(axis=0) - 1e-12)


def test_attention_sampled_rows_match_full():
    q, kp, vp, kc, vc = _rand_attn(c=9)
    o = oracle.canvas_attention(q, kp, vp, kc, vc, causal=True)
    rows = np.array([2, 7])
    o_s = oracle.canvas_attention(q[:, rows], kp, vp, kc, vc, causal=True,
                                  q_pos=rows)
    np.testing.assert_allclose(o_s, o[:, rows], rtol=1e-14)


# ----------------------------------------------------------------- router / MoE

def test_router_topk_hand_example_with_ties():
    logits = np.array([[1.0, 3.0, 3.0, 0.5]])
    idx, w = oracle.router_topk(logits, 2)
    assert idx.tolist() == [[1, 2]]
    np.testing.assert_allclose(w, [[0.5, 0.5]], rtol=1e-15)
    idx, w = oracle.router_topk(logits, 3)
    assert idx.tolist() == [[1, 2, 0]]
    e2 = math.exp(-2.0)
    np.testing.assert_allclose(w[0], [1 / (2 + e2), 1 / (2 + e2),
                                      e2 / (2 + e2)], rtol=1e-14)


def test_router_topk_against_brute_force_comparisons():
    logits = np.round(RNG.standard_normal((50, 16)), 1)  # many ties
    idx, w = oracle.router_topk(logits, 4)
    for t in range(50):
        sel = list(idx[t])
        rest = [e for e in range(16) if e not in sel]
        key = lambda e: (-logits[t, e], e)  # noqa: E731
        assert all(key(a) < key(b) for a in sel for b in rest)
        assert all(key(sel[i]) < key(sel[i + 1]) for i in range(3))
        assert w[t].sum() == pytest.approx(1.0, abs=1e-14)
        assert np.all(np.diff(w[t]) <= 0)


def _scalar_silu(v):
    return v / (1.0 + math.exp(-v))


def test_moe_scalar_closed_form():
    # H = F = 1, two experts, both selected, router weights 3/4 and 1/4
    wgu = np.array([[[1.0], [0.5]], [[-1.0], [2.0]]])   # [E, 2F, H]
    wd = np.array([[[3.0]], [[1.0]]])                   # [E, H, F]
    x = np.array([[2.0]])
    r = np.array([[math.log(3.0), 0.0]])
    idx, w = oracle.router_topk(r, 2)
    y = oracle.moe_mixture(x, idx, w, wgu, wd, mirror=False)
    expect = 0.75 * 3.0 * _scalar_silu(2.0) * 1.0 + \
        0.25 * 1.0 * _scalar_silu(-2.0) * 4.0
    assert y[0, 0] == pytest.approx(expect, rel=1e-14)


def _moe_case(t=9, h=12, f=5, e=6, fp8=False):
    x = RNG.standard_normal((t, h))
    wgu = RNG.standard_normal((e, 2 * f, h)) * 0.3
    wd = RNG.standard_normal((e, h, f)) * 0.3
    r = RNG.standard_normal((t, e))
    return x, wgu, wd, r


def test_moe_all_experts_equals_dense_softmax_mixture():
    x, wgu, wd, r = _moe_case()
    e_count = wgu.shape[0]
    idx, w = oracle.router_topk(r, e_count)
    y = oracle.moe_mixture(x, idx, w, wgu, wd, mirror=False)
    # dense form: every expert on every token, weighted by softmax over all E
    f = wd.shape[2]
    dense = np.zeros_like(x)
    for t in range(x.shape[0]):
        p = np.exp(r[t] - r[t].max())
        p /= p.sum()
        for e in range(e_count):
            gate = wgu[e, :f] @ x[t]
            up = wgu[e, f:] @ x[t]
            act = np.array([_scalar_silu(v) for v in gate]) * up
            dense[t] += p[e] * (wd[e] @ act)
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-13)


def test_moe_top1_is_single_expert_and_identical_experts_ignore_routing():
    x, wgu, wd, r = _moe_case()
    idx, w = oracle.router_topk(r, 1)
    y = oracle.moe_mixture(x, idx, w, wgu, wd, mirror=False)
    f = wd.shape[2]
    for t in range(x.shape[0]):
        e = idx[t, 0]
        act = np.array([_scalar_silu(v) for v in wgu[e, :f] @ x[t]]) * \
            (wgu[e, f:] @ x[t])
        np.testing.assert_allclose(y[t], wd[e] @ act, rtol=1e-12)
    same_gu = np.repeat(wgu[:1], wgu.shape[0], axis=0)
    same_d = np.repeat(wd[:1], wd.shape[0], axis=0)
    idx3, w3 = oracle.router_topk(r, 3)
    y3 = oracle.moe_mixture(x, idx3, w3, same_gu, same_d, mirror=False)
    idx0 = np.zeros((x.shape[0], 1), dtype=np.int64)
    y0 = oracle.moe_mixture(x, idx0, np.ones((x.shape[0], 1)), same_gu,
                            same_d, mirror=False)
    np.testing.assert_allclose(y3, y0, rtol=1e-12, atol=1e-14)


def test_expert_matrix_e4m3_scale():
    codes = RNG.integers(0, 256, size=(2, 3, 4), dtype=np.uint8)
    codes[codes & 0x7F == 0x7F] = 0  # no NaN codes
    scale = RNG.random((2, 3)).astype(np.float32) + 0.5
    ref = torch.from_numpy(codes[1]).view(torch.float8_e4m3fn).to(
        torch.float64).numpy() * scale[1].astype(np.float64)[:, None]
    np.testing.assert_array_equal(oracle.expert_matrix(codes, scale, 1), ref)


# ----------------------------------------------------------------- LM head

def test_entropy_hand_example(golden_dir):
    ex = _load(golden_dir, "entropy_example.json")
    p = np.array(ex["probabilities"])
    embed = (np.log(p) + ex["shift"]).reshape(-1, 1)   # [V, H=1]
    st = oracle.lm_head_stats(np.ones((1, 1)), embed)
    assert st["entropy"][0] == pytest.approx(ex["entropy"], rel=1e-14)
    assert st["lse"][0] == pytest.approx(ex["lse"], rel=1e-14)
    assert st["argmax"][0] == ex["argmax"]


def test_uniform_logits_entropy_is_log_v():
    for v in (7, 4096):
        embed = np.full((v, 3), 0.25)
        st = oracle.lm_head_stats(np.array([[1.0, 2.0, -1.0]]), embed)
        assert st["entropy"][0] == pytest.approx(math.log(v), rel=1e-12)
        assert st["lse"][0] == pytest.approx(math.log(v) + 0.5, rel=1e-12)
        assert st["argmax"][0] == 0


def test_two_tied_maxima_and_dominant_logit():
    z = np.full(64, -1e4)
    z[[37, 11]] = 5.0
    st = oracle.lm_head_stats(np.ones((1, 1)), z.reshape(-1, 1))
    assert st["entropy"][0] == pytest.approx(math.log(2.0), rel=1e-12)
    assert st["argmax"][0] == 11
    z = np.zeros(64)
    z[50] = 200.0
    st = oracle.lm_head_stats(np.ones((1, 1)), z.reshape(-1, 1))
    assert 0.0 <= st["entropy"][0] < 1e-80
    assert st["argmax"][0] == 50


def test_entropy_matches_one_pass_identity_brute_force():
    # H = ln s - t/s with s = sum e^(z-m), t = sum e^(z-m) (z-m): an identity
    # that follows from ln p = z - m - ln s; evaluated here with math.fsum
    for _ in range(20):
        v = int(RNG.integers(2, 65))
        xh = RNG.standard_normal((1, 3))
        embed = RNG.standard_normal((v, 3)) * 2.0
        st = oracle.lm_head_stats(xh, embed)
        z = [float(xh[0] @ embed[i]) for i in range(v)]
        m = max(z)
        s = math.fsum(math.exp(zi - m) for zi in z)
        t = math.fsum(math.exp(zi - m) * (zi - m) for zi in z)
        assert st["entropy"][0] == pytest.approx(math.log(s) - t / s,
                                                 rel=1e-12, abs=1e-14)
        assert st["lse"][0] == pytest.approx(m + math.log(s), rel=1e-14)
        assert st["argmax"][0] == z.index(m)


# ----------------------------------------------------------------- EB sampler

def test_eb_worked_example(golden_dir):
    ex = _load(golden_dir, "eb_worked_example.json")
    ent = np.array([ex["entropy"]], dtype=np.float32)
    for case in ex["cases"]:
        for refine in (True, False):
            com, tok, step, n_new, done = oracle.eb_select(
                ent, np.array([ex["argmax"]]), np.array([ex["committed"]]),
                np.array([ex["tokens"]]), np.array([case["step"]]),
                np.array([case["gamma"]], dtype=np.float32), case["cap"],
                refine=refine)
            assert com[0].tolist() == case["committed"], case["why"]
            want = case["tokens_refine" if refine else "tokens_norefine"]
            assert tok[0].tolist() == want, case["why"]
            assert n_new[0] == case["n_new"] and done[0] == case["done"]
            assert step[0] == case["step"] + 1


def _eb_rand(b=3, c=256, committed_frac=0.3):
    ent = RNG.random((b, c)).astype(np.float32) * 2.0
    com = (RNG.random((b, c)) < committed_frac).astype(np.uint8)
    am = RNG.integers(0, 1000, (b, c))
    tok = RNG.integers(0, 1000, (b, c))
    return ent, am, com, tok


def test_eb_gamma_zero_commits_exactly_the_min_entropy_position():
    ent, am, com, tok = _eb_rand()
    c2, _, _, n_new, _ = oracle.eb_select(ent, am, com, tok, np.zeros(3),
                                          np.zeros(3, np.float32), 256)
    assert n_new.tolist() == [1, 1, 1]
    for b in range(3):
        newly = np.nonzero((c2[b] == 1) & (com[b] == 0))[0]
        unc = np.nonzero(com[b] == 0)[0]
        best = min(unc, key=lambda j: (ent[b, j], j))
        assert newly.tolist() == [best]


def test_eb_infinite_gamma_commits_all_and_block_always_finishes():
    ent, am, com, tok = _eb_rand()
    c2, _, _, n_new, done = oracle.eb_select(
        ent, am, com, tok, np.zeros(3), np.full(3, np.inf, np.float32), 256)
    assert np.all(c2 == 1) and np.all(done == 1)
    assert n_new.tolist() == [(com[b] == 0).sum() for b in range(3)]
    # at least one commit per step: a block finishes within 256 steps
    com = np.zeros((2, 256), np.uint8)
    step = np.zeros(2)
    for it in range(256):
        ent = RNG.random((2, 256)).astype(np.float32) + 1.0
        com, tok, step, n_new, done = oracle.eb_select(
            ent, am[:2], com, tok[:2], step, np.full(2, 0.5, np.float32), 1000)
        assert np.all(n_new == 1)
    assert np.all(done == 1) and np.all(com == 1)


def test_eb_monotone_in_gamma():
    ent, am, com, tok = _eb_rand(b=1)
    prev = None
    for g in np.linspace(0.0, 30.0, 40):
        c2, *_ = oracle.eb_select(ent, am, com, tok, np.zeros(1),
                                  np.array([g], np.float32), 256)
        if prev is not None:
            assert np.all(c2 >= prev)
        prev = c2


def test_eb_exhaustive_subsets_small_canvas():
    # n* is the largest number of uncommitted positions whose entropies can
    # sum to <= gamma (at least 1), and the chosen set is the smallest such
    # set in (entropy, position) order -- checked over all subsets
    for trial in range(40):
        c = 10
        ent = np.round(RNG.random((1, c)) * 4) / 4  # ties on purpose
        ent = ent.astype(np.float32)
        com = (RNG.random((1, c)) < 0.2).astype(np.uint8)
        if com.all():
            continue
        unc = [j for j in range(c) if com[0, j] == 0]
        gamma = float(np.float32(RNG.random() * 2.0))
        c2, *_ = oracle.eb_select(ent, np.zeros((1, c), int), com,
                                  np.zeros((1, c), int), np.zeros(1),
                                  np.array([gamma], np.float32), 256)
        chosen = sorted(j for j in unc if c2[0, j] == 1)
        best_n = 0
        for n in range(len(unc) + 1):
            if any(sum(float(ent[0, j]) for j in s) <= gamma
                   for s in itertools.combinations(unc, n)):
                best_n = n
        assert len(chosen) == max(1, best_n)
        key = lambda s: sorted((float(ent[0, j]), j) for j in s)  # noqa
        smallest = min(itertools.combinations(unc, len(chosen)), key=key)
        assert chosen == sorted(smallest)


def test_eb_finished_canvas_is_left_alone():
    ent, am, com, tok = _eb_rand(b=1)
    com[:] = 1
    c2, t2, s2, n_new, done = oracle.eb_select(
        ent, am, com, tok, np.array([7]), np.array([1.0], np.float32), 256)
    assert np.all(c2 == 1) and np.all(t2 == tok) and s2[0] == 7
    assert n_new[0] == 0 and done[0] == 1


# ----------------------------------------------------------------- full step

def _tiny_model(l_count=2, expert_dtype="bf16"):
    from block_discrete_diffusion_tok_amd import synth
    sh = synth.ModelShape(l_count, 32, 4, 2, 8, 6, 2, 16, 50,
                          expert_dtype=expert_dtype)
    w = synth.to_numpy_weights(synth.make_weights(sh, seed=3, gain_std=0.1))
    osh = oracle.Shapes(sh.n_layers, sh.hidden, sh.n_q_heads, sh.n_kv_heads,
                        sh.head_dim, sh.n_experts, sh.top_k, sh.expert_ffn,
                        sh.vocab, sh.rms_eps)
    return sh, osh, w


def _prefix(sh, p, b=1):
    from block_discrete_diffusion_tok_amd import synth
    out = []
    for r in range(b):
        k, v = synth.make_prefix_kv(sh, p, r, seed=3)
        out.append((k.float().numpy(), v.float().numpy()))
    return out


def test_step_with_zero_output_projections_is_embedding_head():
    sh, osh, w = _tiny_model()
    for lw in w["layers"]:
        lw["w_o"] = np.zeros_like(lw["w_o"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    tokens = RNG.integers(0, sh.vocab, (1, 12))
    committed = np.zeros((1, 12), np.uint8)
    committed[0, [2, 5]] = 1
    out = oracle.denoise_step(osh, w, tokens, committed, _prefix(sh, 4),
                              mirror=False, want_logits=True)
    rows = np.nonzero(committed[0] == 0)[0]
    emb = w["embed"].astype(np.float64)
    x = emb[tokens[0, rows]]
    xh = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + sh.rms_eps) * \
        w["final_norm"]
    np.testing.assert_allclose(out["logits"], xh @ emb.T, rtol=1e-12,
                               atol=1e-14)
    assert np.all(np.isnan(out["entropy"][0, [2, 5]]))


def test_step_is_permutation_equivariant_over_the_canvas():
    sh, osh, w = _tiny_model()
    tokens = RNG.integers(0, sh.vocab, (1, 16))
    committed = (RNG.random((1, 16)) < 0.3).astype(np.uint8)
    pre = _prefix(sh, 5)
    out = oracle.denoise_step(osh, w, tokens, committed, pre, mirror=False)
    perm = RNG.permutation(16)
    out_p = oracle.denoise_step(osh, w, tokens[:, perm], committed[:, perm],
                                pre, mirror=False)
    np.testing.assert_allclose(out_p["entropy"], out["entropy"][:, perm],
                               rtol=1e-10)
    np.testing.assert_array_equal(out_p["argmax"], out["argmax"][:, perm])


def test_step_batch_canvases_are_independent():
    sh, osh, w = _tiny_model(l_count=1)
    tokens = RNG.integers(0, sh.vocab, (2, 10))
    committed = np.zeros((2, 10), np.uint8)
    pre = _prefix(sh, 3, b=2)
    both = oracle.denoise_step(osh, w, tokens, committed, pre, mirror=True)
    for b in range(2):
        one = oracle.denoise_step(osh, w, tokens[b:b + 1], committed[b:b + 1],
                                  pre[b:b + 1], mirror=True)
        np.testing.assert_allclose(one["entropy"][0], both["entropy"][b],
                                   rtol=1e-12)


def test_commit_first_layer_kv_closed_form():
    sh, osh, w = _tiny_model()
    tokens = RNG.integers(0, sh.vocab, (1, 8))
    kv = oracle.commit_block(osh, w, tokens, _prefix(sh, 4), mirror=False)
    x = w["embed"][tokens[0]].astype(np.float64)
    lw = w["layers"][0]
    xh = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + sh.rms_eps) * \
        lw["attn_norm"]
    hd, hq, hkv = sh.head_dim, sh.n_q_heads, sh.n_kv_heads
    wk = lw["w_qkv"][hq * hd:(hq + hkv) * hd].astype(np.float64)
    k0 = (xh @ wk.T).reshape(8, hkv, hd).transpose(1, 0, 2)
    np.testing.assert_allclose(kv[0][0][0], k0, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("expert_dtype", ["bf16", "fp8_e4m3"])
def test_commit_causal_block_equals_sequential_single_token_encodes(
        expert_dtype):
    sh, osh, w = _tiny_model(l_count=3, expert_dtype=expert_dtype)
    n = 7
    tokens = RNG.integers(0, sh.vocab, (1, n))
    pre = _prefix(sh, 4)
    kv = oracle.commit_block(osh, w, tokens, pre, mirror=False)
    kb, vb = kv[0]
    k_cache, v_cache = pre[0]
    for i in range(n):
        got = []
        _layers_forward(osh, w, tokens[:, i:i + 1], [(k_cache, v_cache)],
                        False, False, None, kv_out=got)
        for li, (k1, v1) in enumerate(got):
            np.testing.assert_allclose(k1[:, 0], kb[li][:, i], rtol=1e-10,
                                       atol=1e-12)
            np.testing.assert_allclose(v1[:, 0], vb[li][:, i], rtol=1e-10,
                                       atol=1e-12)
        k_new = np.stack([k1 for k1, _ in got])
        v_new = np.stack([v1 for _, v1 in got])
        k_cache = np.concatenate([k_cache, k_new], axis=2)
        v_cache = np.concatenate([v_cache, v_new], axis=2)


def test_mirror_mode_changes_results_only_by_bf16_rounding_size():
    sh, osh, w = _tiny_model()
    tokens = RNG.integers(0, sh.vocab, (1, 16))
    committed = np.zeros((1, 16), np.uint8)
    pre = _prefix(sh, 5)
    a = oracle.denoise_step(osh, w, tokens, committed, pre, mirror=True,
                            want_logits=True)
    b = oracle.denoise_step(osh, w, tokens, committed, pre, mirror=False,
                            want_logits=True)
    err = np.max(np.abs(a["logits"] - b["logits"])) / np.max(
        np.abs(b["logits"]))
    assert 0 < err < 2e-2


def test_attention_scale_is_one_over_sqrt_head_dim():
    # D = 4, q = (1,1,1,1); key 1 = c (1,1,1,1) with c = ln(3)/2, so
    # q.k1 / sqrt(4) = 4c / 2 = ln 3 and the weights are 1/4, 3/4
    c = math.log(3.0) / 2.0
    q = np.ones((1, 1, 4))
    kc = np.array([[[0.0] * 4, [c] * 4]])
    vc = np.array([[[4.0] * 4, [0.0] * 4]])
    empty = np.zeros((1, 0, 4))
    o = oracle.canvas_attention(q, empty, empty, kc, vc)
    np.testing.assert_allclose(o[0, 0], [1.0] * 4, rtol=1e-14)
