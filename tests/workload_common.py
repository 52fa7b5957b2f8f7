"""Helpers for the parity tests at the larger workload shapes (not collected
by pytest): lazy host copies of device weights and prefixes for the oracle,
and the composition checks (the step's fused kernels against the single-op
entry points on the step's own state)."""
import numpy as np
import torch

from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import (DEV, MARGIN, TOL, cache_scales, log, np32, op_proj,
                        rel_err, routing_margin)


class HostLayers:
    """Sequence of per-layer host copies (numpy, exact values) of device layer
    weights, made when the oracle reaches the layer, so that only one layer's
    copy is alive at a time.  ``count`` truncates the stack to its first
    layers; ``stop(i)``, asked before layer i is handed out, ends the
    sequence there when it returns True (the oracle's layer loop stops)."""

    def __init__(self, layers, count=None, stop=None):
        self.layers = layers
        self.count = len(layers) if count is None else count
        self.stop = stop

    def __len__(self):
        return self.count

    def __getitem__(self, i):
        if not 0 <= i < self.count:
            raise IndexError(i)
        if self.stop is not None and self.stop(i):
            raise IndexError(i)
        return synth.to_numpy_weights({"embed": None, "final_norm": None,
                                       "layers": [self.layers[i]]})["layers"][0]


class HostPerLayer:
    """t[li] as a float32 host array, for a device tensor [L, ...]."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, li):
        return np32(self.t[li])


def host_model(w, count=None, stop=None):
    out = {"embed": np32(w["embed"]), "final_norm": np32(w["final_norm"]),
           "layers": HostLayers(w["layers"], count, stop)}
    for k in ("lm_head", "lm_head_scale"):
        if w.get(k) is not None:
            out[k] = np32(w[k])
    return out


def capture_buffers(shape, T, L, final=True):
    """Device buffers for every per-layer capture of a step over T rows."""
    cap = {
        "attn_out": torch.zeros((L, T, shape.n_q_heads * shape.head_dim),
                                dtype=torch.bfloat16, device=DEV),
        "moe_out": torch.zeros((L, T, shape.hidden), dtype=torch.float32,
                               device=DEV),
        "route_idx": torch.zeros((L, T, shape.top_k), dtype=torch.int32,
                                 device=DEV),
        "route_w": torch.zeros((L, T, shape.top_k), dtype=torch.float32,
                               device=DEV),
        "router_logits": torch.zeros((L, T, shape.n_experts),
                                     dtype=torch.float32, device=DEV),
    }
    if final:
        cap["final_xhat"] = torch.zeros((T, shape.hidden), dtype=torch.float32,
                                        device=DEV)
    return cap


def check_composition(eng, shape, w, tokens, req, plen, cap, tag, layers=None):
    """Every layer of a step (its captures) against the same layer computed
    by the single-op entry points (each compared with the oracle by the op
    tests), from the residual stream rebuilt out of the captures:
    x_0 = E[tokens], x_(l+1) = x_l + attn_out_l W_o^T + moe_out_l.  This
    checks, at the full depth and size, that each layer reads its own
    weights and cache rows and that the fused kernels of the step compute
    what the separate ops compute.  The residual is rebuilt with the step's
    own output-projection kernel and the same float32 additions, so agreement
    is expected to be exact; the bounds are TOL and MARGIN as for the
    oracle."""
    s = shape
    T = tokens.numel()
    H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
    qkv_n = (Hq + 2 * Hkv) * D
    n = len(req)
    layers = range(s.n_layers) if layers is None else layers
    kc_all, vc_all = eng.cache_view("k"), eng.cache_view("v")
    x = w["embed"][tokens.reshape(-1).long()].float()
    worst_att = worst_moe = 0.0
    flips = 0
    for li in range(s.n_layers):
        lw = eng.weights["layers"][li]
        o_cap = cap["attn_out"][li]
        if li in layers:
            xh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
            dg.op_rmsnorm(x, lw["attn_norm"], s.rms_eps, xh)
            qkv = torch.empty((T, qkv_n), dtype=torch.bfloat16, device=DEV)
            op_proj(xh, lw, "w_qkv", qkv, 0)
            o = torch.empty((T, Hq * D), dtype=torch.bfloat16, device=DEV)
            ks, vs = cache_scales(eng, li)
            dg.op_canvas_attention(qkv, n, T // n, Hq, Hkv, D, kc_all[li],
                                   vc_all[li], eng.max_requests,
                                   eng.max_kv_len, req, plen, False, 0, o,
                                   ks, vs)
            e_att = rel_err(np32(o), np32(o_cap))
        op_proj(o_cap, lw, "w_o", x, 2)   # the step's own kernel
        if li in layers:
            xh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
            dg.op_rmsnorm(x, lw["ffn_norm"], s.rms_eps, xh)
            y = torch.zeros((T, H), dtype=torch.float32, device=DEV)
            ridx = torch.empty((T, s.top_k), dtype=torch.int32, device=DEV)
            rw = torch.empty((T, s.top_k), dtype=torch.float32, device=DEV)
            cnt = torch.empty(s.n_experts, dtype=torch.int32, device=DEV)
            dg.op_moe(s, lw, xh, y, ridx, rw, cnt)
            g_idx = cap["route_idx"][li].cpu().numpy()
            diff = np.any(ridx.cpu().numpy() != g_idx, axis=1)
            marg = routing_margin(np32(cap["router_logits"][li]), s.top_k)
            assert np.all(marg[diff] < MARGIN), \
                f"{tag} layer {li}: step and ops route differently"
            e_moe = rel_err(np32(y)[~diff], np32(cap["moe_out"][li])[~diff])
            flips += int(diff.sum())
            worst_att, worst_moe = max(worst_att, e_att), max(worst_moe, e_moe)
            assert e_att < TOL and e_moe < TOL, \
                f"{tag} layer {li}: attn {e_att:.2e} moe {e_moe:.2e}"
        x = x + cap["moe_out"][li]
    log(f"  {tag} composition over {len(layers)} layers: worst attn "
        f"{worst_att:.2e}, moe {worst_moe:.2e}, low-margin routing "
        f"differences {flips}")
    return x


def check_commit_composition(eng, shape, w, tokens, req, plen, tag, C=256):
    """The K/V rows dg_commit_block appended (cache rows [plen, plen + 256)
    of every layer) against the same causal encode run through the
    single-op entry points from the same tokens: embedding, then per layer
    rmsnorm, Q/K/V projection (whose K/V slices must equal the appended
    rows), causal attention, output projection, rmsnorm and MoE, the
    residual carried by the ops themselves (the MoE sum is added once, as
    the step's un-permute adds it)."""
    s = shape
    n = len(req)
    T = n * C
    H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
    qkv_n = (Hq + 2 * Hkv) * D
    kc_all, vc_all = eng.cache_view("k"), eng.cache_view("v")
    x = w["embed"][tokens.reshape(-1).long()].float()
    worst = 0.0
    for li in range(s.n_layers):
        lw = eng.weights["layers"][li]
        xh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        dg.op_rmsnorm(x, lw["attn_norm"], s.rms_eps, xh)
        qkv = torch.empty((T, qkv_n), dtype=torch.bfloat16, device=DEV)
        op_proj(xh, lw, "w_qkv", qkv, 0)
        for b in range(n):
            rows = slice(b * C, (b + 1) * C)
            # after the request's earlier canvases of the batch
            j = 0
            while b - j - 1 >= 0 and req[b - j - 1] == req[b]:
                j += 1
            p = plen[b] + j * C
            k_op = qkv[rows, Hq * D:(Hq + Hkv) * D].reshape(C, Hkv, D).transpose(0, 1)
            v_op = qkv[rows, (Hq + Hkv) * D:].reshape(C, Hkv, D).transpose(0, 1)
            if eng.kv8:
                # an E4M3 cache: the appended codes and scales are those of
                # the ops' K / V rows quantised, bit for bit
                ks, vs = cache_scales(eng, li)
                for cache, scl, rows_op in ((kc_all, ks, k_op), (vc_all, vs, v_op)):
                    r = rows_op.reshape(-1, D).contiguous()
                    q8 = torch.empty(r.shape, dtype=torch.uint8, device=DEV)
                    sc = torch.empty(r.shape[0], dtype=torch.float32, device=DEV)
                    dg.op_quantize_rows(r, q8, None, sc)
                    assert torch.equal(cache[li, req[b], :, p:p + C].reshape(-1, D), q8)
                    assert torch.equal(scl[req[b], :, p:p + C].reshape(-1), sc)
                continue
            ek = rel_err(np32(kc_all[li, req[b], :, p:p + C]), np32(k_op))
            ev = rel_err(np32(vc_all[li, req[b], :, p:p + C]), np32(v_op))
            worst = max(worst, ek, ev)
            assert ek < TOL and ev < TOL, \
                f"{tag} commit layer {li} canvas {b}: K {ek:.2e} V {ev:.2e}"
        if li == s.n_layers - 1:
            break
        o = torch.empty((T, Hq * D), dtype=torch.bfloat16, device=DEV)
        ks, vs = cache_scales(eng, li)
        dg.op_canvas_attention(qkv, n, C, Hq, Hkv, D, kc_all[li], vc_all[li],
                               eng.max_requests, eng.max_kv_len, req, plen,
                               True, 0, o, ks, vs)
        op_proj(o, lw, "w_o", x, 2)
        dg.op_rmsnorm(x, lw["ffn_norm"], s.rms_eps, xh)
        y = torch.empty((T, H), dtype=torch.float32, device=DEV)
        dg.op_moe(s, lw, xh, y)
        x = x + y
    log(f"  {tag} commit composition over {s.n_layers} layers: worst K/V "
        f"rel err {worst:.2e}")
