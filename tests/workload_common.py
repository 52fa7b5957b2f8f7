"""Helpers for the parity tests at the larger workload shapes (not collected
by pytest): lazy host copies of device weights and prefixes for the oracle,
and the layer-by-layer comparison of the step captures."""
import numpy as np
import torch

from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, MARGIN, TOL, log, np32, rel_err, routing_margin


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
    return {"embed": np32(w["embed"]), "final_norm": np32(w["final_norm"]),
            "layers": HostLayers(w["layers"], count, stop)}


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


class ChainChecker:
    """Layer-by-layer comparison of the device captures (rows ``grow``) with
    the oracle's capture ``cap_o`` of the same layers, from the same seeded
    inputs, done while the oracle runs: pass it as the ``stop`` hook of
    HostLayers.

    Attention output, router logits and MoE output within TOL (max relative
    error per tensor); routing bit-exact except where the oracle's margin is
    below MARGIN.  A token routed differently carries a different residual
    from then on, and through attention every later row depends on it, so
    the comparison (and the oracle) ends with the first layer that has such
    a token, its MoE output compared on the other rows."""

    def __init__(self, shape, cap, cap_o, grow, tag):
        self.shape, self.cap, self.cap_o, self.tag = shape, cap, cap_o, tag
        self.gi = torch.as_tensor(np.asarray(grow), device=DEV,
                                  dtype=torch.long)
        self.checked = 0
        self.flipped = False

    def __call__(self, i):
        self.finish()
        return self.flipped

    def finish(self):
        while not self.flipped and self.checked < len(self.cap_o):
            self._check(self.checked)
            self.checked += 1
        return self.checked

    def _check(self, li):
        c, cap, gi = self.cap_o[li], self.cap, self.gi
        att = np32(cap["attn_out"][li].index_select(0, gi))
        moe = np32(cap["moe_out"][li].index_select(0, gi))
        rl = np32(cap["router_logits"][li].index_select(0, gi))
        idx = cap["route_idx"][li].index_select(0, gi).cpu().numpy()
        e_att = rel_err(att, c["attn"])
        e_rl = rel_err(rl, c["router_logits"])
        diff = np.any(idx != c["idx"], axis=1)
        marg = routing_margin(c["router_logits"], self.shape.top_k)
        e_moe = rel_err(moe[~diff], c["moe"][~diff])
        log(f"  {self.tag} layer {li}: attn {e_att:.2e} router {e_rl:.2e} "
            f"moe {e_moe:.2e}; routing differences {int(diff.sum())} at "
            f"relative margins {np.sort(marg[diff]).tolist()}")
        assert np.all(marg[diff] < MARGIN), \
            f"{self.tag} layer {li}: routing differs at a clear margin"
        assert e_att < TOL and e_rl < TOL and e_moe < TOL
        if diff.any():
            self.flipped = True
            log(f"  {self.tag}: low-margin routing difference in layer {li}; "
                "the later layers are checked by composition")


def check_composition(eng, shape, w, tokens, req, plen, cap, tag, layers=None):
    """Every layer of a step (its captures) against the same layer computed
    by the single-op entry points (each compared with the oracle by the op
    tests), from the residual stream rebuilt out of the captures:
    x_0 = E[tokens], x_(l+1) = x_l + attn_out_l W_o^T + moe_out_l.  This
    checks, at the full depth and size, that each layer reads its own
    weights and cache rows and that the fused kernels of the step compute
    what the separate ops compute.  Agreement is to rounding (the rebuilt
    residual is a float32 sum in another order), so the bounds are TOL and
    MARGIN as for the oracle."""
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
        lw = w["layers"][li]
        o_cap = cap["attn_out"][li]
        if li in layers:
            xh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
            dg.op_rmsnorm(x, lw["attn_norm"], s.rms_eps, xh)
            qkv = torch.empty((T, qkv_n), dtype=torch.bfloat16, device=DEV)
            dg.op_linear(xh, lw["w_qkv"], qkv, 0)
            o = torch.empty((T, Hq * D), dtype=torch.bfloat16, device=DEV)
            dg.op_canvas_attention(qkv, n, 256, Hq, Hkv, D, kc_all[li],
                                   vc_all[li], eng.max_requests,
                                   eng.max_kv_len, req, plen, False, 0, o)
            e_att = rel_err(np32(o), np32(o_cap))
        x = x + o_cap.float() @ lw["w_o"].float().t()
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
