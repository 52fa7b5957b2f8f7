"""Lockstep parity at full depth (not collected by pytest).

The oracle runs its own layer chain from the seeded inputs (it never takes a
value the device computed).  As it finishes each layer, the single-op entry
points of the library are fed that layer's oracle inputs -- the residual
entering the layer, its normed rows, its Q/K/V, its attention output, the
residual after the attention, the FFN's normed rows -- and each op's output
is compared with the oracle's next value:

    rmsnorm(x_in)            vs  xh_attn
    linear(xh_attn, W_qkv)   vs  qkv
    attention(qkv, cache)    vs  attn
    x_in + linear(attn, W_o) vs  x_mid
    rmsnorm(x_mid)           vs  xh_ffn
    linear(xh_ffn, W_r)      vs  router logits
    moe(xh_ffn)              vs  routing (bit-exact) and MoE output

then, after the last layer, the final norm, the LM head statistics on the
oracle's final normed rows and the EB selection on the oracle's entropies.
Both sides see identical bf16 operands, so decisions are compared bit for
bit except where the oracle's ABSOLUTE decision margin is below 1e-3; the
positions exempted only by the older relative reading are logged.

The ops run at the batch shape of the step under test: the oracle's
canvases are placed at their rows of the full batch, the other rows hold
seeded filler, so the kernels (and their split counts, MoE path and LM-head
path) are the ones the step uses.  Every row is independent of the others
in these ops except through attention, which reads only its own canvas.
"""
import numpy as np
import torch

from block_discrete_diffusion_tok_amd import dg
from gpu_common import (DEV, MARGIN, TOL, TOL_ROW_FP8_ACT, cache_scales,
                        lm8_decision_bound, op_proj,
                        fp8_act, log,
                        np32, rel_err, row_err,
                        routing_margin, top2_margin)


def _t(a, dtype):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.float32,
                           device=DEV).to(dtype)


class Lockstep:
    """Per-layer op-vs-oracle comparison, driven as the oracle's layer hook
    (see HostLayers' ``stop``): when the oracle asks for layer i, every
    captured layer < i is compared and its capture released.

    shape: model shape; eng: the engine (packed weights, KV caches);
    w: device weights; n_full: canvases of the step's batch; req / plen:
    request slot and prefix length of each of them; sel: the indices (into
    the batch) of the canvases the oracle runs; causal: commit mode."""

    def __init__(self, shape, eng, w, n_full, req, plen, sel, cap_o, tag,
                 causal=False, kv_o=None, seed=0, C=256):
        self.s, self.eng, self.w, self.tag = shape, eng, w, tag
        self.n_full, self.req, self.plen = n_full, list(req), list(plen)
        self.sel, self.cap_o, self.causal = list(sel), cap_o, causal
        self.kv_o = kv_o
        self.C = C                    # positions per canvas
        self.T = n_full * C
        self.rows = np.concatenate([np.arange(b * C, (b + 1) * C)
                                    for b in self.sel])
        self.gi = torch.as_tensor(self.rows, device=DEV, dtype=torch.long)
        self.checked = 0
        self.x_last = None            # oracle residual after the last layer
        self.worst = {}
        self.exempt_abs = 0
        self.exempt_rel_only = 0
        g = torch.Generator(device=DEV)
        g.manual_seed(1000 + seed)
        self.gen = g

    # -- helpers
    def _full(self, a, cols, dtype, scale=1.0):
        """[T, cols] device tensor: the oracle rows at their batch rows, the
        other rows seeded filler N(0, scale^2)."""
        out = torch.randn((self.T, cols), generator=self.gen, device=DEV,
                          dtype=torch.float32).mul_(scale).to(dtype)
        out[self.gi] = _t(a, dtype)
        return out

    def _mine(self, t):
        return np32(t.index_select(0, self.gi))

    def _note(self, key, e):
        self.worst[key] = max(self.worst.get(key, 0.0), e)

    def _cmp(self, key, g, o, li, row_tol=TOL):
        e, er = rel_err(g, o), row_err(g, o)
        self._note(key, e)
        self._note(key + " (per row)", er)
        assert e < TOL and er < row_tol, \
            f"{self.tag} layer {li} {key}: rel err {e:.2e}, per-row {er:.2e}"
        return e

    def __call__(self, i):
        while self.checked < i and self.checked < len(self.cap_o):
            self._layer(self.checked)
            self.checked += 1
        return False

    def finish(self):
        self(len(self.cap_o))
        return self.checked

    # -- one layer
    def _layer(self, li):
        s, c = self.s, self.cap_o[li]
        lw = self.eng.weights["layers"][li]
        H, D, Hq, Hkv = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads
        qkv_n = (Hq + 2 * Hkv) * D
        T = self.T
        # attention norm
        x_in = self._full(c["x_in"], H, torch.float32)
        xh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        dg.op_rmsnorm(x_in, lw["attn_norm"], s.rms_eps, xh)
        self._cmp("attn norm", self._mine(xh), c["xh_attn"], li)
        # Q/K/V projection of the oracle's normed rows
        xh_o = self._full(c["xh_attn"], H, torch.bfloat16)
        qkv = torch.empty((T, qkv_n), dtype=torch.bfloat16, device=DEV)
        op_proj(xh_o, lw, "w_qkv", qkv, 0)
        self._cmp("qkv", self._mine(qkv), c["qkv"], li)
        if self.kv_o is not None:     # commit: the appended K / V rows
            k_o, v_o = self.kv_o[li]
            g = self._mine(qkv)
            k_g = g[:, Hq * D:(Hq + Hkv) * D].reshape(-1, Hkv, D).transpose(1, 0, 2)
            v_g = g[:, (Hq + Hkv) * D:].reshape(-1, Hkv, D).transpose(1, 0, 2)
            self._cmp("commit K", k_g, k_o, li)
            self._cmp("commit V", v_g, v_o, li)
        if "attn" not in c:           # commit: last layer stops at its K/V
            self.cap_o[li] = None
            return
        # attention over the cache and the oracle's Q/K/V
        qkv_o = self._full(c["qkv"], qkv_n, torch.bfloat16)
        o = torch.empty((T, Hq * D), dtype=torch.bfloat16, device=DEV)
        kc, vc = self.eng.cache_view("k"), self.eng.cache_view("v")
        ks, vs = cache_scales(self.eng, li)
        dg.op_canvas_attention(qkv_o, self.n_full, self.C, Hq, Hkv, D, kc[li],
                               vc[li], self.eng.max_requests,
                               self.eng.max_kv_len, self.req, self.plen,
                               self.causal, 0, o, ks, vs)
        self._cmp("attention", self._mine(o), c["attn"], li)
        # output projection added into the oracle's residual
        x = x_in.clone()
        op_proj(self._full(c["attn"], Hq * D, torch.bfloat16), lw, "w_o", x, 2)
        self._cmp("x after attention", self._mine(x), c["x_mid"], li)
        # FFN norm
        x_mid = self._full(c["x_mid"], H, torch.float32)
        dg.op_rmsnorm(x_mid, lw["ffn_norm"], s.rms_eps, xh)
        self._cmp("ffn norm", self._mine(xh), c["xh_ffn"], li)
        # router logits and the MoE on the oracle's normed rows
        xf = self._full(c["xh_ffn"], H, torch.bfloat16)
        rl = torch.empty((T, s.n_experts), dtype=torch.float32, device=DEV)
        dg.op_linear(xf, lw["w_router"], rl, 1)
        self._cmp("router logits", self._mine(rl), c["router_logits"], li)
        y = torch.empty((T, H), dtype=torch.float32, device=DEV)
        ridx = torch.empty((T, s.top_k), dtype=torch.int32, device=DEV)
        rw = torch.empty((T, s.top_k), dtype=torch.float32, device=DEV)
        dg.op_moe(s, lw, xf, y, ridx, rw)
        g_idx = ridx.index_select(0, self.gi).cpu().numpy()
        diff = np.any(g_idx != c["idx"], axis=1)
        m_abs = routing_margin(c["router_logits"], s.top_k, relative=False)
        m_rel = routing_margin(c["router_logits"], s.top_k, relative=True)
        assert np.all(m_abs[diff] < MARGIN), \
            f"{self.tag} layer {li}: routing differs at absolute margins " \
            f"{np.sort(m_abs[diff & (m_abs >= MARGIN)])[:8].tolist()}"
        self.exempt_abs += int(diff.sum())
        self.exempt_rel_only += int(((m_rel < MARGIN) & (m_abs >= MARGIN)).sum())
        ok = ~diff
        self._cmp("moe", self._mine(y)[ok], c["moe"][ok], li,
                  TOL_ROW_FP8_ACT if fp8_act(s) else TOL)
        if li % 5 == 0 or li == len(self.cap_o) - 1:
            log(f"  {self.tag} layer {li}: worst so far " + ", ".join(
                f"{k} {v:.2e}" for k, v in self.worst.items()
                if "per row" not in k) +
                f"; routing differences {int(diff.sum())} (all below the "
                f"absolute margin)")
        self.x_last = c["x"]
        self.cap_o[li] = None

    def report(self):
        log(f"  {self.tag}: {self.checked} layer(s) compared in lockstep; worst "
            + ", ".join(f"{k} {v:.2e}" for k, v in self.worst.items())
            + f"; routing differences below the absolute margin: "
            f"{self.exempt_abs}; positions exempt only under a relative "
            f"reading of the margin (diagnostic): {self.exempt_rel_only}")


def lockstep_head(shape, eng, w, ref, x_last, committed, n_full, sel, tag,
                  seed=0, lm8_host=None):
    """Final norm, LM head statistics and argmax on the oracle's final rows.
    x_last: oracle residual after the last layer [rows of sel canvases, H];
    ref: the oracle's denoise_step output for the sel canvases.  Returns the
    device entropy / argmax of the oracle's rows.  An E4M3 head (reading
    R15) runs its own entry point; lm8_host = its row-major (codes, scales)
    on the host, for the decision bound of its FP8 sums."""
    s = shape
    H = s.hidden
    rows_o = ref["rows"]                        # uncommitted rows, oracle order
    sel = list(sel)
    # the same rows at their places in the full batch
    C = committed.shape[1]
    glob = np.array([sel[r // C] * C + r % C for r in rows_o])
    # final norm of the oracle's residual rows
    xin = torch.as_tensor(x_last[rows_o], dtype=torch.float32, device=DEV)
    xf = torch.empty((len(rows_o), H), dtype=torch.bfloat16, device=DEV)
    dg.op_rmsnorm(xin, w["final_norm"], s.rms_eps, xf)
    e_n, e_nr = rel_err(np32(xf), ref["final_xhat"]), row_err(np32(xf), ref["final_xhat"])
    # LM head over as many rows as the step feeds it: the oracle's final
    # rows at their compacted positions among seeded filler rows
    com = committed.reshape(-1)
    m_full = int((com == 0).sum())
    pos = np.cumsum(com == 0) - 1               # compacted index of each row
    g = torch.Generator(device=DEV)
    g.manual_seed(2000 + seed)
    xh = torch.randn((m_full, H), generator=g, device=DEV).to(torch.bfloat16)
    idx = torch.as_tensor(pos[glob], device=DEV, dtype=torch.long)
    xh[idx] = torch.as_tensor(ref["final_xhat"], dtype=torch.float32,
                              device=DEV).to(torch.bfloat16)
    ent = torch.empty(m_full, dtype=torch.float32, device=DEV)
    lse = torch.empty_like(ent)
    am = torch.empty(m_full, dtype=torch.int32, device=DEV)
    if eng.weights.get("lm_head") is not None:
        dg.op_lmhead_entropy_e4m3(xh, eng.weights["lm_head"],
                                  eng.weights["lm_head_scale"], ent, lse, am)
    else:
        dg.op_lmhead_entropy(xh, eng.weights["embed"], ent, lse, am)
    g_ent = ent[idx].cpu().numpy()
    g_lse = lse[idx].cpu().numpy()
    g_am = am[idx].cpu().numpy()
    o_ent = ref["entropy"].reshape(-1)[rows_o]
    o_lse = ref["lse"].reshape(-1)[rows_o]
    o_am = ref["argmax"].reshape(-1)[rows_o]
    e_ent, e_lse = rel_err(g_ent, o_ent), rel_err(g_lse, o_lse)
    e_ent_el = float(np.max(np.abs(g_ent - o_ent) /
                            np.maximum(np.abs(o_ent), 1e-3 * np.max(np.abs(o_ent)))))
    n_diff = int((g_am != o_am).sum())
    log(f"  {tag} head: final norm {e_n:.2e} (per row {e_nr:.2e}), entropy "
        f"{e_ent:.2e} (elementwise {e_ent_el:.2e}), lse {e_lse:.2e}; "
        f"{len(rows_o)} rows through the LM head of {m_full}; argmax "
        f"differences {n_diff}")
    assert e_n < TOL and e_nr < TOL and e_ent < TOL and e_lse < TOL
    assert e_ent_el < TOL
    if n_diff:
        # margins from the oracle's logits when it kept them
        assert "logits" in ref, "argmax differs and no oracle logits to judge"
        marg = top2_margin(ref["logits"], relative=False)
        bound = np.full(len(marg), MARGIN)
        if eng.weights.get("lm_head") is not None:
            assert lm8_host is not None, "the E4M3 head's bound needs its codes"
            bound = lm8_decision_bound(ref["final_xhat"], ref["logits"], *lm8_host)
        d = g_am != o_am
        assert np.all(marg[d] < bound[d]), \
            "argmax differs at a clear absolute margin"
    return g_ent, g_am


def lockstep_eb(ref_ent, ref_am, committed, tokens, step, gamma, step_cap, tag):
    """EB selection on the oracle's entropies and argmax: the device op and
    the oracle's eb_select from identical fp32 inputs, bit for bit (both take
    the same (entropy, position) order; the EB margin is reported)."""
    import oracle
    B = committed.shape[0]
    ent32 = np.where(np.isnan(ref_ent), 0.0, ref_ent).astype(np.float32)
    am = np.where(ref_am < 0, 0, ref_am).astype(np.int32)
    d = {"ent": torch.as_tensor(ent32, device=DEV),
         "am": torch.as_tensor(am, device=DEV),
         "com": torch.as_tensor(committed.astype(np.uint8), device=DEV),
         "tok": torch.as_tensor(tokens.astype(np.int32), device=DEV),
         "step": torch.as_tensor(step.astype(np.int32), device=DEV)}
    gam = torch.full((B,), gamma, dtype=torch.float32, device=DEV)
    n_new = torch.zeros(B, dtype=torch.int32, device=DEV)
    done = torch.zeros(B, dtype=torch.uint8, device=DEV)
    dg.op_eb_select(d["ent"], d["am"], d["com"], d["tok"], d["step"], gam,
                    step_cap, True, n_new, done)
    o_com, o_tok, o_step, o_new, o_done = oracle.eb_select(
        ent32, am, committed, tokens, step, np.full(B, gamma, np.float32),
        step_cap)
    np.testing.assert_array_equal(d["com"].cpu().numpy(), o_com)
    np.testing.assert_array_equal(d["tok"].cpu().numpy(), o_tok)
    np.testing.assert_array_equal(d["step"].cpu().numpy(), o_step)
    np.testing.assert_array_equal(n_new.cpu().numpy(), o_new)
    np.testing.assert_array_equal(done.cpu().numpy(), o_done)
    log(f"  {tag} EB: committed sets equal bit for bit, n_new "
        f"{o_new.tolist()[:8]}")
