"""The oracle's model: one denoising step, the entropy-bounded sampler and the
block commit, each written as its plain definition in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Readings taken where the pages are silent (all pages: "DiffusionGemma
Technical Report" write-up, "diffusiongemma" model card):

R1  Layer internals are not given (the write-up only says the architecture is
    that of Gemma 4).  Pre-norm residual block: x += Attn(RMSNorm(x));
    x += MoE(RMSNorm(x)); RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g.
    Attention scale 1/sqrt(D).  No positional encoding, no soft-cap, no
    QK-norm, no sliding window, no shared expert, no self-conditioning MLP,
    no embedding scale; the LM head is tied to the embedding.
R2  Query head h reads KV head floor(h / G), G = Hq / Hkv (grouped-query
    attention, consecutive query heads share a KV head).
R3  Every canvas position attends to all cached prefix keys of its own request
    and to all 256 canvas keys, committed or not (write-up Figure 4 stage 2;
    model card "Model Overview").  The commit pass is causal inside the block
    (key j visible to query i iff j <= i), all prefix keys visible (write-up
    Figure 4 stage 3: the clean canvas goes through the causal encoder).
R4  Router: logits r = xhat W_r^T; the k experts with the largest logits are
    selected, ties going to the lower expert id; gate weights are the softmax
    over the k selected logits.  Experts are SwiGLU: W_d (silu(W_g x) * W_u x).
R5  The entropy of a position is -sum_v p_v ln p_v in nats over the full
    vocabulary softmax at temperature 1; it is clamped at 0.  The token taken
    for a position is the argmax of its logits, lowest id on ties.
R6  Entropy-bounded selection over the uncommitted positions U: sort by
    (entropy, position) ascending; C_n is the fp64 running sum of the first n
    entropies; n* = max(1, max{n : C_n <= gamma}) (inclusive); when this step
    is the last one the step budget allows (step + 1 >= cap) n* = |U|.  The
    first n* positions are committed with their argmax token.
R7  Uncommitted positions that are not selected take the step's argmax token
    as well ("refine"), committed ones are frozen; with refine off they keep
    their current token.  The canvas is finished once U is empty.
R8  Precision: the GPU stores GEMM operands in bfloat16 and accumulates in
    fp32.  With ``mirror=True`` the oracle rounds to bfloat16 exactly the
    activations the GPU stores as bfloat16 (norm outputs, Q/K/V, attention
    output, SwiGLU output) and otherwise computes in fp64, so that integer
    decisions are taken on the same operand values.  ``mirror=False`` keeps
    every activation in fp64.
"""
from dataclasses import dataclass

import numpy as np

from .numerics import round_bf16, decode_e4m3

CANVAS = 256


@dataclass(frozen=True)
class Shapes:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_ffn: int
    vocab: int
    rms_eps: float = 1e-6


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _bf(x, mirror):
    return round_bf16(x) if mirror else x


def expert_matrix(w, scale, e):
    """Weights of expert e as fp64.  ``w`` is either a float array
    [E, rows, cols] holding the exact values, or uint8 E4M3 codes with a
    per-output-row fp32 ``scale`` [E, rows] (the stored value times the
    scale is the weight)."""
    if scale is None:
        return _f64(w[e])
    return decode_e4m3(w[e]) * _f64(scale[e])[:, None]


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis (reading R1)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(g)


def canvas_attention(q, k_prefix, v_prefix, k_canvas, v_canvas, causal=False,
                     q_pos=None):
    """Scaled dot-product attention of one canvas (readings R2, R3).

    q        [Hq, n, D]   queries (n canvas positions, ``q_pos`` gives their
                          positions in the canvas; default 0..n-1)
    k_prefix [Hkv, P, D]  cached keys of this request (P may be 0)
    v_prefix [Hkv, P, D]
    k_canvas [Hkv, C, D]  keys / values of the canvas positions
    v_canvas [Hkv, C, D]
    causal   canvas key j visible to the query at position i iff j <= i

    Returns o [Hq, n, D]: for each head and query,
    o = sum_j softmax_j(q . k_j / sqrt(D)) v_j over the visible keys, with the
    full score row materialised and normalised the textbook way.
    """
    q = _f64(q)
    hq, n, d = q.shape
    hkv = k_canvas.shape[0]
    group = hq // hkv
    p_len = k_prefix.shape[1]
    c_len = k_canvas.shape[1]
    if q_pos is None:
        q_pos = np.arange(n)
    q_pos = np.asarray(q_pos)
    out = np.zeros((hq, n, d))
    for h in range(hq):
        g = h // group
        keys = np.concatenate([_f64(k_prefix[g]), _f64(k_canvas[g])], axis=0)
        vals = np.concatenate([_f64(v_prefix[g]), _f64(v_canvas[g])], axis=0)
        s = (q[h] @ keys.T) / np.sqrt(d)
        if causal:
            canvas_j = np.arange(c_len)[None, :]
            hidden = canvas_j > q_pos[:, None]
            s[:, p_len:][hidden] = -np.inf
        s_max = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - s_max)
        p = e / np.sum(e, axis=1, keepdims=True)
        out[h] = p @ vals
    return out


def router_topk(logits, k):
    """Top-k routing (reading R4).  logits [T, E] -> idx [T, k] (int64, in
    rank order: largest logit first, lower id first among equal logits) and
    w [T, k] = softmax over the selected logits."""
    logits = _f64(logits)
    t_count, _ = logits.shape
    idx = np.zeros((t_count, k), dtype=np.int64)
    w = np.zeros((t_count, k))
    for t in range(t_count):
        # stable sort of the negated logits keeps lower ids first on ties
        order = np.argsort(-logits[t], kind="stable")[:k]
        sel = logits[t, order]
        e = np.exp(sel - np.max(sel))
        idx[t] = order
        w[t] = e / np.sum(e)
    return idx, w


def silu(v):
    return v / (1.0 + np.exp(-v))


def moe_mixture(xhat, idx, w, w_gate_up, w_down, gate_up_scale=None,
                down_scale=None, mirror=True, experts=None):
    """Gate-weighted mixture of SwiGLU experts for each token (reading R4):

        y_t = sum_j w[t, j] * W_d,e (silu(W_g,e xhat_t) * W_u,e xhat_t),
        e = idx[t, j],

    where expert e's gate/up matrix holds the F gate rows first, then the F up
    rows.  Each expert is evaluated on the tokens that selected it (a plain
    per-row product; no token is computed twice and no row depends on
    another).  ``experts`` optionally supplies fp64 (W_gu, W_d) per expert id
    to avoid decoding them again.
    """
    xhat = _f64(xhat)
    t_count, hidden = xhat.shape
    out = np.zeros((t_count, hidden))
    for e in np.unique(idx):
        tt, jj = np.nonzero(idx == e)
        if experts is not None:
            wgu, wd = experts[int(e)]
        else:
            wgu = expert_matrix(w_gate_up, gate_up_scale, int(e))
            wd = expert_matrix(w_down, down_scale, int(e))
        f = wd.shape[1]
        gate = xhat[tt] @ wgu[:f].T
        up = xhat[tt] @ wgu[f:].T
        act = _bf(silu(gate) * up, mirror)
        y = act @ wd.T
        out[tt] += w[tt, jj][:, None] * y
    return out


def lm_head_stats(xhat, embed, want_logits=False):
    """Vocabulary softmax statistics per row (reading R5), tied LM head.

    z = xhat E^T;  lse = log sum_v exp(z_v);  p = exp(z - lse);
    entropy = -sum_v p_v ln p_v (terms with p_v = 0 contribute 0), clamped
    at 0;  argmax = lowest v with the largest z_v.
    """
    z = _f64(xhat) @ _f64(embed).T
    z_max = np.max(z, axis=1, keepdims=True)
    lse = z_max[:, 0] + np.log(np.sum(np.exp(z - z_max), axis=1))
    p = np.exp(z - lse[:, None])
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    entropy = np.maximum(-np.sum(plogp, axis=1), 0.0)
    argmax = np.argmax(z, axis=1)  # first occurrence of the maximum
    out = {"lse": lse, "entropy": entropy, "argmax": argmax}
    if want_logits:
        out["logits"] = z
    return out


def eb_select(entropy, argmax, committed, tokens, step, gamma, step_cap,
              refine=True):
    """Entropy-bounded selection for a batch of canvases (readings R6, R7).

    entropy [B, C] float32 (rows of committed positions ignored),
    argmax [B, C], committed [B, C] 0/1, tokens [B, C], step [B],
    gamma [B] float32, step_cap >= 1.

    Returns new (committed, tokens, step, n_new, done) without modifying the
    inputs.  A canvas with no uncommitted position is left unchanged and
    reported done with n_new = 0.
    """
    committed = np.array(committed, dtype=np.uint8, copy=True)
    tokens = np.array(tokens, dtype=np.int64, copy=True)
    step = np.array(step, dtype=np.int64, copy=True)
    b_count, c_len = committed.shape
    n_new = np.zeros(b_count, dtype=np.int64)
    done = np.zeros(b_count, dtype=np.uint8)
    for b in range(b_count):
        unc = [j for j in range(c_len) if committed[b, j] == 0]
        if not unc:
            done[b] = 1
            continue
        ent = [float(np.float32(entropy[b, j])) for j in unc]
        order = [j for _, j in sorted(zip(ent, unc))]  # (entropy, position)
        limit = float(np.float32(gamma[b]))
        total = 0.0
        n = 0
        for j in order:
            total += float(np.float32(entropy[b, j]))
            if total <= limit:
                n += 1
            else:
                break
        n = max(1, n)
        if step[b] + 1 >= step_cap:
            n = len(unc)
        for j in order[:n]:
            committed[b, j] = 1
            tokens[b, j] = argmax[b, j]
        if refine:
            for j in order[n:]:
                tokens[b, j] = argmax[b, j]
        step[b] += 1
        n_new[b] = n
        done[b] = 1 if n == len(unc) else 0
    return committed, tokens, step, n_new, done


def _split_qkv(qkv, sh):
    hq, hkv, d = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    rows = qkv.shape[0]
    q = qkv[:, : hq * d].reshape(rows, hq, d).transpose(1, 0, 2)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(rows, hkv, d).transpose(1, 0, 2)
    v = qkv[:, (hq + hkv) * d:].reshape(rows, hkv, d).transpose(1, 0, 2)
    return q, k, v


def _layers_forward(sh, weights, tokens, prefix, mirror, causal, capture,
                    kv_out=None):
    """Embedding plus the L residual layers over B canvases.

    tokens [B, C]; prefix: list over canvases of (K, V), each [L, Hkv, P_b, D].
    With ``kv_out`` (a list) the per-layer canvas K/V [Hkv, B*C, D] are
    appended to it and the last layer stops after its K/V projection.
    """
    b_count, c_len = tokens.shape
    embed = weights["embed"]
    x = _f64(embed[np.asarray(tokens).reshape(-1)])  # x_t = E[tok_t]
    for li, lw in enumerate(weights["layers"]):
        xh = _bf(rmsnorm(x, lw["attn_norm"], sh.rms_eps), mirror)
        qkv = _bf(xh @ _f64(lw["w_qkv"]).T, mirror)
        q, k, v = _split_qkv(qkv, sh)
        if kv_out is not None:
            kv_out.append((k, v))
            if li == len(weights["layers"]) - 1:
                break
        o = np.zeros((b_count * c_len, sh.n_q_heads * sh.head_dim))
        for b in range(b_count):
            rows = slice(b * c_len, (b + 1) * c_len)
            kp, vp = prefix[b]
            ob = canvas_attention(q[:, rows], kp[li], vp[li], k[:, rows],
                                  v[:, rows], causal=causal)
            o[rows] = ob.transpose(1, 0, 2).reshape(c_len, -1)
        o = _bf(o, mirror)
        x = x + o @ _f64(lw["w_o"]).T
        xh = _bf(rmsnorm(x, lw["ffn_norm"], sh.rms_eps), mirror)
        r = xh @ _f64(lw["w_router"]).T
        idx, w = router_topk(r, sh.top_k)
        y = moe_mixture(xh, idx, w, lw["w_gate_up"], lw["w_down"],
                        lw.get("gate_up_scale"), lw.get("down_scale"),
                        mirror=mirror)
        x = x + y
        if capture is not None:
            capture.append({"attn": o, "router_logits": r, "idx": idx,
                            "w": w, "moe": y, "x": x.copy()})
    return x


def denoise_step(sh, weights, tokens, committed, prefix, mirror=True,
                 want_logits=False, capture=None):
    """One denoising forward over B canvases (write-up Figure 4, stage 2).

    weights: {"embed" [V,H], "final_norm" [H], "layers": [per-layer dict with
    attn_norm, w_qkv [(Hq+2Hkv)D, H], w_o [H, Hq D], ffn_norm, w_router [E, H],
    w_gate_up [E, 2F, H], w_down [E, H, F], optional gate_up_scale [E, 2F] and
    down_scale [E, H] when the expert weights are E4M3 codes]}.

    Returns per-canvas arrays [B, C]: entropy, lse, argmax for the
    uncommitted positions (NaN / -1 at committed ones), plus "rows" (the
    flattened indices of the uncommitted positions, in order) and, with
    ``want_logits``, logits [n_rows, V].
    """
    tokens = np.asarray(tokens)
    committed = np.asarray(committed)
    b_count, c_len = tokens.shape
    x = _layers_forward(sh, weights, tokens, prefix, mirror, False, capture)
    rows = np.nonzero(committed.reshape(-1) == 0)[0]
    xf = _bf(rmsnorm(x[rows], weights["final_norm"], sh.rms_eps), mirror)
    st = lm_head_stats(xf, weights["embed"], want_logits=want_logits)
    ent = np.full(b_count * c_len, np.nan)
    lse = np.full(b_count * c_len, np.nan)
    am = np.full(b_count * c_len, -1, dtype=np.int64)
    ent[rows] = st["entropy"]
    lse[rows] = st["lse"]
    am[rows] = st["argmax"]
    out = {"entropy": ent.reshape(b_count, c_len),
           "lse": lse.reshape(b_count, c_len),
           "argmax": am.reshape(b_count, c_len), "rows": rows,
           "final_xhat": xf}
    if want_logits:
        out["logits"] = st["logits"]
    return out


def commit_block(sh, weights, tokens, prefix, mirror=True):
    """Encode-and-append of finished canvases (write-up Figure 4, stage 3).

    The canvas tokens are run causally through the layers (reading R3) and the
    K/V each layer produces for them are what gets appended to the request's
    cache at rows [P_b, P_b + C).  Returns a list over canvases of (K, V),
    each [L, Hkv, C, D].
    """
    tokens = np.asarray(tokens)
    b_count, c_len = tokens.shape
    kv = []
    _layers_forward(sh, weights, tokens, prefix, mirror, True, None,
                    kv_out=kv)
    out = []
    for b in range(b_count):
        rows = slice(b * c_len, (b + 1) * c_len)
        k_all = np.stack([k[:, rows] for k, _ in kv])
        v_all = np.stack([v[:, rows] for _, v in kv])
        out.append((k_all, v_all))
    return out
