"""The oracle's model: one denoising step, the entropy-bounded sampler and the
block commit, each written as its plain definition in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Readings taken where the pages are silent (all pages: "DiffusionGemma
Technical Report" write-up, "diffusiongemma" model card):

R1  Layer internals are not given (the write-up only says the architecture is
    that of Gemma 4).  Pre-norm residual block: x += Attn(RMSNorm(x));
    x += MoE(RMSNorm(x)); RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g.
    Attention scale 1/sqrt(D).  No positional encoding, no soft-cap, no
    QK-norm, no sliding window, no shared expert (unless the shape has one,
    R10), no self-conditioning MLP,
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
R9  Several canvases of one request (multi-canvas sampling, model card
    feature list "block-autoregressive multi-canvas sampling"; write-up
    Table 7 "number of canvases"): they sit next to each other in the batch,
    in block order, and canvas j attends to the request's cached prefix,
    then to every position of the request's canvases before it (earlier
    blocks are fully visible, later ones not: block-causal), then to its own
    canvas (bidirectional, or causal in the commit pass).
R10 "+ 1 shared" expert (write-up Table 1): a SwiGLU expert of the same
    width that every token uses next to its routed experts, its output
    added with weight 1 (not gated by the router, which scores the routed
    experts only); stored as the last expert group.
R11 Temperature sampling with annealing (write-up Figure 9: "higher N
    yields milder temperature annealing"; Figure 10: "temperature tau_t = 1"
    without annealing): at a canvas's step t (steps already taken in its
    block) the temperature is tau_t = tau_0 (1 - t / N) for a step budget
    N > 0, tau_0 for N = 0, clamped at 0.  With tau_t > 0 the position's
    distribution is softmax(z / tau_t): its entropy is what EB ranks, and
    its token is a draw from it by the Gumbel-max rule, argmax_v
    (z_v / tau_t + g_v) with g_v = -ln(-ln u_v), u_v from Philox4x32-10
    (counter (v div 4, position, t, canvas), key = the 64-bit seed; output
    v mod 4; 24-bit uniforms).  With tau_t = 0 the distribution is the
    point mass on the argmax: entropy 0, token = argmax, and lse reports
    the raw logits' log-sum-exp.  Sampling off (the default) is the greedy
    step of R5.
R12 AR mode (write-up "What they did": the weights still decode left to
    right; model card "Model Overview"): a step takes one token per
    sequence at the next position, runs it through the layers as a canvas of
    one position in the commit pass (causal: it sees the cached prefix and
    itself, no positional term, reading S9), appends the K/V it makes and
    reads the next token's statistics off its final-normed row.  Greedy
    (argmax) decoding only.
R13 FP8 activations (write-up Table 3 and Figure 11 captions: served in
    FP8; the pages fix no scaling): with E4M3 experts and ``act_fp8`` the
    expert products take every row they multiply (a token's FFN-norm row
    for gate/up, a pair's SwiGLU row for down) as OCP E4M3 codes with one
    scale per row: a = max |row|, s = a / 448, r = 448 / a (both 1 for a
    zero row), codes = E4M3(row * r) to nearest, ties to even, saturating,
    each step in fp32; the product is s_row s_w[n] sum_k q_row[k] q_w[n][k].  Per-row dynamic
    scales are the plainest reading for activations that change every
    step.
R14 FP8 KV cache (write-up Table 3 caption, FP8 serving; the cache is
    what long prompts move): with ``kv_fp8`` every cached key or value row
    (one KV head, one position: D values) is stored as E4M3 codes with one
    scale, quantised as in R13 when it enters the cache, and attention
    reads bf16(fp32(code value x scale)) for it.  Keys and values of the
    canvases in the same call (the canvas, the request's earlier canvases
    of the batch) are used as computed; they enter the cache quantised when
    committed.
R15 FP8 LM head (the same captions: the model is served in FP8): with
    ``lm_fp8`` the LM head reads the tied embedding as E4M3 codes with one
    fp32 scale per vocabulary row (the row's max |value| / 448, as the
    expert weights are stored) and takes each final-normed row as E4M3
    codes with its row scale, quantised as in R13; the logit of vocabulary
    id v is s_row s_v sum_k q_row[k] q_v[k].  The embedding lookup at the
    input keeps the bf16 table.
R16 FP8 projections (the same captions): with ``proj_fp8`` the Q/K/V and
    output projections read E4M3 weight codes with one fp32 scale per
    output row (as the experts) and take their input rows (the attention
    norm's rows, the attention output's rows) as E4M3 codes with one scale
    per row, quantised as in R13: out[r, n] = s_r s_n sum_k q_r[k] q_n[k].
    The router keeps bf16 weights and rows: its logits decide the routing,
    and E4M3 rows would move them by whole E4M3 steps (the pages give no
    detail; it is the plainer reading of an FP8 model whose gates keep
    their precision).
R8  Precision: the GPU stores GEMM operands in bfloat16 and accumulates in
    fp32.  With ``mirror=True`` the oracle rounds to bfloat16 exactly the
    activations the GPU stores as bfloat16 (norm outputs, Q/K/V, attention
    output, SwiGLU output) and otherwise computes in fp64, so that integer
    decisions are taken on the same operand values.  ``mirror=False`` keeps
    every activation in fp64.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
from threadpoolctl import threadpool_limits

from .numerics import (round_bf16, decode_e4m3, quantize_rows_e4m3,
                       kv_cache_values)
from .philox import philox4x32_10, uniform24

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
    n_shared_experts: int = 0   # reading R10
    act_fp8: bool = False       # reading R13
    kv_fp8: bool = False        # reading R14
    lm_fp8: bool = False        # reading R15
    proj_fp8: bool = False      # reading R16


# The oracle's real type: fp64, so that every dot product, softmax sum and
# residual addition is a tighter reference than the GPU's fp32
# accumulation.  The ORACLE_ACC32 reading (environment variable, or the
# accumulate_in context) computes the same definitions with fp32 arrays
# instead, so that the pure-fp32 result can be reported beside it.  The
# entropy-bounded sampler's running sum stays fp64 in both (reading R6).
_ACC = [np.float32 if os.environ.get("ORACLE_ACC32") == "1" else np.float64]


class accumulate_in:
    """Context: compute the oracle's arithmetic in the given numpy float
    type (np.float64 by default, np.float32 for the ORACLE_ACC32 reading)."""

    def __init__(self, dtype):
        self.dtype = dtype

    def __enter__(self):
        self.prev = _ACC[0]
        _ACC[0] = self.dtype
        return self

    def __exit__(self, *exc):
        _ACC[0] = self.prev
        return False


def _real(a):
    return np.asarray(a, dtype=_ACC[0])


def _bf(x, mirror):
    return _real(round_bf16(x)) if mirror else x


def _map_independent(fn, items):
    """[fn(i) for i in items] with the items spread over a pool of threads.

    Only used for items whose computations do not depend on each other
    (attention heads, experts); each item's arithmetic is exactly that of a
    serial loop, and the callers combine the results in item order, so the
    results are the same bits as a serial loop's.  BLAS threads are shared
    out among the workers."""
    items = list(items)
    cores = os.cpu_count() or 1
    workers = max(1, min(len(items), cores))
    if workers == 1:
        return [fn(i) for i in items]
    with threadpool_limits(max(1, cores // workers)):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))


def expert_matrix(w, scale, e):
    """Weights of expert e as fp64.  ``w`` is either a float array
    [E, rows, cols] holding the exact values, or uint8 E4M3 codes with a
    per-output-row fp32 ``scale`` [E, rows] (the stored value times the
    scale is the weight)."""
    if scale is None:
        return _real(w[e])
    return decode_e4m3(w[e]) * _real(scale[e])[:, None]


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis (reading R1)."""
    x = _real(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _real(g)


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
    q = _real(q)
    hq, n, d = q.shape
    hkv = k_canvas.shape[0]
    group = hq // hkv
    p_len = k_prefix.shape[1]
    c_len = k_canvas.shape[1]
    if q_pos is None:
        q_pos = np.arange(n)
    q_pos = np.asarray(q_pos)
    def head(h):
        g = h // group
        keys = np.concatenate([_real(k_prefix[g]), _real(k_canvas[g])], axis=0)
        vals = np.concatenate([_real(v_prefix[g]), _real(v_canvas[g])], axis=0)
        s = (q[h] @ keys.T) / np.sqrt(d)
        if causal:
            canvas_j = np.arange(c_len)[None, :]
            hidden = canvas_j > q_pos[:, None]
            s[:, p_len:][hidden] = -np.inf
        s_max = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - s_max)
        p = e / np.sum(e, axis=1, keepdims=True)
        return p @ vals

    out = np.stack(_map_independent(head, range(hq)))
    return out


def router_topk(logits, k):
    """Top-k routing (reading R4).  logits [T, E] -> idx [T, k] (int64, in
    rank order: largest logit first, lower id first among equal logits) and
    w [T, k] = softmax over the selected logits."""
    logits = _real(logits)
    t_count, _ = logits.shape
    idx = np.zeros((t_count, k), dtype=np.int64)
    w = np.zeros((t_count, k), dtype=_ACC[0])
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
                down_scale=None, mirror=True, experts=None, act_fp8=False):
    """Gate-weighted mixture of SwiGLU experts for each token (reading R4):

        y_t = sum_j w[t, j] * W_d,e (silu(W_g,e xhat_t) * W_u,e xhat_t),
        e = idx[t, j],

    where expert e's gate/up matrix holds the F gate rows first, then the F up
    rows.  Each expert is evaluated on the tokens that selected it (a plain
    per-row product; no token is computed twice and no row depends on
    another).  ``experts`` optionally supplies fp64 (W_gu, W_d) per expert id
    to avoid decoding them again.

    With ``act_fp8`` (reading R13; E4M3 expert weights) each token's row
    and each pair's SwiGLU row enter their product as E4M3 codes with one
    scale per row: W q_x is formed from the codes' values and then scaled
    by s_x and the weight rows' scales.
    """
    xhat = _real(xhat)
    t_count, hidden = xhat.shape
    out = np.zeros((t_count, hidden), dtype=_ACC[0])
    if act_fp8:
        qx, sx = quantize_rows_e4m3(xhat)
        xq = _real(decode_e4m3(qx))
        sx = _real(sx)

        def expert8(e):
            tt, jj = np.nonzero(idx == e)
            cgu = _real(decode_e4m3(w_gate_up[e]))
            sgu = _real(gate_up_scale[e])
            cd = _real(decode_e4m3(w_down[e]))
            sd = _real(down_scale[e])
            f = cd.shape[1]
            gate = (xq[tt] @ cgu[:f].T) * sx[tt][:, None] * sgu[:f][None, :]
            up = (xq[tt] @ cgu[f:].T) * sx[tt][:, None] * sgu[f:][None, :]
            act = _bf(silu(gate) * up, mirror)
            qa, sa = quantize_rows_e4m3(act)
            y = (_real(decode_e4m3(qa)) @ cd.T) * _real(sa)[:, None] * sd[None, :]
            return tt, w[tt, jj][:, None] * y

        for tt, contrib in _map_independent(expert8, np.unique(idx)):
            out[tt] += contrib
        return out

    def expert(e):
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
        return tt, w[tt, jj][:, None] * y

    # every expert's products are independent; they are added in expert order
    for tt, contrib in _map_independent(expert, np.unique(idx)):
        out[tt] += contrib
    return out


def linear_w8a8(x, codes, scale):
    """The product of E4M3 rows with E4M3 weight rows (readings R13, R15,
    R16): each row of x is quantised as in R13 (codes q_r, scale s_r);
    codes [N, K] uint8 and scale [N] are the weight rows;
    out[r, n] = s_r scale[n] sum_k q_r[k] q_n[k]."""
    qx, sx = quantize_rows_e4m3(_real(x))
    z = _real(decode_e4m3(qx)) @ _real(decode_e4m3(codes)).T
    return z * _real(sx)[:, None] * _real(scale)[None, :]


def lm_logits(xhat, embed, lm8=None):
    """Logits of the tied LM head: z = xhat E^T.  With ``lm8`` = (codes
    [V, H] uint8, scale [V]) the E4M3 head of reading R15:
    linear_w8a8(xhat, codes, scale)."""
    if lm8 is None:
        return _real(xhat) @ _real(embed).T
    return linear_w8a8(xhat, *lm8)


def projection(sh, x, lw, name):
    """x W^T for the layer matrix ``name`` ("w_qkv" or "w_o"): bf16
    weights, or under reading R16 E4M3 codes with the per-row scales
    lw["qkv_scale"] / lw["o_scale"] and E4M3 rows of x."""
    if sh.proj_fp8:
        sc = lw["qkv_scale" if name == "w_qkv" else "o_scale"]
        return linear_w8a8(x, lw[name], sc)
    return _real(x) @ _real(lw[name]).T


def lm_head_stats(xhat, embed, want_logits=False, lm8=None):
    """Vocabulary softmax statistics per row (reading R5), tied LM head.

    z = xhat E^T (or the E4M3 head of reading R15 with ``lm8``);
    lse = log sum_v exp(z_v);  p = exp(z - lse);
    entropy = -sum_v p_v ln p_v (terms with p_v = 0 contribute 0), clamped
    at 0;  argmax = lowest v with the largest z_v.
    """
    z = lm_logits(xhat, embed, lm8)
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


def temperature(tau0, budget, step):
    """tau_t of reading R11 for the steps already taken in the block."""
    step = np.asarray(step, dtype=np.float64)
    if budget > 0:
        return np.maximum(tau0 * (1.0 - step / budget), 0.0)
    return np.maximum(np.full_like(step, tau0), 0.0)


def gumbel(v, pos, step, canvas, seed):
    """g_v = -ln(-ln u_v) for vocabulary ids v (array) of one position
    (reading R11)."""
    v = np.asarray(v, dtype=np.int64)
    out = philox4x32_10(v // 4, pos, step, canvas, seed & 0xFFFFFFFF,
                        (seed >> 32) & 0xFFFFFFFF)
    x = np.choose(v % 4, out)
    u = uniform24(x)
    return -np.log(-np.log(u))


def lm_head_sample(xhat, embed, tau, ctr, seed, lm8=None):
    """Vocabulary statistics at the rows' temperatures and the sampled
    tokens (reading R11).  xhat [M, H]; tau [M]; ctr [M, 3] = (position,
    step, canvas) of each row; seed: 64-bit key; ``lm8`` as in lm_logits.
    Returns dict with lse, entropy (of softmax(z / tau)), argmax (of z) and
    sample per row."""
    z = lm_logits(xhat, embed, lm8)
    m_rows, v_count = z.shape
    lse = np.zeros(m_rows)
    ent = np.zeros(m_rows)
    sample = np.zeros(m_rows, dtype=np.int64)
    argmax = np.argmax(z, axis=1)
    vids = np.arange(v_count)
    for r in range(m_rows):
        t = float(tau[r])
        if t <= 0.0:
            st = lm_head_stats(xhat[r:r + 1], embed, lm8=lm8)
            lse[r] = st["lse"][0]
            ent[r] = 0.0
            sample[r] = argmax[r]
            continue
        zs = z[r] / t
        zm = np.max(zs)
        lse[r] = zm + np.log(np.sum(np.exp(zs - zm)))
        p = np.exp(zs - lse[r])
        with np.errstate(divide="ignore", invalid="ignore"):
            plogp = np.where(p > 0, p * np.log(p), 0.0)
        ent[r] = max(-np.sum(plogp), 0.0)
        score = zs + gumbel(vids, int(ctr[r][0]), int(ctr[r][1]),
                            int(ctr[r][2]), seed)
        sample[r] = int(np.argmax(score))
    return {"lse": lse, "entropy": ent, "argmax": argmax, "sample": sample,
            "logits": z}


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


def moe_layer(sh, lw, xh, mirror=True):
    """The FFN of one layer on normed rows xh [T, H] (readings R4, R10):
    router logits r = xh W_r^T over the routed experts, top-k routing, and
    the mixture of the routed experts plus, with a shared expert, that
    expert (the last group of the expert matrices) with weight 1.
    Returns (r, idx [T, k], w [T, k], y [T, H])."""
    r = _real(xh) @ _real(lw["w_router"]).T
    idx, w = router_topk(r, sh.top_k)
    idx_all, w_all = idx, w
    if sh.n_shared_experts:
        t_count = idx.shape[0]
        idx_all = np.concatenate(
            [idx, np.full((t_count, 1), sh.n_experts, dtype=idx.dtype)], axis=1)
        w_all = np.concatenate([w, np.ones((t_count, 1))], axis=1)
    y = moe_mixture(xh, idx_all, w_all, lw["w_gate_up"], lw["w_down"],
                    lw.get("gate_up_scale"), lw.get("down_scale"),
                    mirror=mirror, act_fp8=sh.act_fp8)
    return r, idx, w, y


def _split_qkv(qkv, sh):
    hq, hkv, d = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    rows = qkv.shape[0]
    q = qkv[:, : hq * d].reshape(rows, hq, d).transpose(1, 0, 2)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(rows, hkv, d).transpose(1, 0, 2)
    v = qkv[:, (hq + hkv) * d:].reshape(rows, hkv, d).transpose(1, 0, 2)
    return q, k, v


def _earlier_canvases(request, b_count):
    """For each canvas, the batch indices of the earlier canvases of its
    request (reading R9; canvases of a request are contiguous)."""
    if request is None:
        return [[] for _ in range(b_count)]
    request = list(request)
    out = []
    for b in range(b_count):
        first = b
        while first > 0 and request[first - 1] == request[b]:
            first -= 1
        assert request[b] not in request[:first], \
            "canvases of one request must be contiguous"
        out.append(list(range(first, b)))
    return out


def _layers_forward(sh, weights, tokens, prefix, mirror, causal, capture,
                    kv_out=None, request=None, full=False):
    """Embedding plus the L residual layers over B canvases.

    tokens [B, C]; prefix: list over canvases of (K, V), each [L, Hkv, P_b, D].
    request: optional [B] request ids; canvases sharing one see the earlier
    ones (reading R9).
    With ``kv_out`` (a list) the per-layer canvas K/V [Hkv, B*C, D] are
    appended to it and, unless ``full``, the last layer stops after its K/V
    projection.
    """
    b_count, c_len = tokens.shape
    earlier = _earlier_canvases(request, b_count)
    embed = weights["embed"]
    x = _real(embed[np.asarray(tokens).reshape(-1)])  # x_t = E[tok_t]
    for li, lw in enumerate(weights["layers"]):
        x_in = x
        xh = _bf(rmsnorm(x, lw["attn_norm"], sh.rms_eps), mirror)
        qkv = _bf(projection(sh, xh, lw, "w_qkv"), mirror)
        q, k, v = _split_qkv(qkv, sh)
        if kv_out is not None:
            kv_out.append((k, v))
            if li == len(weights["layers"]) - 1 and not full:
                if capture is not None:   # what the last layer computed
                    capture.append({"x_in": x_in, "xh_attn": xh, "qkv": qkv})
                break
        o = np.zeros((b_count * c_len, sh.n_q_heads * sh.head_dim),
                     dtype=_ACC[0])
        for b in range(b_count):
            rows = slice(b * c_len, (b + 1) * c_len)
            kp, vp = prefix[b]
            kp, vp = kp[li], vp[li]
            if sh.kv_fp8:   # reading R14: the cache holds E4M3 rows
                kp, vp = kv_cache_values(kp), kv_cache_values(vp)
            kp, vp = _real(kp), _real(vp)
            if earlier[b]:   # the request's earlier canvases follow its prefix
                sl = [slice(e * c_len, (e + 1) * c_len) for e in earlier[b]]
                kp = np.concatenate([kp] + [k[:, r] for r in sl], axis=1)
                vp = np.concatenate([vp] + [v[:, r] for r in sl], axis=1)
            ob = canvas_attention(q[:, rows], kp, vp, k[:, rows],
                                  v[:, rows], causal=causal)
            o[rows] = ob.transpose(1, 0, 2).reshape(c_len, -1)
        o = _bf(o, mirror)
        x = x + projection(sh, o, lw, "w_o")
        x_mid = x
        xh_attn = xh
        xh = _bf(rmsnorm(x, lw["ffn_norm"], sh.rms_eps), mirror)
        r, idx, w, y = moe_layer(sh, lw, xh, mirror)
        x = x + y
        if capture is not None:
            # every value the layer computed, in order: its input residual,
            # attention norm, Q/K/V, attention output, residual after the
            # attention, FFN norm, router logits, routing, MoE output and
            # the residual it leaves
            capture.append({"x_in": x_in, "xh_attn": xh_attn, "qkv": qkv,
                            "attn": o, "x_mid": x_mid, "xh_ffn": xh,
                            "router_logits": r, "idx": idx, "w": w,
                            "moe": y, "x": x.copy()})
    return x


def _lm8(sh, weights):
    """The E4M3 LM head's (codes, scales) under reading R15, else None."""
    if not sh.lm_fp8:
        return None
    return weights["lm_head"], weights["lm_head_scale"]


def denoise_step(sh, weights, tokens, committed, prefix, mirror=True,
                 want_logits=False, capture=None, request=None, sampling=None,
                 step=None):
    """One denoising forward over B canvases (write-up Figure 4, stage 2).

    weights: {"embed" [V,H], "final_norm" [H], "layers": [per-layer dict with
    attn_norm, w_qkv [(Hq+2Hkv)D, H], w_o [H, Hq D], ffn_norm, w_router [E, H],
    w_gate_up [E, 2F, H], w_down [E, H, F], optional gate_up_scale [E, 2F] and
    down_scale [E, H] when the expert weights are E4M3 codes; with
    ``sh.proj_fp8`` w_qkv and w_o as E4M3 codes with qkv_scale
    [(Hq+2Hkv)D] and o_scale [H]]}, and with ``sh.lm_fp8`` "lm_head" [V, H]
    E4M3 codes and "lm_head_scale" [V].

    Returns per-canvas arrays [B, C]: entropy, lse, argmax for the
    uncommitted positions (NaN / -1 at committed ones), plus "rows" (the
    flattened indices of the uncommitted positions, in order) and, with
    ``want_logits``, logits [n_rows, V].
    """
    tokens = np.asarray(tokens)
    committed = np.asarray(committed)
    b_count, c_len = tokens.shape
    x = _layers_forward(sh, weights, tokens, prefix, mirror, False, capture,
                        request=request)
    rows = np.nonzero(committed.reshape(-1) == 0)[0]
    xf = _bf(rmsnorm(x[rows], weights["final_norm"], sh.rms_eps), mirror)
    lm8 = _lm8(sh, weights)
    if sampling is None:
        st = lm_head_stats(xf, weights["embed"], want_logits=want_logits,
                           lm8=lm8)
    else:   # reading R11: (tau_0, budget N, seed); step [B] of each canvas
        tau0, budget, seed = sampling
        steps = np.asarray(step, dtype=np.int64)
        canvas = rows // c_len
        tau = temperature(tau0, budget, steps[canvas])
        ctr = np.stack([rows % c_len, steps[canvas], canvas], axis=1)
        st = lm_head_sample(xf, weights["embed"], tau, ctr, seed, lm8=lm8)
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
    if sampling is not None:
        smp = np.full(b_count * c_len, -1, dtype=np.int64)
        smp[rows] = st["sample"]
        out["sample"] = smp.reshape(b_count, c_len)
    if want_logits:
        out["logits"] = st["logits"]
    return out


def ar_step(sh, weights, tokens, prefix, mirror=True, request=None,
            want_logits=False, capture=None):
    """One left-to-right decoding step of the same weights (AR mode, reading
    R12): tokens [n] is the token at position P_b of each sequence b (its
    cached prefix holds positions 0..P_b-1); it attends causally to the
    prefix and itself (a canvas of one position in the commit pass), the K/V
    each layer makes for it are what the cache appends at row P_b, and the
    final-normed row's logits give the next-token statistics.

    Returns {"entropy", "lse", "argmax"} [n] (plus "logits" [n, V] with
    ``want_logits``) and "kv": a list over sequences of (K, V), each
    [L, Hkv, 1, D]."""
    tokens = np.asarray(tokens).reshape(-1, 1)
    kv = []
    x = _layers_forward(sh, weights, tokens, prefix, mirror, True, capture,
                        kv_out=kv, request=request, full=True)
    xf = _bf(rmsnorm(x, weights["final_norm"], sh.rms_eps), mirror)
    st = lm_head_stats(xf, weights["embed"], want_logits=want_logits,
                       lm8=_lm8(sh, weights))
    out = {"entropy": st["entropy"], "lse": st["lse"], "argmax": st["argmax"],
           "final_xhat": xf}
    if want_logits:
        out["logits"] = st["logits"]
    out["kv"] = [(np.stack([k[:, b:b + 1] for k, _ in kv]),
                  np.stack([v[:, b:b + 1] for _, v in kv]))
                 for b in range(tokens.shape[0])]
    return out


def commit_block(sh, weights, tokens, prefix, mirror=True, request=None):
    """Encode-and-append of finished canvases (write-up Figure 4, stage 3).

    The canvas tokens are run causally through the layers (reading R3) and the
    K/V each layer produces for them are what gets appended to the request's
    cache at rows [P_b, P_b + C) (after the request's earlier canvases of the
    batch, reading R9, when ``request`` groups canvases).  Returns a list
    over canvases of (K, V), each [L, Hkv, C, D].
    """
    tokens = np.asarray(tokens)
    b_count, c_len = tokens.shape
    kv = []
    _layers_forward(sh, weights, tokens, prefix, mirror, True, None,
                    kv_out=kv, request=request)
    out = []
    for b in range(b_count):
        rows = slice(b * c_len, (b + 1) * c_len)
        k_all = np.stack([k[:, rows] for k, _ in kv])
        v_all = np.stack([v[:, rows] for _, v in kv])
        out.append((k_all, v_all))
    return out
