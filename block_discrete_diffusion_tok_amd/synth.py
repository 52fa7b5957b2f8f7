"""Seeded synthetic inputs: weights, cached prefix K/V and canvas state.

This module holds no arithmetic of the method.  It only draws random numbers
(torch generators seeded per tensor name) and converts them to the storage
formats the engine consumes; the GPU path and the CPU oracle are both fed from
what it returns, so they see identical bytes.

Value recipe (the pages publish no weights; every input is synthetic):
  * matrices (embedding, Q/K/V/O projections, router, experts) ~ N(0, 0.02^2),
    stored as bfloat16 (round to nearest even of the float32 draw);
  * E4M3 expert weights: the same N(0, 0.02^2) draw quantised per output row,
    scale = max|row| / 448, code = RNE(w / scale) in OCP FP8 E4M3;
  * E4M3 LM head (lm_dtype "fp8_e4m3"): the bf16 embedding table quantised
    per vocabulary row the same way (the input lookup keeps the bf16 table);
  * E4M3 projections (proj_dtype "fp8_e4m3"): the bf16 Q/K/V and output
    projection matrices quantised per output row the same way;
  * RMSNorm gains 1 (or 1 + N(0, gain_std^2) when a test asks for it);
  * cached prefix K/V ~ N(0, 1) as bfloat16;
  * canvas tokens i.i.d. uniform over the vocabulary; a "masked" position is
    an uncommitted one, chosen by a seeded uniform permutation.
"""
import zlib
from dataclasses import dataclass

import torch

CANVAS = 256


@dataclass(frozen=True)
class ModelShape:
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
    expert_dtype: str = "bf16"  # "bf16" or "fp8_e4m3"
    canvas_len: int = CANVAS    # positions per canvas (128 or 256)
    n_shared_experts: int = 0   # 0 or 1 shared expert (the last expert group)
    act_dtype: str = "bf16"     # expert GEMM token rows: "bf16" or "fp8_e4m3"
    kv_dtype: str = "bf16"      # KV cache: "bf16" or "fp8_e4m3"
    lm_dtype: str = "bf16"      # LM head: "bf16" or "fp8_e4m3" (W8A8)
    proj_dtype: str = "bf16"    # Q/K/V and output projections (W8A8)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    prefix_len: int
    batch: int
    uncommitted: int          # uncommitted positions per canvas at the start
    gamma: float
    step_cap: int
    blocks: int = 1
    steps: int = 0            # fixed number of denoise steps (0: run to done)
    notes: str = ""


_GEMMA_LAYER = dict(hidden=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                    n_experts=128, top_k=8, expert_ffn=768, vocab=262144)
# FP8 serving: E4M3 weights and E4M3 rows in every dense product but the
# router (attention, norms and the cache stay bf16 / fp32)
_W8A8 = dict(expert_dtype="fp8_e4m3", act_dtype="fp8_e4m3",
             lm_dtype="fp8_e4m3", proj_dtype="fp8_e4m3")

WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_l1_h256_p512",
                 ModelShape(1, 256, 4, 2, 64, 16, 2, 512, 4096),
                 prefix_len=512, batch=1, uncommitted=256, gamma=0.5,
                 step_cap=256,
                 notes="single tiny layer; EB until every position is committed"),
        Workload("moe_layer_h2048_v262k_p2048",
                 ModelShape(1, **_GEMMA_LAYER),
                 prefix_len=2048, batch=1, uncommitted=128, gamma=1.0,
                 step_cap=256,
                 notes="one 128-expert top-8 layer plus the 262k-vocab LM head"),
        Workload("stack30_h2048_p4096",
                 ModelShape(30, **_GEMMA_LAYER),
                 prefix_len=4096, batch=1, uncommitted=256, gamma=1.0,
                 step_cap=64, blocks=4,
                 notes="30 layers, 4 consecutive blocks, step cap 64"),
        Workload("stack30_h2048_p131072",
                 ModelShape(30, **_GEMMA_LAYER),
                 prefix_len=131072, batch=1, uncommitted=256, gamma=1.0,
                 step_cap=256, steps=12,
                 notes="30 layers, 131072-token cached prefix, 12 steps"),
        Workload("stack30_fp8_b32_p2048",
                 ModelShape(30, **_GEMMA_LAYER, expert_dtype="fp8_e4m3"),
                 prefix_len=2048, batch=32, uncommitted=256, gamma=1.0,
                 step_cap=256,
                 notes="30 layers, E4M3 experts, 32 concurrent canvases"),
        Workload("stack30_kv8_h2048_p131072",
                 ModelShape(30, **_GEMMA_LAYER, kv_dtype="fp8_e4m3"),
                 prefix_len=131072, batch=1, uncommitted=256, gamma=1.0,
                 step_cap=256, steps=12,
                 notes="the 131072-token prefix in an E4M3 KV cache"),
        Workload("stack30_w8a8_b32_p2048",
                 ModelShape(30, **_GEMMA_LAYER, **_W8A8),
                 prefix_len=2048, batch=32, uncommitted=256, gamma=1.0,
                 step_cap=256,
                 notes="the 32-canvas batch in W8A8: E4M3 weights and rows "
                       "in the projections, the experts and the LM head"),
        Workload("stack30_w8a8_h2048_p4096",
                 ModelShape(30, **_GEMMA_LAYER, **_W8A8),
                 prefix_len=4096, batch=1, uncommitted=256, gamma=1.0,
                 step_cap=64, blocks=4,
                 notes="the batch-1 stack in W8A8: E4M3 weights and rows "
                       "in the projections, the experts and the LM head"),
    ]
}


def _seed(seed, name):
    return (int(seed) * 1_000_003 + zlib.crc32(name.encode())) % (2 ** 63)


def _gen(seed, name, device):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name))
    return g


def normal(shape, std, seed, name, device="cpu", dtype=torch.bfloat16):
    g = _gen(seed, name, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def quantize_e4m3_rows(w):
    """Per-output-row E4M3 codes and fp32 scales of a float tensor [..., rows,
    cols]: scale = max|row| / 448, code = RNE(w / scale)."""
    w = w.float()
    amax = w.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    scale = amax / 448.0
    q = (w / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.squeeze(-1).contiguous()


def make_weights(shape: ModelShape, seed=0, device="cpu", gain_std=0.0,
                 layers=None, masters=False):
    """Random-init weights in the engine's storage formats (see module doc).

    ``layers`` optionally restricts generation to a subset of layer indices
    (the others are None), e.g. for host copies of sampled layers.
    ``masters``: the matrices as their float32 draws, before the bfloat16
    rounding (bf16-expert shapes only); rounding them gives the default
    weights bit for bit."""
    s = shape
    if masters and (s.expert_dtype != "bf16" or s.proj_dtype != "bf16"):
        raise ValueError("float32 masters exist for bf16-weight shapes only")
    mdt = torch.float32 if masters else torch.bfloat16
    qkv_rows = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim

    def gain(name):
        if gain_std == 0.0:
            return torch.ones(s.hidden, dtype=torch.float32, device=device)
        return 1.0 + normal((s.hidden,), gain_std, seed, name, device,
                            torch.float32)

    w = {"embed": normal((s.vocab, s.hidden), 0.02, seed, "embed", device, mdt),
         "final_norm": gain("final_norm"), "layers": []}
    if s.lm_dtype != "bf16":
        # the E4M3 LM head: per-vocabulary-row codes of the bf16 table
        w["lm_head"], w["lm_head_scale"] = quantize_e4m3_rows(w["embed"])
    for li in range(s.n_layers):
        if layers is not None and li not in layers:
            w["layers"].append(None)
            continue
        p = f"layer{li}."
        lw = {
            "attn_norm": gain(p + "attn_norm"),
            "w_qkv": normal((qkv_rows, s.hidden), 0.02, seed, p + "w_qkv",
                            device, mdt),
            "w_o": normal((s.hidden, s.n_q_heads * s.head_dim), 0.02, seed,
                          p + "w_o", device, mdt),
            "ffn_norm": gain(p + "ffn_norm"),
            "w_router": normal((s.n_experts, s.hidden), 0.02, seed,
                               p + "w_router", device, mdt),
        }
        # the routed experts, then the shared expert (its own draw)
        eg = s.n_experts
        gu_shape = (eg, 2 * s.expert_ffn, s.hidden)
        dn_shape = (eg, s.hidden, s.expert_ffn)
        dt = mdt if s.expert_dtype == "bf16" else torch.float32
        gu = normal(gu_shape, 0.02, seed, p + "w_gate_up", device, dt)
        dn = normal(dn_shape, 0.02, seed, p + "w_down", device, dt)
        if s.n_shared_experts:
            gu = torch.cat([gu, normal((1,) + gu_shape[1:], 0.02, seed,
                                       p + "w_gate_up_shared", device, dt)])
            dn = torch.cat([dn, normal((1,) + dn_shape[1:], 0.02, seed,
                                       p + "w_down_shared", device, dt)])
        if s.expert_dtype == "bf16":
            lw["w_gate_up"], lw["w_down"] = gu, dn
            lw["gate_up_scale"] = None
            lw["down_scale"] = None
        else:
            lw["w_gate_up"], lw["gate_up_scale"] = quantize_e4m3_rows(gu)
            lw["w_down"], lw["down_scale"] = quantize_e4m3_rows(dn)
            del gu, dn
        if s.proj_dtype != "bf16":
            for k, sk in (("w_qkv", "qkv_scale"), ("w_o", "o_scale")):
                lw[k], lw[sk] = quantize_e4m3_rows(lw[k])
        w["layers"].append(lw)
    return w


def make_prefix_kv(shape: ModelShape, prefix_len, request, seed=0,
                   device="cpu", layers=None):
    """Cached K/V of one request's prompt, each [L, Hkv, P, D] bfloat16
    ~ N(0, 1).  ``layers`` restricts to a subset (returned in that order)."""
    s = shape
    ls = range(s.n_layers) if layers is None else layers
    ks, vs = [], []
    for li in ls:
        ks.append(normal((s.n_kv_heads, prefix_len, s.head_dim), 1.0, seed,
                         f"prefix_k.req{request}.layer{li}", device))
        vs.append(normal((s.n_kv_heads, prefix_len, s.head_dim), 1.0, seed,
                         f"prefix_v.req{request}.layer{li}", device))
    return torch.stack(ks), torch.stack(vs)


def make_canvas(shape: ModelShape, batch, uncommitted, seed=0, block=0):
    """Canvas state on the host (C = shape.canvas_len positions per canvas):
    tokens int32 [B, C] uniform over the vocab,
    committed uint8 [B, C] with exactly ``uncommitted`` zeros per canvas at
    seeded uniformly random positions, step int32 [B] zeros."""
    C = shape.canvas_len
    tokens = torch.empty((batch, C), dtype=torch.int32)
    committed = torch.ones((batch, C), dtype=torch.uint8)
    for b in range(batch):
        g = _gen(seed, f"canvas.block{block}.b{b}", "cpu")
        tokens[b] = torch.randint(0, shape.vocab, (C,), generator=g,
                                  dtype=torch.int64).to(torch.int32)
        pos = torch.randperm(C, generator=g)[:uncommitted]
        committed[b, pos] = 0
    return {"tokens": tokens, "committed": committed,
            "step": torch.zeros(batch, dtype=torch.int32)}


def make_entropy_inputs(batch, seed=0, low=0.0, high=2.0, ties=False):
    """Synthetic sampler inputs: entropy float32 [B, C] uniform in [low,
    high) (optionally quantised to a few levels so that ties occur), argmax
    int32 [B, C], committed uint8 [B, C] (about a quarter committed)."""
    g = _gen(seed, "eb_inputs", "cpu")
    ent = low + (high - low) * torch.rand((batch, CANVAS), generator=g)
    if ties:
        ent = torch.floor(ent * 4.0) / 4.0
    argmax = torch.randint(0, 1 << 20, (batch, CANVAS), generator=g,
                           dtype=torch.int64).to(torch.int32)
    committed = (torch.rand((batch, CANVAS), generator=g) < 0.25).to(
        torch.uint8)
    return ent.float(), argmax, committed


def to_numpy_weights(w):
    """Host numpy view of a weight dict for the oracle: bfloat16 tensors as
    float32 arrays (exact), E4M3 codes as uint8, scales as float32."""
    def cv(t):
        if t is None:
            return None
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy()

    out = {"embed": cv(w["embed"]), "final_norm": cv(w["final_norm"]),
           "layers": []}
    for k in ("lm_head", "lm_head_scale"):
        if w.get(k) is not None:
            out[k] = cv(w[k])
    for lw in w["layers"]:
        out["layers"].append(None if lw is None else
                             {k: cv(v) for k, v in lw.items()})
    return out
