"""The C-ABI library loads, exports every function its headers declare, and
rejects bad arguments on the host before any launch.  CPU only: no call here
reaches a kernel."""
import ctypes
import os
import re

import pytest

from block_discrete_diffusion_tok_amd import dg, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in ("dg.h", "dg_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(dg_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    L = dg.lib()
    declared = _declared_functions()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(L, name), name
    assert declared == set(dg.EXPORTS)


def _desc(**kw):
    s = synth.WORKLOADS["moe_layer_h2048_v262k_p2048"].shape
    d = dg.model_desc(s)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_size_queries():
    L = dg.lib()
    d = _desc()
    kv = L.dg_kv_cache_bytes(ctypes.byref(d), 2, 4096)
    assert kv == 1 * 2 * 8 * 4096 * 128 * 2
    ws1 = L.dg_workspace_bytes(ctypes.byref(d), 1)
    ws32 = L.dg_workspace_bytes(ctypes.byref(d), 32)
    assert 0 < ws1 < ws32
    assert L.dg_workspace_bytes(ctypes.byref(d), 0) == 0
    assert L.dg_workspace_bytes(ctypes.byref(d), 65) == 0
    assert L.dg_workspace_bytes(ctypes.byref(_desc(head_dim=96)), 1) == 0
    assert L.dg_workspace_bytes(ctypes.byref(_desc(n_q_heads=12)), 1) == 0
    assert L.dg_workspace_bytes(ctypes.byref(_desc(top_k=17)), 1) == 0
    assert L.dg_workspace_bytes(ctypes.byref(_desc(n_experts=300)), 1) == 0
    assert L.dg_op_moe_workspace_bytes(ctypes.byref(d), 256) > 0
    assert L.dg_op_lmhead_workspace_bytes(128, 262144) >= 128 * 2048 * 16
    assert L.dg_op_attention_workspace_bytes(1, 256, 16, 8, 128, 1) == 256
    assert L.dg_op_attention_workspace_bytes(1, 256, 16, 8, 128, 4) >= \
        4 * 16 * 256 * 129 * 4


def test_create_rejects_bad_arguments_without_touching_memory():
    L = dg.lib()
    d = _desc()
    out = ctypes.c_void_p(123)
    fake = ctypes.c_void_p(0x1000)
    st = L.dg_create(ctypes.byref(d), None, 1, 4096, 1, fake, fake, fake,
                     1 << 40, None, ctypes.byref(out))
    assert st == 1 and out.value is None
    assert b"weights" in L.dg_last_error(None)
    bad = _desc(head_dim=80)
    st = L.dg_create(ctypes.byref(bad), None, 1, 4096, 1, fake, fake, fake,
                     1 << 40, None, ctypes.byref(out))
    assert st == 2
    # weights present but workspace too small: capacity error
    lw = (dg.LayerWeights * 1)(dg.LayerWeights(*([0x1000] * 7 + [None, None])))
    w = dg.Weights(0x1000, 0x1000, lw)
    ws = L.dg_workspace_bytes(ctypes.byref(d), 1)
    st = L.dg_create(ctypes.byref(d), ctypes.byref(w), 1, 4096, 1, fake, fake,
                     fake, ws - 1, None, ctypes.byref(out))
    assert st == 3
    st = L.dg_create(ctypes.byref(d), ctypes.byref(w), 1, 4096, 65, fake, fake,
                     fake, 1 << 40, None, ctypes.byref(out))
    assert st == 1  # max_canvases > 64
    # more canvases than requests (multi-canvas), workspace sized for 2
    st = L.dg_create(ctypes.byref(d), ctypes.byref(w), 1, 4096, 2, fake, fake,
                     fake, ws, None, ctypes.byref(out))
    assert st == 3
    # e4m3 experts without scales
    d8 = _desc(expert_dtype=dg.FP8_E4M3)
    st = L.dg_create(ctypes.byref(d8), ctypes.byref(w), 1, 4096, 1, fake,
                     fake, fake, 1 << 40, None, ctypes.byref(out))
    assert st == 1 and b"scale" in L.dg_last_error(None)


def test_context_host_state_and_validation():
    """A context over fake device addresses: only host-side paths run."""
    L = dg.lib()
    d = _desc()
    lw = (dg.LayerWeights * 1)(dg.LayerWeights(*([0x1000] * 7 + [None, None])))
    w = dg.Weights(0x1000, 0x1000, lw)
    ws = L.dg_workspace_bytes(ctypes.byref(d), 2)
    ctx = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x100000)
    assert L.dg_create(ctypes.byref(d), ctypes.byref(w), 3, 1024, 2, fake,
                       fake, fake, ws, None, ctypes.byref(ctx)) == 0
    try:
        assert L.dg_kv_len(ctx, 0) == 0 and L.dg_kv_len(ctx, 3) == -1
        assert L.dg_set_kv_len(ctx, 1, 800) == 0
        assert L.dg_kv_len(ctx, 1) == 800
        assert L.dg_set_kv_len(ctx, 1, 1025) == 3
        assert L.dg_set_kv_len(ctx, 5, 0) == 1
        # prefill: exactly one of tokens and k/v; capacity and slot checked
        # before any launch, in both modes
        assert L.dg_prefill_kv(ctx, 0, 4, fake, fake, fake) == 1
        assert L.dg_prefill_kv(ctx, 0, 4, None, fake, None) == 1
        assert L.dg_prefill_kv(ctx, 0, 2000, None, fake, fake) == 3
        assert L.dg_prefill_kv(ctx, 0, 2000, fake, None, None) == 3
        assert L.dg_prefill_kv(ctx, 7, 4, fake, None, None) == 1
        assert L.dg_kv_len(ctx, 0) == 0
        # batch validation
        req = (ctypes.c_int32 * 3)(0, 1, 2)
        b = dg.CanvasBatch(3, req, 0x1000, 0x1000, 0x1000)
        out = dg.StepOut(0x1000, 0x1000, 0x1000, None, None)
        assert L.dg_denoise_step(ctx, ctypes.byref(b), ctypes.byref(out)) == 3
        # the canvases of one request must be contiguous
        req2 = (ctypes.c_int32 * 2)(1, 2)
        req2n = (ctypes.c_int32 * 3)(1, 2, 1)
        b2 = dg.CanvasBatch(3, req2n, 0x1000, 0x1000, 0x1000)
        ctx3 = ctypes.c_void_p()
        assert L.dg_create(ctypes.byref(d), ctypes.byref(w), 3, 1024, 3, fake,
                           fake, fake, L.dg_workspace_bytes(ctypes.byref(d), 3),
                           None, ctypes.byref(ctx3)) == 0
        assert L.dg_commit_block(ctx3, ctypes.byref(b2)) == 1
        assert L.dg_denoise_step(ctx3, ctypes.byref(b2), ctypes.byref(
            dg.StepOut(0x1000, 0x1000, 0x1000, None, None))) == 1
        L.dg_destroy(ctx3)
        # two canvases of request 1 after 800 rows: 800 + 2 x 256 > 1024
        b2c = dg.CanvasBatch(2, (ctypes.c_int32 * 2)(1, 1), 0x1000, 0x1000, 0x1000)
        assert L.dg_commit_block(ctx, ctypes.byref(b2c)) == 3
        req3 = (ctypes.c_int32 * 1)(1)
        b3 = dg.CanvasBatch(1, req3, 0x1000, 0x1000, 0x1000)
        # 800 + 256 > max_kv_len 1024: refused before any launch
        assert L.dg_commit_block(ctx, ctypes.byref(b3)) == 3
    finally:
        L.dg_destroy(ctx)


def test_sampler_and_ops_validation():
    L = dg.lib()
    f = ctypes.c_void_p(0x1000)
    assert L.dg_op_eb_select(1, 256, f, f, f, f, f, f, 0, 1, f, f, None) == 1
    assert L.dg_op_eb_select(0, 256, f, f, f, f, f, f, 4, 1, f, f, None) == 3
    assert L.dg_op_eb_select(1, 256, None, f, f, f, f, f, 4, 1, f, f, None) == 1
    assert L.dg_op_eb_select(1, 257, f, f, f, f, f, f, 4, 1, f, f, None) == 2
    assert L.dg_op_router_topk(f, 4, 8, 9, f, f, None) == 2
    assert L.dg_op_linear(f, 4, 100, f, 8, 0, f, None) == 2
    assert L.dg_op_linear(f, 4, 128, f, 8, 7, f, None) == 1
    req = (ctypes.c_int32 * 1)(0)
    plen = (ctypes.c_int32 * 1)(5000)
    assert L.dg_op_canvas_attention(f, 1, 256, 16, 8, 128, f, f, None, None, 1,
                                    4096, req, plen, 0, 0, f, f, 1 << 30,
                                    None) == 3
    plen[0] = 10
    assert L.dg_op_canvas_attention(f, 1, 256, 12, 8, 128, f, f, None, None, 1,
                                    4096, req, plen, 0, 0, f, f, 1 << 30,
                                    None) == 2
    assert L.dg_op_canvas_attention(f, 1, 256, 16, 8, 128, f, f, None, None, 1,
                                    4096, req, plen, 0, 4, f, f, 16, None) == 3
    # an E4M3 cache needs both scale arrays
    assert L.dg_op_canvas_attention(f, 1, 256, 16, 8, 128, f, f, f, None, 1,
                                    4096, req, plen, 0, 0, f, f, 1 << 30,
                                    None) == 1
    row0 = (ctypes.c_int32 * 1)(4000)
    assert L.dg_op_kv_append(f, 1, 256, 16, 8, 128, f, f, None, None, 1, 4096,
                             req, row0, None) == 3
    assert L.dg_op_kv_append(f, 1, 256, 16, 8, 96, f, f, f, f, 1, 4096,
                             req, (ctypes.c_int32 * 1)(0), None) == 2
    assert L.dg_status_string(5) == b"DG_ERR_HIP"


def test_packed_layout_sizes_and_validation():
    L = dg.lib()
    # rows padded to whole 64-row tile groups; K a multiple of 32 (bf16) /
    # 64 (e4m3)
    assert L.dg_packed_bytes(1, 200, 256, dg.BF16) == 256 * 256 * 2
    assert L.dg_packed_bytes(1, 64, 256, dg.BF16) == 64 * 256 * 2
    assert L.dg_packed_bytes(1, 262144, 2048, dg.BF16) == 262144 * 2048 * 2
    assert L.dg_packed_bytes(128, 1536, 2048, dg.FP8_E4M3) == 128 * 1536 * 2048
    assert L.dg_packed_bytes(2, 200, 256, dg.BF16) == 0     # groups need whole tiles
    assert L.dg_packed_bytes(2, 32, 256, dg.BF16) == 0      # ... of 64 rows
    assert L.dg_packed_bytes(2, 128, 256, dg.BF16) == 2 * 128 * 256 * 2
    assert L.dg_packed_bytes(1, 64, 48, dg.BF16) == 0       # K not a multiple of 32
    assert L.dg_packed_bytes(1, 64, 32, dg.FP8_E4M3) == 0   # K not a multiple of 64
    assert L.dg_packed_bytes(1, 64, 64, 7) == 0
    f = ctypes.c_void_p(0x1000)
    assert L.dg_pack_weights(None, 1, 16, 64, dg.BF16, f, None) == 1
    assert L.dg_pack_weights(f, 1, 16, 64, 7, f, None) == 1
    assert L.dg_pack_weights(f, 2, 20, 64, dg.BF16, f, None) == 2
