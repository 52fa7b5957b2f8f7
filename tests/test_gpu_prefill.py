"""Token-mode prefill (dg_prefill_kv with prompt tokens): the causal encode
of the prompt in chunks of up to 256 tokens (write-up Figure 4 stage 1;
model card "Model Overview": the causal encoder fills the cache).

A 300-token prompt (a 256-token chunk and a ragged 44-token chunk) on a
two-layer model:
  * lockstep: the oracle encodes the chunks causally (the second with the
    first's K/V as its prefix; a causal block equals sequential one-token
    encodes, which the oracle pins); the ops are fed the oracle's values per
    layer and chunk (the second chunk's prefix is the oracle's first-chunk
    K/V, installed into a spare slot), and every layer's K/V is compared;
  * composition: the cache rows the prefill wrote against the same chunked
    encode run through the single-op entry points;
  * the slot's length becomes the prompt length; a prompt longer than the
    cache is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from block_discrete_diffusion_tok_amd import dg, synth
from gpu_common import DEV, log, np32, oshape, to_dev
from lockstep import Lockstep
from workload_common import check_commit_composition

pytestmark = pytest.mark.gpu

SHAPE = synth.ModelShape(2, 256, 4, 2, 64, 16, 2, 512, 4096)


def test_token_mode_prefill_lockstep_and_composition():
    n = 300
    w = synth.make_weights(SHAPE, seed=5, gain_std=0.1)
    wd = to_dev(w)
    eng = dg.Engine(SHAPE, wd, max_requests=2, max_kv_len=1024, max_canvases=1)
    g = torch.Generator()
    g.manual_seed(42)
    tok = torch.randint(0, SHAPE.vocab, (n,), generator=g, dtype=torch.int32)
    eng.prefill_tokens(0, tok.to(DEV))
    torch.cuda.synchronize()
    assert eng.kv_len(0) == n
    log("prefill: composition of the two chunks")
    td = tok.to(DEV)
    check_commit_composition(eng, SHAPE, wd, td[:256].reshape(1, 256), [0], [0],
                             "prefill chunk 0")
    check_commit_composition(eng, SHAPE, wd, td[256:].reshape(1, n - 256), [0],
                             [256], "prefill chunk 1", C=n - 256)
    log("prefill: lockstep")
    wn = synth.to_numpy_weights(w)
    osh = oshape(SHAPE)
    empty = np.zeros((SHAPE.n_layers, SHAPE.n_kv_heads, 0, SHAPE.head_dim))
    kv1, cap1 = [], []
    oracle.model._layers_forward(osh, wn, tok.numpy()[None, :256].astype(np.int64),
                                 [(empty, empty)], True, True, cap1, kv_out=kv1)
    ls = Lockstep(SHAPE, eng, eng.weights, 1, [1], [0], [0], cap1,
                  "prefill chunk 0", causal=True, kv_o=kv1)
    assert ls.finish() == SHAPE.n_layers
    ls.report()
    k1 = np.stack([k for k, _ in kv1])      # [L, Hkv, 256, D]
    v1 = np.stack([v for _, v in kv1])
    kv2, cap2 = [], []
    oracle.model._layers_forward(osh, wn, tok.numpy()[None, 256:].astype(np.int64),
                                 [(k1, v1)], True, True, cap2, kv_out=kv2)
    # the second chunk's ops read the oracle's first-chunk K/V from slot 1
    eng.prefill_kv(1, torch.as_tensor(k1, dtype=torch.float32).to(torch.bfloat16)
                   .to(DEV).contiguous(),
                   torch.as_tensor(v1, dtype=torch.float32).to(torch.bfloat16)
                   .to(DEV).contiguous())
    ls2 = Lockstep(SHAPE, eng, eng.weights, 1, [1], [256], [0], cap2,
                   "prefill chunk 1", causal=True, kv_o=kv2, C=n - 256)
    assert ls2.finish() == SHAPE.n_layers
    ls2.report()
    # the one-pass causal encode of the whole prompt equals the two chunks
    kv_all = oracle.commit_block(osh, wn, tok.numpy()[None].astype(np.int64),
                                 [(empty, empty)], mirror=False)[0]
    kv_ch = oracle.commit_block(osh, wn, tok.numpy()[None, 256:].astype(np.int64),
                                [(kv_all[0][:, :, :256], kv_all[1][:, :, :256])],
                                mirror=False)[0]
    np.testing.assert_allclose(kv_ch[0], kv_all[0][:, :, 256:], rtol=1e-9, atol=1e-12)
    # a prompt longer than the cache is refused before any launch
    long_tok = torch.zeros(1025, dtype=torch.int32, device=DEV)
    with pytest.raises(dg.DgError) as ei:
        eng.prefill_tokens(0, long_tok)
    assert ei.value.status == 3
    assert eng.kv_len(0) == n
    eng.close()
