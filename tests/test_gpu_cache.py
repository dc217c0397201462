"""Embeddings cache (aenc_cache_*, aenc_forward_cached) on the device."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def aenc():
    import audio_encoder_tower_amd as a
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    a.lib()
    return a


def test_round_trip_and_lru_eviction(aenc):
    c = aenc.EmbeddingsCache(4096, 3)
    src = {k: torch.full((1024,), float(k), device=DEV) for k in (1, 2, 3, 4)}
    for k in (1, 2, 3):
        c.insert(k, src[k])
    dst = torch.zeros(1024, device=DEV)
    assert c.lookup(1, dst)                      # 1 becomes the most recent; 2 is now the oldest
    torch.cuda.synchronize()
    assert torch.equal(dst, src[1])
    c.insert(4, src[4])                          # evicts 2
    assert 2 not in c and 1 in c and 3 in c and 4 in c
    assert not c.lookup(2, dst)
    for k in (1, 3, 4):
        assert c.lookup(k, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst, src[k])
    assert c.stats() == {"hits": 4, "misses": 1, "inserts": 4, "evictions": 1, "entries": 3}
    c.close()


def test_copies_are_ordered_across_streams(aenc):
    """An insert enqueued behind long work on one stream is seen by a lookup on another."""
    c = aenc.EmbeddingsCache(4 * 4096, 2)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn(4096, 4096, device=DEV)
    src = torch.zeros(4096, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        x = a
        for _ in range(8):
            x = x @ a * 1e-3                     # keeps stream A busy for a while
        src.copy_(x[0])
        c.insert(7, src, stream=sa)
    dst = torch.zeros(4096, device=DEV)
    with torch.cuda.stream(sb):
        assert c.lookup(7, dst, stream=sb)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    c.close()


def test_forward_cached(aenc):
    """Cache hits are the forward's output bit for bit, and both meet the bf16
    bar against the oracle: the first batch (all misses), the all-hit batch,
    and a batch with one new clip (run by the forward, stored alone)."""
    w = synth.get_workload("whisper_large_b1")
    w = w.replace(geom=w.geom.replace(batch=3, n_layers=1, n_frames=400), init="perturbed")
    g = w.geom
    W = synth.make_weights(w)
    enc = aenc.Encoder(g, {k: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for k, v in W.items()})
    mel_np = synth.make_mel(w)
    mel = torch.from_numpy(mel_np).to(DEV).to(torch.bfloat16)
    ref = enc.forward(mel).clone()
    want = oracle.encode(g, W, mel_np)
    cache = aenc.EmbeddingsCache.for_encoder(enc, 8)
    out, hits = enc.forward_cached(cache, [10, 11, 12], mel)
    torch.cuda.synchronize()
    assert hits == 0 and torch.equal(out, ref)
    parity.assert_bf16_parity(out.double().cpu().numpy(), want, "cached forward, all misses")
    enc.profile(True)
    out2, hits2 = enc.forward_cached(cache, [10, 11, 12], mel)
    torch.cuda.synchronize()
    stats = enc.profile_read()
    assert hits2 == 3 and torch.equal(out2, ref)
    assert sum(n for _, n in stats.values()) == 0      # served by copies: no kernel launched
    m = parity.assert_bf16_parity(out2.double().cpu().numpy(), want, "cached forward, all hits")
    print("all hits vs oracle", m)
    # a batch with one new clip runs the forward and stores only the new clip
    mel2_np = mel_np.copy()
    mel2_np[1] = synth.make_mel(w.replace(mel_seed=9), clips=[1])[0]
    mel2 = torch.from_numpy(mel2_np).to(DEV).to(torch.bfloat16)
    ref2 = enc.forward(mel2).clone()
    out3, hits3 = enc.forward_cached(cache, [10, 99, 12], mel2)
    torch.cuda.synchronize()
    assert hits3 == 2 and torch.equal(out3, ref2)
    want2 = oracle.encode(g, W, mel2_np)
    parity.assert_bf16_parity(out3.double().cpu().numpy(), want2, "cached forward, one new clip")
    # the new clip is now served from the cache
    out4, hits4 = enc.forward_cached(cache, [99, 10, 12], mel2[[1, 0, 2]].contiguous())
    torch.cuda.synchronize()
    assert hits4 == 3
    parity.assert_bf16_parity(out4.double().cpu().numpy(), want2[[1, 0, 2]], "cached forward, stored new clip")
    s = cache.stats()
    assert s["entries"] == 4 and s["inserts"] == 4
    enc.profile(False)
    enc.close()
    cache.close()


def test_cache_rejects_bad_arguments(aenc):
    L = aenc.lib()
    assert L.aenc_cache_create(0, 4) is None
    assert L.aenc_cache_create(16, 0) is None
    assert L.aenc_cache_lookup(None, 1, None, None) == -1
    assert L.aenc_cache_insert(None, 1, None, None) == -1
    w = synth.get_workload("whisper_large_b1")
    w = w.replace(geom=w.geom.replace(n_layers=0, n_frames=64))
    enc = aenc.Encoder(w.geom, {k: torch.from_numpy(v).to(DEV).to(torch.bfloat16)
                                for k, v in synth.make_weights(w).items()})
    wrong = aenc.EmbeddingsCache(16, 2)
    mel = torch.zeros(1, w.geom.n_mel, w.geom.n_frames, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(aenc.AencError):
        enc.forward_cached(wrong, [1], mel)
    enc.close()
    wrong.close()
