"""Pins of the oracle's chunked attention (chunk-causal and block-diagonal
key rules).

The rule itself is a reading: "MiniCPM-o-2_6", section "(2) AUDIO", prints
audio_chunk_length 1.0 beside its Whisper encoder and nothing about how the
encoder uses it, so which keys a chunked query sees is parity unpinned. What
is pinned here is that the oracle computes the rule it states, by routes that
do not share its masking code: slicing the sequence into chunks or prefixes
and running plain attention on the slice, chunk sizes that reduce the rule to
full attention, to the identity (a query that sees only itself returns its
value) or to textbook causal attention (PyTorch's scaled_dot_product_attention
in float64), and a brute-force count of the attended pairs. Planted mistakes
in the rule must fail one of these pins.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import encoder as E

H, D = 4, 256


def qkv(t, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((t, D)) for _ in range(3)]


def core(q, k, v, key_mask=None, allowed=None):
    return E.attention_core(q, k, v, H, key_mask, allowed)[0]


@pytest.mark.parametrize("mode", [oracle.CHUNK_CAUSAL, oracle.CHUNK_BLOCK])
def test_chunk_covering_everything_is_full_attention(mode):
    q, k, v = qkv(23)
    full = core(q, k, v)
    assert np.array_equal(core(q, k, v, allowed=oracle.chunk_allowed(23, 23, mode)), full)
    assert np.array_equal(core(q, k, v, allowed=oracle.chunk_allowed(23, 100, mode)), full)


def test_block_chunk_of_one_returns_the_values():
    q, k, v = qkv(17, 1)
    assert np.array_equal(core(q, k, v, allowed=oracle.chunk_allowed(17, 1, oracle.CHUNK_BLOCK)), v)


def test_causal_chunk_of_one_is_causal_attention():
    t = 19
    q, k, v = qkv(t, 2)
    got = core(q, k, v, allowed=oracle.chunk_allowed(t, 1, oracle.CHUNK_CAUSAL))
    heads = lambda x: torch.from_numpy(x.reshape(t, H, D // H).transpose(1, 0, 2).copy())  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
    ref = ref.numpy().transpose(1, 0, 2).reshape(t, D)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def _decomposition_ok(t, chunk, mode, n_valid=None, seed=3):
    """Rows of the chunked attention against plain attention on slices."""
    q, k, v = qkv(t, seed)
    mask = None if n_valid is None else (np.arange(t) < n_valid).astype(np.uint8)
    got = core(q, k, v, mask, oracle.chunk_allowed(t, chunk, mode))
    n = t if n_valid is None else n_valid
    for c in range((t + chunk - 1) // chunk):
        lo, hi = c * chunk, min(t, (c + 1) * chunk)
        first_key = lo if mode == oracle.CHUNK_BLOCK else 0
        last_key = min(hi, n)
        rows = [r for r in range(lo, hi) if r < n]
        if not rows:
            continue
        sl = slice(first_key, last_key)
        ref = core(q[sl], k[sl], v[sl])
        if not np.allclose(got[rows], ref[np.array(rows) - first_key], rtol=1e-12, atol=1e-13):
            return False
    return True


CASES = [(23, 5, None), (23, 5, 17), (40, 8, None), (40, 8, 33), (31, 31, 12), (9, 2, 9)]


@pytest.mark.parametrize("mode", [oracle.CHUNK_CAUSAL, oracle.CHUNK_BLOCK])
@pytest.mark.parametrize("t,chunk,n_valid", CASES)
def test_rows_are_attention_over_their_slice(mode, t, chunk, n_valid):
    assert _decomposition_ok(t, chunk, mode, n_valid)


def test_queries_without_keys_are_zero_and_harmless():
    """Block rule with a key mask: a masked chunk's queries see no key; their
    rows are zero and the valid rows stay finite and unchanged."""
    t, chunk, n_valid = 20, 5, 7
    q, k, v = qkv(t, 4)
    mask = (np.arange(t) < n_valid).astype(np.uint8)
    o = core(q, k, v, mask, oracle.chunk_allowed(t, chunk, oracle.CHUNK_BLOCK))
    assert np.all(np.isfinite(o))
    assert np.array_equal(o[10:], np.zeros((10, D)))
    assert _decomposition_ok(t, chunk, oracle.CHUNK_BLOCK, n_valid, seed=4)


@pytest.mark.parametrize("tb,chunk,mode", [(1500, 50, 1), (1500, 50, 2), (23, 5, 1), (23, 5, 2), (7, 10, 1),
                                           (9, 1, 1), (9, 1, 2), (12, 0, 0)])
def test_attended_pairs_by_brute_force(tb, chunk, mode):
    brute = int(oracle.chunk_allowed(tb, chunk, mode).sum())
    assert oracle.attended_pairs(tb, chunk, mode) == brute
    if mode == oracle.CHUNK_CAUSAL and chunk > 0:
        # closed form for whole chunks: sum over chunks c of chunk * chunk (c + 1)
        n = tb // chunk
        if n * chunk == tb:
            assert brute == chunk * chunk * n * (n + 1) // 2


def test_encoder_with_a_chunk_covering_the_clip_equals_the_full_encoder():
    w = synth.get_workload("tiny_fp32_b1")
    W = synth.make_weights(w)
    mel = synth.make_mel(w)[0]
    full = oracle.encode_clip(w.geom, W, mel)
    for mode in (oracle.CHUNK_CAUSAL, oracle.CHUNK_BLOCK):
        g = w.geom.replace(attn_chunk=w.geom.n_pos, attn_chunk_mode=mode)
        assert np.array_equal(oracle.encode_clip(g, W, mel), full)
    # a real chunk changes the result
    g = w.geom.replace(attn_chunk=16, attn_chunk_mode=oracle.CHUNK_CAUSAL)
    assert not np.allclose(oracle.encode_clip(g, W, mel), full)


# ---- planted mistakes in the rule: each must fail a pin above -------------

def _pins_pass() -> bool:
    for mode in (oracle.CHUNK_CAUSAL, oracle.CHUNK_BLOCK):
        for t, chunk, n_valid in CASES:
            if not _decomposition_ok(t, chunk, mode, n_valid):
                return False
    q, k, v = qkv(17, 1)
    if not np.array_equal(core(q, k, v, allowed=E.chunk_allowed(17, 1, oracle.CHUNK_BLOCK)), v):
        return False
    return True


def m_strict(t, chunk, mode):            # earlier chunks only, not the query's own
    c = np.arange(t) // chunk
    return c[None, :] < c[:, None] if mode == 1 else c[None, :] == c[:, None]


def m_shifted(t, chunk, mode):           # chunk boundaries one position late
    c = (np.arange(t) + 1) // chunk
    return c[None, :] <= c[:, None] if mode == 1 else c[None, :] == c[:, None]


def m_future(t, chunk, mode):            # later chunks instead of earlier ones
    c = np.arange(t) // chunk
    return c[None, :] >= c[:, None] if mode == 1 else c[None, :] == c[:, None]


def m_block_as_causal(t, chunk, mode):   # the block rule forgets its lower edge
    c = np.arange(t) // chunk
    return c[None, :] <= c[:, None]


def m_query_chunk_by_key(t, chunk, mode):  # transposed: the key's chunk decides
    c = np.arange(t) // chunk
    return (c[None, :] <= c[:, None]).T if mode == 1 else c[None, :] == c[:, None]


def test_the_real_rule_passes():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", [m_strict, m_shifted, m_future, m_block_as_causal, m_query_chunk_by_key])
def test_planted_mistake_is_caught(monkeypatch, mutation):
    monkeypatch.setattr(E, "chunk_allowed", mutation)
    monkeypatch.setattr(oracle, "chunk_allowed", mutation)
    assert not _pins_pass()
