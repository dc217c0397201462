"""Why the "sharp" init of the parity tests uses query and key weights of
std 0.05 and not 0.2: an error budget for the bf16 bar (max-abs <= 3e-2,
row cosine >= 0.999), computed with the oracle's own steps on the CPU.

A bf16 path must round Q and K to bf16 before the score product. The test
runs the oracle's blocks twice on the same seeded inputs, once exactly and
once with only Q and K rounded to bf16 (round to nearest even), everything
else in float64. At std 0.2 (scores of std ~47 at d_model 1280) that single
rounding already moves outputs by more than the whole bar, so no bf16 path
could pass; at std 0.05 (scores of std ~3, the sharp init the GPU tests use)
it stays well inside it.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import encoder as E


def _blocks_with_rounded_qk(x, W, n_layers, n_heads, eps):
    """The oracle's pre-LN blocks with Q and K rounded to bf16 before QK^T."""
    for layer in range(n_layers):
        lw = E.layer_weights(W, layer)
        a = E.layer_norm(x, lw["ln1_g"], lw["ln1_b"], eps)
        q = E.linear(a, lw["q_w"], lw["q_b"])
        k = E.linear(a, lw["k_w"])
        v = E.linear(a, lw["v_w"], lw["v_b"])
        rq = synth.round_to_bf16(q.astype(np.float32)).astype(np.float64)
        rk = synth.round_to_bf16(k.astype(np.float32)).astype(np.float64)
        o, _ = E.attention_core(rq, rk, v, n_heads)
        x = x + E.linear(o, lw["o_w"], lw["o_b"])
        h = E.layer_norm(x, lw["ln2_g"], lw["ln2_b"], eps)
        x = x + E.linear(E.gelu(E.linear(h, lw["fc1_w"], lw["fc1_b"])), lw["fc2_w"], lw["fc2_b"])
    return x


@pytest.mark.parametrize("qk_std,within", [(0.2, False), (0.05, True)], ids=["std_0.2", "std_0.05"])
def test_bf16_rounding_of_q_and_k_alone(monkeypatch, qk_std, within):
    base = synth.get_workload("whisper_large_b1")
    w = base.replace(geom=base.geom.replace(n_layers=2, n_frames=600), init="sharp")
    monkeypatch.setattr(synth.inputs, "SHARP_QK_STD", qk_std)
    W = synth.make_weights(w)
    g = w.geom
    mel = synth.make_mel(w)[0]
    x = E.stem(mel, W)
    exact = E.final(E.blocks(x, W, g.n_layers, g.n_heads, None, g.ln_eps), W)
    rounded = E.final(_blocks_with_rounded_qk(x, W, g.n_layers, g.n_heads, g.ln_eps), W)
    err = float(np.abs(rounded - exact).max())
    # the scores' spread, in natural-log units of the softmax, at this init
    a = E.layer_norm(x, W["layers.0.ln1_g"], W["layers.0.ln1_b"])
    s = (E.linear(a, W["layers.0.q_w"])[:, :64] @ E.linear(a, W["layers.0.k_w"])[:, :64].T) / math.sqrt(64)
    print(f"Q/K std {qk_std}: score std {s.std():.2f}, bf16 Q and K alone move outputs by {err:.4f}")
    if within:
        assert err <= 0.5 * 3e-2, err      # leaves more than half the bar to the rest of the path
    else:
        assert err > 3e-2, err             # the bar cannot be met at this init
