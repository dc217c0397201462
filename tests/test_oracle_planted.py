"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation below is a mistake someone could make when writing the
encoder; the pins of test_oracle_pins must reject all of them. The oracle
module is patched only inside each test.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import encoder as E
from tests.test_oracle_pins import (TOWER_CASES, _float64_modules, tiny_workload, torch_encoder,  # noqa: F401
                                    valid_out_rows)


def _tower_pins_pass() -> bool:
    for case, spec in TOWER_CASES.items():
        w = tiny_workload(**spec["geom"]).replace(init=spec["init"], mel_clip=None)
        g = w.geom
        W = synth.make_weights(w)
        mel = synth.make_mel(w)
        mask = None
        if "lengths" in spec:
            n_f = np.array(spec["lengths"])
            for b, n in enumerate(n_f):
                mel[b, :, n:] = 0.0
            mask = (np.arange(g.n_pos)[None, :] < ((n_f + 1) // 2)[:, None]).astype(np.uint8)
        try:
            got = oracle.encode(g, W, mel, mask)
        except Exception:
            return False
        ref = torch_encoder(g, W, mel, mask)
        if got.shape != ref.shape:
            return False
        for b in range(g.batch):
            v = valid_out_rows(g, mask, b)
            if not np.allclose(got[b][v], ref[b][v], rtol=1e-10, atol=1e-11):
                return False
    return True


real = {name: getattr(E, name) for name in
        ("gelu", "layer_norm", "linear", "conv1d_k3", "sinusoids", "attention", "block", "final", "stem",
         "stack_rows")}


def m_unbiased_var(x, g, b, eps=E.LN_EPS):
    mu = x.mean(axis=-1, keepdims=True)
    return g * (x - mu) / np.sqrt(x.var(axis=-1, ddof=1, keepdims=True) + eps) + b


def m_tanh_gelu(x):
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def m_pe_half(n_pos, d, dtype=np.float64):
    half = d // 2
    omega = np.exp(-math.log(10000.0) / half * np.arange(half))
    ang = np.arange(n_pos)[:, None] * omega[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1).astype(dtype)


def m_pe_swapped(n_pos, d, dtype=np.float64):
    pe = real["sinusoids"](n_pos, d, dtype)
    half = d // 2
    return np.concatenate([pe[:, half:], pe[:, :half]], axis=1)


def m_conv_shift(x, w, b, stride):
    # taps x[s*t + k] instead of x[s*t + k - 1]
    y = real["conv1d_k3"](np.concatenate([x[:, 1:], np.zeros_like(x[:, :1])], axis=1), w, b, stride)
    return y


def m_linear_transposed(x, w, b=None):
    y = x @ (w if w.shape[0] == w.shape[1] else w.T)
    return y if b is None else y + b


def m_no_scale_attention(a, lw, n_heads, key_mask=None, k_bias=None, return_probs=False, dtype=np.float64):
    lw = dict(lw, q_w=np.asarray(lw["q_w"], np.float64) * math.sqrt(a.shape[1] // n_heads),
              q_b=np.asarray(lw["q_b"], np.float64) * math.sqrt(a.shape[1] // n_heads))
    return real["attention"](a, lw, n_heads, key_mask, k_bias, return_probs, dtype)


def m_mask_ignored(a, lw, n_heads, key_mask=None, k_bias=None, return_probs=False, dtype=np.float64):
    return real["attention"](a, lw, n_heads, None, k_bias, return_probs, dtype)


def m_post_ln(x, lw, n_heads, key_mask=None, eps=E.LN_EPS, k_bias=None, dtype=np.float64):
    x = real["layer_norm"](x + real["attention"](x, lw, n_heads, key_mask, k_bias=k_bias, dtype=dtype),
                           lw["ln1_g"], lw["ln1_b"], eps)
    h = real["gelu"](real["linear"](x, lw["fc1_w"], lw["fc1_b"]))
    return real["layer_norm"](x + real["linear"](h, lw["fc2_w"], lw["fc2_b"]), lw["ln2_g"], lw["ln2_b"], eps)


def m_no_ffn_residual(x, lw, n_heads, key_mask=None, eps=E.LN_EPS, k_bias=None, dtype=np.float64):
    a = real["layer_norm"](x, lw["ln1_g"], lw["ln1_b"], eps)
    x = x + real["attention"](a, lw, n_heads, key_mask, k_bias=k_bias, dtype=dtype)
    h = real["layer_norm"](x, lw["ln2_g"], lw["ln2_b"], eps)
    return real["linear"](real["gelu"](real["linear"](h, lw["fc1_w"], lw["fc1_b"])), lw["fc2_w"], lw["fc2_b"])


def m_pool_before_ln(x, W, pool_step=1, eps=E.LN_EPS, dtype=np.float64):
    if pool_step == 2:
        n = x.shape[0] // 2
        x = (x[0:2 * n:2] + x[1:2 * n:2]) / 2.0
    return real["final"](x, W, 1, eps, dtype)


def m_no_pe(mel, W, dtype=np.float64):
    x = real["stem"](mel, W, dtype)
    return x - real["sinusoids"](x.shape[0], x.shape[1], dtype)


def m_stack_feature_major(y, k):
    # interleaves the k positions feature by feature instead of concatenating them
    n, d = y.shape[0] // k, y.shape[1]
    return y[:n * k].reshape(n, k, d).transpose(0, 2, 1).reshape(n, k * d)


def m_stack_keeps_partial_run(y, k):
    n, d = -(-y.shape[0] // k), y.shape[1]
    pad = np.zeros((n * k - y.shape[0], d))
    return real["stack_rows"](np.concatenate([y, pad]), k)


MUTATIONS = {
    "unbiased_variance": ("layer_norm", m_unbiased_var),
    "tanh_gelu": ("gelu", m_tanh_gelu),
    "pe_denominator_half": ("sinusoids", m_pe_half),
    "pe_sin_cos_swapped": ("sinusoids", m_pe_swapped),
    "conv_taps_shifted": ("conv1d_k3", m_conv_shift),
    "square_weights_transposed": ("linear", m_linear_transposed),
    "attention_unscaled": ("attention", m_no_scale_attention),
    "key_mask_ignored": ("attention", m_mask_ignored),
    "post_layernorm": ("block", m_post_ln),
    "ffn_residual_dropped": ("block", m_no_ffn_residual),
    "pool_before_final_ln": ("final", m_pool_before_ln),
    "positions_not_added": ("stem", m_no_pe),
    "stack_feature_major": ("stack_rows", m_stack_feature_major),
    "stack_keeps_partial_run": ("stack_rows", m_stack_keeps_partial_run),
}


def test_unmutated_oracle_passes():
    assert _tower_pins_pass()


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    name, fn = MUTATIONS[mutation]
    monkeypatch.setattr(E, name, fn)
    assert not _tower_pins_pass(), f"planted mistake {mutation!r} was not caught"
