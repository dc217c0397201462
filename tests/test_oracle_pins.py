"""Pins of the CPU oracle against facts the pages fix and against mathematics.

Each check uses something other than the oracle itself: numbers printed on
the pages (tests/golden/page_facts.json, each with its citation), closed
forms, invariants, independent library routines (torch.nn modules in
float64, numpy.correlate, math.erf) and brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import encoder as E



@pytest.fixture(autouse=True)
def _float64_modules():
    """torch.nn modules built by these tests hold float64 parameters."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def tiny_workload(**geom_kw):
    base = synth.get_workload("tiny_fp32_b1")
    g = base.geom.replace(**geom_kw)
    return base.replace(geom=g)


def rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def rand_layer(rng, d, f, scale=0.2, perturb=True):
    lw = {
        "ln1_g": 1 + rand(rng, d, scale=0.1 if perturb else 0), "ln1_b": rand(rng, d, scale=0.1 if perturb else 0),
        "q_w": rand(rng, d, d, scale=scale), "q_b": rand(rng, d, scale=0.1),
        "k_w": rand(rng, d, d, scale=scale),
        "v_w": rand(rng, d, d, scale=scale), "v_b": rand(rng, d, scale=0.1),
        "o_w": rand(rng, d, d, scale=scale), "o_b": rand(rng, d, scale=0.1),
        "ln2_g": 1 + rand(rng, d, scale=0.1 if perturb else 0), "ln2_b": rand(rng, d, scale=0.1 if perturb else 0),
        "fc1_w": rand(rng, f, d, scale=scale), "fc1_b": rand(rng, f, scale=0.1),
        "fc2_w": rand(rng, d, f, scale=scale), "fc2_b": rand(rng, d, scale=0.1),
    }
    return lw


# ---------------------------------------------------------------------------
# Geometry and shape facts (P1)
# ---------------------------------------------------------------------------

def test_workload_geometries_match_pages(page_facts):
    large = page_facts["whisper_large_encoder"]
    for name in ("whisper_large_b1", "whisper_large_proj_b16", "whisper_large_varlen_b32"):
        g = synth.get_workload(name).geom
        assert (g.d_model, g.n_layers, g.n_heads, g.d_ffn, g.n_mel) == (
            large["d_model"], large["encoder_layers"], large["encoder_attention_heads"],
            large["encoder_ffn_dim"], large["num_mel_bins"])
        assert g.head_dim == large["head_dim"]
        assert g.n_frames == page_facts["feature_frames"]["nb_max_frames"]
    med = page_facts["whisper_medium_encoder"]
    g = synth.get_workload("whisper_medium_pool2_b1").geom
    assert (g.d_model, g.n_layers, g.n_heads, g.d_ffn, g.pool_step) == (
        med["d_model"], med["encoder_layers"], med["encoder_attention_heads"],
        med["encoder_ffn_dim"], med["audio_pool_step"])
    pj = page_facts["projector"]
    g = synth.get_workload("whisper_large_proj_b16").geom
    assert (g.d_model, g.proj_out) == (pj["d_in"], pj["d_out"])
    ff = page_facts["feature_frames"]
    # 30 s at 16 kHz with hop 160 is 3000 frames.
    assert ff["chunk_seconds"] * ff["sampling_rate"] // ff["hop_length"] == ff["nb_max_frames"]


def test_stem_maps_3000_frames_to_1500_positions(page_facts):
    ff = page_facts["feature_frames"]
    rng = np.random.default_rng(0)
    d, n_mel = 64, ff["feature_size"]
    W = {"conv1_w": rand(rng, d, n_mel, 3, scale=0.05), "conv1_b": np.zeros(d),
         "conv2_w": rand(rng, d, d, 3, scale=0.05), "conv2_b": np.zeros(d)}
    x = E.stem(rand(rng, n_mel, ff["nb_max_frames"]), W)
    assert x.shape == (ff["encoder_positions_per_chunk"], d)
    # The tiny workload: 200 frames -> 100 positions.
    W80 = dict(W, conv1_w=rand(rng, d, 80, 3, scale=0.05))
    assert E.stem(rand(rng, 80, 200), W80).shape == (100, d)


def test_pool_step_2_halves_positions(page_facts):
    p = page_facts["pool"]
    rng = np.random.default_rng(1)
    d = 16
    W = {"lnf_g": np.ones(d), "lnf_b": np.zeros(d)}
    y = E.final(rand(rng, p["positions_in"], d), W, pool_step=p["pool_step"])
    assert y.shape == (p["tokens_out_about"], d)
    # An odd trailing position is dropped.
    assert E.final(rand(rng, 7, d), W, pool_step=2).shape == (3, d)
    # The pool is the pair mean of the normalised rows.
    x = rand(rng, 6, d)
    ln = E.layer_norm(x, W["lnf_g"], W["lnf_b"])
    np.testing.assert_allclose(E.final(x, W, 2)[1], (ln[2] + ln[3]) / 2, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Parameter totals (P2)
# ---------------------------------------------------------------------------

def decoder_params(t):
    h, hd = t["hidden"], t["head_dim"]
    q, kv = t["q_heads"] * hd, t["kv_heads"] * hd
    attn = h * q + 2 * h * kv + q * h
    if t["attention_bias"]:
        attn += q + 2 * kv
    mlp = t["mlp_matrices"] * h * t["intermediate"]
    per_layer = attn + mlp + t["norm_vectors_per_layer"] * h
    return t["layers"] * per_layer + t["embedding_matrices"] * t["vocab"] * h + t["final_norm_vectors"] * h


def large_geom():
    return synth.get_workload("whisper_large_b1").geom


def test_voxtral_total_closes_on_the_oracle_encoder(page_facts):
    v = page_facts["voxtral_total"]
    g = large_geom()
    rest = v["params_total"] - decoder_params(v["text_decoder"])
    pos_table = 1500 * g.d_model                     # stored position table
    adaptor = 4 * g.d_model * 3072 + 3072 * 3072     # bias-free 5120 -> 3072 -> 3072
    assert rest - oracle.param_count(g, with_projector=False) - pos_table == adaptor


def test_voxtral_total_closes_on_the_stacked_projector(page_facts):
    """The same total, now with the oracle's own stacked-projector tensors:
    encoder + 4-position stacked projector (biases aside) + position table."""
    v = page_facts["voxtral_total"]
    g = synth.get_workload("whisper_large_stack4_proj_b16").geom
    rest = v["params_total"] - decoder_params(v["text_decoder"])
    shapes = dict(oracle.param_shapes(g))
    assert shapes["proj1_w"] == (3072, page_facts["downsample"]["adaptor_input_dim"])
    proj_bias = shapes["proj1_b"][0] + shapes["proj2_b"][0]
    assert oracle.param_count(g) - proj_bias + 1500 * g.d_model == rest


def test_stacking_gives_the_page_rate(page_facts):
    """1500 positions per 30 s chunk, stacked by 4, are 12.5 rows per second."""
    f, s = page_facts["feature_frames"], page_facts["downsample"]
    g = synth.get_workload("whisper_large_stack4_proj_b16").geom
    assert g.stack * g.d_model == s["adaptor_input_dim"]
    W = {"lnf_g": np.ones(g.d_model), "lnf_b": np.zeros(g.d_model),
         "proj1_w": np.zeros((8, g.proj_in)), "proj1_b": np.zeros(8),
         "proj2_w": np.zeros((4, 8)), "proj2_b": np.zeros(4)}
    y = E.final(np.random.default_rng(0).standard_normal((f["encoder_positions_per_chunk"], g.d_model)), W,
                stack=g.stack)
    assert y.shape[0] / f["chunk_seconds"] == s["rate_hz"]
    assert y.shape[0] == g.t_out


def test_stacked_projector_is_a_sum_of_block_products():
    """Row j of the stacked projector input is positions kj .. kj+k-1 in
    order: its first linear layer equals the sum over i of position kj+i times
    the i-th column block of Wp1 (an independent way of writing the same
    contraction, which a feature-interleaved or reversed stacking fails)."""
    rng = np.random.default_rng(5)
    d, k, h, o, t = 6, 4, 7, 5, 14
    W = {"lnf_g": 1 + rand(rng, d, scale=0.1), "lnf_b": rand(rng, d, scale=0.1),
         "proj1_w": rand(rng, h, k * d), "proj1_b": rand(rng, h),
         "proj2_w": rand(rng, o, h), "proj2_b": rand(rng, o)}
    x = rand(rng, t, d)
    got = E.final(x, W, stack=k)
    y = E.layer_norm(x, W["lnf_g"], W["lnf_b"])
    assert got.shape == (t // k, o)
    for j in range(t // k):
        pre = W["proj1_b"].copy()
        for i in range(k):
            pre += W["proj1_w"][:, i * d:(i + 1) * d] @ y[k * j + i]
        hid = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in pre])
        np.testing.assert_allclose(got[j], W["proj2_w"] @ hid + W["proj2_b"], rtol=1e-12, atol=1e-12)


def test_qwen2_audio_total_closes_on_the_oracle_encoder(page_facts):
    q = page_facts["qwen2_audio_total"]
    g = large_geom()
    rest = q["params_total"] - decoder_params(q["text_decoder"])
    pos_table = 1500 * g.d_model
    projector = g.d_model * q["text_decoder"]["hidden"] + q["text_decoder"]["hidden"]
    assert rest - oracle.param_count(g, with_projector=False) - pos_table == projector


def test_oracle_reads_every_generated_tensor():
    for name in ("tiny_fp32_b1", "whisper_large_proj_b16", "whisper_large_stack4_proj_b16"):
        w = synth.get_workload(name)
        g = w.geom
        if g.n_layers > 4:
            g = g.replace(n_layers=2)
        shapes = dict(oracle.param_shapes(g))
        gen = dict(synth.inputs.weight_shapes(g) + synth.inputs.proj_shapes(g))
        assert shapes == gen


def test_flop_closed_form():
    g = large_geom()
    assert oracle.flops(g) == pytest.approx(2.27377152e12, rel=1e-12)
    g4 = synth.get_workload("whisper_large_proj_b16").geom
    assert oracle.flops(g4) == pytest.approx(16 * (2.27377152e12 + 2 * 1500 * (1280 * 3072 + 3072 * 3072)))


def test_flop_count_by_counting_matmuls(monkeypatch):
    """Count the multiply-adds of every matmul the oracle performs."""
    w = tiny_workload(n_frames=20, n_layers=2)
    W = synth.make_weights(w)
    mel = synth.make_mel(w)
    count = {"macs": 0}

    class Counting(np.ndarray):
        pass

    real_linear, real_conv = E.linear, E.conv1d_k3

    def linear(x, wt, b=None):
        count["macs"] += x.shape[0] * wt.shape[0] * wt.shape[1]
        return real_linear(x, wt, b)

    def conv(x, wt, b, stride):
        y = real_conv(x, wt, b, stride)
        count["macs"] += y.shape[1] * wt.size
        return y

    monkeypatch.setattr(E, "linear", linear)
    monkeypatch.setattr(E, "conv1d_k3", conv)
    E.encode(w.geom, W, mel)
    t = w.geom.n_frames // 2
    attn_macs = w.geom.n_layers * 2 * t * t * w.geom.d_model
    assert 2 * (count["macs"] + attn_macs) == oracle.flops(w.geom)


# ---------------------------------------------------------------------------
# Elementary functions (P6 iv, P7, P12)
# ---------------------------------------------------------------------------

def test_gelu_identities_and_library():
    x = np.linspace(-12, 12, 100001)
    g = E.gelu(x)
    np.testing.assert_allclose(g - E.gelu(-x), x, rtol=0, atol=1e-14)
    assert E.gelu(np.array([0.0]))[0] == 0.0
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-15)
    # Phi via math.erf at scattered points.
    pts = np.random.default_rng(2).standard_normal(2000) * 4
    want = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in pts])
    np.testing.assert_allclose(E.gelu(pts), want, rtol=1e-14, atol=1e-15)
    # The tanh approximation differs by up to ~4.7e-4: the oracle must not be it.
    tanh = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(g - tanh)) > 1e-4


def test_layer_norm_moments_and_library():
    rng = np.random.default_rng(3)
    x = rand(rng, 64, 96) * 3 + 1.5
    y = E.layer_norm(x, np.ones(96), np.zeros(96), eps=1e-5)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    g, b = 1 + rand(rng, 96, scale=0.3), rand(rng, 96)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(E.layer_norm(x, g, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_conv_matches_textbook_correlation():
    rng = np.random.default_rng(4)
    c_in, c_out, n = 5, 4, 23
    x, w, b = rand(rng, c_in, n), rand(rng, c_out, c_in, 3), rand(rng, c_out)
    for stride in (1, 2):
        y = E.conv1d_k3(x, w, b, stride)
        full = np.stack([
            b[o] + sum(np.correlate(np.pad(x[c], 1), w[o, c], mode="valid") for c in range(c_in))
            for o in range(c_out)])
        np.testing.assert_allclose(y, full[:, ::stride], rtol=1e-12, atol=1e-12)
        ref = torch.nn.functional.conv1d(torch.from_numpy(x)[None], torch.from_numpy(w),
                                         torch.from_numpy(b), stride=stride, padding=1)[0].numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_sinusoids_closed_form():
    d, t = 256, 1500
    pe = E.sinusoids(t, d)
    half = d // 2
    np.testing.assert_array_equal(pe[0, :half], 0.0)
    np.testing.assert_array_equal(pe[0, half:], 1.0)
    np.testing.assert_allclose(pe[:, :half] ** 2 + pe[:, half:] ** 2, 1.0, atol=1e-13)
    # Timescales run from 1 (first pair) to 10000 (last pair): position 1 is
    # sin(1) in the first column and sin(1e-4) in the last sine column.
    assert pe[1, 0] == pytest.approx(math.sin(1.0), abs=1e-15)
    assert pe[1, half - 1] == pytest.approx(math.sin(1e-4), rel=1e-12)
    assert pe[7, half] == pytest.approx(math.cos(7.0), abs=1e-15)
    # Frequencies are geometric: the angle ratio between adjacent columns is constant.
    ang = np.arcsin(pe[1, :half])
    np.testing.assert_allclose(ang[1:] / ang[:-1], 10000.0 ** (-1.0 / (half - 1)), rtol=1e-10)


# ---------------------------------------------------------------------------
# Attention (P4, P5, P6 ii-iii, P9)
# ---------------------------------------------------------------------------

def brute_attention(a, lw, n_heads, key_mask=None):
    """Triple loops over positions, heads and features; [out, in] weights."""
    t, d = a.shape
    dh = d // n_heads
    def lin(w, b, i, o):
        return sum(w[o][c] * a[i][c] for c in range(d)) + (0.0 if b is None else b[o])
    q = [[lin(lw["q_w"], lw["q_b"], i, o) for o in range(d)] for i in range(t)]
    k = [[lin(lw["k_w"], None, i, o) for o in range(d)] for i in range(t)]
    v = [[lin(lw["v_w"], lw["v_b"], i, o) for o in range(d)] for i in range(t)]
    cat = [[0.0] * d for _ in range(t)]
    for h in range(n_heads):
        for i in range(t):
            scores = []
            for j in range(t):
                if key_mask is not None and not key_mask[j]:
                    scores.append(None)
                    continue
                s = sum(q[i][h * dh + e] * k[j][h * dh + e] for e in range(dh)) / math.sqrt(dh)
                scores.append(s)
            m = max(s for s in scores if s is not None)
            ex = [0.0 if s is None else math.exp(s - m) for s in scores]
            z = sum(ex)
            for e in range(dh):
                cat[i][h * dh + e] = sum(ex[j] / z * v[j][h * dh + e] for j in range(t))
    return np.array([[sum(lw["o_w"][o][c] * cat[i][c] for c in range(d)) + lw["o_b"][o]
                      for o in range(d)] for i in range(t)])


@pytest.mark.parametrize("masked", [False, True])
def test_attention_brute_force(masked):
    rng = np.random.default_rng(5)
    t, d, h = 7, 8, 2
    lw = rand_layer(rng, d, 16, scale=0.6)
    a = rand(rng, t, d)
    mask = np.array([1, 1, 0, 1, 1, 1, 0], np.uint8) if masked else None
    got = E.attention(a, lw, h, key_mask=mask)
    np.testing.assert_allclose(got, brute_attention(a, lw, h, mask), rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one_and_masked_columns_are_zero():
    rng = np.random.default_rng(6)
    t, d, h = 40, 32, 4
    lw = rand_layer(rng, d, 64, scale=1.0)
    mask = (rng.random(t) > 0.3).astype(np.uint8)
    mask[0] = 1
    _, p = E.attention(rand(rng, t, d), lw, h, key_mask=mask, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-12)
    assert np.all(p[:, :, mask == 0] == 0.0)
    assert np.all(p[:, :, mask == 1] > 0.0)


def test_attention_vs_torch_sdpa():
    rng = np.random.default_rng(7)
    t, d, h = 33, 64, 4
    lw = rand_layer(rng, d, 64, scale=0.3)
    a = rand(rng, t, d)
    mask = np.ones(t, np.uint8)
    mask[25:] = 0
    got = E.attention(a, lw, h, key_mask=mask)
    mha = torch.nn.MultiheadAttention(d, h, bias=True, batch_first=True)
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([lw["q_w"], lw["k_w"], lw["v_w"]])))
        mha.in_proj_bias.copy_(torch.from_numpy(np.concatenate([lw["q_b"], np.zeros(d), lw["v_b"]])))
        mha.out_proj.weight.copy_(torch.from_numpy(lw["o_w"]))
        mha.out_proj.bias.copy_(torch.from_numpy(lw["o_b"]))
        ref, _ = mha(*(torch.from_numpy(a)[None],) * 3, key_padding_mask=torch.from_numpy(mask == 0)[None],
                     need_weights=False)
    np.testing.assert_allclose(got, ref[0].numpy(), rtol=1e-11, atol=1e-12)


def test_attention_single_position_is_value_projection():
    rng = np.random.default_rng(8)
    d = 16
    lw = rand_layer(rng, d, 32, scale=0.5)
    a = rand(rng, 1, d)
    want = E.linear(E.linear(a, lw["v_w"], lw["v_b"]), lw["o_w"], lw["o_b"])
    np.testing.assert_allclose(E.attention(a, lw, 2), want, rtol=1e-13, atol=1e-13)


def test_zero_queries_give_masked_mean_of_values():
    rng = np.random.default_rng(9)
    t, d, h = 12, 16, 2
    lw = rand_layer(rng, d, 32, scale=0.5)
    lw["q_w"] = np.zeros((d, d))
    lw["q_b"] = np.zeros(d)
    a = rand(rng, t, d)
    mask = np.array([1] * 8 + [0] * 4, np.uint8)
    v = E.linear(a, lw["v_w"], lw["v_b"])
    mean = v[mask == 1].mean(axis=0)
    want = E.linear(np.tile(mean, (t, 1)), lw["o_w"], lw["o_b"])
    np.testing.assert_allclose(E.attention(a, lw, h, key_mask=mask), want, rtol=1e-12, atol=1e-13)


def test_key_bias_does_not_change_the_output():
    rng = np.random.default_rng(10)
    t, d, h = 20, 32, 2
    lw = rand_layer(rng, d, 64, scale=0.5)
    x = rand(rng, t, d)
    mask = np.array([1] * 15 + [0] * 5, np.uint8)
    for m in (None, mask):
        base = E.block(x, lw, h, key_mask=m)
        kb = E.block(x, lw, h, key_mask=m, k_bias=rand(rng, d))
        np.testing.assert_allclose(kb, base, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Blocks and the whole tower (P6 i, P8, P10, P11)
# ---------------------------------------------------------------------------

def torch_layer(lw, d, f, h, eps):
    layer = torch.nn.TransformerEncoderLayer(d, h, dim_feedforward=f, dropout=0.0, activation="gelu",
                                             layer_norm_eps=eps, batch_first=True, norm_first=True)
    with torch.no_grad():
        sa = layer.self_attn
        sa.in_proj_weight.copy_(torch.from_numpy(np.concatenate([lw["q_w"], lw["k_w"], lw["v_w"]])))
        sa.in_proj_bias.copy_(torch.from_numpy(np.concatenate([lw["q_b"], np.zeros(d), lw["v_b"]])))
        sa.out_proj.weight.copy_(torch.from_numpy(lw["o_w"]))
        sa.out_proj.bias.copy_(torch.from_numpy(lw["o_b"]))
        for name, mod in (("ln1", layer.norm1), ("ln2", layer.norm2)):
            mod.weight.copy_(torch.from_numpy(lw[name + "_g"]))
            mod.bias.copy_(torch.from_numpy(lw[name + "_b"]))
        layer.linear1.weight.copy_(torch.from_numpy(lw["fc1_w"]))
        layer.linear1.bias.copy_(torch.from_numpy(lw["fc1_b"]))
        layer.linear2.weight.copy_(torch.from_numpy(lw["fc2_w"]))
        layer.linear2.bias.copy_(torch.from_numpy(lw["fc2_b"]))
    return layer.eval()


def torch_encoder(g, W, mel, mask=None):
    """The tower assembled from torch.nn modules in float64 (independent of the oracle)."""
    t64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    with torch.no_grad():
        x = t64(mel)
        c1 = torch.nn.Conv1d(g.n_mel, g.d_model, 3, stride=1, padding=1)
        c2 = torch.nn.Conv1d(g.d_model, g.d_model, 3, stride=2, padding=1)
        c1.weight.copy_(t64(W["conv1_w"])); c1.bias.copy_(t64(W["conv1_b"]))
        c2.weight.copy_(t64(W["conv2_w"])); c2.bias.copy_(t64(W["conv2_b"]))
        gelu = torch.nn.GELU()
        h = gelu(c2(gelu(c1(x)))).transpose(1, 2)           # [B, T, d]
        t = h.shape[1]
        half = g.d_model // 2
        inv = torch.exp(-math.log(10000.0) / (half - 1) * torch.arange(half, dtype=torch.float64))
        ang = torch.arange(t, dtype=torch.float64)[:, None] * inv[None, :]
        h = h + torch.cat([torch.sin(ang), torch.cos(ang)], dim=1)[None]
        kpm = None if mask is None else torch.from_numpy(np.asarray(mask) == 0)
        for layer in range(g.n_layers):
            lw = {k: np.asarray(v, np.float64) for k, v in E.layer_weights(W, layer).items()}
            mod = torch_layer(lw, g.d_model, g.d_ffn, g.n_heads, g.ln_eps)
            h = mod(h, src_key_padding_mask=kpm)
        ln = torch.nn.LayerNorm(g.d_model, eps=g.ln_eps)
        ln.weight.copy_(t64(W["lnf_g"])); ln.bias.copy_(t64(W["lnf_b"]))
        y = ln(h)
        if g.pool_step == 2:
            y = torch.nn.functional.avg_pool1d(y.transpose(1, 2), 2, 2).transpose(1, 2)
        if g.stack > 1:   # row-major reshape [B, T, d] -> [B, T / k, k d]
            n = y.shape[1] // g.stack
            y = y[:, :n * g.stack].reshape(y.shape[0], n, g.stack * g.d_model)
        if g.proj_hidden:
            l1 = torch.nn.Linear(g.proj_in, g.proj_hidden)
            l2 = torch.nn.Linear(g.proj_hidden, g.proj_out)
            l1.weight.copy_(t64(W["proj1_w"])); l1.bias.copy_(t64(W["proj1_b"]))
            l2.weight.copy_(t64(W["proj2_w"])); l2.bias.copy_(t64(W["proj2_b"]))
            y = l2(gelu(l1(y)))
        return y.numpy()


TOWER_CASES = {
    "plain": dict(geom=dict(n_frames=40, n_layers=2), init="perturbed"),
    "pool": dict(geom=dict(n_frames=42, n_layers=1, pool_step=2), init="perturbed"),
    "projector": dict(geom=dict(n_frames=24, n_layers=1, proj_hidden=96, proj_out=80), init="perturbed"),
    "paper_init": dict(geom=dict(n_frames=30, n_layers=2), init="paper"),
    "batch_mask": dict(geom=dict(n_frames=50, n_layers=2, batch=3), init="perturbed", lengths=[50, 31, 12]),
    "stack4": dict(geom=dict(n_frames=34, n_layers=1, proj_hidden=96, proj_out=80, stack=4), init="perturbed"),
    "stack4_mask": dict(geom=dict(n_frames=34, n_layers=1, proj_hidden=64, proj_out=48, stack=4, batch=2),
                        init="perturbed", lengths=[34, 21]),
}


def valid_out_rows(g, mask, b):
    """Output rows of clip b that the definition fixes: every position they
    read is valid (a stacked row reads `stack` positions, a pooled row two)."""
    if mask is None:
        return np.ones(g.t_out, bool)
    tb = int(mask[b].sum())
    span = g.stack * g.pool_step
    return (np.arange(g.t_out) + 1) * span <= tb if span > 1 else mask[b][:g.t_out] == 1


@pytest.mark.parametrize("case", sorted(TOWER_CASES))
def test_tower_matches_torch_modules(case):
    spec = TOWER_CASES[case]
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
    got = oracle.encode(g, W, mel, mask)
    ref = torch_encoder(g, W, mel, mask)
    assert got.shape == (g.batch, g.t_out, g.d_out)
    for b in range(g.batch):
        v = valid_out_rows(g, mask, b)
        assert v.any()
        np.testing.assert_allclose(got[b][v], ref[b][v], rtol=1e-10, atol=1e-11)


def test_no_layers_is_stem_plus_final_norm():
    w = tiny_workload(n_frames=16, n_layers=0).replace(init="perturbed")
    g = w.geom
    W = synth.make_weights(w)
    mel = synth.make_mel(w)[0].astype(np.float64)
    # Textbook convolutions via numpy.correlate.
    def conv(x, wt, b, stride):
        full = np.stack([b[o] + sum(np.correlate(np.pad(x[c], 1), wt[o, c], mode="valid")
                                    for c in range(x.shape[0])) for o in range(wt.shape[0])])
        return full[:, ::stride]
    gl = lambda v: np.vectorize(lambda s: 0.5 * s * (1 + math.erf(s / math.sqrt(2))))(v)
    h = gl(conv(gl(conv(mel, W["conv1_w"], W["conv1_b"], 1)), W["conv2_w"], W["conv2_b"], 2)).T
    t, d = h.shape
    pe = np.array([[math.sin(p * 10000 ** (-j / (d // 2 - 1))) for j in range(d // 2)] +
                   [math.cos(p * 10000 ** (-j / (d // 2 - 1))) for j in range(d // 2)] for p in range(t)])
    x = h + pe
    mu = x.mean(1, keepdims=True)
    sd = np.sqrt(((x - mu) ** 2).mean(1, keepdims=True) + g.ln_eps)
    want = (x - mu) / sd * W["lnf_g"] + W["lnf_b"]
    np.testing.assert_allclose(oracle.encode(g, W, mel[None])[0], want, rtol=1e-10, atol=1e-11)


def test_blocks_are_permutation_equivariant():
    rng = np.random.default_rng(11)
    t, d, h, f = 24, 32, 2, 64
    W = {f"layers.{l}.{k}": v for l in range(2) for k, v in rand_layer(rng, d, f, scale=0.3).items()}
    x = rand(rng, t, d)
    perm = rng.permutation(t)
    a = E.blocks(x, W, 2, h)[perm]
    b = E.blocks(x[perm], W, 2, h)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # With a mask the permutation carries the mask along.
    mask = (rng.random(t) > 0.25).astype(np.uint8)
    a = E.blocks(x, W, 2, h, key_mask=mask)[perm]
    b = E.blocks(x[perm], W, 2, h, key_mask=mask[perm])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_padded_frames_do_not_change_valid_rows():
    w = tiny_workload(n_frames=60, n_layers=2).replace(init="perturbed")
    g = w.geom
    W = synth.make_weights(w)
    mel = synth.make_mel(w)[0]
    n_f = 37
    tb = (n_f + 1) // 2
    mel[:, n_f:] = 0.0
    mask = (np.arange(g.n_pos) < tb).astype(np.uint8)
    base = oracle.encode(g, W, mel[None], mask[None])[0]
    # Valid position t reads frames up to 2t + 2 <= 2 T_b; garbage beyond that.
    junk = mel.copy()
    rng = np.random.default_rng(12)
    junk[:, 2 * tb + 1:] = rng.choice([-1e4, 1e4], size=junk[:, 2 * tb + 1:].shape)
    other = oracle.encode(g, W, junk[None], mask[None])[0]
    np.testing.assert_array_equal(other[:tb], base[:tb])
    assert not np.allclose(other[tb:], base[tb:])


def test_clip_independent_of_batch():
    w = tiny_workload(n_frames=32, n_layers=1, batch=3).replace(init="perturbed")
    W = synth.make_weights(w)
    mel = synth.make_mel(w)
    full = oracle.encode(w.geom, W, mel)
    alone = oracle.encode(w.geom.replace(batch=1), W, synth.make_mel(w, clips=[2]))
    np.testing.assert_array_equal(full[2], alone[0])


def test_synth_streams_are_stable():
    w = synth.get_workload("whisper_large_varlen_b32")
    lengths = synth.make_lengths(w)
    assert lengths.min() >= 100 and lengths.max() <= 3000
    mask = synth.make_mask(w)
    np.testing.assert_array_equal(mask.sum(1), (lengths + 1) // 2)
    # Clip i's mel does not depend on the batch it is drawn in.
    tiny = synth.get_workload("tiny_fp32_b1")
    a = synth.make_mel(tiny.replace(geom=tiny.geom.replace(batch=4)))[3]
    b = synth.make_mel(tiny, clips=[3])[0]
    np.testing.assert_array_equal(a, b)
    # bf16 rounding is round-to-nearest-even.
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    r = synth.round_to_bf16(x)
    assert r[1] == 1.0 and r[2] == 1.0 + 2 ** -6 and r[3] == -2.5
