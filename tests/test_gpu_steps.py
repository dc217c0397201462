"""Per-step parity of the HIP kernels (through include/aenc_kernels.h) against
the oracle's functions on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import audio_encoder_tower_amd as aenc
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    aenc.lib()
    return aenc


def bf16(rng, *shape, scale=1.0):
    return synth.round_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV).to(torch.bfloat16)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


ATTN_Q_SCALE = 0.18033688011112042   # log2(e) / sqrt(64): the attention kernel's Q units


def scaled_q(q):
    """Q as the attention kernel sees it: q * ATTN_Q_SCALE rounded to bf16,
    returned divided back (float64) for the oracle; the device gets
    exactly q_back * ATTN_Q_SCALE (= the rounded value, up to float64)."""
    qs = synth.round_to_bf16((q * ATTN_Q_SCALE).astype(np.float32)).astype(np.float64)
    return qs / ATTN_Q_SCALE


GEMM_SHAPES = [
    (300, 384, 320),      # ragged M and N against every tile shape
    (64, 64, 64),
    (1, 200, 128),
    (3000, 5120, 1280),   # FC1 of a Whisper-large clip
    (3000, 1280, 5120),   # FC2
    (777, 1284, 4160),    # ragged M and N, 65 slices: a partial trip of the 6-slice buffer cycle
    (70, 196, 64),        # N = 4 mod 8: 4-column tails and rows not 16-byte aligned
    (4000, 4920, 1280),   # 256x256: 40 tiles per XCD, the last 8 run as 128-column halves (ragged M, N)
    (22700, 760, 128),    # 256x256: 267 tiles (not a multiple of 8): 34 or 33 per XCD, tails of 2 and 1 split
    (24000, 3840, 64),    # 256x256: 1410 tiles: 177 per XCD (tail 17, whole) or 176 (tail 16, split)
]


@pytest.mark.parametrize("tile", ["256x256", "128x128"])
@pytest.mark.parametrize("epi", ["bf16", "gelu_bf16", "resid_f32", "f32"])
@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_bf16(_lib, shape, epi, tile):
    M, N, K = shape
    print(f"gemm {shape} {epi} {tile}", flush=True)
    rng = np.random.default_rng(hash((M, N, K)) % 2**32)
    a, w = bf16(rng, M, K), bf16(rng, N, K, scale=0.05)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    ref = oracle.linear(a.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    c_in = None
    if epi == "resid_f32":
        c_in = rng.standard_normal((M, N)).astype(np.float32)
        ref = ref + c_in
        c = dev_f32(c_in)
    elif epi == "f32":
        c = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float32)
    else:
        c = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    if epi == "gelu_bf16":
        ref = oracle.gelu(ref)
    _lib.steps.gemm_bf16(epi, dev_bf16(a), dev_bf16(w), dev_f32(b), c, tile=tile)
    torch.cuda.synchronize()
    got = host(c)
    scale = np.abs(ref).max()
    if epi in ("bf16", "gelu_bf16"):
        # one bf16 rounding of the fp32 result: half an ulp, 2^-9 relative
        np.testing.assert_allclose(got, ref, rtol=2 ** -8, atol=1e-4 * scale)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2e-6 * scale)


@pytest.mark.parametrize("q_scale", [1.0, 0.18033688011112042], ids=["plain", "attention_q_scale"])
@pytest.mark.parametrize("M,d", [(777, 256), (777, 192), (30000, 192), (8448, 640)],
                         ids=["128x128_tiles", "3_heads", "256x256_tiles_3_heads", "256x256_split_tail_10_heads"])
def test_qkv_split_layout(_lib, q_scale, M, d):
    """[Q|K] row-major and V^T, with the Q scale. With 3 heads the Q|K / V
    split (column 384) falls inside a 256-wide tile, whose two waves then take
    different epilogues (bf16 rows stored from registers, V^T through LDS)."""
    rng = np.random.default_rng(1)
    a = bf16(rng, M, d)
    wqkv = bf16(rng, 3 * d, d, scale=0.05)
    bias = (rng.standard_normal(3 * d) * 0.1).astype(np.float32)
    ld_vt = (M + 63) // 64 * 64 + 64
    qk = torch.empty(M, 2 * d, device=DEV, dtype=torch.bfloat16)
    vt = torch.zeros(d, ld_vt, device=DEV, dtype=torch.bfloat16)
    _lib.steps.qkv_bf16(dev_bf16(a), dev_bf16(wqkv), dev_f32(bias), qk, vt, q_scale=q_scale)
    torch.cuda.synchronize()
    ref = oracle.linear(a.astype(np.float64), wqkv.astype(np.float64), bias.astype(np.float64))
    ref[:, :d] *= q_scale                         # Q columns only
    np.testing.assert_allclose(host(qk), ref[:, :2 * d], rtol=2 ** -8, atol=1e-4)
    np.testing.assert_allclose(host(vt)[:, :M], ref[:, 2 * d:].T, rtol=2 ** -8, atol=1e-4)
    assert np.all(host(vt)[:, M:] == 0)


def test_gelu_device_erf(_lib):
    x = np.concatenate([np.linspace(-12, 12, 200001), [0.0, -0.0, 1e-30, -1e-30, 40.0, -40.0]]).astype(np.float32)
    y = torch.empty(x.size, device=DEV, dtype=torch.float32)
    _lib.steps.gelu_f32(dev_f32(x), y)
    torch.cuda.synchronize()
    ref = oracle.gelu(x.astype(np.float64))
    err = np.abs(host(y) - ref)
    # Abramowitz & Stegun 7.1.26 has |erf error| <= 1.5e-7, so GELU is off by at
    # most |x|/2 * 1.5e-7, plus fp32 rounding of the result.
    bound = 0.5 * np.abs(x) * 1.5e-7 + 4 * np.finfo(np.float32).eps * np.abs(ref) + 1e-30
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("d", [256, 1024, 1280])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_layernorm(_lib, d, out):
    rng = np.random.default_rng(d)
    M = 1003
    x = (rng.standard_normal((M, d)) * 2 + 0.5).astype(np.float32)
    g = (1 + rng.standard_normal(d) * 0.1).astype(np.float32)
    b = (rng.standard_normal(d) * 0.1).astype(np.float32)
    y = torch.empty(M, d, device=DEV, dtype=torch.float32 if out == "f32" else torch.bfloat16)
    _lib.steps.layernorm(dev_f32(x), dev_f32(g), dev_f32(b), y, 1e-5)
    torch.cuda.synchronize()
    ref = oracle.layer_norm(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64), 1e-5)
    if out == "f32":
        np.testing.assert_allclose(host(y), ref, rtol=1e-5, atol=1e-5)
    else:
        np.testing.assert_allclose(host(y), ref, rtol=2 ** -8, atol=1e-6)


@pytest.mark.parametrize("rows,d", [(1003, 1280), (37, 1284), (5, 4)])
def test_row_stream(_lib, rows, d):
    """The LayerNorm-traffic calibration kernel writes bf16(x), round to
    nearest even, for every element (its timing is the LayerNorm's ceiling)."""
    x = torch.randn(rows, d, device=DEV) * 3
    x[0, :4] = torch.tensor([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 65504.0], device=DEV)   # ties, sign
    y = torch.empty(rows, d, device=DEV, dtype=torch.bfloat16)
    _lib.steps.row_stream(x, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), x.to(torch.bfloat16).view(torch.int16))


def test_mfma_loop_clock_ticks(_lib):
    """The MFMA-ceiling loop's optional tick record: every workgroup reports a
    positive shader-clock and real-time count, whose ratio gives a clock in
    the part's range, and the loop's sums are the same with or without it."""
    blocks, iters = 512, 64
    a = torch.empty(blocks * 256, device=DEV)
    b = torch.empty(blocks * 256, device=DEV)
    ticks = torch.zeros(blocks, 2, dtype=torch.int64, device=DEV)
    _lib.steps.mfma_loop(a, blocks, iters)
    _lib.steps.mfma_loop(b, blocks, iters, ticks)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(a).all()) and torch.equal(a, b)
    t = ticks.cpu()
    assert bool((t > 0).all()), t[:4]
    ghz = (t[:, 0].double() / t[:, 1].double()) * 0.1
    print(f"mfma loop clock: median {float(ghz.median()):.3f} GHz", flush=True)
    assert 0.3 < float(ghz.median()) < 3.0


def packing_contract(mask):
    """The packing the library promises: valid positions in order, each clip
    starting on a multiple of 8 rows."""
    B, T = mask.shape
    row_map = np.full(B * T, -1, np.int64)
    cu = np.zeros(B + 1, np.int64)
    base = 0
    inv = {}
    for b in range(B):
        base = (base + 7) // 8 * 8
        cu[b] = base
        for t in range(T):
            if mask[b, t]:
                row_map[b * T + t] = base
                inv[base] = b * T + t
                base += 1
    cu[B] = base
    return row_map, cu, inv


@pytest.mark.parametrize("case", ["all_valid", "prefix", "random", "single"])
def test_row_maps(_lib, case):
    rng = np.random.default_rng(3)
    B, T = 5, 1500
    if case == "all_valid":
        mask = np.ones((B, T), np.uint8)
    elif case == "prefix":
        lens = [1500, 1, 731, 64, 1499]
        mask = (np.arange(T)[None, :] < np.array(lens)[:, None]).astype(np.uint8)
    elif case == "random":
        mask = (rng.random((B, T)) > 0.4).astype(np.uint8)
        mask[:, 0] = 1
    else:
        B, T = 1, 1
        mask = np.ones((1, 1), np.uint8)
    rm, inv, cu, lens, mv = _lib.steps.row_maps(torch.from_numpy(mask).to(DEV), B, T)
    torch.cuda.synchronize()
    want_rm, want_cu, want_inv = packing_contract(mask)
    np.testing.assert_array_equal(rm.cpu().numpy(), want_rm)
    np.testing.assert_array_equal(cu.cpu().numpy(), want_cu)
    np.testing.assert_array_equal(lens.cpu().numpy(), mask.sum(1))
    assert int(mv.item()) == want_cu[-1]
    inv_h = inv.cpu().numpy()
    for r in range(int(want_cu[-1])):
        assert inv_h[r] == want_inv.get(r, -1), r
    if case == "all_valid":
        # the null mask gives the same maps
        rm2, inv2, cu2, lens2, mv2 = _lib.steps.row_maps(None, B, T)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(rm2.cpu().numpy(), want_rm)
        np.testing.assert_array_equal(cu2.cpu().numpy(), want_cu)


@pytest.mark.parametrize("lens,heads,scale", [
    ([1500], 20, 1.0),
    ([731, 64, 1, 129, 1500], 2, 1.5),
    ([100], 4, 3.0),
    ([65, 127, 128, 257], 3, 0.5),
], ids=["whisper_large_clip", "ragged_clips", "sharp", "tile_edges"])
def test_attention_bf16(_lib, lens, heads, scale):
    rng = np.random.default_rng(sum(lens) + heads)
    d = 64 * heads
    starts = [0]
    for n in lens[:-1]:
        starts.append((starts[-1] + n + 7) // 8 * 8)
    rows = starts[-1] + lens[-1]
    q, k, v = (bf16(rng, rows, d, scale=scale) for _ in range(3))
    q = scaled_q(q)
    ld_vt = (rows + 63) // 64 * 64 + 64
    qk = np.concatenate([q * ATTN_Q_SCALE, k], axis=1)
    vt = np.zeros((d, ld_vt), np.float32)
    vt[:, :rows] = v.T
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = torch.full((rows, d), float("nan"), device=DEV, dtype=torch.bfloat16)
    _lib.steps.attention_bf16(dev_bf16(qk), dev_bf16(vt), st, ln, max(lens), heads, out)
    torch.cuda.synchronize()
    got = host(out)
    for s, n in zip(starts, lens):
        sl = slice(s, s + n)
        ref, _ = oracle.attention_core(q[sl].astype(np.float64), k[sl].astype(np.float64),
                                       v[sl].astype(np.float64), heads)
        err = np.abs(got[sl] - ref)
        # P is rounded to bf16 before P V, the output to bf16
        assert err.max() <= 1e-2 * max(1.0, np.abs(v).max()), (n, err.max())
        cos = (got[sl] * ref).sum(1) / (np.linalg.norm(got[sl], axis=1) * np.linalg.norm(ref, axis=1))
        assert cos.min() >= 0.9999, (n, cos.min())


def ranges_from_rule(mask, chunk, mode):
    """Expected key ranges: for each valid position, the packed rows of the
    valid keys that oracle.chunk_allowed lets it see, which must be one
    contiguous run; returned clip-relative, keyed by the query's packed row."""
    B, T = mask.shape
    row_map, cu, _ = packing_contract(mask)
    allowed = oracle.chunk_allowed(T, chunk, mode)
    lo, hi = {}, {}
    for b in range(B):
        valid = mask[b].astype(bool)
        for t in np.flatnonzero(valid):
            keys = np.flatnonzero(allowed[t] & valid)
            packed = row_map[b * T + keys] - cu[b]
            assert np.array_equal(packed, np.arange(packed[0], packed[-1] + 1)), "rule not contiguous"
            r = row_map[b * T + t]
            lo[r], hi[r] = packed[0], packed[-1] + 1
    return lo, hi


@pytest.mark.parametrize("mode", ["causal", "block"])
@pytest.mark.parametrize("case,chunk", [("prefix", 50), ("random", 50), ("random", 7), ("all_valid", 1),
                                        ("prefix", 1500), ("single", 1)])
def test_chunk_ranges(_lib, case, chunk, mode):
    rng = np.random.default_rng(11)
    B, T = 4, 1500
    if case == "all_valid":
        mask = np.ones((B, T), np.uint8)
    elif case == "prefix":
        lens = [1500, 1, 731, 64]
        mask = (np.arange(T)[None, :] < np.array(lens)[:, None]).astype(np.uint8)
    elif case == "random":
        mask = (rng.random((B, T)) > 0.4).astype(np.uint8)
        mask[:, 0] = 1
    else:
        B, T = 1, 1
        mask = np.ones((1, 1), np.uint8)
    md = torch.from_numpy(mask).to(DEV)
    rm, inv, cu, lens, mv = _lib.steps.row_maps(md, B, T)
    rows = int(B * ((T + 7) // 8 * 8))
    key_lo = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    key_hi = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    _lib.steps.chunk_ranges(md, B, T, chunk, mode, rm, cu, key_lo, key_hi)
    torch.cuda.synchronize()
    lo, hi = ranges_from_rule(mask, chunk, oracle.CHUNK_CAUSAL if mode == "causal" else oracle.CHUNK_BLOCK)
    got_lo, got_hi = key_lo.cpu().numpy(), key_hi.cpu().numpy()
    for r in lo:
        assert (got_lo[r], got_hi[r]) == (lo[r], hi[r]), (r, got_lo[r], got_hi[r], lo[r], hi[r])
    untouched = np.setdiff1d(np.arange(rows), np.array(list(lo)))
    assert np.all(got_lo[untouched] == -7) and np.all(got_hi[untouched] == -7)


@pytest.mark.parametrize("lens,heads,chunk,mode", [
    ([1500], 4, 50, "causal"),
    ([731, 64, 1, 129], 2, 50, "block"),
    ([300], 2, 1, "block"),
    ([300], 2, 1, "causal"),
    ([257, 511], 3, 128, "causal"),
    ([1000], 2, 37, "block"),
    ([200], 2, 500, "causal"),
], ids=["whisper_large_1s_causal", "ragged_block", "one_block", "one_causal", "tile_aligned", "odd_block",
        "chunk_covers_clip"])
def test_attention_bf16_chunked(_lib, lens, heads, chunk, mode):
    """Ranged attention (ranges from aenc_k_chunk_ranges over all-valid clips)
    against the oracle's chunked attention on every row."""
    rng = np.random.default_rng(sum(lens) + chunk)
    d = 64 * heads
    B, T = len(lens), max(lens)
    mask = (np.arange(T)[None, :] < np.array(lens)[:, None]).astype(np.uint8)
    md = torch.from_numpy(mask).to(DEV)
    rm, inv, cu_d, ln_d, mv = _lib.steps.row_maps(md, B, T)
    cu = cu_d.cpu().numpy()
    rows = int(cu[-1])
    key_lo = torch.zeros(rows + 8, dtype=torch.int32, device=DEV)
    key_hi = torch.zeros(rows + 8, dtype=torch.int32, device=DEV)
    _lib.steps.chunk_ranges(md, B, T, chunk, mode, rm, cu_d, key_lo, key_hi)
    q, k, v = (bf16(rng, rows, d, scale=1.5) for _ in range(3))
    q = scaled_q(q)
    ld_vt = (rows + 63) // 64 * 64 + 64
    qk = np.concatenate([q * ATTN_Q_SCALE, k], axis=1)
    vt = np.zeros((d, ld_vt), np.float32)
    vt[:, :rows] = v.T
    out = torch.full((rows, d), float("nan"), device=DEV, dtype=torch.bfloat16)
    _lib.steps.attention_bf16(dev_bf16(qk), dev_bf16(vt), cu_d, ln_d, T, heads, out, key_lo, key_hi)
    torch.cuda.synchronize()
    got = host(out)
    rule = oracle.CHUNK_CAUSAL if mode == "causal" else oracle.CHUNK_BLOCK
    for b, n in enumerate(lens):
        sl = slice(int(cu[b]), int(cu[b]) + n)
        ref, _ = oracle.attention_core(q[sl].astype(np.float64), k[sl].astype(np.float64),
                                       v[sl].astype(np.float64), heads, None, oracle.chunk_allowed(n, chunk, rule))
        err = np.abs(got[sl] - ref)
        assert err.max() <= 1e-2 * max(1.0, np.abs(v).max()), (n, err.max())
        cos = (got[sl] * ref).sum(1) / (np.linalg.norm(got[sl], axis=1) * np.linalg.norm(ref, axis=1))
        assert cos.min() >= 0.9999, (n, cos.min())
