"""fp64 NumPy oracle of the Whisper-style audio encoder tower.

Test infrastructure only (see the package docstring). Each function states
the passage it follows. The pages fix the geometry and the structure:

  * "Qwen2-Audio-7B-Instruct", section "(1) AUDIO ENCODER": a Whisper-large
    encoder (d_model 1280, 32 layers, 20 heads, FFN 5120, gelu, 128 mel bins,
    1500 positions per 30 s window), a single bidirectional pass with no KV
    cache; linear weights are stored [out, in] (q_proj.weight [1280, 1280]).
  * "Voxtral-Mini-3B-2507", sections "(1) AUDIO ENCODER", "Preprocessor" and
    "PROJECTOR": head_dim 64 with 20 query and 20 KV heads (plain multi-head
    attention), 3000 feature frames per 30 s chunk, and a 2-layer MLP with
    gelu from the 1280-wide encoder to the 3072-wide LLM.
  * "MiniCPM-o-2_6", section "(2) AUDIO": the Whisper-medium encoder
    (1024 / 24 layers / 16 heads / FFN 4096) and audio_pool_step 2, which
    halves 1500 positions to about 750.

Where the pages say nothing, this file takes the plain Whisper reading:
two k=3 convolutions with padding 1 (stride 1, then 2), each followed by
GELU; sinusoidal positions laid out [sin | cos] with timescales from 1 to
10000; pre-LayerNorm blocks (eps 1e-5, biased variance); scores scaled by
1/sqrt(head_dim); no key bias; GELU in its exact erf form; a final
LayerNorm; the pool averages position pairs after the final LayerNorm.

Everything is computed in float64 (or the dtype passed in) from the exact
values of the seeded inputs; there is no blocking, fusion or reordering
beyond what the definitions state.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

LN_EPS = 1e-5
POS_MAX_TIMESCALE = 10000.0


# --------------------------------------------------------------------------
# Elementary steps
# --------------------------------------------------------------------------

def gelu(x: np.ndarray) -> np.ndarray:
    """GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), the exact form.

    The activation is named "gelu" in the encoder configs ("Qwen2-Audio-7B-
    Instruct" and "Voxtral-Mini-3B-2507", "(1) AUDIO ENCODER") and as
    projector_hidden_act ("Voxtral-Mini-3B-2507", "PROJECTOR").
    """
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return gamma * (x - mu) / np.sqrt(var + eps) + beta


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x W^T + b with W stored [out, in] (the checkpoint convention of the
    "Qwen2-Audio-7B-Instruct" record's tensor-shape notes)."""
    y = x @ w.T
    return y if b is None else y + b


def conv1d_k3(x: np.ndarray, w: np.ndarray, b: np.ndarray, stride: int) -> np.ndarray:
    """1-D convolution, kernel 3, zero padding 1, channels-first.

    x [C_in, F], w [C_out, C_in, 3], b [C_out] -> [C_out, F_out] with
    F_out = floor((F + 2 - 3) / stride) + 1 and
    out[o, t] = b[o] + sum_{c, k} w[o, c, k] * x[c, stride*t + k - 1].
    Written as an explicit gather of the three taps and one matmul.
    """
    c_in, n = x.shape
    n_out = (n + 2 * 1 - 3) // stride + 1
    xp = np.zeros((c_in, n + 2), dtype=x.dtype)
    xp[:, 1:n + 1] = x
    cols = np.empty((n_out, c_in, 3), dtype=x.dtype)
    for k in range(3):
        cols[:, :, k] = xp[:, k: k + stride * (n_out - 1) + 1: stride].T
    y = cols.reshape(n_out, c_in * 3) @ w.reshape(w.shape[0], c_in * 3).T
    return (y + b).T


def sinusoids(n_pos: int, d: int, dtype=np.float64) -> np.ndarray:
    """Sinusoidal positions [n_pos, d]: [sin(t w_j) | cos(t w_j)], j < d/2,
    with w_j = exp(-j ln(10000) / (d/2 - 1)) (timescales 1 ... 10000)."""
    half = d // 2
    inc = math.log(POS_MAX_TIMESCALE) / (half - 1)
    omega = np.exp(-inc * np.arange(half, dtype=np.float64))
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * omega[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1).astype(dtype)


# --------------------------------------------------------------------------
# The encoder
# --------------------------------------------------------------------------

def _f(a, dtype):
    return np.asarray(a, dtype=dtype)


CHUNK_CAUSAL = 1
CHUNK_BLOCK = 2


def chunk_allowed(t: int, chunk: int, mode: int) -> np.ndarray:
    """allowed[q, k] of chunked attention over t positions (parity unpinned as
    a reading: "MiniCPM-o-2_6", section "(2) AUDIO", prints audio_chunk_length
    1.0 next to its Whisper encoder but not what the encoder does with it).

    Positions are cut into chunks of `chunk` consecutive positions, c(p) =
    floor(p / chunk). Chunk-causal (mode 1): query q sees key k when
    c(k) <= c(q), i.e. its own chunk and every earlier one, as a streaming
    encoder that is fed one chunk at a time would. Block-diagonal (mode 2):
    c(k) == c(q). chunk 0 or mode 0: every key is allowed.
    """
    if chunk <= 0 or mode == 0:
        return np.ones((t, t), dtype=bool)
    c = np.arange(t) // chunk
    if mode == CHUNK_CAUSAL:
        return c[None, :] <= c[:, None]
    if mode == CHUNK_BLOCK:
        return c[None, :] == c[:, None]
    raise ValueError(f"chunk mode {mode} must be 0, 1 or 2")


def attention(a: np.ndarray, lw: Dict[str, np.ndarray], n_heads: int,
              key_mask: Optional[np.ndarray] = None, k_bias: Optional[np.ndarray] = None,
              return_probs: bool = False, dtype=np.float64, allowed: Optional[np.ndarray] = None):
    """Bidirectional multi-head self-attention with an output projection.

    One pass over all positions, no causal mask and nothing cached ("Qwen2-
    Audio-7B-Instruct", "(1) AUDIO ENCODER": single bidirectional pass); as
    many KV heads as query heads, head_dim = d/H ("Voxtral-Mini-3B-2507",
    "(1) AUDIO ENCODER"). Keys with key_mask == 0 get probability 0.

    a [T, d] (the LayerNorm output) -> concat_h(O_h) W_o^T + b_o, [T, d].
    """
    q = linear(a, _f(lw["q_w"], dtype), _f(lw["q_b"], dtype))
    k = linear(a, _f(lw["k_w"], dtype), None if k_bias is None else _f(k_bias, dtype))
    v = linear(a, _f(lw["v_w"], dtype), _f(lw["v_b"], dtype))
    o, p = attention_core(q, k, v, n_heads, key_mask, allowed)
    out = linear(o, _f(lw["o_w"], dtype), _f(lw["o_b"], dtype))
    return (out, p) if return_probs else out


def attention_core(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int,
                   key_mask: Optional[np.ndarray] = None, allowed: Optional[np.ndarray] = None):
    """Per head h: softmax_j(Q_h K_h^T / sqrt(dh)) V_h, heads concatenated.

    q, k, v [T, d] -> (o [T, d], probabilities [H, T, T]). Keys with
    key_mask == 0, and keys with allowed[q, k] False, get probability 0; each
    row is normalised after subtracting its maximum. A row left with no key
    at all (only possible for a masked query under a chunk rule) is zero.
    """
    t, d = q.shape
    dh = d // n_heads
    qh = q.reshape(t, n_heads, dh).transpose(1, 0, 2)
    kh = k.reshape(t, n_heads, dh).transpose(1, 0, 2)
    vh = v.reshape(t, n_heads, dh).transpose(1, 0, 2)
    s = (qh @ kh.transpose(0, 2, 1)) / math.sqrt(dh)          # [H, T, T]
    ok = np.ones((t, t), dtype=bool)
    if key_mask is not None:
        ok &= np.asarray(key_mask, bool)[None, :]
    if allowed is not None:
        ok &= np.asarray(allowed, bool)
    if key_mask is not None or allowed is not None:
        s = np.where(ok[None], s, -np.inf)
    empty = ~ok.any(axis=1)                                     # [T]
    m = s.max(axis=-1, keepdims=True)
    m = np.where(empty[None, :, None], 0.0, m)
    p = np.exp(s - m)
    den = p.sum(axis=-1, keepdims=True)
    p = p / np.where(empty[None, :, None], 1.0, den)
    o = (p @ vh).transpose(1, 0, 2).reshape(t, d)
    return o, p


def block(x: np.ndarray, lw: Dict[str, np.ndarray], n_heads: int,
          key_mask: Optional[np.ndarray] = None, eps: float = LN_EPS,
          k_bias: Optional[np.ndarray] = None, dtype=np.float64,
          allowed: Optional[np.ndarray] = None) -> np.ndarray:
    """One pre-LayerNorm block: x + Attn(LN1 x), then + FFN(LN2 x) with
    FFN(h) = GELU(h W1^T + b1) W2^T + b2 (encoder_ffn_dim wide)."""
    a = layer_norm(x, _f(lw["ln1_g"], dtype), _f(lw["ln1_b"], dtype), eps)
    x = x + attention(a, lw, n_heads, key_mask, k_bias=k_bias, dtype=dtype, allowed=allowed)
    h = layer_norm(x, _f(lw["ln2_g"], dtype), _f(lw["ln2_b"], dtype), eps)
    h = gelu(linear(h, _f(lw["fc1_w"], dtype), _f(lw["fc1_b"], dtype)))
    return x + linear(h, _f(lw["fc2_w"], dtype), _f(lw["fc2_b"], dtype))


def layer_weights(W: Dict[str, np.ndarray], layer: int) -> Dict[str, np.ndarray]:
    pre = f"layers.{layer}."
    return {k[len(pre):]: v for k, v in W.items() if k.startswith(pre)}


def blocks(x: np.ndarray, W: Dict[str, np.ndarray], n_layers: int, n_heads: int,
           key_mask: Optional[np.ndarray] = None, eps: float = LN_EPS, dtype=np.float64,
           allowed: Optional[np.ndarray] = None) -> np.ndarray:
    for layer in range(n_layers):
        x = block(x, layer_weights(W, layer), n_heads, key_mask, eps, dtype=dtype, allowed=allowed)
    return x


def stem(mel: np.ndarray, W: Dict[str, np.ndarray], dtype=np.float64) -> np.ndarray:
    """Conv stem and positions: mel [n_mel, F] -> X [T, d].

    GELU(conv(k3, s1)) then GELU(conv(k3, s2)), so 3000 frames give the 1500
    positions of a 30 s chunk ("Voxtral-Mini-3B-2507", "Preprocessor"
    nb_max_frames 3000 and "(1) AUDIO ENCODER" 1500 positions); then the
    sinusoidal position table is added.
    """
    x = _f(mel, dtype)
    g1 = gelu(conv1d_k3(x, _f(W["conv1_w"], dtype), _f(W["conv1_b"], dtype), stride=1))
    g2 = gelu(conv1d_k3(g1, _f(W["conv2_w"], dtype), _f(W["conv2_b"], dtype), stride=2))
    xt = g2.T
    return xt + sinusoids(xt.shape[0], xt.shape[1], dtype)


def stack_rows(y: np.ndarray, k: int) -> np.ndarray:
    """Concatenate each run of k consecutive positions into one row:
    row j = [y[k j], y[k j + 1], ..., y[k j + k - 1]]; a trailing partial run
    is dropped.

    Whisper features downsampled from 50 to 12.5 positions per second
    ("[WIP][TSS][Model] Kimi-Audio-7B", Purpose, Audio Tokenizer) into an
    adaptor input of 5120 = 4 x 1280 ("Kimi-Audio-7B-Instruct", (1) AUDIO,
    kimia_adaptor_input_dim).
    """
    n, d = y.shape[0] // k, y.shape[1]
    out = np.empty((n, k * d), dtype=y.dtype)
    for j in range(n):
        for i in range(k):
            out[j, i * d:(i + 1) * d] = y[k * j + i]
    return out


def final(x: np.ndarray, W: Dict[str, np.ndarray], pool_step: int = 1, eps: float = LN_EPS,
          dtype=np.float64, stack: int = 1) -> np.ndarray:
    """Final LayerNorm, then the optional pool or projector.

    pool_step 2 averages positions (2j, 2j+1), j < floor(T/2) ("MiniCPM-o-2_6",
    "(2) AUDIO": audio_pool_step 2, 1500 -> ~750). The projector is
    GELU(Y Wp1^T + bp1) Wp2^T + bp2 ("Voxtral-Mini-3B-2507", "PROJECTOR");
    with stack > 1 its input rows are runs of `stack` consecutive positions
    (stack_rows).
    """
    y = layer_norm(x, _f(W["lnf_g"], dtype), _f(W["lnf_b"], dtype), eps)
    if pool_step == 2:
        n = y.shape[0] // 2
        y = (y[0:2 * n:2] + y[1:2 * n:2]) / 2.0
    elif pool_step != 1:
        raise ValueError("pool_step must be 1 or 2")
    if stack != 1:
        if pool_step != 1 or "proj1_w" not in W:
            raise ValueError("stacking feeds the projector and is not combined with the pool")
        y = stack_rows(y, stack)
    if "proj1_w" in W:
        if pool_step != 1:
            raise ValueError("pool and projector together are not defined")
        h = gelu(linear(y, _f(W["proj1_w"], dtype), _f(W["proj1_b"], dtype)))
        y = linear(h, _f(W["proj2_w"], dtype), _f(W["proj2_b"], dtype))
    return y


def encode_clip(geom, W: Dict[str, np.ndarray], mel: np.ndarray,
                key_mask: Optional[np.ndarray] = None, dtype=np.float64,
                n_layers: Optional[int] = None) -> np.ndarray:
    """One clip: mel [n_mel, F] -> [T_out, D_out]. n_layers overrides the
    geometry's depth (used to time a bounded sample)."""
    depth = geom.n_layers if n_layers is None else n_layers
    x = stem(mel, W, dtype)
    chunk = getattr(geom, "attn_chunk", 0)
    allowed = chunk_allowed(x.shape[0], chunk, getattr(geom, "attn_chunk_mode", 0)) if chunk else None
    x = blocks(x, W, depth, geom.n_heads, key_mask, geom.ln_eps, dtype, allowed=allowed)
    return final(x, W, geom.pool_step, geom.ln_eps, dtype, getattr(geom, "stack", 1))


def encode(geom, W: Dict[str, np.ndarray], mel: np.ndarray, mask: Optional[np.ndarray] = None,
           dtype=np.float64) -> np.ndarray:
    """A batch: mel [B, n_mel, F], mask uint8 [B, T] or None -> [B, T_out, D_out].

    Clips are independent (fixed 30 s chunks, "Voxtral-Mini-3B-2507",
    "STREAMING vs OFFLINE"); rows of masked positions are computed by the same
    definition but carry no meaning.
    """
    outs = [encode_clip(geom, W, mel[b], None if mask is None else mask[b], dtype)
            for b in range(mel.shape[0])]
    return np.stack(outs)


# --------------------------------------------------------------------------
# Closed forms used for accounting
# --------------------------------------------------------------------------

def param_shapes(geom) -> List[Tuple[str, Tuple[int, ...]]]:
    """Every trainable tensor the oracle reads, with its shape."""
    d, f, m = geom.d_model, geom.d_ffn, geom.n_mel
    shapes = [("conv1_w", (d, m, 3)), ("conv1_b", (d,)), ("conv2_w", (d, d, 3)), ("conv2_b", (d,))]
    for layer in range(geom.n_layers):
        p = f"layers.{layer}."
        shapes += [(p + "ln1_g", (d,)), (p + "ln1_b", (d,)),
                   (p + "q_w", (d, d)), (p + "q_b", (d,)), (p + "k_w", (d, d)),
                   (p + "v_w", (d, d)), (p + "v_b", (d,)), (p + "o_w", (d, d)), (p + "o_b", (d,)),
                   (p + "ln2_g", (d,)), (p + "ln2_b", (d,)),
                   (p + "fc1_w", (f, d)), (p + "fc1_b", (f,)), (p + "fc2_w", (d, f)), (p + "fc2_b", (d,))]
    shapes += [("lnf_g", (d,)), ("lnf_b", (d,))]
    if geom.proj_hidden:
        shapes += [("proj1_w", (geom.proj_hidden, getattr(geom, "stack", 1) * d)), ("proj1_b", (geom.proj_hidden,)),
                   ("proj2_w", (geom.proj_out, geom.proj_hidden)), ("proj2_b", (geom.proj_out,))]
    return shapes


def param_count(geom, with_projector: bool = True) -> int:
    return sum(int(np.prod(s)) for n, s in param_shapes(geom)
               if with_projector or not n.startswith("proj"))


def attended_pairs(tb: int, chunk: int = 0, mode: int = 0) -> int:
    """(query, key) pairs among tb valid positions that the chunk rule allows."""
    if chunk <= 0 or mode == 0:
        return tb * tb
    total = 0
    for q in range(tb):
        c = q // chunk
        hi = min(tb, chunk * (c + 1))
        total += hi - (chunk * c if mode == CHUNK_BLOCK else 0)
    return total


def flops(geom, frames: Optional[Sequence[int]] = None) -> float:
    """Algorithmic FLOPs (2 per multiply-add) of one forward.

    frames: valid mel frames per clip (default: all F for every clip). A clip
    of n_f frames has T_b = ceil(n_f/2) valid positions; only valid rows and
    valid key pairs count. LayerNorm, GELU, pool and softmax are not counted.
    """
    d, f, m = geom.d_model, geom.d_ffn, geom.n_mel
    frames = [geom.n_frames] * geom.batch if frames is None else list(frames)
    total = 0.0
    for nf in frames:
        tb = (int(nf) + 1) // 2
        total += 2.0 * nf * d * 3 * m                     # conv1
        total += 2.0 * tb * d * 3 * d                     # conv2
        pairs = attended_pairs(tb, getattr(geom, "attn_chunk", 0), getattr(geom, "attn_chunk_mode", 0))
        per_layer = 2.0 * tb * (3 * d * d + d * d + 2 * d * f) + 4.0 * pairs * d
        total += geom.n_layers * per_layer
        if geom.proj_hidden:
            k = getattr(geom, "stack", 1)
            total += 2.0 * (tb // k) * (k * d * geom.proj_hidden + geom.proj_hidden * geom.proj_out)
    return total
