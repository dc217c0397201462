"""Single steps of the tower (include/aenc_kernels.h) on torch device tensors.

Marshalling only: shapes are checked here, the work is one library kernel
enqueued on torch's current stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import check, lib

EPI = {"bf16": 0, "gelu_bf16": 1, "resid_f32": 2, "f32": 3}
TILE = {"auto": -1, "256x256": 0, "128x128": 1}


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device contiguous tensors only"
    return ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def gemm_bf16(epi: str, a: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], c: torch.Tensor,
              tile: str = "auto") -> torch.Tensor:
    """c = epi(a w^T + bias); a [M, K] bf16, w [N, K] bf16, bias fp32 [N]."""
    M, K = a.shape
    N = w.shape[0]
    assert a.dtype == w.dtype == torch.bfloat16 and w.shape[1] == K and c.shape == (M, N)
    assert bias is None or (bias.dtype == torch.float32 and bias.numel() == N)
    want = torch.bfloat16 if epi in ("bf16", "gelu_bf16") else torch.float32
    assert c.dtype == want, f"epilogue {epi} writes {want}, got a {c.dtype} output"
    check(lib().aenc_k_gemm_bf16(EPI[epi], _p(a), K, _p(w), _p(bias), _p(c), N, M, N, K, TILE[tile], _s()),
          "aenc_k_gemm_bf16")
    return c


# Q scale the attention kernel expects: log2(e) / sqrt(64) (scores as base-2 exponents).
ATTN_Q_SCALE = 0.18033688011112042


def qkv_bf16(a: torch.Tensor, wqkv: torch.Tensor, bias: Optional[torch.Tensor], qk: torch.Tensor,
             vt: torch.Tensor, q_scale: float = 1.0) -> None:
    M, d = a.shape
    assert wqkv.shape == (3 * d, d) and qk.shape == (M, 2 * d) and vt.shape[0] == d
    check(lib().aenc_k_qkv_bf16(_p(a), _p(wqkv), _p(bias), q_scale, _p(qk), _p(vt), vt.shape[1], M, d, _s()),
          "aenc_k_qkv_bf16")


def attention_bf16(qk: torch.Tensor, vt: torch.Tensor, start: torch.Tensor, lens: torch.Tensor, max_len: int,
                   n_heads: int, out: torch.Tensor, key_lo: Optional[torch.Tensor] = None,
                   key_hi: Optional[torch.Tensor] = None) -> torch.Tensor:
    d = 64 * n_heads
    assert qk.shape[1] == 2 * d and vt.shape[0] == d and out.shape == (qk.shape[0], d)
    assert start.dtype == lens.dtype == torch.int32 and start.numel() >= lens.numel()
    assert (key_lo is None) == (key_hi is None)
    if key_lo is not None:
        assert key_lo.dtype == key_hi.dtype == torch.int32
        assert key_lo.numel() >= qk.shape[0] and key_hi.numel() >= qk.shape[0]
    check(lib().aenc_k_attention_bf16(_p(qk), _p(vt), vt.shape[1], _p(start), _p(lens), lens.numel(), max_len,
                                      n_heads, _p(key_lo), _p(key_hi), _p(out), _s()), "aenc_k_attention_bf16")
    return out


CHUNK_MODE = {"causal": 1, "block": 2}


def chunk_ranges(mask: Optional[torch.Tensor], B: int, T: int, chunk: int, mode: str, row_map: torch.Tensor,
                 cu: torch.Tensor, key_lo: torch.Tensor, key_hi: torch.Tensor) -> None:
    """Per packed row, the clip-relative key range of a chunk rule (aenc_k_chunk_ranges)."""
    assert mask is None or (mask.dtype == torch.uint8 and mask.shape == (B, T))
    assert row_map.numel() >= B * T and cu.numel() >= B + 1
    check(lib().aenc_k_chunk_ranges(_p(mask), B, T, chunk, CHUNK_MODE[mode], _p(row_map), _p(cu), _p(key_lo),
                                    _p(key_hi), _s()), "aenc_k_chunk_ranges")


def layernorm(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, y: torch.Tensor, eps: float) -> torch.Tensor:
    M, d = x.shape
    assert x.dtype == gamma.dtype == beta.dtype == torch.float32 and y.shape == (M, d)
    assert y.dtype in (torch.float32, torch.bfloat16)
    y_code = 1 if y.dtype == torch.bfloat16 else 0
    check(lib().aenc_k_layernorm(_p(x), _p(gamma), _p(beta), _p(y), y_code, M, d, eps, _s()), "aenc_k_layernorm")
    return y


def gelu_f32(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    assert x.dtype == y.dtype == torch.float32 and x.numel() == y.numel()
    check(lib().aenc_k_gelu_f32(_p(x), _p(y), x.numel(), _s()), "aenc_k_gelu_f32")
    return y


def row_maps(mask: Optional[torch.Tensor], B: int, T: int):
    """Packing maps of a key mask: (row_map, inv_map, cu, lens, m_valid) int32 device tensors."""
    dev = torch.device("cuda")
    T8 = (T + 7) // 8 * 8
    row_map = torch.empty(B * T, dtype=torch.int32, device=dev)
    inv_map = torch.empty(B * T8, dtype=torch.int32, device=dev)
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    lens = torch.empty(B, dtype=torch.int32, device=dev)
    mv = torch.empty(1, dtype=torch.int32, device=dev)
    check(lib().aenc_k_row_maps(_p(mask), B, T, _p(row_map), _p(inv_map), _p(cu), _p(lens), _p(mv), _s()),
          "aenc_k_row_maps")
    return row_map, inv_map, cu, lens, mv


def copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    check(lib().aenc_k_copy(_p(dst), _p(src), nbytes, _s()), "aenc_k_copy")


def copy_stream(dst: torch.Tensor, src: torch.Tensor) -> None:
    """The streaming copy of the copy ceiling (aenc_k_copy_stream)."""
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    check(lib().aenc_k_copy_stream(_p(dst), _p(src), nbytes, _s()), "aenc_k_copy_stream")


def row_stream(x: torch.Tensor, y: torch.Tensor) -> None:
    """LayerNorm's traffic without its arithmetic (aenc_k_row_stream): y = bf16(x) row by row."""
    assert x.dtype == torch.float32 and y.dtype == torch.bfloat16 and x.dim() == 2 and y.shape == x.shape
    check(lib().aenc_k_row_stream(_p(x), _p(y), x.shape[0], x.shape[1], _s()), "aenc_k_row_stream")


def mfma_loop(out: torch.Tensor, blocks: int, iters: int, ticks: torch.Tensor = None) -> float:
    """The matrix-core loop of the MFMA ceiling (aenc_k_mfma_loop); returns its FLOPs.
    ticks: None or int64 [blocks, 2] for each workgroup's shader-clock and
    100 MHz real-time ticks around its loop."""
    assert out.dtype == torch.float32 and out.numel() >= blocks * 256
    if ticks is not None:
        assert ticks.dtype == torch.int64 and ticks.is_contiguous() and ticks.numel() >= 2 * blocks
    check(lib().aenc_k_mfma_loop(_p(out), blocks, iters, _p(ticks), _s()), "aenc_k_mfma_loop")
    return float(blocks) * 4 * iters * 4 * 32768
