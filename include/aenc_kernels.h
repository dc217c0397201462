/*
 * aenc_kernels.h - single steps of the encoder tower, exported for per-step
 * parity tests and measurement. Each call enqueues one kernel on `stream` (a
 * hipStream_t, NULL = null stream) and returns without synchronising. All
 * pointers are device pointers owned by the caller. Return AENC_OK,
 * AENC_E_INVAL (bad sizes, checked on the host before the launch) or
 * AENC_E_HIP (the launch failed; aenc_last_error() says why).
 *
 * The operations are the pieces of the forward pass declared in aenc.h and
 * come from the same passages: linear maps with [out, in] weights and the
 * gelu activation ("Qwen2-Audio-7B-Instruct", (1) AUDIO ENCODER; "Voxtral-
 * Mini-3B-2507", PROJECTOR), bidirectional multi-head attention with head_dim
 * 64 ("Voxtral-Mini-3B-2507", (1) AUDIO ENCODER), its chunked variant (a
 * reading of audio_chunk_length, "MiniCPM-o-2_6", (2) AUDIO) and the
 * LayerNorms of the pre-LN blocks.
 */
#ifndef AENC_KERNELS_H
#define AENC_KERNELS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of aenc_k_gemm_bf16. */
enum {
  AENC_EPI_BF16 = 0,      /* C (bf16) = A W^T + b                     */
  AENC_EPI_GELU_BF16 = 1, /* C (bf16) = GELU(A W^T + b), erf form     */
  AENC_EPI_RESID_F32 = 2, /* C (fp32) += A W^T + b                    */
  AENC_EPI_F32 = 3        /* C (fp32) = A W^T + b                     */
};

/* Tile shapes of aenc_k_gemm_bf16 (-1 = the library's choice): 256x256 output
 * tiles on 8 waves (one workgroup per CU) or 128x128 tiles on 4 waves. */
enum { AENC_TILE_256x256 = 0, AENC_TILE_128x128 = 1 };

/* C[M, N] = epi(A[M, K] W[N, K]^T + bias[N]) with bf16 A and W (row-major,
 * leading dimensions lda, K and ldc in elements), fp32 accumulate.
 * bias: fp32 [N] or NULL. A, W, C and bias must be 16-byte aligned. K must be
 * a positive multiple of 64; N a positive multiple of 4; lda a multiple of 8
 * and ldc of 4; M >= 1. */
int aenc_k_gemm_bf16(int epi, const void *A, int64_t lda, const void *W, const float *bias, void *C,
                     int64_t ldc, int M, int N, int K, int tile, void *stream);

/* Scale of Q that aenc_k_attention_bf16 expects: log2(e) / sqrt(64), which
 * makes Q K^T the softmax exponent in base 2. */
#define AENC_ATTN_Q_SCALE 0.18033688011112042f

/* The QKV projection of a block: [Q | K | V] = A Wqkv^T + bqkv with A bf16
 * [M, d], Wqkv bf16 [3d, d], bias fp32 [3d] or NULL; the Q columns are then
 * multiplied by q_scale (> 0; 1 for plain Q, AENC_ATTN_Q_SCALE for the input
 * of aenc_k_attention_bf16) before rounding. Q and K go to qk (bf16 [M, 2d]);
 * V goes transposed to vt (bf16, row e of [d, ld_vt] holds feature e of every
 * row; ld_vt >= M + 64, a multiple of 8). d = 64 * heads. A, Wqkv, bias, qk
 * and vt must be 16-byte aligned. */
int aenc_k_qkv_bf16(const void *A, const void *Wqkv, const float *bias, float q_scale, void *qk, void *vt,
                    int64_t ld_vt, int M, int d, void *stream);

/* Bidirectional attention over packed clips: clip b owns rows
 * [start[b], start[b] + len[b]) of qk (Q of head h at column 64h, multiplied
 * by AENC_ATTN_Q_SCALE; K at column d + 64h) and the same columns of vt; every start[b] must be a multiple of 8,
 * every len[b] >= 1 and max_len >= the longest clip; vt must hold 64 columns
 * past the end of the last clip. out: bf16 [rows, d], head h at column 64h;
 * rows outside every clip are not written.
 * key_lo, key_hi: NULL (every query sees its whole clip) or int32 [rows]: the
 * query at packed row r sees the clip-relative keys [key_lo[r], key_hi[r]);
 * within a clip the ranges must be non-empty, inside [0, len[b]] and
 * non-decreasing in r (as aenc_k_chunk_ranges writes them); not checked.
 * qk, vt and out must be 16-byte aligned. */
int aenc_k_attention_bf16(const void *qk, const void *vt, int64_t ld_vt, const int32_t *start, const int32_t *len,
                          int n_clips, int max_len, int n_heads, const int32_t *key_lo, const int32_t *key_hi,
                          void *out, void *stream);

/* Key ranges of chunked attention (aenc.h, AENC_CHUNK_*): positions of a clip
 * are cut into chunks of `chunk` consecutive positions; a valid position sees
 * the valid positions of its own chunk and (mode AENC_CHUNK_CAUSAL) of every
 * earlier chunk, or (AENC_CHUNK_BLOCK) of its own chunk only. From the key
 * mask (uint8 [B, T], NULL = all valid) and the packing maps row_map and cu of
 * aenc_k_row_maps, writes key_lo and key_hi (int32, indexed by packed row,
 * clip-relative) for every valid position's packed row. T <= 4096. */
int aenc_k_chunk_ranges(const uint8_t *mask, int B, int T, int chunk, int mode, const int32_t *row_map,
                        const int32_t *cu, int32_t *key_lo, int32_t *key_hi, void *stream);

/* y[r] = LayerNorm(x[r]; gamma, beta, eps) for r < M, x fp32 [M, d], y in
 * y_dtype (0 fp32, 1 bf16); gamma, beta fp32 [d]. d % 4 == 0, d <= 2048. */
int aenc_k_layernorm(const float *x, const float *gamma, const float *beta, void *y, int y_dtype, int M, int d,
                     float eps, void *stream);

/* y = GELU(x), fp32, the device's erf form used in every GELU epilogue. */
int aenc_k_gelu_f32(const float *x, float *y, int64_t n, void *stream);

/* Packing maps of a key mask uint8 [B, T] (NULL = all valid): row_map [B*T]
 * (packed row or -1), inv_map [B * round_up(T, 8)] (packed row -> b*T + t,
 * -1 in alignment gaps), cu [B + 1] (clip starts, multiples of 8; cu[B] is the
 * end of the last clip), lens [B] (valid positions per clip), m_valid [1]
 * (= cu[B], the packed rows every per-row step covers). */
int aenc_k_row_maps(const uint8_t *mask, int B, int T, int32_t *row_map, int32_t *inv_map, int32_t *cu,
                    int32_t *lens, int32_t *m_valid, void *stream);

/* dst = src, `bytes` (a multiple of 16), by a plain streaming kernel: the
 * reference point for hardware traffic counters. */
int aenc_k_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* Ceilings of this part, measured beside the published peaks (the encoder's
 * kernels are reported against both). Neither is a step of the encoder.
 * aenc_k_copy_stream: dst = src, `bytes` (a multiple of 16; both 16-byte
 * aligned), four 16-byte vectors in flight per lane: the read+write rate a
 * plain streaming kernel reaches.
 * aenc_k_mfma_loop: `blocks` workgroups of 4 waves; each wave runs `iters`
 * rounds of 4 independent v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on
 * register operands with varied non-zero bf16 values, and writes one sum per
 * lane to out (fp32, blocks * 256 elements): the bf16 matrix-core rate with
 * no memory traffic. FLOPs per launch = blocks * 4 * iters * 4 * 32768.
 * ticks: NULL, or uint64 [2 * blocks] (8-byte aligned) that receives, per
 * workgroup, the shader-clock cycles (s_memtime) and the 100 MHz real-time
 * ticks (s_memrealtime) its first wave counted around its loop; 1e8 times
 * their ratio is the shader clock in Hz that the loop ran at. */
int aenc_k_copy_stream(void *dst, const void *src, int64_t bytes, void *stream);
int aenc_k_mfma_loop(float *out, int blocks, int iters, uint64_t *ticks, void *stream);

/* LayerNorm's memory traffic without its arithmetic, the ceiling that kernel
 * is reported against (not a step of the encoder): y[r][j] = bf16(x[r][j])
 * (round to nearest even) for `rows` rows of `d` fp32 values (d a multiple
 * of 4, 4 <= d <= 2048), x row-major and 16-byte aligned, y row-major bf16
 * and 8-byte aligned, both device memory owned by the caller. One wave per
 * row, four rows per workgroup, non-temporal row loads, as the LayerNorm. */
int aenc_k_row_stream(const float *x, void *y, int rows, int d, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AENC_KERNELS_H */
