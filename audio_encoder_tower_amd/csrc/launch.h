// Host-side launchers of the library's kernels (internal to the library).
#pragma once

#include "common.h"
#include "epilogue.h"

namespace aenc {

enum GemmTile { GEMM_TILE_256x256 = 0, GEMM_TILE_128x128 = 1 };

// bf16 MFMA GEMM, C = epi(A W^T + b); K % 64 == 0. rows_vary: *m_dev may be
// well below M (a masked batch), so the split of the last round of tiles is
// decided on the device from it.
hipError_t gemm_bf16(int epi, const bf16_t* A, RowMap arow, const bf16_t* W, int64_t ldw, int M, int N, int K,
                     const int32_t* m_dev, const EpiParams& ep, int tile_cfg, hipStream_t stream,
                     bool rows_vary = false);

// The tile shape gemm_bf16 runs fastest with for an M x N output.
int gemm_pick_tile(int M, int N);

// Split-K for the residual products of short batches: gemm_residual_splits
// gives the number of K ranges (1: none) worth launching for an M x N x K
// product, gemm_bf16_splitk writes split s's partial product A[:, s K/S ..]
// W[:, s K/S ..]^T (fp32, no bias) to parts + s * part_stride, rows ldc apart.
// The consumer adds the partials, the bias and the residual (layernorm and
// final_ln_out with ResidualParts).
int gemm_residual_splits(int M, int N, int K);
hipError_t gemm_bf16_splitk(const bf16_t* A, RowMap arow, const bf16_t* W, int64_t ldw, int M, int N, int K,
                            int splits, const int32_t* m_dev, float* parts, int64_t ldc, int64_t part_stride,
                            hipStream_t stream);

// Partial products of a split residual product, folded into x by the next
// normalisation: x[r] += bias + sum_s parts[s * stride + r * d] (n = 0: nothing).
struct ResidualParts {
  const float* parts;
  int n;
  int64_t stride;
  const float* bias;
};

// fp32 GEMM on the vector ALUs (the fp32 path), same epilogues; K % 16 == 0.
hipError_t gemm_f32(int epi, const float* A, RowMap arow, const float* W, int64_t ldw, int M, int N, int K,
                    const int32_t* m_dev, const EpiParams& ep, hipStream_t stream);

// Bidirectional attention, bf16, head_dim 64. qk: [rows, ld_qk] with Q of head h at
// column h*64 and K at column d + h*64; vt: V transposed, row (h*64 + e) holds
// feature e of head h for every packed row, ld_vt apart. Clip b owns packed rows
// [start[b], start[b] + len[b]); start[b] % 8 == 0. o: [rows, ld_o] bf16, head h at column h*64.
// Q must arrive multiplied by ATT_Q_SCALE = log2(e)/sqrt(64), so that Q K^T is
// the softmax exponent in base 2 (the QKV epilogue applies it).
// key_lo/key_hi (both or neither): per packed row, the clip-relative keys
// [key_lo, key_hi) it sees, non-empty and non-decreasing along the clip.
constexpr float ATT_Q_SCALE = 0.18033688011112042f;
hipError_t attention_bf16(const bf16_t* qk, int64_t ld_qk, const bf16_t* vt, int64_t ld_vt,
                          const int32_t* start, const int32_t* len, int n_clips, int max_len, int n_heads,
                          bf16_t* o, int64_t ld_o, const int32_t* key_lo, const int32_t* key_hi,
                          hipStream_t stream);

// The same for the fp32 path with row-major V: qkv [rows, 3d] (Q | K | V).
hipError_t attention_f32(const float* qkv, int64_t ld, const int32_t* start, const int32_t* len, int n_clips,
                         int max_len, int n_heads, float* o, int64_t ld_o, const int32_t* key_lo,
                         const int32_t* key_hi, hipStream_t stream);

// LayerNorm of fp32 rows: y[r] = LN(x[r]) for r < M (M = *m_dev if set).
// With rp.n > 0, x[r] first becomes x[r] + rp.bias + the partial rows (and is
// written back): the residual update of a split product.
hipError_t layernorm(float* x, const float* gamma, const float* beta, void* y, int y_dtype, int M,
                     const int32_t* m_dev, int d, float eps, hipStream_t stream, ResidualParts rp = {});

// Final LayerNorm written to the output layout [B, T_out, d]: output row (b, j)
// reads packed row map[b*T + j] (pool 1) or the mean of LN rows map[b*T + 2j]
// and map[b*T + 2j + 1] (pool 2); rows whose sources are masked become zeros.
hipError_t final_ln_out(const float* x, const int32_t* map, const float* gamma, const float* beta, void* out,
                        int out_dtype, int B, int T, int pool, int d, float eps, hipStream_t stream,
                        ResidualParts rp = {});

// Zero the output rows of masked positions: out row i (of B*T) when map[i] < 0.
hipError_t zero_masked_rows(const int32_t* map, void* out, int out_dtype, int rows, int width,
                            hipStream_t stream);

// mel [B, C, F] -> melT [B, F + 2, C_pad] (channels last, one zero frame on each
// side, channels >= C zero); also zero the two pad frames of g1 [B, F + 2, d].
hipError_t mel_transpose(const void* mel, int in_dtype, void* melT, int B, int C, int C_pad, int F,
                         void* g1, int g1_dtype, int d, hipStream_t stream);

// Key mask [B, T] -> row_map [B*T] (packed row or -1), inv_map [B*round_up(T,8)]
// (packed row -> b*T + t; -1 in alignment gaps), cu [B + 1] (clip starts, multiples
// of 8; cu[B] = end of the last clip), lens [B] (valid positions per clip),
// m_valid [1] (= cu[B]). mask = null: all valid.
hipError_t build_row_maps(const uint8_t* mask, int B, int T, int32_t* row_map, int32_t* inv_map, int32_t* cu,
                          int32_t* lens, int32_t* m_valid, hipStream_t stream);

// Maps of the stacked projector rows from the clip starts and lengths:
// stacked row r holds packed rows k r .. k r + k - 1. row_map [B * (T / k)]:
// output row b * (T/k) + j -> stacked row cu[b] / k + j when its k positions
// are all valid (k j + k <= lens[b]), else -1. inv_map [B * round_up(T, 8) / k]:
// the inverse, -1 for stacked rows that are no output row. m_valid [1]:
// stacked rows to compute, ceil(cu[B] / k). k divides 8.
// Chunked attention: per packed row, the clip-relative key range [key_lo, key_hi)
// of the chunk rule (mode 1 chunk-causal, 2 block-diagonal, `chunk` positions
// per chunk) from the key mask (NULL = all valid) and the packing maps of
// build_row_maps. T <= CHUNK_MAX_T.
constexpr int CHUNK_MAX_T = 4096;
hipError_t build_chunk_ranges(const uint8_t* mask, int B, int T, int chunk, int mode, const int32_t* row_map,
                              const int32_t* cu, int32_t* key_lo, int32_t* key_hi, hipStream_t stream);
hipError_t build_stack_maps(const int32_t* cu, const int32_t* lens, int B, int T, int k, int32_t* row_map,
                            int32_t* inv_map, int32_t* m_valid, hipStream_t stream);

// Repack conv weight [out, in, 3] (dtype) -> [out, 3, in_pad] in the same dtype.
hipError_t repack_conv(const void* src, int dtype, void* dst, int out, int in, int in_pad, hipStream_t stream);

// Convert n elements (dtype) to fp32; src = null fills `fill`.
hipError_t to_f32(const void* src, int dtype, float* dst, int64_t n, float fill, hipStream_t stream);

// Sinusoidal position table [T, d] fp32.
hipError_t position_table(float* pe, int T, int d, hipStream_t stream);

// y = GELU(x) elementwise (fp32), for tests of the device erf.
hipError_t gelu_f32(const float* x, float* y, int64_t n, hipStream_t stream);

// Zero `bytes` (a multiple of 16) at p with a fill kernel (no memset node, so
// the call is safe inside a captured graph).
hipError_t fill_zero(void* p, int64_t bytes, hipStream_t stream);

// Plain device copy kernel (16-byte vectors), for calibrating traffic counters.
hipError_t copy_bytes(void* dst, const void* src, int64_t bytes, hipStream_t stream);

// Calibration: a streaming copy with four 16-byte vectors in flight per lane
// (the copy ceiling), and an MFMA loop on register operands, `blocks`
// workgroups of 4 waves, each wave `iters` rounds of 4 independent
// 32x32x16 bf16 MFMAs (the matrix-core ceiling); out holds blocks * 256 floats.
hipError_t copy_stream(void* dst, const void* src, int64_t bytes, hipStream_t stream);
hipError_t mfma_loop(float* out, uint64_t* ticks, int blocks, int iters, hipStream_t stream);
hipError_t row_stream(const float* x, bf16_t* y, int rows, int d, hipStream_t stream);

}  // namespace aenc
