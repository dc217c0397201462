// C entry points of include/aenc_kernels.h: host-side checks, then one launch.
#include <cmath>
#include <cstdio>
#include <string>

#include "../../include/aenc.h"
#include "../../include/aenc_kernels.h"
#include "common.h"
#include "launch.h"

using namespace aenc;

namespace aenc {
void set_kernel_error(const char* msg);
}

namespace {
int fail(const char* msg) {
  aenc::set_kernel_error(msg);
  return AENC_E_INVAL;
}
int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return AENC_OK;
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  aenc::set_kernel_error(buf);
  return AENC_E_HIP;
}
// The kernels move 16 bytes per lane (direct-to-LDS copies, fragment loads,
// row stores), so operand base addresses must be 16-byte aligned.
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
}  // namespace

extern "C" int aenc_k_gemm_bf16(int epi, const void* A, int64_t lda, const void* W, const float* bias, void* C,
                                int64_t ldc, int M, int N, int K, int tile, void* stream) {
  if (!A || !W || !C) return fail("NULL operand");
  if (M < 1 || N < 1 || N % 4 || K < 64 || K % 64 || lda < K || lda % 8 || ldc < N || ldc % 4)
    return fail("bad GEMM sizes (need N % 4 == 0, K % 64 == 0, lda % 8 == 0, ldc % 4 == 0)");
  if (!aligned16(A) || !aligned16(W) || !aligned16(C) || !aligned16(bias))
    return fail("GEMM operands must be 16-byte aligned");
  int kind;
  switch (epi) {
    case AENC_EPI_BF16: kind = EPI_STORE_BF16; break;
    case AENC_EPI_GELU_BF16: kind = EPI_GELU_BF16; break;
    case AENC_EPI_RESID_F32: kind = EPI_RESID_F32; break;
    case AENC_EPI_F32: kind = EPI_STORE_F32; break;
    default: return fail("unknown epilogue");
  }
  if (tile < 0) tile = gemm_pick_tile(M, N);
  if (tile != GEMM_TILE_256x256 && tile != GEMM_TILE_128x128) return fail("unknown tile");
  EpiParams ep{};
  ep.bias = bias;
  ep.c = C;
  ep.crow = dense_rows(ldc);
  return hip_status(gemm_bf16(kind, (const bf16_t*)A, dense_rows(lda), (const bf16_t*)W, K, M, N, K, nullptr, ep,
                              tile, (hipStream_t)stream), "gemm");
}

extern "C" int aenc_k_qkv_bf16(const void* A, const void* Wqkv, const float* bias, float q_scale, void* qk,
                               void* vt, int64_t ld_vt, int M, int d, void* stream) {
  if (!A || !Wqkv || !qk || !vt) return fail("NULL operand");
  if (M < 1 || d < 64 || d % 64 || ld_vt < M + 64 || ld_vt % 8) return fail("bad QKV sizes");
  if (!aligned16(A) || !aligned16(Wqkv) || !aligned16(bias) || !aligned16(qk) || !aligned16(vt))
    return fail("QKV operands must be 16-byte aligned");
  if (!(q_scale > 0.0f) || !std::isfinite(q_scale)) return fail("q_scale must be positive and finite");
  EpiParams ep{};
  ep.q_cols = q_scale == 1.0f ? 0 : d;
  ep.q_scale = q_scale;
  ep.bias = bias;
  ep.c = qk;
  ep.crow = dense_rows(2 * d);
  ep.n_split = 2 * d;
  ep.vt = (bf16_t*)vt;
  ep.ld_vt = ld_vt;
  return hip_status(gemm_bf16(EPI_QKV_BF16, (const bf16_t*)A, dense_rows(d), (const bf16_t*)Wqkv, d, M, 3 * d, d,
                              nullptr, ep, gemm_pick_tile(M, 3 * d), (hipStream_t)stream), "qkv");
}

extern "C" int aenc_k_attention_bf16(const void* qk, const void* vt, int64_t ld_vt, const int32_t* start,
                                     const int32_t* len, int n_clips, int max_len, int n_heads,
                                     const int32_t* key_lo, const int32_t* key_hi, void* out, void* stream) {
  if (!qk || !vt || !start || !len || !out) return fail("NULL operand");
  if (!key_lo != !key_hi) return fail("key_lo and key_hi go together");
  if (n_clips < 1 || max_len < 1 || n_heads < 1 || ld_vt % 8) return fail("bad attention sizes");
  if (!aligned16(qk) || !aligned16(vt) || !aligned16(out)) return fail("attention operands must be 16-byte aligned");
  const int d = 64 * n_heads;
  return hip_status(attention_bf16((const bf16_t*)qk, 2 * d, (const bf16_t*)vt, ld_vt, start, len, n_clips, max_len,
                                   n_heads, (bf16_t*)out, d, key_lo, key_hi, (hipStream_t)stream), "attention");
}

extern "C" int aenc_k_chunk_ranges(const uint8_t* mask, int B, int T, int chunk, int mode, const int32_t* row_map,
                                   const int32_t* cu, int32_t* key_lo, int32_t* key_hi, void* stream) {
  if (!row_map || !cu || !key_lo || !key_hi) return fail("NULL operand");
  if (B < 1 || T < 1 || T > CHUNK_MAX_T) return fail("B must be >= 1 and T in 1..4096");
  if (chunk < 1 || (mode != AENC_CHUNK_CAUSAL && mode != AENC_CHUNK_BLOCK))
    return fail("chunk must be >= 1 and mode AENC_CHUNK_CAUSAL or AENC_CHUNK_BLOCK");
  return hip_status(build_chunk_ranges(mask, B, T, chunk, mode, row_map, cu, key_lo, key_hi, (hipStream_t)stream),
                    "chunk ranges");
}

extern "C" int aenc_k_layernorm(const float* x, const float* gamma, const float* beta, void* y, int y_dtype, int M,
                                int d, float eps, void* stream) {
  if (!x || !gamma || !beta || !y) return fail("NULL operand");
  if (M < 1 || d < 4 || d % 4 || d > 2048 || (y_dtype != 0 && y_dtype != 1)) return fail("bad LayerNorm sizes");
  return hip_status(layernorm(const_cast<float*>(x), gamma, beta, y, y_dtype, M, nullptr, d, eps, (hipStream_t)stream),
                    "layernorm");
}

extern "C" int aenc_k_gelu_f32(const float* x, float* y, int64_t n, void* stream) {
  if (!x || !y || n < 0) return fail("bad GELU arguments");
  return hip_status(gelu_f32(x, y, n, (hipStream_t)stream), "gelu");
}

extern "C" int aenc_k_row_maps(const uint8_t* mask, int B, int T, int32_t* row_map, int32_t* inv_map, int32_t* cu,
                               int32_t* lens, int32_t* m_valid, void* stream) {
  if (!row_map || !inv_map || !cu || !lens || !m_valid) return fail("NULL operand");
  if (B < 1 || T < 1) return fail("bad mask sizes");
  return hip_status(build_row_maps(mask, B, T, row_map, inv_map, cu, lens, m_valid, (hipStream_t)stream),
                    "row maps");
}

extern "C" int aenc_k_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes <= 0 || bytes % 16) return fail("bad copy arguments");
  return hip_status(copy_bytes(dst, src, bytes, (hipStream_t)stream), "copy");
}

extern "C" int aenc_k_copy_stream(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes <= 0 || bytes % 16) return fail("bad copy arguments");
  if (!aligned16(dst) || !aligned16(src)) return fail("copy buffers must be 16-byte aligned");
  return hip_status(copy_stream(dst, src, bytes, (hipStream_t)stream), "copy_stream");
}

extern "C" int aenc_k_row_stream(const float* x, void* y, int rows, int d, void* stream) {
  if (!x || !y || rows < 1 || d < 4 || d > 2048 || d % 4) return fail("row stream: need x, y, rows >= 1, d in [4, 2048], d % 4 == 0");
  if (!aligned16(x) || ((uintptr_t)y & 7)) return fail("row stream: x must be 16-byte and y 8-byte aligned");
  return hip_status(row_stream(x, (bf16_t*)y, rows, d, (hipStream_t)stream), "row_stream");
}

extern "C" int aenc_k_mfma_loop(float* out, int blocks, int iters, uint64_t* ticks, void* stream) {
  if (!out || blocks < 1 || iters < 1) return fail("mfma loop: need out, blocks >= 1 and iters >= 1");
  if ((uintptr_t)ticks & 7) return fail("mfma loop: ticks must be 8-byte aligned");
  return hip_status(mfma_loop(out, ticks, blocks, iters, (hipStream_t)stream), "mfma_loop");
}
