// Row addressing and fused epilogues shared by the GEMM kernels.
//
// Every linear map of the tower is a GEMM C = A W^T (A [M, K], W [N, K]) whose
// epilogue adds the bias and does the step that follows it, so that no
// separate elementwise pass touches HBM:
//   conv1     : GELU                               -> bf16 channels-last frames
//   conv2     : GELU, + sinusoidal position        -> fp32 residual rows
//   QKV       : + bias; Q, K row-major, V stored transposed per head
//   O-proj    : + residual (fp32, in place)
//   FC1       : GELU                               -> bf16
//   FC2       : + residual (fp32, in place)
//   projector : GELU -> bf16, then plain store in the output dtype
#pragma once

#include "common.h"

namespace aenc {

// Maps logical row r of a GEMM operand to the element offset of its first
// element: groups of `rpg` rows sit `gstride` elements apart, rows within a
// group `rstride` apart. With `map` set, the physical row is map[r]
// (offset map[r] * rstride + off) and a negative entry drops the row.
struct RowMap {
  int64_t rpg;
  int64_t gstride;
  int64_t rstride;
  int64_t off;
  const int32_t* map;

  __device__ __forceinline__ int64_t offset(int r) const {
    if (map) {
      const int32_t p = map[r];
      return p < 0 ? -1 : (int64_t)p * rstride + off;
    }
    const int64_t g = r / rpg;
    return g * gstride + (int64_t)(r - g * rpg) * rstride + off;
  }
};

static inline RowMap dense_rows(int64_t ld) { return RowMap{INT32_MAX, 0, ld, 0, nullptr}; }

enum EpiKind {
  EPI_STORE_BF16 = 0,   // bf16(v + b)
  EPI_GELU_BF16 = 1,    // bf16(GELU(v + b))
  EPI_RESID_F32 = 2,    // C += v + b          (fp32 residual, in place)
  EPI_STORE_F32 = 3,    // v + b               (fp32)
  EPI_GELU_PE_F32 = 4,  // GELU(v + b) + PE[r % pe_period][n]  (fp32)
  EPI_QKV_BF16 = 5,     // v + b; n < n_split: C (bf16); else VT[(n - n_split) * ld_vt + r]
  EPI_GELU_F32 = 6,     // GELU(v + b)         (fp32)
};

struct EpiParams {
  const float* bias;   // [N] or null
  void* c;             // output base (element type by kind)
  RowMap crow;         // C row addressing
  // EPI_QKV_BF16
  int n_split;
  bf16_t* vt;
  int64_t ld_vt;
  // EPI_GELU_PE_F32
  const float* pe;
  int pe_period;
  int pe_ld;
};

template <int EPI>
struct Epilogue {
  // One element: logical row r, column n (n < N, r < M checked by the caller).
  __device__ __forceinline__ static void one(const EpiParams& p, int r, int n, float x) {
    const int64_t o = p.crow.offset(r);
    if (o < 0) return;
    if (EPI == EPI_STORE_BF16 || EPI == EPI_QKV_BF16) {
      ((bf16_t*)p.c)[o + n] = f32_to_bf16(x);
    } else if (EPI == EPI_GELU_BF16) {
      ((bf16_t*)p.c)[o + n] = f32_to_bf16(gelu_erf(x));
    } else if (EPI == EPI_RESID_F32) {
      float* dst = (float*)p.c + o + n;
      *dst = *dst + x;
    } else if (EPI == EPI_STORE_F32) {
      ((float*)p.c)[o + n] = x;
    } else if (EPI == EPI_GELU_F32) {
      ((float*)p.c)[o + n] = gelu_erf(x);
    } else if (EPI == EPI_GELU_PE_F32) {
      const int t = r % p.pe_period;
      ((float*)p.c)[o + n] = gelu_erf(x) + p.pe[(int64_t)t * p.pe_ld + n];
    }
  }

  // Four consecutive logical rows r0..r0+3 of column n.
  __device__ __forceinline__ static void apply4(const EpiParams& p, int r0, int n, f32x4 v, int M, int N) {
    if (n >= N) return;
    const float b = p.bias ? p.bias[n] : 0.0f;
    if (EPI == EPI_QKV_BF16 && n >= p.n_split) {
      bf16_t* dst = p.vt + (int64_t)(n - p.n_split) * p.ld_vt + r0;
      if (r0 + 3 < M) {
        u32x2 w;
        w.x = pack_bf16x2(v.x + b, v.y + b);
        w.y = pack_bf16x2(v.z + b, v.w + b);
        *(u32x2*)dst = w;
      } else {
        if (r0 + 0 < M) dst[0] = f32_to_bf16(v.x + b);
        if (r0 + 1 < M) dst[1] = f32_to_bf16(v.y + b);
        if (r0 + 2 < M) dst[2] = f32_to_bf16(v.z + b);
      }
      return;
    }
    if (r0 + 0 < M) one(p, r0 + 0, n, v.x + b);
    if (r0 + 1 < M) one(p, r0 + 1, n, v.y + b);
    if (r0 + 2 < M) one(p, r0 + 2, n, v.z + b);
    if (r0 + 3 < M) one(p, r0 + 3, n, v.w + b);
  }
};

}  // namespace aenc
