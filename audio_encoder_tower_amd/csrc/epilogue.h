// Row addressing and fused epilogues shared by the GEMM kernels.
//
// Every linear map of the tower is a GEMM C = A W^T + b (A [M, K], W [N, K])
// whose epilogue does the step that follows it, so that no separate
// elementwise pass touches HBM (the bf16 GEMMs start their accumulators at b;
// the fp32 GEMM adds b in its epilogue):
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
    if (rpg == INT32_MAX) return (int64_t)r * rstride + off;   // dense rows: no division
    const int64_t grp = r / rpg;
    return grp * gstride + (int64_t)(r - grp * rpg) * rstride + off;
  }
};

static inline RowMap dense_rows(int64_t ld) { return RowMap{INT32_MAX, 0, ld, 0, nullptr}; }

// Element offsets of four consecutive logical rows (-1: not stored) and,
// for the positional epilogue, their positions within the clip.
struct RowOffsets {
  int64_t o[4];
  int t[4];
};

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
  // EPI_QKV_BF16: columns n < q_cols (Q) are multiplied by q_scale after the bias
  int n_split;
  bf16_t* vt;
  int64_t ld_vt;
  int q_cols;
  float q_scale;
  // EPI_GELU_PE_F32
  const float* pe;
  int pe_period;
  int pe_ld;
};

template <int EPI>
struct Epilogue {
  __device__ __forceinline__ static void rows(const EpiParams& p, int r0, int M, RowOffsets& ro) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i;
      ro.o[i] = r < M ? p.crow.offset(r) : -1;
      ro.t[i] = EPI == EPI_GELU_PE_F32 ? r % p.pe_period : 0;
    }
  }

  // One element x (bias already added) at element offset o of row-major C, column n.
  __device__ __forceinline__ static void one(const EpiParams& p, int64_t o, int t, int n, float x) {
    if (EPI == EPI_STORE_BF16 || EPI == EPI_QKV_BF16) {
      ((bf16_t*)p.c)[o + n] = f32_to_bf16(x);
    } else if (EPI == EPI_GELU_BF16) {
      ((bf16_t*)p.c)[o + n] = f32_to_bf16(gelu_bf16out(x));
    } else if (EPI == EPI_RESID_F32) {
      float* dst = (float*)p.c + o + n;
      *dst = *dst + x;
    } else if (EPI == EPI_STORE_F32) {
      ((float*)p.c)[o + n] = x;
    } else if (EPI == EPI_GELU_F32) {
      ((float*)p.c)[o + n] = gelu_erf(x);
    } else if (EPI == EPI_GELU_PE_F32) {
      ((float*)p.c)[o + n] = gelu_erf(x) + p.pe[(int64_t)t * p.pe_ld + n];
    }
  }

  // Rows r0..r0+3 (offsets from rows()) of column n; v holds the biased sums.
  __device__ __forceinline__ static void store4(const EpiParams& p, const RowOffsets& ro, int r0, int n, f32x4 v,
                                                int M, int N) {
    if (n >= N) return;
    if (EPI == EPI_QKV_BF16 && n >= p.n_split) {
      // V goes transposed: row (n - n_split) of V^T, columns r0..r0+3 contiguous.
      bf16_t* dst = p.vt + (int64_t)(n - p.n_split) * p.ld_vt + r0;
      if (r0 + 3 < M) {
        u32x2 w;
        w.x = pack_bf16x2(v.x, v.y);
        w.y = pack_bf16x2(v.z, v.w);
        *(u32x2*)dst = w;
      } else {
        if (r0 + 0 < M) dst[0] = f32_to_bf16(v.x);
        if (r0 + 1 < M) dst[1] = f32_to_bf16(v.y);
        if (r0 + 2 < M) dst[2] = f32_to_bf16(v.z);
      }
      return;
    }
    if (EPI == EPI_QKV_BF16 && n < p.q_cols) v *= p.q_scale;
    if (ro.o[0] >= 0) one(p, ro.o[0], ro.t[0], n, v.x);
    if (ro.o[1] >= 0) one(p, ro.o[1], ro.t[1], n, v.y);
    if (ro.o[2] >= 0) one(p, ro.o[2], ro.t[2], n, v.z);
    if (ro.o[3] >= 0) one(p, ro.o[3], ro.t[3], n, v.w);
  }

  // One 32-row slab of a wave's fp32 tile staged in LDS (row stride LDW floats,
  // WN columns starting at col0, rows starting at row0; the sums already hold
  // the bias), written to C four consecutive columns per lane: 8- or 16-byte
  // accesses, whole rows contiguous across lanes. N must be a multiple of 4.
  template <int WN, int LDW>
  __device__ __forceinline__ static void slab32(const EpiParams& p, const float* slab, int row0, int col0, int lane,
                                                int M, int N) {
    if (EPI == EPI_QKV_BF16 && col0 >= p.n_split) {
      // V columns go to V^T: a lane takes 4 consecutive rows of one column.
      constexpr int ITER = WN * 8 / 64;
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int idx = it * 64 + lane;
        const int c = idx >> 3, rq = idx & 7;
        const int n = col0 + c, r0 = row0 + 4 * rq;
        if (n >= N || r0 >= M) continue;
        const float* s = slab + 4 * rq * LDW + c;
        const float v0 = s[0], v1 = s[LDW], v2 = s[2 * LDW], v3 = s[3 * LDW];
        bf16_t* dst = p.vt + (int64_t)(n - p.n_split) * p.ld_vt + r0;
        if (r0 + 3 < M) {
          u32x2 w;
          w.x = pack_bf16x2(v0, v1);
          w.y = pack_bf16x2(v2, v3);
          *(u32x2*)dst = w;
        } else {
          dst[0] = f32_to_bf16(v0);
          if (r0 + 1 < M) dst[1] = f32_to_bf16(v1);
          if (r0 + 2 < M) dst[2] = f32_to_bf16(v2);
        }
      }
      return;
    }
    constexpr int C4 = WN / 4;                 // float4 per slab row
    constexpr int ITER = 32 * C4 / 64;         // float4 per lane
    int64_t off[ITER];
    float4 val[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = it * 64 + lane;
      const int rr = idx / C4, c4 = idx % C4;
      const int r = row0 + rr, n = col0 + 4 * c4;
      float4 v = *(const float4*)(slab + rr * LDW + 4 * c4);
      int64_t o = -1;
      if (r < M && n < N) {
        o = p.crow.offset(r);
        if (o >= 0) o += n;
      }
      if (EPI == EPI_QKV_BF16 && n < p.q_cols) {
        v.x *= p.q_scale; v.y *= p.q_scale; v.z *= p.q_scale; v.w *= p.q_scale;
      }
      if (EPI == EPI_GELU_PE_F32 && o >= 0) {
        const float4 pe = *(const float4*)(p.pe + (int64_t)(r % p.pe_period) * p.pe_ld + n);
        v.x = gelu_erf(v.x) + pe.x; v.y = gelu_erf(v.y) + pe.y;
        v.z = gelu_erf(v.z) + pe.z; v.w = gelu_erf(v.w) + pe.w;
      }
      if (EPI == EPI_GELU_BF16) {
        v.x = gelu_bf16out(v.x); v.y = gelu_bf16out(v.y); v.z = gelu_bf16out(v.z); v.w = gelu_bf16out(v.w);
      }
      if (EPI == EPI_GELU_F32) {
        v.x = gelu_erf(v.x); v.y = gelu_erf(v.y); v.z = gelu_erf(v.z); v.w = gelu_erf(v.w);
      }
      off[it] = o;
      val[it] = v;
    }
    if (EPI == EPI_RESID_F32) {
      // all residual loads first (from a valid address for skipped lanes), then the stores
      float4 old[ITER];
#pragma unroll
      for (int it = 0; it < ITER; ++it) old[it] = *(const float4*)((const float*)p.c + (off[it] >= 0 ? off[it] : 0));
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        if (off[it] < 0) continue;
        const float4 v = val[it];
        *(float4*)((float*)p.c + off[it]) =
            make_float4(old[it].x + v.x, old[it].y + v.y, old[it].z + v.z, old[it].w + v.w);
      }
      return;
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      if (off[it] < 0) continue;
      const float4 v = val[it];
      if (EPI == EPI_STORE_F32 || EPI == EPI_GELU_F32 || EPI == EPI_GELU_PE_F32) {
        *(float4*)((float*)p.c + off[it]) = v;
      } else {
        u32x2 w;
        w.x = pack_bf16x2(v.x, v.y);
        w.y = pack_bf16x2(v.z, v.w);
        *(u32x2*)((bf16_t*)p.c + off[it]) = w;
      }
    }
  }

  // Unbiased sums v of rows r0..r0+3, column n (used by the fp32 GEMM).
  __device__ __forceinline__ static void apply4(const EpiParams& p, int r0, int n, f32x4 v, int M, int N) {
    if (n >= N) return;
    const float b = p.bias ? p.bias[n] : 0.0f;
    RowOffsets ro;
    rows(p, r0, M, ro);
    store4(p, ro, r0, n, f32x4{v.x + b, v.y + b, v.z + b, v.w + b}, M, N);
  }
};

}  // namespace aenc
