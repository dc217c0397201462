// LayerNorm kernels: pre-LN of each block and the final LayerNorm (with the
// optional pair-average pool and the scatter back to the [B, T_out, d] layout).
//
// LN(x) = gamma * (x - mean) / sqrt(var + eps) + beta over the d features of a
// row, biased variance. These kernels are bound by HBM bandwidth: one wave64
// per row, fp32 rows read once as 16-byte vectors and held in registers for
// the two reductions (mean, then the centred second moment), then written
// once (bf16 or fp32).
#include "common.h"
#include "launch.h"

namespace aenc {

constexpr int LN_MAXV = 8;   // float4 per lane: d <= 64 * 4 * 8 = 2048

struct RowStats {
  float mean, rstd;
};

__device__ __forceinline__ RowStats row_stats(const float4 (&v)[LN_MAXV], int n4, int lane, int d, float eps) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i)
    if (lane + 64 * i < n4) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = wave_sum(s) / (float)d;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i)
    if (lane + 64 * i < n4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, e = v[i].w - mean;
      q += (a * a + b * b) + (c * c + e * e);
    }
  const float var = wave_sum(q) / (float)d;
  return RowStats{mean, 1.0f / sqrtf(var + eps)};
}

// Rows are read with non-temporal loads: the residual row is not read again
// before the next residual product rewrites it, and keeping it out of the
// caches leaves them to the products' operands (forward -0.5%, though this
// kernel alone is 3% slower than with plain loads).
__device__ __forceinline__ void load_row(const float* x, float4 (&v)[LN_MAXV], int n4, int lane) {
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i)
    if (lane + 64 * i < n4) {
      const f32x4 t = __builtin_nontemporal_load((const f32x4*)x + lane + 64 * i);
      v[i] = make_float4(t.x, t.y, t.z, t.w);
    }
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// The residual update of a split product: v (row `row` of x) += bias + every
// partial row, in that order. All parts' loads are issued before the first
// add (a loop over a run-time part count would wait for each part in turn).
constexpr int LN_MAX_PARTS = 4;
__device__ __forceinline__ void fold_parts(float4 (&v)[LN_MAXV], const ResidualParts& rp, int64_t row, int d,
                                           int n4, int lane) {
  float4 q[LN_MAX_PARTS][LN_MAXV];
#pragma unroll
  for (int s = 0; s < LN_MAX_PARTS; ++s)
    if (s < rp.n) {
      const float4* src = (const float4*)(rp.parts + s * rp.stride + row * d);
#pragma unroll
      for (int i = 0; i < LN_MAXV; ++i)
        if (lane + 64 * i < n4) q[s][i] = src[lane + 64 * i];
    }
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int j = lane + 64 * i;
    if (j >= n4) continue;
    float4 p = rp.bias ? ((const float4*)rp.bias)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < LN_MAX_PARTS; ++s)
      if (s < rp.n) p = add4(p, q[s][i]);
    v[i] = add4(v[i], p);
  }
}

__device__ __forceinline__ float4 norm4(float4 x, const RowStats& st, float4 g, float4 b) {
  return make_float4((x.x - st.mean) * st.rstd * g.x + b.x, (x.y - st.mean) * st.rstd * g.y + b.y,
                     (x.z - st.mean) * st.rstd * g.z + b.z, (x.w - st.mean) * st.rstd * g.w + b.w);
}

__device__ __forceinline__ void store4(float* y, int j, float4 v) { ((float4*)y)[j] = v; }
__device__ __forceinline__ void store4(bf16_t* y, int j, float4 v) {
  u32x2 w;
  w.x = pack_bf16x2(v.x, v.y);
  w.y = pack_bf16x2(v.z, v.w);
  ((u32x2*)y)[j] = w;
}

// PARTS: fold the partial products of a split residual product into x first
// (and write x back).
template <typename TO, bool PARTS>
__global__ __launch_bounds__(256) void layernorm_kernel(float* __restrict__ x, const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, TO* __restrict__ y,
                                                        int M_arg, const int32_t* m_dev, int d, float eps,
                                                        ResidualParts rp) {
  const int M = m_dev ? *m_dev : M_arg;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int lane = threadIdx.x & 63, n4 = d >> 2;
  float4 v[LN_MAXV];
  load_row(x + (int64_t)row * d, v, n4, lane);
  if (PARTS) {
    fold_parts(v, rp, row, d, n4, lane);
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i)
      if (lane + 64 * i < n4) ((float4*)(x + (int64_t)row * d))[lane + 64 * i] = v[i];
  }
  const RowStats st = row_stats(v, n4, lane, d, eps);
  TO* yr = y + (int64_t)row * d;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int j = lane + 64 * i;
    if (j < n4) store4(yr, j, norm4(v[i], st, ((const float4*)gamma)[j], ((const float4*)beta)[j]));
  }
}

hipError_t layernorm(float* x, const float* gamma, const float* beta, void* y, int y_dtype, int M,
                     const int32_t* m_dev, int d, float eps, hipStream_t stream, ResidualParts rp) {
  if (d % 4 != 0 || d > 64 * 4 * LN_MAXV || M <= 0 || (rp.n > 0 && !rp.parts) || rp.n > LN_MAX_PARTS)
    return hipErrorInvalidValue;
  dim3 grid((M + 3) / 4);
  if (y_dtype == 1 && rp.n > 0)
    hipLaunchKernelGGL((layernorm_kernel<bf16_t, true>), grid, dim3(256), 0, stream, x, gamma, beta, (bf16_t*)y, M,
                       m_dev, d, eps, rp);
  else if (y_dtype == 1)
    hipLaunchKernelGGL((layernorm_kernel<bf16_t, false>), grid, dim3(256), 0, stream, x, gamma, beta, (bf16_t*)y, M,
                       m_dev, d, eps, rp);
  else if (rp.n > 0)
    hipLaunchKernelGGL((layernorm_kernel<float, true>), grid, dim3(256), 0, stream, x, gamma, beta, (float*)y, M,
                       m_dev, d, eps, rp);
  else
    hipLaunchKernelGGL((layernorm_kernel<float, false>), grid, dim3(256), 0, stream, x, gamma, beta, (float*)y, M,
                       m_dev, d, eps, rp);
  return hipGetLastError();
}

// Final LayerNorm into the output layout. Output row (b, j) of B*T_out.
template <typename TO, bool PARTS>
__global__ __launch_bounds__(256) void final_ln_kernel(const float* __restrict__ x, const int32_t* __restrict__ map,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, TO* __restrict__ out, int B,
                                                       int T, int pool, int d, float eps, ResidualParts rp) {
  const int t_out = T / pool;
  const int orow = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (orow >= B * t_out) return;
  const int b = orow / t_out, j = orow - b * t_out;
  const int lane = threadIdx.x & 63, n4 = d >> 2;
  TO* yr = out + (int64_t)orow * d;
  int src[2];
  bool ok = true;
  for (int p = 0; p < pool; ++p) {
    src[p] = map[(int64_t)b * T + pool * j + p];
    ok = ok && src[p] >= 0;
  }
  if (!ok) {
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i)
      if (lane + 64 * i < n4) store4(yr, lane + 64 * i, make_float4(0.f, 0.f, 0.f, 0.f));
    return;
  }
  float4 accv[LN_MAXV];
  for (int p = 0; p < pool; ++p) {
    float4 v[LN_MAXV];
    load_row(x + (int64_t)src[p] * d, v, n4, lane);
    if (PARTS) fold_parts(v, rp, src[p], d, n4, lane);
    const RowStats st = row_stats(v, n4, lane, d, eps);
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int jj = lane + 64 * i;
      if (jj < n4) {
        const float4 y = norm4(v[i], st, ((const float4*)gamma)[jj], ((const float4*)beta)[jj]);
        if (p == 0) accv[i] = y;
        else accv[i] = make_float4(accv[i].x + y.x, accv[i].y + y.y, accv[i].z + y.z, accv[i].w + y.w);
      }
    }
  }
  const float scale = pool == 2 ? 0.5f : 1.0f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int jj = lane + 64 * i;
    if (jj < n4)
      store4(yr, jj, make_float4(accv[i].x * scale, accv[i].y * scale, accv[i].z * scale, accv[i].w * scale));
  }
}

hipError_t final_ln_out(const float* x, const int32_t* map, const float* gamma, const float* beta, void* out,
                        int out_dtype, int B, int T, int pool, int d, float eps, hipStream_t stream,
                        ResidualParts rp) {
  if (d % 4 != 0 || d > 64 * 4 * LN_MAXV || (pool != 1 && pool != 2) || (rp.n > 0 && !rp.parts) ||
      rp.n > LN_MAX_PARTS)
    return hipErrorInvalidValue;
  const int rows = B * (T / pool);
  if (rows <= 0) return hipSuccess;
  dim3 grid((rows + 3) / 4);
  if (out_dtype == 1 && rp.n > 0)
    hipLaunchKernelGGL((final_ln_kernel<bf16_t, true>), grid, dim3(256), 0, stream, x, map, gamma, beta,
                       (bf16_t*)out, B, T, pool, d, eps, rp);
  else if (out_dtype == 1)
    hipLaunchKernelGGL((final_ln_kernel<bf16_t, false>), grid, dim3(256), 0, stream, x, map, gamma, beta,
                       (bf16_t*)out, B, T, pool, d, eps, rp);
  else if (rp.n > 0)
    hipLaunchKernelGGL((final_ln_kernel<float, true>), grid, dim3(256), 0, stream, x, map, gamma, beta, (float*)out,
                       B, T, pool, d, eps, rp);
  else
    hipLaunchKernelGGL((final_ln_kernel<float, false>), grid, dim3(256), 0, stream, x, map, gamma, beta, (float*)out,
                       B, T, pool, d, eps, rp);
  return hipGetLastError();
}

template <typename TO>
__global__ void zero_rows_kernel(const int32_t* __restrict__ map, TO* __restrict__ out, int rows, int width) {
  const int r = blockIdx.x;
  if (r >= rows || map[r] >= 0) return;
  for (int i = threadIdx.x; i < width; i += blockDim.x) out[(int64_t)r * width + i] = TO(0);
}

hipError_t zero_masked_rows(const int32_t* map, void* out, int out_dtype, int rows, int width,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (out_dtype == 1)
    hipLaunchKernelGGL(zero_rows_kernel<bf16_t>, dim3(rows), dim3(256), 0, stream, map, (bf16_t*)out, rows, width);
  else
    hipLaunchKernelGGL(zero_rows_kernel<float>, dim3(rows), dim3(256), 0, stream, map, (float*)out, rows, width);
  return hipGetLastError();
}

}  // namespace aenc
