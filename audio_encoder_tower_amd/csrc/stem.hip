// Data-movement kernels around the encoder: the mel transpose that feeds the
// implicit-GEMM convolutions, the packing maps of a key mask, weight repacks
// and the sinusoidal position table.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace aenc {

// ---------------------------------------------------------------------------
// mel [B, C, F] (channels first, as the feature extractor emits it:
// "Voxtral-Mini-3B-2507", Preprocessor, feature_size x nb_max_frames) ->
// melT [B, F + 2, C_pad]: channels last with one zero frame on each side, so
// that the three taps of frame f are the contiguous rows f, f+1, f+2.
// 64 x 64 tiles transposed through LDS.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mel_transpose_kernel(const T* __restrict__ mel, T* __restrict__ melT, int C,
                                                            int C_pad, int F, T* g1, int d) {
  __shared__ float tile[64][65];
  const int b = blockIdx.z;
  const int fo0 = blockIdx.x * 64;   // output frame rows (0 .. F+1)
  const int c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const T* src = mel + (int64_t)b * C * F;
  for (int cc = ty; cc < 64; cc += 4) {
    const int c = c0 + cc, fin = fo0 + tx - 1;
    float v = 0.0f;
    if (c < C && fin >= 0 && fin < F) v = Elem<T>::load(src + (int64_t)c * F + fin);
    tile[cc][tx] = v;
  }
  __syncthreads();
  T* dst = melT + (int64_t)b * (F + 2) * C_pad;
  for (int ff = ty; ff < 64; ff += 4) {
    const int fo = fo0 + ff;
    if (fo < F + 2 && c0 + tx < C_pad) Elem<T>::store(dst + (int64_t)fo * C_pad + c0 + tx, tile[tx][ff]);
  }
  // The conv1 output buffer has the same padded frame layout; its pad rows stay zero.
  if (g1 && blockIdx.x == 0 && blockIdx.y == 0) {
    T* g = g1 + (int64_t)b * (F + 2) * d;
    for (int i = threadIdx.x; i < d; i += 256) {
      Elem<T>::store(g + i, 0.0f);
      Elem<T>::store(g + (int64_t)(F + 1) * d + i, 0.0f);
    }
  }
}

hipError_t mel_transpose(const void* mel, int in_dtype, void* melT, int B, int C, int C_pad, int F, void* g1,
                         int g1_dtype, int d, hipStream_t stream) {
  if (in_dtype != g1_dtype) return hipErrorInvalidValue;
  dim3 grid((F + 2 + 63) / 64, (C_pad + 63) / 64, B);
  if (in_dtype == 1)
    hipLaunchKernelGGL(mel_transpose_kernel<bf16_t>, grid, dim3(256), 0, stream, (const bf16_t*)mel, (bf16_t*)melT,
                       C, C_pad, F, (bf16_t*)g1, d);
  else
    hipLaunchKernelGGL(mel_transpose_kernel<float>, grid, dim3(256), 0, stream, (const float*)mel, (float*)melT, C,
                       C_pad, F, (float*)g1, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Packing maps of a key-padding mask. Valid positions of clip b get packed
// rows cu[b] + (rank among the clip's valid positions); each clip starts on
// a multiple of 8 rows, so that the transposed value rows of every clip are
// 16-byte aligned. One workgroup scans all clips in order.
// ---------------------------------------------------------------------------
constexpr int SCAN_THREADS = 1024;

__global__ __launch_bounds__(SCAN_THREADS) void row_maps_kernel(const uint8_t* __restrict__ mask, int B, int T,
                                                                int32_t* __restrict__ row_map,
                                                                int32_t* __restrict__ inv_map,
                                                                int32_t* __restrict__ cu,
                                                                int32_t* __restrict__ lens, int32_t* m_valid,
                                                                int inv_cap) {
  __shared__ int wsum[SCAN_THREADS / 64];
  __shared__ int chunk_total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int b = 0; b < B; ++b) {
    base = (base + 7) & ~7;
    const int start = base;
    if (tid == 0) cu[b] = start;
    for (int t0 = 0; t0 < T; t0 += SCAN_THREADS) {
      const int t = t0 + tid;
      const int valid = (t < T) ? (mask ? (mask[(int64_t)b * T + t] != 0) : 1) : 0;
      // inclusive scan within the wave
      int x = valid;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane == 63) wsum[wave] = x;
      __syncthreads();
      if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < SCAN_THREADS / 64; ++w) {
          const int s = wsum[w];
          wsum[w] = acc;
          acc += s;
        }
        chunk_total = acc;
      }
      __syncthreads();
      const int rank = base + wsum[wave] + x - valid;   // exclusive
      if (t < T) {
        row_map[(int64_t)b * T + t] = valid ? rank : -1;
        if (valid) inv_map[rank] = b * T + t;
      }
      base += chunk_total;
      __syncthreads();
    }
    if (tid == 0) lens[b] = base - start;
    // rows of the alignment gap after this clip belong to no position
    const int gap_end = min((base + 7) & ~7, inv_cap);
    for (int r = base + tid; r < gap_end; r += SCAN_THREADS) inv_map[r] = -1;
  }
  if (tid == 0) {
    cu[B] = base;
    *m_valid = base;
  }
}

hipError_t build_row_maps(const uint8_t* mask, int B, int T, int32_t* row_map, int32_t* inv_map, int32_t* cu,
                          int32_t* lens, int32_t* m_valid, hipStream_t stream) {
  const int inv_cap = B * ((T + 7) & ~7);
  hipLaunchKernelGGL(row_maps_kernel, dim3(1), dim3(SCAN_THREADS), 0, stream, mask, B, T, row_map, inv_map, cu,
                     lens, m_valid, inv_cap);
  return hipGetLastError();
}

// Key ranges of chunked attention. Positions t of a clip fall into chunks of
// `chunk` consecutive positions, c(t) = t / chunk; a query sees the keys of its
// own chunk and, chunk-causal (mode 1), every earlier chunk, or, block-diagonal
// (mode 2), only its own. Packing keeps the clip's valid positions in order, so
// those keys are one contiguous range of the clip's packed rows: with cnt[p]
// the number of valid positions before position p, query t sees packed keys
// [mode 2 ? cnt[chunk c] : 0, cnt[min(T, chunk (c + 1))]). One workgroup per
// clip: cnt by a block scan of the mask in LDS, then one range per valid row.
__global__ __launch_bounds__(SCAN_THREADS) void chunk_ranges_kernel(const uint8_t* __restrict__ mask, int T,
                                                                    int chunk, int mode,
                                                                    const int32_t* __restrict__ row_map,
                                                                    const int32_t* __restrict__ cu,
                                                                    int32_t* __restrict__ key_lo,
                                                                    int32_t* __restrict__ key_hi) {
  __shared__ int cnt[CHUNK_MAX_T + 1];
  __shared__ int wsum[SCAN_THREADS / 64];
  __shared__ int carry;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += SCAN_THREADS) {
    const int t = t0 + tid;
    const int valid = (t < T) ? (mask ? (mask[(int64_t)b * T + t] != 0) : 1) : 0;
    int x = valid;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (t < T) cnt[t] = before + x - valid;      // exclusive count
    __syncthreads();
    if (tid == SCAN_THREADS - 1) carry = before + x;
    __syncthreads();
  }
  if (tid == 0) cnt[T] = carry;
  __syncthreads();
  const int base = cu[b];
  for (int t = tid; t < T; t += SCAN_THREADS) {
    if (row_map[(int64_t)b * T + t] < 0) continue;
    const int c = t / chunk;
    const int r = base + cnt[t];
    key_lo[r] = mode == 2 ? cnt[min(T, chunk * c)] : 0;
    key_hi[r] = cnt[min(T, chunk * (c + 1))];
  }
}

hipError_t build_chunk_ranges(const uint8_t* mask, int B, int T, int chunk, int mode, const int32_t* row_map,
                              const int32_t* cu, int32_t* key_lo, int32_t* key_hi, hipStream_t stream) {
  if (B < 1 || T < 1 || T > CHUNK_MAX_T || chunk < 1 || (mode != 1 && mode != 2)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(chunk_ranges_kernel, dim3(B), dim3(SCAN_THREADS), 0, stream, mask, T, chunk, mode, row_map,
                     cu, key_lo, key_hi);
  return hipGetLastError();
}

// One workgroup: clip by clip, every stacked row of the clip's packed range
// gets its output row (or -1), and every output row its stacked row (or -1).
__global__ __launch_bounds__(SCAN_THREADS) void stack_maps_kernel(const int32_t* __restrict__ cu,
                                                                  const int32_t* __restrict__ lens, int B, int T,
                                                                  int k, int32_t* __restrict__ row_map,
                                                                  int32_t* __restrict__ inv_map,
                                                                  int32_t* __restrict__ m_valid, int inv_cap) {
  const int tid = threadIdx.x;
  const int t_out = T / k;
  for (int b = 0; b < B; ++b) {
    const int start = cu[b] / k;
    const int n = min(lens[b] / k, t_out);    // complete runs of k valid positions
    const int end = b + 1 < B ? cu[b + 1] / k : inv_cap;
    for (int j = tid; j < t_out; j += SCAN_THREADS) row_map[(int64_t)b * t_out + j] = j < n ? start + j : -1;
    for (int r = start + tid; r < end; r += SCAN_THREADS) inv_map[r] = r - start < n ? b * t_out + (r - start) : -1;
  }
  if (tid == 0) *m_valid = (cu[B] + k - 1) / k;
}

hipError_t build_stack_maps(const int32_t* cu, const int32_t* lens, int B, int T, int k, int32_t* row_map,
                            int32_t* inv_map, int32_t* m_valid, hipStream_t stream) {
  if (k < 1 || 8 % k != 0) return hipErrorInvalidValue;
  const int inv_cap = B * ((T + 7) & ~7) / k;
  hipLaunchKernelGGL(stack_maps_kernel, dim3(1), dim3(SCAN_THREADS), 0, stream, cu, lens, B, T, k, row_map, inv_map,
                     m_valid, inv_cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight preparation (at create time only).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void repack_conv_kernel(const T* __restrict__ src, T* __restrict__ dst, int out, int in, int in_pad) {
  const int64_t n = (int64_t)out * 3 * in_pad;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % in_pad);
    const int k = (int)((i / in_pad) % 3);
    const int o = (int)(i / (3 * (int64_t)in_pad));
    dst[i] = c < in ? src[((int64_t)o * in + c) * 3 + k] : T(0);
  }
}

hipError_t repack_conv(const void* src, int dtype, void* dst, int out, int in, int in_pad, hipStream_t stream) {
  if (dtype == 1)
    hipLaunchKernelGGL(repack_conv_kernel<bf16_t>, dim3(1024), dim3(256), 0, stream, (const bf16_t*)src,
                       (bf16_t*)dst, out, in, in_pad);
  else
    hipLaunchKernelGGL(repack_conv_kernel<float>, dim3(1024), dim3(256), 0, stream, (const float*)src, (float*)dst,
                       out, in, in_pad);
  return hipGetLastError();
}

template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ src, float* __restrict__ dst, int64_t n, float fill) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src ? Elem<T>::load(src + i) : fill;
}

hipError_t to_f32(const void* src, int dtype, float* dst, int64_t n, float fill, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(to_f32_kernel<bf16_t>, dim3(256), dim3(256), 0, stream, (const bf16_t*)src, dst, n, fill);
  else
    hipLaunchKernelGGL(to_f32_kernel<float>, dim3(256), dim3(256), 0, stream, (const float*)src, dst, n, fill);
  return hipGetLastError();
}

// PE[t, j] = sin(t w_j) for j < d/2 and cos(t w_(j - d/2)) after, with
// w_j = exp(-j ln(10000) / (d/2 - 1)): the sinusoid layout of Whisper-style
// encoders (timescales 1 .. 10000). Computed in double, stored fp32.
__global__ void position_table_kernel(float* pe, int T, int d) {
  const int half = d / 2;
  const int64_t n = (int64_t)T * d;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / d), j = (int)(i % d);
    const int jj = j < half ? j : j - half;
    const double w = exp(-(double)jj * log(10000.0) / (double)(half - 1));
    const double a = (double)t * w;
    pe[i] = (float)(j < half ? sin(a) : cos(a));
  }
}

hipError_t position_table(float* pe, int T, int d, hipStream_t stream) {
  hipLaunchKernelGGL(position_table_kernel, dim3(256), dim3(256), 0, stream, pe, T, d);
  return hipGetLastError();
}

__global__ void gelu_kernel(const float* x, float* y, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = gelu_erf(x[i]);
}

hipError_t gelu_f32(const float* x, float* y, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gelu_kernel, dim3(1024), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(u32x4* __restrict__ p, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t fill_zero(void* p, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)p & 15)) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4*)p, n16);
  return hipGetLastError();
}

__global__ void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t copy_bytes(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, stream, (u32x4*)dst, (const u32x4*)src, bytes / 16);
  return hipGetLastError();
}

}  // namespace aenc
