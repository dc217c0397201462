// Calibration kernels: the ceilings the encoder's kernels are measured against
// on the part itself, beside the published peaks.
//   * a streaming copy (16-byte vectors, four in flight per lane, loads and
//     stores marked non-temporal, 16384 workgroups): the HBM read+write rate a
//     bandwidth-bound kernel reaches (the fastest of the copy forms measured:
//     plain loads and stores 5.76 TB/s, non-temporal 6.06; 8 or 16 vectors in
//     flight per lane slower);
//   * LayerNorm's memory traffic without its arithmetic (fp32 rows in, bf16
//     rows out, the same access pattern): the rate that kernel could reach;
//   * a matrix-core loop: chains of v_mfma_f32_32x32x16_bf16 on register
//     operands (no memory traffic), the bf16 MFMA rate the part sustains. The
//     operands are non-zero bf16 values whose mantissa bits change every
//     iteration, since the matrix cores draw less power, and clock higher, on
//     zeros or constant inputs than on the varied data of a real product.
//     Optionally each workgroup's first wave also counts the shader clock
//     (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around its
//     loop, which gives the clock the loop ran at: the part lowers its clock
//     under a sustained matrix-core load.
#include "common.h"
#include "launch.h"

namespace aenc {

__global__ __launch_bounds__(256) void copy4_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                    int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n16; base += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + 256 * u;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

hipError_t copy_stream(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::min<int64_t>((n16 + 1023) / 1024, 16384);
  hipLaunchKernelGGL(copy4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4*)dst, (const u32x4*)src, n16);
  return hipGetLastError();
}

// LayerNorm's memory traffic without its arithmetic: one wave per row of d
// fp32 values, four rows per workgroup, the row read with non-temporal 16-byte
// loads and written back as bf16 (8 bytes per lane), as the LayerNorm does, but
// with no reductions between the loads and the stores.
__global__ __launch_bounds__(256) void row_stream_kernel(const float* __restrict__ x, bf16_t* __restrict__ y,
                                                         int rows, int d) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63, n4 = d >> 2;
  const f32x4* xr = (const f32x4*)(x + (int64_t)row * d);
  u32x2* yr = (u32x2*)(y + (int64_t)row * d);
  f32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (lane + 64 * i < n4) v[i] = __builtin_nontemporal_load(xr + lane + 64 * i);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (lane + 64 * i < n4) {
      u32x2 w;
      w.x = pack_bf16x2(v[i].x, v[i].y);
      w.y = pack_bf16x2(v[i].z, v[i].w);
      yr[lane + 64 * i] = w;
    }
}

hipError_t row_stream(const float* x, bf16_t* y, int rows, int d, hipStream_t stream) {
  if (rows < 1 || d < 4 || d > 2048 || d % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_stream_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, x, y, rows, d);
  return hipGetLastError();
}

constexpr int MFMA_CHAINS = 4;

// Each wave runs `iters` rounds of MFMA_CHAINS independent 32x32x16 MFMAs and
// writes one sum per lane to out[global thread id]; with ticks, wave 0 of
// workgroup b writes the shader-clock and real-time ticks its loop took to
// ticks[2 b] and ticks[2 b + 1].
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, uint64_t* __restrict__ ticks,
                                                        int iters) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // bf16 pairs with exponent 126..127 (values in [0.5, 2)) and lane-dependent
  // signs and mantissas
  uint32_t sa[4], sb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = (lane * 2654435761u) ^ ((uint32_t)i * 40503u) ^ (wave * 97u) ^ (blockIdx.x * 7919u);
    sa[i] = 0x3F003F00u | (h & 0x807F807Fu);
    sb[i] = 0x3F003F00u | ((h >> 7) & 0x807F807Fu);
  }
  f32x16 acc[MFMA_CHAINS];
#pragma unroll
  for (int c = 0; c < MFMA_CHAINS; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  uint64_t t0 = 0, r0 = 0;
  if (ticks && wave == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{sa[0], sa[1], sa[2], sa[3]});
    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{sb[0], sb[1], sb[2], sb[3]});
#pragma unroll
    for (int c = 0; c < MFMA_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    // new mantissas and signs for the next round (exponents unchanged: finite values)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] ^= 0x80558055u;
      sb[i] ^= 0x002A802Au;
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MFMA_CHAINS; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (ticks && wave == 0) {
    // the accumulators are final here: the sum above waited for the last MFMAs
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      ticks[2 * (int64_t)blockIdx.x] = t1 - t0;
      ticks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
    }
  }
}

hipError_t mfma_loop(float* out, uint64_t* ticks, int blocks, int iters, hipStream_t stream) {
  if (blocks < 1 || iters < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, stream, out, ticks, iters);
  return hipGetLastError();
}

}  // namespace aenc
