// fp32 GEMM on the vector ALUs for the fp32 tower: C = epilogue(A W^T + b).
//
// The fp32 geometry is small (it exists for exact parity), so this is a plain
// LDS-tiled kernel: a 256-thread workgroup computes a 64 x 64 tile, each
// thread a 4 x 4 block, K in slices of 16 staged k-major in LDS. It shares the
// row maps and fused epilogues of the bf16 kernel.
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace aenc {

constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, RowMap arow,
                                                       const float* __restrict__ W, int64_t ldw, int M_arg,
                                                       int N, int K, const int32_t* m_dev, EpiParams ep) {
  __shared__ float As[F_BK][F_BM + 4];
  __shared__ float Bs[F_BK][F_BN + 4];
  const int M = m_dev ? *m_dev : M_arg;
  const int m0 = blockIdx.y * F_BM, n0 = blockIdx.x * F_BN;
  if (m0 >= M) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const float* a_src = A + arow.offset(min(m0 + lr, M - 1)) + lk;
  const float* b_src = W + (int64_t)min(n0 + lr, N - 1) * ldw + lk;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += F_BK) {
    const float4 a = *(const float4*)(a_src + k0);
    const float4 b = *(const float4*)(b_src + k0);
    As[lk + 0][lr] = a.x; As[lk + 1][lr] = a.y; As[lk + 2][lr] = a.z; As[lk + 3][lr] = a.w;
    Bs[lk + 0][lr] = b.x; Bs[lk + 1][lr] = b.y; Bs[lk + 2][lr] = b.z; Bs[lk + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < F_BK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 v = {acc[0][j], acc[1][j], acc[2][j], acc[3][j]};
    Epilogue<EPI>::apply4(ep, m0 + ty * 4, n0 + tx * 4 + j, v, M, N);
  }
}

template <int EPI>
static hipError_t launch(const float* A, RowMap arow, const float* W, int64_t ldw, int M, int N, int K,
                         const int32_t* m_dev, const EpiParams& ep, hipStream_t stream) {
  dim3 grid((N + F_BN - 1) / F_BN, (M + F_BM - 1) / F_BM);
  hipLaunchKernelGGL(gemm_f32_kernel<EPI>, grid, dim3(256), 0, stream, A, arow, W, ldw, M, N, K, m_dev, ep);
  return hipGetLastError();
}

hipError_t gemm_f32(int epi, const float* A, RowMap arow, const float* W, int64_t ldw, int M, int N, int K,
                    const int32_t* m_dev, const EpiParams& ep, hipStream_t stream) {
  if (K % F_BK != 0 || M <= 0 || N <= 0) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE_BF16: return launch<EPI_STORE_BF16>(A, arow, W, ldw, M, N, K, m_dev, ep, stream);
    case EPI_RESID_F32: return launch<EPI_RESID_F32>(A, arow, W, ldw, M, N, K, m_dev, ep, stream);
    case EPI_STORE_F32: return launch<EPI_STORE_F32>(A, arow, W, ldw, M, N, K, m_dev, ep, stream);
    case EPI_GELU_PE_F32: return launch<EPI_GELU_PE_F32>(A, arow, W, ldw, M, N, K, m_dev, ep, stream);
    case EPI_GELU_F32: return launch<EPI_GELU_F32>(A, arow, W, ldw, M, N, K, m_dev, ep, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aenc
