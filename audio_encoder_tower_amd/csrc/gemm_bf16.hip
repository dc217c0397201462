// bf16 GEMM on CDNA4 matrix cores: C = epilogue(A W^T + b), fp32 accumulate.
//
// A [M, K] rows come through a RowMap (dense rows, or the overlapping
// strided rows that turn the k=3 convolutions into implicit GEMMs); W [N, K]
// is row-major (the [out, in] checkpoint layout). K must be a multiple of 64.
//
// Tiling: a 256-thread workgroup (4 wave64s) owns a BM x BN tile of C; each
// wave owns WM x WN and issues v_mfma_f32_32x32x16_bf16 on 32x32 sub-tiles.
// K advances in slices of 64 staged through LDS with two buffers: the global
// loads of slice k+1 are in flight while slice k feeds the matrix cores.
// LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by (row mod 8) so
// that the 128-bit fragment reads of eight consecutive rows hit distinct banks.
// Workgroup ids are remapped so that each of the 8 XCDs (private L2 each)
// works on a contiguous range of tiles, grouped GROUP_M tiles tall, so the A
// and W panels those tiles share stay in that XCD's L2.
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace aenc {

constexpr int GEMM_BK = 64;
constexpr int GEMM_THREADS = 256;
constexpr int GEMM_GROUP_M = 8;
constexpr int N_XCD = 8;

struct GemmArgs {
  const bf16_t* A;
  RowMap arow;
  const bf16_t* W;
  int64_t ldw;
  int M, N, K;
  const int32_t* m_dev;  // if set, M = *m_dev (rows beyond it are not computed)
  int tiles_m, tiles_n, grid;
  EpiParams epi;
};

__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row & 7)); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
  constexpr int SM = WM / 32, SN = WN / 32;        // 32x32 sub-tiles per wave
  constexpr int A_LD = BM * 8 / GEMM_THREADS;       // 16-byte chunks per thread per slice
  constexpr int B_LD = BN * 8 / GEMM_THREADS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* As = (bf16_t*)smem;                       // [2][BM][64]
  bf16_t* Bs = As + 2 * BM * GEMM_BK;               // [2][BN][64]

  // ---- tile selection: XCD-contiguous ranges, then GROUP_M-tall groups ----
  const int total = g.tiles_m * g.tiles_n;
  const int per_xcd = g.grid / N_XCD;
  const int tile = (blockIdx.x % N_XCD) * per_xcd + blockIdx.x / N_XCD;
  if (tile >= total) return;
  const int group_size = GEMM_GROUP_M * g.tiles_n;
  const int group = tile / group_size;
  const int first_m = group * GEMM_GROUP_M;
  const int gm = min(g.tiles_m - first_m, GEMM_GROUP_M);
  const int in_group = tile - group * group_size;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  const int M = g.m_dev ? *g.m_dev : g.M;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---- global load pointers (each thread: fixed chunk column, rows tid/8 + 32 i) ----
  const int ld_row = tid >> 3, ld_ch = tid & 7;
  const bf16_t* a_src[A_LD];
  const bf16_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = min(m0 + ld_row + 32 * i, M - 1);
    a_src[i] = g.A + g.arow.offset(r) + ld_ch * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = min(n0 + ld_row + 32 * i, g.N - 1);
    b_src[i] = g.W + (int64_t)r * g.ldw + ld_ch * 8;
  }
  const int st_off = ld_row * GEMM_BK + swz(ld_row, ld_ch) * 8;  // + 32*64*i per chunk

  u32x4 ra[A_LD], rb[B_LD];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4*)(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4*)(b_src[i] + k0);
  };
  auto lstore = [&](int buf) {
    bf16_t* a = As + buf * BM * GEMM_BK + st_off;
    bf16_t* b = Bs + buf * BN * GEMM_BK + st_off;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4*)(a + i * 32 * GEMM_BK) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *(u32x4*)(b + i * 32 * GEMM_BK) = rb[i];
  };

  f32x16 acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment rows of this lane
  const int fr = lane & 31, fk = lane >> 5;
  const int a_row0 = wm * WM + fr;
  const int b_row0 = wn * WN + fr;

  const int nk = g.K / GEMM_BK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GEMM_BK);
    const bf16_t* a_lds = As + buf * BM * GEMM_BK;
    const bf16_t* b_lds = Bs + buf * BN * GEMM_BK;
#pragma unroll
    for (int s = 0; s < GEMM_BK / 16; ++s) {
      const int ch = 2 * s + fk;
      bf16x8 af[SM], bfr[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        const int r = a_row0 + 32 * i;
        af[i] = *(const bf16x8*)(a_lds + r * GEMM_BK + swz(r, ch) * 8);
      }
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int r = b_row0 + 32 * j;
        bfr[j] = *(const bf16x8*)(b_lds + r * GEMM_BK + swz(r, ch) * 8);
      }
#pragma unroll
      for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 31); rows 8*(v/4) + 4*(lane>>5) + v%4 ----
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = m0 + wm * WM + 32 * i + 8 * q + 4 * fk;
        const int n = n0 + wn * WN + 32 * j + fr;
        const f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
        Epilogue<EPI>::apply4(g.epi, r0, n, v, M, g.N);
      }
}

template <int BM, int BN, int WM, int WN, int EPI>
static hipError_t launch_cfg(const GemmArgs& in, hipStream_t stream) {
  GemmArgs g = in;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  const int total = g.tiles_m * g.tiles_n;
  g.grid = (total + N_XCD - 1) / N_XCD * N_XCD;
  const size_t lds = (size_t)2 * (BM + BN) * GEMM_BK * sizeof(bf16_t);
  static bool attr_set = false;
  if (!attr_set) {
    // Raise the dynamic LDS limit of this instance above 64 KiB (gfx950 has 160 KiB).
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<BM, BN, WM, WN, EPI>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI>), dim3(g.grid), dim3(GEMM_THREADS), lds, stream, g);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, int tile_cfg, hipStream_t stream) {
  switch (tile_cfg) {
    case GEMM_TILE_256x256: return launch_cfg<256, 256, 128, 128, EPI>(g, stream);
    case GEMM_TILE_256x128: return launch_cfg<256, 128, 128, 64, EPI>(g, stream);
    case GEMM_TILE_128x128: return launch_cfg<128, 128, 64, 64, EPI>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_bf16(int epi, const bf16_t* A, RowMap arow, const bf16_t* W, int64_t ldw, int M, int N, int K,
                     const int32_t* m_dev, const EpiParams& ep, int tile_cfg, hipStream_t stream) {
  if (K % GEMM_BK != 0 || M <= 0 || N <= 0) return hipErrorInvalidValue;
  GemmArgs g{};
  g.A = A; g.arow = arow; g.W = W; g.ldw = ldw; g.M = M; g.N = N; g.K = K; g.m_dev = m_dev; g.epi = ep;
  switch (epi) {
    case EPI_STORE_BF16: return launch_epi<EPI_STORE_BF16>(g, tile_cfg, stream);
    case EPI_GELU_BF16: return launch_epi<EPI_GELU_BF16>(g, tile_cfg, stream);
    case EPI_RESID_F32: return launch_epi<EPI_RESID_F32>(g, tile_cfg, stream);
    case EPI_STORE_F32: return launch_epi<EPI_STORE_F32>(g, tile_cfg, stream);
    case EPI_GELU_PE_F32: return launch_epi<EPI_GELU_PE_F32>(g, tile_cfg, stream);
    case EPI_QKV_BF16: return launch_epi<EPI_QKV_BF16>(g, tile_cfg, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aenc
