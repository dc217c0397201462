// bf16 GEMM on CDNA4 matrix cores: C = epilogue(A W^T + b), fp32 accumulate.
//
// A [M, K] rows come through a RowMap (dense rows, or the overlapping
// strided rows that turn the k=3 convolutions into implicit GEMMs); W [N, K]
// is row-major (the [out, in] checkpoint layout). K must be a multiple of 64.
//
// Tiling: a 256-thread workgroup (4 wave64s) owns a BM x BN tile of C; each
// wave owns (BM/2) x (BN/2) and issues v_mfma_f32_32x32x16_bf16 on 32x32
// sub-tiles, accumulating in the AGPR half of the register file.
//
// K advances in slices of 64 through two LDS buffers. Slices are copied
// global -> LDS by global_load_lds_dwordx4 (gfx950): no staging registers
// and no LDS write instructions, so the registers go to the accumulators and
// to double-buffered MFMA fragments. The two buffers are distinct LDS objects
// and the slice loop is unrolled by two, so the copy into one buffer never
// forces a wait in front of the reads of the other.
//
// LDS rows are 128 bytes (64 bf16 of K). The LDS serves a 128-bit read for 16
// lanes per cycle from 64 four-byte banks, i.e. two rows' worth of banks, so
// the 16-byte chunk c of row r is stored at position c ^ ((r / 2) mod 8):
// sixteen consecutive rows reading the same chunk then hit 16 distinct bank
// groups. The direct-to-LDS copy writes 16 bytes per lane at consecutive
// addresses, so each lane fetches the global chunk that belongs at its LDS
// position.
//
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

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// Per-lane element offsets (from the operand base) of the rows this lane
// copies, one per copy instruction.
template <int ROWS>
struct CopyPlan {
  int32_t off[ROWS / 32];
};

// Copy one 64-wide K slice of ROWS rows into an LDS tile: each wave issues
// ROWS/32 instructions of 8 rows (64 lanes x 16 bytes).
template <int ROWS>
__device__ __forceinline__ void copy_slice(const bf16_t* base, const CopyPlan<ROWS>& plan, int k0, bf16_t* lds,
                                           int wave) {
#pragma unroll
  for (int i = 0; i < ROWS / 32; ++i) {
    const int row0 = (wave * (ROWS / 32) + i) * 8;
    __builtin_amdgcn_global_load_lds((gbl_void*)(base + plan.off[i] + k0), (lds_void*)(lds + row0 * GEMM_BK), 16, 0,
                                     0);
  }
}

// vmcnt(0): every global -> LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x3f70); }

// Fragments of one 16-wide K step: rows (lane & 31) of each 32-row sub-tile,
// K half (lane >> 5); the 16-byte chunk index is swizzled by (row / 2) mod 8.
template <int S>
__device__ __forceinline__ void read_frags(const bf16_t* base, int row0, int ch, bf16x8 (&f)[S]) {
#pragma unroll
  for (int i = 0; i < S; ++i) f[i] = *(const bf16x8*)(base + (row0 + 32 * i) * GEMM_BK + ch * 8);
}

template <int SM, int SN>
__device__ __forceinline__ void mma(f32x16 (&acc)[SM][SN], const bf16x8 (&fa)[SM], const bf16x8 (&fb)[SN]) {
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// One 64-wide K slice from LDS tiles (as, bs). Fragments of step s+1 are read
// while step s multiplies; the copies of the next slice (if any) are spread
// over the four steps instead of issued in one burst; the MFMA bursts run at
// raised wave priority so that, with two workgroups per CU, the SIMD's other
// wave does its memory work in the gaps. Scheduler barriers pin this order.
template <int SM, int SN, class Copy>
__device__ __forceinline__ void slice(f32x16 (&acc)[SM][SN], const bf16_t* as, const bf16_t* bs, int a_row0,
                                      int b_row0, int fr, int fk, Copy&& copy_part) {
  bf16x8 fa0[SM], fb0[SN], fa1[SM], fb1[SN];
  const int sw = (fr >> 1) & 7;   // sub-tile rows start on multiples of 16
  read_frags<SM>(as, a_row0, (0 + fk) ^ sw, fa0);
  read_frags<SN>(bs, b_row0, (0 + fk) ^ sw, fb0);
  read_frags<SM>(as, a_row0, (2 + fk) ^ sw, fa1);
  read_frags<SN>(bs, b_row0, (2 + fk) ^ sw, fb1);
  __builtin_amdgcn_sched_barrier(0);
  copy_part(0);
  __builtin_amdgcn_s_setprio(1);
  mma<SM, SN>(acc, fa0, fb0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<SM>(as, a_row0, (4 + fk) ^ sw, fa0);
  read_frags<SN>(bs, b_row0, (4 + fk) ^ sw, fb0);
  copy_part(1);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  mma<SM, SN>(acc, fa1, fb1);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<SM>(as, a_row0, (6 + fk) ^ sw, fa1);
  read_frags<SN>(bs, b_row0, (6 + fk) ^ sw, fb1);
  copy_part(2);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  mma<SM, SN>(acc, fa0, fb0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  copy_part(3);
  __builtin_amdgcn_s_setprio(1);
  mma<SM, SN>(acc, fa1, fb1);
  __builtin_amdgcn_s_setprio(0);
}

// Part q (0..3) of the copy of one K slice: a quarter of this wave's copy
// instructions (A rows first, then W rows).
template <int BM, int BN>
struct SliceCopy {
  const bf16_t* A;
  const bf16_t* W;
  const CopyPlan<BM>* pa;
  const CopyPlan<BN>* pb;
  int k0;
  bf16_t* la;
  bf16_t* lb;
  int wave;
  bool live;   // uniform: false when there is no next slice
  __device__ __forceinline__ void operator()(int q) const {
    constexpr int NA = BM / 32, NB = BN / 32, N = NA + NB, PER = N / 4;
    static_assert(N % 4 == 0, "copy instructions split into four parts");
    if (!live) return;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = q * PER + j;
      if (c < NA) {
        const int row0 = (wave * NA + c) * 8;
        __builtin_amdgcn_global_load_lds((gbl_void*)(A + pa->off[c] + k0), (lds_void*)(la + row0 * GEMM_BK), 16,
                                         0, 0);
      } else {
        const int cb = c - NA;
        const int row0 = (wave * NB + cb) * 8;
        __builtin_amdgcn_global_load_lds((gbl_void*)(W + pb->off[cb] + k0), (lds_void*)(lb + row0 * GEMM_BK), 16,
                                         0, 0);
      }
    }
  }
};

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int SM = WM / 32, SN = WN / 32;   // 32x32 sub-tiles per wave
  // Two slice buffers, A rows then W rows, as distinct LDS objects.
  __shared__ __attribute__((aligned(16))) bf16_t buf0[(BM + BN) * GEMM_BK];
  __shared__ __attribute__((aligned(16))) bf16_t buf1[(BM + BN) * GEMM_BK];

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
  const int wm = wave >> 1, wn = wave & 1;

  // ---- copy plans: lane l of an instruction covers row row0 + l/8 (row0 a
  //      multiple of 8) and LDS chunk l%8, which holds the global chunk
  //      (l%8) ^ ((row / 2) mod 8) ----
  const int c_row = lane >> 3;
  const int c_chunk_lo = (lane & 7) ^ (c_row >> 1);        // rows with (row0/2) % 8 == 0
  const int c_chunk_hi = (lane & 7) ^ ((c_row >> 1) + 4);  // rows with (row0/2) % 8 == 4
  CopyPlan<BM> pa;
  CopyPlan<BN> pb;
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int row0 = (wave * (BM / 32) + i) * 8;
    const int r = row0 + c_row;
    pa.off[i] = (int32_t)g.arow.offset(min(m0 + r, M - 1)) + ((row0 & 8) ? c_chunk_hi : c_chunk_lo) * 8;
  }
#pragma unroll
  for (int i = 0; i < BN / 32; ++i) {
    const int row0 = (wave * (BN / 32) + i) * 8;
    const int r = row0 + c_row;
    pb.off[i] = (int32_t)((int64_t)min(n0 + r, g.N - 1) * g.ldw) + ((row0 & 8) ? c_chunk_hi : c_chunk_lo) * 8;
  }

  f32x16 acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fk = lane >> 5;
  const int a_row0 = wm * WM + fr;
  const int b_row0 = wn * WN + fr;
  bf16_t* const a0 = buf0;
  bf16_t* const b0 = buf0 + BM * GEMM_BK;
  bf16_t* const a1 = buf1;
  bf16_t* const b1 = buf1 + BM * GEMM_BK;

  const int nk = g.K / GEMM_BK;
  copy_slice<BM>(g.A, pa, 0, a0, wave);
  copy_slice<BN>(g.W, pb, 0, b0, wave);
  wait_copies();
  __syncthreads();

  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    // slice kt from buffer 0 while slice kt+1 lands in buffer 1
    slice<SM, SN>(acc, a0, b0, a_row0, b_row0, fr, fk,
                  SliceCopy<BM, BN>{g.A, g.W, &pa, &pb, (kt + 1) * GEMM_BK, a1, b1, wave, true});
    wait_copies();
    __syncthreads();
    // slice kt+1 from buffer 1 while slice kt+2 (if any) lands in buffer 0
    slice<SM, SN>(acc, a1, b1, a_row0, b_row0, fr, fk,
                  SliceCopy<BM, BN>{g.A, g.W, &pa, &pb, (kt + 2) * GEMM_BK, a0, b0, wave, kt + 2 < nk});
    wait_copies();
    __syncthreads();
  }
  if (kt < nk) {   // odd slice count: the last slice sits in buffer 0
    slice<SM, SN>(acc, a0, b0, a_row0, b_row0, fr, fk,
                  SliceCopy<BM, BN>{g.A, g.W, &pa, &pb, 0, a1, b1, wave, false});
    __syncthreads();
  }

  // ---- epilogue through LDS: each wave stages 32-row slabs of its fp32 tile
  //      (lane holds column lane&31 and rows 8*(v/4) + 4*(lane>>5) + v%4 of each
  //      32x32 sub-tile), then writes them back row-contiguously ----
  // Slab rows padded to WN + 8 floats: lanes 32-63 write 4 rows below lanes
  // 0-31, which then lands on the other half of the 64 banks.
  constexpr int LDW = WN + 8;
  float* slab = (float*)(wave < 2 ? buf0 : buf1) + (wave & 1) * (32 * LDW);
  const int col0 = n0 + wn * WN;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) slab[(8 * (v >> 2) + 4 * fk + (v & 3)) * LDW + 32 * j + fr] = acc[i][j][v];
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the slab is written
    __builtin_amdgcn_wave_barrier();
    Epilogue<EPI>::template slab32<WN, LDW>(g.epi, slab, m0 + wm * WM + 32 * i, col0, lane, M, g.N);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next slab overwrites it
    __builtin_amdgcn_wave_barrier();
  }
}

template <int BM, int BN, int EPI>
static hipError_t launch_cfg(const GemmArgs& in, hipStream_t stream) {
  GemmArgs g = in;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  const int total = g.tiles_m * g.tiles_n;
  g.grid = (total + N_XCD - 1) / N_XCD * N_XCD;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, EPI>), dim3(g.grid), dim3(GEMM_THREADS), 0, stream, g);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, int tile_cfg, hipStream_t stream) {
  switch (tile_cfg) {
    case GEMM_TILE_256x256: return launch_cfg<256, 256, EPI>(g, stream);
    case GEMM_TILE_256x128: return launch_cfg<256, 128, EPI>(g, stream);
    case GEMM_TILE_128x128: return launch_cfg<128, 128, EPI>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_bf16(int epi, const bf16_t* A, RowMap arow, const bf16_t* W, int64_t ldw, int M, int N, int K,
                     const int32_t* m_dev, const EpiParams& ep, int tile_cfg, hipStream_t stream) {
  // K in whole slices; N in groups of 4 (the epilogue writes 4 columns per lane).
  if (K % GEMM_BK != 0 || M <= 0 || N <= 0 || N % 4 != 0) return hipErrorInvalidValue;
  // V columns of the QKV epilogue start on a wave boundary.
  if (epi == EPI_QKV_BF16 && ep.n_split % 128 != 0) return hipErrorInvalidValue;
  // The copy plans hold 32-bit element offsets.
  if ((int64_t)N * ldw >= INT32_MAX) return hipErrorInvalidValue;
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
