// bf16 GEMM on CDNA4 matrix cores: C = epilogue(A W^T + b), fp32 accumulate.
//
// A [M, K] rows come through a RowMap (dense rows, or the overlapping
// strided rows that turn the k=3 convolutions into implicit GEMMs); W [N, K]
// is row-major (the [out, in] checkpoint layout). K must be a multiple of 64.
// Every wave issues v_mfma_f32_32x32x16_bf16 on 32x32 sub-tiles of C.
//
// K advances in slices of 64 through LDS buffers. Slices are copied
// global -> LDS by buffer_load_dwordx4 ... lds (direct to LDS, gfx950): no
// staging registers and no LDS write instructions, and the slice's K offset
// rides in the scalar offset, so a copy instruction needs no per-lane address
// arithmetic. The buffers are distinct LDS objects and the slice loop is
// unrolled over them, so a copy into one buffer never forces a wait in front
// of the reads of another.
//
// LDS rows are 128 bytes (64 bf16 of K). The LDS serves a 128-bit read for 16
// lanes per cycle from 64 four-byte banks, i.e. two rows' worth of banks, so
// the 16-byte chunk c of row r is stored at position c ^ ((r / 2) mod 8):
// sixteen consecutive rows reading the same chunk then hit 16 distinct bank
// groups. The direct-to-LDS copy writes 16 bytes per lane at consecutive
// addresses, so each lane fetches the global chunk that belongs at its LDS
// position.
//
// Two tile shapes:
//  * 256x256, 8 waves (two per SIMD), each wave 64x128. The waves form two
//    groups that alternate roles every phase (ping-pong): while one group's
//    waves run a burst of 16 MFMAs at raised priority, the other group's
//    waves, on the same SIMDs, read their next fragments from LDS and issue
//    copies of coming slices; a workgroup barrier ends each phase. Three A
//    and two W slice buffers fill the CU's 160 KiB of LDS (one workgroup per
//    CU), so A slices are requested two slices ahead. Used for the large
//    GEMMs.
//  * 128x128, 4 waves, each wave 64x64, two workgroups per CU that overlap
//    each other's copies and MFMAs. Used when the 256x256 tiles would leave
//    most CUs idle (short batches).
//
// Workgroup ids are remapped so that each of the 8 XCDs (private L2 each)
// works on a contiguous range of tiles, grouped GROUP_M tiles tall, so the A
// and W panels those tiles share stay in that XCD's L2.
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace aenc {

constexpr int GEMM_BK = 64;
constexpr int GEMM_GROUP_M = 4;
constexpr int N_XCD = 8;
constexpr int CUS_PER_XCD = 32;

struct GemmArgs {
  const bf16_t* A;
  RowMap arow;
  const bf16_t* W;
  int64_t ldw;
  int M, N, K;
  const int32_t* m_dev;  // if set, M = min(*m_dev, M) (rows beyond it are not computed)
  uint32_t a_bytes, w_bytes;   // extents of A and W reachable through the row maps
  int tiles_n;
  EpiParams epi;
  // 128x128 kernel only: split-K. `splits` launches' worth of tiles, split s
  // reducing K columns [s K, (s + 1) K) (K above is per split) and writing
  // its partial product (EPI_STORE_F32, no bias) at C offset s * c_split_stride.
  int splits;
  int64_t c_split_stride;
  // the device row count may be well below M (a masked batch): let the
  // workgroups decide the split tail from it
  bool rows_vary;
};

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over [base, base + bytes): raw addressing, 32-bit offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One direct-to-LDS copy: lane l moves 16 bytes from byte voff + soff of the
// buffer to LDS address lds + 16 l.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, bf16_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// vmcnt(0): every copy this wave issued has landed.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x3f70); }
// lgkmcnt(0): every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Workgroup barrier without the memory fences of __syncthreads (which would
// also wait for the copies in flight); the empty asm statements keep the
// compiler from moving memory accesses across it.
#define AENC_BARRIER()                   \
  do {                                   \
    __builtin_amdgcn_sched_barrier(0);   \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_sched_barrier(0);   \
  } while (0)

// Fragments of one 16-wide K step: rows (lane & 31) of each 32-row sub-tile,
// K half (lane >> 5); ch is the (swizzled) 16-byte chunk index.
template <int S>
__device__ __forceinline__ void read_frags(const bf16_t* base, int row0, int ch, bf16x8 (&f)[S]) {
#pragma unroll
  for (int i = 0; i < S; ++i) f[i] = *(const bf16x8*)(base + (row0 + 32 * i) * GEMM_BK + ch * 8);
}

// The MFMA computes the 32x32 block transposed: W rows are its first operand
// (the rows of its result) and A rows its second. A lane then holds one row
// of C (A row lane & 31) and 16 entries of W rows 8*(v/4) + 4*(lane>>5) +
// v%4; the copies place W rows in LDS permuted within each 32-row block (see
// plan_w) so that those are the 16 consecutive columns 16*(lane>>5) + v:
//   acc[i][j][v] = C[row0 + 32 i + (lane & 31)][col0 + 32 j + 16 (lane >> 5) + v].
template <int SM, int SN>
__device__ __forceinline__ void mma(f32x16 (&acc)[SM][SN], const bf16x8 (&fa)[SM], const bf16x8 (&fb)[SN]) {
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
}

// Tile index -> (tm, tn): GROUP_M-tall groups walked column by column.
__device__ __forceinline__ void tile_group_order(int tiles_m, int tiles_n, int tile, int& tm, int& tn) {
  const int group_size = GEMM_GROUP_M * tiles_n;
  const int group = tile / group_size;
  const int first_m = group * GEMM_GROUP_M;
  const int gm = min(tiles_m - first_m, GEMM_GROUP_M);
  const int in_group = tile - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Tile (tm, tn) of workgroup blockIdx.x for an M-row product (M read on the
// device, so a launch sized for the longest batch balances the rows a masked
// batch really has): the tiles are split into 8 contiguous ranges, one per XCD
// (workgroup b runs on XCD b mod 8), of total/8 or total/8 + 1 tiles, walked in
// group order. With SPLIT, when an XCD's range leaves a last round of at most
// 16 tiles on its 32 CUs, those tiles run as two 128-column halves each
// (`half` 0 or 1; -1 for a whole tile). False for workgroups past the work.
template <bool SPLIT>
__device__ __forceinline__ bool tile_of_block(const GemmArgs& g, int M, int BM, int& tm, int& tn, int& half,
                                              int* ksplit = nullptr) {
  const int tiles_m = (M + BM - 1) / BM;
  const int per_split = tiles_m * g.tiles_n;
  const int total = per_split * (ksplit ? g.splits : 1);
  const int x = blockIdx.x % N_XCD, i = blockIdx.x / N_XCD;
  const int base = total / N_XCD, rem = total % N_XCD;
  const int cnt = base + (x < rem ? 1 : 0), first = x * base + min(x, rem);
  int full = cnt;
  if (SPLIT) {
    const int tail = cnt % CUS_PER_XCD;
    if (cnt > CUS_PER_XCD && tail > 0 && 2 * tail <= CUS_PER_XCD) full = cnt - tail;
  }
  int t = i;
  half = -1;
  if (i >= full) {
    if (i >= full + 2 * (cnt - full)) return false;
    t = full + (i - full) / 2;
    half = (i - full) & 1;
  }
  if (t >= cnt) return false;
  int tile = first + t;
  if (ksplit) {
    *ksplit = tile / per_split;   // the split is the slowest index: an XCD's range stays within few splits
    tile -= *ksplit * per_split;
  }
  tile_group_order(tiles_m, g.tiles_n, tile, tm, tn);
  return true;
}

// Per-lane byte offsets of the rows this lane copies, one per copy
// instruction: instruction i of wave w covers rows (w * NI + i) * 8 ..+8;
// lane l takes row +l/8 and LDS chunk l%8, which holds global chunk
// (l%8) ^ ((row / 2) mod 8).
template <int NI>
struct CopyPlan {
  uint32_t off[NI];
};

template <int NI>
__device__ __forceinline__ CopyPlan<NI> plan_a(const GemmArgs& g, int m0, int M, int wave, int lane) {
  const int c_row = lane >> 3;
  CopyPlan<NI> p;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row0 = (wave * NI + i) * 8;
    const int ch = (lane & 7) ^ ((c_row >> 1) + ((row0 & 8) ? 4 : 0));
    p.off[i] = (uint32_t)((g.arow.offset(min(m0 + row0 + c_row, M - 1)) + ch * 8) * 2);
  }
  return p;
}

// W rows go to LDS permuted within each 32-row block: LDS row r = 8 g + 4 h + q
// (g < 4, h < 2, q < 4) holds W row 16 h + 4 g + q of the block, which makes
// the MFMA result rows a lane holds (see mma) consecutive output columns.
__device__ __forceinline__ int w_row_of_lds_row(int r) {
  return (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}

template <int NI>
__device__ __forceinline__ CopyPlan<NI> plan_w(const GemmArgs& g, int n0, int wave, int lane) {
  const int c_row = lane >> 3;
  CopyPlan<NI> p;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row0 = (wave * NI + i) * 8;
    const int ch = (lane & 7) ^ ((c_row >> 1) + ((row0 & 8) ? 4 : 0));
    const int n = n0 + w_row_of_lds_row(row0 + c_row);
    p.off[i] = (uint32_t)(((int64_t)min(n, g.N - 1) * g.ldw + ch * 8) * 2);
  }
  return p;
}

// Accumulators start at the bias of their columns (zero past N, or without a
// bias), so the epilogues add none: the bias loads are issued with the first
// slice copies instead of waited for in the epilogue, where they cost 5% of
// fc1. acc[i][j] holds columns col0 + 32 j + 16 (lane >> 5) + 0..15.
template <int SM, int SN>
__device__ __forceinline__ void init_acc(f32x16 (&acc)[SM][SN], const float* bias, int col0, int N, int lane) {
  const int fk = lane >> 5;
#pragma unroll
  for (int j = 0; j < SN; ++j) {
    f32x16 b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = col0 + 32 * j + 16 * fk + 4 * q;   // N is a multiple of 4
      const float4 v = (bias && n < N) ? *(const float4*)(bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
      b[4 * q] = v.x;
      b[4 * q + 1] = v.y;
      b[4 * q + 2] = v.z;
      b[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[i][j] = b;
  }
}

// Epilogue. A lane holds 16 consecutive columns of one row per 32x32 block
// (see mma), so bf16 outputs are finished in registers and written directly,
// 16 bytes per lane (8 columns). fp32 outputs and the V^T part of the QKV
// epilogue go through LDS instead: a wave stages its accumulators as 32-row
// slabs SW columns wide (16-byte writes; rows padded to SW + 4 floats so that
// the 16 lanes of one write cycle cover all 64 banks), then writes each slab
// back row-contiguously (or column-contiguously for V^T). Staging measured
// faster for the fp32 residual update (its loads and stores stay fully
// coalesced) and slower for bf16 stores.
template <int EPI, int SM, int SN>
__device__ __forceinline__ void store_direct_bf16(const GemmArgs& g, const f32x16 (&acc)[SM][SN], int row0, int col0,
                                                  int lane, int M) {
  const EpiParams& p = g.epi;
  const int fr = lane & 31, fk = lane >> 5;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int m = row0 + 32 * i + fr;
    const int64_t o = m < M ? p.crow.offset(m) : -1;
    if (o < 0) continue;
    bf16_t* const crow = (bf16_t*)p.c + o;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int n = col0 + 32 * j + 16 * fk + 8 * c;
        if (n >= g.N) continue;
        const bool full = n + 8 <= g.N;   // else 4 columns (N is a multiple of 4)
        float v[8];   // biased sums (init_acc)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[i][j][8 * c + e];
        if (EPI == EPI_QKV_BF16 && n < p.q_cols) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= p.q_scale;
        }
        if (EPI == EPI_GELU_BF16) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_bf16out(v[e]);
        }
        u32x2 lo, hi;
        lo.x = pack_bf16x2(v[0], v[1]);
        lo.y = pack_bf16x2(v[2], v[3]);
        hi.x = pack_bf16x2(v[4], v[5]);
        hi.y = pack_bf16x2(v[6], v[7]);
        if (full && ((o + n) & 7) == 0) {
          *(uint4*)(crow + n) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          *(u32x2*)(crow + n) = lo;
          if (full) *(u32x2*)(crow + n + 4) = hi;
        }
      }
    }
  }
}

template <int EPI, int SM, int SN, int SW>
__device__ __forceinline__ void store_tile(const GemmArgs& g, const f32x16 (&acc)[SM][SN], float* slab, int row0,
                                           int col0, int lane, int M) {
  if (EPI == EPI_STORE_BF16 || EPI == EPI_GELU_BF16 || (EPI == EPI_QKV_BF16 && col0 < g.epi.n_split)) {
    store_direct_bf16<EPI, SM, SN>(g, acc, row0, col0, lane, M);
    return;
  }
  constexpr int LDW = SW + 4, JW = SW / 32;
  const int fr = lane & 31, fk = lane >> 5;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
#pragma unroll
    for (int jh = 0; jh < SN / JW; ++jh) {
#pragma unroll
      for (int j = 0; j < JW; ++j) {
        const f32x16& a = acc[i][jh * JW + j];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(slab + fr * LDW + 32 * j + 16 * fk + 4 * q) =
              make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
      }
      wait_lds();   // the slab is written
      __builtin_amdgcn_wave_barrier();
      Epilogue<EPI>::template slab32<SW, LDW>(g.epi, slab, row0 + 32 * i, col0 + SW * jh, lane, M, g.N);
      wait_lds();   // reads done before the next slab overwrites it
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 tiles, 4 waves (2 x 2), two workgroups per CU.
// ---------------------------------------------------------------------------
constexpr int SMALL_THREADS = 256;

// The copies of one slice split in four parts (A rows first, then W rows),
// spread over the four K steps of the slice being multiplied.
struct SmallCopy {
  __amdgpu_buffer_rsrc_t ra, rw;
  const CopyPlan<4>* pa;
  const CopyPlan<4>* pw;
  uint32_t k_bytes;
  bf16_t* la;
  bf16_t* lw;
  int wave;
  bool live;   // uniform: false when there is no next slice
  __device__ __forceinline__ void operator()(int q) const {
    if (!live) return;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = q * 2 + j;
      if (c < 4) copy16(ra, la + (wave * 4 + c) * 8 * GEMM_BK, pa->off[c], k_bytes);
      else copy16(rw, lw + (wave * 4 + c - 4) * 8 * GEMM_BK, pw->off[c - 4], k_bytes);
    }
  }
};

// One 64-wide K slice from LDS tiles (as, bs). Fragments of step s+1 are read
// while step s multiplies; the copies of the next slice are spread over the
// four steps; the MFMA bursts run at raised wave priority so that the other
// workgroup's wave on the SIMD does its memory work in the gaps. Scheduler
// barriers pin this order.
template <int SM, int SN>
__device__ __forceinline__ void small_slice(f32x16 (&acc)[SM][SN], const bf16_t* as, const bf16_t* bs, int a_row0,
                                            int b_row0, int fr, int fk, const SmallCopy& copy_part) {
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

// SPLITK: the launch splits K (GemmArgs.splits); a separate instantiation.
template <int EPI, bool SPLITK>
__global__ __launch_bounds__(SMALL_THREADS) void gemm_bf16_128_kernel(GemmArgs g) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64;
  constexpr int SM = WM / 32, SN = WN / 32;
  __shared__ __attribute__((aligned(16))) bf16_t buf0[(BM + BN) * GEMM_BK];
  __shared__ __attribute__((aligned(16))) bf16_t buf1[(BM + BN) * GEMM_BK];

  const int M = g.m_dev ? min(*g.m_dev, g.M) : g.M;
  int tm, tn, half, ks = 0;
  if (!tile_of_block<false>(g, M, BM, tm, tn, half, SPLITK ? &ks : nullptr)) return;
  const int m0 = tm * BM, n0 = tn * BN;
  // split ks reads K columns from ks * K on: a scalar byte offset on every copy
  const uint32_t kb0 = SPLITK ? (uint32_t)ks * (uint32_t)g.K * 2u : 0u;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const CopyPlan<4> pa = plan_a<4>(g, m0, M, wave, lane);
  const CopyPlan<4> pw = plan_w<4>(g, n0, wave, lane);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes), rw = make_rsrc(g.W, g.w_bytes);

  f32x16 acc[SM][SN];
  init_acc<SM, SN>(acc, g.epi.bias, n0 + wn * WN, g.N, lane);   // no bias on split-K partials (null)

  const int fr = lane & 31, fk = lane >> 5;
  const int a_row0 = wm * WM + fr;
  const int b_row0 = wn * WN + fr;
  bf16_t* const a0 = buf0;
  bf16_t* const b0 = buf0 + BM * GEMM_BK;
  bf16_t* const a1 = buf1;
  bf16_t* const b1 = buf1 + BM * GEMM_BK;

  const int nk = g.K / GEMM_BK;
  {
    const SmallCopy first{ra, rw, &pa, &pw, kb0, a0, b0, wave, true};
    first(0);
    first(1);
    first(2);
    first(3);
  }
  wait_copies();
  __syncthreads();

  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    // slice kt from buffer 0 while slice kt+1 lands in buffer 1
    small_slice<SM, SN>(acc, a0, b0, a_row0, b_row0, fr, fk,
                        SmallCopy{ra, rw, &pa, &pw, kb0 + (uint32_t)(kt + 1) * GEMM_BK * 2, a1, b1, wave, true});
    wait_copies();
    __syncthreads();
    // slice kt+1 from buffer 1 while slice kt+2 (if any) lands in buffer 0
    small_slice<SM, SN>(acc, a1, b1, a_row0, b_row0, fr, fk,
                        SmallCopy{ra, rw, &pa, &pw, kb0 + (uint32_t)(kt + 2) * GEMM_BK * 2, a0, b0, wave, kt + 2 < nk});
    wait_copies();
    __syncthreads();
  }
  if (kt < nk) {   // odd slice count: the last slice sits in buffer 0
    small_slice<SM, SN>(acc, a0, b0, a_row0, b_row0, fr, fk, SmallCopy{ra, rw, &pa, &pw, 0, a1, b1, wave, false});
    __syncthreads();
  }

  constexpr int SW = WN;
  float* slab = (float*)(wave < 2 ? buf0 : buf1) + (wave & 1) * (32 * (SW + 4));
  if (SPLITK) {
    GemmArgs gs = g;   // split ks writes its partial product at C + ks * c_split_stride
    gs.epi.crow.off += (int64_t)ks * g.c_split_stride;
    store_tile<EPI, SM, SN, SW>(gs, acc, slab, m0 + wm * WM, n0 + wn * WN, lane, M);
  } else {
    store_tile<EPI, SM, SN, SW>(g, acc, slab, m0 + wm * WM, n0 + wn * WN, lane, M);
  }
}

// ---------------------------------------------------------------------------
// 256x256 tiles, 8 waves (4 x 2) in two ping-pong groups, one workgroup per CU.
// ---------------------------------------------------------------------------
constexpr int BIG_THREADS = 512;

typedef int i32x4_asm __attribute__((ext_vector_type(4)));

// The fragments of half a slice (two K steps) and the wait for them, as one
// asm block: the compiler's wait insertion then never sees these LDS reads, so
// it does not make them wait for the direct-to-LDS copies in flight (it cannot
// tell that those target other buffers once there are more than two).
template <int SM, int SN>
__device__ __forceinline__ void read_half_wait(const bf16_t* as, const bf16_t* bs, int a_row0, int b_row0, int sw,
                                               int fk, int h, bf16x8 (&fa)[2][SM], bf16x8 (&fb)[2][SN]) {
  static_assert(SM == 2 && (SN == 4 || SN == 2), "written for the 64x128 and 64x64 wave tiles");
  const uint32_t ab = (uint32_t)(uintptr_t)(lds_void*)as, bb = (uint32_t)(uintptr_t)(lds_void*)bs;
  const uint32_t pa0 = ab + (a_row0 * GEMM_BK + ((4 * h + 0 + fk) ^ sw) * 8) * 2;
  const uint32_t pa1 = ab + (a_row0 * GEMM_BK + ((4 * h + 2 + fk) ^ sw) * 8) * 2;
  const uint32_t pb0 = bb + (b_row0 * GEMM_BK + ((4 * h + 0 + fk) ^ sw) * 8) * 2;
  const uint32_t pb1 = bb + (b_row0 * GEMM_BK + ((4 * h + 2 + fk) ^ sw) * 8) * 2;
  if constexpr (SN == 2) {
    i32x4_asm r[8];
    asm volatile(
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %8 offset:4096\n"
        "ds_read_b128 %2, %9\n"
        "ds_read_b128 %3, %9 offset:4096\n"
        "ds_read_b128 %4, %10\n"
        "ds_read_b128 %5, %10 offset:4096\n"
        "ds_read_b128 %6, %11\n"
        "ds_read_b128 %7, %11 offset:4096\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(pa0), "v"(pb0), "v"(pa1), "v"(pb1)
        : "memory");
    fa[0][0] = __builtin_bit_cast(bf16x8, r[0]);
    fa[0][1] = __builtin_bit_cast(bf16x8, r[1]);
    fb[0][0] = __builtin_bit_cast(bf16x8, r[2]);
    fb[0][1] = __builtin_bit_cast(bf16x8, r[3]);
    fa[1][0] = __builtin_bit_cast(bf16x8, r[4]);
    fa[1][1] = __builtin_bit_cast(bf16x8, r[5]);
    fb[1][0] = __builtin_bit_cast(bf16x8, r[6]);
    fb[1][1] = __builtin_bit_cast(bf16x8, r[7]);
  } else {
    i32x4_asm r[12];
    asm volatile(
        "ds_read_b128 %0, %12\n"
        "ds_read_b128 %1, %12 offset:4096\n"
        "ds_read_b128 %2, %13\n"
        "ds_read_b128 %3, %13 offset:4096\n"
        "ds_read_b128 %4, %13 offset:8192\n"
        "ds_read_b128 %5, %13 offset:12288\n"
        "ds_read_b128 %6, %14\n"
        "ds_read_b128 %7, %14 offset:4096\n"
        "ds_read_b128 %8, %15\n"
        "ds_read_b128 %9, %15 offset:4096\n"
        "ds_read_b128 %10, %15 offset:8192\n"
        "ds_read_b128 %11, %15 offset:12288\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
        : "v"(pa0), "v"(pb0), "v"(pa1), "v"(pb1)
        : "memory");
    fa[0][0] = __builtin_bit_cast(bf16x8, r[0]);
    fa[0][1] = __builtin_bit_cast(bf16x8, r[1]);
    fb[0][0] = __builtin_bit_cast(bf16x8, r[2]);
    fb[0][1] = __builtin_bit_cast(bf16x8, r[3]);
    fb[0][2] = __builtin_bit_cast(bf16x8, r[4]);
    fb[0][3] = __builtin_bit_cast(bf16x8, r[5]);
    fa[1][0] = __builtin_bit_cast(bf16x8, r[6]);
    fa[1][1] = __builtin_bit_cast(bf16x8, r[7]);
    fb[1][0] = __builtin_bit_cast(bf16x8, r[8]);
    fb[1][1] = __builtin_bit_cast(bf16x8, r[9]);
    fb[1][2] = __builtin_bit_cast(bf16x8, r[10]);
    fb[1][3] = __builtin_bit_cast(bf16x8, r[11]);
  }
}

template <int SM, int SN>
__device__ __forceinline__ void compute_half(f32x16 (&acc)[SM][SN], const bf16x8 (&fa)[2][SM],
                                             const bf16x8 (&fb)[2][SN]) {
  __builtin_amdgcn_s_setprio(1);
  mma<SM, SN>(acc, fa[0], fb[0]);
  mma<SM, SN>(acc, fa[1], fb[1]);
  __builtin_amdgcn_s_setprio(0);
}

struct BigCopy {
  __amdgpu_buffer_rsrc_t ra, rw;
  CopyPlan<4> pa, pw;
  int wave;
  bool w_on;   // uniform: false for the waves whose W rows lie outside a half tile
  // this wave's 4 copy instructions of the A (or W) part of the slice at K byte offset k_bytes
  __device__ __forceinline__ void slice_a(uint32_t k_bytes, bf16_t* la) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) copy16(ra, la + (wave * 4 + i) * 8 * GEMM_BK, pa.off[i], k_bytes);
  }
  __device__ __forceinline__ void slice_w(uint32_t k_bytes, bf16_t* lw) const {
    if (!w_on) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) copy16(rw, lw + (wave * 4 + i) * 8 * GEMM_BK, pw.off[i], k_bytes);
  }
  // both parts: this wave's 8 copy instructions
  __device__ __forceinline__ void slice(uint32_t k_bytes, bf16_t* la, bf16_t* lw) const {
    slice_a(k_bytes, la);
    slice_w(k_bytes, lw);
  }
};

// vmcnt(4): everything but this wave's 4 most recent copies has landed.
__device__ __forceinline__ void wait_copies_but4() { __builtin_amdgcn_s_waitcnt(0x3f74); }

// One K slice in four phases, each closed by a workgroup barrier. Group 0
// reads fragments (half 0, then half 1) in phases 0 and 2 and multiplies in
// 1 and 3; group 1 runs one phase later (its phase-0 work is the second half
// of the previous slice). A slices run through three LDS buffers and W slices
// through two (160 KiB in all). As each group reads the first half of slice
// j it copies W slice j+1, and as it reads the second half, A slice j+2 (the
// buffers' last readers finished in slice j-1); at the end of the slice it
// waits for all but the A copies just issued. A (the activations, streamed
// from memory) thus has about one and a half slices of lead and W (shared by
// many tiles, mostly L2 hits) about one, and the copy path carries a quarter
// slice per phase: issuing a whole slice in one phase (two of four phases
// with copies) saturated the ~64 B/clk per CU of direct-to-LDS copies and
// left the phases without copies idle (fc2 6% slower). The fragment reads are
// asm blocks: with five DMA targets the compiler's wait insertion would
// otherwise make every LDS read wait for all copies in flight.
template <int G, int SM, int SN>
__device__ __forceinline__ void big_slice(f32x16 (&acc)[SM][SN], bf16x8 (&fa)[2][SM], bf16x8 (&fb)[2][SN],
                                           const bf16_t* ca, const bf16_t* cb, bf16_t* na, bf16_t* nb, int a_row0,
                                           int b_row0, int sw, int fk, const BigCopy& cp, int j, int nk,
                                           bool first) {
  const bool live_w = j + 1 < nk, live_a = j + 2 < nk;
  const uint32_t kb_w = (uint32_t)(j + 1) * GEMM_BK * 2, kb_a = (uint32_t)(j + 2) * GEMM_BK * 2;
  // phase 0
  if (G == 0) {
    if (live_w) cp.slice_w(kb_w, nb);
    read_half_wait<SM, SN>(ca, cb, a_row0, b_row0, sw, fk, 0, fa, fb);
  } else if (!first) {
    compute_half<SM, SN>(acc, fa, fb);
  }
  AENC_BARRIER();
  // phase 1
  if (G == 0) {
    compute_half<SM, SN>(acc, fa, fb);
  } else {
    if (live_w) cp.slice_w(kb_w, nb);
    read_half_wait<SM, SN>(ca, cb, a_row0, b_row0, sw, fk, 0, fa, fb);
  }
  AENC_BARRIER();
  // phase 2
  if (G == 0) {
    if (live_a) cp.slice_a(kb_a, na);
    read_half_wait<SM, SN>(ca, cb, a_row0, b_row0, sw, fk, 1, fa, fb);
  } else {
    compute_half<SM, SN>(acc, fa, fb);
  }
  AENC_BARRIER();
  // phase 3
  if (G == 0) {
    compute_half<SM, SN>(acc, fa, fb);
  } else {
    if (live_a) cp.slice_a(kb_a, na);
    read_half_wait<SM, SN>(ca, cb, a_row0, b_row0, sw, fk, 1, fa, fb);
  }
  if (live_a) wait_copies_but4();   // A slice j+1 and W slice j+1 have landed
  else wait_copies();
  AENC_BARRIER();
}

// Slice j sits in A buffer j mod 3 and W buffer j mod 2: six slices per trip.
template <int G, int SM, int SN>
__device__ __forceinline__ void big_loop(f32x16 (&acc)[SM][SN], bf16_t* a0, bf16_t* a1, bf16_t* a2, bf16_t* w0,
                                          bf16_t* w1, int a_row0, int b_row0, int sw, int fk, const BigCopy& cp,
                                          int nk) {
  bf16x8 fa[2][SM], fb[2][SN];
#define AENC_BIG_SLICE(T, CA, CB, NA, NB) \
  if (j + T < nk)                          \
    big_slice<G, SM, SN>(acc, fa, fb, CA, CB, NA, NB, a_row0, b_row0, sw, fk, cp, j + T, nk, T == 0 && j == 0);
  for (int j = 0; j < nk; j += 6) {
    AENC_BIG_SLICE(0, a0, w0, a2, w1)
    AENC_BIG_SLICE(1, a1, w1, a0, w0)
    AENC_BIG_SLICE(2, a2, w0, a1, w1)
    AENC_BIG_SLICE(3, a0, w1, a2, w0)
    AENC_BIG_SLICE(4, a1, w0, a0, w1)
    AENC_BIG_SLICE(5, a2, w1, a1, w0)
  }
#undef AENC_BIG_SLICE
  if (G == 1) compute_half<SM, SN>(acc, fa, fb);   // group 1's last half slice
  AENC_BARRIER();
}

// One 256-row tile of C, 256 columns wide (SN 4: 64x128 per wave) or, for a
// split tail, 128 wide (SN 2: 64x64 per wave; only waves 0-3 copy W, whose
// 128 rows fill the first half of each W buffer).
template <int EPI, int SN>
__device__ __forceinline__ void big_tile(const GemmArgs& g, int m0, int n0, int M, bf16_t* la0, bf16_t* la1,
                                         bf16_t* la2, bf16_t* lw0, bf16_t* lw1) {
  constexpr int WM = 64, WN = 32 * SN;
  constexpr int SM = WM / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  BigCopy cp;
  cp.ra = make_rsrc(g.A, g.a_bytes);
  cp.rw = make_rsrc(g.W, g.w_bytes);
  cp.pa = plan_a<4>(g, m0, M, wave, lane);
  cp.pw = plan_w<4>(g, n0, wave, lane);
  cp.wave = wave;
  cp.w_on = SN == 4 || wave < 4;

  f32x16 acc[SM][SN];
  init_acc<SM, SN>(acc, g.epi.bias, n0 + wn * WN, g.N, lane);

  const int fr = lane & 31, fk = lane >> 5;
  const int a_row0 = wm * WM + fr;
  const int b_row0 = wn * WN + fr;
  const int sw = (fr >> 1) & 7;
  const int nk = g.K / GEMM_BK;

  // A slices 0 and 1 and W slice 0 in flight; wait for A 0 and W 0
  cp.slice(0, la0, lw0);
  if (nk > 1) {
    cp.slice_a(GEMM_BK * 2, la1);
    wait_copies_but4();
  } else {
    wait_copies();
  }
  AENC_BARRIER();
  if (wave < 4)
    big_loop<0, SM, SN>(acc, la0, la1, la2, lw0, lw1, a_row0, b_row0, sw, fk, cp, nk);
  else
    big_loop<1, SM, SN>(acc, la0, la1, la2, lw0, lw1, a_row0, b_row0, sw, fk, cp, nk);

  constexpr int SW = 64;   // two waves' slabs (2 x 8.5 KiB) per 32 KiB buffer
  float* slab = (float*)(wave < 2 ? la0 : wave < 4 ? la1 : wave < 6 ? la2 : lw0) + (wave & 1) * (32 * (SW + 4));
  store_tile<EPI, SM, SN, SW>(g, acc, slab, m0 + wm * WM, n0 + wn * WN, lane, M);
}

// SPLIT: the launch has a split tail (a separate instantiation, so that
// launches without one run the whole-tile code alone).
template <int EPI, bool SPLIT>
__global__ __launch_bounds__(BIG_THREADS) void gemm_bf16_256_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 256;
  __shared__ __attribute__((aligned(16))) bf16_t la0[BM * GEMM_BK];
  __shared__ __attribute__((aligned(16))) bf16_t la1[BM * GEMM_BK];
  __shared__ __attribute__((aligned(16))) bf16_t la2[BM * GEMM_BK];
  __shared__ __attribute__((aligned(16))) bf16_t lw0[BN * GEMM_BK];
  __shared__ __attribute__((aligned(16))) bf16_t lw1[BN * GEMM_BK];

  const int M = g.m_dev ? min(*g.m_dev, g.M) : g.M;
  int tm, tn, half;
  if (!tile_of_block<SPLIT>(g, M, BM, tm, tn, half)) return;
  const int m0 = tm * BM, n0 = tn * BN;
  if (!SPLIT || half < 0) {
    big_tile<EPI, 4>(g, m0, n0, M, la0, la1, la2, lw0, lw1);
  } else {
    if (n0 + 128 * half >= g.N) return;
    big_tile<EPI, 2>(g, m0, n0 + 128 * half, M, la0, la1, la2, lw0, lw1);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Whether some XCD's tile range leaves a last round that the split tail halves
// (the same rule as tile_of_block<true>, for the host's row count).
static bool split_pays(int total) {
  for (int x = 0; x < N_XCD; ++x) {
    const int cnt = total / N_XCD + (x < total % N_XCD ? 1 : 0), tail = cnt % CUS_PER_XCD;
    if (cnt > CUS_PER_XCD && tail > 0 && 2 * tail <= CUS_PER_XCD) return true;
  }
  return false;
}

template <int EPI>
static hipError_t launch_epi(GemmArgs g, int tile_cfg, hipStream_t stream) {
  const int bt = tile_cfg == GEMM_TILE_256x256 ? 256 : 128;
  g.tiles_n = (g.N + bt - 1) / bt;
  // sized for g.M rows; a device row count below it leaves workgroups idle
  const int total = (g.M + bt - 1) / bt * g.tiles_n;
  const int per_xcd = (total + N_XCD - 1) / N_XCD;
  if (tile_cfg == GEMM_TILE_256x256 && (split_pays(total) || g.rows_vary)) {
    // a split XCD runs at most 16 extra half-tile workgroups
    hipLaunchKernelGGL((gemm_bf16_256_kernel<EPI, true>), dim3(N_XCD * (per_xcd + CUS_PER_XCD / 2)),
                       dim3(BIG_THREADS), 0, stream, g);
  } else if (tile_cfg == GEMM_TILE_256x256) {
    hipLaunchKernelGGL((gemm_bf16_256_kernel<EPI, false>), dim3(N_XCD * per_xcd), dim3(BIG_THREADS), 0, stream, g);
  } else if (g.splits > 1) {
    if constexpr (EPI == EPI_STORE_F32) {
      const int per_xcd_all = (total * g.splits + N_XCD - 1) / N_XCD;
      hipLaunchKernelGGL((gemm_bf16_128_kernel<EPI, true>), dim3(N_XCD * per_xcd_all), dim3(SMALL_THREADS), 0,
                         stream, g);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((gemm_bf16_128_kernel<EPI, false>), dim3(N_XCD * per_xcd), dim3(SMALL_THREADS), 0, stream, g);
  }
  return hipGetLastError();
}

int gemm_pick_tile(int M, int N) {
  // The 256x256 kernel is faster per tile but runs one workgroup per CU: use
  // it when its tiles fill the 256 CUs at least once.
  const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  return big_tiles >= 256 ? GEMM_TILE_256x256 : GEMM_TILE_128x128;
}

// Largest element offset (+1) reachable through a row map over rows [0, M).
static int64_t row_extent(const RowMap& r, int M, int K) {
  if (r.rpg == INT32_MAX) return (int64_t)(M - 1) * r.rstride + r.off + K;
  const int64_t groups = (M - 1) / r.rpg;
  return groups * r.gstride + (int64_t)(r.rpg - 1) * r.rstride + r.off + K;
}

hipError_t gemm_bf16(int epi, const bf16_t* A, RowMap arow, const bf16_t* W, int64_t ldw, int M, int N, int K,
                     const int32_t* m_dev, const EpiParams& ep, int tile_cfg, hipStream_t stream, bool rows_vary) {
  // K in whole slices; N in groups of 4 (the epilogue writes 4 columns per lane).
  if (K % GEMM_BK != 0 || M <= 0 || N <= 0 || N % 4 != 0) return hipErrorInvalidValue;
  if (tile_cfg != GEMM_TILE_256x256 && tile_cfg != GEMM_TILE_128x128) return hipErrorInvalidValue;
  // V columns of the QKV epilogue start on a slab boundary.
  if (epi == EPI_QKV_BF16 && ep.n_split % 128 != 0) return hipErrorInvalidValue;
  // A is addressed through a closed-form row map (no per-row table), and the
  // copies use 32-bit byte offsets.
  if (arow.map) return hipErrorInvalidValue;
  const int64_t a_elems = row_extent(arow, M, K), w_elems = (int64_t)(N - 1) * ldw + K;
  if (a_elems * 2 >= (int64_t)UINT32_MAX || w_elems * 2 >= (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  GemmArgs g{};
  g.A = A; g.arow = arow; g.W = W; g.ldw = ldw; g.M = M; g.N = N; g.K = K; g.m_dev = m_dev; g.epi = ep;
  g.a_bytes = (uint32_t)(a_elems * 2);
  g.w_bytes = (uint32_t)(w_elems * 2);
  g.splits = 1;
  g.rows_vary = rows_vary && m_dev;
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

int gemm_residual_splits(int M, int N, int K) {
  if (gemm_pick_tile(M, N) != GEMM_TILE_128x128) return 1;
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  // two 128x128 workgroups per CU: below 384 tiles most of the 512 slots idle
  if (tiles >= 384) return 1;
  for (int s = 4; s >= 2; s /= 2)
    if (tiles * s <= 1024 && (K / GEMM_BK) % s == 0 && K / s >= 4 * GEMM_BK) return s;
  return 1;
}

hipError_t gemm_bf16_splitk(const bf16_t* A, RowMap arow, const bf16_t* W, int64_t ldw, int M, int N, int K,
                            int splits, const int32_t* m_dev, float* parts, int64_t ldc, int64_t part_stride,
                            hipStream_t stream) {
  if (splits < 2 || K % (GEMM_BK * splits) != 0 || M <= 0 || N <= 0 || N % 4 != 0 || arow.map || !parts)
    return hipErrorInvalidValue;
  const int64_t a_elems = row_extent(arow, M, K), w_elems = (int64_t)(N - 1) * ldw + K;
  if (a_elems * 2 >= (int64_t)UINT32_MAX || w_elems * 2 >= (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  if ((uint64_t)K * 2 * (splits - 1) >= UINT32_MAX) return hipErrorInvalidValue;
  GemmArgs g{};
  g.A = A; g.arow = arow; g.W = W; g.ldw = ldw; g.M = M; g.N = N; g.K = K / splits; g.m_dev = m_dev;
  g.epi.c = parts;
  g.epi.crow = dense_rows(ldc);
  g.a_bytes = (uint32_t)(a_elems * 2);
  g.w_bytes = (uint32_t)(w_elems * 2);
  g.splits = splits;
  g.c_split_stride = part_stride;
  return launch_epi<EPI_STORE_F32>(g, GEMM_TILE_128x128, stream);
}

}  // namespace aenc
