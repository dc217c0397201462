// Bidirectional multi-head attention of the encoder blocks, head_dim 64.
//
// Every position attends to every valid position of its own clip: one pass,
// no causal mask, nothing cached ("Qwen2-Audio-7B-Instruct", (1) AUDIO
// ENCODER: single bidirectional pass; "Voxtral-Mini-3B-2507", (1) AUDIO
// ENCODER: 20 heads and 20 KV heads, head_dim 64). Clips are packed: clip b
// owns rows [start[b], start[b] + len[b]) and masked positions were removed
// beforehand, so the only masking left is the ragged end of each clip, or,
// for chunked attention, each query's key range.
//
// bf16 kernel (flash-style, one pass over the keys with an online softmax):
//   - workgroup = (128-query tile, head, clip), four wave64s with 32 queries each
//     (two wave64s and 64 queries when the 4-wave grid would leave CUs idle);
//   - 64-key tiles of K (row-major) and V (already transposed by the QKV
//     GEMM's epilogue) are staged in LDS, double-buffered through registers;
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so each lane holds 32 scores of
//     a single query (its partner lane l^32 holds the other 32): the row sum
//     needs one cross-lane exchange at the end, the row max one only when the
//     reference maximum moves (below);
//   - P^T in registers is exactly the B operand of O^T = V^T P^T, so P never
//     goes through LDS: K rows are placed in LDS so that each lane's scores
//     cover runs of 8 consecutive keys, and V^T tiles are stored as loaded;
//   - Q arrives pre-scaled by log2(e)/sqrt(64) (the QKV epilogue applies it
//     before rounding), and each tile's score accumulator starts at minus the
//     row's reference maximum, so the MFMAs yield base-2 exponents ready for
//     v_exp_f32; softmax statistics and the output accumulate in fp32;
//   - the running maximum is moved (and the sums rescaled) only when a row's
//     tile maximum exceeds it by more than 2^8 in probability: until then the
//     stale maximum only scales every term of the row by the same factor
//     (at most 256), which the final division by the row sum cancels. With
//     32 queries per wave, an exact running maximum would rescale on most
//     tiles.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace aenc {

constexpr int ATT_BQ = 128;   // queries per workgroup of 4 waves (32 per wave)
constexpr int ATT_BK = 64;
constexpr int ATT_D = 64;

// LDS tiles have 128-byte rows; a 128-bit read is served for 16 lanes per
// cycle from 64 banks (two rows), so chunk c of row r sits at c ^ ((r/2) mod 8)
// and 16 consecutive rows reading the same chunk use 16 distinct bank groups.
__device__ __forceinline__ int att_swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// K rows sit in LDS with bits 2 and 3 of the key index swapped (an involution:
// LDS row r holds key key_row(r)). The score MFMA gives lane half hh the rows
// 8a + 4hh + (0..3) of each 32-row block; through the swap those are keys
// 16(a/2) + 8hh + 4(a%2) + (0..3), so each lane half holds runs of 8
// consecutive keys: exactly the K-index order in which the P V MFMA takes its
// B operand, with V^T's keys in their natural order.
__device__ __forceinline__ int key_row(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// RANGED: query row r (clip-relative index i) sees only the clip's keys
// [key_lo[r], key_hi[r]), non-empty and non-decreasing in i (the chunk rules);
// the workgroup walks the key tiles between its first query's key_lo and its
// last query's key_hi and masks per query.
// NW waves per workgroup (4, or 2 for short batches, whose 4-wave grids leave
// CUs idle): BQ = 32 NW queries per workgroup.
template <bool RANGED, int NW>
__global__ __launch_bounds__(64 * NW) void attention_bf16_kernel(const bf16_t* __restrict__ qk, int64_t ld_qk,
                                                             const bf16_t* __restrict__ vt, int64_t ld_vt,
                                                             const int32_t* __restrict__ starts,
                                                             const int32_t* __restrict__ lens, int d,
                                                             bf16_t* __restrict__ o, int64_t ld_o,
                                                             const int32_t* __restrict__ key_lo,
                                                             const int32_t* __restrict__ key_hi, int n_qb,
                                                             int n_clips, int pair_group) {
  __shared__ __align__(16) bf16_t Ks[2][ATT_BK * ATT_D];   // [key][dim], swizzled 16-byte chunks
  __shared__ __align__(16) bf16_t Vs[2][ATT_D * ATT_BK];   // [dim][key position], swizzled

  // RANGED: the grid is (head, clip, query block) with the query blocks in
  // reverse, so the blocks that see the most keys (the last ones under the
  // chunk-causal rule) are dispatched first and the short ones fill in behind.
  // Otherwise the grid is 1-D: workgroup b runs on XCD b mod 8 (private L2
  // each), and the (clip, head) pairs are dealt to the XCDs in turn, all
  // query blocks of a pair on its XCD (see below).
  int b, h, qb;
  if (RANGED) {
    b = blockIdx.y;
    h = blockIdx.x;
    qb = gridDim.z - 1 - blockIdx.z;
  } else {
    // (clip, head) pairs in runs of pair_group consecutive ones (heads of
    // one clip) dealt round-robin to the XCDs, each XCD taking all query
    // blocks of its pairs: the query blocks that stream one pair's K and V
    // share an L2, and clips of unequal lengths spread over the XCDs
    const int n_pairs = (d / ATT_D) * n_clips;
    const int i = (int)(blockIdx.x / 8);
    const int lp = i / n_qb;
    const int pair = ((lp / pair_group) * 8 + (int)(blockIdx.x % 8)) * pair_group + lp % pair_group;
    if (pair >= n_pairs) return;
    qb = i % n_qb;
    h = pair % (d / ATT_D);
    b = pair / (d / ATT_D);
  }
  const int start = starts[b];
  const int len = lens[b];
  constexpr int BQ = 32 * NW, THREADS = 64 * NW, CH = 512 / THREADS;   // CH: 16-byte chunks per thread and tile
  const int q0 = qb * BQ;
  if (q0 >= len) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fq = lane & 31, hh = lane >> 5;
  const int qi = q0 + wave * 32 + fq;                       // this lane's query (clip-relative)
  // keys this lane's query may see, and the key tiles the workgroup visits
  int k_lo = 0, k_hi = len, kt_first = 0, kt_last = (len - 1) / ATT_BK;
  if (RANGED) {
    k_lo = key_lo[start + min(qi, len - 1)];
    k_hi = key_hi[start + min(qi, len - 1)];
    kt_first = key_lo[start + q0] / ATT_BK;
    kt_last = (key_hi[start + min(q0 + BQ, len) - 1] - 1) / ATT_BK;
  }

  // Q fragments (B operand of S^T = K Q^T): dims 16s + 8hh .. +7. Q arrives
  // multiplied by log2(e)/sqrt(64), so scores are base-2 exponents.
  bf16x8 qf[4];
  {
    const bf16_t* qrow = qk + (int64_t)(start + min(qi, len - 1)) * ld_qk + h * ATT_D + 8 * hh;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *(const bf16x8*)(qrow + 16 * s);
  }

  // Cooperative tile loads: CH 16-byte chunks of K and CH of V^T per thread.
  // Whole tiles come through buffer loads based at the clip's first row: the
  // per-lane offset is fixed and the tile's key offset rides in the scalar
  // offset, so a tile costs no address arithmetic. A tile that runs past the
  // clip clamps its key rows (plain loads) and zeroes the values of keys past
  // the clip (a zero probability times a non-finite value would still poison
  // the sum).
  const bf16_t* kbase = qk + (int64_t)start * ld_qk + d + h * ATT_D;
  const bf16_t* vbase = vt + (int64_t)(h * ATT_D) * ld_vt + start;
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kbase), (short)0,
                                                                       0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vbase), (short)0,
                                                                       0x7fffffff, 0x00020000);
  uint32_t koff[CH], voff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + THREADS * i;
    koff[i] = (uint32_t)(((c >> 3) * ld_qk + (c & 7) * 8) * 2);
    voff[i] = (uint32_t)(((c >> 3) * ld_vt + (c & 7) * 8) * 2);
  }
  u32x4 rk[CH], rv[CH];
  auto gload = [&](int k0, auto ragged) {
    constexpr bool RAGGED = decltype(ragged)::value;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + THREADS * i;
      const int key = c >> 3, ch = c & 7;
      if (RAGGED) {
        rk[i] = *(const u32x4*)(kbase + (int64_t)min(k0 + key, len - 1) * ld_qk + ch * 8);
        u32x4 v = *(const u32x4*)(vbase + (int64_t)key * ld_vt + k0 + ch * 8);
        const int first = k0 + ch * 8;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = v[w];
          if (first + 2 * w >= len) word &= 0xFFFF0000u;
          if (first + 2 * w + 1 >= len) word &= 0x0000FFFFu;
          v[w] = word;
        }
        rv[i] = v;
      } else {
        rk[i] = __builtin_amdgcn_raw_buffer_load_b128(rsk, koff[i], (uint32_t)(k0 * ld_qk * 2), 0);
        rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rsv, voff[i], (uint32_t)(k0 * 2), 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + THREADS * i;
      const int key = c >> 3, ch = c & 7;
      // K row `key` goes to LDS row key_row(key) (bits 2 and 3 of the key
      // swapped; see tile), V^T chunks to their own places
      const int kr = key_row(key);
      *(u32x4*)(&Ks[buf][kr * ATT_D + att_swz(kr, ch) * 8]) = rk[i];
      const int e = c >> 3, kc = c & 7;
      *(u32x4*)(&Vs[buf][e * ATT_BK + att_swz(e, kc) * 8]) = rv[i];
    }
  };

  // Online softmax in base 2. m_run is the row's reference maximum; every
  // tile's score accumulator starts at -m_run (negm), so the MFMAs produce
  // s - m_run directly and p = 2^acc needs no per-score arithmetic. The
  // reference moves (and the sums are rescaled) only when a row's tile maximum
  // exceeds it by more than 2^8 in probability: until then the stale maximum
  // scales every term of the row by the same factor (at most 256), which the
  // final division by the row sum cancels.
  constexpr float slack = 8.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 negm;                                                // -m_run, or 0 before the first key
#pragma unroll
  for (int v = 0; v < 16; ++v) negm[v] = 0.0f;
  f32x16 oacc[2];
#pragma unroll
  for (int es = 0; es < 2; ++es)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[es][v] = 0.0f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // One 64-key tile from LDS buffer `buf`; MASKED: keys past the clip (or, RANGED,
  // outside the query's range) are masked.
  auto tile = [&](int buf, int k0, auto masked, auto first) {
    constexpr bool MASKED = decltype(masked)::value;
    // Without ranges every row sees key 0 in the first tile, so no row can
    // still be waiting for its first key after it.
    constexpr bool MAYBE_FRESH = RANGED || decltype(first)::value;
    // ---- S^T - m_run = K Q^T - m_run for two 32-key sub-tiles ----
    f32x16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int key = 32 * sub + fq;
      s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *(const bf16x8*)(&Ks[buf][key * ATT_D + att_swz(key, hh) * 8]), qf[0], negm, 0, 0, 0);
#pragma unroll
      for (int st = 1; st < 4; ++st) {
        const bf16x8 kf = *(const bf16x8*)(&Ks[buf][key * ATT_D + att_swz(key, 2 * st + hh) * 8]);
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[sub], 0, 0, 0);
      }
    }
    // lane holds keys 32 sub + 16 (v >> 3) + 8 hh + (v & 7) of query qi
    if (MASKED) {
      const int lo = RANGED ? k_lo : 0, hi = RANGED ? k_hi : len;
      // per-key masking only where the tile crosses some query's range edge
      if (!__all(k0 >= lo && k0 + ATT_BK <= hi)) {
        const int first = k0 + 8 * hh;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = first + 32 * sub + 16 * (v >> 3) + (v & 7);
            if (key < lo || key >= hi) s[sub][v] = -INFINITY;
          }
      }
    }
    // this lane's maximum; the row's is the larger of it and its partner's
    // (lane ^ 32), needed only when the reference moves
    float mx = s[0][0];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[sub][v]);
    // Move the reference when some row outgrew it by more than the slack, or
    // sees its first key (a uniform branch, rarely taken after the first tile;
    // some row passes the test exactly when some lane's own maximum does).
    const bool fresh = MAYBE_FRESH && m_run == -INFINITY;
    if (__any(fresh ? mx > -INFINITY : mx > slack)) {
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));                // the row's tile maximum, relative to m_run
      const float shift = fresh ? (mx == -INFINITY ? 0.0f : mx) : fmaxf(mx, 0.0f);
      const float alpha = fresh ? 1.0f : __builtin_amdgcn_exp2f(-shift);
      if (!(fresh && mx == -INFINITY)) m_run = fresh ? mx : m_run + shift;
      l_run *= alpha;
#pragma unroll
      for (int es = 0; es < 2; ++es)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[es][v] *= alpha;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[sub][v] -= shift;
      const float nm = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
      for (int v = 0; v < 16; ++v) negm[v] = nm;
    }

    bf16x8 pb[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[sub][u][j] = (__bf16)__builtin_amdgcn_exp2f(s[sub][8 * u + j]);
    // row sum of the rounded probabilities (the values P V multiplies), two per instruction
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; j += 2)
          l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[sub][u][j], pb[sub][u][j + 1]}, ones, l_run, false);

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int es = 0; es < 2; ++es) {
      const int e = 32 * es + fq;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 vf = *(const bf16x8*)(&Vs[buf][e * ATT_BK + att_swz(e, 4 * sub + 2 * u + hh) * 8]);
          oacc[es] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[sub][u], oacc[es], 0, 0, 0);
        }
    }
  };

  // Tiles kt_first .. kt_last; a tile that runs past the clip is loaded ragged.
  // Without ranges only the last tile can cross the clip's end (masked, peeled).
  if ((kt_first + 1) * ATT_BK > len) gload(kt_first * ATT_BK, std::true_type{});
  else gload(kt_first * ATT_BK, std::false_type{});
  lstore(0);
  __syncthreads();
  // full tile kt from buffer buf, with the next one loaded meanwhile
  auto step = [&](int kt, int buf, auto first) {
    if ((kt + 2) * ATT_BK > len) gload((kt + 1) * ATT_BK, std::true_type{});
    else gload((kt + 1) * ATT_BK, std::false_type{});
    tile(buf, kt * ATT_BK, std::integral_constant<bool, RANGED>{}, first);
    lstore(buf ^ 1);
    __syncthreads();
  };
  if (kt_first < kt_last) step(kt_first, 0, std::true_type{});
  for (int kt = kt_first + 1; kt < kt_last; ++kt) step(kt, (kt - kt_first) & 1, std::false_type{});
  // the last tile (masked); it is also the first when the workgroup visits one tile
  if (kt_last == kt_first) tile(0, kt_last * ATT_BK, std::true_type{}, std::true_type{});
  else tile((kt_last - kt_first) & 1, kt_last * ATT_BK, std::true_type{}, std::false_type{});

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qi < len) {
    bf16_t* orow = o + (int64_t)(start + qi) * ld_o + h * ATT_D;
#pragma unroll
    for (int es = 0; es < 2; ++es)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e0 = 32 * es + 8 * i + 4 * hh;
        u32x2 w;
        w.x = pack_bf16x2(oacc[es][4 * i + 0] * inv, oacc[es][4 * i + 1] * inv);
        w.y = pack_bf16x2(oacc[es][4 * i + 2] * inv, oacc[es][4 * i + 3] * inv);
        *(u32x2*)(orow + e0) = w;
      }
  }
}

hipError_t attention_bf16(const bf16_t* qk, int64_t ld_qk, const bf16_t* vt, int64_t ld_vt, const int32_t* start,
                          const int32_t* len, int n_clips, int max_len, int n_heads, bf16_t* o, int64_t ld_o,
                          const int32_t* key_lo, const int32_t* key_hi, hipStream_t stream) {
  if (n_clips <= 0 || max_len <= 0 || n_heads <= 0 || (!key_lo != !key_hi)) return hipErrorInvalidValue;
  // buffer-load offsets within one clip stay below 2^31 bytes
  if ((int64_t)(max_len + ATT_BK) * ld_qk * 2 >= INT32_MAX || (int64_t)ATT_D * ld_vt * 2 >= INT32_MAX)
    return hipErrorInvalidValue;
  // 4-wave workgroups of 128 queries, or 2-wave ones of 64 when the 4-wave
  // grid would give the 256 CUs fewer than two workgroups each
  const int n_qb4 = (max_len + ATT_BQ - 1) / ATT_BQ;
  const bool two = (int64_t)n_qb4 * n_heads * n_clips < 512;
  const int n_qb = two ? (max_len + ATT_BQ / 2 - 1) / (ATT_BQ / 2) : n_qb4;
  if (key_lo) {
    if (two)
      hipLaunchKernelGGL((attention_bf16_kernel<true, 2>), dim3(n_heads, n_clips, n_qb), dim3(128), 0, stream, qk,
                         ld_qk, vt, ld_vt, start, len, n_heads * ATT_D, o, ld_o, key_lo, key_hi, n_qb, n_clips, 1);
    else
      hipLaunchKernelGGL((attention_bf16_kernel<true, 4>), dim3(n_heads, n_clips, n_qb), dim3(256), 0, stream, qk,
                         ld_qk, vt, ld_vt, start, len, n_heads * ATT_D, o, ld_o, key_lo, key_hi, n_qb, n_clips, 1);
  } else {
    const int64_t n_pairs = (int64_t)n_heads * n_clips;
    // pairs of heads: on the 32-clip variable-length batch (1-30 s clips)
    // runs of 1, 2 or 5 heads per XCD turn are 15% faster than one
    // contiguous range per XCD; on equal-length clips all are alike
    const int G = 2;
    // each XCD runs at most ceil(groups / 8) groups of G pairs
    const int64_t n = (n_pairs + 8LL * G - 1) / (8LL * G) * G * 8 * n_qb;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    const int grid = (int)n;
    if (two)
      hipLaunchKernelGGL((attention_bf16_kernel<false, 2>), dim3(grid), dim3(128), 0, stream, qk, ld_qk, vt, ld_vt,
                         start, len, n_heads * ATT_D, o, ld_o, nullptr, nullptr, n_qb, n_clips, G);
    else
      hipLaunchKernelGGL((attention_bf16_kernel<false, 4>), dim3(grid), dim3(256), 0, stream, qk, ld_qk, vt, ld_vt,
                         start, len, n_heads * ATT_D, o, ld_o, nullptr, nullptr, n_qb, n_clips, G);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per query, 64-key tiles of K and V in LDS, online
// softmax with one rescale per tile.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attention_f32_kernel(const float* __restrict__ qkv, int64_t ld,
                                                           const int32_t* __restrict__ starts,
                                                           const int32_t* __restrict__ lens, int d,
                                                           float* __restrict__ o, int64_t ld_o,
                                                           const int32_t* __restrict__ key_lo,
                                                           const int32_t* __restrict__ key_hi) {
  __shared__ float Ks[ATT_BK][ATT_D + 1];
  __shared__ float Vs[ATT_BK][ATT_D + 1];
  const int b = blockIdx.z, h = blockIdx.y;
  const int start = starts[b];
  const int len = lens[b];
  const int q0 = blockIdx.x * 64;
  if (q0 >= len) return;
  const int t = threadIdx.x;
  const int qi = min(q0 + t, len - 1);
  float q[ATT_D], acc[ATT_D];
  const float* qrow = qkv + (int64_t)(start + qi) * ld + h * ATT_D;
#pragma unroll
  for (int e = 0; e < ATT_D; ++e) { q[e] = qrow[e] * 0.125f; acc[e] = 0.0f; }
  // keys [lo, hi) of this query (all of the clip without ranges)
  const int lo = key_lo ? key_lo[start + qi] : 0;
  const int hi = key_hi ? key_hi[start + qi] : len;
  float m_run = -INFINITY, l_run = 0.0f;
  for (int k0 = 0; k0 < len; k0 += ATT_BK) {
    __syncthreads();
    for (int i = t; i < ATT_BK * ATT_D; i += 64) {
      const int key = i / ATT_D, e = i % ATT_D;
      const int64_t row = (int64_t)(start + min(k0 + key, len - 1)) * ld;
      Ks[key][e] = qkv[row + d + h * ATT_D + e];
      Vs[key][e] = qkv[row + 2 * d + h * ATT_D + e];
    }
    __syncthreads();
    const int nk = min(ATT_BK, len - k0);
    float s[ATT_BK];
    float mx = -INFINITY;
    for (int j = 0; j < ATT_BK; ++j) {
      float v = 0.0f;
#pragma unroll
      for (int e = 0; e < ATT_D; ++e) v = fmaf(q[e], Ks[j][e], v);
      s[j] = (j < nk && k0 + j >= lo && k0 + j < hi) ? v : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) continue;   // no key of this query in the tile yet
    const float alpha = expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < ATT_D; ++e) acc[e] *= alpha;
    for (int j = 0; j < nk; ++j) {
      const float p = expf(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int e = 0; e < ATT_D; ++e) acc[e] = fmaf(p, Vs[j][e], acc[e]);
    }
    m_run = m_new;
  }
  if (q0 + t < len) {
    float* orow = o + (int64_t)(start + q0 + t) * ld_o + h * ATT_D;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int e = 0; e < ATT_D; ++e) orow[e] = acc[e] * inv;
  }
}

hipError_t attention_f32(const float* qkv, int64_t ld, const int32_t* start, const int32_t* len, int n_clips,
                         int max_len, int n_heads, float* o, int64_t ld_o, const int32_t* key_lo,
                         const int32_t* key_hi, hipStream_t stream) {
  if (n_clips <= 0 || max_len <= 0 || n_heads <= 0 || (!key_lo != !key_hi)) return hipErrorInvalidValue;
  dim3 grid((max_len + 63) / 64, n_heads, n_clips);
  hipLaunchKernelGGL(attention_f32_kernel, grid, dim3(64), 0, stream, qkv, ld, start, len, n_heads * ATT_D, o,
                     ld_o, key_lo, key_hi);
  return hipGetLastError();
}

}  // namespace aenc
