// Host runtime behind include/aenc.h: validation, the weight arena, the
// workspace, and the launch sequence of one forward.
//
// One forward (clip-packed rows; M = valid positions of all clips):
//   mask -> packing maps (or the precomputed all-valid maps)
//   mel -> channels-last padded frames
//   conv1  implicit GEMM, + bias, GELU                  -> padded frames (bf16)
//   conv2  implicit GEMM (stride 2), + bias, GELU, + PE -> fp32 residual X [M, d]
//   per block: LN1 -> QKV GEMM (V stored transposed) -> attention
//              -> O GEMM (+= X) -> LN2 -> FC1 GEMM (GELU) -> FC2 GEMM (+= X)
//   final LN (+ pool) -> out, or final LN -> proj1 (GELU) -> proj2 -> out
// Everything is enqueued on the caller's stream; nothing is allocated.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/aenc.h"
#include "common.h"
#include "launch.h"

using namespace aenc;

namespace {

thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

namespace aenc {
void set_kernel_error(const char* msg) { g_last_error = msg; }
}  // namespace aenc

namespace {

enum Kind {
  K_MAPS = 0, K_MEL, K_CONV1, K_CONV2, K_LN, K_QKV, K_ATTN, K_OPROJ, K_FC1, K_FC2, K_FINAL, K_PROJ1, K_PROJ2,
  K_ZERO, K_CLEAR, N_KINDS
};
const char* kKindNames[N_KINDS] = {"mask_maps", "mel_transpose", "conv1", "conv2", "layernorm", "qkv",
                                   "attention", "o_proj", "fc1", "fc2", "final_ln", "proj1", "proj2",
                                   "zero_masked", "scratch_clear"};
constexpr int PROF_RING = 64;

}  // namespace

// One array per GPU the library runs on, held until the process ends. Calls on
// one GPU share it (and race if they overlap); it keeps the last call's
// contents, so each call clears the part it uses first.
static __device__ __align__(256) unsigned char scratch[AENC_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device: the address of `scratch` there (null until looked up)

// The device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept; the array's name in host code is not it.
bool scratch_of_device(int dev, void** ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return false;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return true;
}

}  // namespace

struct aenc_handle {
  aenc_geometry g{};
  int device = 0;
  int T = 0, T8 = 0, C_pad = 0;
  int64_t M_cap = 0, ld_vt = 0;
  size_t esz = 2;  // bytes per activation/weight element

  void* arena = nullptr;
  size_t arena_bytes = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;

  // weights
  void *conv1_w = nullptr, *conv2_w = nullptr;
  float *conv1_b = nullptr, *conv2_b = nullptr;
  struct Layer {
    float *ln1_g, *ln1_b, *qkv_b, *o_b, *ln2_g, *ln2_b, *fc1_b, *fc2_b;
    void *qkv_w, *o_w, *fc1_w, *fc2_w;
  };
  std::vector<Layer> layers;
  float *lnf_g = nullptr, *lnf_b = nullptr;
  void *proj1_w = nullptr, *proj2_w = nullptr;
  float *proj1_b = nullptr, *proj2_b = nullptr;
  float* pe = nullptr;

  // workspace: activations and the packing maps (Ws, defined below)
  struct Ws {
    void *melT, *g1, *a, *qk, *vt, *hmid;
    float* x;
    float* parts;   // [parts][M_cap][d] fp32, or null
    int64_t ld_vt;
    // maps written per forward
    int32_t *row_map, *inv_map, *cu, *lens, *m_valid;
    int32_t *sk_row_map, *sk_inv_map, *sk_m_valid;   // stacked projector rows (stack > 1)
    int32_t *key_lo, *key_hi;                        // chunked attention: per packed row, keys [lo, hi)
    // the same maps for an all-valid batch, built once at create (null: built per forward)
    const int32_t *id_row_map, *id_inv_map, *id_cu, *id_lens, *id_m_valid;
    const int32_t *id_sk_row_map, *id_sk_inv_map, *id_sk_m_valid;
    const int32_t *id_key_lo, *id_key_hi;
  } w{};

  // this device's copy of the static scratch array of aenc_forward_noalloc
  void* scratch = nullptr;

  // profiling
  bool prof = false;
  int launches_per_forward = 0;
  std::vector<hipEvent_t> events;          // PROF_RING x (launches + 1)
  std::vector<int> kinds;                  // PROF_RING x launches
  int ring_head = 0, ring_count = 0;
  int cur_slot = -1, cur_launch = 0;
};

// ---------------------------------------------------------------------------
// Host-only helpers
// ---------------------------------------------------------------------------

extern "C" const char* aenc_last_error(void) { return g_last_error.c_str(); }

extern "C" int aenc_validate(const aenc_geometry* g) {
  if (!g) { set_error("geometry is NULL"); return AENC_E_INVAL; }
  if (g->batch < 1 || g->batch > 4096) { set_error("batch %d outside 1..4096", g->batch); return AENC_E_INVAL; }
  if (g->n_mel < 1 || g->n_mel > 512) { set_error("n_mel %d outside 1..512", g->n_mel); return AENC_E_INVAL; }
  if (g->n_frames < 2 || g->n_frames > 3000 || g->n_frames % 2) {
    set_error("n_frames %d must be even and in 2..3000 (at most 1500 positions)", g->n_frames);
    return AENC_E_INVAL;
  }
  if (g->n_heads < 1 || g->d_model != 64 * g->n_heads) {
    set_error("d_model %d must equal 64 * n_heads (%d): head_dim is 64", g->d_model, g->n_heads);
    return AENC_E_INVAL;
  }
  if (g->d_model % 128 || g->d_model > 2048) {
    set_error("d_model %d must be a multiple of 128 and at most 2048", g->d_model);
    return AENC_E_INVAL;
  }
  if (g->d_ffn < 64 || g->d_ffn % 64 || g->d_ffn > 65536) {
    set_error("d_ffn %d must be a positive multiple of 64", g->d_ffn);
    return AENC_E_INVAL;
  }
  if (g->n_layers < 0 || g->n_layers > 1024) { set_error("n_layers %d outside 0..1024", g->n_layers); return AENC_E_INVAL; }
  if (g->pool_step != 1 && g->pool_step != 2) { set_error("pool_step %d must be 1 or 2", g->pool_step); return AENC_E_INVAL; }
  const bool proj = g->proj_hidden != 0 || g->proj_out != 0;
  if (proj && (g->proj_hidden < 64 || g->proj_out < 64 || g->proj_hidden % 64 || g->proj_out % 64 ||
               g->proj_hidden > 65536 || g->proj_out > 65536)) {
    set_error("projector widths %d, %d must be positive multiples of 64", g->proj_hidden, g->proj_out);
    return AENC_E_INVAL;
  }
  if (g->dtype != AENC_F32 && g->dtype != AENC_BF16) { set_error("dtype %d unknown", g->dtype); return AENC_E_INVAL; }
  if (g->out_dtype != AENC_F32 && g->out_dtype != AENC_BF16) {
    set_error("out_dtype %d unknown", g->out_dtype);
    return AENC_E_INVAL;
  }
  if (!(g->ln_eps > 0.0f) || !std::isfinite(g->ln_eps)) { set_error("ln_eps must be positive and finite"); return AENC_E_INVAL; }
  if (proj && g->pool_step == 2) {
    set_error("pool_step 2 together with a projector is not defined");
    return AENC_E_UNSUPPORTED;
  }
  if (g->stack != 0 && g->stack != 1 && g->stack != 4) {
    set_error("stack %d must be 0, 1 or 4", g->stack);
    return AENC_E_INVAL;
  }
  if (g->stack == 4 && !proj) {
    set_error("stack 4 feeds the projector: set proj_hidden and proj_out");
    return AENC_E_UNSUPPORTED;
  }
  if (g->stack == 4 && g->n_frames / 2 < 4) {
    set_error("stack 4 needs at least 4 positions (n_frames >= 8)");
    return AENC_E_INVAL;
  }
  if (g->attn_chunk < 0 || g->attn_chunk > g->n_frames / 2) {
    set_error("attn_chunk %d outside 0..n_frames/2", g->attn_chunk);
    return AENC_E_INVAL;
  }
  if (g->attn_chunk == 0 ? g->attn_chunk_mode != AENC_CHUNK_NONE
                         : (g->attn_chunk_mode != AENC_CHUNK_CAUSAL && g->attn_chunk_mode != AENC_CHUNK_BLOCK)) {
    set_error("attn_chunk_mode %d: AENC_CHUNK_CAUSAL or AENC_CHUNK_BLOCK with attn_chunk > 0, else AENC_CHUNK_NONE",
              g->attn_chunk_mode);
    return AENC_E_INVAL;
  }
  if (g->dtype == AENC_BF16) {
    // The bf16 GEMMs copy A and W through buffer resources, whose byte offsets
    // are 32-bit: every operand must stay under 4 GiB. Per clip, the largest A
    // operands are the conv stem's padded frames and the FFN (or projector)
    // hidden rows.
    const int64_t lim = (int64_t)UINT32_MAX;
    const int64_t F2 = g->n_frames + 2, T8 = round_up(g->n_frames / 2, 8), d = g->d_model;
    const int64_t mid = std::max<int64_t>(g->d_ffn, g->proj_hidden);
    const int64_t per_clip = 2 * std::max({F2 * round_up(g->n_mel, 64), F2 * d, T8 * mid});
    if ((int64_t)g->batch * per_clip >= lim) {
      set_error("batch %d: a bf16 GEMM operand would span %lld bytes, over the 4 GiB that 32-bit buffer offsets "
                "reach; at most %lld clips of this geometry per forward",
                g->batch, (long long)(g->batch * per_clip), (long long)((lim - 1) / per_clip));
      return AENC_E_INVAL;
    }
    const int64_t proj_in = d * std::max(1, g->stack);
    if (proj && (2 * g->proj_hidden * proj_in >= lim || 2 * (int64_t)g->proj_out * g->proj_hidden >= lim)) {
      set_error("projector weights of %d x %lld and %d x %d bf16 must each stay under 4 GiB", g->proj_hidden,
                (long long)proj_in, g->proj_out, g->proj_hidden);
      return AENC_E_INVAL;
    }
  }
  return AENC_OK;
}

namespace {
// Positions concatenated into one projector input row (0 means 1).
int stack_of(const aenc_geometry* g) { return g->stack > 1 ? g->stack : 1; }
}  // namespace

extern "C" int64_t aenc_param_count(const aenc_geometry* g) {
  if (aenc_validate(g) != AENC_OK) return -1;
  const int64_t d = g->d_model, f = g->d_ffn, m = g->n_mel, L = g->n_layers;
  int64_t n = 3 * m * d + d + 3 * d * d + d;                         // conv stem
  n += L * (4 * d * d + 3 * d + 2 * d * f + f + d + 4 * d);          // blocks (no key bias)
  n += 2 * d;                                                        // final LN
  if (g->proj_hidden)
    n += stack_of(g) * d * g->proj_hidden + g->proj_hidden + (int64_t)g->proj_hidden * g->proj_out + g->proj_out;
  return n;
}

extern "C" int aenc_output_shape(const aenc_geometry* g, int64_t shape[3]) {
  const int st = aenc_validate(g);
  if (st != AENC_OK) return st;
  if (!shape) { set_error("shape is NULL"); return AENC_E_INVAL; }
  shape[0] = g->batch;
  shape[1] = (g->n_frames / 2) / g->pool_step / stack_of(g);
  shape[2] = g->proj_hidden ? g->proj_out : g->d_model;
  return AENC_OK;
}

namespace {

struct Layout {
  int T, T8, C_pad;
  int64_t M_cap, ld_vt;
  size_t esz;
  size_t off_melT, off_g1, off_x, off_a, off_qk, off_vt, off_hmid, off_parts, off_maps, total;
  int parts;   // partial products of the split residual GEMMs (0: not split)
};

Layout workspace_layout(const aenc_geometry* g) {
  Layout L{};
  L.T = g->n_frames / 2;
  L.T8 = (int)round_up(L.T, 8);
  L.C_pad = (int)round_up(g->n_mel, 64);
  L.esz = g->dtype == AENC_BF16 ? 2 : 4;
  L.M_cap = (int64_t)g->batch * L.T8;
  L.ld_vt = round_up(L.M_cap, 64) + 64;
  const int64_t B = g->batch, F = g->n_frames, d = g->d_model;
  const int64_t mid = std::max<int64_t>(g->d_ffn, g->proj_hidden);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += round_up((int64_t)bytes, 256); return o; };
  L.off_melT = take(B * (F + 2) * L.C_pad * L.esz);
  L.off_g1 = take(B * (F + 2) * d * L.esz);
  L.off_x = take(L.M_cap * d * 4);
  L.off_a = take(L.M_cap * d * L.esz);
  // bf16: Q|K rows [M, 2d] and V^T [d, ld_vt]; fp32: Q|K|V rows [M, 3d]
  L.off_qk = take(L.M_cap * (g->dtype == AENC_BF16 ? 2 : 3) * d * L.esz);
  L.off_vt = take(g->dtype == AENC_BF16 ? d * L.ld_vt * 2 : 0);
  L.off_hmid = take(L.M_cap * mid * L.esz);
  // short bf16 batches split the residual products along K; the partials wait
  // here for the next LayerNorm, which adds them to the residual stream
  L.parts = 0;
  if (g->dtype == AENC_BF16 && g->n_layers > 0) {
    const int M_rows = (int)((int64_t)(B - 1) * L.T8 + L.T);
    L.parts = std::max(gemm_residual_splits(M_rows, (int)d, (int)d), gemm_residual_splits(M_rows, (int)d, g->d_ffn));
    if (L.parts < 2) L.parts = 0;
  }
  L.off_parts = take((size_t)L.parts * L.M_cap * d * 4);
  // row_map, inv_map, cu, lens, m_valid twice (per-forward and all-valid),
  // then the stacked-row maps twice when the projector reads stacked rows
  const int k = stack_of(g);
  const size_t maps = (size_t)(B * L.T + L.M_cap + (B + 1) + B + 1) * 4;
  const size_t sk_maps = k > 1 ? (size_t)(B * (L.T / k) + L.M_cap / k + 1) * 4 : 0;
  // chunked attention: key_lo and key_hi per packed row, twice
  const size_t ranges = g->attn_chunk > 0 ? (size_t)2 * L.M_cap * 4 : 0;
  L.off_maps = take(2 * maps + 2 * sk_maps + 2 * ranges + 64);
  L.total = off;
  return L;
}

// Pointers into a workspace laid out by workspace_layout for `batch` clips.
// The all-valid maps are left null; create() builds them in its own workspace.
aenc_handle::Ws carve(const aenc_geometry* g, const Layout& L, int batch, char* base) {
  aenc_handle::Ws w{};
  w.melT = base + L.off_melT;
  w.g1 = base + L.off_g1;
  w.x = (float*)(base + L.off_x);
  w.a = base + L.off_a;
  w.qk = base + L.off_qk;
  w.vt = base + L.off_vt;
  w.hmid = base + L.off_hmid;
  w.parts = L.parts ? (float*)(base + L.off_parts) : nullptr;
  w.ld_vt = L.ld_vt;
  int32_t* maps = (int32_t*)(base + L.off_maps);
  const int64_t BT = (int64_t)batch * L.T;
  w.row_map = maps; maps += BT;
  w.inv_map = maps; maps += L.M_cap;
  w.cu = maps; maps += batch + 1;
  w.lens = maps; maps += batch;
  w.m_valid = maps; maps += 1;
  // room for the all-valid copies (used by create's workspace only)
  maps += BT + L.M_cap + batch + 1 + batch + 1;
  const int k = g->stack > 1 ? g->stack : 1;
  if (k > 1) {
    w.sk_row_map = maps; maps += (int64_t)batch * (L.T / k);
    w.sk_inv_map = maps; maps += L.M_cap / k;
    w.sk_m_valid = maps; maps += 1;
    maps += (int64_t)batch * (L.T / k) + L.M_cap / k + 1;
  }
  if (g->attn_chunk > 0) {
    w.key_lo = maps; maps += L.M_cap;
    w.key_hi = maps; maps += L.M_cap;
  }
  return w;
}

}  // namespace

extern "C" int64_t aenc_workspace_bytes(const aenc_geometry* g) {
  if (aenc_validate(g) != AENC_OK) return -1;
  return (int64_t)workspace_layout(g).total;
}

extern "C" int aenc_profile_kind_count(void) { return N_KINDS; }
extern "C" const char* aenc_profile_kind_name(int kind) {
  return (kind >= 0 && kind < N_KINDS) ? kKindNames[kind] : "";
}

// ---------------------------------------------------------------------------
// create / destroy
// ---------------------------------------------------------------------------

namespace {

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) {                                                                \
      set_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, __LINE__); \
      return false;                                                                        \
    }                                                                                      \
  } while (0)

bool check_weights(const aenc_geometry* g, const aenc_weights* w) {
  if (!w) { set_error("weights is NULL"); return false; }
  if (!w->conv1_w || !w->conv2_w) { set_error("conv weights must not be NULL"); return false; }
  if (g->n_layers > 0 && !w->layers) { set_error("layers array is NULL"); return false; }
  for (int l = 0; l < g->n_layers; ++l) {
    const aenc_layer_weights& L = w->layers[l];
    if (!L.q_w || !L.k_w || !L.v_w || !L.o_w || !L.fc1_w || !L.fc2_w) {
      set_error("layer %d: weight matrices must not be NULL", l);
      return false;
    }
  }
  if (g->proj_hidden && (!w->proj1_w || !w->proj2_w)) { set_error("projector weights must not be NULL"); return false; }
  return true;
}

struct Builder {
  aenc_handle* h;
  char* cursor;
  void* staging;
  size_t staging_bytes;

  void* take(size_t bytes) {
    void* p = cursor;
    cursor += round_up((int64_t)bytes, 256);
    return p;
  }
  bool copy(void* dst, const void* src, size_t bytes) {
    HIP_TRY(hipMemcpy(dst, src, bytes, hipMemcpyDefault));
    return true;
  }
  // vector of n elements in the geometry dtype (or null) -> fp32 in the arena
  bool vec(float* dst, const void* src, int64_t n, float fill) {
    if (src) {
      if (!copy(staging, src, n * h->esz)) return false;
      HIP_TRY(to_f32(staging, h->g.dtype, dst, n, fill, nullptr));
    } else {
      HIP_TRY(to_f32(nullptr, h->g.dtype, dst, n, fill, nullptr));
    }
    HIP_TRY(hipStreamSynchronize(nullptr));
    return true;
  }
  bool conv(void* dst, const void* src, int out, int in, int in_pad) {
    if (!copy(staging, src, (size_t)out * in * 3 * h->esz)) return false;
    HIP_TRY(repack_conv(staging, h->g.dtype, dst, out, in, in_pad, nullptr));
    HIP_TRY(hipStreamSynchronize(nullptr));
    return true;
  }
};

size_t arena_size(const aenc_geometry* g, int C_pad, size_t esz, int T) {
  const int64_t d = g->d_model, f = g->d_ffn, L = g->n_layers;
  int64_t elems = d * 3 * C_pad + d * 3 * d + L * (3 * d * d + d * d + f * d + d * f);
  int64_t floats = 2 * d + L * (2 * d + 3 * d + d + 2 * d + f + d) + 2 * d + (int64_t)T * d;
  if (g->proj_hidden) {
    elems += (int64_t)g->proj_hidden * stack_of(g) * d + (int64_t)g->proj_out * g->proj_hidden;
    floats += g->proj_hidden + g->proj_out;
  }
  // + 256 B alignment slack per tensor
  return (size_t)(elems * esz + floats * 4) + (size_t)(16 + 16 * L) * 256 + 4096;
}

bool build(aenc_handle* h, const aenc_weights* w) {
  const aenc_geometry& g = h->g;
  const int d = g.d_model, f = g.d_ffn;
  const size_t esz = h->esz;

  h->arena_bytes = arena_size(&g, h->C_pad, esz, h->T);
  HIP_TRY(hipMalloc(&h->arena, h->arena_bytes));
  const size_t stage = (size_t)std::max<int64_t>(3LL * d * d, std::max<int64_t>(3LL * d * g.n_mel,
                                                 std::max<int64_t>(f, std::max(g.proj_hidden, g.proj_out)))) * esz;
  Builder B{h, (char*)h->arena, nullptr, stage};
  HIP_TRY(hipMalloc(&B.staging, stage));
  struct Free { void* p; ~Free() { if (p) (void)hipFree(p); } } free_staging{B.staging};

  h->conv1_w = B.take((size_t)d * 3 * h->C_pad * esz);
  h->conv1_b = (float*)B.take(d * 4);
  h->conv2_w = B.take((size_t)d * 3 * d * esz);
  h->conv2_b = (float*)B.take(d * 4);
  if (!B.conv(h->conv1_w, w->conv1_w, d, g.n_mel, h->C_pad) || !B.vec(h->conv1_b, w->conv1_b, d, 0.0f)) return false;
  if (!B.conv(h->conv2_w, w->conv2_w, d, d, d) || !B.vec(h->conv2_b, w->conv2_b, d, 0.0f)) return false;

  h->layers.resize(g.n_layers);
  for (int l = 0; l < g.n_layers; ++l) {
    const aenc_layer_weights& s = w->layers[l];
    aenc_handle::Layer& L = h->layers[l];
    L.ln1_g = (float*)B.take(d * 4); L.ln1_b = (float*)B.take(d * 4);
    L.qkv_w = B.take((size_t)3 * d * d * esz); L.qkv_b = (float*)B.take(3 * d * 4);
    L.o_w = B.take((size_t)d * d * esz); L.o_b = (float*)B.take(d * 4);
    L.ln2_g = (float*)B.take(d * 4); L.ln2_b = (float*)B.take(d * 4);
    L.fc1_w = B.take((size_t)f * d * esz); L.fc1_b = (float*)B.take(f * 4);
    L.fc2_w = B.take((size_t)d * f * esz); L.fc2_b = (float*)B.take(d * 4);
    const size_t mat = (size_t)d * d * esz;
    bool ok = B.vec(L.ln1_g, s.ln1_g, d, 1.0f) && B.vec(L.ln1_b, s.ln1_b, d, 0.0f) &&
              B.copy(L.qkv_w, s.q_w, mat) && B.copy((char*)L.qkv_w + mat, s.k_w, mat) &&
              B.copy((char*)L.qkv_w + 2 * mat, s.v_w, mat) && B.vec(L.qkv_b, s.q_b, d, 0.0f) &&
              B.vec(L.qkv_b + d, nullptr, d, 0.0f) && B.vec(L.qkv_b + 2 * d, s.v_b, d, 0.0f) &&
              B.copy(L.o_w, s.o_w, mat) && B.vec(L.o_b, s.o_b, d, 0.0f) && B.vec(L.ln2_g, s.ln2_g, d, 1.0f) &&
              B.vec(L.ln2_b, s.ln2_b, d, 0.0f) && B.copy(L.fc1_w, s.fc1_w, (size_t)f * d * esz) &&
              B.vec(L.fc1_b, s.fc1_b, f, 0.0f) && B.copy(L.fc2_w, s.fc2_w, (size_t)d * f * esz) &&
              B.vec(L.fc2_b, s.fc2_b, d, 0.0f);
    if (!ok) return false;
  }
  h->lnf_g = (float*)B.take(d * 4);
  h->lnf_b = (float*)B.take(d * 4);
  if (!B.vec(h->lnf_g, w->lnf_g, d, 1.0f) || !B.vec(h->lnf_b, w->lnf_b, d, 0.0f)) return false;
  if (g.proj_hidden) {
    const int ph = g.proj_hidden, po = g.proj_out;
    const size_t p1 = (size_t)ph * stack_of(&g) * d * esz;
    h->proj1_w = B.take(p1); h->proj1_b = (float*)B.take(ph * 4);
    h->proj2_w = B.take((size_t)po * ph * esz); h->proj2_b = (float*)B.take(po * 4);
    if (!B.copy(h->proj1_w, w->proj1_w, p1) || !B.vec(h->proj1_b, w->proj1_b, ph, 0.0f) ||
        !B.copy(h->proj2_w, w->proj2_w, (size_t)po * ph * esz) || !B.vec(h->proj2_b, w->proj2_b, po, 0.0f))
      return false;
  }
  h->pe = (float*)B.take((size_t)h->T * d * 4);
  HIP_TRY(position_table(h->pe, h->T, d, nullptr));
  if ((size_t)(B.cursor - (char*)h->arena) > h->arena_bytes) {
    set_error("internal: arena overflow");
    return false;
  }

  // workspace
  const Layout Ly = workspace_layout(&g);
  h->ws_bytes = Ly.total;
  HIP_TRY(hipMalloc(&h->ws, h->ws_bytes));
  HIP_TRY(hipMemset(h->ws, 0, h->ws_bytes));
  char* ws = (char*)h->ws;
  h->w = carve(&g, Ly, g.batch, ws);
  aenc_handle::Ws& W = h->w;
  // the all-valid maps sit right after the per-forward ones (see carve)
  int32_t* id = (int32_t*)(ws + Ly.off_maps);
  const int64_t BT = (int64_t)g.batch * h->T;
  id += BT + h->M_cap + g.batch + 1 + g.batch + 1;
  int32_t* id_row_map = id; id += BT;
  int32_t* id_inv_map = id; id += h->M_cap;
  int32_t* id_cu = id; id += g.batch + 1;
  int32_t* id_lens = id; id += g.batch;
  int32_t* id_m_valid = id; id += 1;
  HIP_TRY(build_row_maps(nullptr, g.batch, h->T, id_row_map, id_inv_map, id_cu, id_lens, id_m_valid, nullptr));
  W.id_row_map = id_row_map; W.id_inv_map = id_inv_map; W.id_cu = id_cu; W.id_lens = id_lens;
  W.id_m_valid = id_m_valid;
  const int k = stack_of(&g);
  if (k > 1) {
    int32_t* sk = W.sk_m_valid + 1;
    int32_t* id_sk_row_map = sk; sk += (int64_t)g.batch * (h->T / k);
    int32_t* id_sk_inv_map = sk; sk += h->M_cap / k;
    int32_t* id_sk_m_valid = sk;
    HIP_TRY(build_stack_maps(id_cu, id_lens, g.batch, h->T, k, id_sk_row_map, id_sk_inv_map, id_sk_m_valid,
                             nullptr));
    W.id_sk_row_map = id_sk_row_map; W.id_sk_inv_map = id_sk_inv_map; W.id_sk_m_valid = id_sk_m_valid;
  }
  if (g.attn_chunk > 0) {
    int32_t* r = W.key_hi + h->M_cap;
    int32_t* id_key_lo = r; r += h->M_cap;
    int32_t* id_key_hi = r;
    HIP_TRY(build_chunk_ranges(nullptr, g.batch, h->T, g.attn_chunk, g.attn_chunk_mode, id_row_map, id_cu,
                               id_key_lo, id_key_hi, nullptr));
    W.id_key_lo = id_key_lo; W.id_key_hi = id_key_hi;
  }
  HIP_TRY(hipDeviceSynchronize());
  return true;
}

void release(aenc_handle* h) {
  if (!h) return;
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.clear();
  if (h->ws) (void)hipFree(h->ws);
  if (h->arena) (void)hipFree(h->arena);
  h->ws = h->arena = nullptr;
}

}  // namespace

extern "C" aenc_handle* aenc_create(const aenc_geometry* g, const aenc_weights* w) {
  g_last_error.clear();
  if (aenc_validate(g) != AENC_OK) return nullptr;
  if (!check_weights(g, w)) return nullptr;

  int n_dev = 0;
  hipError_t e = hipGetDeviceCount(&n_dev);
  if (e != hipSuccess || n_dev < 1) {
    set_error("no HIP device available (%s)", e != hipSuccess ? hipGetErrorString(e) : "0 devices");
    return nullptr;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { set_error("hipGetDevice failed"); return nullptr; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) { set_error("hipGetDeviceProperties failed"); return nullptr; }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_error("device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    return nullptr;
  }

  void* scratch_ptr = nullptr;
  if (!scratch_of_device(dev, &scratch_ptr)) return nullptr;

  aenc_handle* h = new aenc_handle();
  h->g = *g;
  h->device = dev;
  h->scratch = scratch_ptr;
  const Layout Ly = workspace_layout(g);
  h->T = Ly.T; h->T8 = Ly.T8; h->C_pad = Ly.C_pad; h->M_cap = Ly.M_cap; h->ld_vt = Ly.ld_vt; h->esz = Ly.esz;
  h->launches_per_forward = 7 * g->n_layers + 11;
  if (!build(h, w)) {
    std::string msg = g_last_error;
    release(h);
    delete h;
    g_last_error = msg;
    return nullptr;
  }
  return h;
}

extern "C" void aenc_destroy(aenc_handle* h) {
  if (!h) return;
  (void)hipSetDevice(h->device);
  (void)hipDeviceSynchronize();
  release(h);
  delete h;
}

// ---------------------------------------------------------------------------
// profiling
// ---------------------------------------------------------------------------

extern "C" int aenc_profile_enable(aenc_handle* h, int on) {
  if (!h) { set_error("handle is NULL"); return AENC_E_INVAL; }
  if (on && h->events.empty()) {
    const int per = h->launches_per_forward + 1;
    h->events.resize((size_t)PROF_RING * per);
    h->kinds.assign((size_t)PROF_RING * h->launches_per_forward, -1);
    for (auto& ev : h->events) {
      if (hipEventCreate(&ev) != hipSuccess) { set_error("hipEventCreate failed"); return AENC_E_HIP; }
    }
  }
  h->prof = on != 0;
  h->ring_head = h->ring_count = 0;
  return AENC_OK;
}

extern "C" int aenc_profile_read(aenc_handle* h, double* ms, int64_t* calls, int n_kinds) {
  if (!h || !ms || !calls) { set_error("NULL argument"); return AENC_E_INVAL; }
  const int per = h->launches_per_forward + 1;
  const int n = h->ring_count;
  const int first = (h->ring_head - n + PROF_RING) % PROF_RING;
  for (int i = 0; i < n; ++i) {
    const int slot = (first + i) % PROF_RING;
    hipEvent_t* ev = &h->events[(size_t)slot * per];
    const int* kd = &h->kinds[(size_t)slot * h->launches_per_forward];
    for (int k = 0; k < h->launches_per_forward; ++k) {
      if (kd[k] < 0) break;
      if (hipEventSynchronize(ev[k + 1]) != hipSuccess) { set_error("hipEventSynchronize failed"); return AENC_E_HIP; }
      float t = 0.0f;
      if (hipEventElapsedTime(&t, ev[k], ev[k + 1]) != hipSuccess) { set_error("hipEventElapsedTime failed"); return AENC_E_HIP; }
      if (kd[k] < n_kinds) {
        ms[kd[k]] += t;
        calls[kd[k]] += 1;
      }
    }
  }
  h->ring_count = 0;
  return n;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

namespace {

struct Enq {
  aenc_handle* h;
  hipStream_t s;
  int slot;
  int n;

  bool begin() {
    if (!h->prof) return true;
    slot = h->ring_head;
    h->ring_head = (h->ring_head + 1) % PROF_RING;
    h->ring_count = std::min(h->ring_count + 1, PROF_RING);
    n = 0;
    int* kd = &h->kinds[(size_t)slot * h->launches_per_forward];
    std::fill(kd, kd + h->launches_per_forward, -1);
    return hipEventRecord(h->events[(size_t)slot * (h->launches_per_forward + 1)], s) == hipSuccess;
  }
  bool done(int kind, hipError_t e, const char* what) {
    if (e != hipSuccess) {
      set_error("%s launch failed: %s", what, hipGetErrorString(e));
      return false;
    }
    if (h->prof && n < h->launches_per_forward) {
      const size_t per = h->launches_per_forward + 1;
      h->kinds[(size_t)slot * h->launches_per_forward + n] = kind;
      ++n;
      if (hipEventRecord(h->events[slot * per + n], s) != hipSuccess) {
        set_error("hipEventRecord failed");
        return false;
      }
    }
    return true;
  }
};

int pick_tile(int M, int N) { return gemm_pick_tile(M, N); }

}  // namespace

extern "C" int aenc_handle_geometry(const aenc_handle* h, aenc_geometry* g) {
  if (!h || !g) { set_error("handle and geometry must not be NULL"); return AENC_E_INVAL; }
  *g = h->g;
  return AENC_OK;
}

namespace {

// One forward of B clips (B <= the geometry's batch) with workspace w on stream s.
int forward_impl(aenc_handle* h, const aenc_handle::Ws& w, int B, const void* mel, const uint8_t* mask, void* out,
                 hipStream_t s, const void* clear, size_t clear_bytes) {
  const aenc_geometry& g = h->g;
  const int T = h->T, F = g.n_frames, d = g.d_model, f = g.d_ffn, C = g.n_mel;
  const int64_t T8 = h->T8;
  const bool bf = g.dtype == AENC_BF16;
  Enq q{h, s, 0, 0};
  if (!q.begin()) { set_error("hipEventRecord failed"); return AENC_E_HIP; }
  if (clear && !q.done(K_CLEAR, fill_zero((void*)clear, (int64_t)clear_bytes, s), "scratch clear"))
    return AENC_E_HIP;

  // packing maps: the all-valid ones built at create, or built now (a mask,
  // or a workspace without them)
  const bool build = mask || !w.id_row_map;
  const int32_t *row_map = w.id_row_map, *inv_map = w.id_inv_map, *cu = w.id_cu, *lens = w.id_lens,
                *mv = w.id_m_valid;
  const int k = stack_of(&g);
  const int32_t *sk_row_map = w.id_sk_row_map, *sk_inv_map = w.id_sk_inv_map, *sk_mv = w.id_sk_m_valid;
  const int32_t *key_lo = w.id_key_lo, *key_hi = w.id_key_hi;
  if (build) {
    if (!q.done(K_MAPS, build_row_maps(mask, B, T, w.row_map, w.inv_map, w.cu, w.lens, w.m_valid, s), "mask maps"))
      return AENC_E_HIP;
    row_map = w.row_map; inv_map = w.inv_map; cu = w.cu; lens = w.lens; mv = w.m_valid;
    if (k > 1) {
      if (!q.done(K_MAPS, build_stack_maps(cu, lens, B, T, k, w.sk_row_map, w.sk_inv_map, w.sk_m_valid, s),
                  "stack maps"))
        return AENC_E_HIP;
      sk_row_map = w.sk_row_map; sk_inv_map = w.sk_inv_map; sk_mv = w.sk_m_valid;
    }
    if (g.attn_chunk > 0) {
      if (!q.done(K_MAPS, build_chunk_ranges(mask, B, T, g.attn_chunk, g.attn_chunk_mode, row_map, cu, w.key_lo,
                                             w.key_hi, s),
                  "chunk ranges"))
        return AENC_E_HIP;
      key_lo = w.key_lo; key_hi = w.key_hi;
    }
  }
  // Rows of the packed layout the GEMMs must cover at most (all clips full);
  // under a mask the valid rows (on the device) may be far fewer
  const int M_rows = (int)((int64_t)(B - 1) * T8 + T);
  const bool vary = mask != nullptr;
  // Without a mask every one of those rows exists: the kernels then take
  // M_rows as given instead of first reading the row count from the device.
  const int32_t* const mvr = vary ? mv : nullptr;

  if (!q.done(K_MEL, mel_transpose(mel, g.dtype, w.melT, B, C, h->C_pad, F, w.g1, g.dtype, d, s), "mel transpose"))
    return AENC_E_HIP;

  // conv1: rows (b, f) read padded frames f, f+1, f+2 (= f-1, f, f+1), K = 3 C_pad
  EpiParams e1{};
  e1.bias = h->conv1_b;
  e1.c = w.g1;
  e1.crow = RowMap{F, (int64_t)(F + 2) * d, d, d, nullptr};
  const RowMap a1{F, (int64_t)(F + 2) * h->C_pad, h->C_pad, 0, nullptr};
  hipError_t e;
  if (bf)
    e = gemm_bf16(EPI_GELU_BF16, (const bf16_t*)w.melT, a1, (const bf16_t*)h->conv1_w, 3 * h->C_pad, B * F, d,
                  3 * h->C_pad, nullptr, e1, pick_tile(B * F, d), s);
  else
    e = gemm_f32(EPI_GELU_F32, (const float*)w.melT, a1, (const float*)h->conv1_w, 3 * h->C_pad, B * F, d,
                 3 * h->C_pad, nullptr, e1, s);
  if (!q.done(K_CONV1, e, "conv1")) return AENC_E_HIP;

  // conv2: rows (b, t) read conv1 frames 2t-1, 2t, 2t+1 (padded rows 2t .. 2t+2), K = 3 d
  EpiParams e2{};
  e2.bias = h->conv2_b;
  e2.c = w.x;
  e2.crow = RowMap{INT32_MAX, 0, d, 0, row_map};
  e2.pe = h->pe;
  e2.pe_period = T;
  e2.pe_ld = d;
  const RowMap a2{T, (int64_t)(F + 2) * d, 2 * d, 0, nullptr};
  if (bf)
    e = gemm_bf16(EPI_GELU_PE_F32, (const bf16_t*)w.g1, a2, (const bf16_t*)h->conv2_w, 3 * d, B * T, d, 3 * d,
                  nullptr, e2, pick_tile(B * T, d), s);
  else
    e = gemm_f32(EPI_GELU_PE_F32, (const float*)w.g1, a2, (const float*)h->conv2_w, 3 * d, B * T, d, 3 * d, nullptr,
                 e2, s);
  if (!q.done(K_CONV2, e, "conv2")) return AENC_E_HIP;

  const RowMap dense_d = dense_rows(d);
  // Short batches split the residual products (O-proj, FC2) along K; the next
  // LayerNorm adds the partials and the bias to the residual stream.
  const int split_o = (bf && w.parts) ? gemm_residual_splits(M_rows, d, d) : 1;
  const int split_f = (bf && w.parts) ? gemm_residual_splits(M_rows, d, f) : 1;
  const int64_t part_stride = (int64_t)B * T8 * d;
  ResidualParts pending{};   // partials the next LayerNorm folds in
  for (int l = 0; l < g.n_layers; ++l) {
    const aenc_handle::Layer& L = h->layers[l];
    if (!q.done(K_LN, layernorm(w.x, L.ln1_g, L.ln1_b, w.a, g.dtype, M_rows, mvr, d, g.ln_eps, s, pending), "ln1"))
      return AENC_E_HIP;
    pending = ResidualParts{};
    EpiParams eq{};
    eq.bias = L.qkv_b;
    eq.c = w.qk;
    if (bf) {
      eq.crow = dense_rows(2 * d);
      eq.n_split = 2 * d;
      eq.vt = (bf16_t*)w.vt;
      eq.ld_vt = w.ld_vt;
      eq.q_cols = d;                 // the attention kernel takes Q in base-2 score units
      eq.q_scale = ATT_Q_SCALE;
      e = gemm_bf16(EPI_QKV_BF16, (const bf16_t*)w.a, dense_d, (const bf16_t*)L.qkv_w, d, M_rows, 3 * d, d, mvr, eq,
                    pick_tile(M_rows, 3 * d), s, vary);
    } else {
      eq.crow = dense_rows(3 * d);
      e = gemm_f32(EPI_STORE_F32, (const float*)w.a, dense_d, (const float*)L.qkv_w, d, M_rows, 3 * d, d, mvr, eq, s);
    }
    if (!q.done(K_QKV, e, "qkv")) return AENC_E_HIP;

    if (bf)
      e = attention_bf16((const bf16_t*)w.qk, 2 * d, (const bf16_t*)w.vt, w.ld_vt, cu, lens, B, T, g.n_heads,
                         (bf16_t*)w.a, d, key_lo, key_hi, s);
    else
      e = attention_f32((const float*)w.qk, 3 * d, cu, lens, B, T, g.n_heads, (float*)w.a, d, key_lo, key_hi, s);
    if (!q.done(K_ATTN, e, "attention")) return AENC_E_HIP;

    if (split_o > 1) {
      e = gemm_bf16_splitk((const bf16_t*)w.a, dense_d, (const bf16_t*)L.o_w, d, M_rows, d, d, split_o, mvr, w.parts,
                           d, part_stride, s);
      pending = ResidualParts{w.parts, split_o, part_stride, L.o_b};
    } else {
      EpiParams eo{};
      eo.bias = L.o_b;
      eo.c = w.x;
      eo.crow = dense_d;
      e = bf ? gemm_bf16(EPI_RESID_F32, (const bf16_t*)w.a, dense_d, (const bf16_t*)L.o_w, d, M_rows, d, d, mvr, eo,
                         pick_tile(M_rows, d), s, vary)
             : gemm_f32(EPI_RESID_F32, (const float*)w.a, dense_d, (const float*)L.o_w, d, M_rows, d, d, mvr, eo, s);
    }
    if (!q.done(K_OPROJ, e, "o_proj")) return AENC_E_HIP;

    if (!q.done(K_LN, layernorm(w.x, L.ln2_g, L.ln2_b, w.a, g.dtype, M_rows, mvr, d, g.ln_eps, s, pending), "ln2"))
      return AENC_E_HIP;
    pending = ResidualParts{};

    EpiParams ef1{};
    ef1.bias = L.fc1_b;
    ef1.c = w.hmid;
    ef1.crow = dense_rows(f);
    e = bf ? gemm_bf16(EPI_GELU_BF16, (const bf16_t*)w.a, dense_d, (const bf16_t*)L.fc1_w, d, M_rows, f, d, mvr, ef1,
                       pick_tile(M_rows, f), s, vary)
           : gemm_f32(EPI_GELU_F32, (const float*)w.a, dense_d, (const float*)L.fc1_w, d, M_rows, f, d, mvr, ef1, s);
    if (!q.done(K_FC1, e, "fc1")) return AENC_E_HIP;

    if (split_f > 1) {
      e = gemm_bf16_splitk((const bf16_t*)w.hmid, dense_rows(f), (const bf16_t*)L.fc2_w, f, M_rows, d, f, split_f,
                           mvr, w.parts, d, part_stride, s);
      pending = ResidualParts{w.parts, split_f, part_stride, L.fc2_b};
    } else {
      EpiParams ef2{};
      ef2.bias = L.fc2_b;
      ef2.c = w.x;
      ef2.crow = dense_d;
      e = bf ? gemm_bf16(EPI_RESID_F32, (const bf16_t*)w.hmid, dense_rows(f), (const bf16_t*)L.fc2_w, f, M_rows, d,
                         f, mvr, ef2, pick_tile(M_rows, d), s, vary)
             : gemm_f32(EPI_RESID_F32, (const float*)w.hmid, dense_rows(f), (const float*)L.fc2_w, f, M_rows, d, f,
                        mvr, ef2, s);
    }
    if (!q.done(K_FC2, e, "fc2")) return AENC_E_HIP;
  }

  if (!g.proj_hidden) {
    if (!q.done(K_FINAL, final_ln_out(w.x, row_map, h->lnf_g, h->lnf_b, out, g.out_dtype, B, T, g.pool_step, d,
                                      g.ln_eps, s, pending), "final ln"))
      return AENC_E_HIP;
    return AENC_OK;
  }

  const int ph = g.proj_hidden, po = g.proj_out;
  if (!q.done(K_FINAL, layernorm(w.x, h->lnf_g, h->lnf_b, w.a, g.dtype, M_rows, mvr, d, g.ln_eps, s, pending),
              "final ln"))
    return AENC_E_HIP;
  // Projector rows: the packed LN rows themselves, or (stack k) runs of k
  // packed rows read as one k*d-wide row. Clip starts are multiples of 8, so
  // a run never straddles two clips; stacked row r holds packed rows
  // k r .. k r + k - 1, all inside the workspace (M_cap is a multiple of 8).
  const int pin = k * d;
  const int Mp = k > 1 ? (M_rows + k - 1) / k : M_rows;
  const int32_t* mvp = k > 1 ? sk_mv : mv;
  EpiParams ep1{};
  ep1.bias = h->proj1_b;
  ep1.c = w.hmid;
  ep1.crow = dense_rows(ph);
  e = bf ? gemm_bf16(EPI_GELU_BF16, (const bf16_t*)w.a, dense_rows(pin), (const bf16_t*)h->proj1_w, pin, Mp, ph,
                     pin, mvp, ep1, pick_tile(Mp, ph), s)
         : gemm_f32(EPI_GELU_F32, (const float*)w.a, dense_rows(pin), (const float*)h->proj1_w, pin, Mp, ph, pin, mvp,
                    ep1, s);
  if (!q.done(K_PROJ1, e, "proj1")) return AENC_E_HIP;

  EpiParams ep2{};
  ep2.bias = h->proj2_b;
  ep2.c = out;
  // packed (or stacked) row -> output row b * T_out + j, or -1 (not written)
  ep2.crow = RowMap{INT32_MAX, 0, po, 0, k > 1 ? sk_inv_map : inv_map};
  const int epi2 = g.out_dtype == AENC_BF16 ? EPI_STORE_BF16 : EPI_STORE_F32;
  e = bf ? gemm_bf16(epi2, (const bf16_t*)w.hmid, dense_rows(ph), (const bf16_t*)h->proj2_w, ph, Mp, po, ph, mvp,
                     ep2, pick_tile(Mp, po), s)
         : gemm_f32(epi2, (const float*)w.hmid, dense_rows(ph), (const float*)h->proj2_w, ph, Mp, po, ph, mvp, ep2, s);
  if (!q.done(K_PROJ2, e, "proj2")) return AENC_E_HIP;
  if (mask) {
    const int32_t* zmap = k > 1 ? sk_row_map : row_map;
    if (!q.done(K_ZERO, zero_masked_rows(zmap, out, g.out_dtype, B * (T / k), po, s), "zero masked rows"))
      return AENC_E_HIP;
  }
  return AENC_OK;
}

}  // namespace

extern "C" int aenc_forward(aenc_handle* h, const void* mel, const uint8_t* mask, void* out, void* stream) {
  if (!h) { set_error("handle is NULL"); return AENC_E_INVAL; }
  if (!mel || !out) { set_error("mel and out must not be NULL"); return AENC_E_INVAL; }
  if (((uintptr_t)mel | (uintptr_t)out) & 15) { set_error("mel and out must be 16-byte aligned"); return AENC_E_INVAL; }
  return forward_impl(h, h->w, h->g.batch, mel, mask, out, (hipStream_t)stream, nullptr, 0);
}

// ---------------------------------------------------------------------------
// forward without allocation: the workspace is a static device array
// ---------------------------------------------------------------------------

extern "C" int64_t aenc_noalloc_scratch_bytes(const aenc_geometry* g, int n_clips) {
  if (aenc_validate(g) != AENC_OK) return -1;
  if (n_clips < 1 || n_clips > g->batch) { set_error("n_clips %d outside 1..batch (%d)", n_clips, g->batch); return -1; }
  aenc_geometry gb = *g;
  gb.batch = n_clips;
  return (int64_t)workspace_layout(&gb).total;
}

extern "C" int aenc_forward_noalloc(aenc_handle* h, int n_clips, const void* mel, const uint8_t* mask, void* out,
                                    void* stream) {
  if (!h) { set_error("handle is NULL"); return AENC_E_INVAL; }
  if (!mel || !out) { set_error("mel and out must not be NULL"); return AENC_E_INVAL; }
  if (((uintptr_t)mel | (uintptr_t)out) & 15) { set_error("mel and out must be 16-byte aligned"); return AENC_E_INVAL; }
  if (n_clips < 1 || n_clips > h->g.batch) {
    set_error("n_clips %d outside 1..%d (the handle's batch)", n_clips, h->g.batch);
    return AENC_E_INVAL;
  }
  if (!h->scratch) { set_error("no scratch array on this handle's device"); return AENC_E_DEVICE; }
  aenc_geometry gb = h->g;
  gb.batch = n_clips;
  const Layout Ly = workspace_layout(&gb);
  if (Ly.total > (size_t)AENC_NOALLOC_SCRATCH_BYTES) {
    set_error("%d clip(s) of this geometry need %zu bytes of workspace, over the %lld-byte static scratch of "
              "aenc_forward_noalloc; pass fewer clips",
              n_clips, Ly.total, (long long)AENC_NOALLOC_SCRATCH_BYTES);
    return AENC_E_INVAL;
  }
  const aenc_handle::Ws w = carve(&gb, Ly, n_clips, (char*)h->scratch);
  return forward_impl(h, w, n_clips, mel, mask, out, (hipStream_t)stream, h->scratch, Ly.total);
}
