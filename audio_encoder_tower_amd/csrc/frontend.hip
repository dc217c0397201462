// Log-mel front end: 16 kHz audio [B, n_samples] -> features [B, n_mel, n_samples / 160],
// the input of the encoder tower.
//
// The pages fix the extractor's geometry (a Whisper feature extractor: 16 kHz,
// 480,000 samples per 30 s chunk, n_fft 400, hop 160, 128 features, 3000
// frames: "Voxtral-Mini-3B-2507", Preprocessor). Its steps follow the Whisper
// extractor's recipe: centred frames (reflect padding by n_fft/2), periodic
// Hann window, power spectrum of bins 0..200 with the last centred frame
// dropped, Slaney-scale triangular mel filters of unit area, log10 floored
// at 1e-10 and then at the clip maximum minus 8, and (x + 4) / 4.
//
// On the device:
//   1. reflect padding of each clip into a workspace row of n_samples + 400;
//   2. the windowed DFT and the power spectrum in one kernel: a GEMM in fp64
//      on the vector ALUs whose A rows are the overlapping frames (read
//      straight from the padded clip, fp32 samples widened to fp64) and whose
//      B rows are w[n] cos(2 pi k n / 400) and w[n] sin(...) interleaved
//      (bin k in columns 2k and 2k + 1), so one thread holds the real and
//      imaginary parts of its bins and writes |X|^2 (rounded to fp32) into
//      rows of 224 (bins past 200 zero). fp64 sums keep spectral valleys next
//      to loud bins exact: in fp32 a bin 80 dB under its frame's energy loses
//      about 1e-3 of its power to cancellation;
//   3. the mel filters as an fp32 GEMM (K = 224; sums of non-negative terms,
//      accurate to a few fp32 ulps);
//   4. log10 with the floor, a per-clip maximum, then the 80 dB floor, the
//      affine map and a transpose to [B, n_mel, frames] through LDS tiles.
// The DFT matrix (fp64) and the filters are built once, in double precision,
// at create time.
#include <cmath>
#include <cstring>
#include <vector>

#include "aenc.h"
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace aenc {
void set_kernel_error(const char* msg);
}

namespace {

using namespace aenc;

constexpr int FE_NFFT = 400;
constexpr int FE_HOP = 160;
constexpr int FE_BINS = FE_NFFT / 2 + 1;   // 201
constexpr int FE_PK = 224;                 // bins in a power row: 201, zero padded to 7 tiles of 32
constexpr int FE_DFT_N = 2 * FE_PK;        // DFT matrix rows: cos and sin of each (padded) bin, interleaved

__global__ void reflect_pad_kernel(const float* __restrict__ x, float* __restrict__ xp, int n, int B) {
  const int padded = n + FE_NFFT;
  const int64_t total = (int64_t)B * padded;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(i / padded);
    int j = (int)(i - (int64_t)b * padded) - FE_NFFT / 2;   // position in the unpadded clip
    if (j < 0) j = -j;                                        // reflect (the edge sample is not repeated)
    if (j >= n) j = 2 * (n - 1) - j;
    xp[i] = x[(int64_t)b * n + j];
  }
}

// Power spectrum of the frames: P[r, k] = (sum_n x_r[n] C[2k, n])^2 + (sum_n x_r[n] C[2k+1, n])^2
// in fp64, stored as fp32. Frame r = b F + f reads padded samples [b n_pad + 160 f, + 400).
// A workgroup takes 128 frames x 64 DFT columns (32 bins); thread (ty, tx) holds
// frames 8 ty .. 8 ty + 7 and columns 4 tx .. 4 tx + 3 (bins 2 tx and 2 tx + 1 of the tile).
// K advances 16 samples at a time through LDS, k-major.
constexpr int DP_BM = 128, DP_BN = 64, DP_BK = 16;

__global__ __launch_bounds__(256) void dft_power_kernel(const float* __restrict__ xp, int n_pad, int F, int rows,
                                                        const double* __restrict__ dft, float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) double As[DP_BK][DP_BM + 2];
  __shared__ __attribute__((aligned(16))) double Bs[DP_BK][DP_BN + 2];
  const int m0 = blockIdx.y * DP_BM, n0 = blockIdx.x * DP_BN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  // A loader: frame m0 + (tid >> 1), samples 8 (tid & 1) .. +7 of the slice
  const int ar = tid >> 1, ak = (tid & 1) * 8;
  const int r_ld = min(m0 + ar, rows - 1);
  const int b_ld = r_ld / F;
  const float* a_src = xp + (int64_t)b_ld * n_pad + (int64_t)FE_HOP * (r_ld - b_ld * F) + ak;
  // B loader: DFT row n0 + (tid >> 2), samples 4 (tid & 3) .. +3 of the slice
  const int br = tid >> 2, bk = (tid & 3) * 4;
  const double* b_src = dft + (int64_t)(n0 + br) * FE_NFFT + bk;

  double acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < FE_NFFT; k0 += DP_BK) {
    const float4 a0 = *(const float4*)(a_src + k0);
    const float4 a1 = *(const float4*)(a_src + k0 + 4);
    const double2 b0 = *(const double2*)(b_src + k0);
    const double2 b1 = *(const double2*)(b_src + k0 + 2);
    As[ak + 0][ar] = a0.x; As[ak + 1][ar] = a0.y; As[ak + 2][ar] = a0.z; As[ak + 3][ar] = a0.w;
    As[ak + 4][ar] = a1.x; As[ak + 5][ar] = a1.y; As[ak + 6][ar] = a1.z; As[ak + 7][ar] = a1.w;
    Bs[bk + 0][br] = b0.x; Bs[bk + 1][br] = b0.y; Bs[bk + 2][br] = b1.x; Bs[bk + 3][br] = b1.y;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < DP_BK; ++k) {
      double av[8], bv[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const double2 t = *(const double2*)&As[k][ty * 8 + i];
        av[i] = t.x;
        av[i + 1] = t.y;
      }
      const double2 u0 = *(const double2*)&Bs[k][tx * 4];
      const double2 u1 = *(const double2*)&Bs[k][tx * 4 + 2];
      bv[0] = u0.x; bv[1] = u0.y; bv[2] = u1.x; bv[3] = u1.y;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int bin = (n0 >> 1) + 2 * tx;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = m0 + ty * 8 + i;
    if (r >= rows) break;
    float2 p;
    p.x = (float)fma(acc[i][0], acc[i][0], acc[i][1] * acc[i][1]);
    p.y = (float)fma(acc[i][2], acc[i][2], acc[i][3] * acc[i][3]);
    *(float2*)(P + (int64_t)r * FE_PK + bin) = p;
  }
}

// log10(max(mel, 1e-10)) in place, and the maximum of each clip (rows [b F, (b+1) F)).
__global__ __launch_bounds__(1024) void log_max_kernel(float* __restrict__ L, int frames, int n_mel,
                                                       float* __restrict__ clip_max) {
  const int b = blockIdx.x;
  float* base = L + (int64_t)b * frames * n_mel;
  const int64_t n = (int64_t)frames * n_mel;
  float m = -INFINITY;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float v = log10f(fmaxf(base[i], 1e-10f));
    base[i] = v;
    m = fmaxf(m, v);
  }
  m = wave_max(m);
  __shared__ float part[16];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = part[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, part[w]);
    clip_max[b] = r;
  }
}

// out[b, m, f] = (max(L[b F + f, m], max_b - 8) + 4) / 4, through 32 x 32 LDS tiles.
template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ L, const float* __restrict__ clip_max,
                                                       T* __restrict__ out, int frames, int n_mel) {
  __shared__ float tile[32][33];
  const int b = blockIdx.z;
  const int f0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const float floor_v = clip_max[b] - 8.0f;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int f = f0 + r, m = m0 + tx;
    tile[r][tx] = (f < frames && m < n_mel) ? L[((int64_t)b * frames + f) * n_mel + m] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int m = m0 + r, f = f0 + tx;
    if (m < n_mel && f < frames) {
      const float v = (fmaxf(tile[tx][r], floor_v) + 4.0f) * 0.25f;
      T* dst = out + ((int64_t)b * n_mel + m) * frames + f;
      if constexpr (std::is_same<T, float>::value) *dst = v;
      else *dst = f32_to_bf16(v);
    }
  }
}

// Slaney mel scale: linear (3 f / 200) below 1 kHz, logarithmic above.
double hz_to_mel(double f) { return f < 1000.0 ? 3.0 * f / 200.0 : 15.0 + 27.0 * std::log(f / 1000.0) / std::log(6.4); }
double mel_to_hz(double m) { return m < 15.0 ? 200.0 * m / 3.0 : 1000.0 * std::exp((m - 15.0) * std::log(6.4) / 27.0); }

}  // namespace

struct aenc_frontend {
  aenc_frontend_config cfg{};
  int frames = 0;
  double* dft = nullptr;      // [448, 400]: row 2k cos, row 2k + 1 sin of bin k (rows past bin 200 zero)
  float* filters = nullptr;   // [n_mel, 224]
  float* ws = nullptr;        // padded audio | P | mel | clip max
  float *xp = nullptr, *P = nullptr, *mel = nullptr, *cmax = nullptr;
};

namespace {

void fe_error(const char* msg) { aenc::set_kernel_error(msg); }

bool fe_release(aenc_frontend* h) {
  if (h->dft) (void)hipFree(h->dft);
  if (h->filters) (void)hipFree(h->filters);
  if (h->ws) (void)hipFree(h->ws);
  return false;
}

}  // namespace

extern "C" int aenc_frontend_output_shape(const aenc_frontend_config* c, int64_t shape[3]) {
  if (!c || !shape) { fe_error("NULL argument"); return AENC_E_INVAL; }
  if (c->batch < 1 || c->n_samples <= FE_NFFT / 2 || c->n_samples % FE_HOP || c->n_mel < 1 || c->n_mel > 512 ||
      (c->out_dtype != AENC_F32 && c->out_dtype != AENC_BF16)) {
    fe_error("front end config: need batch >= 1, n_samples a multiple of 160 above 200, 1 <= n_mel <= 512, "
             "out_dtype AENC_F32 or AENC_BF16");
    return AENC_E_INVAL;
  }
  if ((int64_t)c->batch * c->n_samples > (int64_t)1 << 31) { fe_error("front end config: too many samples"); return AENC_E_INVAL; }
  shape[0] = c->batch;
  shape[1] = c->n_mel;
  shape[2] = c->n_samples / FE_HOP;
  return AENC_OK;
}

extern "C" aenc_frontend* aenc_frontend_create(const aenc_frontend_config* c) {
  int64_t shape[3];
  if (aenc_frontend_output_shape(c, shape) != AENC_OK) return nullptr;
  auto* h = new aenc_frontend;
  h->cfg = *c;
  h->frames = (int)shape[2];
  const int B = c->batch, n_mel = c->n_mel;
  // DFT rows: w[n] cos(2 pi k n / N) and w[n] sin(2 pi k n / N) of bin k at
  // rows 2k and 2k + 1 (the sign of the imaginary part does not matter for
  // the power).
  std::vector<double> dft((size_t)FE_DFT_N * FE_NFFT, 0.0);
  for (int k = 0; k < FE_BINS; ++k)
    for (int n = 0; n < FE_NFFT; ++n) {
      const double w = 0.5 - 0.5 * std::cos(2.0 * M_PI * n / FE_NFFT);
      const double a = 2.0 * M_PI * (double)((int64_t)k * n % FE_NFFT) / FE_NFFT;
      dft[(size_t)(2 * k) * FE_NFFT + n] = w * std::cos(a);
      dft[(size_t)(2 * k + 1) * FE_NFFT + n] = w * std::sin(a);
    }
  // Triangular filters between mel-spaced edges, each of unit area in Hz.
  std::vector<float> fb((size_t)n_mel * FE_PK, 0.0f);
  const double mel_hi = hz_to_mel(8000.0);
  std::vector<double> edge(n_mel + 2);
  for (int i = 0; i < n_mel + 2; ++i) edge[i] = mel_to_hz(mel_hi * i / (n_mel + 1));
  for (int m = 0; m < n_mel; ++m)
    for (int k = 0; k < FE_BINS; ++k) {
      const double f = 8000.0 * k / (FE_BINS - 1);
      const double rise = (f - edge[m]) / (edge[m + 1] - edge[m]);
      const double fall = (edge[m + 2] - f) / (edge[m + 2] - edge[m + 1]);
      const double v = std::fmax(0.0, std::fmin(rise, fall)) * 2.0 / (edge[m + 2] - edge[m]);
      fb[(size_t)m * FE_PK + k] = (float)v;
    }
  const int64_t rows = (int64_t)B * h->frames;
  const size_t n_xp = (size_t)B * (c->n_samples + FE_NFFT), n_P = (size_t)rows * FE_PK,
               n_mel_el = (size_t)rows * n_mel;
  hipError_t e;
  if ((e = hipMalloc(&h->dft, dft.size() * 8)) != hipSuccess || (e = hipMalloc(&h->filters, fb.size() * 4)) != hipSuccess ||
      (e = hipMalloc(&h->ws, (n_xp + n_P + n_mel_el + B + 64) * 4)) != hipSuccess ||
      (e = hipMemcpy(h->dft, dft.data(), dft.size() * 8, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(h->filters, fb.data(), fb.size() * 4, hipMemcpyHostToDevice)) != hipSuccess) {
    fe_error(hipGetErrorString(e));
    fe_release(h);
    delete h;
    return nullptr;
  }
  h->xp = h->ws;
  h->P = h->xp + n_xp;
  h->mel = h->P + n_P;
  h->cmax = h->mel + n_mel_el;
  return h;
}

extern "C" int aenc_frontend_run(aenc_frontend* h, const float* audio, void* mel_out, void* stream) {
  if (!h || !audio || !mel_out) { fe_error("NULL argument"); return AENC_E_INVAL; }
  if (((uintptr_t)audio | (uintptr_t)mel_out) & 15) { fe_error("audio and mel must be 16-byte aligned"); return AENC_E_INVAL; }
  const aenc_frontend_config& c = h->cfg;
  hipStream_t s = (hipStream_t)stream;
  const int B = c.batch, n = c.n_samples, F = h->frames, n_mel = c.n_mel;
  const int64_t rows = (int64_t)B * F;
  auto check = [](hipError_t e) {
    if (e != hipSuccess) { fe_error(hipGetErrorString(e)); return false; }
    return true;
  };
  hipLaunchKernelGGL(reflect_pad_kernel, dim3(2048), dim3(256), 0, s, audio, h->xp, n, B);
  if (!check(hipGetLastError())) return AENC_E_HIP;
  // frames: row r = b F + f starts at padded sample b (n + 400) + 160 f
  hipLaunchKernelGGL(dft_power_kernel, dim3(FE_DFT_N / DP_BN, (unsigned)((rows + DP_BM - 1) / DP_BM)), dim3(256), 0, s,
                     h->xp, n + FE_NFFT, F, (int)rows, h->dft, h->P);
  if (!check(hipGetLastError())) return AENC_E_HIP;
  EpiParams e2{};
  e2.c = h->mel;
  e2.crow = dense_rows(n_mel);
  if (!check(gemm_f32(EPI_STORE_F32, h->P, dense_rows(FE_PK), h->filters, FE_PK, (int)rows, n_mel, FE_PK, nullptr, e2,
                      s)))
    return AENC_E_HIP;
  hipLaunchKernelGGL(log_max_kernel, dim3(B), dim3(1024), 0, s, h->mel, F, n_mel, h->cmax);
  if (!check(hipGetLastError())) return AENC_E_HIP;
  dim3 grid((F + 31) / 32, (n_mel + 31) / 32, B);
  if (c.out_dtype == AENC_BF16)
    hipLaunchKernelGGL(finalize_kernel<bf16_t>, grid, dim3(256), 0, s, h->mel, h->cmax, (bf16_t*)mel_out, F, n_mel);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, grid, dim3(256), 0, s, h->mel, h->cmax, (float*)mel_out, F, n_mel);
  return check(hipGetLastError()) ? AENC_OK : AENC_E_HIP;
}

extern "C" void aenc_frontend_destroy(aenc_frontend* h) {
  if (!h) return;
  fe_release(h);
  delete h;
}
