/*
 * aenc.h - C ABI of the Whisper-style audio encoder tower for AMD MI355X (gfx950).
 *
 * What the library computes (one forward, per clip b):
 *
 *   mel [n_mel, F] --conv1d(k3, s1, pad 1) + GELU--> [d, F]
 *                  --conv1d(k3, s2, pad 1) + GELU--> [d, T],  T = F/2
 *   + sinusoidal positions ([sin | cos], timescales 1 .. 10000)
 *   L pre-LayerNorm blocks: x += Attn(LN1 x); x += W2 GELU(W1 LN2 x + b1) + b2
 *     with bidirectional multi-head attention over all T positions (no causal
 *     mask, nothing cached), head_dim 64, as many KV heads as query heads
 *   final LayerNorm, then either nothing, a pair-average pool (pool_step 2) or
 *   a 2-layer GELU projector.
 *
 * Where this comes from:
 *   - Whisper-large geometry (d_model 1280, 32 layers, 20 heads, FFN 5120,
 *     128 mel bins, 1500 positions per 30 s window) and the single bidirectional
 *     pass without a KV cache: "Qwen2-Audio-7B-Instruct", section (1) AUDIO ENCODER.
 *   - head_dim 64 with 20 KV heads (MHA), 3000 feature frames per 30 s chunk and
 *     the 2-layer gelu projector 1280 -> 3072: "Voxtral-Mini-3B-2507", sections
 *     (1) AUDIO ENCODER, Preprocessor and PROJECTOR.
 *   - Whisper-medium geometry and audio_pool_step 2 (1500 -> ~750 tokens):
 *     "MiniCPM-o-2_6", section (2) AUDIO.
 *   - The encoder runs as its own precompute pass, on a schedule separate from
 *     decode: the SERVICEABILITY JOIN / REQUIRED KERNEL CLASS passages of the
 *     Kimi-Audio, Qwen2-Audio and MiniCPM-o records. Hence forward() only
 *     enqueues on a caller-chosen stream.
 *
 * Conventions
 *   - Linear weights are row-major [out, in] (the checkpoint convention the
 *     Qwen2-Audio record reads from tensor shapes: q_proj.weight [1280, 1280]);
 *     conv weights are [out, in, 3]; vectors are [n].
 *   - Tensors are in the geometry's dtype (AENC_BF16 or AENC_F32). bf16 is the
 *     IEEE-754 binary32 upper half (bfloat16).
 *   - There is no key bias slot: a bias on the keys adds a constant to every
 *     score of a query row and cannot change the softmax.
 *   - All functions are thread-safe across distinct handles; one handle must
 *     not be used from two threads at once.
 */
#ifndef AENC_H
#define AENC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
enum { AENC_F32 = 0, AENC_BF16 = 1 };

/* Chunked attention rules (aenc_geometry.attn_chunk_mode). */
enum {
  AENC_CHUNK_NONE = 0,    /* every position sees every valid position of its clip */
  AENC_CHUNK_CAUSAL = 1,  /* its own chunk and every earlier chunk                */
  AENC_CHUNK_BLOCK = 2    /* its own chunk only                                   */
};

/* Status codes returned by the int-valued functions. */
typedef enum {
  AENC_OK = 0,
  AENC_E_INVAL = -1,        /* bad argument or geometry (nothing was touched) */
  AENC_E_UNSUPPORTED = -2,  /* valid request this build does not serve (e.g. non-gfx950 device) */
  AENC_E_NOMEM = -3,        /* device allocation failed */
  AENC_E_DEVICE = -4,       /* no usable HIP device */
  AENC_E_HIP = -5           /* a HIP runtime call failed; see aenc_last_error() */
} aenc_status;

/* Encoder geometry. Field names follow the checkpoint config fields the model
 * records print (d_model, encoder_layers, encoder_attention_heads,
 * encoder_ffn_dim, num_mel_bins, audio_pool_step, projector width). */
typedef struct aenc_geometry {
  int32_t batch;        /* clips per forward, 1 .. 4096; the workspace is sized for it.
                         * bf16: each GEMM operand must stay under 4 GiB (32-bit buffer
                         * offsets), e.g. at most 278 clips of 3000 frames with d_ffn
                         * 5120; aenc_validate reports the largest batch allowed.     */
  int32_t n_mel;        /* num_mel_bins (1 .. 512)                                           */
  int32_t n_frames;     /* F mel frames per clip, even, 2 .. 3000; T = F/2 positions         */
  int32_t d_model;      /* d = 64 * n_heads, a multiple of 128, <= 2048                       */
  int32_t n_layers;     /* encoder_layers (>= 0)                                             */
  int32_t n_heads;      /* encoder_attention_heads; head_dim = d_model / n_heads must be 64  */
  int32_t d_ffn;        /* encoder_ffn_dim, a multiple of 64                                 */
  int32_t pool_step;    /* 1 (none) or 2 (average of positions 2j, 2j+1; T/2 outputs)        */
  int32_t proj_hidden;  /* 0 = no projector; else the projector's hidden width (mult. of 64) */
  int32_t proj_out;     /* projector output width (multiple of 64); 0 when proj_hidden is 0  */
  int32_t dtype;        /* AENC_BF16 (fp32 accumulate, fp32 residual) or AENC_F32           */
  int32_t out_dtype;    /* element type of `out`: AENC_F32 or AENC_BF16                       */
  float ln_eps;         /* LayerNorm epsilon (> 0), e.g. 1e-5                                */
  int32_t stack;        /* 0 or 1: none. 4: the projector reads runs of 4 consecutive final-LN
                         * positions concatenated in order ([T, d] -> [T/4, 4d], a trailing
                         * partial run dropped), i.e. 12.5 rows per second of audio with a
                         * 4d-wide projector input (Whisper features downsampled to 12.5 Hz,
                         * "[WIP][TSS][Model] Kimi-Audio-7B", Purpose; kimia_adaptor_input_dim
                         * 5120, "Kimi-Audio-7B-Instruct", (1) AUDIO). Needs a projector and
                         * pool_step 1.                                                    */
  int32_t attn_chunk;   /* 0: full bidirectional attention. > 0: positions are cut into
                         * chunks of attn_chunk consecutive positions (by their position in
                         * the clip, masked ones included) and attention follows
                         * attn_chunk_mode. A reading of audio_chunk_length 1.0 printed beside
                         * MiniCPM-o's Whisper encoder ("MiniCPM-o-2_6", (2) AUDIO): 1 s of
                         * audio is 50 positions. 0 .. n_frames/2.                          */
  int32_t attn_chunk_mode; /* AENC_CHUNK_CAUSAL or AENC_CHUNK_BLOCK when attn_chunk > 0,
                            * AENC_CHUNK_NONE (0) otherwise.                               */
} aenc_geometry;

/* One block's tensors (d = d_model, f = d_ffn). Pointers may be host or device
 * memory; create() copies them. Bias and beta pointers may be NULL (zero);
 * gamma pointers may be NULL (one). Weight matrices must not be NULL. */
typedef struct aenc_layer_weights {
  const void *ln1_g, *ln1_b;            /* [d]                       */
  const void *q_w, *q_b;                /* [d, d], [d]               */
  const void *k_w;                      /* [d, d]  (no key bias)     */
  const void *v_w, *v_b;                /* [d, d], [d]               */
  const void *o_w, *o_b;                /* [d, d], [d]               */
  const void *ln2_g, *ln2_b;            /* [d]                       */
  const void *fc1_w, *fc1_b;            /* [f, d], [f]               */
  const void *fc2_w, *fc2_b;            /* [d, f], [d]               */
} aenc_layer_weights;

typedef struct aenc_weights {
  const void *conv1_w, *conv1_b;        /* [d, n_mel, 3], [d]        */
  const void *conv2_w, *conv2_b;        /* [d, d, 3], [d]            */
  const aenc_layer_weights *layers;     /* host array of n_layers    */
  const void *lnf_g, *lnf_b;            /* [d]                       */
  const void *proj1_w, *proj1_b;        /* [proj_hidden, stack*d], [proj_hidden]  (projector only) */
  const void *proj2_w, *proj2_b;        /* [proj_out, proj_hidden], [proj_out]    (projector only) */
} aenc_weights;

typedef struct aenc_handle aenc_handle;

/* Check a geometry on the host. No device call. Returns AENC_OK, AENC_E_INVAL
 * (a field out of range, or a bf16 batch whose largest GEMM operand would
 * reach 4 GiB: aenc_last_error() names the largest batch allowed) or
 * AENC_E_UNSUPPORTED (pool_step 2 together with a projector: the pages never
 * combine them, so their order is not defined). */
int aenc_validate(const aenc_geometry *g);

/* Build an encoder on the current HIP device. Validates g and w (before any
 * device call), checks for a gfx950 device, allocates a library-owned device
 * arena, copies and repacks the weights into it (the caller may free its
 * copies afterwards), allocates the workspace for g->batch clips and
 * synchronises once. Returns NULL on error; aenc_last_error() says why. */
aenc_handle *aenc_create(const aenc_geometry *g, const aenc_weights *w);

/* Run the tower on g->batch clips. Enqueues kernels on `stream` (a
 * hipStream_t; NULL = the null stream) and returns without synchronising; it
 * allocates nothing, so it may be captured into a HIP graph.
 *   mel  : device, [batch, n_mel, n_frames], dtype. Row-major, channels first.
 *   mask : device uint8 [batch, T] key-padding mask (1 = valid position) or
 *          NULL (all valid). Masked positions take no part as keys; their own
 *          output rows are written as zeros, so a clip with no valid
 *          position at all comes out as zeros. Frames that only masked
 *          positions read may hold anything finite.
 *   out  : device, [batch, T_out, D_out] in out_dtype, with T_out = T /
 *          pool_step and D_out = proj_out or d_model (see aenc_output_shape).
 * mel and out must be 16-byte aligned (hipMalloc and torch allocations are).
 * Forwards on one handle share its workspace and must be ordered (one stream
 * or explicit dependencies). Returns AENC_OK, AENC_E_INVAL (NULL handle, NULL
 * or misaligned pointer) or AENC_E_HIP (launch failure); device faults
 * surface at the caller's next synchronisation. */
int aenc_forward(aenc_handle *h, const void *mel, const uint8_t *mask, void *out, void *stream);

/* Release the handle's device memory. NULL is ignored. Synchronises the device
 * first so that no enqueued forward still uses the workspace. */
void aenc_destroy(aenc_handle *h);

/* Message for the last error on the calling thread ("" if none). */
const char *aenc_last_error(void);

/* Trainable parameters of g (conv stem, blocks, final LN, projector), a
 * closed form on the host; -1 for an invalid geometry. */
int64_t aenc_param_count(const aenc_geometry *g);

/* Output shape {batch, T_out, D_out} of g. Host only. */
int aenc_output_shape(const aenc_geometry *g, int64_t shape[3]);

/* Workspace bytes create() allocates for g (activations, masks, tables),
 * excluding the weight arena. Host only; -1 for an invalid geometry. */
int64_t aenc_workspace_bytes(const aenc_geometry *g);

/* Per-step timing with HIP events, for measurement. When enabled, forward()
 * records an event before the first and after every kernel it launches.
 * aenc_profile_read() waits for the events of the forwards recorded since the
 * last read (at most 64) and adds each kernel's duration, in milliseconds, to
 * ms[kind] and the number of launches to calls[kind], for kind < n_kinds.
 * Kind names: aenc_profile_kind_name(). Returns the number of forwards read,
 * or a negative status. */
int aenc_profile_enable(aenc_handle *h, int on);
int aenc_profile_read(aenc_handle *h, double *ms, int64_t *calls, int n_kinds);
int aenc_profile_kind_count(void);
const char *aenc_profile_kind_name(int kind);

/* The geometry a handle was created with (NULL arguments: AENC_E_INVAL). */
int aenc_handle_geometry(const aenc_handle *h, aenc_geometry *g);

/* ---------------------------------------------------------------------------
 * Forward without allocation, for callers that cannot allocate device memory
 * while they run (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the activations live in a static device array of
 * AENC_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, instead of the handle's workspace.
 *
 * aenc_forward_noalloc runs aenc_forward's kernels on the first n_clips clips
 * of the buffers (1 <= n_clips <= the handle's batch): mel [n_clips, n_mel,
 * n_frames], mask [n_clips, T] or NULL, out [n_clips, T_out, D_out], in the
 * layouts and types of aenc_forward, and enqueues on `stream` without
 * synchronising. It allocates nothing and calls no allocating routine; the
 * packing maps are built into the array on every call, and the part of the
 * array a call uses is cleared first by a fill kernel (the array keeps the
 * last call's contents otherwise). Every call on one GPU shares that GPU's
 * array, whatever the handle: calls that overlap in time on one GPU race and
 * must be ordered by the caller (one stream, or events). Returns AENC_OK,
 * AENC_E_INVAL (NULL handle or pointer, misaligned pointer, n_clips out of
 * range, or a workspace for n_clips clips over AENC_NOALLOC_SCRATCH_BYTES:
 * aenc_last_error() gives the size needed) or AENC_E_HIP (launch failure).
 * A Whisper-large clip (3000 frames, d_model 1280, FFN 5120) needs about
 * 78 MB (its residual products are split along K, whose partials take 31 MB),
 * so the array holds one such clip per call.
 *
 * aenc_noalloc_scratch_bytes: the bytes n_clips clips of g need in the array
 * (host only; -1 for an invalid geometry or n_clips outside 1..g->batch). */
#define AENC_NOALLOC_SCRATCH_BYTES (96LL << 20)
int aenc_forward_noalloc(aenc_handle *h, int n_clips, const void *mel, const uint8_t *mask, void *out,
                         void *stream);
int64_t aenc_noalloc_scratch_bytes(const aenc_geometry *g, int n_clips);

/* ---------------------------------------------------------------------------
 * Embeddings cache: encoder outputs kept on the device under caller-given
 * 64-bit content keys (for instance a hash of the clip's audio and length),
 * so a clip seen before is served by a device copy. Serving stacks pair such
 * a cache with a separately scheduled encoder (TRT-LLM's "Multimodal
 * Embeddings Cache" and "Multimodal Encoder Side Stream", cited by the
 * "Kimi-Audio-7B-Instruct" and "Qwen2-Audio-7B-Instruct" records, (1) under
 * SERVICEABILITY JOIN).
 *
 * The pool of `capacity` slots of `entry_bytes` each is allocated at create;
 * lookups and inserts allocate nothing and enqueue device-to-device copies on
 * the given stream, ordered after any earlier copy of the same slot (on any
 * stream). Least recently used slots are recycled. Host calls may come from
 * several threads.
 * ------------------------------------------------------------------------- */
typedef struct aenc_cache aenc_cache;

aenc_cache *aenc_cache_create(int64_t entry_bytes, int64_t capacity);   /* NULL on error */
void aenc_cache_destroy(aenc_cache *c);                                 /* NULL-safe */
/* 1 if `key` is cached, else 0 (no copy, no statistics). */
int aenc_cache_contains(aenc_cache *c, uint64_t key);
/* Hit: enqueue a copy of the entry into device `dst` (entry_bytes), return 1.
 * Miss: return 0 and enqueue nothing. */
int aenc_cache_lookup(aenc_cache *c, uint64_t key, void *dst, void *stream);
/* Store entry_bytes from device `src` under `key` (replacing its entry, or
 * taking a free or the least recently used slot). AENC_OK or an error. */
int aenc_cache_insert(aenc_cache *c, uint64_t key, const void *src, void *stream);
/* out = {hits, misses, inserts, evictions, entries}. */
int aenc_cache_stats(aenc_cache *c, int64_t out[5]);
/* aenc_forward through the cache: keys[b] names clip b (entry_bytes must be
 * one clip's output, T_out * D_out * element size). If every clip is cached,
 * only copies are enqueued; otherwise the whole batch runs (its shape is
 * fixed) and the new clips are stored. *hits (if not NULL) receives the
 * number of clips found. */
int aenc_forward_cached(aenc_handle *h, aenc_cache *c, const uint64_t *keys, const void *mel,
                        const uint8_t *mask, void *out, void *stream, int32_t *hits);

/* ---------------------------------------------------------------------------
 * Log-mel front end: 16 kHz audio -> the encoder's input features.
 *
 * The extractor's geometry is the pages' Whisper feature extractor (16 kHz,
 * 480,000 samples per 30 s chunk, n_fft 400, hop 160, 128 features, 3000
 * frames: "Voxtral-Mini-3B-2507", Preprocessor). Its steps follow the Whisper
 * recipe: centred frames with reflect padding of 200 samples, periodic Hann
 * window, power spectrum of bins 0..200 with the last centred frame dropped,
 * Slaney-scale triangular mel filters of unit area (0 to 8 kHz), log10
 * floored at 1e-10, then floored at the clip's maximum minus 8, then
 * (x + 4) / 4.
 * ------------------------------------------------------------------------- */
typedef struct aenc_frontend_config {
  int32_t batch;        /* clips per call; the workspace is sized for it            */
  int32_t n_samples;    /* samples per clip: a multiple of 160, above 200 (480000) */
  int32_t n_mel;        /* filters (1 .. 512): 128 or 80                             */
  int32_t out_dtype;    /* AENC_F32 or AENC_BF16                                     */
} aenc_frontend_config;

typedef struct aenc_frontend aenc_frontend;

/* [batch, n_mel, n_samples / 160]: the frame count is the hop count (3000 for
 * 480,000 samples). Validates the config (AENC_E_INVAL when it is bad). */
int aenc_frontend_output_shape(const aenc_frontend_config *c, int64_t shape[3]);

/* Build the DFT matrix and the filters on the current device and allocate the
 * workspace (about 4 * batch * n_samples * 8 bytes). NULL on error. */
aenc_frontend *aenc_frontend_create(const aenc_frontend_config *c);

/* audio: device fp32 [batch, n_samples]; mel: device [batch, n_mel, frames]
 * in out_dtype, channels first (the layout aenc_forward reads); both 16-byte
 * aligned. Enqueues on `stream` without synchronising and allocates nothing.
 * Calls on one handle must be stream-ordered (one workspace). */
int aenc_frontend_run(aenc_frontend *h, const float *audio, void *mel, void *stream);

/* Free the handle (NULL is accepted). */
void aenc_frontend_destroy(aenc_frontend *h);

#ifdef __cplusplus
}
#endif

#endif /* AENC_H */
