/*
 * atlas.h -- C ABI of the MI355X (gfx950) W4 decode-step library (libatlas.so).
 *
 * The library computes the single-token decode step of an OLMo-3-32B-shaped dense
 * decoder whose linear layers hold 4-bit group-quantised weights, plus a prefill
 * entry point. Sources (page titles):
 *   [card]  "ATLAS-OLMo-3-32B-Think-v4" model card -- Quantization recipe (packed
 *           int4 layout, per-group scales, W4 x f32 activations, bf16 lm_head),
 *           Architecture deep-dive (GQA 40/8, head_dim 128, [SWA,SWA,SWA,full] x16,
 *           window 4,096, post-norm + full-projection QK-norm, RoPE theta 5e5,
 *           YaRN x8 with attention_factor ~1.208), Limitations & roadmap (prefill
 *           runs token by token through the decode path).
 *   [arch]  "Olmo 3 32B" field table (post norms only, q_norm/k_norm, rotary on the
 *           full head, untied embeddings, 100,278 vocabulary).
 *   [kb]    "OLMo 3 32B" knowledge-base page (reordered post-norm inside the
 *           residual branch; RMSNorm on Q and K before the dot product; YaRN only on
 *           global layers).
 *   [db]    "Olmo-3-1125-32B" database page (RMSNorm eps 1e-6, no biases, SwiGLU).
 *
 * Conventions for every entry point:
 *  - Returns an atlas_status code; nothing is thrown across the ABI.
 *  - All tensor pointers are DEVICE pointers owned by the caller (the library never
 *    allocates, frees or keeps them past the enqueued work); descriptor structs and
 *    their host arrays are HOST memory read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued and the call returns; kernel faults surface at the caller's sync.
 *  - Arguments are validated on the host before anything is launched; a failed
 *    check returns ATLAS_ERR_INVALID_ARG / ATLAS_ERR_UNSUPPORTED_SHAPE /
 *    ATLAS_ERR_WORKSPACE_TOO_SMALL and enqueues nothing. atlas_last_error() gives a
 *    message (thread-local).
 *  - Positions are read from device memory (`d_pos`) so a captured step replays for
 *    every token. A position outside [0, T_max) is detected on the device: the step
 *    writes nothing to the KV cache and sets the status word returned by
 *    atlas_device_status() to ATLAS_ERR_INVALID_ARG.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef ATLAS_H
#define ATLAS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define ATLAS_API __attribute__((visibility("default")))
#else
#define ATLAS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum atlas_status {
    ATLAS_OK = 0,
    ATLAS_ERR_INVALID_ARG = 1,
    ATLAS_ERR_UNSUPPORTED_SHAPE = 2,
    ATLAS_ERR_WORKSPACE_TOO_SMALL = 3,
    ATLAS_ERR_HIP = 4
} atlas_status;

/* A 4-bit group-quantised linear layer W[N][K] ([card] Quantization recipe).
 *  qweight: u32 [N][K/8]; code of column j is nibble j%8 (bits 4(j%8)..+3) of word
 *           j/8, the lowest nibble holding the lowest column.
 *  scales : [N][G] 16-bit floats, G = ceil(K/group); binary16 (scale_dtype 0) or
 *           bfloat16 (scale_dtype 1, the card's own choice).
 *  zeros  : u32 [N][ceil(G/8)] packed uint4 zero points in the same nibble order,
 *           or NULL for the card's symmetric form (stored nibble = q + 8, i.e. a
 *           zero point of 8).
 *  Dequantised weight: W[n][k] = (code - zero[n][k/group]) * scale[n][k/group].
 *  Requirements: K % 32 == 0, group % 32 == 0, N >= 1; 16-byte aligned qweight. */
typedef struct atlas_w4 {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* zeros;
    int32_t N, K, group, scale_dtype;
} atlas_w4;

/* Rotary embedding parameters ([card] RoPE row; [db] YaRN on full layers only).
 * inv_i = theta^(-2i/D); with yarn_factor > 1 the YaRN by-parts blend over the
 * correction range [floor b(beta_fast), ceil b(beta_slow)],
 * b(beta) = D ln(orig_max_pos / (2 pi beta)) / (2 ln theta), divides low
 * frequencies by yarn_factor; q and k are then scaled by attention_factor
 * (<= 0 selects 0.1 ln(yarn_factor) + 1, i.e. 1.2079 for x8). */
typedef struct atlas_rope {
    double theta;
    double yarn_factor;       /* <= 1: plain RoPE */
    double orig_max_pos;
    double beta_fast, beta_slow;
    double attention_factor;  /* <= 0: default 0.1 ln s + 1 (1 when no YaRN) */
} atlas_rope;

/* One decoder layer ([card] Architecture deep-dive; [kb]; [db]). qkv stacks the q
 * (Hq*D rows), k (Hkv*D) and v (Hkv*D) projections; gate and up are the two SwiGLU
 * inputs, down the output projection. Gains are f32. The caches are [Hkv][slots][D]
 * in the model's KV format (atlas_model.kv_dtype, swa_ring): slots = window on a
 * sliding-window layer kept as a ring (key j in slot j mod window), else t_max (key j
 * in slot j). type: 0 = sliding window, 1 = full attention. */
typedef struct atlas_layer {
    atlas_w4 qkv, o, gate, up, down;
    const float *g_q, *g_k, *g_pa, *g_pf;
    void *k_cache, *v_cache;
    int32_t type;
} atlas_layer;

typedef struct atlas_model {
    int32_t d, hq, hkv, hd, dff, n_layers, window, vocab;
    float eps;
    int64_t t_max;
    atlas_rope rope_swa, rope_full;
    const atlas_layer* layers;   /* host array [n_layers] */
    const uint16_t* embedding;   /* bf16 [vocab][d] (device), or NULL */
    const float* g_final;        /* f32 [d] final RMSNorm gain (device), or NULL */
    const uint16_t* lm_head;     /* bf16 [vocab][d] (device), or NULL */
    /* KV format ([card] Limitations & roadmap: a bf16 cache that keeps only the
     * window on the sliding-window layers). kv_dtype 0: f32 elements; 1: bfloat16,
     * rounded to nearest even (ties to even) when a key or value is stored and read
     * back exactly. swa_ring != 0: every type-0 layer keeps a ring of `window` slots
     * (needs window > 0); full layers always keep t_max. */
    int32_t kv_dtype;
    int32_t swa_ring;
} atlas_model;

ATLAS_API const char* atlas_version(void);
ATLAS_API const char* atlas_status_string(int status);
ATLAS_API const char* atlas_last_error(void);

/* ---- W4 GEMV ---------------------------------------------------------------------
 * y[n] = sum_k W[n][k] x[k] for an atlas_w4 W ([card] Quantization recipe: W4 x f32
 * activations with inline dequantisation). x: f32 [K], y: f32 [N] (device).
 * ws: device workspace of atlas_w4_gemv_workspace_bytes(W) bytes (x is re-encoded
 * there once per call). Result within 1e-6 relative of the f64 definition. */
ATLAS_API size_t atlas_w4_gemv_workspace_bytes(const atlas_w4* W);
ATLAS_API int atlas_w4_gemv(const atlas_w4* W, const float* x, float* y, void* ws, size_t ws_bytes, void* stream);

/* Batched W4 GEMV: y[v][n] = sum_k W[n][k] x[v][k] for B <= 8 activation vectors, the
 * weights read once for all of them (the projections of batched decode, [card]
 * Limitations & roadmap: batched decode after the batch-1 path). x: f32 [B][K], y: f32
 * [B][N] (device, row-major). Requires K % 64 == 0 and a group that is a multiple of
 * 128; else ATLAS_ERR_UNSUPPORTED_SHAPE. Each x[v] is encoded per block of 128 columns
 * as 24-bit block fixed point (n = rint(x / 2^e) with |n| < 2^23) and multiplied on the
 * int8 matrix cores in exact integer digit sums; result within 1e-6 relative of the f64
 * definition. ws: device workspace of atlas_w4_gemv_batch_workspace_bytes(W, B) bytes
 * (0 when the shape is unsupported). */
ATLAS_API size_t atlas_w4_gemv_batch_workspace_bytes(const atlas_w4* W, int32_t B);
ATLAS_API int atlas_w4_gemv_batch(const atlas_w4* W, const float* x, int32_t B, float* y, void* ws, size_t ws_bytes,
                                  void* stream);

/* Materialise the dequantised matrix out[N][K] f32 (device); exact (bit-for-bit
 * (code - zero) * scale). For checking the unpacking. */
ATLAS_API int atlas_w4_dequant(const atlas_w4* W, float* out, void* stream);

/* ---- W4 GEMM (the prefill projections) -------------------------------------------
 * C[m][n] = sum_k W[n][k] A[m][k] for M rows of f32 activations A [M][K] (row-major,
 * device) and an atlas_w4 W; C: f32 [M][N] (device). Runs on the matrix cores, per
 * quantisation group:
 *   A is first held as two bf16 planes (hi + lo, 16 significant bits); then
 *   - groups of 128, 256 or 512 dividing K, M > 16: int8 products. The planes are
 *     rounded per row and group to 24-bit integers v times a power-of-two scale s
 *     with max|A| / (127 * 2^16) <= s (error <= s/2 per element), carried as three int8
 *     digit planes; the raw codes multiply each plane exactly in int32, the digit sums
 *     and the zero point are combined in f32, and the group's sum is scaled and
 *     accumulated in f32;
 *   - other groups (32 or multiples of 64), or M <= 16: bf16 products of the planes
 *     with W as exact bf16 integers (code - zero), per group summed in f32.
 *   Either way the result is within about 1e-5 relative of the f64 definition.
 * Needs group == 32 or a multiple of 64 (else ATLAS_ERR_UNSUPPORTED_SHAPE).
 * ws: atlas_w4_gemm_workspace_bytes(W, M) bytes (the planes of A). */
ATLAS_API size_t atlas_w4_gemm_workspace_bytes(const atlas_w4* W, int32_t M);
ATLAS_API int atlas_w4_gemm(const atlas_w4* W, const float* A, int32_t M, float* C, void* ws, size_t ws_bytes,
                            void* stream);

/* ---- RMSNorm + residual -----------------------------------------------------------
 * out = resid + g * x / sqrt(mean(x^2) + eps) over n elements; with resid == NULL,
 * out = g * x / sqrt(mean(x^2) + eps) ([kb] reordered post-norm: the norm sits on
 * the sublayer output inside the residual branch; [db] RMSNorm eps 1e-6).
 * out may alias resid. All f32 device vectors. */
ATLAS_API int atlas_rmsnorm_residual(const float* x, const float* g, const float* resid, float* out, int32_t n,
                           float eps, void* stream);

/* ---- QK-norm + RoPE ---------------------------------------------------------------
 * In place on q [Hq][D] and k [Hkv][D] (f32 device): RMSNorm over the whole q
 * projection (Hq*D values, gain gq) and over the whole k projection (gain gk)
 * ([card] Architecture deep-dive: QK-norm spans the full projections), then rotary
 * embedding at position
 * *d_pos (device int32) on pairs (i, i + D/2) of every head with angle
 * pos * inv_i (angles in double) and magnitude factor m (rope->attention_factor
 * rule above). D must be even and <= 256. */
ATLAS_API int atlas_qk_norm_rope(float* q, float* k, const float* gq, const float* gk, int32_t Hq, int32_t Hkv,
                       int32_t D, const int32_t* d_pos, const atlas_rope* rope, float eps, void* stream);

/* ---- GQA decode attention ---------------------------------------------------------
 * out[h] = sum_j softmax_j(scale * q[h] . K[kv][j]) V[kv][j], kv = h / (Hq/Hkv), over
 * keys j in [max(0, pos - window + 1), pos] (window > 0: sliding window counting
 * the current token; window == 0: full context) with pos = *d_pos
 * ([card] sliding window 4,096, GQA 40/8). Caches f32 [Hkv][T_max][D]; slot pos
 * must already hold the new key/value. Split over the key range with an
 * online-softmax merge. q, out: f32 [Hq][D]. Requires D == 128, Hq % Hkv == 0,
 * Hq/Hkv <= 8. ws: atlas_gqa_decode_workspace_bytes(...) bytes. */
ATLAS_API size_t atlas_gqa_decode_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int64_t T_max);
ATLAS_API int atlas_gqa_decode(const float* q, const float* k_cache, const float* v_cache, int32_t Hq, int32_t Hkv,
                     int32_t D, int64_t T_max, const int32_t* d_pos, int32_t window, float softmax_scale,
                     float* out, void* ws, size_t ws_bytes, void* stream);

/* The same over caches in any KV format ([card] Limitations & roadmap: bf16 KV and
 * a window-sized cache on the sliding-window layers). layout (host memory):
 *   kv_dtype 0 = f32, 1 = bfloat16 elements;
 *   slots    = positions stored per KV head (caches are [Hkv][slots][D]);
 *   ring     != 0: key j lives in slot j mod slots and any pos >= 0 is accepted
 *              (needs 0 < window <= slots); else key j in slot j and pos < slots.
 * Slot of pos must already hold the new key/value. ws: at least
 * atlas_gqa_decode_workspace_bytes(Hq, Hkv, D, slots) bytes. A position outside the
 * accepted range (checked on the device) makes every output row zero. */
typedef struct atlas_kv_layout {
    int32_t kv_dtype;
    int32_t ring;
    int64_t slots;
} atlas_kv_layout;
ATLAS_API int atlas_gqa_decode_kv(const float* q, const void* k_cache, const void* v_cache,
                        const atlas_kv_layout* layout, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* d_pos,
                        int32_t window, float softmax_scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* ---- decode step ------------------------------------------------------------------
 * One token through m->n_layers layers ([card] Architecture deep-dive; [kb]):
 *   x = embedding[*d_token] (bf16 -> f32) if d_token != NULL, else d_hidden_in;
 *   per layer: qkv = W_qkv x; q,k <- full-projection RMSNorm; RoPE (YaRN and its
 *   factor on type-1 layers); K/V cache slot pos <- k, v; o = GQA attention over
 *   the layer's window; h = x + RMSNorm_pa(W_o o); z = silu(W_gate h) * (W_up h);
 *   x = h + RMSNorm_pf(W_down z).
 * d_hidden_out (f32 [d], may be NULL) receives the last layer's output. When
 * d_logits or d_argmax is non-NULL the final RMSNorm (g_final), the bf16 lm_head
 * GEMV (logits f32 [vocab]) and the greedy argmax (lowest index on ties, int32) run
 * as well. pos = *d_pos (device int32). ws: atlas_decode_workspace_bytes(m).
 * Shapes: head_dim 128, Hq % Hkv == 0 with Hq/Hkv <= 8, d a multiple of 32 in
 * [32, 6144], dff a multiple of 32; otherwise ATLAS_ERR_UNSUPPORTED_SHAPE. */
ATLAS_API size_t atlas_decode_workspace_bytes(const atlas_model* m);
ATLAS_API int atlas_decode_step(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in,
                      const int32_t* d_pos, float* d_hidden_out, float* d_logits, int32_t* d_argmax,
                      void* ws, size_t ws_bytes, void* stream);

/* ---- decode step without a workspace argument -------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. The same step as
 * atlas_decode_step (same arguments, results and shape limits), with its workspace
 * taken from a scratch area of ATLAS_NOALLOC_SCRATCH_BYTES (4 MiB) that the library
 * keeps in device memory, one per GPU, until the process ends. The call allocates
 * nothing and every step writes the parts of the scratch area it reads, so a call
 * does not depend on what an earlier call left there.
 *  - A model whose atlas_decode_workspace_bytes() exceeds the scratch size returns
 *    ATLAS_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the 32B shape needs
 *    about 1.4 MB at 16,385 slots and 2.1 MB at 65,536).
 *  - d_status_out (device int32, may be NULL) receives the step's status word, the
 *    value atlas_device_status() reads from a workspace, at the end of the step.
 *  - All calls on one GPU share that GPU's scratch area: calls that overlap in time on
 *    one GPU (from other streams or threads) race and must be serialised by the
 *    caller. Calls on different GPUs are independent. */
#define ATLAS_NOALLOC_SCRATCH_BYTES (4u << 20)
ATLAS_API int atlas_decode_step_noalloc(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in,
                              const int32_t* d_pos, float* d_hidden_out, float* d_logits, int32_t* d_argmax,
                              int32_t* d_status_out, void* stream);

/* Device status word of the last step that used this workspace (ATLAS_OK, or
 * ATLAS_ERR_INVALID_ARG when a position was out of range). Synchronises stream. */
ATLAS_API int atlas_device_status(const void* ws, void* stream, int32_t* status_out);

/* ---- prefill ----------------------------------------------------------------------
 * Processes n_tokens prompt tokens (device int32) at positions start_pos ..
 * start_pos + n_tokens - 1 through every layer, writing those KV slots, and
 * returns the last token's logits (f32 [vocab], may be NULL) and greedy argmax
 * (int32, may be NULL). By definition it equals n_tokens teacher-forced decode
 * steps ([card] Limitations: prefill currently runs token by token through the
 * decode path, with a batched GEMM prefill as the planned fix); here the projections
 * run as W4 GEMMs on the matrix cores over all tokens (see atlas_w4_gemm: int8
 * products for groups of 128-512, bf16 otherwise), QK norm, rotary and the KV write
 * per token, and causal attention within each layer's window on bf16 matrix cores
 * with hi/lo operands (about 2^-16 per product). Linear layers need group 32 or a
 * multiple of 64.
 * ws: atlas_prefill_workspace_bytes(m, n_tokens) bytes; its first word is the status
 * word of atlas_device_status (ATLAS_ERR_INVALID_ARG when a token id is out of range;
 * such ids read embedding row 0). */
ATLAS_API size_t atlas_prefill_workspace_bytes(const atlas_model* m, int32_t n_tokens);
ATLAS_API int atlas_prefill(const atlas_model* m, const int32_t* d_tokens, int32_t n_tokens, int32_t start_pos,
                  float* d_last_logits, int32_t* d_argmax, void* ws, size_t ws_bytes, void* stream);

/* ---- batched decode ------------------------------------------------------------------
 * One token for each of `batch` sequences (1..16) through m->n_layers layers ([card]
 * Limitations & roadmap: batched decode planned after batch-1 serving). By definition
 * the result is `batch` independent decode steps (atlas_decode_step) with shared
 * weights: sequence b feeds token d_tokens[b] at position d_pos[b] (device int32
 * [batch]) into its own KV cache. Each layer's k_cache/v_cache hold the sequences back
 * to back: [batch][Hkv][slots][D] in the model's KV format. The weights are read once
 * per step for the whole batch: the projections run as W4 GEMMs on the matrix cores
 * (the prefill's, split over K where the batch alone gives too few tiles), the lm_head
 * as one bf16 matrix-core pass. Outputs (device, each may be NULL): d_hidden_out f32
 * [batch][d] (last layer), d_logits f32 [batch][vocab], d_argmax int32 [batch] (first
 * index of the maximum). Needs an embedding table, d % 64 == 0 and group 32 or a
 * multiple of 64. ws: atlas_decode_batch_workspace_bytes(m, batch) bytes; its first
 * word is the status word of atlas_device_status (ATLAS_ERR_INVALID_ARG for a token id
 * or position out of range; such a sequence's cache is not written). */
ATLAS_API size_t atlas_decode_batch_workspace_bytes(const atlas_model* m, int32_t batch);
ATLAS_API int atlas_decode_batch(const atlas_model* m, const int32_t* d_tokens, const int32_t* d_pos, int32_t batch,
                       float* d_hidden_out, float* d_logits, int32_t* d_argmax, void* ws, size_t ws_bytes,
                       void* stream);

/* ---- on-device sampling -------------------------------------------------------------
 * Draws the next token from logits (f32 [vocab], device) with temperature and nucleus
 * (top-p) filtering ([card] Benchmarks and Prompting guide: served with temperature
 * 0.6, top-p 0.95). p_i is proportional to exp((l_i - max l) / temperature); the
 * nucleus is the fewest most-probable tokens whose mass reaches top_p, with tokens
 * tied with the last one included; the token is the first nucleus member, in
 * ascending index order, whose cumulative mass exceeds u times the nucleus mass,
 * u = *d_u (device float, clamped into [0, 1)). Masses are summed exactly in 2^-32
 * units, so the draw is deterministic. temperature == 0: greedy (first index of the
 * maximum; d_u and top_p unused). *d_token (device int32) receives the token.
 * vocab in [1, 2^21]; top_p in (0, 1]; ws: atlas_sample_workspace_bytes(vocab) bytes
 * of device memory. Asynchronous on `stream`; calls sharing a workspace must not
 * overlap. */
ATLAS_API size_t atlas_sample_workspace_bytes(int32_t vocab);
ATLAS_API int atlas_sample(const float* d_logits, int32_t vocab, float temperature, float top_p, const float* d_u,
                 int32_t* d_token, void* ws, size_t ws_bytes, void* stream);

/* ---- read-bandwidth probe (measurement aid) -------------------------------------------
 * Reads `bytes` (a positive multiple of 16) of the device buffer d_buf (16-byte
 * aligned) with a plain grid-stride streaming kernel of `blocks` blocks (1..65536) of
 * 256 threads, and nothing else: the achievable read bandwidth that the decode
 * kernels are compared with beside the device's peak. d_sink: one device uint32 that
 * is written only in the rare case that the XOR of all words read equals a fixed
 * sentinel. Asynchronous on `stream`; timed like any launch by atlas_profile_*
 * (label "stream_read"). ATLAS_ERR_INVALID_ARG on a null pointer, misaligned buffer,
 * bad size or block count. */
ATLAS_API int atlas_stream_read(const void* d_buf, size_t bytes, uint32_t* d_sink, int32_t blocks, void* stream);

/* ---- launch timing (measurement aid) -------------------------------------------------
 * Between atlas_profile_start(capacity) and atlas_profile_stop(), every kernel launch
 * of the library (at most `capacity` launches) carries a start and a stop hipEvent
 * that its dispatch stamps when the kernel begins and ends (hipExtLaunchKernel).
 * atlas_profile_stop synchronises the stream of the last launch, then reports per
 * launch label the number of launches and their summed execution time. Returns
 * ATLAS_ERR_INVALID_ARG if not started or if more than `capacity` launches were made.
 * Not thread-safe; meant for a single stream. */
typedef struct atlas_profile_entry {
    char name[48];
    int32_t count;
    double total_ms;
} atlas_profile_entry;

ATLAS_API int atlas_profile_start(int32_t capacity);
ATLAS_API int atlas_profile_stop(atlas_profile_entry* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif
#endif /* ATLAS_H */
