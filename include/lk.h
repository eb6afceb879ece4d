/*
 * lk.h -- C ABI of the MI355X (gfx950) lightning-indexer hot path.
 *
 * The indexer of DeepSeek-V3.2-Exp's sparse attention scores every cached key
 * position against each query token and keeps the best positions per token:
 *
 *   S[t,s] = k_scale[s] * sum_{h<64} w_eff[t,h] * ReLU( q8[t,h,:] . k8[s,:] )
 *
 * (page "Index scores": the score formula, with 1/sqrt(64) folded into the
 * weights and 1/sqrt(128) folded together with each query's fp8 scale; the
 * fp8_index docstring excerpt: fp8 q @ fp8 k -> fp32 logits, ReLU, times the
 * folded weights, head sum, times the e8m0 key scale).  Keys and queries reach
 * fp8 through a scaled Hadamard-128 rotation and a per-128-feature power-of-two
 * scale (page "Hadamard rotation"; page "Index key cache").  Masked positions
 * get -inf and each row keeps its top-k positions (Indexer.forward excerpt).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE memory owned by the caller (for example
 *     PyTorch tensors).  The library never allocates, frees, copies to the host
 *     or synchronizes; each call only enqueues kernels on `stream` and returns.
 *   - `lk_rows` structures are HOST memory, read during the call only.
 *   - Validation happens on the host before any HIP call; a failed validation
 *     enqueues nothing.  LK_E_HIP reports a failed kernel launch (the status the
 *     launch call itself returned; errors pending from earlier HIP calls are not
 *     read or cleared).
 *   - bf16 data is passed as its uint16 bit pattern; fp8 data is e4m3fn bytes.
 *   - The library keeps no state (apart from the per-thread profiling events of
 *     lk_profile_next_launch), prints nothing and never aborts; calls are
 *     thread-safe.  Non-finite inputs are outside the contract.
 *   - Zero-sized work (no rows, no keys) returns LK_OK and enqueues nothing.
 */
#ifndef LK_H
#define LK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LK_API __attribute__((visibility("default")))

#define LK_ABI_VERSION 1
#define LK_DIM 128          /* features per index head and per key (page "Index scores") */
#define LK_HEADS 64         /* index heads (page "Index scores")                       */
#define LK_TOPK_MAX_T 16384 /* longest score row lk_topk accepts (one row in LDS)      */
#define LK_SELECT_FUSED_MAX_T 1024 /* rows lk_decode_select scores and selects in one launch */
#define LK_ROPE_DIM 64      /* leading features RoPE rotates (Indexer.forward excerpt)  */
#define LK_MLA_HEADS 128    /* attention heads of the MLA decode (page "Join query parts") */
#define LK_MLA_LATENT 512   /* latent (content) features per head and per cached row    */
#define LK_MLA_ROPE 64      /* rotary features per head and per cached row              */
#define LK_MLA_SCRATCH_BYTES (64u << 20) /* static workspace of lk_sparse_mla_decode_static */

typedef enum lk_status {
    LK_OK = 0,
    LK_E_NULL = -1,        /* a required pointer is NULL                               */
    LK_E_SHAPE = -2,       /* negative size, or sizes that do not fit together          */
    LK_E_UNSUPPORTED = -3, /* valid request outside what the library implements:
                              heads != 64 in lk_index_score, T > LK_TOPK_MAX_T in
                              lk_topk, a launch grid beyond the HIP limits, or a
                              pointer not aligned to 16 bytes (4 for float tensors)    */
    LK_E_HIP = -4,         /* the HIP runtime rejected a kernel launch                 */
    LK_E_SCRATCH = -5      /* lk_sparse_mla_decode_static: the request needs more
                              workspace than LK_MLA_SCRATCH_BYTES                      */
} lk_status;

/*
 * Which (sequence b, query token t, key s) triples are valid.  Valid keys always
 * form a prefix [0, L) of the score row of (b, t), with
 *
 *   L(b,t) = min( T,  seq_len ? clamp(seq_len[b], 0, T) : T,
 *                 causal ? start_pos + t + 1 : T )          (clamped below at 0)
 *
 * Slots L <= s < T of the score row are -inf (Indexer.forward adds the causal
 * mask; a ragged batch masks each sequence's unused cache slots the same way).
 */
typedef struct lk_rows {
    int32_t B;               /* sequences                                            */
    int32_t S;               /* query tokens per sequence in this call (decode: 1)   */
    int64_t T;               /* key slots per score row (= end_pos)                  */
    int64_t start_pos;       /* absolute position of query token 0 (causal masking)  */
    const int32_t *seq_len;  /* DEVICE [B] valid cache length per sequence, or NULL  */
    int32_t causal;          /* nonzero: key s > start_pos + t is masked              */
} lk_rows;

/*
 * Key write: rotate_activation + act_quant + cache write of Indexer.forward
 * (page "Hadamard rotation": kbar = ktilde (1/sqrt 128) H_128 with a bf16 result,
 * then fp8 quantization in groups of 128 features; page "Index key cache": an
 * e4m3fn cache [B, T, 128] plus one float32 scale per position).
 *
 * For each sequence b < n_seq and row i < n_rows, the 128 bf16 values at
 *   x + (b * x_seq_stride + i) * 128
 * are rotated with Sylvester's Hadamard-128 (exact sum, one fp64 multiply by
 * fl64(128^-0.5), one round-to-nearest-even to bf16), scaled by the smallest
 * power of two 2^j (j >= -126) with amax <= 448 * 2^j, and encoded as e4m3fn
 * (nearest-even, sign kept, never NaN).  The 128 bytes go to cache row
 *   p = (positions ? positions[b] : row_offset) + i
 * at  cache + (b * cache_seq_stride + p) * 128, and 2^j to
 * cache_scale[b * cache_seq_stride + p].  positions is DEVICE [n_seq] int32 or NULL.
 * Without positions the host checks the destination: 0 <= row_offset and
 * row_offset + n_rows <= cache_rows, else LK_E_SHAPE (the cache write at
 * [start_pos, end_pos) of Indexer.forward never leaves the cache).  With positions,
 * which the host cannot read, the kernel checks each row and skips (does not write)
 * a row whose p falls outside [0, cache_rows).
 * Results are bit-exact for every row whose nonzero magnitudes span at most
 * 2^38 and whose values are below 2^120 in magnitude.
 * Requires: cache_rows <= cache_seq_stride; x and cache 16-byte aligned.
 */
LK_API lk_status lk_quantize_keys(const uint16_t *x, int64_t n_seq, int64_t n_rows,
                                  int64_t x_seq_stride, uint8_t *cache, float *cache_scale,
                                  int64_t cache_seq_stride, int64_t cache_rows,
                                  int64_t row_offset, const int32_t *positions,
                                  hipStream_t stream);

/*
 * Query side of Indexer.forward: rotate_activation + act_quant of every head
 * row (same recipe as lk_quantize_keys, one 128-feature group per head) and
 * the weight fold
 *   w_eff = fl32( fl32(w * q_scale) * fl32(128^-0.5) )
 * (page "Index scores": 1/sqrt(128) is folded with each query's fp8 scale; `w`
 * already carries the 1/sqrt(64) factor).
 *   q      [n_tokens, heads, 128] bf16 bits     -> q_fp8 [n_tokens, heads, 128]
 *   w      [n_tokens, heads] float32           -> w_eff [n_tokens, heads] float32
 *   q_scale (optional, may be NULL) receives the [n_tokens, heads] scales 2^j.
 * Requires q and q_fp8 16-byte aligned.
 */
LK_API lk_status lk_quantize_queries(const uint16_t *q, const float *w, int64_t n_tokens,
                                     int32_t heads, uint8_t *q_fp8, float *w_eff,
                                     float *q_scale, hipStream_t stream);

/*
 * lk_quantize_keys and lk_quantize_queries in ONE kernel launch: the key write of
 * a step's new tokens and the query preparation are independent, and a decode step
 * is short enough that a second launch costs more than either job.  Arguments,
 * results and errors are those of the two calls (either job may be empty), plus
 * optional RoPE (Indexer.forward excerpt: q_pe / k_pe rotated, "not interleaved",
 * before rotate_activation; the NKI page takes cos / sin tables of rope_dim / 2
 * entries per token): feature pairs (i, i + 32) of the leading LK_ROPE_DIM = 64
 * features become
 *   y_i = fl32(fl32(x_i c_i) - fl32(x_{i+32} s_i)),  y_{i+32} = fl32(fl32(x_i s_i) + fl32(x_{i+32} c_i)),
 * each rounded to bf16 (nearest-even), before the Hadamard rotation.
 *   k_rope_cos / k_rope_sin: float32 [n_seq * n_rows][32], one row per key row
 *   (row b * n_rows + i), or both NULL for keys that need no rotation;
 *   q_rope_cos / q_rope_sin: float32 [n_tokens][32], one row per query token (shared
 *   by its heads), or both NULL.  Tables must be 16-byte aligned.
 */
LK_API lk_status lk_prepare(const uint16_t *x, int64_t n_seq, int64_t n_rows, int64_t x_seq_stride,
                            uint8_t *cache, float *cache_scale, int64_t cache_seq_stride,
                            int64_t cache_rows, int64_t row_offset, const int32_t *positions,
                            const uint16_t *q, const float *w, int64_t n_tokens, int32_t heads,
                            uint8_t *q_fp8, float *w_eff, float *q_scale,
                            const float *k_rope_cos, const float *k_rope_sin,
                            const float *q_rope_cos, const float *q_rope_sin, hipStream_t stream);

/*
 * fp8_index + mask (page "Index scores"): for every valid (b, t, s)
 *   scores[(b*S + t)*T + s] = k_scale[b*cache_seq_stride + s]
 *        * sum_h w_eff[(b*S + t)*heads + h] * ReLU( q8[(b*S+t), h, :] . k8[b, s, :] )
 * and -inf (0xFF800000) for masked slots (see lk_rows).
 *   q_fp8  [B, S, heads, 128] e4m3fn;  w_eff [B, S, heads] float32 (folded)
 *   k_cache: key s of sequence b at k_cache + (b*cache_seq_stride + s)*128
 *   k_scale: float32 power-of-two scale of the same key at b*cache_seq_stride + s
 *   scores [B, S, T] float32.
 * The fp8 values are converted exactly to f16 and contracted on the MFMA unit
 * with float32 accumulation; ReLU, the head weighting and sum, the key scale and
 * the mask are applied in registers; each score is written once.
 * Requires heads == 64 (else LK_E_UNSUPPORTED), T <= cache_seq_stride,
 * q_fp8 and k_cache 16-byte aligned, w_eff 16-byte aligned.  LK_E_UNSUPPORTED past
 * the launch grid limits: B > 65535, or (S > 1) B * ceil(S / 8) * ceil(T / 4096)
 * blocks above 2^31 - 8.
 */
LK_API lk_status lk_index_score(const uint8_t *q_fp8, const float *w_eff, int32_t heads,
                                const uint8_t *k_cache, const float *k_scale,
                                int64_t cache_seq_stride, const lk_rows *rows,
                                float *scores, hipStream_t stream);

/*
 * One decode step of Indexer.forward up to the scores, in ONE kernel launch: the
 * new token's key write (the cache update at [start_pos, end_pos) of the forward
 * excerpt), the query quantization with the weight fold, and fp8_index + mask.
 * Rows have S == 1.  For sequence b with valid length L = row length of lk_rows
 * (L >= 1), the new key k_new[b] goes to cache slot L-1 -- the decode token's own
 * position -- exactly as lk_quantize_keys would write it, and the scores of keys
 * [0, L) include it.  A row with L == 0 writes nothing to the cache and scores -inf.
 *   q      [B, heads, 128] bf16 bits;   w [B, heads] float32 (raw, 1/sqrt(64) included)
 *   k_new  [B, 128] bf16 bits
 *   k_cache / k_scale as in lk_index_score (written at slot L-1 of each sequence)
 *   scores [B, 1, T] float32, identical to lk_prepare + lk_index_score on the same inputs.
 *   q_fp8_out [B, heads, 128], w_eff_out [B, heads]: optional (both NULL or both set)
 *   copies of the quantized query and folded weights.
 *   rope_cos / rope_sin: optional (both NULL or both set) float32 [B][32] tables of the
 *   step's token, applied to the query heads and the new key as in lk_prepare.
 * Every block of the kernel quantizes its row's query while its key loads are in
 * flight, so the query preparation costs no separate launch.
 * Requires S == 1, heads == 64, T <= cache_seq_stride; q, k_new, k_cache and
 * q_fp8_out 16-byte aligned, w and w_eff_out 4-byte aligned.
 */
LK_API lk_status lk_decode_score(const uint16_t *q, const float *w, int32_t heads, const uint16_t *k_new,
                                 uint8_t *k_cache, float *k_scale, int64_t cache_seq_stride,
                                 const lk_rows *rows, float *scores, uint8_t *q_fp8_out,
                                 float *w_eff_out, const float *rope_cos, const float *rope_sin,
                                 hipStream_t stream);

/*
 * The decode step's scores and their per-row top-k from ONE call, as the NKI indexer
 * returns both (page "DeepSeek-V3.2 Sparse Indexer Kernel API Reference", the call's
 * returns: scores and top-k indices).  Arguments and results as lk_decode_score, then
 * idx [B, 1, k] exactly as lk_topk would produce from those scores (same indices in the
 * same order).  Rows of at most LK_SELECT_FUSED_MAX_T key slots (the pages' stated
 * decode step, 1001 keys at position 1000, is one) run as ONE kernel launch in which
 * each block keeps its row's scores in LDS and selects from them there, so the scores
 * make no round trip through memory; `scores` may then be NULL (not written).  Longer
 * rows run as lk_decode_score's launch followed by lk_topk's, and need `scores`.
 * Requires what lk_decode_score and lk_topk require: S == 1, heads == 64,
 * T <= cache_seq_stride, 1 <= k <= T, T <= LK_TOPK_MAX_T; idx 4-byte aligned.
 */
LK_API lk_status lk_decode_select(const uint16_t *q, const float *w, int32_t heads, const uint16_t *k_new,
                                  uint8_t *k_cache, float *k_scale, int64_t cache_seq_stride,
                                  const lk_rows *rows, float *scores, uint8_t *q_fp8_out,
                                  float *w_eff_out, const float *rope_cos, const float *rope_sin,
                                  int32_t k, int32_t *idx, hipStream_t stream);

/*
 * Per-row top-k of Indexer.forward (index_score.topk), with the NKI indexer's
 * int32 unordered-set result (page "DeepSeek-V3.2 Sparse Indexer Kernel API
 * Reference", Notes).  For row r = b*S + t with valid length L (see lk_rows):
 * idx[r*k + j] for j < min(k, L) holds the indices of the min(k, L) largest
 * scores among scores[r*T + 0 .. r*T + L-1]; ties go to the lower index and
 * -0 equals +0.  Slots j >= min(k, L) hold -1.  The set is written as two runs,
 * each in increasing index order: an upper group, then a cut group; every score
 * of the upper group is above every score of the cut group, and within the cut
 * group's lowest score the lower indices are the ones taken.
 * Requires 1 <= k <= T (else LK_E_SHAPE: the reference asks for
 * min(index_topk, end_pos) entries, never more than the row holds) and
 * T <= LK_TOPK_MAX_T (else LK_E_UNSUPPORTED).
 */
LK_API lk_status lk_topk(const float *scores, const lk_rows *rows, int32_t k, int32_t *idx,
                         hipStream_t stream);

/*
 * Sparse MLA decode attention over the indexer's selection (page "Join query parts",
 * the MQA-decode excerpt: scores of the absorbed latent query and the rotary query
 * against the cached latent and rotary rows, the index mask keeping only the top-k
 * slots, softmax, weighted sum of the latent rows).  For sequence b and head h:
 *   s_t = scale * (q_latent[b,h,:] . kv_latent[b,t,:] + q_rope[b,h,:] . kv_rope[b,t,:])
 *   for t in I_b = { idx[b*n_idx + j] : 0 <= idx < cache_rows },
 *   out[b,h,:] = sum_{t in I_b} softmax_t(s) * kv_latent[b,t,:];  zeros if I_b is empty.
 *   q_latent [B][128][512], q_rope [B][128][64]: bf16 bits
 *   kv_latent: row t of sequence b at kv_latent + (b*cache_seq_stride + t)*512 (bf16)
 *   kv_rope:   row t of sequence b at kv_rope + (b*cache_seq_stride + t)*64 (bf16)
 *   idx [B][n_idx] int32: distinct slots; -1 (or any value outside [0, cache_rows))
 *   marks an unused entry, as lk_topk pads its result
 *   out [B][128][512] float32
 *   workspace: device memory of at least lk_sparse_mla_workspace_size(B, n_idx) bytes
 *   (per-split partial results), owned by the caller, contents need no initialisation.
 * Logits and the softmax run in fp32 on bf16 MFMA products; p is rounded to bf16 for
 * the weighted sum (fp32 accumulation).  Requires cache_rows <= cache_seq_stride; all
 * tensors 16-byte aligned except idx (4).  LK_E_SHAPE if the workspace is too small;
 * LK_E_UNSUPPORTED past the launch grid limits: B > 65535, or
 * ceil(n_idx / 256) * B > 4194303 (one 512-thread block per 256 entries and 64 heads).
 */
LK_API size_t lk_sparse_mla_workspace_size(int32_t B, int32_t n_idx);
LK_API lk_status lk_sparse_mla_decode(const uint16_t *q_latent, const uint16_t *q_rope, const uint16_t *kv_latent,
                                      const uint16_t *kv_rope, int64_t cache_seq_stride, int64_t cache_rows,
                                      const int32_t *idx, int32_t B, int32_t n_idx, float scale, float *out,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lk_sparse_mla_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the per-split partials go to a static buffer of
 * LK_MLA_SCRATCH_BYTES (64 MiB) that the library holds on each device from the first
 * use until the process ends.  Arguments and results are those of
 * lk_sparse_mla_decode minus the workspace; the output is the same, bit for bit.
 * LK_E_SCRATCH when lk_sparse_mla_workspace_size(B, n_idx) > LK_MLA_SCRATCH_BYTES
 * (for example B = 16 with n_idx = 2048 needs 33.7 MB and fits; B = 32 does not).
 * The call allocates nothing (no hipMalloc, no hipFree); the buffer's device address
 * is looked up once per device (hipGetSymbolAddress), on the current device, which
 * must be the one `stream` runs on.  Every call on a device shares that device's
 * buffer: calls that overlap on one device (other streams, other threads) race and
 * must be serialised by the caller.  The buffer needs no clearing between calls.
 */
LK_API lk_status lk_sparse_mla_decode_static(const uint16_t *q_latent, const uint16_t *q_rope,
                                             const uint16_t *kv_latent, const uint16_t *kv_rope,
                                             int64_t cache_seq_stride, int64_t cache_rows, const int32_t *idx,
                                             int32_t B, int32_t n_idx, float scale, float *out,
                                             hipStream_t stream);

/*
 * Measurement aids, outside the indexer computation (they serve the benchmark's
 * floors and the accuracy test of the fp8 matrix core; nothing in the hot path calls
 * them):
 *   lk_probe_empty: an empty kernel of `blocks` 64-thread blocks (the fixed cost of
 *     one launch).  LK_E_SHAPE unless 1 <= blocks <= 2^31 / 64.
 *   lk_probe_read: `blocks` 256-thread blocks read the `bytes` at src once (16-byte
 *     loads, contiguous span per block) and write one word per wave to
 *     sink[blocks * 4] (DEVICE).  bytes must be a multiple of 16 (else LK_E_SHAPE).
 *   lk_probe_fp8_mfma_score: lk_index_score for decode rows (S == 1) with the
 *     contraction on the fp8 MFMA (v_mfma_f32_16x16x32_fp8_fp8) instead of exactly
 *     converted f16 operands; arguments as lk_index_score (heads fixed at 64),
 *     LK_E_SHAPE if S > 1.  q_fp8 and k_cache 8-byte aligned.
 */
LK_API lk_status lk_probe_empty(int32_t blocks, hipStream_t stream);
LK_API lk_status lk_probe_read(const void *src, size_t bytes, uint32_t *sink, int32_t blocks,
                               hipStream_t stream);
LK_API lk_status lk_probe_fp8_mfma_score(const uint8_t *q_fp8, const float *w_eff, const uint8_t *k_cache,
                                         const float *k_scale, int64_t cache_seq_stride, const lk_rows *rows,
                                         float *scores, hipStream_t stream);

/*
 * Profiling aid, outside the indexer computation: arm two HIP events for the next
 * kernel that the calling thread launches through an lk_* entry point.  The runtime
 * records `start` when that kernel begins executing and `stop` when it ends
 * (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is the kernel's own
 * duration without queueing gaps.  The next lk_* call consumes the pair whether or
 * not it launches a kernel.  Events are caller-owned (hipEventCreate); LK_E_NULL if
 * either is NULL.  The armed pair is per thread; nothing else is kept.
 */
LK_API lk_status lk_profile_next_launch(hipEvent_t start, hipEvent_t stop);

/* Human-readable name of a status code (static storage). */
LK_API const char *lk_status_string(lk_status s);

/* LK_ABI_VERSION of the built library. */
LK_API int32_t lk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LK_H */
