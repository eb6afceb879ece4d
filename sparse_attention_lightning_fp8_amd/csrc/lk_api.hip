// lk_api.hip -- host side of the C ABI declared in include/lk.h: argument validation
// (before any HIP call) and kernel dispatch on the caller's stream.
#include <stdint.h>

#include "lk_device.h"

namespace lk {
hipError_t launch_quantize(const KeyJobArgs &ka, const QueryJobArgs &qa, hipStream_t stream);
hipError_t launch_index_score(const uint8_t *q_fp8, const float *w_eff, const uint8_t *k_cache,
                              const float *k_scale, int64_t cache_seq_stride, const RowsDev &rows,
                              float *scores, hipStream_t stream);
bool index_score_grid_fits(const RowsDev &rows);
hipError_t launch_topk(const float *scores, const RowsDev &rows, int32_t k, int32_t *idx, hipStream_t stream);
hipError_t launch_decode_score(const uint16_t *q, const float *w, const uint16_t *k_new, uint8_t *k_cache,
                               float *k_scale, int64_t cache_seq_stride, const RowsDev &rows, float *scores,
                               uint8_t *q_fp8_out, float *w_eff_out, const float *rope_cos,
                               const float *rope_sin, hipStream_t stream);
hipError_t launch_decode_select(const uint16_t *q, const float *w, const uint16_t *k_new, uint8_t *k_cache,
                                float *k_scale, int64_t cache_seq_stride, const RowsDev &rows, float *scores,
                                uint8_t *q_fp8_out, float *w_eff_out, const float *rope_cos,
                                const float *rope_sin, int32_t k, int32_t *idx, hipStream_t stream);
hipError_t launch_probe_empty(int32_t blocks, hipStream_t stream);
hipError_t launch_probe_read(const void *src, uint64_t bytes, uint32_t *sink, int32_t blocks, hipStream_t stream);
hipError_t launch_probe_fp8_score(const uint8_t *q_fp8, const float *w_eff, const uint8_t *k_cache,
                                  const float *k_scale, int64_t cache_seq_stride, const RowsDev &rows, float *scores,
                                  hipStream_t stream);
size_t mla_workspace_bytes(int32_t B, int32_t n_idx);
size_t mla_scratch_capacity();
hipError_t launch_sparse_mla_static(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *kv_lat,
                                    const uint16_t *kv_rope, int64_t stride, int64_t cap, const int32_t *idx,
                                    int32_t B, int32_t n_idx, float scale, float *out, hipStream_t stream);
bool mla_grid_fits(int32_t B, int32_t n_idx);
hipError_t launch_sparse_mla(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *kv_lat,
                             const uint16_t *kv_rope, int64_t stride, int64_t cap, const int32_t *idx, int32_t B,
                             int32_t n_idx, float scale, float *out, void *workspace, hipStream_t stream);
}  // namespace lk

namespace lk {
LaunchEvents &armed_events() {
    static thread_local LaunchEvents ev;
    return ev;
}
}  // namespace lk

namespace {

// Every entry point consumes the armed profiling events, launched or not.
struct DisarmOnExit {
    ~DisarmOnExit() { lk::armed_events() = lk::LaunchEvents{}; }
};

constexpr int64_t kMaxGridX = 0x7FFFFFFFLL;
constexpr int64_t kMaxGridYZ = 65535;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

lk_status from_hip(hipError_t e) { return e == hipSuccess ? LK_OK : LK_E_HIP; }

lk_status check_rows(const lk_rows *rows) {
    if (!rows) return LK_E_NULL;
    if (rows->B < 0 || rows->S < 0 || rows->T < 0) return LK_E_SHAPE;
    return LK_OK;
}

lk::RowsDev to_dev(const lk_rows &r) {
    lk::RowsDev d;
    d.B = r.B;
    d.S = r.S;
    d.T = r.T;
    d.start_pos = r.start_pos;
    d.seq_len = r.seq_len;
    d.causal = r.causal;
    return d;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// Validate a key-write request and fill `a` (n_seq == 0 or n_rows == 0: empty job).
lk_status check_keys(const uint16_t *x, int64_t n_seq, int64_t n_rows, int64_t x_seq_stride, uint8_t *cache,
                     float *cache_scale, int64_t cache_seq_stride, int64_t cache_rows, int64_t row_offset,
                     const int32_t *positions, lk::KeyJobArgs &a) {
    if (n_seq < 0 || n_rows < 0 || x_seq_stride < 0 || cache_seq_stride < 0 || cache_rows < 0)
        return LK_E_SHAPE;
    if (cache_rows > cache_seq_stride) return LK_E_SHAPE;
    if (n_seq == 0 || n_rows == 0) return LK_OK;
    if (!x || !cache || !cache_scale) return LK_E_NULL;
    if (!aligned(x, 16) || !aligned(cache, 16) || !aligned(cache_scale, 4) || !aligned(positions, 4))
        return LK_E_UNSUPPORTED;
    if (n_rows > INT64_MAX / n_seq || (n_seq * n_rows + 31) / 32 > kMaxGridX / 2) return LK_E_UNSUPPORTED;
    // A host-known destination must fit the cache; device positions are checked per row
    // by the kernel, which skips rows outside [0, cache_rows).
    if (!positions && (row_offset < 0 || row_offset > cache_rows - n_rows)) return LK_E_SHAPE;
    a = lk::KeyJobArgs{x, n_seq, n_rows, x_seq_stride, cache, cache_scale, cache_seq_stride, cache_rows,
                       row_offset, positions};
    return LK_OK;
}

// Validate a query request and fill `a` (n_tokens == 0: empty job).
lk_status check_queries(const uint16_t *q, const float *w, int64_t n_tokens, int32_t heads, uint8_t *q_fp8,
                        float *w_eff, float *q_scale, lk::QueryJobArgs &a) {
    if (n_tokens < 0 || heads < 1) return LK_E_SHAPE;
    if (n_tokens == 0) return LK_OK;
    if (!q || !w || !q_fp8 || !w_eff) return LK_E_NULL;
    if (!aligned(q, 16) || !aligned(q_fp8, 16) || !aligned(w, 4) || !aligned(w_eff, 4) || !aligned(q_scale, 4))
        return LK_E_UNSUPPORTED;
    if (n_tokens > INT64_MAX / heads) return LK_E_UNSUPPORTED;
    const int64_t n_rows = n_tokens * heads;
    if ((n_rows + 31) / 32 > kMaxGridX / 2) return LK_E_UNSUPPORTED;
    a = lk::QueryJobArgs{q, w, n_rows, q_fp8, w_eff, q_scale, heads};
    return LK_OK;
}

// Optional RoPE tables: both or neither, 16-byte aligned.
lk_status check_rope(const float *c, const float *s) {
    if ((c == nullptr) != (s == nullptr)) return LK_E_NULL;
    if (!aligned(c, 16) || !aligned(s, 16)) return LK_E_UNSUPPORTED;
    return LK_OK;
}

lk_status run_quantize(const lk::KeyJobArgs &ka, const lk::QueryJobArgs &qa, hipStream_t stream) {
    if (ka.n_seq * ka.n_rows == 0 && qa.n_rows == 0) return LK_OK;
    return from_hip(lk::launch_quantize(ka, qa, stream));
}

}  // namespace

extern "C" {

LK_API lk_status lk_quantize_keys(const uint16_t *x, int64_t n_seq, int64_t n_rows, int64_t x_seq_stride,
                                  uint8_t *cache, float *cache_scale, int64_t cache_seq_stride,
                                  int64_t cache_rows, int64_t row_offset, const int32_t *positions,
                                  hipStream_t stream) {
    DisarmOnExit disarm;
    lk::KeyJobArgs ka;
    lk_status st = check_keys(x, n_seq, n_rows, x_seq_stride, cache, cache_scale, cache_seq_stride, cache_rows,
                              row_offset, positions, ka);
    if (st != LK_OK) return st;
    return run_quantize(ka, lk::QueryJobArgs{}, stream);
}

LK_API lk_status lk_quantize_queries(const uint16_t *q, const float *w, int64_t n_tokens, int32_t heads,
                                     uint8_t *q_fp8, float *w_eff, float *q_scale, hipStream_t stream) {
    DisarmOnExit disarm;
    lk::QueryJobArgs qa;
    lk_status st = check_queries(q, w, n_tokens, heads, q_fp8, w_eff, q_scale, qa);
    if (st != LK_OK) return st;
    return run_quantize(lk::KeyJobArgs{}, qa, stream);
}

LK_API lk_status lk_prepare(const uint16_t *x, int64_t n_seq, int64_t n_rows, int64_t x_seq_stride,
                            uint8_t *cache, float *cache_scale, int64_t cache_seq_stride, int64_t cache_rows,
                            int64_t row_offset, const int32_t *positions, const uint16_t *q, const float *w,
                            int64_t n_tokens, int32_t heads, uint8_t *q_fp8, float *w_eff, float *q_scale,
                            const float *k_rope_cos, const float *k_rope_sin, const float *q_rope_cos,
                            const float *q_rope_sin, hipStream_t stream) {
    DisarmOnExit disarm;
    lk::KeyJobArgs ka;
    lk::QueryJobArgs qa;
    lk_status st = check_keys(x, n_seq, n_rows, x_seq_stride, cache, cache_scale, cache_seq_stride, cache_rows,
                              row_offset, positions, ka);
    if (st != LK_OK) return st;
    st = check_queries(q, w, n_tokens, heads, q_fp8, w_eff, q_scale, qa);
    if (st != LK_OK) return st;
    st = check_rope(k_rope_cos, k_rope_sin);
    if (st != LK_OK) return st;
    st = check_rope(q_rope_cos, q_rope_sin);
    if (st != LK_OK) return st;
    ka.rope_cos = k_rope_cos;
    ka.rope_sin = k_rope_sin;
    qa.rope_cos = q_rope_cos;
    qa.rope_sin = q_rope_sin;
    return run_quantize(ka, qa, stream);
}

LK_API lk_status lk_index_score(const uint8_t *q_fp8, const float *w_eff, int32_t heads,
                                const uint8_t *k_cache, const float *k_scale, int64_t cache_seq_stride,
                                const lk_rows *rows, float *scores, hipStream_t stream) {
    DisarmOnExit disarm;
    lk_status st = check_rows(rows);
    if (st != LK_OK) return st;
    if (cache_seq_stride < 0 || rows->T > cache_seq_stride) return LK_E_SHAPE;
    if (heads != LK_HEADS) return LK_E_UNSUPPORTED;
    if (rows->B == 0 || rows->S == 0 || rows->T == 0) return LK_OK;
    if (!q_fp8 || !w_eff || !k_cache || !k_scale || !scores) return LK_E_NULL;
    if (!aligned(q_fp8, 16) || !aligned(w_eff, 16) || !aligned(k_cache, 16) || !aligned(k_scale, 4) ||
        !aligned(scores, 4) || !aligned(rows->seq_len, 4))
        return LK_E_UNSUPPORTED;
    if (rows->T > kMaxGridX || !lk::index_score_grid_fits(to_dev(*rows))) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_index_score(q_fp8, w_eff, k_cache, k_scale, cache_seq_stride, to_dev(*rows),
                                           scores, stream));
}

LK_API lk_status lk_decode_score(const uint16_t *q, const float *w, int32_t heads, const uint16_t *k_new,
                                 uint8_t *k_cache, float *k_scale, int64_t cache_seq_stride,
                                 const lk_rows *rows, float *scores, uint8_t *q_fp8_out,
                                 float *w_eff_out, const float *rope_cos, const float *rope_sin,
                                 hipStream_t stream) {
    DisarmOnExit disarm;
    lk_status st = check_rows(rows);
    if (st != LK_OK) return st;
    st = check_rope(rope_cos, rope_sin);
    if (st != LK_OK) return st;
    if (cache_seq_stride < 0 || rows->T > cache_seq_stride) return LK_E_SHAPE;
    if (rows->S > 1) return LK_E_SHAPE;
    if (heads != LK_HEADS) return LK_E_UNSUPPORTED;
    if ((q_fp8_out == nullptr) != (w_eff_out == nullptr)) return LK_E_NULL;
    if (rows->B == 0 || rows->S == 0 || rows->T == 0) return LK_OK;
    if (!q || !w || !k_new || !k_cache || !k_scale || !scores) return LK_E_NULL;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(k_cache, 16) || !aligned(q_fp8_out, 16) ||
        !aligned(w, 4) || !aligned(w_eff_out, 4) || !aligned(k_scale, 4) || !aligned(scores, 4) ||
        !aligned(rows->seq_len, 4))
        return LK_E_UNSUPPORTED;
    if (rows->B > kMaxGridYZ || rows->T > kMaxGridX) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_decode_score(q, w, k_new, k_cache, k_scale, cache_seq_stride, to_dev(*rows), scores,
                                            q_fp8_out, w_eff_out, rope_cos, rope_sin, stream));
}

LK_API lk_status lk_decode_select(const uint16_t *q, const float *w, int32_t heads, const uint16_t *k_new,
                                  uint8_t *k_cache, float *k_scale, int64_t cache_seq_stride,
                                  const lk_rows *rows, float *scores, uint8_t *q_fp8_out, float *w_eff_out,
                                  const float *rope_cos, const float *rope_sin, int32_t k, int32_t *idx,
                                  hipStream_t stream) {
    DisarmOnExit disarm;
    lk_status st = check_rows(rows);
    if (st != LK_OK) return st;
    st = check_rope(rope_cos, rope_sin);
    if (st != LK_OK) return st;
    if (cache_seq_stride < 0 || rows->T > cache_seq_stride) return LK_E_SHAPE;
    if (rows->S > 1) return LK_E_SHAPE;
    if (k < 1 || k > rows->T) return LK_E_SHAPE;
    if (heads != LK_HEADS) return LK_E_UNSUPPORTED;
    if (rows->T > LK_TOPK_MAX_T) return LK_E_UNSUPPORTED;
    if ((q_fp8_out == nullptr) != (w_eff_out == nullptr)) return LK_E_NULL;
    if (rows->B == 0 || rows->S == 0) return LK_OK;
    if (!q || !w || !k_new || !k_cache || !k_scale || !idx) return LK_E_NULL;
    if (!scores && rows->T > LK_SELECT_FUSED_MAX_T) return LK_E_NULL;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(k_cache, 16) || !aligned(q_fp8_out, 16) ||
        !aligned(w, 4) || !aligned(w_eff_out, 4) || !aligned(k_scale, 4) || !aligned(scores, 4) ||
        !aligned(idx, 4) || !aligned(rows->seq_len, 4))
        return LK_E_UNSUPPORTED;
    if (rows->B > kMaxGridYZ || rows->T > kMaxGridX) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_decode_select(q, w, k_new, k_cache, k_scale, cache_seq_stride, to_dev(*rows), scores,
                                             q_fp8_out, w_eff_out, rope_cos, rope_sin, k, idx, stream));
}

LK_API lk_status lk_topk(const float *scores, const lk_rows *rows, int32_t k, int32_t *idx, hipStream_t stream) {
    DisarmOnExit disarm;
    lk_status st = check_rows(rows);
    if (st != LK_OK) return st;
    if (k < 1 || k > rows->T) return LK_E_SHAPE;
    if (rows->T > LK_TOPK_MAX_T) return LK_E_UNSUPPORTED;
    if (rows->B == 0 || rows->S == 0) return LK_OK;
    if (!scores || !idx) return LK_E_NULL;
    if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(rows->seq_len, 4)) return LK_E_UNSUPPORTED;
    if ((int64_t)rows->B * rows->S > kMaxGridX) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_topk(scores, to_dev(*rows), k, idx, stream));
}

LK_API size_t lk_sparse_mla_workspace_size(int32_t B, int32_t n_idx) {
    if (B <= 0 || n_idx <= 0) return 0;
    return lk::mla_workspace_bytes(B, n_idx);
}

LK_API lk_status lk_sparse_mla_decode(const uint16_t *q_latent, const uint16_t *q_rope, const uint16_t *kv_latent,
                                      const uint16_t *kv_rope, int64_t cache_seq_stride, int64_t cache_rows,
                                      const int32_t *idx, int32_t B, int32_t n_idx, float scale, float *out,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    DisarmOnExit disarm;
    if (B < 0 || n_idx < 0 || cache_seq_stride < 0 || cache_rows < 0) return LK_E_SHAPE;
    if (cache_rows > cache_seq_stride) return LK_E_SHAPE;
    if (B == 0) return LK_OK;
    if (!q_latent || !q_rope || !out || (n_idx > 0 && (!kv_latent || !kv_rope || !idx || !workspace)))
        return LK_E_NULL;
    if (workspace_bytes < lk_sparse_mla_workspace_size(B, n_idx)) return LK_E_SHAPE;
    if (!aligned(q_latent, 16) || !aligned(q_rope, 16) || !aligned(kv_latent, 16) || !aligned(kv_rope, 16) ||
        !aligned(out, 16) || !aligned(workspace, 16) || !aligned(idx, 4))
        return LK_E_UNSUPPORTED;
    if (B > kMaxGridYZ || !lk::mla_grid_fits(B, n_idx)) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_sparse_mla(q_latent, q_rope, kv_latent, kv_rope, cache_seq_stride, cache_rows, idx, B,
                                          n_idx, scale, out, workspace, stream));
}

LK_API lk_status lk_sparse_mla_decode_static(const uint16_t *q_latent, const uint16_t *q_rope,
                                             const uint16_t *kv_latent, const uint16_t *kv_rope,
                                             int64_t cache_seq_stride, int64_t cache_rows, const int32_t *idx,
                                             int32_t B, int32_t n_idx, float scale, float *out,
                                             hipStream_t stream) {
    DisarmOnExit disarm;
    if (B < 0 || n_idx < 0 || cache_seq_stride < 0 || cache_rows < 0) return LK_E_SHAPE;
    if (cache_rows > cache_seq_stride) return LK_E_SHAPE;
    if (B == 0) return LK_OK;
    if (!q_latent || !q_rope || !out || (n_idx > 0 && (!kv_latent || !kv_rope || !idx))) return LK_E_NULL;
    if (!aligned(q_latent, 16) || !aligned(q_rope, 16) || !aligned(kv_latent, 16) || !aligned(kv_rope, 16) ||
        !aligned(out, 16) || !aligned(idx, 4))
        return LK_E_UNSUPPORTED;
    if (B > kMaxGridYZ || !lk::mla_grid_fits(B, n_idx)) return LK_E_UNSUPPORTED;
    if (lk_sparse_mla_workspace_size(B, n_idx) > lk::mla_scratch_capacity()) return LK_E_SCRATCH;
    return from_hip(lk::launch_sparse_mla_static(q_latent, q_rope, kv_latent, kv_rope, cache_seq_stride, cache_rows,
                                                 idx, B, n_idx, scale, out, stream));
}

LK_API lk_status lk_probe_empty(int32_t blocks, hipStream_t stream) {
    DisarmOnExit disarm;
    if (blocks < 1 || blocks > kMaxGridX / 64) return LK_E_SHAPE;
    return from_hip(lk::launch_probe_empty(blocks, stream));
}

LK_API lk_status lk_probe_read(const void *src, size_t bytes, uint32_t *sink, int32_t blocks, hipStream_t stream) {
    DisarmOnExit disarm;
    if (blocks < 1 || blocks > kMaxGridX / 256 || bytes % 16 != 0) return LK_E_SHAPE;
    if (bytes == 0) return LK_OK;
    if (!src || !sink) return LK_E_NULL;
    if (!aligned(src, 16) || !aligned(sink, 4)) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_probe_read(src, (uint64_t)bytes, sink, blocks, stream));
}

LK_API lk_status lk_probe_fp8_mfma_score(const uint8_t *q_fp8, const float *w_eff, const uint8_t *k_cache,
                                         const float *k_scale, int64_t cache_seq_stride, const lk_rows *rows,
                                         float *scores, hipStream_t stream) {
    DisarmOnExit disarm;
    lk_status st = check_rows(rows);
    if (st != LK_OK) return st;
    if (cache_seq_stride < 0 || rows->T > cache_seq_stride || rows->S > 1) return LK_E_SHAPE;
    if (rows->B == 0 || rows->S == 0 || rows->T == 0) return LK_OK;
    if (!q_fp8 || !w_eff || !k_cache || !k_scale || !scores) return LK_E_NULL;
    if (!aligned(q_fp8, 8) || !aligned(k_cache, 8) || !aligned(w_eff, 4) || !aligned(k_scale, 4) ||
        !aligned(scores, 4) || !aligned(rows->seq_len, 4))
        return LK_E_UNSUPPORTED;
    if (rows->B > kMaxGridYZ || (rows->T + 63) / 64 > kMaxGridX) return LK_E_UNSUPPORTED;
    return from_hip(lk::launch_probe_fp8_score(q_fp8, w_eff, k_cache, k_scale, cache_seq_stride, to_dev(*rows),
                                               scores, stream));
}

LK_API lk_status lk_profile_next_launch(hipEvent_t start, hipEvent_t stop) {
    if (!start || !stop) return LK_E_NULL;
    lk::armed_events() = lk::LaunchEvents{start, stop};
    return LK_OK;
}

LK_API const char *lk_status_string(lk_status s) {
    switch (s) {
    case LK_OK: return "LK_OK";
    case LK_E_NULL: return "LK_E_NULL: a required pointer is NULL";
    case LK_E_SHAPE: return "LK_E_SHAPE: sizes are negative or do not fit together";
    case LK_E_UNSUPPORTED: return "LK_E_UNSUPPORTED: outside what this library implements (heads, row length, alignment or grid limits)";
    case LK_E_HIP: return "LK_E_HIP: the HIP runtime rejected a kernel launch";
    case LK_E_SCRATCH: return "LK_E_SCRATCH: the request needs more workspace than the static scratch buffer (LK_MLA_SCRATCH_BYTES) holds";
    }
    return "unknown lk_status";
}

LK_API int32_t lk_abi_version(void) { return LK_ABI_VERSION; }

}  // extern "C"
