// C ABI of liblrkv.so: host-side validation, workspace sizing and dispatch.
// Every check runs before anything is enqueued; a failing call touches no
// device memory. The library allocates nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "common.h"

namespace lrkv {

bool latent_shape_supported(int mode, const LatentGeom& g);

LatentGeom latent_geom(const lrkv_latent_cache* c) {
    LatentGeom g;
    g.B = c->batch;
    g.U = c->units;
    g.s = c->kv_per_unit;
    g.gq = c->q_per_kv;
    g.dh = c->head_dim;
    g.r = c->rank;
    g.cap = c->capacity;
    g.fmt = c->fmt;
    g.theta = c->rope_theta;
    g.Hq = c->units * c->kv_per_unit * c->q_per_kv;
    return g;
}

// Chunking of the sequence: enough workgroups to cover the 256 compute units
// a couple of times, chunks a multiple of the 32-token tile. `cap_split` is an
// upper bound of the split count for every length <= host_max_len, so that a
// workspace sized for one length also serves every shorter one.
static void pick_split(int per_split_groups, int host_max_len, int n_split, int target,
                       int max_chunk_tiles, int* out_split, int* out_chunk, int* cap_split) {
    const int tiles = (host_max_len + kTile - 1) / kTile;
    if (n_split <= 0) n_split = (target + per_split_groups - 1) / per_split_groups;
    const int min_split = (tiles + max_chunk_tiles - 1) / max_chunk_tiles;
    if (n_split < min_split) n_split = min_split;
    if (n_split > kMaxSplit) n_split = kMaxSplit;
    if (n_split > tiles) n_split = tiles;
    if (n_split < 1) n_split = 1;
    const int chunk_tiles = (tiles + n_split - 1) / n_split;
    *out_chunk = chunk_tiles * kTile;
    *out_split = (tiles + chunk_tiles - 1) / chunk_tiles;
    *cap_split = n_split;
}

LatentWorkspace latent_workspace(int mode, const LatentGeom& g, int host_max_len, int n_split) {
    LatentWorkspace w;
    // RoPE: ~256 (chunk, unit, sequence) groups at rank 256 (one workgroup per CU),
    // more for the smaller ranks, whose tiles carry less work each and need more
    // workgroups in flight; absorbed: ~1024 workgroups of 4 independent waves
    // the grouped-query RoPE kernel: one chunk per wave, two waves per SIMD
    int target = mode == LRKV_MODE_ROPE_RECON ? (g.r >= 256 ? 256 : g.r >= 128 ? 512 : 1024) : 1024;
    if (mode == LRKV_MODE_ROPE_RECON && use_gqa_kernel(g)) target = 2048;
    int cap_split = 1;
    const int max_chunk_tiles = mode == LRKV_MODE_ROPE_RECON ? kMaxRopeTiles : 1 << 30;
    pick_split(g.B * g.U, host_max_len, n_split, target, max_chunk_tiles, &w.n_split, &w.chunk,
               &cap_split);
    size_t off = 0;
    w.part_off = off;
    off += align_up((size_t)g.B * g.Hq * cap_split * (g.r + 2) * sizeof(float), 256);
    w.qp_off = off;
    w.qs_off = off;
    w.ang_off = off;
    if (mode == LRKV_MODE_ROPE_RECON) {
        off += align_up((size_t)g.B * g.Hq * g.dh * g.r * sizeof(half_t), 256);
        w.qs_off = off;
        off += align_up((size_t)g.B * g.U * (g.dh / 2) * sizeof(float), 256);
        w.ang_off = off;
        off += align_up((size_t)(33 + g.B * cap_split) * (g.dh / 2) * 2 * sizeof(float), 256);
    }
    w.total = off;
    return w;
}

PagedWorkspace paged_workspace(const lrkv_paged_cache* c, int host_max_len, int n_split) {
    PagedWorkspace w;
    int npg = (host_max_len + c->page_size - 1) / c->page_size;
    if (npg > c->max_pages) npg = c->max_pages;
    const int groups = c->batch * c->kv_heads;
    // default chunking, a wave taking at most 64 pages: with fp16 page factors
    // about one wave per SIMD, with int4 factors two (each measured the faster on
    // 8 sequences x 8 KV heads at 32K tokens: 105 vs 110 us and 65 vs 72 us)
    if (n_split <= 0) {
        const int waves = c->factor_fmt == LRKV_FMT_INT4_G32 ? 2048 : 1024;
        n_split = (waves + groups - 1) / groups;
    }
    if (n_split < (npg + 63) / 64) n_split = (npg + 63) / 64;
    if (n_split > kMaxSplit) n_split = kMaxSplit;
    if (n_split > npg) n_split = npg;
    if (n_split < 1) n_split = 1;
    w.pages_per_split = (npg + n_split - 1) / n_split;
    w.n_split = (npg + w.pages_per_split - 1) / w.pages_per_split;
    w.part_off = 0;
    w.total = align_up((size_t)c->batch * c->kv_heads * c->q_per_kv * n_split *
                           (c->head_dim + 2) * sizeof(float), 256);
    return w;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int32_t check_latent(const lrkv_latent_cache* c) {
    if (!c) return LRKV_ERR_INVALID_ARG;
    if (c->batch < 1 || c->units < 1 || c->kv_per_unit < 1 || c->q_per_kv < 1 ||
        c->head_dim < 2 || (c->head_dim & 1) || c->rank < 8 || (c->rank % 8) ||
        c->capacity < kTile || (c->capacity % kTile))
        return LRKV_ERR_INVALID_ARG;
    if (c->fmt != LRKV_FMT_FP16 && c->fmt != LRKV_FMT_INT4_G32) return LRKV_ERR_INVALID_ARG;
    if (!(c->rope_theta >= 0.0f) || !isfinite(c->rope_theta)) return LRKV_ERR_INVALID_ARG;
    if (!c->hk || !c->hv || !c->lens) return LRKV_ERR_INVALID_ARG;
    if (!aligned16(c->hk) || !aligned16(c->hv)) return LRKV_ERR_INVALID_ARG;
    if (c->fmt == LRKV_FMT_INT4_G32) {
        if (!c->sk || !c->sv) return LRKV_ERR_INVALID_ARG;
        if (c->rank % 32) return LRKV_ERR_UNSUPPORTED;
    }
    if ((long)c->batch * c->units * (long)c->capacity * c->rank > (1L << 40)) return LRKV_ERR_INVALID_ARG;
    return LRKV_OK;
}

static int32_t check_paged(const lrkv_paged_cache* c) {
    if (!c) return LRKV_ERR_INVALID_ARG;
    if (c->batch < 1 || c->kv_heads < 1 || c->q_per_kv < 1 || c->head_dim < 8 ||
        c->page_size < 1 || c->sink_pages < 0 || c->window_pages < 1 || c->rank_k < 1 ||
        c->rank_v < 1 || c->max_pages < 1)
        return LRKV_ERR_INVALID_ARG;
    if (!c->dense_k || !c->dense_v || !c->lk || !c->rk || !c->lv || !c->rv || !c->page_table ||
        !c->lens)
        return LRKV_ERR_INVALID_ARG;
    if (c->head_dim != 128 || c->page_size != 32 || c->q_per_kv > 16 || c->rank_k > 32 ||
        c->rank_v > 32 || (c->rank_k % 4) || (c->rank_v % 4))
        return LRKV_ERR_UNSUPPORTED;
    // one (sequence, head)'s factor arrays are addressed with 32-bit byte offsets
    if ((size_t)c->max_pages * 32 * 128 * 2 >= ((size_t)1 << 31)) return LRKV_ERR_UNSUPPORTED;
    if (c->max_pages > 64 * kMaxSplit) return LRKV_ERR_UNSUPPORTED;
    if (!aligned16(c->dense_k) || !aligned16(c->dense_v) || !aligned16(c->rk) || !aligned16(c->rv))
        return LRKV_ERR_INVALID_ARG;
    if (c->factor_fmt != LRKV_FMT_FP16 && c->factor_fmt != LRKV_FMT_INT4_G32) return LRKV_ERR_INVALID_ARG;
    if (c->factor_fmt == LRKV_FMT_INT4_G32 && (!c->lk_s || !c->rk_s || !c->lv_s || !c->rv_s))
        return LRKV_ERR_INVALID_ARG;
    if (c->factor_fmt == LRKV_FMT_INT4_G32 && (c->rank_k > 16 || c->rank_v > 16)) return LRKV_ERR_UNSUPPORTED;
    // int4 factor codes are written as 16-byte groups
    if (c->factor_fmt == LRKV_FMT_INT4_G32 && (!aligned16(c->lk) || !aligned16(c->lv))) return LRKV_ERR_INVALID_ARG;
    return LRKV_OK;
}

}  // namespace lrkv

using namespace lrkv;

// Every check lrkv_append_latent makes before it enqueues anything.
static int32_t check_append(int32_t mode, const void* cache, const void* new_k, const void* new_v,
                            int32_t n_new, int32_t host_max_len) {
    if (!cache || !new_k || !new_v || n_new < 1 || host_max_len < 0) return LRKV_ERR_INVALID_ARG;
    if (!aligned16(new_k) || !aligned16(new_v)) return LRKV_ERR_INVALID_ARG;
    if (mode == LRKV_MODE_HYBRID_PAGED) {
        const lrkv_paged_cache* c = (const lrkv_paged_cache*)cache;
        int32_t rc = check_paged(c);
        if (rc != LRKV_OK) return rc;
        if ((long)host_max_len + n_new > (long)c->max_pages * c->page_size) return LRKV_ERR_CAPACITY;
        return LRKV_OK;
    }
    if (mode != LRKV_MODE_ROPE_RECON && mode != LRKV_MODE_ABSORBED) return LRKV_ERR_INVALID_ARG;
    const lrkv_latent_cache* c = (const lrkv_latent_cache*)cache;
    int32_t rc = check_latent(c);
    if (rc != LRKV_OK) return rc;
    if ((long)host_max_len + n_new > c->capacity) return LRKV_ERR_CAPACITY;
    return LRKV_OK;
}

extern "C" {

const char* lrkv_status_string(int32_t s) {
    switch (s) {
        case LRKV_OK: return "ok";
        case LRKV_ERR_INVALID_ARG: return "invalid argument";
        case LRKV_ERR_UNSUPPORTED: return "unsupported shape or format";
        case LRKV_ERR_CAPACITY: return "cache capacity exceeded";
        case LRKV_ERR_WORKSPACE: return "workspace missing or too small";
        case LRKV_ERR_HIP: return "HIP error";
        case LRKV_ERR_SCRATCH: return "call needs more than the no-allocation entry point's static scratch";
        default: return "unknown status";
    }
}

int32_t lrkv_version(void) { return 100; }

size_t lrkv_decode_workspace_bytes(int32_t mode, const void* cache, int32_t host_max_len,
                                   int32_t n_split) {
    if (host_max_len < 1) return 0;
    if (mode == LRKV_MODE_HYBRID_PAGED) {
        const lrkv_paged_cache* c = (const lrkv_paged_cache*)cache;
        if (check_paged(c) != LRKV_OK) return 0;
        if (host_max_len > c->max_pages * c->page_size) return 0;
        return paged_workspace(c, host_max_len, n_split).total;
    }
    if (mode != LRKV_MODE_ROPE_RECON && mode != LRKV_MODE_ABSORBED) return 0;
    const lrkv_latent_cache* c = (const lrkv_latent_cache*)cache;
    if (check_latent(c) != LRKV_OK) return 0;
    if (host_max_len > c->capacity) return 0;
    return latent_workspace(mode, latent_geom(c), host_max_len, n_split).total;
}

int32_t lrkv_append_latent(int32_t mode, const void* cache, const void* new_k, const void* new_v,
                           int32_t n_new, int32_t host_max_len, void* stream) {
    const int32_t rc = check_append(mode, cache, new_k, new_v, n_new, host_max_len);
    if (rc != LRKV_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (mode == LRKV_MODE_HYBRID_PAGED)
        return launch_append_paged((const lrkv_paged_cache*)cache, (const half_t*)new_k, (const half_t*)new_v,
                                   n_new, st);
    return launch_append_latent((const lrkv_latent_cache*)cache, (const float*)new_k, (const float*)new_v,
                                n_new, st);
}

}  // extern "C"

// Shared validation and dispatch of the decode entry points. `phases` selects
// which of prepare / partials / merge are enqueued; the pointers each phase
// needs are checked here. With `ws_need` non-null nothing is enqueued: after the
// argument checks the workspace size the call needs is stored there.
int32_t lrkv::decode_common(int32_t mode, int phases, const void* cache, const float* q,
                             const void* bk, const int32_t* q_pos, float sm_scale, float* out,
                             void* workspace, size_t ws_bytes, int32_t host_max_len, int32_t n_split,
                             void* stream, size_t* ws_need, const FusedAppend* app) {
    if (!cache || host_max_len < 1) return LRKV_ERR_INVALID_ARG;
    if ((phases & kPhaseMerge) && !out) return LRKV_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (mode == LRKV_MODE_HYBRID_PAGED) {
        const lrkv_paged_cache* c = (const lrkv_paged_cache*)cache;
        int32_t rc = check_paged(c);
        if (rc != LRKV_OK) return rc;
        if (bk || q_pos) return LRKV_ERR_INVALID_ARG;
        if ((phases & kPhasePartials) && !q) return LRKV_ERR_INVALID_ARG;
        if (host_max_len > c->max_pages * c->page_size) return LRKV_ERR_INVALID_ARG;
        const PagedWorkspace w = paged_workspace(c, host_max_len, n_split);
        if (ws_need) {
            *ws_need = w.total;
            return LRKV_OK;
        }
        if (!workspace || ws_bytes < w.total || !aligned16(workspace)) return LRKV_ERR_WORKSPACE;
        const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)c->head_dim);
        return launch_decode_hybrid(phases, c, q, scale, out, workspace, w, st);
    }
    if (mode != LRKV_MODE_ROPE_RECON && mode != LRKV_MODE_ABSORBED) return LRKV_ERR_INVALID_ARG;
    const lrkv_latent_cache* c = (const lrkv_latent_cache*)cache;
    int32_t rc = check_latent(c);
    if (rc != LRKV_OK) return rc;
    if (host_max_len > c->capacity) return LRKV_ERR_INVALID_ARG;
    if (mode == LRKV_MODE_ROPE_RECON) {
        if ((phases & kPhasePrepare) && (!bk || !q)) return LRKV_ERR_INVALID_ARG;
    } else {
        if (bk || q_pos) return LRKV_ERR_INVALID_ARG;
        if ((phases & kPhasePartials) && !q) return LRKV_ERR_INVALID_ARG;
    }
    const LatentGeom g = latent_geom(c);
    if (g.r % 32) return LRKV_ERR_UNSUPPORTED;
    if (!latent_shape_supported(mode, g)) return LRKV_ERR_UNSUPPORTED;
    const LatentWorkspace w = latent_workspace(mode, g, host_max_len, n_split);
    if (ws_need) {
        *ws_need = w.total;
        return LRKV_OK;
    }
    if (!workspace || ws_bytes < w.total || !aligned16(workspace)) return LRKV_ERR_WORKSPACE;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)c->head_dim);
    return launch_decode_latent(mode, phases, c, q, (const half_t*)bk, q_pos, scale, out, workspace,
                                w, st, app);
}

extern "C" {

int32_t lrkv_decode_attn(int32_t mode, const void* cache, const float* q, const void* bk,
                         const int32_t* q_pos, float sm_scale, float* out, void* workspace,
                         size_t ws_bytes, int32_t host_max_len, int32_t n_split, void* stream) {
    if (!q) return LRKV_ERR_INVALID_ARG;
    return decode_common(mode, kPhaseAll, cache, q, bk, q_pos, sm_scale, out, workspace, ws_bytes,
                         host_max_len, n_split, stream);
}

int32_t lrkv_decode_step(int32_t mode, const void* cache, const void* new_k, const void* new_v,
                         int32_t n_new, const float* q, const void* bk, const int32_t* q_pos,
                         float sm_scale, float* out, void* workspace, size_t ws_bytes,
                         int32_t host_max_len, int32_t n_split, void* stream) {
    // both halves validated before anything is enqueued
    int32_t rc = check_append(mode, cache, new_k, new_v, n_new, host_max_len);
    if (rc != LRKV_OK) return rc;
    if (!q) return LRKV_ERR_INVALID_ARG;
    const int32_t len_after = host_max_len + n_new;
    size_t need = 0;
    rc = decode_common(mode, kPhaseAll, cache, q, bk, q_pos, sm_scale, out, workspace, ws_bytes, len_after,
                       n_split, stream, &need);
    if (rc != LRKV_OK) return rc;
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return LRKV_ERR_WORKSPACE;
    if (mode == LRKV_MODE_ROPE_RECON) {
        const lrkv_latent_cache* c = (const lrkv_latent_cache*)cache;
        if (fused_append_fits(c, n_new)) {
            const FusedAppend app{(const float*)new_k, (const float*)new_v, n_new};
            return decode_common(mode, kPhaseAll, cache, q, bk, q_pos, sm_scale, out, workspace, ws_bytes,
                                 len_after, n_split, stream, nullptr, &app);
        }
    }
    rc = lrkv_append_latent(mode, cache, new_k, new_v, n_new, host_max_len, stream);
    if (rc != LRKV_OK) return rc;
    return decode_common(mode, kPhaseAll, cache, q, bk, q_pos, sm_scale, out, workspace, ws_bytes, len_after,
                         n_split, stream);
}

int32_t lrkv_decode_prepare(int32_t mode, const void* cache, const float* q, const void* bk,
                            const int32_t* q_pos, float sm_scale, void* workspace, size_t ws_bytes,
                            int32_t host_max_len, int32_t n_split, void* stream) {
    return decode_common(mode, kPhasePrepare, cache, q, bk, q_pos, sm_scale, nullptr, workspace,
                         ws_bytes, host_max_len, n_split, stream);
}

int32_t lrkv_decode_partials(int32_t mode, const void* cache, const float* q, float sm_scale,
                             void* workspace, size_t ws_bytes, int32_t host_max_len,
                             int32_t n_split, void* stream) {
    return decode_common(mode, kPhasePartials, cache, q, nullptr, nullptr, sm_scale, nullptr,
                         workspace, ws_bytes, host_max_len, n_split, stream);
}

int32_t lrkv_merge_partials(int32_t mode, const void* cache, float* out, void* workspace,
                            size_t ws_bytes, int32_t host_max_len, int32_t n_split, void* stream) {
    return decode_common(mode, kPhaseMerge, cache, nullptr, nullptr, nullptr, 0.0f, out, workspace,
                         ws_bytes, host_max_len, n_split, stream);
}

int32_t lrkv_factor_page(const lrkv_paged_cache* cache, const int32_t* pages, int32_t n_pages,
                         const void* src_k, const void* src_v, int32_t src_len,
                         int32_t max_sweeps, void* stream) {
    int32_t rc = check_paged(cache);
    if (rc != LRKV_OK) return rc;
    if (n_pages < 0 || (n_pages > 0 && !pages)) return LRKV_ERR_INVALID_ARG;
    if ((src_k == nullptr) != (src_v == nullptr)) return LRKV_ERR_INVALID_ARG;
    if (src_k && (src_len < cache->page_size || !aligned16(src_k) || !aligned16(src_v)))
        return LRKV_ERR_INVALID_ARG;
    if (max_sweeps <= 0) max_sweeps = 15;
    if (max_sweeps > 100) return LRKV_ERR_INVALID_ARG;
    return launch_factor_page(cache, pages, n_pages, (const half_t*)src_k, (const half_t*)src_v,
                              src_k ? src_len : 0, max_sweeps, (hipStream_t)stream);
}

int32_t lrkv_paged_plan(const lrkv_paged_cache* c, const int32_t* host_lens, int32_t n_new,
                        int32_t* out, int32_t max_out) {
    int32_t rc = check_paged(c);
    if (rc != LRKV_OK) return rc;
    if (!host_lens || n_new < 0 || max_out < 0 || (max_out > 0 && !out)) return LRKV_ERR_INVALID_ARG;
    const long P = c->page_size;
    long count = 0;
    for (int b = 0; b < c->batch; ++b) {
        const long len = host_lens[b];
        if (len < 0 || len + n_new > (long)c->max_pages * P) return LRKV_ERR_INVALID_ARG;
        // pages factored at length n: sink <= p < ceil(n / P) - window
        const long before = (len + P - 1) / P - c->window_pages;
        const long after = (len + n_new + P - 1) / P - c->window_pages;
        const long lo = before > c->sink_pages ? before : c->sink_pages;
        for (int h = 0; h < c->kv_heads; ++h) {
            for (long p = lo; p < after; ++p) {
                if (count < max_out) {
                    out[3 * count + 0] = b;
                    out[3 * count + 1] = h;
                    out[3 * count + 2] = (int32_t)p;
                }
                ++count;
            }
        }
    }
    return count > 0x7fffffff ? LRKV_ERR_INVALID_ARG : (int32_t)count;
}

static int32_t check_skinny(const void* X, const void* Wt, const void* C, int M, int N, int K) {
    if (!X || !Wt || !C || M < 1 || N < 1 || K < 1) return LRKV_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(Wt)) return LRKV_ERR_INVALID_ARG;
    if ((K % 32) || (N % 16)) return LRKV_ERR_UNSUPPORTED;
    if ((long)M * N >= (1L << 31) || (long)N * K >= (1L << 40)) return LRKV_ERR_INVALID_ARG;
    return LRKV_OK;
}

size_t lrkv_project_workspace_bytes(int32_t m, int32_t n, int32_t k) {
    if (m < 1 || n < 1 || k < 1 || (k % 32) || (n % 16) || (long)m * n >= (1L << 31)) return 0;
    return skinny_plan(m, n, k).ws_bytes;
}

int32_t lrkv_latent_project(const float* x, int32_t n_tok, int32_t d_model, const void* a_t, int32_t units,
                            int32_t rank, float* h, void* workspace, size_t ws_bytes, void* stream) {
    if (units < 1 || rank < 1 || (long)units * rank >= (1L << 30)) return LRKV_ERR_INVALID_ARG;
    const int N = units * rank;
    int32_t rc = check_skinny(x, a_t, h, n_tok, N, d_model);
    if (rc != LRKV_OK) return rc;
    const SkinnyPlan p = skinny_plan(n_tok, N, d_model);
    if (!workspace || ws_bytes < p.ws_bytes) return LRKV_ERR_WORKSPACE;
    return launch_skinny(x, (const half_t*)a_t, h, n_tok, N, d_model, workspace, p, (hipStream_t)stream);
}

int32_t lrkv_output_project(const float* o, int32_t batch, int32_t q_heads, int32_t rank, const void* w_t,
                            int32_t d_model, float* y, void* workspace, size_t ws_bytes, void* stream) {
    if (q_heads < 1 || rank < 1 || (long)q_heads * rank >= (1L << 30)) return LRKV_ERR_INVALID_ARG;
    const int K = q_heads * rank;
    int32_t rc = check_skinny(o, w_t, y, batch, d_model, K);
    if (rc != LRKV_OK) return rc;
    const SkinnyPlan p = skinny_plan(batch, d_model, K);
    if (!workspace || ws_bytes < p.ws_bytes) return LRKV_ERR_WORKSPACE;
    return launch_skinny(o, (const half_t*)w_t, y, batch, d_model, K, workspace, p, (hipStream_t)stream);
}

// prefill: fp16 latents, rank 256, head_dim 128; host_max_len bounds p0[b] + m_tokens
static int32_t check_prefill(const lrkv_latent_cache* c, int32_t m_tokens, int32_t host_max_len) {
    int32_t rc = check_latent(c);
    if (rc != LRKV_OK) return rc;
    if (m_tokens < 1 || host_max_len < 1 || host_max_len > c->capacity) return LRKV_ERR_INVALID_ARG;
    if ((long)c->batch * m_tokens * c->units * c->kv_per_unit * c->q_per_kv * c->head_dim >= (1L << 31))
        return LRKV_ERR_INVALID_ARG;
    if (c->fmt != LRKV_FMT_FP16 || c->rank != 256 || c->head_dim != 128) return LRKV_ERR_UNSUPPORTED;
    return LRKV_OK;
}

size_t lrkv_prefill_workspace_bytes(const lrkv_latent_cache* c, int32_t m_tokens, int32_t host_max_len) {
    if (check_prefill(c, m_tokens, host_max_len) != LRKV_OK) return 0;
    return prefill_workspace_bytes(c->batch, c->units, c->kv_per_unit, c->q_per_kv, m_tokens, c->head_dim, c->rank,
                                   (host_max_len + kTile - 1) / kTile);
}

int32_t lrkv_prefill_attn(const lrkv_latent_cache* c, const float* q, const void* bk, const int32_t* p0,
                          int32_t m_tokens, int32_t host_max_len, float sm_scale, float* out, void* workspace,
                          size_t ws_bytes, void* stream) {
    int32_t rc = check_prefill(c, m_tokens, host_max_len);
    if (rc != LRKV_OK) return rc;
    if (!q || !bk || !p0 || !out || !aligned16(out) || !aligned16(q)) return LRKV_ERR_INVALID_ARG;
    if (!isfinite(sm_scale)) return LRKV_ERR_INVALID_ARG;
    const int n_tiles = (host_max_len + kTile - 1) / kTile;
    if (!workspace || ws_bytes < prefill_workspace_bytes(c->batch, c->units, c->kv_per_unit, c->q_per_kv, m_tokens,
                                                          c->head_dim, c->rank, n_tiles))
        return LRKV_ERR_WORKSPACE;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)c->head_dim);
    return launch_prefill(c, q, (const half_t*)bk, p0, m_tokens, n_tiles, scale, out, workspace,
                          (hipStream_t)stream);
}

int32_t lrkv_probe_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, void* stream) {
    if (!buf || !out || bytes == 0 || (bytes % 16) || (((uintptr_t)buf) & 15) || blocks < 1 || blocks > 65535)
        return LRKV_ERR_INVALID_ARG;
    return launch_stream_read(buf, bytes, out, blocks, (hipStream_t)stream);
}

}  // extern "C"
