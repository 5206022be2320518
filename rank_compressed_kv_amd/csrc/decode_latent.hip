// Dispatch of the Palu latent-cache decode steps: query preparation, per-chunk
// partial states, split merge.
#include "common.h"

namespace lrkv {

bool rope_shape_supported(int r, int dh, int nh);
bool rope_fragment_layout(const lrkv_latent_cache* c);
bool absorbed_shape_supported(int r, int nh);
void launch_rope_prep(const float* q, const half_t* bk, const int32_t* q_pos, const int32_t* lens,
                      half_t* qp, float* qs, float2* angles, int B, int U, int s, int gq, int DH,
                      int R, int n_split, int chunk, double theta, float scale, int qmode,
                      bool int4, hipStream_t st, int pending, const float* nk, const float* nv,
                      void* hk, void* hv, half_t* sk, half_t* sv, int cap);
int32_t launch_rope_decode(const lrkv_latent_cache* c, const half_t* qp, const float* qs,
                           const float2* angles, float* part, int n_split, int chunk, hipStream_t st,
                           int pending);
int32_t launch_rope_gqa(const lrkv_latent_cache* c, const half_t* qbuf, const float2* angles, float* part,
                        int n_split, int chunk, hipStream_t st, int pending);
int32_t launch_absorbed_decode(const lrkv_latent_cache* c, const float* q, float* part, int n_split,
                               int chunk, float qscale, hipStream_t st);
void launch_merge(const float* part, float* out, int BH, int n_split, int D, hipStream_t st);
void launch_merge_bump(const float* part, float* out, int BH, int n_split, int D, hipStream_t st,
                       int32_t* lens, int B, int bump);

bool latent_shape_supported(int mode, const LatentGeom& g) {
    const int nh = g.s * g.gq;
    if (mode == LRKV_MODE_ROPE_RECON) return use_gqa_kernel(g) || rope_shape_supported(g.r, g.dh, nh);
    return absorbed_shape_supported(g.r, nh);
}

// `app` (lrkv_decode_step, RoPE mode, fp16 latents, all phases): the step's new
// tokens, appended by the preparation launch and counted as `pending` by every
// kernel until the merge adds them to lens.
int32_t launch_decode_latent(int mode, int phases, const lrkv_latent_cache* c, const float* q,
                             const half_t* bk, const int32_t* q_pos, float sm_scale, float* out,
                             void* ws, const LatentWorkspace& w, hipStream_t st, const FusedAppend* app) {
    const int pending = app ? app->n_new : 0;
    const LatentGeom g = latent_geom(c);
    char* base = (char*)ws;
    float* part = (float*)(base + w.part_off);
    if (mode == LRKV_MODE_ROPE_RECON) {
        half_t* qp = (half_t*)(base + w.qp_off);
        float* qs = (float*)(base + w.qs_off);
        float2* angles = (float2*)(base + w.ang_off);
        const bool gqa = use_gqa_kernel(g);
        const int qmode = gqa ? kQpGqaFragments : rope_fragment_layout(c) ? kQpFragments : kQpRowMajor;
        if (phases & kPhasePrepare)
            launch_rope_prep(q, bk, q_pos, c->lens, qp, qs, angles, g.B, g.U, g.s, g.gq, g.dh, g.r,
                             w.n_split, w.chunk, (double)g.theta, sm_scale * kLog2e, qmode,
                             g.fmt == LRKV_FMT_INT4_G32, st, pending, app ? app->nk : nullptr,
                             app ? app->nv : nullptr, c->hk, c->hv, (half_t*)c->sk, (half_t*)c->sv,
                             c->capacity);
        if (phases & kPhasePartials) {
            const int32_t rc = gqa ? launch_rope_gqa(c, qp, angles, part, w.n_split, w.chunk, st, pending)
                                   : launch_rope_decode(c, qp, qs, angles, part, w.n_split, w.chunk, st,
                                                        pending);
            if (rc != LRKV_OK) return rc;
        }
    } else if (phases & kPhasePartials) {
        const int32_t rc = launch_absorbed_decode(c, q, part, w.n_split, w.chunk, sm_scale * kLog2e, st);
        if (rc != LRKV_OK) return rc;
    }
    if (phases & kPhaseMerge) {
        if (pending) launch_merge_bump(part, out, g.B * g.Hq, w.n_split, g.r, st, c->lens, g.B, pending);
        else launch_merge(part, out, g.B * g.Hq, w.n_split, g.r, st);
    }
    return last_launch_status();
}

}  // namespace lrkv
