// C ABI of v4attn: argument validation (on the host, before anything is
// enqueued), launch planning and workspace layout. The operations themselves
// are described in include/v4attn.h; the kernels live in the .hip files.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "v4attn.h"
#include "v4attn_internal.hpp"

using namespace v4a;

namespace {

thread_local std::string g_last_error = "no error";

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(v4a_strerror(status)) + ": " + buf;
    return status;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return V4A_OK;
    return fail(V4A_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool aligned(int64_t v, int64_t a) { return (v % a) == 0; }

void fill_inv_freq(double base, double *f) {
    for (int i = 0; i < ROPE_PAIRS; ++i) f[i] = pow(base, -2.0 * (double)i / (double)ROPE_DIM);
}

int check_plane(const v4a_plane &pl, const char *name, size_t align) {
    if (!pl.ptr) return fail(V4A_ENULL, "%s: plane pointer is NULL", name);
    if (!aligned(pl.ptr, align) || !aligned(pl.row_stride, (int64_t)align) || !aligned(pl.batch_stride, (int64_t)align))
        return fail(V4A_EALIGN, "%s: pointer and strides must be %zu-byte aligned", name, align);
    if (pl.row_stride <= 0 || pl.batch_stride < 0) return fail(V4A_EINVAL, "%s: bad strides", name);
    return V4A_OK;
}

// Validates a KV store; `fp8_dim` is the only dim allowed for E4M3_BF16.
int check_kv(const v4a_kv_store *s, const char *name, KvView *v) {
    if (!s) return fail(V4A_ENULL, "%s is NULL", name);
    if (s->rows <= 0 || s->ring < 0 || s->ring > s->rows) return fail(V4A_EINVAL, "%s: bad rows/ring", name);
    memset(v, 0, sizeof *v);
    v->fmt = s->fmt;
    v->dim = s->dim;
    v->rows = s->rows;
    v->ring = s->ring;
    int r;
    if (s->fmt == V4A_KV_F32) {
        if (s->dim < 128 || s->dim > 256 || s->dim % 64) return fail(V4A_EFORMAT, "%s: F32 dim must be 128..256, multiple of 64", name);
        if ((r = check_plane(s->f32, name, 16))) return r;
        if (s->f32.row_stride < 4 * s->dim) return fail(V4A_EINVAL, "%s: f32 row stride too small", name);
        v->f32 = (const char *)s->f32.ptr;
        v->f32_rs = s->f32.row_stride;
        v->f32_bs = s->f32.batch_stride;
    } else if (s->fmt == V4A_KV_E4M3_BF16) {
        if (s->dim != 192) return fail(V4A_EFORMAT, "%s: E4M3_BF16 stores need dim 192", name);
        if ((r = check_plane(s->nope, name, 16)) || (r = check_plane(s->rope, name, 16)) ||
            (r = check_plane(s->scale, name, 4)))
            return r;
        if (s->nope.row_stride < s->dim - 64 || s->rope.row_stride < 128)
            return fail(V4A_EINVAL, "%s: plane row stride too small", name);
        v->nope = (const char *)s->nope.ptr;
        v->nope_rs = s->nope.row_stride;
        v->nope_bs = s->nope.batch_stride;
        v->rope = (const char *)s->rope.ptr;
        v->rope_rs = s->rope.row_stride;
        v->rope_bs = s->rope.batch_stride;
        v->scale = (const char *)s->scale.ptr;
        v->scale_rs = s->scale.row_stride;
        v->scale_bs = s->scale.batch_stride;
    } else {
        return fail(V4A_EFORMAT, "%s: unknown KV format %d", name, s->fmt);
    }
    return V4A_OK;
}

int check_ik(const v4a_ik_store *s, const char *name, IkView *v) {
    if (!s) return fail(V4A_ENULL, "%s is NULL", name);
    if (s->rows <= 0) return fail(V4A_EINVAL, "%s: bad rows", name);
    memset(v, 0, sizeof *v);
    v->fmt = s->fmt;
    v->dim = s->dim;
    v->rows = s->rows;
    int r;
    if (s->fmt == V4A_IK_F32) {
        if (s->dim <= 0 || s->dim > 256 || s->dim % 4) return fail(V4A_EFORMAT, "%s: F32 dim must be 4..256, multiple of 4", name);
        if ((r = check_plane(s->f32, name, 16))) return r;
        v->f32 = (const char *)s->f32.ptr;
        v->f32_rs = s->f32.row_stride;
        v->f32_bs = s->f32.batch_stride;
    } else if (s->fmt == V4A_IK_MXFP4) {
        if (s->dim <= 0 || s->dim > 256 || s->dim % 32) return fail(V4A_EFORMAT, "%s: MXFP4 dim must be a multiple of 32, <= 256", name);
        if ((r = check_plane(s->e2m1, name, 16)) || (r = check_plane(s->e8m0, name, 1))) return r;
        if (s->e2m1.row_stride >= (1 << 20) || s->e8m0.row_stride >= (1 << 20))
            return fail(V4A_EINVAL, "%s: row strides must be below 1 MiB", name);
        v->e2m1 = (const char *)s->e2m1.ptr;
        v->e2m1_rs = s->e2m1.row_stride;
        v->e2m1_bs = s->e2m1.batch_stride;
        v->e8m0 = (const char *)s->e8m0.ptr;
        v->e8m0_rs = s->e8m0.row_stride;
        v->e8m0_bs = s->e8m0.batch_stride;
    } else {
        return fail(V4A_EFORMAT, "%s: unknown indexer-key format %d", name, s->fmt);
    }
    return V4A_OK;
}

// ------------------------------------------------------- index planning ----

struct IndexLayout {
    int chunk, n_chunks, s_local, region_cap;
    size_t off_meta, off_key, off_idx, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

IndexLayout index_layout(const v4a_index_args *a) {
    IndexLayout L;
    const int64_t Q = (int64_t)a->B * a->Tq;
    const int64_t rows = a->keys->rows;
    // several queries per sequence over more than one sub-chunk (chunked
    // prefill, drafts): a chunk of IDX_CPW sub-chunks per workgroup (MXFP4 keys)
    const bool multi = a->keys->fmt != V4A_IK_F32 && a->Tq > 1 && rows > IDX_CHUNK;
    L.chunk = multi ? IDX_CHUNK * IDX_CPW : IDX_CHUNK;
    L.n_chunks = (int)std::max<int64_t>(1, (rows + L.chunk - 1) / L.chunk);
    L.s_local = 2 * ((a->k + L.n_chunks - 1) / L.n_chunks) + 8;
    // a multiple of 4 slots and at least 32: the merge reads a region's first
    // 32 slots with 16-byte loads
    L.region_cap = std::min(L.chunk, (std::max(2 * L.s_local + 64, 128) + 3) / 4 * 4);
    L.off_meta = 0;
    L.off_key = align_up(L.off_meta + (size_t)Q * L.n_chunks * 8, 256);
    L.off_idx = align_up(L.off_key + (size_t)Q * L.n_chunks * L.region_cap * 4, 256);
    L.total = align_up(L.off_idx + (size_t)Q * L.n_chunks * L.region_cap * 4, 256);
    return L;
}

int check_index(const v4a_index_args *a) {
    if (!a) return fail(V4A_ENULL, "args is NULL");
    if (a->B <= 0 || a->Tq <= 0) return fail(V4A_EINVAL, "B and Tq must be positive");
    if (a->k < 1 || a->k > 4096) return fail(V4A_EINVAL, "k must be in 1..4096 (got %d)", a->k);
    if (a->m < 1) return fail(V4A_EINVAL, "m must be >= 1");
    if (!a->q_pos || !a->iq || !a->w || !a->out_idx || !a->keys) return fail(V4A_ENULL, "a required pointer is NULL");
    if (a->keys->fmt == V4A_IK_MXFP4) {
        if (a->keys->dim != 128) return fail(V4A_EFORMAT, "MXFP4 indexer keys need dim 128");
        if (a->H_I <= 0 || a->H_I > 64 || a->H_I % 16) return fail(V4A_EFORMAT, "MXFP4 indexer needs H_I in {16,32,48,64}");
        if (!a->iq_scale) return fail(V4A_ENULL, "iq_scale is NULL");
        if (!aligned(a->iq, 16)) return fail(V4A_EALIGN, "iq must be 16-byte aligned");
        if (!aligned(a->keys->e8m0.ptr, 4) || a->keys->e8m0.row_stride % 4 || a->keys->e8m0.batch_stride % 4)
            return fail(V4A_EALIGN, "MXFP4 indexer keys: e8m0 pointer and strides must be 4-byte aligned");
    } else if (a->keys->fmt == V4A_IK_F32) {
        if (a->H_I <= 0 || a->H_I > 16) return fail(V4A_EFORMAT, "F32 indexer needs H_I in 1..16");
        if (!aligned(a->iq, 4)) return fail(V4A_EALIGN, "iq must be 4-byte aligned");
    }
    if (!aligned(a->w, 4) || !aligned(a->q_pos, 8) || !aligned(a->out_idx, 4) || (a->out_score && !aligned(a->out_score, 4)))
        return fail(V4A_EALIGN, "w/q_pos/out_idx/out_score misaligned");
    IkView v;
    int r = check_ik(a->keys, "keys", &v);
    if (r) return r;
    if ((int64_t)a->B * a->Tq > (1 << 24)) return fail(V4A_EINVAL, "too many queries");
    return V4A_OK;
}

// --------------------------------------------------- attention planning ----

constexpr int KS_MIN = 32;      // keys per split: one tile at least
constexpr int KS_MAX = 2048;    // the FP8 kernel resolves a split's rows into LDS
constexpr int WG_TARGET = 512;  // about two resident workgroups per compute unit
constexpr int WG_TARGET_NS2 = 256;  // two-stream workgroups: one per compute unit
constexpr int64_t NS2_MIN_KEYS = 4096;  // key lists at least this long take two streams

constexpr int MAX_SPLITS = 1024;  // splits per query the combine kernel merges
// Longest key list (entries + window) one query may have: every split resolves
// its keys' store rows into LDS first, at most KS_MAX of them.
constexpr int64_t MAX_KEY_LIST = (int64_t)MAX_SPLITS * KS_MAX;

struct AttnLayout {
    int n_split, keys_per_split, n_streams;
    size_t off_ml, total;
};

// Upper bound of a query's key list: the sparse list, or every entry of the
// store (capped by the override), plus the window.
int64_t key_list_cap(const v4a_attn_args *a, bool sparse, int k, int64_t n_override) {
    int64_t n_list = 0;
    if (a->ent_k) {
        if (sparse) n_list = k;
        else {
            n_list = a->ent_k->rows;
            if (n_override >= 0) n_list = std::min(n_list, n_override);
        }
    }
    return n_list + a->W;
}

int check_key_list(const v4a_attn_args *a, bool sparse, int k, int64_t n_override) {
    const int64_t cap = key_list_cap(a, sparse, k, n_override);
    if (cap > MAX_KEY_LIST)
        return fail(V4A_EINVAL, "a key list of up to %lld keys exceeds the supported %lld (%d splits of %d keys)",
                    (long long)cap, (long long)MAX_KEY_LIST, MAX_SPLITS, KS_MAX);
    return V4A_OK;
}

AttnLayout attn_layout(const v4a_attn_args *a, bool sparse, int k, int64_t n_override) {
    AttnLayout L;
    const int64_t Q = (int64_t)a->B * a->Tq;
    const int64_t cap = key_list_cap(a, sparse, k, n_override);
    // Long key lists (FP8 path) run two key streams per workgroup, one
    // workgroup per compute unit; short ones one stream, about two per unit.
    const bool fp8 = a->win_k && a->win_k->fmt == V4A_KV_E4M3_BF16;
    L.n_streams = (fp8 && cap >= NS2_MIN_KEYS) ? 2 : 1;
    const int64_t target = L.n_streams == 2 ? WG_TARGET_NS2 : WG_TARGET;
    // enough splits to fill the device when the queries alone cannot, at least
    // one tile per stream, and no split longer than KS_MAX keys
    int64_t n_split = std::min((cap + KS_MIN * L.n_streams - 1) / (KS_MIN * L.n_streams), (target + Q - 1) / Q);
    n_split = std::max<int64_t>(n_split, (cap + KS_MAX - 1) / KS_MAX);
    n_split = std::max<int64_t>(1, std::min<int64_t>(n_split, MAX_SPLITS));
    int64_t ks = (cap + n_split - 1) / n_split;
    ks = std::max<int64_t>(KS_MIN, (ks + 31) / 32 * 32);
    n_split = std::max<int64_t>(1, (cap + ks - 1) / ks);
    L.n_split = (int)n_split;
    L.keys_per_split = (int)ks;
    if (n_split == 1) {
        L.off_ml = 0;
        L.total = 0;
        return L;
    }
    const size_t n_part = (size_t)Q * n_split * a->H_q;
    L.off_ml = align_up(n_part * a->dim * 4, 256);
    L.total = align_up(L.off_ml + n_part * 8, 256);
    return L;
}

int check_attn(const v4a_attn_args *a, AttnPlan *P) {
    if (!a) return fail(V4A_ENULL, "args is NULL");
    if (a->B <= 0 || a->Tq <= 0) return fail(V4A_EINVAL, "B and Tq must be positive");
    if (a->W < 0 || a->W > 4096) return fail(V4A_EINVAL, "W must be in 0..4096");
    if (!a->q_pos || !a->q || !a->o || !a->win_k || !a->win_v) return fail(V4A_ENULL, "a required pointer is NULL");
    if ((a->ent_k == nullptr) != (a->ent_v == nullptr)) return fail(V4A_ENULL, "ent_k and ent_v must both be given or both NULL");
    if (a->ent_k && a->m < 1) return fail(V4A_EINVAL, "m must be >= 1");
    memset(P, 0, sizeof *P);
    int r;
    if ((r = check_kv(a->win_k, "win_k", &P->wk)) || (r = check_kv(a->win_v, "win_v", &P->wv))) return r;
    if (a->ent_k && ((r = check_kv(a->ent_k, "ent_k", &P->ek)) || (r = check_kv(a->ent_v, "ent_v", &P->ev)))) return r;
    if (a->ent_k && (a->ent_k->ring != 0 || a->ent_v->ring != 0)) return fail(V4A_EINVAL, "entry stores cannot be rings");
    // rows are addressed as 30-bit codes (bit 30 marks a window-store row)
    for (auto *s : {a->win_k, a->win_v, a->ent_k, a->ent_v})
        if (s && s->rows >= ((int64_t)1 << 30))
            return fail(V4A_EINVAL, "a store of %lld rows exceeds the 2^30 rows attention addresses", (long long)s->rows);
    const int fmt = a->win_k->fmt;
    const v4a_kv_store *all[4] = {a->win_k, a->win_v, a->ent_k, a->ent_v};
    for (auto *s : all)
        if (s && (s->fmt != fmt || s->dim != a->dim)) return fail(V4A_EFORMAT, "all stores must share format and dim");
    if (a->win_v->rows < a->win_k->rows || a->win_v->ring != a->win_k->ring)
        return fail(V4A_EINVAL, "win_k and win_v must have the same rows and ring");
    // a ring shorter than the window would map two window positions to one slot
    if (a->win_k->ring > 0 && a->win_k->ring < a->W)
        return fail(V4A_EINVAL, "a window ring of %lld slots cannot hold a window of %d positions",
                    (long long)a->win_k->ring, a->W);
    if (a->ent_k && a->ent_v->rows < a->ent_k->rows) return fail(V4A_EINVAL, "ent_v has fewer rows than ent_k");
    if (fmt == V4A_KV_F32) {
        if (a->dim > 128) return fail(V4A_EFORMAT, "the fp32 path supports dim <= 128");
        if (a->H_q <= 0 || a->H_q > 64 || a->H_q * a->dim > 4096) return fail(V4A_EFORMAT, "fp32 path needs H_q*dim <= 4096");
        if (a->q_fmt != V4A_ACT_F32 || a->o_fmt != V4A_ACT_F32) return fail(V4A_EFORMAT, "fp32 stores need float32 q and o");
        if (!aligned(a->q, 4) || !aligned(a->o, 4)) return fail(V4A_EALIGN, "q/o misaligned");
    } else {
        if (a->H_q <= 0 || a->H_q > 64 || a->H_q % 16) return fail(V4A_EFORMAT, "the FP8 path needs H_q in {16,32,48,64}");
        if (a->q_fmt != V4A_ACT_BF16) return fail(V4A_EFORMAT, "FP8 stores need a bfloat16 q");
        if (a->o_fmt != V4A_ACT_BF16 && a->o_fmt != V4A_ACT_F32) return fail(V4A_EFORMAT, "unknown output format");
        if (!aligned(a->q, 16) || !aligned(a->o, 16)) return fail(V4A_EALIGN, "q and o must be 16-byte aligned");
    }
    if (!aligned(a->q_pos, 8) || (a->lse && !aligned(a->lse, 4))) return fail(V4A_EALIGN, "q_pos/lse misaligned");
    if (a->append_k || a->append_v) {
        if (!a->append_k || !a->append_v) return fail(V4A_ENULL, "append_k and append_v must both be given or both NULL");
        if (fmt != V4A_KV_E4M3_BF16) return fail(V4A_EFORMAT, "the fused window append needs E4M3_BF16 stores");
        if (a->Tq != 1) return fail(V4A_EINVAL, "the fused window append needs Tq == 1 (got %d)", a->Tq);
        if (a->W < 1) return fail(V4A_EINVAL, "the fused window append needs W >= 1");
        if (!aligned(a->append_k, 4) || !aligned(a->append_v, 4)) return fail(V4A_EALIGN, "append_k/append_v must be 4-byte aligned");
    }
    if (!(a->sm_scale >= 0.0f) || !isfinite(a->sm_scale)) return fail(V4A_EINVAL, "sm_scale must be finite and >= 0");
    if ((int64_t)a->B * a->Tq > (1 << 24)) return fail(V4A_EINVAL, "too many queries");
    P->Q = a->B * a->Tq;
    P->Tq = a->Tq;
    P->H = a->H_q;
    P->D = a->dim;
    P->W = a->W;
    P->m = a->ent_k ? a->m : 1;
    P->has_ent = a->ent_k != nullptr;
    P->q_pos = a->q_pos;
    P->q = a->q;
    P->sm_scale = a->sm_scale > 0.0f ? a->sm_scale : (float)(1.0 / sqrt((double)a->dim));
    fill_inv_freq(a->rope_base, P->inv_freq);
    P->o = a->o;
    P->o_bf16 = a->o_fmt == V4A_ACT_BF16;
    P->lse = a->lse;
    P->has_app = a->append_k != nullptr;
    P->app_k = (const uint16_t *)(P->has_app ? a->append_k : a->q);
    P->app_v = (const uint16_t *)(P->has_app ? a->append_v : a->q);
    return V4A_OK;
}

int run_attn(AttnPlan &P, const AttnLayout &L, void *ws, size_t ws_bytes, hipStream_t s) {
    P.n_split = L.n_split;
    P.keys_per_split = L.keys_per_split;
    P.n_streams = L.n_streams;
    if (L.total > 0) {
        if (!ws) return fail(V4A_EWORKSPACE, "a workspace of %zu bytes is required", L.total);
        if (ws_bytes < L.total) return fail(V4A_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
        if (!aligned(ws, 256)) return fail(V4A_EALIGN, "workspace must be 256-byte aligned");
        P.part_o = (float *)ws;
        P.part_ml = (float *)((char *)ws + L.off_ml);
    }
    return hip_status(launch_attn(P, s), "attention launch");
}

}  // namespace

extern "C" {

const char *v4a_strerror(int status) {
    switch (status) {
        case V4A_OK: return "ok";
        case V4A_EINVAL: return "invalid argument";
        case V4A_ENULL: return "null pointer";
        case V4A_EALIGN: return "misaligned pointer or stride";
        case V4A_EFORMAT: return "unsupported format or shape";
        case V4A_EWORKSPACE: return "workspace missing or too small";
        case V4A_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *v4a_last_error(void) { return g_last_error.c_str(); }

const char *v4a_version(void) { return "v4attn 0.1 gfx950"; }

int v4a_workspace_init(void *ws, size_t bytes, v4a_stream stream) {
    if (bytes == 0) return V4A_OK;
    if (!ws) return fail(V4A_ENULL, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(V4A_EALIGN, "workspace must be 256-byte aligned");
    return hip_status(launch_fill_zero(ws, bytes, (hipStream_t)stream), "workspace init");
}

int csa_compress(const v4a_compress_args *a, v4a_stream stream) {
    if (!a) return fail(V4A_ENULL, "args is NULL");
    if (a->B <= 0 || a->t_new < 0) return fail(V4A_EINVAL, "B must be positive and t_new >= 0");
    if (a->B > MAX_GRID_Y) return fail(V4A_EINVAL, "B must be at most %d (got %d)", MAX_GRID_Y, a->B);
    if (a->m < 1 || a->m > 1024) return fail(V4A_EINVAL, "m must be in 1..1024 (got %d)", a->m);
    if (a->pos0 < 0 || a->pos0 % a->m || a->t_new % a->m)
        return fail(V4A_EINVAL, "pos0 and t_new must be non-negative multiples of m");
    // a launch's grid holds 512 threads for each output of each block
    if (a->t_new / a->m > V4A_MAX_COMPRESS_BLOCKS)
        return fail(V4A_EINVAL, "at most %d blocks of m tokens per call (got %lld)", V4A_MAX_COMPRESS_BLOCKS,
                    (long long)(a->t_new / a->m));
    if (a->variant < V4A_POOL_BLOCK || a->variant > V4A_POOL_CHANNEL_GATE)
        return fail(V4A_EFORMAT, "unknown compressor variant %d", a->variant);
    const int span = a->variant == V4A_POOL_OVERLAP ? 2 * a->m : a->m;  // tokens one entry pools
    if (a->variant == V4A_POOL_OVERLAP && a->m > 512) return fail(V4A_EINVAL, "overlapping windows need m <= 512");
    if (a->block_end) {
        if (a->pos0 != 0) return fail(V4A_EINVAL, "block mode (block_end given) needs pos0 == 0");
        if (a->t_new < span)
            return fail(V4A_EINVAL, "block mode: the raw ring (t_new rows) must hold the %d tokens an entry pools", span);
        if (!aligned(a->block_end, 8)) return fail(V4A_EALIGN, "block_end must be 8-byte aligned");
    }
    if (a->act_fmt != V4A_ACT_F32 && a->act_fmt != V4A_ACT_BF16) return fail(V4A_EFORMAT, "unknown activation format");
    if (a->t_new == 0) return V4A_OK;  // nothing to compress: no pointer is read, nothing is launched
    if (!a->gate || !a->pos_bias) return fail(V4A_ENULL, "gate and pos_bias are required");
    if ((a->k_out == nullptr) != (a->v_out == nullptr)) return fail(V4A_ENULL, "k_out and v_out must both be given or both NULL");
    if ((a->ik_out == nullptr) != (a->raw_ik == nullptr)) return fail(V4A_ENULL, "raw_ik and ik_out go together");
    if (!a->k_out && !a->ik_out) return fail(V4A_EINVAL, "no output store given");
    CompressPlan P;
    memset(&P, 0, sizeof P);
    P.B = a->B;
    P.t_new = a->t_new;
    P.m = a->m;
    P.act = a->act_fmt;
    P.pos0 = a->pos0;
    P.gate = a->gate;
    P.pos_bias = a->pos_bias;
    P.block_end = a->block_end;
    P.variant = a->variant;
    const int64_t e0 = a->pos0 / a->m, ne = a->t_new / a->m;
    const size_t esz = a->act_fmt == V4A_ACT_F32 ? 4 : 2;
    int r;
    if (a->k_out) {
        if (!a->raw_k || !a->raw_v) return fail(V4A_ENULL, "raw_k/raw_v are NULL");
        if ((r = check_kv(a->k_out, "k_out", &P.k)) || (r = check_kv(a->v_out, "v_out", &P.v))) return r;
        if (a->k_out->fmt != a->v_out->fmt || a->k_out->dim != a->v_out->dim || a->k_out->ring != a->v_out->ring)
            return fail(V4A_EFORMAT, "k_out and v_out must share format, dim and ring");
        for (const v4a_kv_store *s : {a->k_out, a->v_out}) {
            if (!a->block_end && s->ring == 0 && e0 + ne > s->rows)
                return fail(V4A_EINVAL, "entries %lld..%lld do not fit in %lld rows", (long long)e0,
                            (long long)(e0 + ne - 1), (long long)s->rows);
        }
        // the compressors read raw rows as pairs of elements
        if (!aligned(a->raw_k, 2 * esz) || !aligned(a->raw_v, 2 * esz))
            return fail(V4A_EALIGN, "raw_k/raw_v must be aligned to two elements");
        P.has_kv = 1;
        P.D = a->k_out->dim;
        P.raw_k = a->raw_k;
        P.raw_v = a->raw_v;
    }
    if (a->ik_out) {
        if ((r = check_ik(a->ik_out, "ik_out", &P.ik))) return r;
        if (!a->block_end && e0 + ne > a->ik_out->rows) return fail(V4A_EINVAL, "indexer entries do not fit in the store");
        if (a->ik_out->fmt == V4A_IK_F32 && a->ik_out->dim % 4) return fail(V4A_EFORMAT, "bad indexer dim");
        if (!aligned(a->raw_ik, 2 * esz)) return fail(V4A_EALIGN, "raw_ik must be aligned to two elements");
        P.has_ik = 1;
        P.dI = a->ik_out->dim;
        P.raw_ik = a->raw_ik;
    }
    if (a->variant == V4A_POOL_CHANNEL_GATE) P.gate_c = (P.has_kv ? 2 * P.D : 0) + (P.has_ik ? P.dI : 0);
    fill_inv_freq(a->rope_base, P.inv_freq);
    if (a->t_new == 0) return V4A_OK;
    return hip_status(launch_compress(P, (hipStream_t)stream), "compress launch");
}

size_t lightning_index_topk_workspace(const v4a_index_args *a) {
    if (check_index(a)) return 0;
    return index_layout(a).total;
}

int lightning_index_topk(const v4a_index_args *a, void *ws, size_t ws_bytes, v4a_stream stream) {
    return v4a::index_call(a, ws, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"

namespace v4a {

int report(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return fail(status, "%s", buf);
}

int index_workspace(const v4a_index_args *a, size_t *bytes) {
    const int r = check_index(a);
    *bytes = r ? 0 : index_layout(a).total;
    return r;
}

int index_call(const v4a_index_args *a, void *ws, size_t ws_bytes, hipStream_t stream) {
    int r = check_index(a);
    if (r) return r;
    const IndexLayout L = index_layout(a);
    if (!ws) return fail(V4A_EWORKSPACE, "a workspace of %zu bytes is required", L.total);
    if (ws_bytes < L.total) return fail(V4A_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    if (!aligned(ws, 256)) return fail(V4A_EALIGN, "workspace must be 256-byte aligned");
    IndexPlan P;
    memset(&P, 0, sizeof P);
    check_ik(a->keys, "keys", &P.keys);
    P.Q = a->B * a->Tq;
    P.Tq = a->Tq;
    P.H = a->H_I;
    P.dI = a->keys->dim;
    P.k = a->k;
    P.m = a->m;
    P.chunk = L.chunk;
    P.n_chunks = L.n_chunks;
    P.s_local = L.s_local;
    P.region_cap = L.region_cap;
    P.q_pos = a->q_pos;
    P.iq = a->iq;
    P.iq_scale = a->iq_scale;
    P.w = a->w;
    P.out_idx = a->out_idx;
    P.out_score = a->out_score;
    char *w = (char *)ws;
    P.meta = (uint32_t *)(w + L.off_meta);
    P.reg_key = (uint32_t *)(w + L.off_key);
    P.reg_idx = (int32_t *)(w + L.off_idx);
    return hip_status(launch_index(P, stream), "index launch");
}

int fill_zero(void *ptr, size_t bytes, hipStream_t stream) {
    return hip_status(launch_fill_zero(ptr, bytes, stream), "scratch initialisation");
}

}  // namespace v4a

extern "C" {

size_t sparse_window_attn_workspace(const v4a_attn_args *a, int32_t k) {
    AttnPlan P;
    if (check_attn(a, &P) || k < 1 || k > 65536 || check_key_list(a, true, k, -1)) return 0;
    return attn_layout(a, true, k, -1).total;
}

int sparse_window_attn(const v4a_attn_args *a, const int32_t *idx, int32_t k, void *ws, size_t ws_bytes,
                       v4a_stream stream) {
    AttnPlan P;
    int r = check_attn(a, &P);
    if (r) return r;
    if (!a->ent_k) return fail(V4A_ENULL, "sparse attention needs entry stores");
    if (k < 1 || k > 65536) return fail(V4A_EINVAL, "k must be in 1..65536");
    if (!idx) return fail(V4A_ENULL, "topk_idx is NULL");
    if (!aligned(idx, 4)) return fail(V4A_EALIGN, "topk_idx misaligned");
    if ((r = check_key_list(a, true, k, -1))) return r;
    P.sparse = 1;
    P.k = k;
    P.idx = idx;
    P.id_src = idx;
    P.id_stride = k;
    P.id_jmax = k - 1;
    P.n_override = -1;
    return run_attn(P, attn_layout(a, true, k, -1), ws, ws_bytes, (hipStream_t)stream);
}

size_t hca_attn_workspace(const v4a_attn_args *a, int64_t n_override) {
    AttnPlan P;
    if (check_attn(a, &P) || check_key_list(a, false, 0, n_override)) return 0;
    return attn_layout(a, false, 0, n_override).total;
}

int hca_attn(const v4a_attn_args *a, int64_t n_override, void *ws, size_t ws_bytes, v4a_stream stream) {
    AttnPlan P;
    int r = check_attn(a, &P);
    if (r) return r;
    if ((r = check_key_list(a, false, 0, n_override))) return r;
    P.sparse = 0;
    P.k = 0;
    P.idx = nullptr;
    P.id_src = (const int32_t *)a->q_pos;
    P.id_stride = 0;
    P.id_jmax = 0;
    P.n_override = n_override;
    if (n_override == 0) P.has_ent = 0;
    return run_attn(P, attn_layout(a, false, 0, n_override), ws, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"
