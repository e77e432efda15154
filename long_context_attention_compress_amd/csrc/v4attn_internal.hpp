// Internal plans passed from the C ABI layer (abi.cpp) to the kernel launchers.
// Plain structs, copied by value into kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "v4attn.h"

namespace v4a {

constexpr int ROPE_DIM = 64;
constexpr int ROPE_PAIRS = 32;

// Device view of a v4a_kv_store: byte pointers and byte strides.
struct KvView {
    int fmt;       // 0 f32, 1 e4m3+bf16
    int dim;
    int64_t rows;
    int64_t ring;  // 0: linear
    const char *f32;   int64_t f32_rs, f32_bs;
    const char *nope;  int64_t nope_rs, nope_bs;
    const char *rope;  int64_t rope_rs, rope_bs;
    const char *scale; int64_t scale_rs, scale_bs;
};

struct IkView {
    int fmt;       // 0 f32, 1 mxfp4
    int dim;
    int64_t rows;
    const char *f32;  int64_t f32_rs, f32_bs;
    const char *e2m1; int64_t e2m1_rs, e2m1_bs;
    const char *e8m0; int64_t e8m0_rs, e8m0_bs;
};

struct CompressPlan {
    int B, t_new, m, act;  // act: 0 f32, 1 bf16
    int64_t pos0;
    // block mode: device positions [B] of the last token of the block to write
    // (the raw inputs are rings of t_new rows); null: the chunk at pos0
    const int64_t *block_end;
    int variant;      // v4a_pool_variant
    int gate_c;       // channel gates: logits per token (0 otherwise)
    int D, dI;
    int has_kv, has_ik;
    const void *raw_k, *raw_v, *raw_ik;
    const float *gate, *pos_bias;
    KvView k, v;
    IkView ik;
    double inv_freq[ROPE_PAIRS];
};

// Entries scored by one indexer workgroup in one unrolled pass (a sub-chunk).
// A compile-time constant: the scoring loop over it is fully unrolled.
constexpr int IDX_CHUNK = 1024;
// With several queries per sequence over more than IDX_CHUNK entries (chunked
// prefill, drafts) a chunk is IDX_CPW sub-chunks: one workgroup scores them
// and keeps one candidate set for all of them.
constexpr int IDX_CPW = 4;

// Launches put queries on grid y, whose extent is at most 65535: larger
// query counts run as several launches, each with its first query in q_base.
constexpr int MAX_GRID_Y = 65535;

struct IndexPlan {
    int Q, Tq, H, dI, k, m;
    int q_base;      // first query of this launch (score kernel)
    int chunk;       // entries per chunk: IDX_CHUNK, or IDX_CHUNK x IDX_CPW (several queries per sequence)
    int n_chunks;    // workgroups per query
    int s_local;     // candidates a chunk keeps at least (its local top-s)
    int region_cap;  // candidate slots per chunk in the workspace
    const int64_t *q_pos;
    const void *iq;
    const uint8_t *iq_scale;
    const float *w;
    IkView keys;
    int32_t *out_idx;
    float *out_score;
    uint32_t *meta;      // [Q][n_chunks][2]: candidate count, lower key bound
    uint32_t *reg_key;   // [Q][n_chunks][region_cap]
    int32_t *reg_idx;    // [Q][n_chunks][region_cap]
};

// What a query's key list needs besides the query position, in one
// block at the start of the plan, so that the first scalar loads bring it in
// before the position arrives (launch_attn fills it from the plan's other
// fields). Rows and counts are below 2^30 (the host checks).
struct KeyConsts {
    int32_t W;       // window length
    int32_t ring;    // window stores' ring (0: linear)
    int32_t wrows;   // window store rows
    int32_t erows;   // entry store rows (0 without entries)
    int32_t cap;     // list length bound: k (sparse), else the entry rows capped by the override; 0 without entries
    uint32_t misc;   // bit 0: sparse; bits 8..15: m_sh; bits 16..23: r_sh
    uint32_t m_mul;  // x / m == (x * m_mul) >> m_sh for 0 <= x < 2^31 (x as 64-bit product)
    uint32_t r_mul;  // x / ring == (x * r_mul) >> r_sh likewise (ring > 0)
    int32_t m;       // positions per entry (1 without entries)
};

struct AttnPlan {
    KeyConsts kc;
    int Q, Tq, H, D, W, m;
    int q_base;        // first query of this launch (attention kernels)
    int sparse;        // 1: key list is idx[q][0..k); 0: entries 0..n_ent-1
    int k;             // sparse list length
    int64_t n_override;  // dense: cap on entries (< 0: none)
    int has_ent;
    int n_split;       // workgroups per query
    int keys_per_split;
    int n_streams;     // FP8 path: key streams per workgroup (1 or 2)
    const int64_t *q_pos;
    const void *q;
    KvView ek, ev, wk, wv;
    const int32_t *idx;
    // where the FP8 kernel reads the ids of query q's list (position j <=
    // id_jmax): id_src + q * id_stride; a dense call reads a valid dummy
    // (q_pos) there, so the loads need no branch
    const int32_t *id_src;
    int64_t id_stride, id_jmax;
    float sm_scale;
    double inv_freq[ROPE_PAIRS];
    void *o;
    int o_bf16;      // output format: 1 bfloat16, 0 float32
    float *lse;
    float *part_o;   // [Q][n_split][H][D]
    float *part_ml;  // [Q][n_split][H][2]
    // fused window append (FP8 path, one query token per sequence): raw BF16
    // K and V rows [Q][D] of the query tokens, written into the window stores
    // at the query positions before they are attended (has_app = 1); without
    // an append both point at q (read, never used)
    int has_app;
    const uint16_t *app_k, *app_v;
};

// Entry-point pieces shared between translation units (abi.cpp defines them):
// the index call's validation, workspace size and launch; the error report
// behind v4a_last_error(); a zero fill of device memory on a stream.
int report(int status, const char *fmt, ...);
int index_workspace(const v4a_index_args *a, size_t *bytes);
int index_call(const v4a_index_args *a, void *ws, size_t ws_bytes, hipStream_t stream);
int fill_zero(void *ptr, size_t bytes, hipStream_t stream);

hipError_t launch_compress(const CompressPlan &p, hipStream_t s);
hipError_t launch_index(const IndexPlan &p, hipStream_t s);
hipError_t launch_attn(const AttnPlan &p, hipStream_t s);
hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t s);

}  // namespace v4a
