/*
 * v4attn: hybrid compressed attention (CSA / HCA) for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the hot path. Four operations, named after the steps the pages
 * describe:
 *
 *   csa_compress          softmax-gated pooling of m raw tokens into one cache
 *                         entry (m = 4 for CSA, 128 for HCA, 1 appends a raw
 *                         window row), encoded as FP8 + BF16 (or float32), plus
 *                         the MXFP4 (or float32) indexer key.
 *                         [chaosnode.de, "DeepSeek-V4: 1 Million Token Context
 *                         endlich nutzbar", section "Hybrid Attention: CSA und
 *                         HCA"; webconsulting.at, "DeepSeek V4-Pro: Architektur,
 *                         KV-Cache-Kompression und Hyper-Connections im Detail",
 *                         section "Kompression und Selektion"]
 *   lightning_index_topk  per query, score every visible compressed entry with
 *                         the low-precision indexer and keep the top k.
 *                         [same sections; golem.de, "Chinas KI-Unabhängigkeit?:
 *                         Bei Deepseek V4 haben kleine Änderungen große
 *                         Wirkung", section "Komprimierte Erinnerung für längere
 *                         Kontexte"]
 *   sparse_window_attn    CSA attention: the selected entries plus the raw
 *                         window of the last W tokens, one joint softmax.
 *   hca_attn              HCA attention: every visible entry plus the window
 *                         (no selection); with n_entries_override = 0 it is the
 *                         window-only attention of the first layers.
 *                         [golem.de, same section; chaosnode.de, same section]
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every data pointer is a DEVICE pointer (hipMalloc'd or equivalent) owned
 *   by the caller. The library never allocates, frees or synchronises, and
 *   keeps no pointer after a call returns. Work is enqueued on `stream`
 *   (NULL = the default stream); outputs are valid once the stream reaches
 *   that point, and inputs must stay unchanged until then.
 * - Calls return V4A_OK (0) or a negative v4a_status. All argument checks run
 *   on the host before anything is enqueued, so a failed call launches
 *   nothing. v4a_last_error() gives a message for the calling thread's last
 *   failure. No C++ exception crosses this interface.
 * - Query positions (q_pos) live on the device and are not checked on the
 *   host; kernels clamp every derived index to the store bounds, so a bad
 *   position yields unspecified values but never an out-of-bounds access.
 * - Results are deterministic: identical inputs give bitwise identical
 *   outputs (no floating-point atomics on result paths).
 * - Calls that take a workspace must be given one of at least the size the
 *   matching *_workspace() function returns, initialised once with
 *   v4a_workspace_init(); the library leaves it in the initialised state after
 *   every call, so it can be reused. Calls that overlap in time on different
 *   streams need different workspaces.
 *
 * Positions, entries and the window
 * ---------------------------------
 * A raw token at position p belongs to compressed entry e = p / m; entry e
 * is visible to a query at position t when e*m + m - 1 <= t. The window of a
 * query at t is the raw positions max(0, t-W+1) .. t (the query's own token
 * included). Entries and window rows may cover the same position; both count.
 * The last 64 dims of every key, value and query are the RoPE dims
 * (interleaved pairs, angle p * base^(-2i/64), i < 32); keys are rotated at
 * their raw token's position before pooling, queries at their own position,
 * values never.
 */
#ifndef V4ATTN_H
#define V4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *v4a_stream; /* a hipStream_t */

typedef enum {
    V4A_OK = 0,
    V4A_EINVAL = -1,     /* a size, count or ratio is out of range */
    V4A_ENULL = -2,      /* a required pointer is NULL */
    V4A_EALIGN = -3,     /* a pointer or stride breaks the required alignment */
    V4A_EFORMAT = -4,    /* an unsupported format or shape combination */
    V4A_EWORKSPACE = -5, /* workspace missing or too small */
    V4A_EHIP = -6        /* the HIP runtime reported an error at enqueue */
} v4a_status;

typedef enum { V4A_KV_F32 = 0, V4A_KV_E4M3_BF16 = 1 } v4a_kv_format;
typedef enum { V4A_IK_F32 = 0, V4A_IK_MXFP4 = 1 } v4a_ik_format;
typedef enum { V4A_ACT_F32 = 0, V4A_ACT_BF16 = 1 } v4a_act_format;
/* Compressor variants of csa_compress (readings of the pages; see csa_compress). */
typedef enum {
    V4A_POOL_BLOCK = 0,          /* blocks of m, keys rotated then pooled, one gate per token */
    V4A_POOL_OVERLAP = 1,        /* windows of 2m: the block and the one before it */
    V4A_POOL_ROPE_AFTER = 2,     /* keys pooled unrotated, rotated at the block's last position */
    V4A_POOL_CHANNEL_GATE = 3    /* one gate logit per token and output channel */
} v4a_pool_variant;

/* One plane of a store: element (b, row, ...) starts at
 * ptr + b*batch_stride + row*row_stride (strides in BYTES). */
typedef struct {
    void *ptr;
    int64_t row_stride;
    int64_t batch_stride;
} v4a_plane;

/* A key or value store (compressed entries or raw window rows).
 *  fmt  V4A_KV_F32:       plane f32   [rows][dim] float32.
 *       V4A_KV_E4M3_BF16: plane nope  [rows][dim-64] OCP E4M3 codes,
 *                         plane rope  [rows][64] bfloat16 bits,
 *                         plane scale [rows][(dim-64)/128] float32;
 *                         value of nope element i = E4M3(code) * scale[i/128].
 *  rows  rows per batch element (below 2^30 for the attention calls, which
 *        reject larger stores with V4A_EINVAL).
 *  ring  0: entry/position n is row n (n < rows);
 *        > 0: entry/position n is row n % ring (ring <= rows), for a window
 *        kept as a ring buffer.
 * Alignment: nope and rope pointers and strides 16-byte aligned; scale and
 * f32 4-byte aligned. */
typedef struct {
    int32_t fmt;
    int32_t dim;
    int64_t rows;
    int64_t ring;
    v4a_plane f32;
    v4a_plane nope;
    v4a_plane rope;
    v4a_plane scale;
} v4a_kv_store;

/* An indexer-key store, one key of `dim` values per compressed entry.
 *  fmt  V4A_IK_F32:   plane f32  [rows][dim] float32.
 *       V4A_IK_MXFP4: plane e2m1 [rows][dim/2] bytes, byte i holding element
 *                     2i in its low nibble and 2i+1 in its high nibble;
 *                     plane e8m0 [rows][dim/32] shared exponents (value of
 *                     element j = E2M1(code_j) * 2^(e8m0[j/32] - 127)).
 * Alignment: e2m1 pointer and row stride 16-byte aligned. */
typedef struct {
    int32_t fmt;
    int32_t dim;
    int64_t rows;
    v4a_plane f32;
    v4a_plane e2m1;
    v4a_plane e8m0;
} v4a_ik_store;

/* ------------------------------------------------------------------------
 * csa_compress: pool blocks of m raw tokens into cache entries.
 *
 * For block j of the chunk (raw tokens pos0 + j*m + r, r < m):
 *   alpha_r = softmax_r(gate[b][j*m + r] + pos_bias[r])
 *   K = sum_r alpha_r * RoPE(raw_k[b][j*m + r], pos0 + j*m + r)
 *   V = sum_r alpha_r * raw_v[b][j*m + r]
 *   U = sum_r alpha_r * raw_ik[b][j*m + r]
 * computed in float64, rounded to float32, then encoded into the stores at
 * entry pos0/m + j. E4M3_BF16 stores: scale = amax/448 per 128 no-RoPE dims
 * (1 when amax = 0; NaN when the group holds a NaN, which then makes every
 * code of the group NaN), code = E4M3(x/scale) rounded to nearest even with
 * saturation to +-448 (NaN -> 0x7F); RoPE dims rounded to BF16. MXFP4 keys:
 * OCP MX v1.0 scale rule, E = floor(log2 amax) - 2 clamped to [-127, 127],
 * elements rounded to nearest even E2M1 with saturation to +-6; a block with a
 * non-finite value gets scale 0xFF and zero elements.
 * m = 1 turns the call into an append of raw rows (RoPE + encode), which is
 * how the window is filled.
 *
 *  B, t_new    batch size (1 .. 65535) and raw tokens per batch element
 *              (t_new % m == 0, and at most V4A_MAX_COMPRESS_BLOCKS blocks:
 *              t_new / m <= 2^21). t_new = 0 returns V4A_OK once B, m, pos0
 *              and act_fmt are valid; then no pointer is read and nothing is
 *              enqueued.
 *  pos0        position of the first raw token (pos0 % m == 0, >= 0).
 *  m           1 .. 1024.
 *  act_fmt     format of raw_k, raw_v, raw_ik (float32 or bfloat16).
 *  rope_base   RoPE base (e.g. 10000).
 *  raw_k/raw_v [B][t_new][dim of k_out/v_out], contiguous; may be NULL
 *              together with k_out/v_out. raw_k, raw_v and raw_ik are read as
 *              pairs of elements: 8-byte aligned (float32) or 4-byte aligned
 *              (bfloat16), else V4A_EALIGN.
 *  gate        [B][t_new] float32 gate logits.
 *  pos_bias    [m] float32 positional bias.
 *  raw_ik      [B][t_new][ik_out->dim] or NULL (then ik_out must be NULL).
 *  k_out/v_out key and value stores (same fmt and dim), or both NULL.
 *  ik_out      indexer-key store or NULL.
 * At least one output must be given. Entries written: pos0/m .. pos0/m +
 * t_new/m - 1, which must fit in the rows of linear stores. A ring store
 * (k_out/v_out with ring > 0, e.g. the window) receives only the last `ring`
 * of them, at row entry % ring.
 *
 *  block_end   NULL, or (block mode, decode) a DEVICE array [B] of positions:
 *              for each batch element b the call compresses the one block of m
 *              tokens ending at t = block_end[b] into entry (t+1)/m - 1, when
 *              t + 1 is a positive multiple of m; otherwise (or when the entry
 *              is past a linear store's rows) nothing is written for b. The
 *              raw inputs are then rings of t_new rows per batch element (a
 *              multiple of m): position p is row p % t_new of raw_k, raw_v and
 *              raw_ik and element p % t_new of gate. pos0 must be 0. Positions
 *              are read on the device, so the call can be captured once in a
 *              HIP graph while the positions advance from replay to replay
 *              (the block is written at the step it completes).
 *              [chaosnode.de, "DeepSeek-V4: 1 Million Token Context endlich
 *              nutzbar", section "Hybrid Attention: CSA und HCA": blocks of 4
 *              (CSA) or 128 (HCA) consecutive tokens become one entry]
 *  variant     a v4a_pool_variant (0 = V4A_POOL_BLOCK, the pooling above).
 *              V4A_POOL_OVERLAP [webconsulting.at, section "Kompression und
 *              Selektion": CSA lets information flow across group
 *              boundaries]: entry e pools the 2m tokens (e-1)m .. (e+1)m - 1
 *              with alpha = softmax over the 2m of (gate + pos_bias[offset]),
 *              pos_bias [2m] (offsets below m: the block before); positions
 *              below 0 do not take part. The raw inputs and gate then hold
 *              t_new + m rows, positions pos0 - m .. pos0 + t_new - 1 (the
 *              first m unread when pos0 = 0); in block mode the ring needs at
 *              least 2m rows. m <= 512.
 *              V4A_POOL_ROPE_AFTER [golem.de, same section as above: the last
 *              64 values carry RoPE]: K = RoPE(sum_r alpha_r raw_k[r], p_last),
 *              p_last the block's last position; V and U as above.
 *              V4A_POOL_CHANNEL_GATE [chaosnode.de, same section: softmax
 *              gating with a learned positional bias, per channel]: gate
 *              [B][t_new][C] and pos_bias [m][C], C = 2 dim (when k_out is
 *              given) + ik dim (when ik_out is given), channels ordered K, V, U;
 *              channel c of an entry pools with its own softmax over r of
 *              gate[.][r][c] + pos_bias[r][c].
 *              Every variant keeps the store formats and the visibility rule,
 *              so the attention calls read their entries unchanged.
 * ---------------------------------------------------------------------- */
/* Blocks of m tokens one csa_compress call may compress per batch element. */
#define V4A_MAX_COMPRESS_BLOCKS (1 << 21)

typedef struct {
    int32_t B;
    int32_t t_new;
    int64_t pos0;
    int32_t m;
    int32_t act_fmt;
    double rope_base;
    const void *raw_k;
    const void *raw_v;
    const float *gate;
    const float *pos_bias;
    const void *raw_ik;
    const v4a_kv_store *k_out;
    const v4a_kv_store *v_out;
    const v4a_ik_store *ik_out;
    const int64_t *block_end;
    int32_t variant;
} v4a_compress_args;

int csa_compress(const v4a_compress_args *a, v4a_stream stream);

/* ------------------------------------------------------------------------
 * lightning_index_topk: per query, score the visible entries and keep the
 * top k.
 *
 * Query (b, i) at position t = q_pos[b][i] sees entries e < min(rows,
 * (t+1)/m). Score (float32):
 *   I_e = sum_h w[b][i][h] * max(0, iq[b][i][h] . key_e)
 * max(0, x) propagates NaN (IEEE 754-2019 maximum): a NaN dot product, for
 * example from an E8M0 NaN scale (0xFF) in a key or a query head, makes I_e
 * NaN. The selection is the min(k, n_visible) entries with the largest score,
 * equal scores going to the lower entry id (-0 equals +0; NaN ranks lowest).
 * out_idx[b][i][0..k) receives the selected ids in ascending order, padded
 * with -1. out_score (optional) receives the matching scores (0 for padding).
 *
 *  iq      MXFP4 keys: [B][Tq][H_I][dim/2] packed E2M1 bytes (same nibble
 *          order as the store) with iq_scale [B][Tq][H_I][dim/32] E8M0;
 *          F32 keys: [B][Tq][H_I][dim] float32 (iq_scale unused).
 *  w       [B][Tq][H_I] float32 head weights.
 * Supported: F32 keys with dim % 4 == 0, dim <= 256, H_I <= 16; MXFP4 keys
 * with dim == 128 and H_I in {16, 32, 48, 64}, iq 16-byte aligned and the
 * keys' e8m0 plane (pointer and strides) 4-byte aligned: each key's four
 * exponents are read as one 32-bit word. 1 <= k <= 4096.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t B;
    int32_t Tq;
    int32_t H_I;
    int32_t k;
    int32_t m;
    const int64_t *q_pos;
    const void *iq;
    const uint8_t *iq_scale;
    const float *w;
    const v4a_ik_store *keys;
    int32_t *out_idx;
    float *out_score;
} v4a_index_args;

size_t lightning_index_topk_workspace(const v4a_index_args *a);
int lightning_index_topk(const v4a_index_args *a, void *workspace, size_t workspace_bytes,
                         v4a_stream stream);

/* lightning_index_topk without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, results and errors as
 * lightning_index_topk; its scratch is a static device array of
 * V4A_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends), zero-filled
 * on the first call on each device (on that call's stream). A call needing more
 * scratch than that (lightning_index_topk_workspace() above the limit; about
 * 264 KB per query at 262,144 entries) returns V4A_EWORKSPACE before anything
 * is enqueued. It allocates nothing. All calls on one GPU share the array:
 * calls that overlap in time on one GPU (other streams or host threads) race. */
#define V4A_NOALLOC_SCRATCH_BYTES (32u << 20)
int lightning_index_topk_noalloc(const v4a_index_args *a, v4a_stream stream);

/* ------------------------------------------------------------------------
 * Attention over compressed entries plus the raw window, one KV head shared
 * by H_q query heads.
 *
 * For query (b, i) at t = q_pos[b][i], head h: q = RoPE(q[b][i][h], t);
 * logits sm_scale * (q . key) over the key list [entries] ++ [window rows];
 * one softmax; o = sum p * value. lse (optional) = log sum exp of the logits
 * (natural log). A query with an empty key list gets o = 0, lse = -inf.
 *
 *  q         [B][Tq][H_q][dim] in q_fmt (pre-RoPE).
 *  ent_k/v   entry stores (ring = 0); may be NULL for window-only use.
 *  m         compression ratio of the entries (visibility rule above).
 *  win_k/v   raw window rows, indexed by position (usually a ring; a ring
 *            needs at least W slots, else V4A_EINVAL).
 *  W         window length (0 .. 4096).
 *  sm_scale  logit scale; 0 means 1/sqrt(dim).
 *  o         [B][Tq][H_q][dim] in o_fmt.
 *  lse       [B][Tq][H_q] float32 or NULL.
 *  append_k/v  optional fused window append (decode): the query tokens' raw
 *          K and V rows [B][Tq][dim] bfloat16, 4-byte aligned. Each is first
 *          written into win_k/win_v at its query position t, with the bytes
 *          that csa_compress with m = 1 at pos0 = t writes (the pooling of
 *          one token is the identity; K is rotated at t), and the attention
 *          then sees it as the window row of t. Needs E4M3_BF16 stores,
 *          Tq == 1 and W >= 1 (else EFORMAT / EINVAL); both NULL: no append.
 *          A position past a linear window store's rows writes nothing.
 *          [chaosnode.de, "DeepSeek-V4: 1 Million Token Context endlich
 *          nutzbar", section "Hybrid Attention: CSA und HCA"]: the window
 *          of the last 128 raw tokens includes the current one.
 * Key lists (entries + window) of up to 2,097,152 keys per query (1024 splits
 * of 2048 keys); a longer one returns V4A_EINVAL and its *_workspace() 0.
 * Supported: all stores F32 with q and o float32, dim 128, H_q * dim <= 4096;
 * or all stores E4M3_BF16 with dim == 192, q bfloat16, o float32 or bfloat16,
 * and H_q in {16, 32, 48, 64}. (A bfloat16 output carries its own rounding of
 * 2^-8 relative per element; float32 keeps the kernel's full accuracy.)
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t B;
    int32_t Tq;
    int32_t H_q;
    int32_t dim;
    const int64_t *q_pos;
    int32_t q_fmt;
    const void *q;
    const v4a_kv_store *ent_k;
    const v4a_kv_store *ent_v;
    int32_t m;
    const v4a_kv_store *win_k;
    const v4a_kv_store *win_v;
    int32_t W;
    float sm_scale;
    double rope_base;
    int32_t o_fmt;
    void *o;
    float *lse;
    const void *append_k;
    const void *append_v;
} v4a_attn_args;

/* CSA: keys are the entries listed in topk_idx[b][i][0..k) (ids < 0 or not
 * below the store's rows are skipped), then the window. */
size_t sparse_window_attn_workspace(const v4a_attn_args *a, int32_t k);
int sparse_window_attn(const v4a_attn_args *a, const int32_t *topk_idx, int32_t k, void *workspace,
                       size_t workspace_bytes, v4a_stream stream);

/* HCA: keys are every visible entry (at most n_entries_override when it is
 * >= 0; 0 gives window-only attention), then the window. */
size_t hca_attn_workspace(const v4a_attn_args *a, int64_t n_entries_override);
int hca_attn(const v4a_attn_args *a, int64_t n_entries_override, void *workspace,
             size_t workspace_bytes, v4a_stream stream);

/* Bring a workspace into the initialised state (zero-fills it on `stream`).
 * Needed once after allocation, before its first use by any call above. */
int v4a_workspace_init(void *workspace, size_t workspace_bytes, v4a_stream stream);

/* Static text for a status code. */
const char *v4a_strerror(int status);
/* Message describing the calling thread's most recent failed call. */
const char *v4a_last_error(void);
/* Library version string. */
const char *v4a_version(void);

#ifdef __cplusplus
}
#endif

#endif /* V4ATTN_H */
