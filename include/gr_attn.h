/*
 * gr_attn.h -- C ABI of the MI355X (gfx950) decode-attention library for
 * large-beam generative recommendation.
 *
 * The operation (GR-Inference blog on developer.nvidia.cn, section on kernel
 * design; xGR paper review on xllm-io, section "xAttention", three-stage
 * computation; SID-GR Inference README, section "Design Highlights"):
 *
 *   Every request b owns one long ContextKV written at prefill and shared by
 *   all of its W_b live beams, plus short per-beam BeamKV tokens reached
 *   through a BeamPath index table.  For every packed query row r of request
 *   b and every query head h (KV head g = h / (Hq/Hkv)), the library computes
 *   softmax attention over the concatenation
 *       ContextKV tokens 0 .. ctx_len[b]-1            (shared stage)
 *    ++ BeamKV tokens beam_path[r][0 .. beam_len[b]-1]  (per-beam stage)
 *   and combines the two parts by their log-sum-exp (merge stage):
 *       out[r][h][:] = sum_j softmax_j(scale * q.K_j) V_j        (bf16)
 *       lse[r][h]    = ln sum_j exp(scale * q.K_j)               (fp32)
 *   A row with no key at all gets out = 0 and lse = -inf.
 *
 * Layouts (all row-major, contiguous; bf16 = raw 16-bit bfloat16):
 *   q          bf16  [R][Hq][D]                 query rows of all requests, packed
 *   ctx_k/v    bf16  [B][ctx_cap][Hkv][D]       dense ContextKV per request
 *   ctx_len    int32 [B]                        0 <= ctx_len[b] <= ctx_cap
 *   beam_k/v   bf16  [B][beam_cap][Hkv][D]      BeamKV pool per request
 *   beam_path  int32 [R][T_cap]                 per-request BeamKV token indices
 *   beam_len   int32 [B]                        0 <= beam_len[b] <= T_cap
 *   row_offset int32 [B+1]                      request b owns rows
 *                                               row_offset[b] .. row_offset[b+1]-1
 *   out        bf16  [R][Hq][D]
 *   lse        fp32  [R][Hq]                    natural log, scale included
 *
 * Ownership and threading: the caller owns every buffer (device memory,
 * except the dims struct, which is host memory and is read during the call
 * only), including the workspace (see gr_decode_attn_workspace_bytes).  A
 * call only enqueues work on `stream` (a hipStream_t; NULL = the null stream)
 * and returns; it never allocates, frees, copies between host and device,
 * synchronises, or reads device memory from the host, so it may be captured
 * into a HIP graph.  The library keeps no mutable global state:
 * concurrent calls on different streams are safe as long as their out/lse
 * buffers differ.  out and lse must not alias any input.
 *
 * Errors: every entry point returns GR_OK (0) or a negative GR_ERR_* code and
 * then has enqueued nothing, except GR_ERR_LAUNCH, which reports a failed
 * kernel launch.  GR_ERR_WORKSPACE: the dims' workspace is NULL, smaller than
 * gr_decode_attn_workspace_bytes(dims) or not 256-byte aligned.
 * Device-resident metadata (ctx_len, beam_len, row_offset, beam_path) is not
 * read by the host: its bounds above are preconditions.
 * gr_check_metadata() verifies them on the device when a caller cannot
 * guarantee them.
 */
#ifndef GR_ATTN_H
#define GR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GR_OK = 0,
    GR_ERR_NULL = -1,        /* a required pointer is NULL */
    GR_ERR_DIMS = -2,        /* inconsistent sizes (Hq % Hkv, R < 0, scale < 0, ...) */
    GR_ERR_UNSUPPORTED = -3, /* D not 64/128, G > 8, no gfx950 device, ... */
    GR_ERR_ALIGN = -4,       /* a bf16 tensor pointer is not 16-byte aligned */
    GR_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
    GR_ERR_DEVICE = -6,      /* a HIP runtime query failed */
    GR_ERR_WORKSPACE = -7    /* workspace NULL, too small or not 256-byte aligned */
};

/* Sizes of one call.  Host memory; read only during the call. */
typedef struct gr_decode_attn_dims {
    int32_t B;        /* requests (>= 0) */
    int32_t R;        /* packed query rows = row_offset[B] (>= 0) */
    int32_t Hq;       /* query heads */
    int32_t Hkv;      /* KV heads; Hq % Hkv == 0 and G = Hq / Hkv <= 8 */
    int32_t D;        /* head dim: 64 or 128 */
    int32_t W_max;    /* upper bound on any request's row count W_b (>= 0) */
    int32_t T_cap;    /* row stride of beam_path; upper bound on beam_len[b] */
    int32_t reserved; /* must be 0 */
    int64_t ctx_cap;  /* ContextKV tokens per request in ctx_k / ctx_v */
    int64_t beam_cap; /* BeamKV tokens per request in beam_k / beam_v */
    float scale;      /* softmax scale applied to q.k; 0 selects 1/sqrt(D) */
    int32_t flags;    /* 0 (the library plans the work), or GR_TILING(...) */
    void *workspace;  /* DEVICE scratch owned by the caller (see below); may be
                         NULL when gr_decode_attn_workspace_bytes() is 0 */
    uint64_t workspace_bytes; /* size of `workspace` in bytes */
} gr_decode_attn_dims;

/*
 * Per-call choice of the work decomposition, for tuning and tests (dims
 * flags; 0 lets the library choose): workgroups of nqt query waves (32
 * stacked query rows each) by nks key streams, with each (request, KV head,
 * query tile) unit's context split over n_split workgroups.  nqt, nks in
 * 1 .. 255, n_split in 1 .. 8 (1 with GR_FLAG_ROW16); a tiling the library
 * does not compile, or whose LDS does not fit, gives GR_ERR_UNSUPPORTED.  The
 * result is the same (up to rounding order) for every tiling.
 */
#define GR_FLAG_TILING 0x40000000
#define GR_TILING(nqt, nks, n_split) \
    ((int32_t)(GR_FLAG_TILING | (nqt) | ((nks) << 8) | ((n_split) << 16)))
/* The same with waves of 16 stacked query rows instead of 32 (more waves per
 * SIMD for short stacks; no context split across workgroups). */
#define GR_FLAG_ROW16 0x20000000
#define GR_TILING16(nqt, nks) ((int32_t)(GR_TILING(nqt, nks, 1) | GR_FLAG_ROW16))

/*
 * Workspace gr_decode_attn / gr_decode_attn_paged need for these sizes, in
 * bytes (0 when the call is planned without a cross-workgroup context split).
 * The pages split the long ContextKV over several workers (Split-KV:
 * GR-Inference blog, section on kernel design); when the (request, KV head)
 * pairs alone cannot fill the GPU and each pair has few query rows for its
 * context length, the library splits each pair's context over several
 * workgroups, which leave fp32 partial results (unnormalised output, running
 * maximum and sums) in the workspace, and the last of them to finish combines
 * them by log-sum-exp.  Layout: arrival counters first, then the partials;
 * it is private to the library.
 *
 * Contract: the caller allocates at least this many bytes, 256-byte aligned,
 * and ZERO-FILLS it once before its first use (the counters must start at
 * zero; every completed call leaves them at zero again, so later calls,
 * including graph replays, need no clearing).  One workspace must not be used
 * by two calls that can run at the same time.  The size depends only on
 * the dims (and on the GR_ATTN_TILE tuning override, read once per process).
 * Returns 0 for a NULL or invalid dims.
 */
size_t gr_decode_attn_workspace_bytes(const gr_decode_attn_dims *dims);

/*
 * The work decomposition gr_decode_attn / gr_decode_attn_paged plan for these
 * dims, by the same rules (for reporting and tuning; the pages leave the
 * decomposition to the implementation).  On GR_OK, plan (host memory, 5
 * int32) holds: [0] nqt, [1] nks, [2] n_split, [3] 1 for waves of 16 stacked
 * query rows (0: 32), [4] the launch's workgroup count (all 0 when the call
 * has nothing to compute).  Errors as gr_decode_attn for invalid dims
 * (GR_ERR_NULL also for a NULL plan; GR_ERR_UNSUPPORTED for a forced tiling
 * the library does not compile); no device is touched.
 */
int gr_decode_attn_plan(const gr_decode_attn_dims *dims, int32_t plan[5]);

/*
 * Large-beam decode attention (shared ContextKV stage on bf16 MFMA with an
 * online softmax, per-beam BeamPath gather, log-sum-exp merge), one launch
 * on `stream`.  row_offset is a DEVICE pointer to int32[B+1]; it is a
 * positional argument (not a dims field) because it is device memory that a
 * decode loop updates every step, while the dims struct holds host values.
 * The ContextKV of each (request, KV head) is read from HBM once per call
 * rather than once per beam.  dims->workspace must hold
 * gr_decode_attn_workspace_bytes(dims) bytes (see there).
 */
int gr_decode_attn(const gr_decode_attn_dims *dims, const int32_t *row_offset,
                   const void *q, const void *ctx_k, const void *ctx_v,
                   const int32_t *ctx_len, const void *beam_k, const void *beam_v,
                   const int32_t *beam_path, const int32_t *beam_len, void *out,
                   float *lse, void *stream);

/*
 * gr_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid allocation.
 * Same arguments, results, ownership of the caller's buffers and errors as
 * gr_decode_attn, except that dims->workspace and dims->workspace_bytes are
 * ignored: when the call is planned with a context split, its counters and
 * partials live in a scratch array inside the library, one per device (16 MiB,
 * held until the process ends; its address is looked up once per device on
 * that device's first call, which also clears its counters with a kernel on
 * `stream`).  A call whose split would not fit the scratch (more than 16384
 * (request, KV head, query tile) units, or partials beyond 16 MiB - 64 KiB)
 * returns GR_ERR_WORKSPACE and enqueues nothing.  Nothing is allocated or
 * freed.  Every call on one device shares that device's scratch: two calls
 * that can run at the same time on one device (different streams, or
 * different host threads) race and may give wrong results; callers order
 * them (one stream) or use gr_decode_attn with a workspace each.
 */
int gr_decode_attn_noalloc(const gr_decode_attn_dims *dims, const int32_t *row_offset,
                           const void *q, const void *ctx_k, const void *ctx_v,
                           const int32_t *ctx_len, const void *beam_k, const void *beam_v,
                           const int32_t *beam_path, const int32_t *beam_len, void *out,
                           float *lse, void *stream);

/*
 * The same operation computed the way a generic decode-attention kernel
 * does it: every (row, head) independently reads its request's whole
 * ContextKV (SID-GR README, section "Performance Breakdown": the
 * general path treats B x W beams as independent decode rows).  Same
 * arguments, layouts and results; kept as an in-library comparator.
 * Requires ctx_cap + T_cap <= 16384; needs no workspace (the dims' workspace
 * fields are ignored).
 */
int gr_decode_attn_generic(const gr_decode_attn_dims *dims, const int32_t *row_offset,
                           const void *q, const void *ctx_k, const void *ctx_v,
                           const int32_t *ctx_len, const void *beam_k, const void *beam_v,
                           const int32_t *beam_path, const int32_t *beam_len, void *out,
                           float *lse, void *stream);

/* Paged ContextKV: fixed-size pages of a shared pool.  Host memory; read
 * only during the call (the pointers are DEVICE pointers). */
typedef struct gr_paged_ctx {
    const void *k_pages;       /* bf16 [n_pages][page_size][Hkv][D] */
    const void *v_pages;       /* bf16 [n_pages][page_size][Hkv][D] */
    const int32_t *page_table; /* int32 [B][pages_per_req]: page of each request's
                                  logical page j (tokens j*page_size ..) */
    int32_t page_size;         /* tokens per page: a positive multiple of 16 */
    int32_t pages_per_req;     /* row stride of page_table */
    int64_t n_pages;           /* pages in each pool (>= 1) */
} gr_paged_ctx;

/*
 * gr_decode_attn with the ContextKV read through a page table instead of a
 * dense per-request slice.  Page tables in decode attention are on the SID-GR
 * roadmap (SID-GR README, "Roadmap").  Token j < ctx_len[b] of request b is
 * row j % page_size of page page_table[b][j / page_size]; within a page the
 * rows have the dense layout ([Hkv][D] per token).  Every other argument,
 * the result, the ownership and the errors are those of gr_decode_attn;
 * dims->ctx_cap must not exceed pages_per_req * page_size and bounds
 * ctx_len.  Entries of page_table for tokens < ctx_len[b] must lie in
 * [0, n_pages) (an entry outside is clamped into the pool: wrong data, no
 * access outside the buffers).
 */
int gr_decode_attn_paged(const gr_decode_attn_dims *dims, const gr_paged_ctx *ctx,
                         const int32_t *row_offset, const void *q, const int32_t *ctx_len,
                         const void *beam_k, const void *beam_v, const int32_t *beam_path,
                         const int32_t *beam_len, void *out, float *lse, void *stream);

/*
 * Device-side check of the metadata preconditions above: row_offset is
 * non-decreasing with row_offset[0] = 0, row_offset[B] = R and every
 * W_b <= W_max; every ctx_len[b] in [0, ctx_cap]; every beam_len[b] in
 * [0, T_cap]; every used beam_path entry in [0, beam_cap).  Writes the number
 * of violations (0 = valid) to the DEVICE int32 *violations; enqueued on
 * `stream` like the other calls.
 */
int gr_check_metadata(const gr_decode_attn_dims *dims, const int32_t *row_offset,
                      const int32_t *ctx_len, const int32_t *beam_path,
                      const int32_t *beam_len, int32_t *violations, void *stream);

/* Sizes of one beam step.  Host memory; read only during the call. */
typedef struct gr_beam_step_dims {
    int32_t B;        /* requests (>= 0) */
    int32_t R_old;    /* rows before the step = row_offset_old[B] (>= 0) */
    int32_t R_new;    /* rows after beam selection = row_offset_new[B] (>= 0) */
    int32_t Hkv;      /* KV heads (>= 1) */
    int32_t D;        /* head dim: 64 or 128 */
    int32_t T_cap;    /* row stride of both BeamPath tables (>= 0) */
    int32_t W_cap;    /* BeamKV slots per step: step s, beam k -> s * W_cap + k */
    int32_t reserved; /* must be 0 */
    int64_t beam_cap; /* BeamKV tokens per request in beam_k / beam_v (>= 0) */
} gr_beam_step_dims;

/*
 * One decode step of the per-beam state: BeamKV append and BeamPath update.
 * BeamKV keeps each beam's short decode history.  BeamPath records how beams
 * fork and reorder by index, so that beam selection never copies KV (GR-Inference
 * blog, section on system design; SID-GR README, "Design Highlights": BeamPath
 * keeps the parent-child relation).  The history is reached token by token through
 * direct indices (xGR review, section "xAttention", KV cache management).
 *
 * Request b had W_old = row_offset_old[b+1] - row_offset_old[b] beams with
 * paths of s = beam_len_old[b] tokens.  Beam selection left it W_new =
 * row_offset_new[b+1] - row_offset_new[b] beams.  New beam k (packed row
 * r = row_offset_new[b] + k) descends from old beam parent[r] of request b
 * (read only when s > 0), and its current token is step s:
 *   path_new[r][t]              = path_old[row_offset_old[b] + parent[r]][t]   t < s
 *   path_new[r][s]              = s * W_cap + k
 *   beam_k[b][s * W_cap + k][:] = new_k[r][:]      (all KV heads; beam_v likewise)
 *   beam_len_new[b]             = W_new > 0 ? s + 1 : s
 * Nothing else is written: entries t > s of path_new and every other BeamKV
 * slot keep their contents.  The paths go to a second table, so no row is
 * overwritten before another reads it.
 *
 * Layouts (row-major, contiguous; DEVICE memory except dims):
 *   row_offset_old, row_offset_new  int32 [B+1]
 *   parent                          int32 [R_new]
 *   path_old                        int32 [R_old][T_cap]
 *   path_new                        int32 [R_new][T_cap]
 *   beam_len_old, beam_len_new      int32 [B]
 *   new_k, new_v                    bf16  [R_new][Hkv][D]
 *   beam_k, beam_v                  bf16  [B][beam_cap][Hkv][D], updated in place
 *   violations                      int32 [1] or NULL
 *
 * A row whose step or slot is out of range (s >= T_cap, k >= W_cap,
 * s * W_cap + k >= beam_cap), or with s > 0 and parent[r] outside
 * [0, W_old), writes nothing.  When violations is not NULL, the number of
 * such rows is added to *violations (the caller zeroes it).
 *
 * path_new must not overlap path_old, and beam_len_new must not overlap
 * beam_len_old (both are checked: GR_ERR_DIMS).  new_k / new_v must not overlap
 * beam_k / beam_v.  Ownership, threading, graph capture and the other error codes
 * are as for gr_decode_attn.  Writes are bit copies, so results are exact.
 */
int gr_beam_step(const gr_beam_step_dims *dims, const int32_t *row_offset_old,
                 const int32_t *row_offset_new, const int32_t *parent,
                 const int32_t *path_old, const int32_t *beam_len_old, const void *new_k,
                 const void *new_v, int32_t *path_new, int32_t *beam_len_new, void *beam_k,
                 void *beam_v, int32_t *violations, void *stream);

/* Sizes of one beam selection.  Host memory; read only during the call. */
typedef struct gr_beam_select_dims {
    int32_t B;        /* requests (>= 0) */
    int32_t R_old;    /* beam rows before the step = row_offset_old[B] (>= 0) */
    int32_t R_new;    /* beams kept = row_offset_new[B] (>= 0) */
    int32_t V;        /* vocabulary: logits per row, 1 .. 16384 */
    int32_t K_max;    /* upper bound on any request's kept beams, 1 .. 1024 */
    int32_t reserved; /* must be 0 */
} gr_beam_select_dims;

/* Workspace gr_beam_select needs for these sizes (bytes, 256-byte aligned). */
size_t gr_beam_select_workspace_bytes(const gr_beam_select_dims *dims);

/*
 * Beam selection of one decode step: log_softmax + top-K over every (beam,
 * token) candidate of a request, with early-terminated sorting.  Sorting
 * stops for a beam once its candidates fall below the beam width's least
 * kept element (xGR review, section "xBeam"); log_softmax, top-K and
 * selection run on the device (SID-GR README, "Roadmap").
 *
 * Request b had W_old = row_offset_old[b+1] - row_offset_old[b] beams with
 * cumulative scores score_old (natural-log probabilities).  It keeps
 * K_b = row_offset_new[b+1] - row_offset_new[b] <= K_max beams: the K_b best
 * candidates (w, v), w < W_old, v < V, valued
 *     score_old[w] + logits[w][v] - ln sum_u exp(logits[w][u])      (fp32)
 * ranked by value (larger first) and, among equal values, by w*V + v
 * (smaller first).  For k < K_b the packed outputs at row_offset_new[b] + k are
 *     score_new = the value, parent = w (beam within the request), token = v,
 * in rank order.  A request with fewer than K_b candidates (or more than
 * K_max to keep) fills the rest with (-inf, -1, -1).  (parent, token) feed
 * gr_beam_step and the next decode step.
 *
 * Layouts (DEVICE memory except dims): row_offset_old, row_offset_new int32
 * [B+1]; score_old fp32 [R_old]; logits fp32 [R_old][V] (every row with at
 * least one finite logit); score_new fp32 [R_new]; parent, token int32
 * [R_new]; workspace of gr_beam_select_workspace_bytes(dims) bytes (caller-
 * owned, not shared by concurrent calls).  Values are computed in fp32:
 * candidates within rounding of each other may rank in either order.  Other
 * properties as for gr_decode_attn (GR_ERR_DIMS for a short workspace).
 */
int gr_beam_select(const gr_beam_select_dims *dims, const int32_t *row_offset_old,
                   const int32_t *row_offset_new, const float *score_old, const float *logits,
                   float *score_new, int32_t *parent, int32_t *token, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Item catalog as a prefix trie of semantic-ID tokens in CSR form, resident
 * in device memory (GR-Inference blog, kernel design: the SID trie stored as
 * CSR).  Node 0 is the root.  Node u's children are edges node_ptr[u] ..
 * node_ptr[u+1]-1; edge e carries token edge_tok[e] (in [0, V), strictly
 * increasing within a node) and leads to node edge_child[e].  max_fanout
 * bounds every node's child count (1 .. V): it sizes the launch, and a node
 * with more children has only its first max_fanout considered.
 */
typedef struct gr_sid_trie {
    const int32_t *node_ptr;   /* DEVICE int32 [n_nodes + 1] */
    const int32_t *edge_tok;   /* DEVICE int32 [n_edges] */
    const int32_t *edge_child; /* DEVICE int32 [n_edges] */
    int32_t n_nodes;           /* >= 1 */
    int32_t n_edges;           /* >= 0 */
    int32_t max_fanout;        /* 1 .. V */
    int32_t reserved;          /* must be 0 */
} gr_sid_trie;

/*
 * Item-constrained beam selection: gr_beam_select where beam w's candidates
 * are only the legal next tokens, the labels of the edges leaving its trie
 * node node_old[w] (none if node_old[w] is -1 or out of range).  The prefix
 * traversal, the gather of the legal logits and the top-K run in one call
 * (GR-Inference blog, kernel design: item-constrained fused kernel; xGR
 * review, section "xBeam").  A legal candidate (w, t) is valued
 *     score_old[w] + logits[w][t] - ln sum_{legal u} exp(logits[w][u])
 * (log_softmax over the legal tokens: every other logit masked to -inf),
 * ranked and packed as in gr_beam_select.  node_new[k] is the trie node of
 * the kept beam's prefix extended by its token (the child on that edge),
 * -1 for padding: the next step's node_old.  Only the legal logits of a row
 * are read.
 *
 * Layouts as gr_beam_select, plus node_old int32 [R_old] and node_new int32
 * [R_new] (DEVICE); trie is host memory holding device pointers.  The same
 * workspace size applies.  Errors as gr_beam_select; a NULL or inconsistent
 * trie (n_nodes < 1, n_edges < 0, max_fanout outside 1 .. V, reserved != 0)
 * gives GR_ERR_NULL or GR_ERR_DIMS.  Trie contents are read as given:
 * out-of-range node or edge ranges are clamped (wrong results, no access
 * outside the arrays); labels outside [0, V) count as -inf logits.
 */
int gr_beam_select_trie(const gr_beam_select_dims *dims, const gr_sid_trie *trie,
                        const int32_t *row_offset_old, const int32_t *row_offset_new,
                        const float *score_old, const float *logits, const int32_t *node_old,
                        float *score_new, int32_t *parent, int32_t *token, int32_t *node_new,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *gr_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int gr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GR_ATTN_H */
