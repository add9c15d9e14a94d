// Internal interface between the host-side API and the device code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr {

// Everything a kernel needs about one call (passed by value).
struct Params {
    const uint16_t *q, *ctx_k, *ctx_v, *beam_k, *beam_v;
    const int32_t *ctx_len, *beam_len, *beam_path, *row_offset;
    uint16_t *out;
    float *lse;
    int B, R, Hq, Hkv, G, D, T_cap;
    int64_t ctx_cap, beam_cap;
    float scale_log2;   // softmax scale * log2(e)
    int n_qt;           // query tiles per (request, KV head) pair in the fused grid
    // Cross-workgroup context split (fused kernel): the n_split workgroups of
    // one (pair, query tile) unit each sweep 1/n_split of the context and
    // leave fp32 partials in ws_part; the last to arrive (counted in
    // ws_count[unit], which it resets to 0) combines them.  n_split == 1:
    // no workspace is touched.
    int n_split;
    int32_t *ws_count;  // [pairs * n_qt] arrival counters, zero between calls
    char *ws_part;      // [pairs * n_qt][n_split][NQT] wave partials of fused_part_bytes(D)
    // Paged ContextKV (fused kernel only): when page_table is set, ctx_k /
    // ctx_v are page pools [n_pages][page_size][Hkv][D] and token j of request
    // b is row j % page_size of page page_table[b * pages_per_req + j / page_size].
    const int32_t *page_table;
    int page_size, pages_per_req;
    int64_t n_pages;
};

struct MetaCheck {
    const int32_t *row_offset, *ctx_len, *beam_len, *beam_path;
    int32_t *violations;
    int B, R, W_max, T_cap;
    int64_t ctx_cap, beam_cap;
};

// One beam step (BeamKV append + BeamPath update).
struct StepParams {
    const int32_t *row_offset_old, *row_offset_new, *parent, *path_old, *len_old;
    const uint16_t *new_k, *new_v;
    int32_t *path_new, *len_new;
    uint16_t *beam_k, *beam_v;
    int32_t *violations;   // may be null
    int B, R_old, R_new, Hkv, D, T_cap, W_cap;
    int64_t beam_cap;
};

// Beam selection (log_softmax + top-K over beams x vocabulary).
constexpr int SEL_MAX_V = 16384;   // vocabulary held in registers by one workgroup
constexpr int SEL_MAX_K = 1024;    // beams kept per request (one sort in registers)
constexpr int SEL_LIST = 32;       // best keys kept per row for the request stage
struct SelParams {
    const int32_t *row_offset_old, *row_offset_new;
    const float *score_old, *logits;
    float *score_new;
    int32_t *parent, *token;
    uint64_t *ws_list;   // [R_old][SEL_LIST] each row's best keys, descending
    float *ws_off;       // [R_old] score_old - LSE of each row
    int32_t *ws_ovf;     // [R_old] rows to select again, per request from row_offset_old[b]
    uint64_t *ws_surv;   // [R_old][K_max] survivors, per request from row_offset_old[b]*K_max
    int32_t *ws_n;       // [R_old] candidates of each row (V when unconstrained)
    int32_t *ws_e0;      // [R_old] first trie edge of each row's node
    // item-constrained selection (node_ptr == nullptr: every token is legal)
    const int32_t *node_ptr, *edge_tok, *edge_child;
    const int32_t *node_old;   // [R_old] trie node of each beam (-1: none)
    int32_t *node_new;         // [R_new]
    int n_nodes, n_edges, max_fanout;
    int B, R_old, R_new, V, K_max;
};
// Workspace bytes of the six tables above (each 256-byte aligned).
inline size_t beam_select_workspace(int R_old, int K_max)
{
    auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
    const size_t R = static_cast<size_t>(R_old);
    return al(R * SEL_LIST * sizeof(uint64_t)) + al(R * sizeof(float)) +
           al(R * sizeof(int32_t)) + al(R * static_cast<size_t>(K_max) * sizeof(uint64_t)) +
           2 * al(R * sizeof(int32_t));
}

// Longest key list the generic comparator keeps in LDS.
constexpr int GENERIC_MAX_KEYS = 16320;

// Fused-kernel instantiations: (head dim, query waves per stream NQT, key
// streams NKS, LDS tile buffers per stream NBUF, target waves per SIMD OCC).
// A workgroup has NQT*NKS waves and covers 32*NQT stacked query rows.
#define GR_FOR_EACH_FUSED_CONFIG(X)                                            \
    X(128, 8, 1, 4, 2) X(128, 4, 1, 4, 2) X(128, 4, 2, 4, 2) X(128, 2, 2, 4, 2)    \
    X(64, 4, 1, 4, 2) X(64, 2, 2, 4, 2) X(64, 2, 4, 3, 2)

// LDS of the fused kernel (host and device agree on it): the ring of NKS *
// NBUF context tiles of FUSED_KT keys (K then V rows, D bf16 each), which the
// beam gathers and the merge of the key streams reuse, then the staged
// BeamPath entries.
constexpr int FUSED_KT = 32;
constexpr int FUSED_PTAB_BYTES = 4096;
constexpr int fused_lds_main(int D, int nqt, int nks, int nbuf)
{
    const int tile = 2 * FUSED_KT * D * 2;
    const int stage = nks * nbuf * tile;
    const int oslot = 32 * (D + 4) * 4 + 32 * 16;  // one wave's O partial + (max, sums)
    const int merge = (nks - 1) * nqt * oslot;
    return stage > merge ? stage : merge;
}
constexpr int fused_lds_total(int D, int nqt, int nks, int nbuf)
{
    return fused_lds_main(D, nqt, nks, nbuf) + FUSED_PTAB_BYTES;
}
// The 16-row-wave kernel (gr_attn16.hip): NQT waves of 16 stacked query
// rows per key stream; its merge slot is a wave's O^T in lane order.
// Columns: (head dim, NQT, NKS, NBUF, OCC, BW).  BW = 1 adds NQT beam waves,
// one per query tile, which fold the BeamKV steps of the tile's rows while
// the NQT*NKS sweep waves run the context; their partials merge with the
// key streams' through LDS (one slot per key stream past the first and per
// beam wave, in the tile ring's space).
#define GR_FOR_EACH_FUSED16_CONFIG(X)                                          \
    X(128, 4, 2, 4, 3, 1) X(128, 8, 1, 4, 4, 0) X(128, 4, 1, 4, 4, 0)             \
    X(128, 6, 1, 4, 3, 0) X(128, 2, 2, 4, 2, 0) X(64, 4, 2, 4, 3, 1) X(64, 8, 1, 4, 4, 0)
constexpr int fused16_lds_main(int D, int nqt, int nks, int nbuf, int bw)
{
    const int stage = nks * nbuf * 2 * FUSED_KT * D * 2;
    const int merge = (nks - 1 + bw) * nqt * (D / 16 + 1) * 64 * 16;
    return stage > merge ? stage : merge;
}
inline int fused16_lds_bytes(int D, int nqt, int nks)
{
#define GR_LDS16_CASE(d, a, c, nb, oc, bw)                                            \
    if (D == d && nqt == a && nks == c)                                               \
        return fused16_lds_main(d, a, c, nb, bw);
    GR_FOR_EACH_FUSED16_CONFIG(GR_LDS16_CASE)
#undef GR_LDS16_CASE
    return -1;
}
hipError_t launch_fused16(const Params &p, int nqt, int nks, int grid, hipStream_t s);

// Dynamic LDS of a compiled (D, NQT, NKS) instantiation, -1 if not compiled.
inline int fused_lds_bytes(int D, int nqt, int nks)
{
#define GR_LDS_CASE(d, a, c, nb, oc)                                                  \
    if (D == d && nqt == a && nks == c)                                               \
        return fused_lds_total(d, a, c, nb);
    GR_FOR_EACH_FUSED_CONFIG(GR_LDS_CASE)
#undef GR_LDS_CASE
    return -1;
}
// Bytes of one wave's partial result in the split workspace: the unnormalised
// O^T fragments (D/2 floats per lane) and (max, sum, sum) per lane, in the
// wave's own lane order (16-byte vectors, lane-contiguous).
constexpr int fused_part_bytes(int D) { return (D / 8 + 1) * 64 * 16; }
hipError_t launch_fused(const Params &p, int nqt, int nks, int grid, hipStream_t s);
// Scratch of gr_decode_attn_noalloc, per device: fixed layout, the split
// counters in the first NOALLOC_COUNTER_BYTES (never reused for partials, so
// they stay zero between calls), the partials after them.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
constexpr size_t NOALLOC_COUNTER_BYTES = (size_t)64 << 10;
// The current device's scratch address (looked up once per device; the
// counters are cleared by a kernel on `s` before the first use).
hipError_t noalloc_scratch(void **out, hipStream_t s);
hipError_t launch_generic(const Params &p, hipStream_t s);
hipError_t launch_check(const MetaCheck &c, hipStream_t s);
hipError_t launch_beam_step(const StepParams &p, hipStream_t s);
hipError_t launch_beam_select(const SelParams &p, hipStream_t s);

}  // namespace gr
