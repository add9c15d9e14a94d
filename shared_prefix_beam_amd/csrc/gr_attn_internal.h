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
size_t beam_select_workspace(int R_old, int K_max);

// Longest key list the generic comparator keeps in LDS.
constexpr int GENERIC_MAX_KEYS = 16320;

// Fused-kernel instantiations: (head dim, query waves per stream NQT, key
// streams NKS, LDS tile buffers per stream NBUF, target waves per SIMD OCC).
// A workgroup has NQT*NKS waves and covers 32*NQT stacked query rows.
#define GR_FOR_EACH_FUSED_CONFIG(X)                                            \
    X(128, 8, 1, 4, 2) X(128, 4, 1, 4, 2) X(128, 4, 2, 4, 2) X(128, 2, 2, 4, 2)    \
    X(64, 4, 1, 4, 2) X(64, 2, 2, 4, 2) X(64, 2, 4, 3, 2)

int fused_lds_bytes(int D, int nqt, int nks);
hipError_t launch_fused(const Params &p, int nqt, int nks, int grid, hipStream_t s);
hipError_t launch_generic(const Params &p, hipStream_t s);
hipError_t launch_check(const MetaCheck &c, hipStream_t s);
hipError_t launch_beam_step(const StepParams &p, hipStream_t s);
hipError_t launch_beam_select(const SelParams &p, hipStream_t s);

}  // namespace gr
