// Host side of the C ABI declared in include/gr_attn.h: argument validation,
// the work decomposition of the fused kernel, and launches on the caller's
// stream.  Nothing here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gr_attn.h"
#include "gr_attn_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// gfx950 check, cached per device ordinal (the only global state: immutable
// after first use).
int device_ok()
{
    static std::once_flag once;
    static int ok_mask[64];
    static int ndev = 0;
    std::call_once(once, [] {
        if (hipGetDeviceCount(&ndev) != hipSuccess)
            ndev = 0;
        if (ndev > 64)
            ndev = 64;
        for (int d = 0; d < ndev; ++d) {
            hipDeviceProp_t prop;
            ok_mask[d] = hipGetDeviceProperties(&prop, d) == hipSuccess &&
                         std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        }
    });
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ndev)
        return GR_ERR_DEVICE;
    return ok_mask[dev] ? GR_OK : GR_ERR_UNSUPPORTED;
}

int validate(const gr_decode_attn_dims *d)
{
    if (!d)
        return GR_ERR_NULL;
    if (d->B < 0 || d->R < 0 || d->Hq <= 0 || d->Hkv <= 0 || d->W_max < 0 || d->T_cap < 0 ||
        d->ctx_cap < 0 || d->beam_cap < 0 || d->reserved != 0)
        return GR_ERR_DIMS;
    if (d->flags != 0) {
        const int nqt = d->flags & 255, nks = (d->flags >> 8) & 255, sp = (d->flags >> 16) & 255;
        if ((d->flags & ~(GR_FLAG_TILING | GR_FLAG_ROW16 | 0xffffff)) != 0 ||
            !(d->flags & GR_FLAG_TILING) || nqt < 1 || nks < 1 || sp < 1 || sp > 8 ||
            ((d->flags & GR_FLAG_ROW16) && sp != 1))
            return GR_ERR_DIMS;
    }
    if (d->Hq % d->Hkv != 0)
        return GR_ERR_DIMS;
    if (!(d->scale >= 0.f) || std::isinf(d->scale))
        return GR_ERR_DIMS;
    if (d->D != 64 && d->D != 128)
        return GR_ERR_UNSUPPORTED;
    if (d->Hq / d->Hkv > 8)
        return GR_ERR_UNSUPPORTED;
    // index arithmetic of the kernels is 32-bit per request token index
    if (d->ctx_cap > INT32_MAX || d->beam_cap > INT32_MAX ||
        static_cast<int64_t>(d->W_max) * (d->Hq / d->Hkv) > INT32_MAX)
        return GR_ERR_DIMS;
    return GR_OK;
}

int validate_buffers(const gr_decode_attn_dims *d, const int32_t *row_offset, const void *q,
                     const void *ctx_k, const void *ctx_v, const int32_t *ctx_len,
                     const void *beam_k, const void *beam_v, const int32_t *beam_path,
                     const int32_t *beam_len, const void *out, const float *lse)
{
    if (d->B > 0 && (!row_offset || !ctx_len || !beam_len || !ctx_k || !ctx_v || !beam_k ||
                     !beam_v))
        return GR_ERR_NULL;
    if (d->R > 0 && (!q || !out || !lse || (!beam_path && d->T_cap > 0)))
        return GR_ERR_NULL;
    const void *bf[] = {q, ctx_k, ctx_v, beam_k, beam_v, out};
    for (const void *p : bf)
        if (p && !aligned16(p))
            return GR_ERR_ALIGN;
    if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) ||
        (beam_path && (reinterpret_cast<uintptr_t>(beam_path) & 3u)))
        return GR_ERR_ALIGN;
    return GR_OK;
}

gr::Params make_params(const gr_decode_attn_dims *d, const int32_t *row_offset, const void *q,
                       const void *ctx_k, const void *ctx_v, const int32_t *ctx_len,
                       const void *beam_k, const void *beam_v, const int32_t *beam_path,
                       const int32_t *beam_len, void *out, float *lse)
{
    gr::Params p{};
    p.q = static_cast<const uint16_t *>(q);
    p.ctx_k = static_cast<const uint16_t *>(ctx_k);
    p.ctx_v = static_cast<const uint16_t *>(ctx_v);
    p.beam_k = static_cast<const uint16_t *>(beam_k);
    p.beam_v = static_cast<const uint16_t *>(beam_v);
    p.ctx_len = ctx_len;
    p.beam_len = beam_len;
    p.beam_path = beam_path;
    p.row_offset = row_offset;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    p.B = d->B;
    p.R = d->R;
    p.Hq = d->Hq;
    p.Hkv = d->Hkv;
    p.G = d->Hq / d->Hkv;
    p.D = d->D;
    p.T_cap = d->T_cap;
    p.ctx_cap = d->ctx_cap;
    p.beam_cap = d->beam_cap;
    const double scale = d->scale > 0.f ? d->scale : 1.0 / std::sqrt((double)d->D);
    p.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
    return p;
}

// Work decomposition.  A workgroup covers 32*NQT stacked query rows of one
// (request, KV head) pair (a wave owns 32 rows) and splits its share of that
// pair's context over NKS key streams.  Wide query tiles share each K/V tile
// in LDS between more waves; more key streams keep the grid large when the
// stacks are short.  (4,1) is preferred: two of its workgroups share a
// compute unit, and as their barriers are independent the two waves of a
// SIMD drift out of phase, so one's softmax overlaps the other's matrix work
// (measured: 78 us against 96 us for (8,1) at 4 requests x 900 beams x 2048
// context tokens).  When its grid cannot fill the GPU (few pairs, short
// stacks), the context of each (pair, query tile) is split over n_split
// workgroups that combine their partials through the workspace; only when
// the context is too short for that do wider key streams take over.
struct Plan {
    int nqt, nks, n_split, n_qt, grid;
    bool row16 = false;   // waves of 16 stacked rows (gr_attn16.hip)
};

constexpr int kSIMDs = 256 * 4;
constexpr int kLdsBytes = 160 * 1024;     // LDS per compute unit
// The fused kernel's own static LDS (the block-wide vote of its re-sweep
// check and the split-arrival flag); the dynamic segment, aligned to 1 KB,
// starts after it.
constexpr int kStaticLds = 1024;
constexpr int kMaxSplit = 8;              // workgroups per (pair, query tile)
constexpr int kMinSplitTiles = 4;         // 32-key tiles each split sweeps, at least
constexpr int kKeyTile = 32;

bool tiling_fits(int D, int nqt, int nks, bool row16 = false)
{
    const int lds = row16 ? gr::fused16_lds_bytes(D, nqt, nks) : gr::fused_lds_bytes(D, nqt, nks);
    return lds > 0 && lds + kStaticLds <= kLdsBytes;
}

// "NQT,NKS[,SPLIT]" from GR_ATTN_TILE (tuning and tests), read once per
// process; a tiling that is not compiled or does not fit the LDS is ignored.
struct TileOverride {
    int nqt = 0, nks = 0, split = 0;
};
const TileOverride &tile_override()
{
    static const TileOverride o = [] {
        TileOverride t;
        const char *env = std::getenv("GR_ATTN_TILE");
        int a = 0, b = 0, c = 0;
        const int n = env ? std::sscanf(env, "%d,%d,%d", &a, &b, &c) : 0;
        if (n >= 2 && a > 0 && b > 0) {
            t.nqt = a;
            t.nks = b;
            t.split = n >= 3 && c > 0 ? (c < kMaxSplit ? c : kMaxSplit) : 1;
        }
        return t;
    }();
    return o;
}

Plan plan(const gr_decode_attn_dims *d)
{
    const int G = d->Hq / d->Hkv;
    const int64_t M = static_cast<int64_t>(d->W_max) * G;
    const int64_t pairs = static_cast<int64_t>(d->B) * d->Hkv;
    const int64_t n_tiles = (d->ctx_cap + kKeyTile - 1) / kKeyTile;
    const int64_t want = 7 * 2 * kSIMDs / 8;   // 7/8 of two waves per SIMD
    auto waves = [&](int nqt, int nks) {
        return pairs * ((M + 32 * nqt - 1) / (32 * nqt)) * nqt * nks;
    };
    Plan best{1, 4, 1, 0, 0};
    const TileOverride &o = tile_override();
    if (d->flags & GR_FLAG_TILING) {
        best.nqt = d->flags & 255;
        best.nks = (d->flags >> 8) & 255;
        best.n_split = (d->flags >> 16) & 255;
        best.row16 = (d->flags & GR_FLAG_ROW16) != 0;
        if (!tiling_fits(d->D, best.nqt, best.nks, best.row16))
            best.grid = -2;                     // not compiled or too large
    } else if (o.nqt > 0 && tiling_fits(d->D, o.nqt, o.nks)) {
        best.nqt = o.nqt;
        best.nks = o.nks;
        best.n_split = o.split;
    } else {
        static const int cand[][2] = {{4, 1}, {8, 1}, {4, 2}, {2, 2}, {2, 4}};
        bool chosen = false;
        if (tiling_fits(d->D, 4, 1)) {
            // A split pays only while its partials (written and read back
            // once per wave and split) stay well below the pair's ContextKV
            // bytes: measured at 8 requests x 128 beams x 1024 tokens, where
            // they are as large as the context, splits of 2 / 4 / 8 took 29 /
            // 38 / 58 us against 27 us for the (2,2) tiling without a split.
            const int64_t w = waves(4, 1);
            // waves with query rows write a partial (write + read back)
            const int64_t part_per_split =
                2 * ((M + 31) / 32) * static_cast<int64_t>(gr::fused_part_bytes(d->D));
            const int64_t ctx_bytes = d->ctx_cap * 4 * d->D;
            int s = 1;
            while (w * s < want && 2 * s <= kMaxSplit && n_tiles >= 2 * s * kMinSplitTiles &&
                   2 * s * part_per_split * 4 <= ctx_bytes)
                s *= 2;
            if (w * s >= want || s > 1) {
                best = Plan{4, 1, s, 0, 0};
                chosen = true;
            }
        }
        bool filled = chosen;
        for (const auto &c : cand) {
            if (chosen)
                break;
            if (!tiling_fits(d->D, c[0], c[1]))
                continue;
            best.nqt = c[0];
            best.nks = c[1];
            best.n_split = 1;
            if (waves(c[0], c[1]) >= want) {
                filled = true;
                break;
            }
        }
        // Few stacked rows per pair: waves of 16 rows, two key streams and
        // beam waves.  Measured at 8 requests x 128 beams (G = 2, 1024
        // tokens): 23.2 us against 28.3 us for the (2,2) tiling, and at one
        // request of 4 beams 5.3 us against 8.1 us; where a 32-row tiling
        // fills two waves per SIMD it is 1.4-1.5 times slower (its LDS reads
        // per row double).
        if (!filled && tiling_fits(d->D, 4, 2, true)) {
            best = Plan{4, 2, 1, 0, 0};
            best.row16 = true;
        }
    }
    if (best.grid == -2)
        return best;
    const int rows = best.row16 ? 16 * best.nqt : 32 * best.nqt;   // stacked rows per workgroup
    best.n_qt = static_cast<int>((M + rows - 1) / rows);
    const int64_t pairs_per_xcd = (pairs + 7) / 8;
    const int64_t grid = 8 * pairs_per_xcd * best.n_qt * best.n_split;
    best.grid = grid > INT32_MAX ? -1 : static_cast<int>(grid);
    return best;
}

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

hipError_t launch_plan(const gr::Params &p, const Plan &pl, void *stream)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return pl.row16 ? gr::launch_fused16(p, pl.nqt, pl.nks, pl.grid, s)
                    : gr::launch_fused(p, pl.nqt, pl.nks, pl.grid, s);
}

// Workspace layout of a plan: arrival counters, then the wave partials.
size_t workspace_bytes(const gr_decode_attn_dims *d, const Plan &pl)
{
    if (pl.n_split <= 1 || pl.grid <= 0)
        return 0;
    const size_t units = static_cast<size_t>(d->B) * d->Hkv * pl.n_qt;
    return align256(units * sizeof(int32_t)) +
           units * pl.n_split * pl.nqt * static_cast<size_t>(gr::fused_part_bytes(d->D));
}

// Checks the dims' workspace against the plan and points the kernel
// parameters at it.
int bind_workspace(const gr_decode_attn_dims *d, const Plan &pl, gr::Params &p)
{
    p.n_split = pl.n_split;
    const size_t need = workspace_bytes(d, pl);
    if (need == 0)
        return GR_OK;
    if (!d->workspace || d->workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(d->workspace) & 255u))
        return GR_ERR_WORKSPACE;
    const size_t units = static_cast<size_t>(d->B) * d->Hkv * pl.n_qt;
    char *w = static_cast<char *>(d->workspace);
    p.ws_count = reinterpret_cast<int32_t *>(w);
    p.ws_part = w + align256(units * sizeof(int32_t));
    return GR_OK;
}

}  // namespace

extern "C" {

size_t gr_decode_attn_workspace_bytes(const gr_decode_attn_dims *d)
{
    if (validate(d) != GR_OK || d->R == 0 || d->B == 0 || d->W_max == 0)
        return 0;
    return workspace_bytes(d, plan(d));
}

int gr_decode_attn_plan(const gr_decode_attn_dims *d, int32_t plan_out[5])
{
    if (!plan_out)
        return GR_ERR_NULL;
    const int st = validate(d);
    if (st != GR_OK)
        return st;
    for (int i = 0; i < 5; ++i)
        plan_out[i] = 0;
    if (d->R == 0 || d->B == 0 || d->W_max == 0)
        return GR_OK;
    const Plan pl = plan(d);
    if (pl.grid < 0)
        return pl.grid == -2 ? GR_ERR_UNSUPPORTED : GR_ERR_DIMS;
    plan_out[0] = pl.nqt;
    plan_out[1] = pl.nks;
    plan_out[2] = pl.n_split;
    plan_out[3] = pl.row16 ? 1 : 0;
    plan_out[4] = pl.grid;
    return GR_OK;
}

int gr_decode_attn(const gr_decode_attn_dims *d, const int32_t *row_offset, const void *q,
                   const void *ctx_k, const void *ctx_v, const int32_t *ctx_len,
                   const void *beam_k, const void *beam_v, const int32_t *beam_path,
                   const int32_t *beam_len, void *out, float *lse, void *stream)
{
    int st = validate(d);
    if (st != GR_OK)
        return st;
    st = validate_buffers(d, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path,
                          beam_len, out, lse);
    if (st != GR_OK)
        return st;
    if (d->R == 0 || d->B == 0 || d->W_max == 0)
        return GR_OK;
    gr::Params p = make_params(d, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v,
                               beam_path, beam_len, out, lse);
    const Plan pl = plan(d);
    if (pl.grid < 0)
        return pl.grid == -2 ? GR_ERR_UNSUPPORTED : GR_ERR_DIMS;
    p.n_qt = pl.n_qt;
    st = bind_workspace(d, pl, p);
    if (st != GR_OK)
        return st;
    if (pl.grid == 0)
        return GR_OK;
    st = device_ok();
    if (st != GR_OK)
        return st;
    const hipError_t e = launch_plan(p, pl, stream);
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

int gr_decode_attn_noalloc(const gr_decode_attn_dims *d, const int32_t *row_offset,
                           const void *q, const void *ctx_k, const void *ctx_v,
                           const int32_t *ctx_len, const void *beam_k, const void *beam_v,
                           const int32_t *beam_path, const int32_t *beam_len, void *out,
                           float *lse, void *stream)
{
    int st = validate(d);
    if (st != GR_OK)
        return st;
    st = validate_buffers(d, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path,
                          beam_len, out, lse);
    if (st != GR_OK)
        return st;
    if (d->R == 0 || d->B == 0 || d->W_max == 0)
        return GR_OK;
    gr::Params p = make_params(d, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v,
                               beam_path, beam_len, out, lse);
    const Plan pl = plan(d);
    if (pl.grid < 0)
        return pl.grid == -2 ? GR_ERR_UNSUPPORTED : GR_ERR_DIMS;
    p.n_qt = pl.n_qt;
    p.n_split = pl.n_split;
    if (pl.grid == 0)
        return GR_OK;
    // the split's counters and partials must fit the fixed scratch layout
    const size_t units = static_cast<size_t>(d->B) * d->Hkv * pl.n_qt;
    const size_t part = units * pl.n_split * pl.nqt * static_cast<size_t>(gr::fused_part_bytes(d->D));
    if (pl.n_split > 1 && (units * sizeof(int32_t) > gr::NOALLOC_COUNTER_BYTES ||
                           part > gr::NOALLOC_SCRATCH_BYTES - gr::NOALLOC_COUNTER_BYTES))
        return GR_ERR_WORKSPACE;
    st = device_ok();
    if (st != GR_OK)
        return st;
    if (pl.n_split > 1) {
        void *sp = nullptr;
        if (gr::noalloc_scratch(&sp, static_cast<hipStream_t>(stream)) != hipSuccess)
            return GR_ERR_DEVICE;
        p.ws_count = static_cast<int32_t *>(sp);
        p.ws_part = static_cast<char *>(sp) + gr::NOALLOC_COUNTER_BYTES;
    }
    const hipError_t e = launch_plan(p, pl, stream);
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

int gr_decode_attn_paged(const gr_decode_attn_dims *d, const gr_paged_ctx *c,
                         const int32_t *row_offset, const void *q, const int32_t *ctx_len,
                         const void *beam_k, const void *beam_v, const int32_t *beam_path,
                         const int32_t *beam_len, void *out, float *lse, void *stream)
{
    int st = validate(d);
    if (st != GR_OK)
        return st;
    if (!c)
        return GR_ERR_NULL;
    if (c->page_size <= 0 || c->page_size % 16 != 0 || c->pages_per_req <= 0 ||
        c->n_pages <= 0 || c->n_pages > INT32_MAX ||
        d->ctx_cap > static_cast<int64_t>(c->pages_per_req) * c->page_size)
        return GR_ERR_DIMS;
    if (d->B > 0 && (!c->k_pages || !c->v_pages || !c->page_table))
        return GR_ERR_NULL;
    if ((c->k_pages && !aligned16(c->k_pages)) || (c->v_pages && !aligned16(c->v_pages)) ||
        (reinterpret_cast<uintptr_t>(c->page_table) & 3u))
        return GR_ERR_ALIGN;
    st = validate_buffers(d, row_offset, q, c->k_pages, c->v_pages, ctx_len, beam_k, beam_v,
                          beam_path, beam_len, out, lse);
    if (st != GR_OK)
        return st;
    if (d->R == 0 || d->B == 0 || d->W_max == 0)
        return GR_OK;
    gr::Params p = make_params(d, row_offset, q, c->k_pages, c->v_pages, ctx_len, beam_k, beam_v,
                               beam_path, beam_len, out, lse);
    p.page_table = c->page_table;
    p.page_size = c->page_size;
    p.pages_per_req = c->pages_per_req;
    p.n_pages = c->n_pages;
    const Plan pl = plan(d);
    if (pl.grid < 0)
        return pl.grid == -2 ? GR_ERR_UNSUPPORTED : GR_ERR_DIMS;
    p.n_qt = pl.n_qt;
    st = bind_workspace(d, pl, p);
    if (st != GR_OK)
        return st;
    if (pl.grid == 0)
        return GR_OK;
    st = device_ok();
    if (st != GR_OK)
        return st;
    const hipError_t e = launch_plan(p, pl, stream);
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

int gr_decode_attn_generic(const gr_decode_attn_dims *d, const int32_t *row_offset,
                           const void *q, const void *ctx_k, const void *ctx_v,
                           const int32_t *ctx_len, const void *beam_k, const void *beam_v,
                           const int32_t *beam_path, const int32_t *beam_len, void *out,
                           float *lse, void *stream)
{
    int st = validate(d);
    if (st != GR_OK)
        return st;
    st = validate_buffers(d, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v, beam_path,
                          beam_len, out, lse);
    if (st != GR_OK)
        return st;
    if (d->ctx_cap + d->T_cap > gr::GENERIC_MAX_KEYS)
        return GR_ERR_UNSUPPORTED;
    if (d->R == 0 || d->B == 0)
        return GR_OK;
    st = device_ok();
    if (st != GR_OK)
        return st;
    const gr::Params p = make_params(d, row_offset, q, ctx_k, ctx_v, ctx_len, beam_k, beam_v,
                                     beam_path, beam_len, out, lse);
    const hipError_t e = gr::launch_generic(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

int gr_check_metadata(const gr_decode_attn_dims *d, const int32_t *row_offset,
                      const int32_t *ctx_len, const int32_t *beam_path,
                      const int32_t *beam_len, int32_t *violations, void *stream)
{
    int st = validate(d);
    if (st != GR_OK)
        return st;
    if (!violations || (d->B > 0 && (!row_offset || !ctx_len || !beam_len)) ||
        (d->R > 0 && d->T_cap > 0 && !beam_path))
        return GR_ERR_NULL;
    st = device_ok();
    if (st != GR_OK)
        return st;
    gr::MetaCheck c{};
    c.row_offset = row_offset;
    c.ctx_len = ctx_len;
    c.beam_len = beam_len;
    c.beam_path = beam_path;
    c.violations = violations;
    c.B = d->B;
    c.R = d->R;
    c.W_max = d->W_max;
    c.T_cap = d->T_cap;
    c.ctx_cap = d->ctx_cap;
    c.beam_cap = d->beam_cap;
    const hipError_t e = gr::launch_check(c, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

int gr_beam_step(const gr_beam_step_dims *d, const int32_t *row_offset_old,
                 const int32_t *row_offset_new, const int32_t *parent, const int32_t *path_old,
                 const int32_t *beam_len_old, const void *new_k, const void *new_v,
                 int32_t *path_new, int32_t *beam_len_new, void *beam_k, void *beam_v,
                 int32_t *violations, void *stream)
{
    if (!d)
        return GR_ERR_NULL;
    if (d->B < 0 || d->R_old < 0 || d->R_new < 0 || d->Hkv <= 0 || d->T_cap < 0 ||
        d->W_cap < 0 || d->beam_cap < 0 || d->reserved != 0)
        return GR_ERR_DIMS;
    if (d->D != 64 && d->D != 128)
        return GR_ERR_UNSUPPORTED;
    if (d->B > 0 && (!row_offset_old || !row_offset_new || !beam_len_old || !beam_len_new))
        return GR_ERR_NULL;
    if (d->R_new > 0 && (!parent || !new_k || !new_v || !beam_k || !beam_v ||
                         (d->T_cap > 0 && !path_new)))
        return GR_ERR_NULL;
    if (d->R_old > 0 && d->T_cap > 0 && !path_old)
        return GR_ERR_NULL;
    const void *bf[] = {new_k, new_v, beam_k, beam_v};
    for (const void *p : bf)
        if (p && !aligned16(p))
            return GR_ERR_ALIGN;
    const void *i32[] = {row_offset_old, row_offset_new, parent, path_old, beam_len_old,
                         path_new, beam_len_new, violations};
    for (const void *p : i32)
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u))
            return GR_ERR_ALIGN;
    // the step reads path_old / beam_len_old while it writes path_new /
    // beam_len_new: the ranges must be disjoint
    auto overlap = [](const void *a, int64_t na, const void *b, int64_t nb) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
        return a && b && na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
    };
    if (overlap(path_old, (int64_t)d->R_old * d->T_cap * 4, path_new,
                (int64_t)d->R_new * d->T_cap * 4) ||
        overlap(beam_len_old, (int64_t)d->B * 4, beam_len_new, (int64_t)d->B * 4))
        return GR_ERR_DIMS;
    if (d->B == 0)
        return GR_OK;
    int st = device_ok();
    if (st != GR_OK)
        return st;
    gr::StepParams p{};
    p.row_offset_old = row_offset_old;
    p.row_offset_new = row_offset_new;
    p.parent = parent;
    p.path_old = path_old;
    p.len_old = beam_len_old;
    p.new_k = static_cast<const uint16_t *>(new_k);
    p.new_v = static_cast<const uint16_t *>(new_v);
    p.path_new = path_new;
    p.len_new = beam_len_new;
    p.beam_k = static_cast<uint16_t *>(beam_k);
    p.beam_v = static_cast<uint16_t *>(beam_v);
    p.violations = violations;
    p.B = d->B;
    p.R_old = d->R_old;
    p.R_new = d->R_new;
    p.Hkv = d->Hkv;
    p.D = d->D;
    p.T_cap = d->T_cap;
    p.W_cap = d->W_cap;
    p.beam_cap = d->beam_cap;
    const hipError_t e = gr::launch_beam_step(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

size_t gr_beam_select_workspace_bytes(const gr_beam_select_dims *d)
{
    if (!d || d->R_old < 0 || d->K_max <= 0)
        return 0;
    return gr::beam_select_workspace(d->R_old, d->K_max);
}

static int beam_select_common(const gr_beam_select_dims *d, const gr_sid_trie *trie,
                              const int32_t *row_offset_old, const int32_t *row_offset_new,
                              const float *score_old, const float *logits,
                              const int32_t *node_old, float *score_new, int32_t *parent,
                              int32_t *token, int32_t *node_new, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    if (!d)
        return GR_ERR_NULL;
    if (d->B < 0 || d->R_old < 0 || d->R_new < 0 || d->V <= 0 || d->K_max <= 0 ||
        d->reserved != 0)
        return GR_ERR_DIMS;
    if (d->V > gr::SEL_MAX_V || d->K_max > gr::SEL_MAX_K ||
        static_cast<int64_t>(d->R_old) * d->V > INT32_MAX)
        return GR_ERR_UNSUPPORTED;
    if (trie) {
        if (trie->n_nodes < 1 || trie->n_edges < 0 || trie->max_fanout < 1 ||
            trie->max_fanout > d->V || trie->reserved != 0)
            return GR_ERR_DIMS;
        if (!trie->node_ptr || (trie->n_edges > 0 && (!trie->edge_tok || !trie->edge_child)))
            return GR_ERR_NULL;
        if ((d->R_old > 0 && !node_old) || (d->R_new > 0 && !node_new))
            return GR_ERR_NULL;
    }
    if (d->B > 0 && (!row_offset_old || !row_offset_new))
        return GR_ERR_NULL;
    if (d->R_old > 0 && (!score_old || !logits))
        return GR_ERR_NULL;
    if (d->R_new > 0 && (!score_new || !parent || !token))
        return GR_ERR_NULL;
    const size_t need = gr_beam_select_workspace_bytes(d);
    if (need > 0 && !workspace)
        return GR_ERR_NULL;
    if (workspace_bytes < need)
        return GR_ERR_DIMS;
    const void *al4[] = {row_offset_old, row_offset_new, score_old, logits, score_new, parent,
                         token, node_old, node_new,
                         trie ? trie->node_ptr : nullptr, trie ? trie->edge_tok : nullptr,
                         trie ? trie->edge_child : nullptr};
    for (const void *p : al4)
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u))
            return GR_ERR_ALIGN;
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GR_ERR_ALIGN;
    if (d->B == 0)
        return GR_OK;
    int st = device_ok();
    if (st != GR_OK)
        return st;
    gr::SelParams p{};
    p.row_offset_old = row_offset_old;
    p.row_offset_new = row_offset_new;
    p.score_old = score_old;
    p.logits = logits;
    p.score_new = score_new;
    p.parent = parent;
    p.token = token;
    {
        auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
        char *w = static_cast<char *>(workspace);
        const size_t R = static_cast<size_t>(d->R_old);
        p.ws_list = reinterpret_cast<uint64_t *>(w);
        w += al(R * gr::SEL_LIST * sizeof(uint64_t));
        p.ws_off = reinterpret_cast<float *>(w);
        w += al(R * sizeof(float));
        p.ws_ovf = reinterpret_cast<int32_t *>(w);
        w += al(R * sizeof(int32_t));
        p.ws_surv = reinterpret_cast<uint64_t *>(w);
        w += al(R * static_cast<size_t>(d->K_max) * sizeof(uint64_t));
        p.ws_n = reinterpret_cast<int32_t *>(w);
        w += al(R * sizeof(int32_t));
        p.ws_e0 = reinterpret_cast<int32_t *>(w);
    }
    if (trie) {
        p.node_ptr = trie->node_ptr;
        p.edge_tok = trie->edge_tok;
        p.edge_child = trie->edge_child;
        p.n_nodes = trie->n_nodes;
        p.n_edges = trie->n_edges;
        p.max_fanout = trie->max_fanout;
        p.node_old = node_old;
        p.node_new = node_new;
    }
    p.B = d->B;
    p.R_old = d->R_old;
    p.R_new = d->R_new;
    p.V = d->V;
    p.K_max = d->K_max;
    const hipError_t e = gr::launch_beam_select(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GR_OK : GR_ERR_LAUNCH;
}

int gr_beam_select(const gr_beam_select_dims *d, const int32_t *row_offset_old,
                   const int32_t *row_offset_new, const float *score_old, const float *logits,
                   float *score_new, int32_t *parent, int32_t *token, void *workspace,
                   size_t workspace_bytes, void *stream)
{
    return beam_select_common(d, nullptr, row_offset_old, row_offset_new, score_old, logits,
                              nullptr, score_new, parent, token, nullptr, workspace,
                              workspace_bytes, stream);
}

int gr_beam_select_trie(const gr_beam_select_dims *d, const gr_sid_trie *trie,
                        const int32_t *row_offset_old, const int32_t *row_offset_new,
                        const float *score_old, const float *logits, const int32_t *node_old,
                        float *score_new, int32_t *parent, int32_t *token, int32_t *node_new,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    if (!trie)
        return GR_ERR_NULL;
    return beam_select_common(d, trie, row_offset_old, row_offset_new, score_old, logits,
                              node_old, score_new, parent, token, node_new, workspace,
                              workspace_bytes, stream);
}

const char *gr_status_str(int status)
{
    switch (status) {
    case GR_OK: return "ok";
    case GR_ERR_NULL: return "a required pointer is NULL";
    case GR_ERR_DIMS: return "inconsistent or out-of-range dimensions";
    case GR_ERR_UNSUPPORTED: return "unsupported configuration or device";
    case GR_ERR_ALIGN: return "misaligned tensor pointer";
    case GR_ERR_LAUNCH: return "kernel launch failed";
    case GR_ERR_DEVICE: return "HIP device query failed";
    case GR_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    default: return "unknown status";
    }
}

int gr_version(void) { return 200; }

}  // extern "C"
