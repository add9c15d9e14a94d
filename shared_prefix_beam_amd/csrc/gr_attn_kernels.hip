// Device code of the gfx950 large-beam decode-attention library.
//
// The method (GR-Inference blog, section on kernel design; xGR paper review,
// section "xAttention"): per (request, KV head), attention over a long
// ContextKV that all beams share is computed once for the whole stack of
// beam query rows on the matrix cores, split over the context length; each
// beam's few BeamKV tokens are gathered along its BeamPath on the vector
// units; the parts are combined through their log-sum-exp.
//
// gfx950 mapping of the fused kernel (one launch does all three stages):
//   * A workgroup owns one (request b, KV head g) pair and a tile of
//     32*NQT stacked query rows: stacked row m = beam * G + i is query head
//     g*G+i of beam `beam`.  Its NQT*NKS waves form NKS key streams of NQT
//     waves; stream ks walks a contiguous 1/NKS share of the context in
//     32-key tiles.  Tiles move HBM -> LDS with direct loads (no register
//     staging), NBUF-deep, with one workgroup barrier per tile.
//   * Each wave holds 32 query columns.  Scores are produced transposed,
//     S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16: the A operand is a K tile
//     fragment read from LDS, the B operand is the wave's Q^T kept in
//     registers for the whole pass.  In the 32x32 accumulator layout every
//     lane holds 16 keys of ONE query, so a row maximum is an in-lane max
//     chain plus one v_permlane32_swap.
//   * Probabilities are rounded to bf16 in registers and fed straight back
//     as the B operand of O^T += V^T * P^T.  The keys' order inside that
//     contraction is the order in which the accumulator layout holds them;
//     the matching V^T operand comes from transposing LDS reads
//     (ds_read_b64_tr_b16) of the row-major V tile, so P never leaves
//     registers and V is never transposed in memory.
//   * Softmax in the log2 domain against a per-query reference maximum that
//     stays fixed during the context sweep (the first tile's maximum), so the
//     O^T accumulators are written only by the matrix cores inside the loop;
//     a second, exact sweep runs only if a row sum leaves the safe range.
//   * BeamKV steps are spread over the key streams; before its context
//     sweep, each stream folds its steps into its own (max, sum, O) from
//     rows gathered along the BeamPath into the still empty tile ring; that
//     partial seeds the accumulators, and the streams merge through LDS by
//     log-sum-exp at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "gr_attn_internal.h"
#include "gr_attn_device.h"

namespace gr {

template <int D, int NQT, int NKS, int NBUF, int OCC, bool PAGED>
__global__ __launch_bounds__(64 * NQT * NKS) __attribute__((amdgpu_waves_per_eu(OCC)))
void fused_decode_attn(const Params p)
{
    using Gm = Geo<D>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // ---- work item: (pair, query tile), XCD-aware ----------------------
    // Workgroups are dispatched round-robin over the 8 XCDs; all query tiles
    // of one (request, KV head) pair go to the same XCD so that its L2 holds
    // the pair's ContextKV for every tile.
    // With a context split, the n_split workgroups of one (pair, query tile)
    // unit have consecutive ids on the XCD, so they run together and their
    // partials meet in that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int j = bid >> 3;
    const int per_pair = p.n_qt * p.n_split;
    const int pair = (j / per_pair) * 8 + xcd;
    const int qtile = (j % per_pair) / p.n_split;
    const int split = j % p.n_split;
    if (pair >= p.B * p.Hkv)
        return;
    const int b = pair / p.Hkv;
    const int g = pair - b * p.Hkv;
    const int G = p.G;
    const int r0 = p.row_offset[b];
    const int Wb = p.row_offset[b + 1] - r0;
    const int M = Wb * G;
    const int tile_row0 = qtile * 32 * NQT;
    if (tile_row0 >= M)
        return;                                   // uniform for the workgroup
    const int L = p.ctx_len[b];
    const int T = p.beam_len[b];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int lane = tid & 63;
    const int qt = wave % NQT;
    const int ks = wave / NQT;
    // global key stream: the unit's n_split * NKS streams share its context
    const int gs = split * NKS + ks;
    const int GS = p.n_split * NKS;
    const int h = lane >> 5;
    const int c32 = lane & 31;
    const int wrow0 = tile_row0 + qt * 32;        // first stacked row of this wave
    const bool wave_live = wrow0 < M;

    // ---- the lane's query column and its Q^T fragments (B operand) -------
    const int m_row = wrow0 + c32;
    const bool qvalid = m_row < M;
    const int beam = qvalid ? m_row / G : 0;
    const int qhead = g * G + (qvalid ? m_row - beam * G : 0);
    const int qrow = r0 + beam;
    u32x4 qf[Gm::DC];
    {
        const uint16_t *src = p.q + ((int64_t)qrow * p.Hq + qhead) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < Gm::DC; ++c)
            qf[c] = qvalid ? ldg16(src + 16 * c) : u32x4{0, 0, 0, 0};
    }

    // ---- BeamPath entries of the workgroup's beams, staged in LDS ---------
    // Loaded with Q, so that the beam stage after the context sweep finds
    // its gather indices in LDS instead of waiting on memory for them.  The
    // tile's beam beta (beam tile_row0/G + beta) keeps step s at entry
    // beta*T + s; entries of beams past the request's last are 0.
    constexpr int NTHR = 64 * NQT * NKS;
    constexpr int PT_PER = (PTAB_BYTES / 4 + NTHR - 1) / NTHR;
    int32_t *const ptab_l = reinterpret_cast<int32_t *>(smem + lds_main<D, NQT, NKS, NBUF>());
    const int nb_wg = (32 * NQT) / G;             // the tile's beams (G divides 32)
    const bool use_tab = (32 % G == 0) && T > 0 && nb_wg * T * 4 <= PTAB_BYTES;
    const int beam0 = tile_row0 / G;
    int ptv[PT_PER];
#pragma unroll
    for (int i = 0; i < PT_PER; ++i) {
        const int e = tid + i * NTHR;
        const int beta = use_tab ? e / T : 0;
        const int sidx = e - beta * T;
        const bool ok = use_tab && e < nb_wg * T && beam0 + beta < Wb;
        ptv[i] = ok ? p.beam_path[(int64_t)(r0 + beam0 + beta) * p.T_cap + sidx] : 0;
    }
    // consume the loads here, so that no wait for them is left inside the
    // tile loop (where it would also wait for the tile prefetches)
#pragma unroll
    for (int c = 0; c < Gm::DC; ++c)
        asm volatile("" : "+v"(qf[c]));
#pragma unroll
    for (int i = 0; i < PT_PER; ++i) {
        const int e = tid + i * NTHR;
        if (use_tab && e < nb_wg * T)
            ptab_l[e] = ptv[i];                    // read after the next barrier
    }

    float m_ref = NEG_INF;                        // reference maximum, log2 units
    // this lane-half's share of the row sum, twice: l_run adds the bf16
    // values the matrix cores multiply (it normalises the output, so the
    // weights sum to one exactly); l_lse adds the unrounded values (it
    // gives the log-sum-exp, free of the bf16 rounding of the weights)
    float l_run = 0.f;
    float l_lse = 0.f;
    f32x16 acc[Gm::DB];
    f32x16 o[Gm::DB];                             // vector-unit copy (beam stage, merge)
#pragma unroll
    for (int db = 0; db < Gm::DB; ++db) {
        acc[db] = f32x16{};
        o[db] = f32x16{};
    }
    const float cs = p.scale_log2;

    // ---- shared (context) stage -----------------------------------------
    const int n_tiles = (L + KT - 1) / KT;
    const int t_begin = (gs * n_tiles) / GS;
    const int n_mine = ((gs + 1) * n_tiles) / GS - t_begin;
    const int iters = (n_tiles + GS - 1) / GS;    // same for every wave (barrier count)
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    const uint32_t stream_off = ks * (NBUF * Gm::TILE);        // byte offset of this stream
    // dense: request b's slice; paged: the pools (pages are located per load)
    const uint16_t *kv_k = p.ctx_k + ((PAGED ? 0 : (int64_t)b * p.ctx_cap * p.Hkv) + g) * D;
    const uint16_t *kv_v = p.ctx_v + ((PAGED ? 0 : (int64_t)b * p.ctx_cap * p.Hkv) + g) * D;
    const int kv_tok = p.Hkv * D;                 // elements between consecutive tokens
    const int32_t *ptab = PAGED ? p.page_table + (int64_t)b * p.pages_per_req : nullptr;
    // element offset, within a pool, of token `tok`'s row (KV head 0): the
    // rows of one page are consecutive, as in the dense layout.  A page index
    // outside the pool is clamped into it (a broken table reads wrong data,
    // never outside the buffer).
    // Page arithmetic without integer division when the page size is a
    // power of two (a runtime divide costs dozens of scalar instructions,
    // and every tile needs two).
    const int ps = PAGED ? p.page_size : 1;
    const bool ps_pow2 = (ps & (ps - 1)) == 0;
    const int ps_shift = __builtin_ctz((unsigned)ps);
    auto page_idx = [&](int tok) { return ps_pow2 ? tok >> ps_shift : tok / ps; };
    auto page_off = [&](int tok) { return ps_pow2 ? (tok & (ps - 1)) : tok % ps; };
    // An entry outside the pool is clamped into it (the pool size fits 32
    // bits): a broken table reads wrong data, never outside the buffer.
    const int pg_last = PAGED ? (int)(p.n_pages - 1) : 0;
    auto page_clamp = [&](int pg) { return pg < 0 ? 0 : (pg > pg_last ? pg_last : pg); };
    auto page_entry = [&](int tok) -> int {    // wave-uniform table read
        return ((const __attribute__((address_space(4))) int32_t *)(uintptr_t)ptab)[page_idx(tok)];
    };
    // element offset of row `tok - sub` in the pool, `tok` lying in page `pg`
    auto page_base = [&](int pg, int tok, int sub) -> int64_t {
        return ((int64_t)page_clamp(pg) * ps + page_off(tok) - sub) * kv_tok;
    };
    constexpr int RPL = 1024 / Gm::ROW;           // rows covered by one 1 KB load
    constexpr int LPW = (Gm::LOADS + NQT - 1) / NQT;   // loads per wave per tile (max)

    // Direct loads of a stream tile: this wave issues loads u = qt + i*NQT.
    // Load u < LOADS/2 fills K rows, the rest V rows; lane `lane` of load u
    // writes tile row r = (u % (LOADS/2))*RPL + lane/CH, slot lane%CH, with
    // the chunk that the row's swizzle puts there.  Its byte offset from the
    // tile's first token is loop-invariant for full tiles.
    uint32_t loff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int u = qt + i * NQT;
        const bool is_v = u >= Gm::LOADS / 2;
        const int uu = is_v ? u - Gm::LOADS / 2 : u;
        const int r = uu * RPL + lane / Gm::CH;
        const int c = (lane % Gm::CH) ^ (is_v ? vswz<D>(r) : kswz<D>(r));
        loff[i] = (uint32_t)(r * kv_tok + 8 * c) * 2u;
    }
    // Every load index u < LOADS when NQT divides LOADS (all configurations
    // but the guard keeps other shapes correct).
    constexpr bool EVEN = Gm::LOADS % NQT == 0;
    auto issue_tile = [&](int t, int buf) {
        const int key0 = (t_begin + t) * KT;
        const uint32_t dst0 = lds0 + stream_off + buf * Gm::TILE;
        if constexpr (PAGED) {
            // Rows past the context end repeat row L-1, each lane finding
            // its page.
            if (key0 + KT <= L) {
                // the tile's first and last 16 keys each lie in one page
                // (page sizes are multiples of 16, tiles start at multiples
                // of 32): one wave-uniform base per half, the lane offsets
                // the dense ones
                const int64_t base0 = page_base(page_entry(key0), key0, 0);
                const int64_t base1 = page_base(page_entry(key0 + 16), key0 + 16, 16);
#pragma unroll
                for (int i = 0; i < LPW; ++i) {
                    const int u = qt + i * NQT;
                    if (EVEN || u < Gm::LOADS) {
                        const bool is_v = u >= Gm::LOADS / 2;
                        const int uu = is_v ? u - Gm::LOADS / 2 : u;
                        dma16_s((is_v ? kv_v : kv_k) + (uu * RPL < 16 ? base0 : base1), loff[i],
                                dst0 + (is_v ? Gm::KBYTES : 0) + uu * 1024);
                    }
                }
            } else {
                // the context's last tile: per-lane rows and pages, one load
                // at a time (rolled, so that no address is held across loads)
#pragma unroll 1
                for (int i = 0; i < LPW; ++i) {
                    const int u = qt + i * NQT;
                    if (!EVEN && u >= Gm::LOADS)
                        break;
                    const bool is_v = u >= Gm::LOADS / 2;
                    const int uu = is_v ? u - Gm::LOADS / 2 : u;
                    const int r = uu * RPL + lane / Gm::CH;
                    const int c = (lane % Gm::CH) ^ (is_v ? vswz<D>(r) : kswz<D>(r));
                    const int tok = key0 + r < L ? key0 + r : L - 1;
                    const int64_t row = page_base(ptab[page_idx(tok)], tok, 0);
                    dma16((is_v ? kv_v : kv_k) + row + 8 * c,
                          dst0 + (is_v ? Gm::KBYTES : 0) + uu * 1024);
                }
            }
            return;
        }
        if (key0 + KT <= L) {
            // full tile: loop-invariant offsets, no per-lane arithmetic
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int u = qt + i * NQT;
                if (EVEN || u < Gm::LOADS) {
                    const bool is_v = u >= Gm::LOADS / 2;
                    const int uu = is_v ? u - Gm::LOADS / 2 : u;
                    dma16_s((is_v ? kv_v : kv_k) + (int64_t)key0 * kv_tok, loff[i],
                            dst0 + (is_v ? Gm::KBYTES : 0) + uu * 1024);
                }
            }
        } else {
            // the context's last, partial tile: rows past the end repeat row
            // L-1 (their scores are masked and their probabilities are 0)
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int u = qt + i * NQT;
                if (EVEN || u < Gm::LOADS) {
                    const bool is_v = u >= Gm::LOADS / 2;
                    const int uu = is_v ? u - Gm::LOADS / 2 : u;
                    const int r = uu * RPL + lane / Gm::CH;
                    const int rr = key0 + r < L ? r : L - 1 - key0;
                    const uint32_t off = loff[i] - (uint32_t)((r - rr) * kv_tok) * 2u;
                    dma16_s((is_v ? kv_v : kv_k) + (int64_t)key0 * kv_tok, off,
                            dst0 + (is_v ? Gm::KBYTES : 0) + uu * 1024);
                }
            }
        }
    };
    // loads this wave issues per tile (waves of a stream share LOADS)
    const int my_loads = EVEN ? Gm::LOADS / NQT : (Gm::LOADS - qt + NQT - 1) / NQT;
    // wait until at most `pending` later tiles of this wave are still loading
    auto wait_tiles = [&](int pending) {
        const int n = pending > 0 ? pending * my_loads : 0;
        if (n >= 48)
            wait_vm<48>();
        else if (n >= 32)
            wait_vm<32>();
        else if (n >= 16)
            wait_vm<16>();
        else if (n >= 8)
            wait_vm<8>();
        else if (n >= 4)
            wait_vm<4>();
        else if (n >= 2)
            wait_vm<2>();
        else
            wait_vm<0>();
    };

    // Loop-invariant per-lane LDS byte offsets (stream base included), so
    // that every fragment read is one instruction with an immediate offset.
    // K: lane row c32, d chunk 2c+h.  V (transposing reads): lane group
    // (h, dh) reads keys 16kc+4h+{0..3} (then +8) at d = 32db+16dh+{0..15};
    // the row swizzle depends only on key & 3, the same for all four keys of
    // a read, so kc and the +8 rows are immediate offsets too.
    uint32_t koff[Gm::DC];
#pragma unroll
    for (int c = 0; c < Gm::DC; ++c)
        koff[c] = stream_off + c32 * Gm::ROW + 16 * ((2 * c + h) ^ kswz<D>(c32));
    uint32_t voff[Gm::DB];
    {
        const int dh = (lane >> 4) & 1;
        const int sl = lane & 15;
        const int key_a = 4 * h + (sl >> 2);
#pragma unroll
        for (int db = 0; db < Gm::DB; ++db) {
            const int cidx = 4 * db + 2 * dh + ((sl & 3) >> 1);
            voff[db] = stream_off + Gm::KBYTES + key_a * Gm::ROW + 16 * (cidx ^ vswz<D>(key_a)) +
                       8 * (sl & 1);
        }
    }

    // Per-tile compute of a live wave on LDS buffer BUF.  ACCUM: p =
    // exp2(s*c - m_ref) against the fixed reference; otherwise only the exact
    // maxima are tracked.  The accumulators are written only by the matrix
    // cores, on every iteration of the compute loop, so they stay in
    // accumulation registers.
    auto compute_tile = [&](int it, auto buf_tag, bool want_max, auto accum_tag) {
        constexpr bool ACCUM = decltype(accum_tag)::value;
        constexpr int BUF = decltype(buf_tag)::value;
        const char *kl = smem + BUF * Gm::TILE;
        const int kbase = (t_begin + it) * KT;
        // S^T = K * Q^T
        f32x16 s = f32x16{};
#pragma unroll
        for (int c = 0; c < Gm::DC; ++c) {
            const u32x4 kf = *reinterpret_cast<const u32x4 *>(kl + koff[c]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                        __builtin_bit_cast(bf16x8, qf[c]), s, 0,
                                                        0, 0);
        }
        if (kbase + KT > L) {                      // keys past the context end
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
                if (key >= L)
                    s[r] = NEG_INF;
            }
        }
        if (want_max) {
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                mx = __builtin_fmaxf(mx, s[r]);
            mx = __builtin_fmaxf(mx, swap32(mx, h));
            m_ref = __builtin_fmaxf(m_ref, mx * cs);
        }
        if constexpr (ACCUM) {
            // probabilities as bf16 B operands; l_run adds the rounded
            // values, l_lse the unrounded ones
            u32x4 pb[2];
            const float nm = -m_ref;
            float sum = l_run, sum_x = l_lse;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 8 * kc + 2 * e;
                    const float p0 = exp2_fast(__builtin_fmaf(s[r], cs, nm));
                    const float p1 = exp2_fast(__builtin_fmaf(s[r + 1], cs, nm));
                    const uint32_t pk = pack_bf16(p0, p1);
                    pb[kc][e] = pk;
                    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                          __builtin_bit_cast(bf16x2, BF16_ONES),
                                                          sum, false);
                    sum_x += p0 + p1;
                }
            l_run = sum;
            l_lse = sum_x;
            // O^T += V^T * P^T
#pragma unroll
            for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const char *va_p = kl + voff[db] + 16 * kc * Gm::ROW;
                    const i16x4 va = lds_tr16(va_p);
                    const i16x4 vb = lds_tr16(va_p + 8 * Gm::ROW);
                    const bf16x8 vf = __builtin_shufflevector(
                        __builtin_bit_cast(bf16x4_t, va), __builtin_bit_cast(bf16x4_t, vb), 0, 1,
                        2, 3, 4, 5, 6, 7);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        vf, __builtin_bit_cast(bf16x8, pb[kc]), acc[db], 0, 0, 0);
                }
        }
    };

    // One sweep over the stream's tiles with NBUF-deep direct-load
    // prefetch and one workgroup barrier per tile.  Every wave executes the
    // same number of barriers; waves without query rows only load.  The
    // compute loop is unrolled NBUF times so that buffer offsets are
    // immediates.
    auto sweep = [&](bool first_max, auto accum_tag) {
#pragma unroll
        for (int t = 0; t < NBUF - 1; ++t)
            if (t < n_mine)
                issue_tile(t, t);
        auto step = [&](int it) {
            const int issued_last = (it + NBUF - 2 < n_mine - 1) ? it + NBUF - 2 : n_mine - 1;
            wait_tiles(issued_last - it);
            block_barrier();
            if (it + NBUF - 1 < n_mine)
                issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
        };
        if (wave_live) {
            int it = 0;
            auto one = [&](auto buf_tag) {
                if (it < n_mine) {
                    step(it);
                    // a max-only pass takes every tile's maximum; an
                    // accumulating one fixes its reference at the first tile
                    compute_tile(it, buf_tag, !decltype(accum_tag)::value || (first_max && it == 0),
                                 accum_tag);
                    ++it;
                }
            };
            while (it < n_mine) {
                one(std::integral_constant<int, 0>{});
                one(std::integral_constant<int, 1 % NBUF>{});
                if constexpr (NBUF > 2)
                    one(std::integral_constant<int, 2 % NBUF>{});
                if constexpr (NBUF > 3)
                    one(std::integral_constant<int, 3 % NBUF>{});
            }
            for (; it < iters; ++it)
                step(it);
        } else {
            for (int it = 0; it < iters; ++it)
                step(it);
        }
        wait_vm<0>();
        block_barrier();                           // buffers free for the next user
    };

    // Software-pipelined accumulation sweep.  Iteration `it` runs the softmax
    // of tile it on the vector units while the matrix cores compute the
    // scores of tile it+1, then P.V of tile it; so each wave keeps its VALU,
    // MFMA and LDS work overlapped instead of alternating between them.
    // Buffers in use in iteration it: K(it+1) and V(it); the direct loads of
    // tile it+NBUF-1 refill the buffer of tile it-1 (NBUF >= 3).
    auto sweep_acc = [&](bool first_max) {
        static_assert(NBUF >= 3, "the pipelined sweep reads two tiles per iteration");
#pragma unroll
        for (int t = 0; t < NBUF - 1; ++t)
            if (t < n_mine)
                issue_tile(t, t);
        // tile t in LDS for every wave, called at the top of iteration `cur`,
        // when tiles 0 .. min(cur+NBUF-2, n_mine-1) have been issued
        auto sync_tile = [&](int t, int cur) {
            if (EVEN && t == cur + 1 && cur + NBUF - 2 < n_mine - 1)
                wait_vm<(NBUF - 3) * (Gm::LOADS / NQT)>();   // steady state
            else
                wait_tiles(((cur + NBUF - 2 < n_mine - 1) ? cur + NBUF - 2 : n_mine - 1) - t);
            block_barrier();
        };
        if (!wave_live) {
            sync_tile(0, 0);
            for (int it = 0; it < iters; ++it) {
                if (it + 1 < n_mine)
                    sync_tile(it + 1, it);
                else
                    block_barrier();
                if (it + NBUF - 1 < n_mine)
                    issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
            }
        } else {
            auto kread = [&](int buf, u32x4 (&kf)[Gm::DC]) {
                const char *kl = smem + buf * Gm::TILE;
#pragma unroll
                for (int c = 0; c < Gm::DC; ++c)
                    kf[c] = *reinterpret_cast<const u32x4 *>(kl + koff[c]);
            };
            auto mask = [&](f32x16 &s, int it) {
                const int kbase = (t_begin + it) * KT;
                if (kbase + KT > L) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (key >= L)
                            s[r] = NEG_INF;
                    }
                }
            };
            f32x16 s_cur = f32x16{};
            if (n_mine > 0) {
                sync_tile(0, 0);
                u32x4 kf[Gm::DC];
                kread(0, kf);
#pragma unroll
                for (int c = 0; c < Gm::DC; ++c)
                    s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, kf[c]), __builtin_bit_cast(bf16x8, qf[c]),
                        s_cur, 0, 0, 0);
                mask(s_cur, 0);
                if (first_max) {
                    float mx = s_cur[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r)
                        mx = __builtin_fmaxf(mx, s_cur[r]);
                    mx = __builtin_fmaxf(mx, swap32(mx, h));
                    // the beam partial, folded before the sweep, moves to
                    // the sweep's reference and seeds the accumulators
                    const float m_new = __builtin_fmaxf(m_ref, mx * cs);
                    const float a = m_ref == NEG_INF ? 0.f : exp2_fast(m_ref - m_new);
                    l_run *= a;
                    l_lse *= a;
#pragma unroll
                    for (int db = 0; db < Gm::DB; ++db)
                        acc[db] = o[db] * a;
                    m_ref = m_new;
                }
            } else {
                if (first_max) {
#pragma unroll
                    for (int db = 0; db < Gm::DB; ++db)
                        acc[db] = o[db];
                }
                block_barrier();
            }
            // one pipelined iteration; HAS_NEXT (compile time) keeps the
            // steady-state body free of branches around its MFMAs
            auto body = [&](int it, auto next_tag) {
                constexpr bool HAS_NEXT = decltype(next_tag)::value;
                if constexpr (HAS_NEXT)
                    sync_tile(it + 1, it);
                else
                    block_barrier();
                if (it + NBUF - 1 < n_mine)
                    issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
                const int bcur = it % NBUF, bnext = (it + 1) % NBUF;
                // (1) all LDS fragment reads of the iteration: V^T of tile it,
                // K of tile it+1; they land while the vector units work
                bf16x8 vf[Gm::DB][2];
                {
                    const char *vl = smem + bcur * Gm::TILE;
#pragma unroll
                    for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc) {
                            const char *va_p = vl + voff[db] + 16 * kc * Gm::ROW;
                            const i16x4 va = lds_tr16(va_p);
                            const i16x4 vb = lds_tr16(va_p + 8 * Gm::ROW);
                            vf[db][kc] = __builtin_shufflevector(
                                __builtin_bit_cast(bf16x4_t, va), __builtin_bit_cast(bf16x4_t, vb),
                                0, 1, 2, 3, 4, 5, 6, 7);
                        }
                }
                u32x4 kf[Gm::DC];
                if constexpr (HAS_NEXT)
                    kread(bnext, kf);
                __builtin_amdgcn_sched_barrier(0);
                // (2) softmax of tile it on the vector units: bf16 B operands,
                // l_run adds the rounded values, l_lse the unrounded ones.
                // Only a stream's last tile can hold keys past the context end.
                if constexpr (!HAS_NEXT)
                    mask(s_cur, it);
                u32x4 pb[2];
                {
                    const float nm = -m_ref;
                    float sum = l_run, sum_x = l_lse;
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) {
                        const int r = 2 * e2;
                        const float p0 = exp2_fast(__builtin_fmaf(s_cur[r], cs, nm));
                        const float p1 = exp2_fast(__builtin_fmaf(s_cur[r + 1], cs, nm));
                        const uint32_t pk = pack_bf16(p0, p1);
                        pb[e2 >> 2][e2 & 3] = pk;
                        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                              __builtin_bit_cast(bf16x2, BF16_ONES),
                                                              sum, false);
                        sum_x += p0 + p1;
                    }
                    l_run = sum;
                    l_lse = sum_x;
                }
                __builtin_amdgcn_sched_barrier(0);
                // (3) matrix cores: O^T += V^T * P^T for tile it, then the
                // scores of tile it+1
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            vf[db][kc], __builtin_bit_cast(bf16x8, pb[kc]), acc[db], 0, 0, 0);
                f32x16 s_next = f32x16{};
                if constexpr (HAS_NEXT) {
#pragma unroll
                    for (int c = 0; c < Gm::DC; ++c)
                        s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, kf[c]), __builtin_bit_cast(bf16x8, qf[c]),
                            s_next, 0, 0, 0);
                }
                if constexpr (HAS_NEXT)
                    s_cur = s_next;
            };
            int it = 0;
            for (; it + 1 < n_mine; ++it)
                body(it, std::true_type{});
            if (it < n_mine) {
                body(it, std::false_type{});
                ++it;
            }
            for (int it = n_mine; it < iters; ++it) {
                block_barrier();
                if (it + NBUF - 1 < n_mine)
                    issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
            }
        }
        wait_vm<0>();
        block_barrier();                           // buffers free for the next user
    };

    // ---- per-beam stage: BeamKV steps gs, gs+GS, ... along BeamPath ------
    // Each lane folds the K and V rows of its query's path token for a step
    // into its (max, sums, O) online.  When G divides 32 the 32/G beams of a
    // wave are gathered first into the (still unused) tile buffers with
    // direct loads, each covering whole rows (a 1 KB load takes 1024/ROW
    // rows: few cache lines per instruction), up to `sch` steps at a time;
    // row beta's 16-byte chunks sit at slot chunk ^ (beta & (CH-1)).  The
    // path entries come from the staged table (else from the lane beta*G,
    // which loads its own).  Otherwise each lane loads its rows from memory.
    const int n_steps = T > gs ? (T - gs + GS - 1) / GS : 0;
    auto step_idx = [&](int i) __attribute__((always_inline)) {
        int qr = qrow;
        asm volatile("" : "+v"(qr));
        return qvalid ? p.beam_path[(int64_t)qr * p.T_cap + gs + i * GS] : 0;
    };
    auto fold = [&](const u32x4 (&kr)[Gm::DC], const u32x2 (&vr)[Gm::DB][4])
                    __attribute__((always_inline)) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < Gm::DC; ++c)
            dot = dot8(qf[c], kr[c], dot);
        dot += swap32(dot, h);
        const float tz = dot * cs;
        const float mn = __builtin_fmaxf(m_ref, tz);
        const float alpha = exp2_fast(m_ref - mn);
        const float pw = exp2_fast(tz - mn);
        m_ref = mn;
        l_run = l_run * alpha + (h == 0 ? pw : 0.f);
        l_lse = l_lse * alpha + (h == 0 ? pw : 0.f);
#pragma unroll
        for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const u32x2 v = vr[db][rg];
                f32x16 &ov = o[db];
                ov[4 * rg + 0] = ov[4 * rg + 0] * alpha + pw * bf16lo(v[0]);
                ov[4 * rg + 1] = ov[4 * rg + 1] * alpha + pw * bf16hi(v[0]);
                ov[4 * rg + 2] = ov[4 * rg + 2] * alpha + pw * bf16lo(v[1]);
                ov[4 * rg + 3] = ov[4 * rg + 3] * alpha + pw * bf16hi(v[1]);
            }
    };
    constexpr int RING = NKS * NBUF * Gm::TILE;
    const int nb = 32 / G;                         // beams of a wave (G divides 32)
    const int sb = 2 * nb * Gm::ROW;               // LDS bytes per gathered step
    const int fit = RING / (NQT * NKS * sb);
    // The LDS gather moves whole 1 KB loads of 1024/ROW rows, so it needs at
    // least that many beams per wave (not so for D = 64 at G = 8: 4 beams of
    // 128 bytes); other shapes take the per-lane gather.
    const int sch = (32 % G == 0 && nb * Gm::ROW >= 1024) ? (fit < PSTEPS ? fit : PSTEPS) : 0;
    auto beam_stage = [&]() __attribute__((always_inline)) {
        if (wave_live && sch > 0) {
            const uint32_t area = lds0 + wave * sch * sb;
            const char *area_p = smem + wave * sch * sb;
            const int lpr = nb * Gm::ROW / 1024;       // 1 KB loads per step for K (and V)
            const int beta_l = lane / Gm::CH;
            const int beta_q = c32 / G;                // this lane's beam within the wave
            const int sw = beta_q & (Gm::CH - 1);
            const uint16_t *bk = p.beam_k + ((int64_t)b * p.beam_cap * p.Hkv + g) * D;
            const uint16_t *bv = p.beam_v + ((int64_t)b * p.beam_cap * p.Hkv + g) * D;
            constexpr int MAXL = 32 * Gm::ROW / 1024;  // 1 KB loads per step at G = 1
            const int tb_w = qt * nb;                  // the wave's first beam in the table
            for (int s0 = 0; s0 < n_steps; s0 += sch) {
                const int cnt = sch < n_steps - s0 ? sch : n_steps - s0;
                // path entries of the chunk's steps for the rows each lane's
                // direct loads cover: from the staged table, or one global load
                // per lane and step followed by shuffles; all before the first
                // direct load
                int rid[PSTEPS][MAXL];
                if (use_tab) {
#pragma unroll
                    for (int i = 0; i < PSTEPS; ++i)
#pragma unroll
                        for (int u = 0; u < MAXL; ++u) {
                            const int beta = u * (1024 / Gm::ROW) + beta_l;
                            rid[i][u] = (i < cnt && u < lpr)
                                            ? ptab_l[(tb_w + beta) * T + gs + (s0 + i) * GS]
                                            : 0;
                        }
                } else {
                    int myidx[PSTEPS];
#pragma unroll
                    for (int i = 0; i < PSTEPS; ++i)
                        myidx[i] = i < cnt ? step_idx(s0 + i) : 0;
#pragma unroll
                    for (int i = 0; i < PSTEPS; ++i)
#pragma unroll
                        for (int u = 0; u < MAXL; ++u) {
                            const int beta = u * (1024 / Gm::ROW) + beta_l;
                            rid[i][u] = (i < cnt && u < lpr) ? __shfl(myidx[i], beta * G) : 0;
                        }
                }
#pragma unroll
                for (int i = 0; i < PSTEPS; ++i)
#pragma unroll
                    for (int u = 0; u < MAXL; ++u)
                        if (i < cnt && u < lpr) {
                            const int beta = u * (1024 / Gm::ROW) + beta_l;
                            const int64_t src = (int64_t)rid[i][u] * p.Hkv * D +
                                                8 * ((lane % Gm::CH) ^ (beta & (Gm::CH - 1)));
                            const uint32_t dst = area + i * sb + u * 1024;
                            dma16(bk + src, dst);
                            dma16(bv + src, dst + nb * Gm::ROW);
                        }
                wait_vm<0>();
                for (int i = 0; i < cnt; ++i) {
                    const char *krow = area_p + i * sb + beta_q * Gm::ROW;
                    const char *vrow = krow + nb * Gm::ROW;
                    u32x4 kr[Gm::DC];
                    u32x2 vr[Gm::DB][4];
#pragma unroll
                    for (int c = 0; c < Gm::DC; ++c)
                        kr[c] = *reinterpret_cast<const u32x4 *>(krow + 16 * ((2 * c + h) ^ sw));
#pragma unroll
                    for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg)
                            vr[db][rg] = *reinterpret_cast<const u32x2 *>(
                                vrow + 16 * ((4 * db + rg) ^ sw) + 8 * h);
                    fold(kr, vr);
                }
                // this wave's reads of the area are done before it is refilled
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        } else if (wave_live) {
            for (int i = 0; i < n_steps; ++i) {
                const int idx = step_idx(i);
                const int64_t base = (((int64_t)b * p.beam_cap + idx) * p.Hkv + g) * D;
                const uint16_t *kp = p.beam_k + base + 8 * h;
                const uint16_t *vp = p.beam_v + base + 4 * h;
                u32x4 kr[Gm::DC];
                u32x2 vr[Gm::DB][4];
#pragma unroll
                for (int c = 0; c < Gm::DC; ++c)
                    kr[c] = qvalid ? ldg16(kp + 16 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg)
                        vr[db][rg] = qvalid ? ldg8(vp + 32 * db + 8 * rg) : u32x2{0, 0};
                fold(kr, vr);
            }
        }
    };

    // The BeamKV steps are folded first, while the tile ring is still empty:
    // their gathers overlap the start of the other workgroups' sweeps, and
    // the partial seeds the accumulators at the first tile, rescaled to the
    // sweep's reference.
    block_barrier();                               // staged BeamPath entries written
    beam_stage();
    block_barrier();                               // gather area read before the tiles land

    // Pass 0 takes the larger of the beam partial's maximum and each
    // stream's first-tile maximum as the fixed reference:
    // later tiles may exceed it, so probabilities can grow past 1.  As long
    // as every row sum stays below 2^64 nothing can overflow and the final
    // normalisation is exact.  Otherwise (scores rising by more than ~44
    // nats along the context) the workgroup sweeps again: exact maxima
    // first, then the accumulation against them.
    // The re-sweep starts from nothing and folds the BeamKV steps again
    // after it.
    sweep_acc(true);
    bool beam_again = false;
    if (__syncthreads_or(qvalid && !(l_lse < SAFE_SUM))) {
        beam_again = true;                         // the beam partial is dropped with the rest
        m_ref = NEG_INF;
        l_run = 0.f;
        l_lse = 0.f;
#pragma unroll
        for (int db = 0; db < Gm::DB; ++db)
            acc[db] = f32x16{};
        sweep(true, std::false_type{});
        sweep_acc(false);
    }

    // The vector-unit stages below work on a copy of the accumulators pinned
    // in ordinary VGPRs; the context loop above then keeps its accumulators
    // in the matrix cores' accumulation registers without per-iteration moves.
#pragma unroll
    for (int db = 0; db < Gm::DB; ++db) {
        o[db] = acc[db];
        asm volatile("" : "+v"(o[db]));
    }
    if (beam_again)
        beam_stage();
    if constexpr (NKS > 1)
        block_barrier();                           // gathered rows read before the merge
    // full row sums (the two lane halves held different keys)
    l_run += swap32(l_run, h);
    l_lse += swap32(l_lse, h);

    // ---- merge of the key streams through LDS (log-sum-exp) ---------------
    if constexpr (NKS > 1) {
        char *ml = smem;                           // staging buffers are free now
        if (ks > 0 && wave_live) {
            char *sp = ml + ((ks - 1) * NQT + qt) * Gm::OSLOT;
            float *stats = reinterpret_cast<float *>(sp + 32 * Gm::OPITCH);
            if (h == 0) {
                stats[4 * c32] = m_ref;
                stats[4 * c32 + 1] = l_run;
                stats[4 * c32 + 2] = l_lse;
            }
#pragma unroll
            for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const f32x4 v = {o[db][4 * rg], o[db][4 * rg + 1], o[db][4 * rg + 2],
                                     o[db][4 * rg + 3]};
                    *reinterpret_cast<f32x4 *>(sp + c32 * Gm::OPITCH +
                                               (32 * db + 8 * rg + 4 * h) * 4) = v;
                }
        }
        __syncthreads();
        if (ks == 0 && wave_live) {
#pragma unroll
            for (int k2 = 1; k2 < NKS; ++k2) {
                const char *sp = ml + ((k2 - 1) * NQT + qt) * Gm::OSLOT;
                const float *stats = reinterpret_cast<const float *>(sp + 32 * Gm::OPITCH);
                const float mo = stats[4 * c32], lo = stats[4 * c32 + 1];
                const float lxo = stats[4 * c32 + 2];
                const float mn = __builtin_fmaxf(m_ref, mo);
                const float a = m_ref == NEG_INF ? 0.f : exp2_fast(m_ref - mn);
                const float bw = mo == NEG_INF ? 0.f : exp2_fast(mo - mn);
                m_ref = mn;
                l_run = l_run * a + lo * bw;
                l_lse = l_lse * a + lxo * bw;
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(
                            sp + c32 * Gm::OPITCH + (32 * db + 8 * rg + 4 * h) * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[db][4 * rg + e] = o[db][4 * rg + e] * a + v[e] * bw;
                    }
            }
        }
    }

    // ---- context split: partials through the workspace --------------------
    // Every workgroup of the unit leaves its waves' (O, max, sums) in the
    // workspace in lane order, then counts itself in; the last to arrive
    // resets the counter for the next call and combines all n_split partials
    // in ascending split order, its own included and read back like the
    // others, so the result does not depend on which workgroup finishes
    // last.  Partials are written and read with device-scope (sc1) accesses,
    // which are coherent across XCDs without an L2 writeback: the writer
    // waits for its stores to complete before it counts itself in, and the
    // last workgroup reads only after its count has returned.
    if (p.n_split > 1) {
        __shared__ int s_last;
        const int unit = pair * p.n_qt + qtile;
        constexpr int PB = fused_part_bytes(D);
        constexpr int NV = D / 8;                  // f32x4 per lane of a wave's O^T
        constexpr int SC1 = 16;                    // cache policy: device scope
        const int unit_bytes = p.n_split * NQT * PB;
        const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
            p.ws_part + (size_t)unit * unit_bytes, 0, unit_bytes, 0x00020000);
        if (ks == 0 && wave_live) {
            const int mine = (split * NQT + qt) * PB + 16 * lane;
            if (m_ref != NEG_INF) {                // nothing to add otherwise
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(u32x4, f32x4{o[db][4 * rg], o[db][4 * rg + 1],
                                                            o[db][4 * rg + 2], o[db][4 * rg + 3]}),
                            part, mine + (db * 4 + rg) * 1024, 0, SC1);
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, f32x4{m_ref, l_run, l_lse, 0.f}), part,
                mine + NV * 1024, 0, SC1);
        }
        wait_vm<0>();                              // this wave's partial is complete
        __syncthreads();
        if (tid == 0) {
            const int last = atomicAdd(p.ws_count + unit, 1) == p.n_split - 1;
            if (last)
                p.ws_count[unit] = 0;              // next call starts from zero
            s_last = last;
        }
        __syncthreads();
        if (!s_last)
            return;
        if (ks == 0 && wave_live) {
            float mm = NEG_INF, lr = 0.f, ll = 0.f;
#pragma unroll
            for (int db = 0; db < Gm::DB; ++db)
                o[db] = f32x16{};                  // the combined O^T
#pragma unroll 1
            for (int sp = 0; sp < p.n_split; ++sp) {
                const int src = (sp * NQT + qt) * PB + 16 * lane;
                const f32x4 st = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(part, src + NV * 1024, 0, SC1));
                const float ms = st[0];
                if (ms == NEG_INF)
                    continue;                      // an empty partial
                const float mn = __builtin_fmaxf(mm, ms);
                const float a = mm == NEG_INF ? 0.f : exp2_fast(mm - mn);
                const float bw = exp2_fast(ms - mn);
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const f32x4 v = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       part, src + (db * 4 + rg) * 1024, 0, SC1));
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[db][4 * rg + e] = o[db][4 * rg + e] * a + v[e] * bw;
                    }
                mm = mn;
                lr = lr * a + st[1] * bw;
                ll = ll * a + st[2] * bw;
            }
            m_ref = mm;
            l_run = lr;
            l_lse = ll;
        }
    }

    // ---- epilogue: normalise, bf16 output, fp32 natural-log LSE ----------
    if (ks == 0 && wave_live && qvalid) {
        // recomputed here from opaque copies: the 64-bit row offset of the Q
        // load would otherwise be kept (and spilled) across the context loop
        int qr = qrow, qh = qhead;
        asm volatile("" : "+v"(qr), "+v"(qh));
        const int64_t orow = (int64_t)qr * p.Hq + qh;
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        uint16_t *dst = p.out + orow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const u32x2 v = {pack_bf16(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv),
                                 pack_bf16(o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv)};
                *reinterpret_cast<u32x2 *>(dst + 32 * db + 8 * rg) = v;
            }
        if (h == 0)
            p.lse[orow] = l_lse > 0.f ? (m_ref + __builtin_log2f(l_lse)) * 0.69314718055994531f
                                      : NEG_INF;
    }
}

// ---------------------------------------------------------------------------
// Generic comparator: one workgroup of 64 threads per (row, head); two passes
// over that row's keys, reading the whole ContextKV again for every row.
template <int D>
__global__ __launch_bounds__(64) void generic_decode_attn(const Params p)
{
    __shared__ float z[GENERIC_MAX_KEYS];
    __shared__ float red[64];
    const int rh = blockIdx.x;
    const int r = rh / p.Hq;
    const int hq = rh - r * p.Hq;
    const int g = hq / p.G;
    const int lane = threadIdx.x;
    int b = 0;
    while (b + 1 < p.B && p.row_offset[b + 1] <= r)
        ++b;
    const int L = p.ctx_len[b];
    const int T = p.beam_len[b];
    const int N = L + T;
    const uint16_t *qv = p.q + ((int64_t)r * p.Hq + hq) * D;
    const int64_t kv_tok = (int64_t)p.Hkv * D;
    const int64_t ctx_base = ((int64_t)b * p.ctx_cap * p.Hkv + g) * D;
    const int64_t beam_base = ((int64_t)b * p.beam_cap * p.Hkv + g) * D;
    auto key_ptr = [&](const uint16_t *ctx, const uint16_t *beam, int j) -> const uint16_t * {
        if (j < L)
            return ctx + ctx_base + j * kv_tok;
        const int idx = p.beam_path[(int64_t)r * p.T_cap + (j - L)];
        return beam + beam_base + (int64_t)idx * kv_tok;
    };
    // pass 1: scores (lane per key)
    float mx = NEG_INF;
    for (int jj = lane; jj < N; jj += 64) {
        const uint16_t *k = key_ptr(p.ctx_k, p.beam_k, jj);
        float dot = 0.f;
        for (int c = 0; c < D / 8; ++c)
            dot = dot8(ldg16(qv + 8 * c), ldg16(k + 8 * c), dot);
        z[jj] = dot * p.scale_log2;
        mx = __builtin_fmaxf(mx, z[jj]);
    }
    red[lane] = mx;
    __syncthreads();
    for (int o = 32; o > 0; o >>= 1) {
        if (lane < o)
            red[lane] = __builtin_fmaxf(red[lane], red[lane + o]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    float sum = 0.f;
    for (int jj = lane; jj < N; jj += 64) {
        const float e = exp2_fast(z[jj] - M);
        z[jj] = e;
        sum += e;
    }
    red[lane] = sum;
    __syncthreads();
    for (int o = 32; o > 0; o >>= 1) {
        if (lane < o)
            red[lane] += red[lane + o];
        __syncthreads();
    }
    const float Z = red[0];
    // pass 2: weighted values (lanes split D)
    constexpr int PER = D / 64;
    float o[PER] = {};
    for (int jj = 0; jj < N; ++jj) {
        const uint16_t *v = key_ptr(p.ctx_v, p.beam_v, jj);
        const float w = z[jj];
#pragma unroll
        for (int e = 0; e < PER; ++e)
            o[e] += w * __uint_as_float((uint32_t)v[lane * PER + e] << 16);
    }
    const float inv = Z > 0.f ? 1.f / Z : 0.f;
    uint16_t *dst = p.out + ((int64_t)r * p.Hq + hq) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        dst[lane * PER + e] = static_cast<uint16_t>(pack_bf16(o[e] * inv, 0.f) & 0xffffu);
    if (lane == 0)
        p.lse[(int64_t)r * p.Hq + hq] =
            N > 0 ? (M + __builtin_log2f(Z)) * 0.69314718055994531f : NEG_INF;
}

// ---------------------------------------------------------------------------
// Metadata checker: one thread per request row plus per-request checks.
__global__ void check_metadata(const MetaCheck c)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (t < c.B) {
        const int lo = c.row_offset[t], hi = c.row_offset[t + 1];
        bad += (hi < lo) || (hi - lo > c.W_max) || (lo < 0) || (hi > c.R);
        bad += (c.ctx_len[t] < 0) || (c.ctx_len[t] > c.ctx_cap);
        bad += (c.beam_len[t] < 0) || (c.beam_len[t] > c.T_cap);
        if (t == 0)
            bad += (lo != 0) || (c.row_offset[c.B] != c.R);
    }
    if (t < c.R) {
        int b = 0;
        while (b + 1 < c.B && c.row_offset[b + 1] <= t)
            ++b;
        int T = c.beam_len[b];
        T = T < 0 ? 0 : (T > c.T_cap ? c.T_cap : T);
        for (int s = 0; s < T; ++s) {
            const int idx = c.beam_path[(int64_t)t * c.T_cap + s];
            bad += (idx < 0) || ((int64_t)idx >= c.beam_cap);
        }
    }
    if (bad)
        atomicAdd(c.violations, bad);
}

__global__ void zero_i32(int32_t *p) { *p = 0; }

// ---------------------------------------------------------------------------
template <int D, int NQT, int NKS, int NBUF, int OCC, bool PAGED>
static hipError_t launch_fused_t(const Params &p, int grid, hipStream_t s)
{
    constexpr int lds = lds_bytes<D, NQT, NKS, NBUF>();
    auto kern = fused_decode_attn<D, NQT, NKS, NBUF, OCC, PAGED>;
    // the dynamic-LDS limit is raised once per instantiation and device
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess)
            return e;
        attr_set.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NQT * NKS), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_fused(const Params &p, int nqt, int nks, int grid, hipStream_t s)
{
#define GR_LAUNCH_CASE(d, a, c, nb, oc)                                               \
    if (p.D == d && nqt == a && nks == c)                                             \
        return p.page_table ? launch_fused_t<d, a, c, nb, oc, true>(p, grid, s)         \
                            : launch_fused_t<d, a, c, nb, oc, false>(p, grid, s);
    GR_FOR_EACH_FUSED_CONFIG(GR_LAUNCH_CASE)
#undef GR_LAUNCH_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_generic(const Params &p, hipStream_t s)
{
    const int grid = p.R * p.Hq;
    if (grid == 0)
        return hipSuccess;
    if (p.D == 128)
        hipLaunchKernelGGL(generic_decode_attn<128>, dim3(grid), dim3(64), 0, s, p);
    else if (p.D == 64)
        hipLaunchKernelGGL(generic_decode_attn<64>, dim3(grid), dim3(64), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_check(const MetaCheck &c, hipStream_t s)
{
    hipLaunchKernelGGL(zero_i32, dim3(1), dim3(1), 0, s, c.violations);
    const int n = (c.R > c.B ? c.R : c.B);
    if (n > 0)
        hipLaunchKernelGGL(check_metadata, dim3((n + 255) / 256), dim3(256), 0, s, c);
    return hipGetLastError();
}

}  // namespace gr
