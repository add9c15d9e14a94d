// Fused decode attention with 16-row waves (gfx950).
//
// The method is the one of gr_attn_kernels.hip (GR-Inference blog, section
// on kernel design; xGR paper review, section "xAttention"): per (request,
// KV head), the stacked beam query rows against one ContextKV on the matrix
// cores with an online softmax, each beam's BeamKV tokens gathered along its
// BeamPath, the parts combined by their log-sum-exp.  This variant gives
// each wave 16 stacked query rows instead of 32, so that a wave needs about
// half the registers and more waves share each SIMD: it is meant for shapes
// whose (request, KV head) pairs have few rows (the 32-row kernel then runs
// one wave per SIMD, and nothing hides a wave's own latency chain).
//
// gfx950 mapping (v_mfma_f32_16x16x32_bf16; lane l = 16*lg + n):
//   * S^T = K * Q^T per 16-key block: A = K rows (lane: key n, 8 d values
//     of its 32-wide d chunk), B = Q^T held in registers.  The 16x16
//     accumulator gives lane (n, lg) keys 4*lg + i of query n (i < 4); with
//     the tile's two key blocks, 8 keys of one query per lane.
//   * O^T += V^T * P^T with the tile's 32 keys as the contraction: the order
//     of the keys in that contraction is free, so it is taken as the order
//     in which each lane already holds them (keys 4*lg..4*lg+3, then
//     16+4*lg..16+4*lg+3): the rounded probabilities are the B operand as
//     they are, and the matching V^T operand is two transposing LDS reads
//     (ds_read_b64_tr_b16) of the row-major V tile per 16-row d block.
//   * Tiles, direct loads, the ring, the fixed-reference softmax with its
//     exact re-sweep and the merge of key streams are those of the 32-row
//     kernel.  No context split across workgroups.
//   * BeamKV rows are gathered by each lane with vector loads and folded
//     online on the vector units: either by the sweep waves before their
//     sweep (BW = 0), or (BW = 1) by NQT extra beam waves, one per query
//     tile, while the sweep waves run the context.  A beam wave takes part
//     in every barrier of the sweep (it does its gathers and folds between
//     them), and its partial joins the key streams' in the LDS merge.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "gr_attn_device.h"
#include "gr_attn_internal.h"

namespace gr {

template <int D>
struct Geo16 {
    static constexpr int DC = D / 32;                     // 32-wide d chunks (QK)
    static constexpr int DB = D / 16;                     // 16-row d blocks of O^T
    static constexpr int OSLOT = (DB + 1) * 64 * 16;      // a wave's O^T + stats, lane order
};

// Chunk swizzles of this kernel's K and V tile rows (16-byte chunk c of row
// r sits in slot c ^ swz(r)), chosen for its own fragment reads: the K read
// has the 16 lanes of a group on rows 0..15, the V^T read has lane groups
// lg and lg+1 on rows four apart.  A row spans all 64 four-byte banks at D
// = 128 and half of them at D = 64; with these swizzles no two lanes of one
// LDS pass (16 lanes of a 16-byte read, 32 of an 8-byte read) share a bank.
template <int D>
__device__ __forceinline__ constexpr int kswz16(int r)
{
    return (D == 64 ? r >> 1 : r) & (Geo<D>::CH - 1);
}
template <int D>
__device__ __forceinline__ constexpr int vswz16(int r)
{
    return (D == 64 ? r : 2 * r) & (Geo<D>::CH - 1);
}

template <int D, int NQT, int NKS, int NBUF, bool BW>
constexpr int lds16_bytes()
{
    constexpr int stage = NKS * NBUF * Geo<D>::TILE;
    constexpr int merge = (NKS - 1 + (BW ? 1 : 0)) * NQT * Geo16<D>::OSLOT;
    static_assert((stage > merge ? stage : merge) == fused16_lds_main(D, NQT, NKS, NBUF, BW),
                  "host and device LDS layouts differ");
    return stage > merge ? stage : merge;
}

// sweep barriers a beam wave lets pass between issuing a chunk's BeamKV
// loads and folding them
#ifndef BW_SLACK
#define BW_SLACK 3
#endif

__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16); }
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

template <int D, int NQT, int NKS, int NBUF, int OCC, bool BW, bool PAGED>
__global__ __launch_bounds__(64 * (NQT * NKS + (BW ? NQT : 0)))
__attribute__((amdgpu_waves_per_eu(OCC)))
void fused_decode_attn16(const Params p)
{
    using Gm = Geo<D>;
    using G16 = Geo16<D>;
    constexpr int WR = 16;                        // stacked query rows per wave
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // ---- work item: (pair, query tile), XCD-aware (as the 32-row kernel)
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int j = bid >> 3;
    const int pair = (j / p.n_qt) * 8 + xcd;
    const int qtile = j % p.n_qt;
    if (pair >= p.B * p.Hkv)
        return;
    const int b = pair / p.Hkv;
    const int g = pair - b * p.Hkv;
    const int G = p.G;
    const int r0 = p.row_offset[b];
    const int Wb = p.row_offset[b + 1] - r0;
    const int M = Wb * G;
    const int tile_row0 = qtile * WR * NQT;
    if (tile_row0 >= M)
        return;                                   // uniform for the workgroup
    const int L = p.ctx_len[b];
    const int T = p.beam_len[b];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // waves 0 .. NQT*NKS-1 sweep the context (query tile qt, key stream
    // ks); with BW the next NQT waves are the beam waves of the query tiles
    const bool bwave = BW && wave >= NQT * NKS;
    const int qt = bwave ? wave - NQT * NKS : wave % NQT;
    const int ks = bwave ? 0 : wave / NQT;
    const int n = lane & 15;                      // the lane's query within the wave
    const int lg = lane >> 4;                     // the lane's 16-lane group
    const int wrow0 = tile_row0 + qt * WR;
    const bool wave_live = wrow0 < M;

    // ---- the lane's query and its Q^T fragments: d = 32c + 8lg .. +8 ------
    const int m_row = wrow0 + n;
    const bool qvalid = m_row < M;
    const int beam = qvalid ? m_row / G : 0;
    const int qhead = g * G + (qvalid ? m_row - beam * G : 0);
    const int qrow = r0 + beam;
    // BeamPath entries of the beam stage's first two steps (this stream's
    // steps ks and ks + NKS), loaded first: the beam stage's gathers wait on
    // them
    const int n_steps = T > ks ? (T - ks + NKS - 1) / NKS : 0;
    int pidx0[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const bool on = !BW && wave_live && qvalid && u < n_steps;
        pidx0[u] = on ? p.beam_path[(int64_t)qrow * p.T_cap + ks + u * NKS] : 0;
    }
    u32x4 qf[G16::DC];
    {
        const uint16_t *src = p.q + ((int64_t)qrow * p.Hq + qhead) * D + 8 * lg;
#pragma unroll
        for (int c = 0; c < G16::DC; ++c)
            qf[c] = qvalid ? ldg16(src + 32 * c) : u32x4{0, 0, 0, 0};
    }
    // consume the loads here, so that no wait for them is left inside the
    // tile loop (where it would also wait for the tile prefetches)
#pragma unroll
    for (int c = 0; c < G16::DC; ++c)
        asm volatile("" : "+v"(qf[c]));

    float m_ref = NEG_INF;                        // reference maximum, log2 units
    // this lane's share of its query's row sums (its 8 keys of each tile):
    // l_run of the bf16 values the matrix cores multiply, l_lse unrounded
    float l_run = 0.f;
    float l_lse = 0.f;
    f32x4 acc[G16::DB];
    f32x4 o[G16::DB];                             // vector-unit accumulators
#pragma unroll
    for (int db = 0; db < G16::DB; ++db) {
        acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float cs = p.scale_log2;

    // ---- the stream's context tiles and their direct loads ----------------
    const int n_tiles = (L + KT - 1) / KT;
    const int t_begin = (ks * n_tiles) / NKS;
    const int n_mine = ((ks + 1) * n_tiles) / NKS - t_begin;
    const int iters = (n_tiles + NKS - 1) / NKS;  // same for every wave (barrier count)
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    const uint32_t stream_off = ks * (NBUF * Gm::TILE);
    const uint16_t *kv_k = p.ctx_k + ((PAGED ? 0 : (int64_t)b * p.ctx_cap * p.Hkv) + g) * D;
    const uint16_t *kv_v = p.ctx_v + ((PAGED ? 0 : (int64_t)b * p.ctx_cap * p.Hkv) + g) * D;
    const int kv_tok = p.Hkv * D;
    const int32_t *ptab = PAGED ? p.page_table + (int64_t)b * p.pages_per_req : nullptr;
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
    constexpr int RPL = 1024 / Gm::ROW;
    constexpr int LPW = (Gm::LOADS + NQT - 1) / NQT;
    uint32_t loff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int u = qt + i * NQT;
        const bool is_v = u >= Gm::LOADS / 2;
        const int uu = is_v ? u - Gm::LOADS / 2 : u;
        const int r = uu * RPL + lane / Gm::CH;
        const int c = (lane % Gm::CH) ^ (is_v ? vswz16<D>(r) : kswz16<D>(r));
        loff[i] = (uint32_t)(r * kv_tok + 8 * c) * 2u;
    }
    constexpr bool EVEN = Gm::LOADS % NQT == 0;
    auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
        const int key0 = (t_begin + t) * KT;
        const uint32_t dst0 = lds0 + stream_off + buf * Gm::TILE;
        if constexpr (PAGED) {
            if (key0 + KT <= L) {
                // the tile's first and last 16 keys each lie in one page
                // (page sizes are multiples of 16, tiles start at multiples
                // of 32): one base per half, the lane offsets the dense ones
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
#pragma unroll 1
                for (int i = 0; i < LPW; ++i) {
                    const int u = qt + i * NQT;
                    if (!EVEN && u >= Gm::LOADS)
                        break;
                    const bool is_v = u >= Gm::LOADS / 2;
                    const int uu = is_v ? u - Gm::LOADS / 2 : u;
                    const int r = uu * RPL + lane / Gm::CH;
                    const int c = (lane % Gm::CH) ^ (is_v ? vswz16<D>(r) : kswz16<D>(r));
                    const int tok = key0 + r < L ? key0 + r : L - 1;
                    const int64_t row = page_base(ptab[page_idx(tok)], tok, 0);
                    dma16((is_v ? kv_v : kv_k) + row + 8 * c,
                          dst0 + (is_v ? Gm::KBYTES : 0) + uu * 1024);
                }
            }
            return;
        }
        if (key0 + KT <= L) {
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
    const int my_loads = EVEN ? Gm::LOADS / NQT : (Gm::LOADS - qt + NQT - 1) / NQT;
    auto wait_tiles = [&](int pending) __attribute__((always_inline)) {
        const int nn = pending > 0 ? pending * my_loads : 0;
        if (nn >= 48)
            wait_vm<48>();
        else if (nn >= 32)
            wait_vm<32>();
        else if (nn >= 16)
            wait_vm<16>();
        else if (nn >= 8)
            wait_vm<8>();
        else if (nn >= 4)
            wait_vm<4>();
        else if (nn >= 2)
            wait_vm<2>();
        else
            wait_vm<0>();
    };

    // ---- fragment offsets (stream base included) -------------------------
    // K: lane (n, lg) reads key row 16kb + n, 16-byte chunk 4c + lg; the row
    // swizzle depends on n only, so the second key block is +16 rows.
    uint32_t koff[G16::DC];
#pragma unroll
    for (int c = 0; c < G16::DC; ++c)
        koff[c] = stream_off + n * Gm::ROW + 16 * ((4 * c + lg) ^ kswz16<D>(n));
    // V^T: in a transposing read, lane a of a 16-lane group receives element
    // a % 4 of the words addressed by lanes a/4 + 4j (j < 4); lane a here
    // addresses row 4lg + a/4, columns 16db + 4(a % 4) .. +3, so lane a
    // receives V[4lg + j][16db + a] for j < 4 (and rows +16 for the second
    // read).
    uint32_t voff[G16::DB];
    {
        const int vrow = 4 * lg + (n >> 2);
#pragma unroll
        for (int db = 0; db < G16::DB; ++db)
            voff[db] = stream_off + Gm::KBYTES + vrow * Gm::ROW +
                       16 * ((2 * db + ((n & 3) >> 1)) ^ vswz16<D>(vrow)) + 8 * (n & 1);
    }

    auto kread = [&](int buf, u32x4 (&kf)[2][G16::DC]) __attribute__((always_inline)) {
        const char *kl = smem + buf * Gm::TILE;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < G16::DC; ++c)
                kf[kb][c] = *reinterpret_cast<const u32x4 *>(kl + koff[c] + kb * 16 * Gm::ROW);
    };
    auto qk = [&](const u32x4 (&kf)[2][G16::DC], f32x4 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < G16::DC; ++c)
                s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kf[kb][c]), __builtin_bit_cast(bf16x8, qf[c]),
                    s[kb], 0, 0, 0);
        }
    };
    auto vread = [&](int buf, bf16x8 (&vf)[G16::DB]) __attribute__((always_inline)) {
        const char *vl = smem + buf * Gm::TILE;
#pragma unroll
        for (int db = 0; db < G16::DB; ++db) {
            const i16x4 va = lds_tr16(vl + voff[db]);
            const i16x4 vb = lds_tr16(vl + voff[db] + 16 * Gm::ROW);
            vf[db] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, va),
                                             __builtin_bit_cast(bf16x4_t, vb), 0, 1, 2, 3, 4,
                                             5, 6, 7);
        }
    };
    auto mask = [&](f32x4 (&s)[2], int it) __attribute__((always_inline)) {
        const int kbase = (t_begin + it) * KT;
        if (kbase + KT > L) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kbase + 16 * kb + 4 * lg + i >= L)
                        s[kb][i] = NEG_INF;
        }
    };
    auto rowmax = [&](const f32x4 (&s)[2]) __attribute__((always_inline)) {
        float mx = s[0][0];
#pragma unroll
        for (int i = 1; i < 4; ++i)
            mx = __builtin_fmaxf(mx, s[0][i]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = __builtin_fmaxf(mx, s[1][i]);
        mx = __builtin_fmaxf(mx, xor16(mx));
        return __builtin_fmaxf(mx, xor32(mx));
    };
    // probabilities as the PV B operand (keys 4lg+i, then 16+4lg+i), and
    // this lane's share of the row sums
    auto softmax = [&](const f32x4 (&s)[2], u32x4 &pb) __attribute__((always_inline)) {
        const float nm = -m_ref;
        float sum = l_run, sum_x = l_lse;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kb = e >> 1, i = 2 * (e & 1);
            const float p0 = exp2_fast(__builtin_fmaf(s[kb][i], cs, nm));
            const float p1 = exp2_fast(__builtin_fmaf(s[kb][i + 1], cs, nm));
            const uint32_t pk = pack_bf16(p0, p1);
            pb[e] = pk;
            sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                  __builtin_bit_cast(bf16x2, BF16_ONES), sum,
                                                  false);
            sum_x += p0 + p1;
        }
        l_run = sum;
        l_lse = sum_x;
    };
    auto pv = [&](const bf16x8 (&vf)[G16::DB], const u32x4 &pb) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < G16::DB; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                vf[db], __builtin_bit_cast(bf16x8, pb), acc[db], 0, 0, 0);
    };

    // Max-only sweep (the exact pass of the re-sweep): one barrier per tile.
    auto sweep_max = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NBUF - 1; ++t)
            if (t < n_mine)
                issue_tile(t, t);
        for (int it = 0; it < iters; ++it) {
            const int last = (it + NBUF - 2 < n_mine - 1) ? it + NBUF - 2 : n_mine - 1;
            wait_tiles(last - it);
            block_barrier();
            if (it + NBUF - 1 < n_mine)
                issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
            if (wave_live && it < n_mine) {
                u32x4 kf[2][G16::DC];
                kread(it % NBUF, kf);
                f32x4 s[2];
                qk(kf, s);
                mask(s, it);
                m_ref = __builtin_fmaxf(m_ref, rowmax(s) * cs);
            }
        }
        wait_vm<0>();
        block_barrier();
    };

    // Software-pipelined accumulation sweep (as the 32-row kernel):
    // iteration it reads V^T(it) and K(it+1), runs the softmax of tile it,
    // then the P.V MFMAs of tile it and the score MFMAs of tile it+1.
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NBUF - 1; ++t)
            if (t < n_mine)
                issue_tile(t, t);
    };
    auto sweep_acc = [&](bool first_max, bool issued) __attribute__((always_inline)) {
        static_assert(NBUF >= 3, "the pipelined sweep reads two tiles per iteration");
        if (!issued)
            prefetch();
        auto sync_tile = [&](int t, int cur) __attribute__((always_inline)) {
            if (EVEN && t == cur + 1 && cur + NBUF - 2 < n_mine - 1)
                wait_vm<(NBUF - 3) * (Gm::LOADS / NQT)>();
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
            f32x4 s_cur[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            if (n_mine > 0) {
                sync_tile(0, 0);
                u32x4 kf[2][G16::DC];
                kread(0, kf);
                qk(kf, s_cur);
                mask(s_cur, 0);
                if (first_max) {
                    // the beam partial, folded before the sweep, moves to
                    // the sweep's reference and seeds the accumulators
                    const float m_new = __builtin_fmaxf(m_ref, rowmax(s_cur) * cs);
                    const float a = m_ref == NEG_INF ? 0.f : exp2_fast(m_ref - m_new);
                    l_run *= a;
                    l_lse *= a;
#pragma unroll
                    for (int db = 0; db < G16::DB; ++db)
                        acc[db] = o[db] * a;
                    m_ref = m_new;
                }
            } else {
                if (first_max) {
#pragma unroll
                    for (int db = 0; db < G16::DB; ++db)
                        acc[db] = o[db];
                }
                block_barrier();
            }
            auto body = [&](int it, auto next_tag) __attribute__((always_inline)) {
                constexpr bool HAS_NEXT = decltype(next_tag)::value;
                if constexpr (HAS_NEXT)
                    sync_tile(it + 1, it);
                else
                    block_barrier();
                // the V reads go first into the LDS queue, then this wave's
                // share of the refill (measured ~1% faster than the refill
                // first), then the K reads
                bf16x8 vf[G16::DB];
                vread(it % NBUF, vf);
                if (it + NBUF - 1 < n_mine)
                    issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
                u32x4 kf[2][G16::DC];
                if constexpr (HAS_NEXT)
                    kread((it + 1) % NBUF, kf);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!HAS_NEXT)
                    mask(s_cur, it);
                u32x4 pb;
                softmax(s_cur, pb);
                __builtin_amdgcn_sched_barrier(0);
                pv(vf, pb);
                if constexpr (HAS_NEXT)
                    qk(kf, s_cur);
            };
            int it = 0;
            for (; it + 1 < n_mine; ++it)
                body(it, std::true_type{});
            if (it < n_mine) {
                body(it, std::false_type{});
                ++it;
            }
            for (int it2 = n_mine; it2 < iters; ++it2) {
                block_barrier();
                if (it2 + NBUF - 1 < n_mine)
                    issue_tile(it2 + NBUF - 1, (it2 + NBUF - 1) % NBUF);
            }
        }
        wait_vm<0>();
        block_barrier();
    };

    // ---- per-beam stage: the stream's BeamKV steps ks, ks+NKS, ... --------
    // Each lane loads its query's rows (K: d = 32c + 8lg .. +8; V: d = 16db +
    // 4lg .. +3) and folds them online into `o`; up to two steps' loads are
    // in flight together.
    // online fold of one BeamKV step into (m_ref, l_run, l_lse, o); l_run
    // and l_lse hold the step weights on the lanes of group 0 only
    auto fold_step = [&](const u32x4 (&kr)[G16::DC], const u32x2 (&vr)[G16::DB])
        __attribute__((always_inline)) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < G16::DC; ++c)
            dot = dot8(qf[c], kr[c], dot);
        dot += xor16(dot);
        dot += xor32(dot);
        const float tz = dot * cs;
        const float mn = __builtin_fmaxf(m_ref, tz);
        const float alpha = m_ref == NEG_INF ? 0.f : exp2_fast(m_ref - mn);
        const float pw = exp2_fast(tz - mn);
        m_ref = mn;
        l_run = l_run * alpha + (lg == 0 ? pw : 0.f);
        l_lse = l_lse * alpha + (lg == 0 ? pw : 0.f);
#pragma unroll
        for (int db = 0; db < G16::DB; ++db) {
            const u32x2 v = vr[db];
            o[db][0] = o[db][0] * alpha + pw * bf16lo(v[0]);
            o[db][1] = o[db][1] * alpha + pw * bf16hi(v[0]);
            o[db][2] = o[db][2] * alpha + pw * bf16lo(v[1]);
            o[db][3] = o[db][3] * alpha + pw * bf16hi(v[1]);
        }
    };
    auto beam_stage = [&](bool pre) __attribute__((always_inline)) {
        if (!wave_live)
            return;
        const int64_t req = (int64_t)b * p.beam_cap;
        for (int i0 = 0; i0 < n_steps; i0 += 2) {
            u32x4 kr[2][G16::DC];
            u32x2 vr[2][G16::DB];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bool on = i0 + u < n_steps && qvalid;
                int qr = qrow;
                asm volatile("" : "+v"(qr));
                const int idx =
                    pre && i0 == 0 ? pidx0[u]
                                   : (on ? p.beam_path[(int64_t)qr * p.T_cap + ks + (i0 + u) * NKS] : 0);
                const int64_t base = ((req + idx) * p.Hkv + g) * D;
#pragma unroll
                for (int c = 0; c < G16::DC; ++c)
                    kr[u][c] = on ? ldg16(p.beam_k + base + 32 * c + 8 * lg) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int db = 0; db < G16::DB; ++db)
                    vr[u][db] = on ? ldg8(p.beam_v + base + 16 * db + 4 * lg) : u32x2{0, 0};
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (i0 + u >= n_steps)
                    break;
                fold_step(kr[u], vr[u]);
            }
        }
    };

    // ---- beam wave (BW): all BeamKV steps of the query tile's rows --------
    // BSTEP steps at a time: their BeamKV rows are issued, BW_SLACK of the
    // sweep's barriers pass while they travel, then they are folded; the
    // BeamPath entries of the next chunk are fetched a chunk ahead.  It then
    // takes the rest of the sweep's barriers (and those of an exact
    // re-sweep), and leaves its partial in its merge slot.  One step at a
    // time spreads the BeamKV reads over the sweep instead of adding them
    // to the first tiles' burst (measured at 8 requests x 128 beams, three
    // steps: 22.6 us with all three issued at once, 21.9 us one at a time).
    auto beam_wave_run = [&]() __attribute__((always_inline)) {
        constexpr int BSTEP = 1;
        const int bars = iters + 2;               // barriers of the accumulation sweep
        int done = 0;
        auto tick = [&]() __attribute__((always_inline)) {
            if (done < bars) {
                block_barrier();
                ++done;
            }
        };
        const bool on_row = wave_live && qvalid;
        int qr = qrow;
        asm volatile("" : "+v"(qr));
        const int32_t *prow = p.beam_path + (int64_t)qr * p.T_cap;
        const int64_t req = (int64_t)b * p.beam_cap;
        int idx_next[BSTEP];
#pragma unroll
        for (int u = 0; u < BSTEP; ++u)
            idx_next[u] = on_row && u < T ? prow[u] : 0;
        if (T > 0)
            tick();
        for (int i0 = 0; i0 < T; i0 += BSTEP) {
            u32x4 kr[BSTEP][G16::DC];
            u32x2 vr[BSTEP][G16::DB];
#pragma unroll
            for (int u = 0; u < BSTEP; ++u) {
                const bool on = on_row && i0 + u < T;
                const int64_t base = ((req + idx_next[u]) * p.Hkv + g) * D;
#pragma unroll
                for (int c = 0; c < G16::DC; ++c)
                    kr[u][c] = on ? ldg16(p.beam_k + base + 32 * c + 8 * lg) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int db = 0; db < G16::DB; ++db)
                    vr[u][db] = on ? ldg8(p.beam_v + base + 16 * db + 4 * lg) : u32x2{0, 0};
            }
#pragma unroll
            for (int u = 0; u < BSTEP; ++u) {
                const int st = i0 + BSTEP + u;
                idx_next[u] = on_row && st < T ? prow[st] : 0;
            }
            for (int k = 0; k < BW_SLACK; ++k)
                tick();
#pragma unroll
            for (int u = 0; u < BSTEP; ++u) {
                if (i0 + u >= T)
                    break;
                fold_step(kr[u], vr[u]);
            }
        }
        while (done < bars) {
            block_barrier();
            ++done;
        }
        if (__syncthreads_or(0)) {                 // the sweep waves sweep again
            for (int i = 0; i < 2 * iters + 3; ++i)
                block_barrier();
        }
        l_run += xor16(l_run);
        l_run += xor32(l_run);
        l_lse += xor16(l_lse);
        l_lse += xor32(l_lse);
        if (wave_live) {
            char *sp = smem + ((NKS - 1) * NQT + qt) * G16::OSLOT;
#pragma unroll
            for (int db = 0; db < G16::DB; ++db)
                *reinterpret_cast<f32x4 *>(sp + (db * 64 + lane) * 16) = o[db];
            *reinterpret_cast<f32x4 *>(sp + (G16::DB * 64 + lane) * 16) =
                f32x4{m_ref, l_run, l_lse, 0.f};
        }
        __syncthreads();                           // the merge's barrier
    };
    if constexpr (BW) {
        if (bwave) {
            beam_wave_run();
            return;
        }
    }

    // The first tiles' direct loads go out before the beam stage, so that
    // their latency overlaps the BeamPath and BeamKV loads (the beam stage's
    // waits may also wait for them: they were issued first).
    prefetch();
    if constexpr (!BW)
        beam_stage(true);
    sweep_acc(true, true);
    bool beam_again = false;
    if (__syncthreads_or(qvalid && !(l_lse < SAFE_SUM))) {
        beam_again = !BW;                          // the beam partial is dropped with the rest
        m_ref = NEG_INF;
        l_run = 0.f;
        l_lse = 0.f;
#pragma unroll
        for (int db = 0; db < G16::DB; ++db) {
            acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
            o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        sweep_max();
        sweep_acc(false, false);
    }
#pragma unroll
    for (int db = 0; db < G16::DB; ++db) {
        o[db] = acc[db];
        asm volatile("" : "+v"(o[db]));
    }
    if (beam_again)
        beam_stage(false);
    // full row sums (the four lanes of a query held different keys)
    l_run += xor16(l_run);
    l_run += xor32(l_run);
    l_lse += xor16(l_lse);
    l_lse += xor32(l_lse);

    // ---- merge of the key streams through LDS (log-sum-exp) ---------------
    if constexpr (NKS > 1 || BW) {
        char *ml = smem;                           // the tile ring is free now
        if (ks > 0 && wave_live) {
            char *sp = ml + ((ks - 1) * NQT + qt) * G16::OSLOT;
#pragma unroll
            for (int db = 0; db < G16::DB; ++db)
                *reinterpret_cast<f32x4 *>(sp + (db * 64 + lane) * 16) = o[db];
            *reinterpret_cast<f32x4 *>(sp + (G16::DB * 64 + lane) * 16) =
                f32x4{m_ref, l_run, l_lse, 0.f};
        }
        __syncthreads();
        if (ks == 0 && wave_live) {
#pragma unroll
            // the other key streams' partials, then (BW) the beam wave's
            for (int k2 = 1; k2 < NKS + (BW ? 1 : 0); ++k2) {
                const char *sp = ml + ((k2 - 1) * NQT + qt) * G16::OSLOT;
                const f32x4 st = *reinterpret_cast<const f32x4 *>(sp + (G16::DB * 64 + lane) * 16);
                const float mo = st[0];
                const float mn = __builtin_fmaxf(m_ref, mo);
                const float a = m_ref == NEG_INF ? 0.f : exp2_fast(m_ref - mn);
                const float bw = mo == NEG_INF ? 0.f : exp2_fast(mo - mn);
                m_ref = mn;
                l_run = l_run * a + st[1] * bw;
                l_lse = l_lse * a + st[2] * bw;
#pragma unroll
                for (int db = 0; db < G16::DB; ++db) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(sp + (db * 64 + lane) * 16);
                    o[db] = o[db] * a + v * bw;
                }
            }
        }
    }

    // ---- epilogue: normalise, bf16 output, fp32 natural-log LSE ----------
    if (ks == 0 && wave_live && qvalid) {
        int qr = qrow, qh = qhead;
        asm volatile("" : "+v"(qr), "+v"(qh));
        const int64_t orow = (int64_t)qr * p.Hq + qh;
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        uint16_t *dst = p.out + orow * D + 4 * lg;
#pragma unroll
        for (int db = 0; db < G16::DB; ++db) {
            const u32x2 v = {pack_bf16(o[db][0] * inv, o[db][1] * inv),
                             pack_bf16(o[db][2] * inv, o[db][3] * inv)};
            *reinterpret_cast<u32x2 *>(dst + 16 * db) = v;
        }
        if (lg == 0)
            p.lse[orow] = l_lse > 0.f ? (m_ref + __builtin_log2f(l_lse)) * 0.69314718055994531f
                                      : NEG_INF;
    }
}

template <int D, int NQT, int NKS, int NBUF, int OCC, bool BW, bool PAGED>
static hipError_t launch_fused16_t(const Params &p, int grid, hipStream_t s)
{
    constexpr int lds = lds16_bytes<D, NQT, NKS, NBUF, BW>();
    auto kern = fused_decode_attn16<D, NQT, NKS, NBUF, OCC, BW, PAGED>;
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
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * (NQT * NKS + (BW ? NQT : 0))), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_fused16(const Params &p, int nqt, int nks, int grid, hipStream_t s)
{
#define GR_LAUNCH16_CASE(d, a, c, nb, oc, bw)                                         \
    if (p.D == d && nqt == a && nks == c)                                             \
        return p.page_table ? launch_fused16_t<d, a, c, nb, oc, bw, true>(p, grid, s)   \
                            : launch_fused16_t<d, a, c, nb, oc, bw, false>(p, grid, s);
    GR_FOR_EACH_FUSED16_CONFIG(GR_LAUNCH16_CASE)
#undef GR_LAUNCH16_CASE
    return hipErrorInvalidValue;
}

}  // namespace gr
