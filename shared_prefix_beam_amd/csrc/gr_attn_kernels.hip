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
//     64*NQT stacked query rows: stacked row m = beam * G + i is query head
//     g*G+i of beam `beam`.  Its NQT*NKS waves form NKS key streams of NQT
//     waves; stream ks walks a contiguous 1/NKS share of the context in
//     32-key tiles staged through LDS (double buffered, one barrier per tile).
//   * Each wave holds 64 query columns.  Scores are produced transposed,
//     S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16: the A operand is a K tile
//     fragment read from LDS, the B operand is the wave's Q^T kept in
//     registers for the whole pass.  In the 32x32 accumulator layout every
//     lane holds 16 keys of ONE query, so the row max is an in-lane max3
//     chain plus one v_permlane32_swap.
//   * Probabilities are rounded to bf16 in registers and fed straight back
//     as the B operand of O^T += V^T * P^T; the keys' order inside the
//     contraction follows the accumulator layout, and V is stored transposed
//     in LDS in that same order, so P never leaves registers.
//   * Softmax in the log2 domain against a per-query reference maximum that
//     stays fixed during the context sweep (the first tile's maximum), so the
//     O^T accumulators are written only by the matrix cores inside the loop;
//     a second, exact sweep runs only if a row sum leaves the safe range.
//   * BeamKV steps are spread over the key streams; each stream folds its
//     steps into its own running (max, sum, O) with vector loads along the
//     BeamPath, before the streams merge through LDS by log-sum-exp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gr_attn_internal.h"

namespace gr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 32;          // keys per context tile
constexpr float SAFE_SUM = 1.8446744e19f;  // 2^64: largest row sum accepted in pass 0
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr uint32_t BF16_ONES = 0x3f803f80u;  // two bf16 ones

template <int D>
struct Geo {
    static constexpr int KPITCH = D * 2 + 16;            // bytes per K row in LDS
    static constexpr int VPITCH = KT * 2 + 16;           // bytes per transposed V row (one d)
    static constexpr int KBYTES = KT * KPITCH;
    static constexpr int VBYTES = D * VPITCH;
    static constexpr int TILE = KBYTES + VBYTES;
    static constexpr int STREAM = 2 * TILE;              // double buffered
    static constexpr int DC = D / 16;                    // 16-wide d chunks (QK contraction)
    static constexpr int DB = D / 32;                    // 32-row d blocks of O^T
    static constexpr int OPITCH = (D + 4) * 4;           // bytes per query row in the merge area
    static constexpr int OSLOT = 64 * OPITCH;            // one wave's O partial
};

template <int D, int NQT, int NKS>
constexpr int lds_bytes()
{
    constexpr int stage = NKS * Geo<D>::STREAM;
    constexpr int merge = (NKS - 1) * NQT * (Geo<D>::OSLOT + 64 * 8);
    return stage > merge ? stage : merge;
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x2 ldg8(const uint16_t *p)
{
    return *reinterpret_cast<const u32x2 *>(p);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l^32.  v_permlane32_swap exchanges lanes 32..63 of its
// first operand with lanes 0..31 of its second; with both operands equal to
// x, lanes 0..31 find their partner's value in the second result and lanes
// 32..63 in the first.  `h` is lane / 32.
__device__ __forceinline__ float swap32(float x, int h)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const uint32_t lo = r[0], hi = r[1];
    return __uint_as_float(h ? lo : hi);
}

// position of key x (0..31) of a tile inside the transposed-V row: within
// each 16-key chunk bits 2 and 3 are swapped, matching the order in which a
// lane's accumulator registers hold the keys (see file comment)
__device__ __forceinline__ int vpos(int x)
{
    return (x & 0x13) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc)
{
    // vector elements are copied to scalars before the bit casts: a bit cast
    // applied directly to a subscripted vector element reads element 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = a[i], y = b[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                              __builtin_bit_cast(bf16x2, y), acc, false);
    }
    return acc;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

template <int D, int NQT, int NKS>
__global__ __launch_bounds__(64 * NQT * NKS, 1) void fused_decode_attn(const Params p)
{
    using Gm = Geo<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // ---- work item: (pair, query tile), XCD-aware ----------------------
    // Workgroups are dispatched round-robin over the 8 XCDs; all query tiles
    // of one (request, KV head) pair go to the same XCD so that its L2 holds
    // the pair's ContextKV for every tile.
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
    const int tile_row0 = qtile * 64 * NQT;
    if (tile_row0 >= M)
        return;                                   // uniform for the workgroup
    const int L = p.ctx_len[b];
    const int T = p.beam_len[b];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int qt = wave % NQT;
    const int ks = wave / NQT;
    const int h = lane >> 5;
    const int c32 = lane & 31;
    const int wrow0 = tile_row0 + qt * 64;        // first stacked row of this wave
    const bool wave_live = wrow0 < M;

    // ---- Q^T fragments (B operand), resident for the whole pass -----------
    u32x4 qf[2][Gm::DC];
    int qrow[2];
    bool qvalid[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int m = wrow0 + qb * 32 + c32;
        qvalid[qb] = m < M;
        const int w = qvalid[qb] ? m / G : 0;
        const int i = qvalid[qb] ? m - w * G : 0;
        qrow[qb] = r0 + w;
        const uint16_t *src = p.q + ((int64_t)(r0 + w) * p.Hq + g * G + i) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < Gm::DC; ++c)
            qf[qb][c] = qvalid[qb] ? ldg16(src + 16 * c) : u32x4{0, 0, 0, 0};
    }

    float m_ref[2] = {NEG_INF, NEG_INF};          // reference maximum, log2 units
    float l_run[2] = {0.f, 0.f};                  // this lane-half's share of the sum
    f32x16 acc[2][Gm::DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < Gm::DB; ++db)
            acc[qb][db] = f32x16{};
    const float cs = p.scale_log2;

    // ---- shared (context) stage -----------------------------------------
    const int n_tiles = (L + KT - 1) / KT;
    const int t_begin = (ks * n_tiles) / NKS;
    const int t_end = ((ks + 1) * n_tiles) / NKS;
    const int iters = (n_tiles + NKS - 1) / NKS;  // same for every wave (barrier count)
    char *stream_lds = smem + ks * Gm::STREAM;
    const int64_t kv_base = ((int64_t)b * p.ctx_cap * p.Hkv + g) * D;
    const int64_t kv_tok = (int64_t)p.Hkv * D;    // elements between consecutive tokens
    const int lt = qt * 64 + lane;                // loader id inside the stream

    constexpr int K_CHUNKS = KT * D / 8;          // 16-byte pieces of a K tile
    constexpr int K_PER = (K_CHUNKS + 64 * NQT - 1) / (64 * NQT);
    constexpr int V_UNITS = (KT / 2) * (D / 8);   // (key pair, d octet) units of a V tile
    constexpr int V_PER = (V_UNITS + 64 * NQT - 1) / (64 * NQT);
    u32x4 kreg[K_PER];
    u32x4 vreg[V_PER][2];

    auto load_tile = [&](int t) {
        const int kbase = t * KT;
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int u = lt + i * 64 * NQT;
            const int row = u / (D / 8), col = u % (D / 8);
            const int key = kbase + row;
            kreg[i] = (u < K_CHUNKS && key < L)
                          ? ldg16(p.ctx_k + kv_base + key * kv_tok + col * 8)
                          : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int u = lt + i * 64 * NQT;
            const int kp = u / (D / 8), oc = u % (D / 8);
            const int key = kbase + 2 * kp;
            const bool ok = u < V_UNITS;
            vreg[i][0] = (ok && key < L) ? ldg16(p.ctx_v + kv_base + key * kv_tok + oc * 8)
                                         : u32x4{0, 0, 0, 0};
            vreg[i][1] = (ok && key + 1 < L)
                             ? ldg16(p.ctx_v + kv_base + (key + 1) * kv_tok + oc * 8)
                             : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf) {
        char *kl = stream_lds + buf * Gm::TILE;
        char *vl = kl + Gm::KBYTES;
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int u = lt + i * 64 * NQT;
            if (u < K_CHUNKS) {
                const int row = u / (D / 8), col = u % (D / 8);
                *reinterpret_cast<u32x4 *>(kl + row * Gm::KPITCH + col * 16) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int u = lt + i * 64 * NQT;
            if (u < V_UNITS) {
                const int kp = u / (D / 8), oc = u % (D / 8);
                char *dst = vl + (8 * oc) * Gm::VPITCH + vpos(2 * kp) * 2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t a = vreg[i][0][e], c = vreg[i][1][e];
                    *reinterpret_cast<uint32_t *>(dst + (2 * e) * Gm::VPITCH) =
                        __builtin_amdgcn_perm(c, a, 0x05040100u);
                    *reinterpret_cast<uint32_t *>(dst + (2 * e + 1) * Gm::VPITCH) =
                        __builtin_amdgcn_perm(c, a, 0x07060302u);
                }
            }
        }
    };

    // One sweep over the stream's tiles.  ACCUM: p = exp2(s*c - m_ref) with a
    // fixed per-query reference m_ref (taken from the stream's first tile
    // unless `given_ref`); the accumulators are touched only by the matrix
    // cores inside the loop.  MAXONLY: exact per-query maxima, no values.
    auto sweep = [&](bool accum, bool given_ref) {
        if (iters > 0) {
            if (t_begin < t_end) {
                load_tile(t_begin);
                store_tile(0);
            }
            __syncthreads();
        }
        for (int it = 0; it < iters; ++it) {
            const int t = t_begin + it;
            const bool active = t < t_end;
            const bool has_next = t + 1 < t_end;
            if (has_next)
                load_tile(t + 1);
            if (active && wave_live) {
                const char *kl = stream_lds + (it & 1) * Gm::TILE;
                const char *vl = kl + Gm::KBYTES;
                // S^T = K * Q^T for both query blocks
                f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int c = 0; c < Gm::DC; ++c) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(kl + c32 * Gm::KPITCH +
                                                                     (2 * c + h) * 16);
                    const bf16x8 av = __builtin_bit_cast(bf16x8, a);
                    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        av, __builtin_bit_cast(bf16x8, qf[0][c]), s[0], 0, 0, 0);
                    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        av, __builtin_bit_cast(bf16x8, qf[1][c]), s[1], 0, 0, 0);
                }
                // keys past the context end (only in the last tile)
                const int kbase = t * KT;
                if (kbase + KT > L) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (key >= L) {
                            s[0][r] = NEG_INF;
                            s[1][r] = NEG_INF;
                        }
                    }
                }
                if (!accum || (it == 0 && !given_ref)) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        float mx = s[qb][0];
#pragma unroll
                        for (int r = 1; r < 16; ++r)
                            mx = __builtin_fmaxf(mx, s[qb][r]);
                        mx = __builtin_fmaxf(mx, swap32(mx, h));
                        m_ref[qb] = __builtin_fmaxf(m_ref[qb], mx * cs);
                    }
                }
                if (accum) {
                    // probabilities, row sums, bf16 B operands
                    u32x4 pb[2][2];
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        const float nm = -m_ref[qb];
                        float pr[16];
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            pr[r] = exp2_fast(__builtin_fmaf(s[qb][r], cs, nm));
                        // the row sum adds the bf16-rounded probabilities that
                        // the matrix cores multiply, so the normalisation
                        // matches the weighted sum exactly
                        float sum = l_run[qb];
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const uint32_t pk =
                                    pack_bf16(pr[8 * kc + 2 * e], pr[8 * kc + 2 * e + 1]);
                                pb[qb][kc][e] = pk;
                                sum = __builtin_amdgcn_fdot2_f32_bf16(
                                    __builtin_bit_cast(bf16x2, pk),
                                    __builtin_bit_cast(bf16x2, BF16_ONES), sum, false);
                            }
                        l_run[qb] = sum;
                    }
                    // O^T += V^T * P^T
#pragma unroll
                    for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc) {
                            const u32x4 a = *reinterpret_cast<const u32x4 *>(
                                vl + (32 * db + c32) * Gm::VPITCH + (16 * kc + 8 * h) * 2);
                            const bf16x8 av = __builtin_bit_cast(bf16x8, a);
                            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                av, __builtin_bit_cast(bf16x8, pb[0][kc]), acc[0][db], 0, 0, 0);
                            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                av, __builtin_bit_cast(bf16x8, pb[1][kc]), acc[1][db], 0, 0, 0);
                        }
                }
            }
            if (has_next)
                store_tile((it + 1) & 1);
            __syncthreads();
        }
    };

    // Pass 0 takes each stream's first-tile maximum as the fixed reference:
    // later tiles may exceed it, so probabilities can grow past 1.  As long
    // as every row sum stays below 2^64 nothing can overflow and the final
    // normalisation is exact.  Otherwise (scores rising by more than ~44
    // nats along the context) the workgroup sweeps again: exact maxima
    // first, then the accumulation against them.
    sweep(true, false);
    {
        bool bad = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
            bad |= qvalid[qb] && !(l_run[qb] < SAFE_SUM);
        if (__syncthreads_or(bad)) {
            m_ref[0] = m_ref[1] = NEG_INF;
            l_run[0] = l_run[1] = 0.f;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
                    acc[qb][db] = f32x16{};
            sweep(false, false);
            sweep(true, true);
        }
    }

    // ---- per-beam stage: BeamKV steps ks, ks+NKS, ... along BeamPath ------
    if (wave_live) {
        for (int s = ks; s < T; s += NKS) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int idx = qvalid[qb] ? p.beam_path[(int64_t)qrow[qb] * p.T_cap + s] : 0;
                const int64_t base = (((int64_t)b * p.beam_cap + idx) * p.Hkv + g) * D;
                const uint16_t *kr = p.beam_k + base + 8 * h;
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < Gm::DC; ++c)
                    dot = dot8(qf[qb][c], qvalid[qb] ? ldg16(kr + 16 * c) : u32x4{0, 0, 0, 0},
                               dot);
                dot += swap32(dot, h);
                const float tz = dot * cs;
                const float mn = __builtin_fmaxf(m_ref[qb], tz);
                const float alpha = exp2_fast(m_ref[qb] - mn);
                const float pw = exp2_fast(tz - mn);
                m_ref[qb] = mn;
                l_run[qb] = l_run[qb] * alpha + (h == 0 ? pw : 0.f);
                const uint16_t *vr = p.beam_v + base + 4 * h;
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const u32x2 v = qvalid[qb] ? ldg8(vr + 32 * db + 8 * rg) : u32x2{0, 0};
                        f32x16 &o = acc[qb][db];
                        o[4 * rg + 0] = o[4 * rg + 0] * alpha + pw * bf16lo(v[0]);
                        o[4 * rg + 1] = o[4 * rg + 1] * alpha + pw * bf16hi(v[0]);
                        o[4 * rg + 2] = o[4 * rg + 2] * alpha + pw * bf16lo(v[1]);
                        o[4 * rg + 3] = o[4 * rg + 3] * alpha + pw * bf16hi(v[1]);
                    }
            }
        }
    }
    // full row sums (the two lane halves held different keys)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
        l_run[qb] += swap32(l_run[qb], h);

    // ---- merge of the key streams through LDS (log-sum-exp) ---------------
    if constexpr (NKS > 1) {
        char *ml = smem;                           // staging buffers are free now
        if (ks > 0 && wave_live) {
            const int slot = (ks - 1) * NQT + qt;
            char *o = ml + slot * (Gm::OSLOT + 64 * 8);
            float *stats = reinterpret_cast<float *>(o + Gm::OSLOT);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int qc = qb * 32 + c32;
                if (h == 0) {
                    stats[2 * qc] = m_ref[qb];
                    stats[2 * qc + 1] = l_run[qb];
                }
#pragma unroll
                for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        f32x4 v = {acc[qb][db][4 * rg], acc[qb][db][4 * rg + 1],
                                   acc[qb][db][4 * rg + 2], acc[qb][db][4 * rg + 3]};
                        *reinterpret_cast<f32x4 *>(o + qc * Gm::OPITCH +
                                                   (32 * db + 8 * rg + 4 * h) * 4) = v;
                    }
            }
        }
        __syncthreads();
        if (ks == 0 && wave_live) {
            for (int k2 = 1; k2 < NKS; ++k2) {
                const int slot = (k2 - 1) * NQT + qt;
                const char *o = ml + slot * (Gm::OSLOT + 64 * 8);
                const float *stats = reinterpret_cast<const float *>(o + Gm::OSLOT);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const int qc = qb * 32 + c32;
                    const float mo = stats[2 * qc], lo = stats[2 * qc + 1];
                    const float mn = __builtin_fmaxf(m_ref[qb], mo);
                    const float a = m_ref[qb] == NEG_INF ? 0.f : exp2_fast(m_ref[qb] - mn);
                    const float bw = mo == NEG_INF ? 0.f : exp2_fast(mo - mn);
                    m_ref[qb] = mn;
                    l_run[qb] = l_run[qb] * a + lo * bw;
#pragma unroll
                    for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg) {
                            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                                o + qc * Gm::OPITCH + (32 * db + 8 * rg + 4 * h) * 4);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[qb][db][4 * rg + e] = acc[qb][db][4 * rg + e] * a + v[e] * bw;
                        }
                }
            }
        }
    }

    // ---- epilogue: normalise, bf16 output, fp32 natural-log LSE ----------
    if (ks == 0 && wave_live) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            if (!qvalid[qb])
                continue;
            const int m = wrow0 + qb * 32 + c32;
            const int w = m / G;
            const int i = m - w * G;
            const int hq = g * G + i;
            const int64_t orow = ((int64_t)(r0 + w) * p.Hq + hq);
            const float l = l_run[qb];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            uint16_t *dst = p.out + orow * D + 4 * h;
#pragma unroll
            for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const f32x16 &o = acc[qb][db];
                    u32x2 v = {pack_bf16(o[4 * rg] * inv, o[4 * rg + 1] * inv),
                               pack_bf16(o[4 * rg + 2] * inv, o[4 * rg + 3] * inv)};
                    *reinterpret_cast<u32x2 *>(dst + 32 * db + 8 * rg) = v;
                }
            if (h == 0)
                p.lse[orow] = l > 0.f ? (m_ref[qb] + __builtin_log2f(l)) * 0.69314718055994531f
                                      : NEG_INF;
        }
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
template <int D, int NQT, int NKS>
static hipError_t launch_fused_t(const Params &p, int grid, hipStream_t s)
{
    constexpr int lds = lds_bytes<D, NQT, NKS>();
    auto kern = fused_decode_attn<D, NQT, NKS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NQT * NKS), lds, s, p);
    return hipGetLastError();
}

int fused_lds_bytes(int D, int nqt, int nks)
{
#define GR_LDS_CASE(d, a, c)                                                          \
    if (D == d && nqt == a && nks == c)                                               \
        return lds_bytes<d, a, c>();
    GR_FOR_EACH_FUSED_CONFIG(GR_LDS_CASE)
#undef GR_LDS_CASE
    return -1;
}

hipError_t launch_fused(const Params &p, int nqt, int nks, int grid, hipStream_t s)
{
#define GR_LAUNCH_CASE(d, a, c)                                                       \
    if (p.D == d && nqt == a && nks == c)                                             \
        return launch_fused_t<d, a, c>(p, grid, s);
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
