// Device code of beam selection: log_softmax + top-K over (beam, token)
// candidates with early-terminated sorting (xGR review, section "xBeam":
// a global heap of the beam width; a beam's candidates stop being sorted
// once they fall below the heap's least element; SID-GR README, "Roadmap":
// log_softmax + top-K + beam selection moved onto the device).
//
// Candidate (w, v) of request b has value score_old[w] + logits[w][v] -
// LSE_w.  It is ranked by a distinct 64-bit key: the order-preserving bits of
// its fp32 value above the complemented flat index w*V + v, so that larger
// values come first and, among equal values, smaller indices.
//
// gfx950 mapping, two launches:
//  1. select_rows: one 256-thread workgroup per beam row reads the row's
//     logits once into registers, reduces max and log-sum-exp, and keeps the
//     row's L = min(K, 32) best keys, sorted.  The L-th best of the 256
//     thread maxima bounds the row's L-th best key from below, so the radix
//     select (8-bit digits, LDS histograms) only sees the few keys above it.
//  2. select_request: one 1024-thread workgroup per request.  The K-th best
//     of the rows' 8 best keys bounds the request's K-th best candidate from
//     below; every row's list is cut at that bound (the early termination),
//     and a row whose whole list clears it while it has more candidates is
//     selected again from its logits.  The exact K best of the survivors
//     (held in LDS) are selected, sorted in registers and written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gr_attn_internal.h"

namespace gr {

constexpr int SEL_ROW_THREADS = 256;
constexpr int SEL_REQ_THREADS = 1024;
constexpr int SEL_HEAD = 8;                               // keys per row behind the bound
constexpr int SEL_HEAD_FAR = 6;                           // the same, rows beyond one chunk
constexpr int SEL_HEAD_REG = 8;                           // head keys per thread in registers
constexpr int SEL_SURV_REG = 4;                           // survivors per thread in registers
constexpr int SEL_SURV_LDS = SEL_SURV_REG * SEL_REQ_THREADS;
constexpr int SEL_REQ_NV = SEL_MAX_V / SEL_REQ_THREADS;   // logits per thread, re-selection
// (512 threads of 16 candidates per row for vocabularies up to 8192, each
// row's chain half as long, measured slower than 256 of 32: 8 x 128 beams
// 27.1 -> 28.2 us, 4 x 900 55.1 -> 60.3 us.)
constexpr int SEL_WCAND = 256;                            // the same, one wave per row

// Order-preserving bits of a float: negative values complemented, the sign
// bit set on the others (the sign, spread by an arithmetic shift, picks the
// mask: three vector instructions)
__device__ __forceinline__ uint32_t ord_f32(float f)
{
    const uint32_t u = __float_as_uint(f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(uint32_t ord, uint32_t flat)
{
    return ((uint64_t)ord << 32) | (uint32_t)~flat;
}

// Value of lane (lane ^ J) for J in {1, 2, 4, 8}, through DPP moves (VALU,
// no LDS traffic): quad permutations for 1 and 2; for 4 and 8 a row shift
// up (lane + J) or down (lane - J), picked by the lane's bit J.
template <int J>
__device__ __forceinline__ uint32_t dpp_xor_u32(uint32_t v)
{
    const int x = (int)v;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    } else {
        const int up = __builtin_amdgcn_update_dpp(0, x, 0x100 + J, 0xF, 0xF, false);
        const int dn = __builtin_amdgcn_update_dpp(0, x, 0x110 + J, 0xF, 0xF, false);
        return (uint32_t)((threadIdx.x & J) ? dn : up);
    }
}

template <int J>
__device__ __forceinline__ uint64_t dpp_xor_u64(uint64_t v)
{
    const uint32_t lo = dpp_xor_u32<J>((uint32_t)v), hi = dpp_xor_u32<J>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Value of lane (lane ^ J) for any power of two J < 64 without LDS traffic:
// the DPP moves above for J <= 8; for 16 and 32 one v_permlane16_swap /
// v_permlane32_swap with both operands equal to v (it exchanges the odd
// 16-lane rows, resp. the upper half, of its first operand with the even
// rows, resp. the lower half, of its second: a lane finds its partner's
// value in the first result when its bit J is set, else in the second).
template <int J>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v)
{
    if constexpr (J <= 8) {
        return dpp_xor_u32<J>(v);
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & 16) ? (uint32_t)r[0] : (uint32_t)r[1];
    } else {
        static_assert(J == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? (uint32_t)r[0] : (uint32_t)r[1];
    }
}

template <int J>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v)
{
    const uint32_t lo = lane_xor_u32<J>((uint32_t)v), hi = lane_xor_u32<J>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Butterfly over the wave: every lane ends with op over all 64 lanes.
template <class T, class Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op)
{
    auto x = [](T a, auto tag) -> T {
        constexpr int J = decltype(tag)::value;
        if constexpr (sizeof(T) == 8) {
            return __builtin_bit_cast(T, lane_xor_u64<J>(__builtin_bit_cast(uint64_t, a)));
        } else {
            return __builtin_bit_cast(T, lane_xor_u32<J>(__builtin_bit_cast(uint32_t, a)));
        }
    };
    v = op(v, x(v, std::integral_constant<int, 32>{}));
    v = op(v, x(v, std::integral_constant<int, 16>{}));
    v = op(v, x(v, std::integral_constant<int, 8>{}));
    v = op(v, x(v, std::integral_constant<int, 4>{}));
    v = op(v, x(v, std::integral_constant<int, 2>{}));
    v = op(v, x(v, std::integral_constant<int, 1>{}));
    return v;
}

// Inclusive prefix sum over the lanes in order, with DPP: shifts by 1, 2, 4
// and 8 lanes inside each 16-lane row (a lane with no source adds 0), then
// the last lane of rows 0 and 2 broadcast into rows 1 and 3, then lane 31
// into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Value of a wave-uniform lane `src`.
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// Largest and smallest 64-bit key over the block (every thread passes its
// own; threads with no key pass kmax = 0, kmin = ~0).  One barrier; `red`
// may be written again only after a later barrier.
template <int NT>
__device__ void block_minmax(uint64_t &kmax, uint64_t &kmin, uint64_t *red)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    kmax = wave_allreduce(kmax, [](uint64_t a, uint64_t c) { return a > c ? a : c; });
    kmin = wave_allreduce(kmin, [](uint64_t a, uint64_t c) { return a < c ? a : c; });
    if (lane == 0) {
        red[2 * wv] = kmax;
        red[2 * wv + 1] = kmin;
    }
    __syncthreads();
    kmax = red[0];
    kmin = red[1];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
        kmax = red[2 * w] > kmax ? red[2 * w] : kmax;
        kmin = red[2 * w + 1] < kmin ? red[2 * w + 1] : kmin;
    }
}

// Sum over the block; one barrier, `red` reusable after a later barrier.
template <int NT>
__device__ int block_sum(int v, int *red)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    v = wave_allreduce(v, [](int a, int c) { return a + c; });
    if (lane == 0)
        red[wv] = v;
    __syncthreads();
    v = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
        v += red[w];
    return v;
}

// Inclusive prefix sum over the threads in order, and the total.  One
// barrier; `wsum` reusable after a later barrier.
template <int NT>
__device__ int block_incl_scan(int v, int *wsum, int &total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    v = wave_incl_scan(v);
    if (lane == 63)
        wsum[wv] = v;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int s = wsum[w];
        before += w < wv ? s : 0;
        total += s;
    }
    return v + before;
}

// In a complete 256-bin histogram h (published by a barrier), the digit d
// where the count from the top digit down reaches `remaining`, the count
// above d and d's own count; every lane of every wave gets the same three.
// Lane l holds bins 4l .. 4l+3; suffix sums over the lanes find the lane.
__device__ __forceinline__ void hist_find(const uint32_t *h, int remaining, int &d, int &above,
                                          int &cnt)
{
    const int lane = threadIdx.x & 63;
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        b[j] = h[4 * lane + j];
    const uint32_t own = b[0] + b[1] + b[2] + b[3];
    // suffix sum over the lanes: the total less the prefix before this lane
    const int incl = wave_incl_scan((int)own);
    const uint32_t suf = (uint32_t)(lane_value(incl, 63) - incl) + own;
    const uint32_t above_lane = suf - own;
    const bool here = suf >= (uint32_t)remaining && above_lane < (uint32_t)remaining;
    int d_l = 0, above_l = 0, cnt_l = 0;
    if (here) {
        uint32_t cum = above_lane;
        for (int j = 3; j >= 0; --j) {
            if (cum + b[j] >= (uint32_t)remaining || j == 0) {
                d_l = 4 * lane + j;
                above_l = (int)cum;
                cnt_l = (int)b[j];
                break;
            }
            cum += b[j];
        }
    }
    const int src = __ffsll((unsigned long long)__ballot(here)) - 1;
    d = lane_value(d_l, src);
    above = lane_value(above_l, src);
    cnt = lane_value(cnt_l, src);
}

// Threshold of the k-th largest of n distinct keys lying in [kmin, kmax], as
// (prefix, mask): the k largest keys are exactly those with (key & mask) >=
// prefix.  The bits kmin and kmax share are shared by every key and decided
// at once; the rest are resolved 8 bits per pass from the top.  Each pass
// counts the keys still matching into a 256-bin LDS histogram; after one
// barrier every wave reads it and finds the digit where the count from the
// top reaches k.  The passes stop once every key of the chosen bin is
// needed.  Three histograms rotate (hist3, 3 x 256): on entry
// hist3[256*hbuf ..] is zero and published by a barrier; on exit hbuf names
// the one zeroed by the last pass.  visit(f) calls f(key) for each key the
// calling thread owns.  Requires 1 <= k <= n; all NT threads call it.
template <int NT, class Visit>
__device__ void radix_kth(int k, uint64_t kmax, uint64_t kmin, Visit visit, uint32_t *hist3,
                          int &hbuf, uint64_t &prefix_out, uint64_t &mask_out)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const uint64_t diff = kmax ^ kmin;
    const int common = diff ? __clzll(diff) : 64;
    uint64_t mask = common == 0 ? 0 : (~0ull << (64 - common));
    uint64_t prefix = kmax & mask;
    int hi = 64 - common;                    // bits [0, hi) still undecided
    int remaining = k;
    while (hi > 0) {
        uint32_t *h = hist3 + 256 * hbuf;
        const int nb = hbuf == 2 ? 0 : hbuf + 1;
        uint32_t *hn = hist3 + 256 * nb;
        for (int i = tid; i < 256; i += NT)
            hn[i] = 0;                            // the histogram of the next pass
        const int lo = hi > 8 ? hi - 8 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        visit([&](uint64_t key) {
            if ((key & mask) == prefix)
                atomicAdd(&h[(uint32_t)(key >> lo) & dmask], 1u);
        });
        __syncthreads();
        int d, above, cnt;
        hist_find(h, remaining, d, above, cnt);
        prefix |= (uint64_t)d << lo;
        mask |= (uint64_t)dmask << lo;
        remaining -= above;
        hi = lo;
        hbuf = nb;
        if (cnt == remaining)
            break;
    }
    prefix_out = prefix;
    mask_out = mask;
}

// Slot of this lane's item in an append to *counter (one atomic per wave);
// called by the lanes that reach it, `take` says which of them append.
__device__ __forceinline__ int wave_append(bool take, int *counter)
{
    const uint64_t ballot = __ballot(take);
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((unsigned long long)ballot) - 1;
    int base = 0;
    if (ballot) {
        if (lane == leader)
            base = atomicAdd(counter, __popcll(ballot));
        base = lane_value(base, leader);
    }
    return base + __popcll(ballot & ((1ull << lane) - 1ull));
}

// Bitonic sort of one key per thread into descending order over threads
// 0 .. ns-1 (ns a power of two <= NT; threads from ns on hold 0).  Each
// stage is its own instantiation, so its partner distance J and block size
// K are constants: 1, 2, 4 and 8 lanes away exchange through DPP, 16 and 32
// through lane shuffles, wider ones through one of two LDS buffers in turn
// (xch2: 2 x NT keys), one barrier each.  A thread takes its partner's key
// when (partner > own) matches (lower of the pair == block sorts descending).
template <int NT, int K, int J>
__device__ __forceinline__ void bitonic_stage(uint64_t &key, uint64_t *xch2, int &buf)
{
    const int tid = threadIdx.x;
    uint64_t other;
    if constexpr (J >= 64) {
        uint64_t *x = xch2 + NT * buf;
        x[tid] = key;
        __syncthreads();
        other = x[tid ^ J];
        buf ^= 1;
    } else if constexpr (J <= 8) {
        other = dpp_xor_u64<J>(key);
    } else {
        other = lane_xor_u64<J>(key);
    }
    const bool same = ((tid & J) == 0) == ((tid & K) == 0);
    key = ((other > key) == same) ? other : key;
    if constexpr (J > 1)
        bitonic_stage<NT, K, J / 2>(key, xch2, buf);
}

template <int NT, int K>
__device__ __forceinline__ void bitonic_from(uint64_t &key, int ns, uint64_t *xch2, int &buf)
{
    if (K <= ns) {                                  // wave-uniform
        bitonic_stage<NT, K, K / 2>(key, xch2, buf);
        if constexpr (K < NT)
            bitonic_from<NT, 2 * K>(key, ns, xch2, buf);
    }
}

template <int NT>
__device__ uint64_t block_sort_desc(uint64_t key, int ns, uint64_t *xch2)
{
    int buf = 0;
    bitonic_from<NT, 2>(key, ns, xch2, buf);
    return key;
}

__device__ __forceinline__ int pow2_at_least(int n)
{
    int p = 1;
    while (p < n)
        p <<= 1;
    return p;
}

// request b with row_offset[b] <= r < row_offset[b+1]
__device__ __forceinline__ int request_of(const int32_t *row_offset, int B, int r)
{
    int lo = 0, hi = B;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (row_offset[mid] <= r)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// Candidates of a beam row: every token (TRIE false), or the labels of the
// edges leaving the beam's trie node (TRIE true): candidate v is edge e0 + v,
// token edge_tok[e0 + v].  A key's index part is w * V + v; the edge labels
// increase with v, so ties still go to the smaller token.
__device__ __forceinline__ void row_candidates(const SelParams &p, int r, bool trie, int cap,
                                               int &n, int &e0)
{
    n = p.V;
    e0 = 0;
    if (trie) {
        n = 0;
        const int node = p.node_old[r];
        if (node >= 0 && node < p.n_nodes) {
            int a = p.node_ptr[node], z = p.node_ptr[node + 1];
            a = a < 0 ? 0 : (a > p.n_edges ? p.n_edges : a);
            z = z < a ? a : (z > p.n_edges ? p.n_edges : z);
            e0 = a;
            n = z - a < p.V ? z - a : p.V;          // distinct labels below V
            n = n < p.max_fanout ? n : p.max_fanout;  // a node's first max_fanout edges
            n = n < cap ? n : cap;
        }
    }
}

// One beam row per workgroup of NT threads; NV candidates per thread (n <=
// NV * NT).  With NV <= 32 the kernel fits 96 registers, i.e. five waves per
// SIMD: a row's loads are a third of its time, so more resident rows keep
// HBM busy (measured: four waves 79.1 us, five 75.2 us per 4 x 900 x 8192
// call); with NV <= 16, 64 registers (eight waves).
template <int NV, int NT, bool TRIE>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(NV <= 16 ? 8 : (NV <= 32 ? 5 : 2)))) void select_rows(const SelParams p)
{
    constexpr int NW = NT / 64;
    static_assert(NT % 64 == 0 && NT >= 256, "whole waves; the histograms need 256 threads");
    __shared__ float red[NW];
    __shared__ int wsum[NW];
    __shared__ uint64_t tq[NW];
    __shared__ uint64_t cand[NT];
    __shared__ uint64_t red64[2 * NW];
    // used only when many keys tie around the bound
    __shared__ uint32_t hist3[3 * 256];
    __shared__ uint64_t buf[SEL_LIST];
    __shared__ int n_buf;

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int b = request_of(p.row_offset_old, p.B, r);
    const int wl = r - p.row_offset_old[b];
    int k_row = p.row_offset_new[b + 1] - p.row_offset_new[b];
    k_row = k_row < p.V ? k_row : p.V;
    k_row = k_row < p.K_max ? k_row : p.K_max;
    if (k_row <= 0)
        return;
    const int L = k_row < SEL_LIST ? k_row : SEL_LIST;
    int n, e0;
    row_candidates(p, r, TRIE, NV * NT, n, e0);
    if (tid == 0) {
        p.ws_n[r] = n;
        p.ws_e0[r] = e0;
    }
    uint64_t *list = p.ws_list + (int64_t)r * SEL_LIST;
    if (n == 0) {                                 // no legal token: an empty list
        if (tid < L)
            list[tid] = 0;
        return;
    }

    const float *row = p.logits + (int64_t)r * p.V;
    const uint32_t flat0 = (uint32_t)wl * (uint32_t)p.V + (uint32_t)tid;
    // The body, for rows whose NV*NT candidate slots are all taken (every
    // unconstrained row of an NV*NT vocabulary: no per-slot validity test
    // at all) and for the others.  Validity and key comparisons are kept to
    // 32 bits where the 64-bit keys allow it: every bound below has zero
    // index bits, so key >= bound is value bits >= the bound's value bits.
    auto run = [&](auto full_tag) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        auto valid = [&](int i) { return FULL || tid + NT * i < n; };
        float x[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + NT * i;
            int t = v;
            if (TRIE && valid(i))
                t = p.edge_tok[e0 + v];
            x[i] = (valid(i) && t >= 0 && t < p.V) ? row[t] : -__builtin_huge_valf();
        }
        // max and log-sum-exp over the row
        float m = x[0];
#pragma unroll
        for (int i = 1; i < NV; ++i)
            m = __builtin_fmaxf(m, x[i]);
        m = wave_allreduce(m, [](float a, float c) { return __builtin_fmaxf(a, c); });
        if (lane == 0)
            red[wv] = m;
        __syncthreads();
        m = red[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            m = __builtin_fmaxf(m, red[w]);
        __syncthreads();
        // exp(x - m) as 2^(x log2 e - m log2 e): one fused multiply-add and
        // one v_exp_f32 per logit
        constexpr float L2E = 1.4426950408889634f;
        const float nm = -m * L2E;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            s += __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], L2E, nm));
        s = wave_allreduce(s, [](float a, float c) { return a + c; });
        if (lane == 0)
            red[wv] = s;
        __syncthreads();
        s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            s += red[w];
        const float off_w = p.score_old[r] - (m + __logf(s));
        if (tid == 0)
            p.ws_off[r] = off_w;

        // the candidates' ordered value bits replace the logits; invalid
        // slots hold 0, below every bound used with them
        uint32_t o[NV];
        uint32_t omax = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            o[i] = valid(i) ? ord_f32(off_w + x[i]) : 0u;
            omax = o[i] > omax ? o[i] : omax;
        }
        // t0: when every thread holds keys (n >= NT), each wave's q-th best
        // thread maximum value (q = ceil(L / NW)), found bit by bit with
        // ballots over the 32 value bits: at least q distinct keys of the
        // wave have that value or more, so the key with that value and zero
        // index bits bounds them from below (ties at the value only loosen
        // the bound).  The smallest of the NW bounds has L distinct keys at
        // or above it; otherwise t0 = 0 (fewer than NT keys)
        uint32_t th = 0;                          // t0 = th << 32
        if (n >= NT) {
            const int q = (L + NW - 1) / NW;
            uint32_t res = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand_bits = res | (1u << bit);
                if (__popcll(__ballot(omax >= cand_bits)) >= q)
                    res = cand_bits;
            }
            if (lane == 0)
                tq[wv] = res;
            __syncthreads();
            th = (uint32_t)tq[0];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                th = (uint32_t)tq[w] < th ? (uint32_t)tq[w] : th;
        }
        // the keys >= t0, compacted in thread order
        auto above = [&](int i) { return valid(i) && o[i] >= th; };
        int c = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            c += above(i) ? 1 : 0;
        int M;
        const int incl = block_incl_scan<NT>(c, wsum, M);
        if (M <= NT) {
            int at = incl - c;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (above(i))
                    cand[at++] = make_key(o[i], flat0 + NT * i);
            __syncthreads();
            // rank among the candidates: the L best land in the row's list in order
            if (tid < M) {
                const uint64_t mine = cand[tid];
                int rk = 0;
                for (int j = 0; j < M; ++j)
                    rk += cand[j] > mine ? 1 : 0;
                if (rk < L)
                    list[rk] = mine;
            }
            if (tid >= M && tid < L)              // fewer candidates than L: pad
                list[tid] = 0;
            return;
        }
        // many keys at or above t0: radix select of the L best among them
        const uint64_t t0 = (uint64_t)th << 32;
        if (tid < 256)
            hist3[tid] = 0;
        uint64_t best = 0, unused = ~0ull;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint64_t key = make_key(o[i], flat0 + NT * i);
            if (above(i) && key > best)
                best = key;
        }
        block_minmax<NT>(best, unused, red64);    // its barrier publishes hist3
        int hb = 0;
        uint64_t pf, mk;
        radix_kth<NT>(
            L, best, t0,
            [&](auto f) {
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (above(i))
                        f(make_key(o[i], flat0 + NT * i));
            },
            hist3, hb, pf, mk);
        if (tid == 0)
            n_buf = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint64_t key = make_key(o[i], flat0 + NT * i);
            const bool take = above(i) && (key & mk) >= pf;
            const int at = wave_append(take, &n_buf);
            if (take && at < L)
                buf[at] = key;
        }
        __syncthreads();
        if (tid < L) {
            const uint64_t mine = buf[tid];
            int rk = 0;
            for (int j = 0; j < L; ++j)
                rk += buf[j] > mine ? 1 : 0;
            list[rk] = mine;
        }
    };
    if (n == NV * NT)                             // uniform for the workgroup
        run(std::true_type{});
    else
        run(std::false_type{});
}

__device__ __forceinline__ float wave_max(float v)
{
    return wave_allreduce(v, [](float a, float c) { return __builtin_fmaxf(a, c); });
}

__device__ __forceinline__ float wave_sum(float v)
{
    return wave_allreduce(v, [](float a, float c) { return a + c; });
}

__device__ __forceinline__ int wave_sum_i(int v)
{
    return wave_allreduce(v, [](int a, int c) { return a + c; });
}

// One beam row per wave, four rows per 256-thread workgroup, no block
// barriers: candidate v = lane + 64 i (i < NL) sits in a register.  The
// row's L best keys all have ordered value bits >= res, the L-th largest of
// the 64 lane maxima (L distinct keys reach it), found by a 32-step ballot
// search; the few keys above it are compacted in order into the wave's LDS
// slice and ranked by counting.  With more than SEL_WCAND of them (ties at
// the bound) the exact L-th largest value is searched instead and the ties
// at it are taken in index order.
template <int NL, bool TRIE>
__global__ __launch_bounds__(256) void select_rows_wave(const SelParams p)
{
    __shared__ uint64_t cand_all[4][SEL_WCAND];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = blockIdx.x * 4 + wv;
    if (r >= p.R_old)
        return;
    uint64_t *cand = cand_all[wv];
    // the candidate chain (node, its edges, their logits) first: it does
    // not depend on the request lookup, which overlaps with it
    int n, e0;
    row_candidates(p, r, TRIE, 64 * NL, n, e0);
    const float *row = p.logits + (int64_t)r * p.V;
    float x[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int v = lane + 64 * i;
        int t = v;
        if (TRIE && v < n)
            t = p.edge_tok[e0 + v];
        x[i] = (v < n && t >= 0 && t < p.V) ? row[t] : -__builtin_huge_valf();
    }
    const float score = p.score_old[r];
    const int b = request_of(p.row_offset_old, p.B, r);
    const int wl = r - p.row_offset_old[b];
    int k_row = p.row_offset_new[b + 1] - p.row_offset_new[b];
    k_row = k_row < p.V ? k_row : p.V;
    k_row = k_row < p.K_max ? k_row : p.K_max;
    if (k_row <= 0)
        return;
    const int L = k_row < SEL_LIST ? k_row : SEL_LIST;
    if (lane == 0) {
        p.ws_n[r] = n;
        p.ws_e0[r] = e0;
    }
    uint64_t *list = p.ws_list + (int64_t)r * SEL_LIST;
    if (n == 0) {                                 // no legal token: an empty list
        if (lane < L)
            list[lane] = 0;
        return;
    }
    float m = x[0];
#pragma unroll
    for (int i = 1; i < NL; ++i)
        m = __builtin_fmaxf(m, x[i]);
    m = wave_max(m);
    constexpr float L2E = 1.4426950408889634f;   // exp(x - m) = 2^(x log2 e - m log2 e)
    const float nm = -m * L2E;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i)
        s += __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], L2E, nm));
    s = wave_sum(s);
    const float off_w = score - (m + __logf(s));
    if (lane == 0)
        p.ws_off[r] = off_w;

    // ordered value bits of candidate i, 0 when there is none (every real
    // one is >= 1); rebuilt from x in each pass (an opaque copy of off_w
    // keeps the compiler from holding all of them in registers)
    struct Pass {
        float ow;
        int lim;                                  // candidates of this lane: v < n
    };
    auto ord_at = [&](int i, Pass q) -> uint32_t {
        return 64 * i < q.lim ? ord_f32(q.ow + x[i]) : 0u;
    };
    auto fresh = [&]() {
        Pass q{off_w, n - lane};
        asm volatile("" : "+v"(q.ow), "+v"(q.lim));
        return q;
    };
    uint32_t omax = 0;
    {
        const Pass ow = fresh();
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t oi = ord_at(i, ow);
            omax = oi > omax ? oi : omax;
        }
    }
    const uint32_t flat0 = (uint32_t)wl * (uint32_t)p.V + (uint32_t)lane;
    uint32_t res = 1;
    if (n >= L) {                                 // min(n, 64) >= L lanes hold candidates
        uint32_t acc = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = acc | (1u << bit);
            if (__popcll(__ballot(omax >= c)) >= L)
                acc = c;
        }
        res = acc > 1u ? acc : 1u;
    }
    int c = 0;
    {
        const Pass ow = fresh();
#pragma unroll
        for (int i = 0; i < NL; ++i)
            c += ord_at(i, ow) >= res ? 1 : 0;
    }
    int incl = wave_incl_scan(c);
    int M = lane_value(incl, 63);
    int n_keys = 0;                               // keys placed in cand
    if (M <= SEL_WCAND) {
        int at = incl - c;
        const Pass ow = fresh();
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t oi = ord_at(i, ow);
            if (oi >= res)
                cand[at++] = make_key(oi, flat0 + 64 * i);
        }
        n_keys = M;
    } else {
        // the exact L-th largest value (with repeats), bit by bit
        uint32_t acc = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t t = acc | (1u << bit);
            const Pass ow = fresh();
            int k = 0;
#pragma unroll
            for (int i = 0; i < NL; ++i)
                k += ord_at(i, ow) >= t ? 1 : 0;
            if (wave_sum_i(k) >= L)
                acc = t;
        }
        // everything above it, then the ties at it by increasing index
        c = 0;
        {
            const Pass ow = fresh();
#pragma unroll
            for (int i = 0; i < NL; ++i)
                c += ord_at(i, ow) > acc ? 1 : 0;
        }
        incl = wave_incl_scan(c);
        const int A = lane_value(incl, 63);       // < L
        int at = incl - c;
        const Pass ow = fresh();
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t oi = ord_at(i, ow);
            if (oi > acc)
                cand[at++] = make_key(oi, flat0 + 64 * i);
        }
        int taken = 0;
        const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (A + taken < L) {                  // wave-uniform: stop once L are placed
                const uint32_t oi = ord_at(i, ow);
                const bool tie = oi == acc;
                const uint64_t bal = __ballot(tie);
                const int rank = taken + __popcll(bal & below);
                if (tie && A + rank < L)
                    cand[A + rank] = make_key(oi, flat0 + 64 * i);
                taken += __popcll(bal);
            }
        }
        n_keys = L;
    }
    __builtin_amdgcn_wave_barrier();              // this wave's LDS writes precede its reads
    // rank by counting; the L best land in the row's list in order
    uint64_t mine[SEL_WCAND / 64];
    int rk[SEL_WCAND / 64];
#pragma unroll
    for (int k = 0; k < SEL_WCAND / 64; ++k) {
        mine[k] = lane + 64 * k < n_keys ? cand[lane + 64 * k] : 0;
        rk[k] = 0;
    }
    for (int j = 0; j < n_keys; ++j) {
        const uint64_t cj = cand[j];
#pragma unroll
        for (int k = 0; k < SEL_WCAND / 64; ++k)
            rk[k] += cj > mine[k] ? 1 : 0;
    }
#pragma unroll
    for (int k = 0; k < SEL_WCAND / 64; ++k)
        if (lane + 64 * k < n_keys && rk[k] < L)
            list[rk[k]] = mine[k];
    if (lane < L && lane >= n_keys)               // fewer candidates than L: pad
        list[lane] = 0;
}

__global__ __launch_bounds__(SEL_REQ_THREADS) void select_request(const SelParams p)
{
    constexpr int NT = SEL_REQ_THREADS, NW = NT / 64;
    constexpr int WROWS = 32;                           // rows per wave and chunk
    constexpr int CHUNK = WROWS * NW;
    constexpr int RPL = 64 / (SEL_LIST / 2);            // rows per wave-wide 16-byte load
    constexpr int LOADS = WROWS / RPL;
    __shared__ uint32_t hist3[3 * 256];
    __shared__ uint64_t red64a[2 * NW], red64b[2 * NW];
    __shared__ int redi[NW], wsum[NW];
    __shared__ int cnt_lds[NT];
    __shared__ uint64_t xch2[2 * NT];
    __shared__ uint64_t surv_lds[SEL_SURV_LDS];
    __shared__ int n_sel, n_ovf;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    // offsets clamped to the tables' sizes: inconsistent ones give wrong
    // results, never accesses outside the buffers
    auto clamp = [](int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); };
    const int r0 = clamp(p.row_offset_old[b], 0, p.R_old);
    const int W = clamp(p.row_offset_old[b + 1], r0, p.R_old) - r0;
    const int k0 = clamp(p.row_offset_new[b], 0, p.R_new);
    const int K = clamp(p.row_offset_new[b + 1], k0, p.R_new) - k0;
    if (K <= 0)
        return;
    int k_row = K < p.V ? K : p.V;
    k_row = k_row < p.K_max ? k_row : p.K_max;
    const int L = k_row < SEL_LIST ? k_row : SEL_LIST;
    // Head keys per row behind the bound: all SEL_HEAD when the rows' lists
    // fit one chunk (their heads are then read from registers), else 6 (the
    // heads are loaded and each costs an LDS atomic in the bound's first
    // pass; fewer of them loosen the bound a little).  Measured: 4 x 900
    // beams 58.0 -> 55.5 us with 6 (60.7 with 4: too many survivors), 8 x
    // 128 beams 27.2 with 8 against 27.6 with 6.
    const int head_cap = W <= CHUNK ? SEL_HEAD : SEL_HEAD_FAR;
    const int head = L < head_cap ? L : head_cap;
    const int K_eff = K < p.K_max ? K : p.K_max;      // keys that can be produced
    const uint64_t *lists = p.ws_list + (int64_t)r0 * SEL_LIST;
    uint64_t *surv = p.ws_surv + (int64_t)r0 * p.K_max;
    int32_t *ovf_rows = p.ws_ovf + r0;
    if (tid < 256)
        hist3[tid] = 0;
    if (tid == 0)
        n_ovf = 0;
    __syncthreads();
    int hb = 0;

    // Lists of a chunk of CHUNK rows: wave wv reads rows wv*WROWS .. of the
    // chunk with 16-byte lanes (keys 2kp, 2kp+1 of row g of each load), RPL
    // rows per load.  The first chunk stays in registers for steps 1 and 2.
    const int g = lane / (SEL_LIST / 2), kp = lane % (SEL_LIST / 2);
    uint64_t ka[LOADS], kb[LOADS];
    auto load_chunk = [&](int base, int rows_here) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int rl = wv * WROWS + i * RPL + g;
            ka[i] = kb[i] = 0;
            if (rl < rows_here && 2 * kp < L) {
                const uint4 v = *reinterpret_cast<const uint4 *>(
                    lists + (int64_t)(base + rl) * SEL_LIST + 2 * kp);
                ka[i] = ((uint64_t)v.y << 32) | v.x;
                kb[i] = ((uint64_t)v.w << 32) | v.z;
            }
        }
    };
    load_chunk(0, W < CHUNK ? W : CHUNK);

    // 1. Lower bound tau of the K-th best candidate: the K-th best among the
    //    first `head` keys of every row (distinct candidates).  Without K
    //    head keys there is no bound.
    uint64_t tau = 0;
    const int n_head = W * head;
    if (W > 0 && n_head >= K_eff) {
        // heads: from the chunk in registers when it holds every row, else
        // loaded into SEL_HEAD_REG registers per thread, else streamed
        auto head_key = [&](int i) { return lists[(int64_t)(i / head) * SEL_LIST + i % head]; };
        const int mode = W <= CHUNK ? 0 : (n_head <= SEL_HEAD_REG * NT ? 1 : 2);
        uint64_t hk[SEL_HEAD_REG];
        if (mode == 1) {
#pragma unroll
            for (int j = 0; j < SEL_HEAD_REG; ++j) {
                const int i = tid + NT * j;
                hk[j] = i < n_head ? head_key(i) : 0;
            }
        }
        auto visit = [&](auto f) {
            if (mode == 0) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    if (wv * WROWS + i * RPL + g < W) {
                        if (2 * kp < head)
                            f(ka[i]);
                        if (2 * kp + 1 < head)
                            f(kb[i]);
                    }
                }
            } else if (mode == 1) {
#pragma unroll
                for (int j = 0; j < SEL_HEAD_REG; ++j)
                    if (tid + NT * j < n_head)
                        f(hk[j]);
            } else {
                for (int i = tid; i < n_head; i += NT)
                    f(head_key(i));
            }
        };
        // the K_eff-th best head key, exactly, by radix select over the
        // keys where they sit (registers or memory); the K_eff selected
        // keys are >= pf, so pf bounds the request's K_eff-th best
        // candidate from below.  (One LDS histogram pass per 8-bit digit;
        // measured much cheaper than a bit-by-bit ballot search of each
        // wave's share, and exact, so fewer candidates survive the cut.
        // A first pass over equal-width value bins instead of the exponent
        // digit was measured no faster: the first pass costs its LDS
        // atomics, about one key per clock per compute unit, however the
        // keys spread.)
        uint64_t kmax = 0, kmin = ~0ull;
        visit([&](uint64_t key) {
            kmax = key > kmax ? key : kmax;
            kmin = key < kmin ? key : kmin;
        });
        block_minmax<NT>(kmax, kmin, red64a);
        uint64_t pf, mk;
        radix_kth<NT>(K_eff, kmax, kmin, visit, hist3, hb, pf, mk);
        tau = pf;
    }
    tau = tau > 1 ? tau : 1;                        // every real key is >= 1; 0 pads

    // 2. Survivors: each row's list entries >= tau (a prefix: the lists are
    //    sorted); a row's count is the popcount of its lanes in two ballots.
    //    A row whose whole list clears tau while it has more candidates is
    //    selected again below.
    int N = 0;
    for (int base = 0; base < W; base += CHUNK) {
        const int rows_here = W - base < CHUNK ? W - base : CHUNK;
        if (base > 0)
            load_chunk(base, rows_here);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int rl = wv * WROWS + i * RPL + g;
            const bool in = rl < rows_here;
            const uint64_t ba = __ballot(in && 2 * kp < L && ka[i] >= tau);
            const uint64_t bb = __ballot(in && 2 * kp + 1 < L && kb[i] >= tau);
            const int sh = (SEL_LIST / 2) * g;
            const uint64_t gm = (1ull << (SEL_LIST / 2)) - 1ull;
            const int c = __popcll((ba >> sh) & gm) + __popcll((bb >> sh) & gm);
            if (kp == 0 && in) {
                // the whole list clears tau and the row has more candidates
                const bool ovf = c == L && L < k_row && p.ws_n[r0 + base + rl] > L;
                cnt_lds[rl] = ovf ? 0 : c;
                if (ovf)
                    ovf_rows[atomicAdd(&n_ovf, 1)] = base + rl;
            }
        }
        __syncthreads();
        int tot;
        const int incl = block_incl_scan<NT>(tid < rows_here ? cnt_lds[tid] : 0, wsum, tot);
        __syncthreads();                            // every count read
        if (tid < rows_here)
            cnt_lds[tid] = incl;                    // end of the row's survivors
        __syncthreads();
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int rl = wv * WROWS + i * RPL + g;
            if (rl < rows_here) {
                const int end = cnt_lds[rl];
                const int c = end - (rl ? cnt_lds[rl - 1] : 0);
                const int at = N + end - c + 2 * kp;
                if (2 * kp < c) {
                    surv[at] = ka[i];
                    if (at < SEL_SURV_LDS)
                        surv_lds[at] = ka[i];
                }
                if (2 * kp + 1 < c) {
                    surv[at + 1] = kb[i];
                    if (at + 1 < SEL_SURV_LDS)
                        surv_lds[at + 1] = kb[i];
                }
            }
        }
        N += tot;
        __syncthreads();                            // cnt_lds and wsum reused
    }
    const int n_over = n_ovf;

    // 3. Rows selected again from their logits: every key >= tau competes,
    //    the row's k_row best of them are appended.
    for (int j = 0; j < n_over; ++j) {
        const int w = ovf_rows[j];
        const int r = r0 + w;
        const float off_w = p.ws_off[r];
        const float *row = p.logits + (int64_t)r * p.V;
        const int n = p.ws_n[r], e0 = p.ws_e0[r];
        const bool trie = p.node_ptr != nullptr;
        const uint32_t flat0 = (uint32_t)w * (uint32_t)p.V + (uint32_t)tid;
        uint32_t o[SEL_REQ_NV];
        uint64_t kmax = 0, kmin = ~0ull;
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < SEL_REQ_NV; ++i) {
            const int v = tid + NT * i;
            int t = v;
            if (trie && v < n)
                t = p.edge_tok[e0 + v];
            const float xv = (v < n && t >= 0 && t < p.V) ? row[t] : -__builtin_huge_valf();
            o[i] = v < n ? ord_f32(off_w + xv) : 0;
            const uint64_t key = make_key(o[i], flat0 + NT * i);
            if (v < n && key >= tau) {
                kmax = key > kmax ? key : kmax;
                kmin = key < kmin ? key : kmin;
                ++cnt;
            }
        }
        const int M = block_sum<NT>(cnt, redi);
        block_minmax<NT>(kmax, kmin, red64b);
        const int take = k_row < M ? k_row : M;     // M >= L >= 1: the list's keys
        uint64_t pf, mk;
        auto visit = [&](auto f) {
#pragma unroll
            for (int i = 0; i < SEL_REQ_NV; ++i) {
                const uint64_t key = make_key(o[i], flat0 + NT * i);
                if (tid + NT * i < n && key >= tau)
                    f(key);
            }
        };
        radix_kth<NT>(take, kmax, kmin, visit, hist3, hb, pf, mk);
        if (tid == 0)
            n_sel = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SEL_REQ_NV; ++i) {
            const uint64_t key = make_key(o[i], flat0 + NT * i);
            const bool sel = tid + NT * i < n && key >= tau && (key & mk) >= pf;
            const int at = wave_append(sel, &n_sel);
            if (sel && at < take)
                surv[N + at] = key;
        }
        __syncthreads();                            // n_sel, redi and red64b reused
        N += take;
    }

    // 4. The K_eff best survivors, sorted, decoded and written.  Up to NT
    //    survivors are sorted as they are; more are first cut to the K_eff
    //    best by a radix select.
    const bool from_lds = n_over == 0 && N <= SEL_SURV_LDS;
    const uint64_t *sv = from_lds ? surv_lds : surv;
    const int take = K_eff < N ? K_eff : N;
    uint64_t key = 0;
    int ns = 1;
    if (N <= NT) {
        key = tid < N ? sv[tid] : 0;
        ns = pow2_at_least(N > 0 ? N : 1);
    } else {
        uint64_t pf = 0, mk = 0;
        const bool in_reg = N <= SEL_SURV_REG * NT;
        uint64_t sk[SEL_SURV_REG];
        uint64_t kmax = 0, kmin = ~0ull;
        if (in_reg) {
#pragma unroll
            for (int j = 0; j < SEL_SURV_REG; ++j) {
                const int i = tid + NT * j;
                sk[j] = i < N ? sv[i] : 0;
                if (i < N) {
                    kmax = sk[j] > kmax ? sk[j] : kmax;
                    kmin = sk[j] < kmin ? sk[j] : kmin;
                }
            }
        } else {
            for (int i = tid; i < N; i += NT) {
                const uint64_t k2 = sv[i];
                kmax = k2 > kmax ? k2 : kmax;
                kmin = k2 < kmin ? k2 : kmin;
            }
        }
        block_minmax<NT>(kmax, kmin, red64a);
        radix_kth<NT>(
            take, kmax, kmin,
            [&](auto f) {
                if (in_reg) {
#pragma unroll
                    for (int j = 0; j < SEL_SURV_REG; ++j)
                        if (tid + NT * j < N)
                            f(sk[j]);
                } else {
                    for (int i = tid; i < N; i += NT)
                        f(sv[i]);
                }
            },
            hist3, hb, pf, mk);
        if (tid == 0)
            n_sel = 0;
        __syncthreads();
        if (in_reg) {
#pragma unroll
            for (int j = 0; j < SEL_SURV_REG; ++j) {
                const bool sel = tid + NT * j < N && (sk[j] & mk) >= pf;
                const int at = wave_append(sel, &n_sel);
                if (sel && at < take)
                    xch2[at] = sk[j];
            }
        } else {
            for (int base = 0; base < N; base += NT) {
                const int i = base + tid;
                const uint64_t k2 = i < N ? sv[i] : 0;
                const bool sel = i < N && (k2 & mk) >= pf;
                const int at = wave_append(sel, &n_sel);
                if (sel && at < take)
                    xch2[at] = k2;
            }
        }
        __syncthreads();
        key = tid < take ? xch2[tid] : 0;           // take <= K_max <= NT
        ns = pow2_at_least(take);
    }
    __syncthreads();                                // xch2 is the sort's exchange
    key = block_sort_desc<NT>(key, ns, xch2);
    const bool trie = p.node_ptr != nullptr;
    if (tid < K) {
        if (tid < take) {
            const uint32_t flat = ~(uint32_t)key;
            const int w = (int)(flat / (uint32_t)p.V), v = (int)(flat % (uint32_t)p.V);
            p.score_new[k0 + tid] = unord_f32((uint32_t)(key >> 32));
            p.parent[k0 + tid] = w;
            if (trie) {
                const int e = p.ws_e0[r0 + w] + v;
                p.token[k0 + tid] = p.edge_tok[e];
                p.node_new[k0 + tid] = p.edge_child[e];
            } else {
                p.token[k0 + tid] = v;
            }
        } else {
            p.score_new[k0 + tid] = -__builtin_huge_valf();
            p.parent[k0 + tid] = -1;
            p.token[k0 + tid] = -1;
            if (trie)
                p.node_new[k0 + tid] = -1;
        }
    }
    for (int i = tid + NT; i < K; i += NT) {        // kept beyond K_max: padding
        p.score_new[k0 + i] = -__builtin_huge_valf();
        p.parent[k0 + i] = -1;
        p.token[k0 + i] = -1;
        if (trie)
            p.node_new[k0 + i] = -1;
    }
}

hipError_t launch_beam_select(const SelParams &p, hipStream_t s)
{
    if (p.R_old > 0) {
        // one wave per row up to 64 * 16 candidates (short rows: latency of
        // the dependent loads dominates), else one workgroup per row (long
        // rows: a wave holding 64 * 32 or more keys runs at low occupancy)
        const int n = p.node_ptr ? p.max_fanout : p.V;
        const dim3 gw((p.R_old + 3) / 4), g(p.R_old), t(SEL_ROW_THREADS), t2(2 * SEL_ROW_THREADS);
        if (p.node_ptr) {
            if (n <= 64 * 4)
                hipLaunchKernelGGL((select_rows_wave<4, true>), gw, t, 0, s, p);
            else if (n <= 64 * 16)
                hipLaunchKernelGGL((select_rows_wave<16, true>), gw, t, 0, s, p);
            else if (n <= 32 * SEL_ROW_THREADS)
                hipLaunchKernelGGL((select_rows<32, SEL_ROW_THREADS, true>), g, t, 0, s, p);
            else
                hipLaunchKernelGGL((select_rows<32, 2 * SEL_ROW_THREADS, true>), g, t2, 0, s, p);
        } else if (n <= 64 * 4) {
            hipLaunchKernelGGL((select_rows_wave<4, false>), gw, t, 0, s, p);
        } else if (n <= 64 * 16) {
            hipLaunchKernelGGL((select_rows_wave<16, false>), gw, t, 0, s, p);
        } else if (n <= 32 * SEL_ROW_THREADS) {
            hipLaunchKernelGGL((select_rows<32, SEL_ROW_THREADS, false>), g, t, 0, s, p);
        } else {
            hipLaunchKernelGGL((select_rows<32, 2 * SEL_ROW_THREADS, false>), g, t2, 0, s, p);
        }
    }
    if (p.B > 0)
        hipLaunchKernelGGL(select_request, dim3(p.B), dim3(SEL_REQ_THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace gr
