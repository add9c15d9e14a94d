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
//  1. select_rows: one 256-thread workgroup per beam row holds the row's
//     logits in registers, reduces its max and log-sum-exp, and selects the
//     row's K best keys (K = beams its request keeps) with a radix select over
//     8-bit digits (LDS histograms, one wave finding the digit), then sorts
//     them with a bitonic network in LDS and writes them to the workspace.
//  2. select_request: one 1024-thread workgroup per request.  The K-th best
//     of the rows' best keys bounds the K-th best candidate from below (when
//     the request has at least K rows); each row's sorted list is cut where it
//     falls below that bound (binary search: the early termination), the
//     survivors are gathered, and the exact K best are selected among them,
//     sorted, decoded and written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gr_attn_internal.h"

namespace gr {

constexpr int SEL_ROW_THREADS = 256;
constexpr int SEL_REQ_THREADS = 1024;
constexpr int SEL_HEAD = 8;            // keys per row that set the pruning bound

__device__ __forceinline__ uint32_t ord_f32(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float value, uint32_t flat)
{
    return ((uint64_t)ord_f32(value) << 32) | (uint32_t)~flat;
}

// Largest and smallest 64-bit key over the block (every thread passes its
// own; threads with no key pass kmax = 0, kmin = ~0).
template <int NT>
__device__ void block_minmax(uint64_t &kmax, uint64_t &kmin, uint64_t *red)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t a = __shfl_xor(kmax, off), c = __shfl_xor(kmin, off);
        kmax = a > kmax ? a : kmax;
        kmin = c < kmin ? c : kmin;
    }
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
    __syncthreads();
}

// Threshold of the k-th largest of n distinct keys lying in [kmin, kmax], as
// (prefix, mask): the k largest keys are exactly those with (key & mask) >=
// prefix.  The bits kmin and kmax share are shared by every key and decided
// at once; the rest are resolved 8 bits per pass from the top (LDS histogram,
// one wave finding the digit where the count from the top reaches k), and
// the passes stop once every key of the chosen bin is needed.  visit(f)
// calls f(key) for each key the calling thread owns.  Requires 1 <= k <= n;
// all NT threads call it.
template <int NT, class Visit>
__device__ void radix_kth(int k, uint64_t kmax, uint64_t kmin, Visit visit, uint32_t *hist,
                          int *st, uint64_t &prefix_out, uint64_t &mask_out)
{
    const int tid = threadIdx.x;
    const uint64_t diff = kmax ^ kmin;
    const int common = diff ? __clzll(diff) : 64;
    uint64_t mask = common == 0 ? 0 : (~0ull << (64 - common));
    uint64_t prefix = kmax & mask;
    int hi = 64 - common;                    // bits [0, hi) still undecided
    int remaining = k;
    while (hi > 0) {
        const int lo = hi > 8 ? hi - 8 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        for (int i = tid; i < 256; i += NT)
            hist[i] = 0;
        __syncthreads();
        visit([&](uint64_t key) {
            if ((key & mask) == prefix)
                atomicAdd(&hist[(uint32_t)(key >> lo) & dmask], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 4l .. 4l+3; suffix sums over lanes find the
            // bin where the count from the top reaches `remaining`
            const int lane = tid;
            uint32_t b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = hist[4 * lane + j];
            const uint32_t own = b[0] + b[1] + b[2] + b[3];
            uint32_t suf = own;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t t = __shfl_down(suf, off);
                if (lane + off < 64)
                    suf += t;
            }
            const uint32_t above_lane = suf - own;
            if (suf >= (uint32_t)remaining && above_lane < (uint32_t)remaining) {
                uint32_t cum = above_lane;
                for (int j = 3; j >= 0; --j) {
                    if (cum + b[j] >= (uint32_t)remaining || j == 0) {
                        st[0] = 4 * lane + j;
                        st[1] = (int)cum;
                        st[2] = (int)b[j];
                        break;
                    }
                    cum += b[j];
                }
            }
        }
        __syncthreads();
        const int d = st[0], above = st[1], cnt = st[2];
        __syncthreads();                          // st and hist are reused next pass
        prefix |= (uint64_t)d << lo;
        mask |= (uint64_t)dmask << lo;
        remaining -= above;
        hi = lo;
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
        base = __shfl(base, leader);
    }
    return base + __popcll(ballot & ((1ull << lane) - 1ull));
}

// Bitonic sort of buf[0 .. ns) into descending order (ns a power of two).
template <int NT>
__device__ void block_sort_desc(uint64_t *buf, int ns)
{
    const int tid = threadIdx.x;
    for (int k = 2; k <= ns; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < ns; i += NT) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t a = buf[i], c = buf[ixj];
                    const bool desc = (i & k) == 0;
                    if (desc ? (a < c) : (a > c)) {
                        buf[i] = c;
                        buf[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
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

// One beam row per workgroup; NV logits per thread (V <= NV * 256).
template <int NV>
__global__ __launch_bounds__(SEL_ROW_THREADS) void select_rows(const SelParams p)
{
    __shared__ uint32_t hist[256];
    __shared__ int st[4];
    __shared__ float red[SEL_ROW_THREADS / 64];
    __shared__ uint64_t red64[2 * SEL_ROW_THREADS / 64];
    __shared__ uint64_t buf[SEL_MAX_K];
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

    const float *row = p.logits + (int64_t)r * p.V;
    float x[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = tid + SEL_ROW_THREADS * i;
        x[i] = v < p.V ? row[v] : -__builtin_huge_valf();
    }
    // max and log-sum-exp over the row
    float m = x[0];
#pragma unroll
    for (int i = 1; i < NV; ++i)
        m = __builtin_fmaxf(m, x[i]);
    for (int off = 32; off > 0; off >>= 1)
        m = __builtin_fmaxf(m, __shfl_xor(m, off));
    if (lane == 0)
        red[wv] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < SEL_ROW_THREADS / 64; ++w)
        m = __builtin_fmaxf(m, red[w]);
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
        s += __expf(x[i] - m);
    for (int off = 32; off > 0; off >>= 1)
        s += __shfl_xor(s, off);
    if (lane == 0)
        red[wv] = s;
    __syncthreads();
    s = 0.f;
#pragma unroll
    for (int w = 0; w < SEL_ROW_THREADS / 64; ++w)
        s += red[w];
    const float off_w = p.score_old[r] - (m + __logf(s));

    // the candidates' ordered value bits replace the logits
    uint32_t o[NV];
    uint64_t kmax = 0, kmin = ~0ull;
    const uint32_t flat0 = (uint32_t)wl * (uint32_t)p.V + (uint32_t)tid;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        o[i] = ord_f32(off_w + x[i]);
        if (tid + SEL_ROW_THREADS * i < p.V) {
            const uint64_t key = ((uint64_t)o[i] << 32) | ~(flat0 + SEL_ROW_THREADS * i);
            kmax = key > kmax ? key : kmax;
            kmin = key < kmin ? key : kmin;
        }
    }
    block_minmax<SEL_ROW_THREADS>(kmax, kmin, red64);
    auto visit = [&](auto f) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (tid + SEL_ROW_THREADS * i < p.V)
                f(((uint64_t)o[i] << 32) | ~(flat0 + SEL_ROW_THREADS * i));
    };
    uint64_t prefix, mask;
    radix_kth<SEL_ROW_THREADS>(k_row, kmax, kmin, visit, hist, st, prefix, mask);

    // gather the k_row selected keys, sort them, write the row's list
    if (tid == 0)
        n_buf = 0;
    const int ns = pow2_at_least(k_row);
    for (int i = tid; i < ns; i += SEL_ROW_THREADS)
        buf[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const uint64_t key = ((uint64_t)o[i] << 32) | ~(flat0 + SEL_ROW_THREADS * i);
        const bool take = tid + SEL_ROW_THREADS * i < p.V && (key & mask) >= prefix;
        const int at = wave_append(take, &n_buf);
        if (take && at < k_row)
            buf[at] = key;
    }
    __syncthreads();
    block_sort_desc<SEL_ROW_THREADS>(buf, ns);
    uint64_t *dst = p.ws_rows + (int64_t)r * p.K_max;
    for (int i = tid; i < k_row; i += SEL_ROW_THREADS)
        dst[i] = buf[i];
}

__global__ __launch_bounds__(SEL_REQ_THREADS) void select_request(const SelParams p)
{
    constexpr int NW = SEL_REQ_THREADS / 64;
    __shared__ uint32_t hist[256];
    __shared__ int st[4];
    __shared__ uint64_t red64[2 * NW];
    __shared__ int scan[SEL_REQ_THREADS];
    __shared__ uint64_t buf[SEL_MAX_K];
    __shared__ int n_buf;
    __shared__ int carry;

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
    const int K_eff = K < p.K_max ? K : p.K_max;      // keys that can be produced
    const uint64_t *rows = p.ws_rows + (int64_t)r0 * p.K_max;

    // Lower bound of the K-th best candidate: the K-th best among the first
    // `head` keys of every row (distinct candidates).  Keys below it cannot
    // be among the K best; without K head keys there is no bound.
    const int head = k_row < SEL_HEAD ? k_row : SEL_HEAD;
    const int n_head = W * head;
    uint64_t tau = 0;
    if (W > 0 && n_head >= K_eff) {
        auto head_key = [&](int i) { return rows[(int64_t)(i / head) * p.K_max + i % head]; };
        uint64_t kmax = 0, kmin = ~0ull;
        for (int i = tid; i < n_head; i += SEL_REQ_THREADS) {
            const uint64_t key = head_key(i);
            kmax = key > kmax ? key : kmax;
            kmin = key < kmin ? key : kmin;
        }
        block_minmax<SEL_REQ_THREADS>(kmax, kmin, red64);
        uint64_t pf, mk;
        radix_kth<SEL_REQ_THREADS>(
            K_eff, kmax, kmin,
            [&](auto f) {
                for (int i = tid; i < n_head; i += SEL_REQ_THREADS)
                    f(head_key(i));
            },
            hist, st, pf, mk);
        // the K_eff selected head keys are all >= pf
        tau = pf;
    }
    // survivors: the prefix of each row's sorted list at or above tau (the
    // early termination of that row's candidates)
    uint64_t *surv = p.ws_surv + (int64_t)r0 * p.K_max;
    if (tid == 0)
        carry = 0;
    __syncthreads();
    for (int base = 0; base < W; base += SEL_REQ_THREADS) {
        const int w = base + tid;
        int c = 0;
        if (w < W) {
            const uint64_t *lst = rows + (int64_t)w * p.K_max;
            int lo = 0, hi = k_row;              // count of keys >= tau in a descending list
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (lst[mid] >= tau)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            c = lo;
        }
        scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < SEL_REQ_THREADS; off <<= 1) {   // inclusive scan
            const int t = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += t;
            __syncthreads();
        }
        // one wave copies one row's survivors
        const int n_rows = W - base < SEL_REQ_THREADS ? W - base : SEL_REQ_THREADS;
        for (int j = wv; j < n_rows; j += NW) {
            const int end = scan[j];
            const int cj = end - (j ? scan[j - 1] : 0);
            const uint64_t *lst = rows + (int64_t)(base + j) * p.K_max;
            uint64_t *out = surv + carry + end - cj;
            for (int i = lane; i < cj; i += 64)
                out[i] = lst[i];
        }
        __syncthreads();
        if (tid == SEL_REQ_THREADS - 1)
            carry += scan[tid];
        __syncthreads();
    }
    const int N = carry;

    // exact best K_eff among the N survivors, sorted
    const int take = K_eff < N ? K_eff : N;
    uint64_t pf = 0, mk = 0;
    if (take > 0) {
        uint64_t kmax = 0, kmin = ~0ull;
        for (int i = tid; i < N; i += SEL_REQ_THREADS) {
            const uint64_t key = surv[i];
            kmax = key > kmax ? key : kmax;
            kmin = key < kmin ? key : kmin;
        }
        block_minmax<SEL_REQ_THREADS>(kmax, kmin, red64);
        radix_kth<SEL_REQ_THREADS>(
            take, kmax, kmin,
            [&](auto f) {
                for (int i = tid; i < N; i += SEL_REQ_THREADS)
                    f(surv[i]);
            },
            hist, st, pf, mk);
    }
    if (tid == 0)
        n_buf = 0;
    const int ns = pow2_at_least(take > 0 ? take : 1);
    for (int i = tid; i < ns; i += SEL_REQ_THREADS)
        buf[i] = 0;
    __syncthreads();
    if (take > 0) {
        for (int base = 0; base < N; base += SEL_REQ_THREADS) {
            const int i = base + tid;
            const uint64_t key = i < N ? surv[i] : 0;
            const bool sel = i < N && (key & mk) >= pf;
            const int at = wave_append(sel, &n_buf);
            if (sel && at < take)
                buf[at] = key;
        }
    }
    __syncthreads();
    block_sort_desc<SEL_REQ_THREADS>(buf, ns);
    for (int i = tid; i < K; i += SEL_REQ_THREADS) {
        if (i < take) {
            const uint64_t key = buf[i];
            const uint32_t flat = ~(uint32_t)key;
            p.score_new[k0 + i] = unord_f32((uint32_t)(key >> 32));
            p.parent[k0 + i] = (int)(flat / (uint32_t)p.V);
            p.token[k0 + i] = (int)(flat % (uint32_t)p.V);
        } else {
            p.score_new[k0 + i] = -__builtin_huge_valf();
            p.parent[k0 + i] = -1;
            p.token[k0 + i] = -1;
        }
    }
}

hipError_t launch_beam_select(const SelParams &p, hipStream_t s)
{
    if (p.R_old > 0) {
        if (p.V <= 16 * SEL_ROW_THREADS)
            hipLaunchKernelGGL(select_rows<16>, dim3(p.R_old), dim3(SEL_ROW_THREADS), 0, s, p);
        else if (p.V <= 32 * SEL_ROW_THREADS)
            hipLaunchKernelGGL(select_rows<32>, dim3(p.R_old), dim3(SEL_ROW_THREADS), 0, s, p);
        else
            hipLaunchKernelGGL(select_rows<64>, dim3(p.R_old), dim3(SEL_ROW_THREADS), 0, s, p);
    }
    if (p.B > 0)
        hipLaunchKernelGGL(select_request, dim3(p.B), dim3(SEL_REQ_THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace gr
