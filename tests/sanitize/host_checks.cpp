// Sanitizer test program for the host-side C code: argument validation, the work
// decomposition and workspace layout of gr_attn_api.cpp (through the C ABI,
// with the launchers stubbed: they check each planned launch against the
// caller's buffers), and the C oracle on small random inputs.  Built with
// g++ -fsanitize=address,undefined and run on the CPU; prints SANITIZE_OK.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "gr_attn.h"
#include "stub_state.h"

extern "C" int oracle_decode_attn(int B, int R, int Hq, int Hkv, int D, int T_cap,
                                  int64_t ctx_cap, int64_t beam_cap, double scale,
                                  const uint16_t *q, const uint16_t *ctx_k,
                                  const uint16_t *ctx_v, const int32_t *ctx_len,
                                  const uint16_t *beam_k, const uint16_t *beam_v,
                                  const int32_t *beam_path, const int32_t *beam_len,
                                  const int32_t *row_offset, const int32_t *rows, int n_rows,
                                  double *out, double *lse, int n_threads);
extern "C" int oracle_beam_step(int B, int Hkv, int D, int T_cap, int W_cap, int64_t beam_cap,
                                const int32_t *row_offset_old, const int32_t *row_offset_new,
                                const int32_t *parent, const int32_t *path_old,
                                const int32_t *beam_len_old, const uint16_t *new_k,
                                const uint16_t *new_v, int32_t *path_new,
                                int32_t *beam_len_new, uint16_t *beam_k, uint16_t *beam_v);

static std::mt19937_64 rng(20261203);
static int pick(const std::vector<int> &v) { return v[rng() % v.size()]; }
static int64_t pick64(const std::vector<int64_t> &v) { return v[rng() % v.size()]; }

#define CHECK(c)                                                                       \
    do {                                                                               \
        if (!(c)) {                                                                    \
            std::fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #c); \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

// Fake device addresses: 256-byte aligned, never dereferenced (the stubs
// launch nothing).
static void *fake(uintptr_t k) { return reinterpret_cast<void *>((k + 1) << 20); }

static bool known_status(int st) { return st <= 0 && st >= -7; }

static int fuzz_decode_attn(int iters)
{
    long ok = 0;
    for (int it = 0; it < iters; ++it) {
        gr_decode_attn_dims d{};
        d.B = pick({-1, 0, 1, 2, 3, 8, 16, 33});
        d.Hkv = pick({-1, 0, 1, 2, 4, 8});
        d.Hq = d.Hkv * pick({1, 2, 3, 4, 5, 8, 9}) + (rng() % 16 == 0 ? 1 : 0);
        d.D = pick({0, 32, 64, 96, 128, 256});
        d.W_max = pick({-1, 0, 1, 4, 37, 128, 900, 3600});
        d.R = pick({-1, 0, 1, 10}) + (d.B > 0 && d.W_max > 0 ? (int)(rng() % (d.B * d.W_max + 1)) : 0);
        d.T_cap = pick({-1, 0, 1, 3, 5, 17});
        d.ctx_cap = pick64({-1, 0, 1, 31, 64, 513, 1024, 2048, 4096, 1LL << 31, 1LL << 40});
        d.beam_cap = pick64({-1, 0, 1, 16, 4500, 1LL << 33});
        d.scale = (float)pick({0, 0, 1, -1, 2});
        if (rng() % 32 == 0)
            d.scale = NAN;
        if (rng() % 32 == 0)
            d.scale = INFINITY;
        d.reserved = rng() % 64 == 0;
        const int f = rng() % 8;
        d.flags = f < 5 ? 0
                  : f == 5 ? GR_TILING(pick({1, 2, 3, 4, 8}), pick({1, 2, 4}), pick({1, 2, 3, 8}))
                  : f == 6 ? GR_TILING(pick({0, 4, 300}), pick({0, 1}), pick({0, 1, 9}))
                           : (int32_t)rng();
        const size_t need = gr_decode_attn_workspace_bytes(&d);
        const int wsm = rng() % 5;
        d.workspace = wsm == 0 ? nullptr : (char *)fake(7) + (wsm == 4 ? 128 : 0);
        d.workspace_bytes = wsm == 1 && need > 0 ? need - 1 : need + (wsm == 3 ? 4096 : 0);
        g_call = StubCall{d.workspace, (size_t)d.workspace_bytes, d.W_max};
        void *P = fake(1);
        const int32_t *I = static_cast<const int32_t *>(fake(2));
        int st = gr_decode_attn(&d, I, P, P, P, I, P, P, I, I, fake(3), (float *)fake(4), nullptr);
        CHECK(known_status(st));
        if (st == GR_OK)
            ++ok;
        if (st == GR_OK && need > 0)
            CHECK(d.workspace && d.workspace_bytes >= need);
        // the no-alloc variant: the split goes to the library's scratch
        {
            const StubCall saved = g_call;
            st = gr_decode_attn_noalloc(&d, I, P, P, P, I, P, P, I, I, fake(3), (float *)fake(4),
                                        nullptr);
            CHECK(known_status(st));
            g_call = saved;
        }
        // paged: the same dims through a page table
        gr_paged_ctx c{P, P, I, pick({0, 8, 16, 32, 48}), pick({0, 1, 64, 300}),
                       pick64({0, 1, 1000, 1LL << 32})};
        st = gr_decode_attn_paged(&d, &c, I, P, I, P, P, I, I, fake(3), (float *)fake(4), nullptr);
        CHECK(known_status(st));
        st = gr_decode_attn_generic(&d, I, P, P, P, I, P, P, I, I, fake(3), (float *)fake(4),
                                    nullptr);
        CHECK(known_status(st));
        st = gr_check_metadata(&d, I, I, I, I, (int32_t *)fake(5), nullptr);
        CHECK(known_status(st));
        // misaligned and missing pointers are refused before any launch
        st = gr_decode_attn(&d, I, (char *)P + 2, P, P, I, P, P, I, I, fake(3),
                            (float *)fake(4), nullptr);
        CHECK(st != GR_OK || d.R == 0 || d.B == 0 || d.W_max == 0);
    }
    std::printf("decode_attn: %d calls, %ld accepted\n", iters, ok);
    CHECK(ok > iters / 50);
    return 0;
}

static int fuzz_step_and_select(int iters)
{
    for (int it = 0; it < iters; ++it) {
        gr_beam_step_dims s{};
        s.B = pick({-1, 0, 1, 4});
        s.R_old = pick({-1, 0, 5, 900});
        s.R_new = pick({-1, 0, 7, 900});
        s.Hkv = pick({0, 1, 8});
        s.D = pick({64, 96, 128});
        s.T_cap = pick({-1, 0, 4});
        s.W_cap = pick({-1, 0, 900});
        s.beam_cap = pick64({-1, 0, 3601});
        s.reserved = rng() % 64 == 0;
        void *P = fake(1);
        int32_t *I = static_cast<int32_t *>(fake(2));
        int st = gr_beam_step(&s, I, I, I, I, I, P, P, (int32_t *)fake(8), (int32_t *)fake(9),
                              P, P, nullptr, nullptr);
        CHECK(known_status(st));
        st = gr_beam_step(&s, I, I, I, I, I, P, P, I, I, P, P, nullptr, nullptr);
        CHECK(known_status(st));       // overlapping tables are refused when both are used

        gr_beam_select_dims d{};
        d.B = pick({-1, 0, 1, 4, 8});
        d.R_old = pick({-1, 0, 1, 900, 3600});
        d.R_new = pick({-1, 0, 1, 900, 3600});
        d.V = pick({0, 1, 300, 8192, 16384, 16385});
        d.K_max = pick({0, 1, 24, 900, 1024, 1025});
        d.reserved = rng() % 64 == 0;
        const size_t need = gr_beam_select_workspace_bytes(&d);
        const int wsm = rng() % 4;
        void *ws = wsm == 0 ? nullptr : (char *)fake(11) + (wsm == 3 ? 8 : 0);
        const size_t wsb = wsm == 1 && need > 0 ? need - 1 : need;
        g_call = StubCall{ws, wsb, 0};
        float *F = static_cast<float *>(fake(12));
        st = gr_beam_select(&d, I, I, F, F, F, I, I, ws, wsb, nullptr);
        CHECK(known_status(st));
        gr_sid_trie t{I, I, I, pick({0, 1, 1000}), pick({-1, 0, 5000}), pick({0, 1, 122, 20000}),
                      0};
        st = gr_beam_select_trie(&d, &t, I, I, F, F, I, F, I, I, I, ws, wsb, nullptr);
        CHECK(known_status(st));
    }
    for (int c = -10; c <= 2; ++c)
        CHECK(gr_status_str(c) != nullptr && std::strlen(gr_status_str(c)) > 0);
    std::printf("beam_step / beam_select: %d calls each\n", iters);
    return 0;
}

// The oracle on small random inputs: every buffer exactly as large as its
// layout says, so an index outside it is a sanitizer report.
static int oracle_cases(int n)
{
    std::uniform_int_distribution<int> bits(0, 0xffff);
    for (int it = 0; it < n; ++it) {
        const int B = 1 + rng() % 3, Hkv = 1 + rng() % 2, G = 1 + rng() % 3, Hq = Hkv * G;
        const int D = 4 * (1 + rng() % 4), T_cap = rng() % 4;
        const int64_t ctx_cap = rng() % 9, W_cap = 1 + rng() % 3;
        const int64_t beam_cap = T_cap * W_cap + 1;
        std::vector<int32_t> ro(B + 1, 0), ctx_len(B), beam_len(B);
        for (int b = 0; b < B; ++b) {
            ro[b + 1] = ro[b] + (int)(rng() % (W_cap + 1));
            ctx_len[b] = (int)(rng() % (ctx_cap + 1));
            beam_len[b] = T_cap ? (int)(rng() % (T_cap + 1)) : 0;
        }
        const int R = ro[B];
        auto rnd = [&](size_t m) {
            std::vector<uint16_t> v(m);
            for (auto &x : v)
                x = (uint16_t)((bits(rng) & 0x3fff) | 0x3c00);   // finite, moderate
            return v;
        };
        auto q = rnd((size_t)R * Hq * D), ck = rnd((size_t)B * ctx_cap * Hkv * D);
        auto cv = rnd(ck.size()), bk = rnd((size_t)B * beam_cap * Hkv * D), bv = rnd(bk.size());
        std::vector<int32_t> path((size_t)R * T_cap);
        for (auto &x : path)
            x = (int32_t)(rng() % beam_cap);
        std::vector<double> out((size_t)R * Hq * D), lse((size_t)R * Hq);
        // (with no rows the output vectors are empty and their data() may be
        // NULL, which the oracle refuses; there is nothing to evaluate then)
        const int st = R == 0 ? 0 : oracle_decode_attn(B, R, Hq, Hkv, D, T_cap, ctx_cap, beam_cap, 0.5,
                                          q.data(), ck.data(), cv.data(), ctx_len.data(),
                                          bk.data(), bv.data(), path.data(), beam_len.data(),
                                          ro.data(), nullptr, R, out.data(), lse.data(),
                                          1 + (int)(rng() % 3));
        if (st != 0)
            std::fprintf(stderr, "oracle status %d (B=%d R=%d Hq=%d D=%d T_cap=%d)\n", st, B, R,
                         Hq, D, T_cap);
        CHECK(st == 0);
        // one step of the per-beam state on the same pools
        std::vector<int32_t> ro_new(B + 1, 0);
        for (int b = 0; b < B; ++b)
            ro_new[b + 1] = ro_new[b] + (int)(rng() % (W_cap + 1));
        const int R_new = ro_new[B];
        std::vector<int32_t> parent(R_new), path_new((size_t)R_new * T_cap, -1), len_new(B);
        for (int b = 0; b < B; ++b) {
            const int w_old = ro[b + 1] - ro[b];
            for (int r = ro_new[b]; r < ro_new[b + 1]; ++r)
                parent[r] = w_old > 0 ? (int)(rng() % w_old) : (int)(rng() % 3) - 1;
        }
        auto nk = rnd((size_t)R_new * Hkv * D), nv = rnd(nk.size());
        const int sk = oracle_beam_step(B, Hkv, D, T_cap, (int)W_cap, beam_cap, ro.data(),
                                        ro_new.data(), parent.data(), path.data(),
                                        beam_len.data(), nk.data(), nv.data(), path_new.data(),
                                        len_new.data(), bk.data(), bv.data());
        CHECK(sk >= 0 && sk <= R_new);
    }
    std::printf("oracle: %d random cases\n", n);
    return 0;
}

int main()
{
    if (fuzz_decode_attn(200000) || fuzz_step_and_select(50000) || oracle_cases(3000))
        return 1;
    std::printf("launches checked: %ld\nSANITIZE_OK\n", g_launches);
    return 0;
}
