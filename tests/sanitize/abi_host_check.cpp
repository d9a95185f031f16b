// abi_host_check.cpp -- CPU check of the library's host-side logic under
// AddressSanitizer and UndefinedBehaviorSanitizer (built with g++ by
// tests/test_sanitizers.py, together with hqq_abi.cpp and hqq_stream.cpp).
//
// The kernel launchers and the few HIP runtime calls of those files are
// replaced by recording stubs, so every entry point runs its argument checks,
// the shrink certificate, the planning of batched launches (tensor tables,
// depth, workgroup counts) and the chunking of streamed weights without a GPU.
// Exit status 0: every check passed.
#include "hqq.h"
#include "hqq_internal.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

static int g_fail = 0;
#define CHECK(c)                                                                    \
    do {                                                                            \
        if (!(c)) {                                                                 \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);   \
            ++g_fail;                                                               \
        }                                                                           \
    } while (0)

// ---------------------------------------------------------------- stubs
static std::vector<hqq::SolveArgs> g_solve;
static std::vector<int> g_seg;   // the mapping of each launch

// linear layer routes: a log of (kind, weight's Y or W_hat, ...) in call order
struct LinCall {
    char kind;   // 'd' dequantize, 'g' GEMM, 'f' fused launch
    const void *a, *b;
    int64_t M, N, K;
    size_t ws;
};
static std::vector<LinCall> g_lin;
static bool g_gemm_ok = true;

namespace hqq {
hipError_t launch_solve(int nbits, int gs, int axis, bool bf16, int seg, const SolveArgs &a, hipStream_t)
{
    if ((seg == kMapSeg && !seg_format(nbits, gs, axis, bf16)) ||
        (seg == kMapSeg16 && !seg16_format(nbits, gs, axis, bf16)))
        return hipErrorInvalidValue;
    g_solve.push_back(a);
    g_seg.push_back(seg);
    return hipSuccess;
}
hipError_t launch_dequantize(int nbits, int axis, const CodecArgs &a, hipStream_t)
{
    g_lin.push_back({'d', a.packed_in, a.W_hat, a.rows, nbits, axis, (size_t)a.n_words});
    return hipSuccess;
}
hipError_t launch_pack(int, int, const CodecArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_unpack(int, int, const CodecArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_linear(int, bool, LinearBatch &b, hipStream_t)
{
    g_lin.push_back({'f', b.Y[0], nullptr, b.a.M, b.count, b.a.K, 0});
    return hipSuccess;
}
bool gemm_available(int64_t, int64_t, int64_t, bool, size_t) { return g_gemm_ok; }
hipError_t gemm_xwt(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, bool, void *ws,
                    size_t ws_bytes, hipStream_t)
{
    g_lin.push_back({'g', Y, W, M, N, K, ws_bytes});
    (void)X;
    (void)ws;
    return hipSuccess;
}
hipError_t launch_quantize_meta(MetaBatch &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_dequantize_meta(MetaBatch &, int, hipStream_t) { return hipSuccess; }
}  // namespace hqq

struct Copy {
    char *dst;
    const char *src;
    size_t bytes;
};
static std::vector<Copy> g_copies;
static int g_events = 0, g_events_live = 0;
static std::vector<int> g_event_log;   // +1 record, +2 wait, per call order

hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned)
{
    ++g_events;
    ++g_events_live;
    *e = reinterpret_cast<hipEvent_t>((intptr_t)(0x1000 + g_events));
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t)
{
    --g_events_live;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t)
{
    g_event_log.push_back(1);
    return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned)
{
    g_event_log.push_back(2);
    return hipSuccess;
}
static const void *g_symbol = nullptr;   // the static staging array's (host) address
static int g_symbol_lookups = 0;
hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void **p, const void *symbol)
{
    ++g_symbol_lookups;
    g_symbol = symbol;
    *p = const_cast<void *>(symbol);
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t)
{
    g_copies.push_back(Copy{(char *)dst, (const char *)src, bytes});
    return hipSuccess;
}

// ---------------------------------------------------------------- helpers
static void *aligned(size_t bytes)
{
    void *p = nullptr;
    if (posix_memalign(&p, 256, bytes < 256 ? 256 : bytes) != 0)
        abort();
    return p;
}

// Every launch's tensor table describes the given tensors in order, with
// workgroup ranges that tile the grid.
static void check_launches(const std::vector<hqq_tensor> &ts, int nbits, int gs, int axis)
{
    const int C = hqq::codes_per_word(nbits);
    const int64_t lb = hqq::lcm_c(gs, C);
    size_t k = 0;
    const char *force = getenv("HQQ_SOLVE_MAPPING");
    for (size_t li = 0; li < g_solve.size(); ++li) {
        const hqq::SolveArgs &a = g_solve[li];
        const int seg = g_seg[li];
        CHECK(a.n >= 1 && a.n <= hqq::kMaxBatch);
        CHECK(a.depth >= 1 && a.depth <= hqq::kMaxDepth);
        // several lanes per group: only where the format allows it, always
        // when forced (16 per lane: where the format has it), never when one
        // lane per item is forced
        const bool ok8 = hqq::seg_format(nbits, gs, axis, false), ok16 = hqq::seg16_format(nbits, gs, axis, false);
        if (!ok8)
            CHECK(seg == hqq::kMapLane);
        else if (force && strcmp(force, "seg") == 0)
            CHECK(seg == hqq::kMapSeg);
        else if (force && strcmp(force, "seg16") == 0)
            CHECK(seg == (ok16 ? hqq::kMapSeg16 : hqq::kMapLane));
        else if (force && strcmp(force, "lane") == 0)
            CHECK(seg == hqq::kMapLane);
        const int64_t per = (seg != hqq::kMapLane ? (int64_t)(hqq::kSolveBlock / 64) * hqq::seg_groups_per_wave(gs, seg)
                                                  : (int64_t)hqq::kSolveBlock) * a.depth;
        int64_t items = 0;
        for (int j = 0; j < a.n; ++j)
            items += a.t[j].n_items;
        if (!force && ok8)
            CHECK(seg == (items >= hqq::seg_max_items(nbits) ? hqq::kMapLane
                          : ok16 && nbits >= 4             ? hqq::kMapSeg16
                                                           : hqq::kMapSeg));
        int64_t b = 0;
        for (int j = 0; j < a.n; ++j, ++k) {
            CHECK(k < ts.size());
            if (k >= ts.size())
                return;
            const hqq::SolveTensor &t = a.t[j];
            CHECK(t.W == ts[k].W && t.packed == ts[k].packed && t.scale == ts[k].scale && t.zero == ts[k].zero);
            CHECK(t.rows == ts[k].rows && t.cols == ts[k].cols);
            const int64_t L = axis == 1 ? t.cols : t.rows;
            CHECK(t.nblk == (L + lb - 1) / lb);
            CHECK(t.n_items == t.nblk * (axis == 1 ? t.rows : t.cols));
            CHECK(a.block0[j] == b);
            b += (t.n_items + per - 1) / per;
        }
        CHECK(a.blocks == b);
    }
    CHECK(k == ts.size());
}

static void test_validation()
{
    uint16_t *W = (uint16_t *)aligned(1 << 16);
    uint32_t *pk = (uint32_t *)aligned(1 << 16);
    float *sc = (float *)aligned(1 << 16), *ze = (float *)aligned(1 << 16);
    CHECK(hqq_quantize(W, 64, 128, 5, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_NBITS);
    CHECK(hqq_quantize(W, 64, 128, 4, 64, 2, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_AXIS);
    CHECK(hqq_quantize(W, 64, 100, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_GROUP);
    CHECK(hqq_quantize(W, 64, 128, 4, 48, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_GROUP);
    CHECK(hqq_quantize(W, 0, 128, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_SHAPE);
    CHECK(hqq_quantize(W, 64, (int64_t)1 << 32, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) ==
          HQQ_EINVAL_SHAPE);
    CHECK(hqq_quantize(nullptr, 64, 128, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_PTR);
    CHECK(hqq_quantize(W + 1, 64, 128, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_PTR);
    CHECK(hqq_quantize(W, 64, 128, 4, 64, 1, -1, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_PARAM);
    CHECK(hqq_quantize(W, 64, 128, 4, 64, 1, 20, NAN, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_PARAM);
    CHECK(hqq_quantize(W, 64, 128, 4, 64, 1, 20, 0.7f, 0.f, 1.01f, pk, sc, ze, nullptr) == HQQ_EINVAL_PARAM);
    CHECK(hqq_quantize(W, 64, 128, 4, 64, 1, 20, 0.7f, 10.f, INFINITY, pk, sc, ze, nullptr) == HQQ_EINVAL_PARAM);
    CHECK(hqq_quantize_batch_ex(nullptr, 0, 7, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, nullptr) == HQQ_EINVAL_DTYPE);
    CHECK(hqq_quantize_batch(nullptr, -1, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, nullptr) == HQQ_EINVAL_SHAPE);
    CHECK(hqq_quantize_batch(nullptr, 3, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, nullptr) == HQQ_EINVAL_PTR);
    CHECK(hqq_dequantize(pk, sc, ze, 64, 128, 3, 64, 1, W, nullptr) == HQQ_OK);
    CHECK(hqq_dequantize_ex(pk, sc, ze, 64, 128, 3, 64, 1, 9, W, nullptr) == HQQ_EINVAL_DTYPE);
    CHECK(hqq_pack((const uint8_t *)W, 64, 128, 2, 16, 0, pk, nullptr) == HQQ_OK);
    CHECK(hqq_unpack(pk, 64, 128, 2, 16, 0, (uint8_t *)W + 4, nullptr) == HQQ_EINVAL_PTR);
    CHECK(hqq_linear(W, 1, 128, pk, sc, ze, 64, 3, 64, W, nullptr) == HQQ_EINVAL_NBITS);
    CHECK(hqq_linear(W, 1, 100, pk, sc, ze, 64, 4, 64, W, nullptr) == HQQ_EINVAL_SHAPE);
    CHECK(hqq_quantize_meta((const float *)sc, 0, 128, (uint8_t *)W, sc, ze, nullptr) == HQQ_EINVAL_SHAPE);
    CHECK(hqq_quantize_meta((const float *)sc, 100, 0, (uint8_t *)W, sc, ze, nullptr) == HQQ_EINVAL_GROUP);
    CHECK(hqq_packed_words(10, 33, 3, 1) == 10 * 4);
    CHECK(hqq_packed_words(33, 10, 3, 0) == 4 * 10);
    CHECK(hqq_packed_words(10, 10, 5, 0) == HQQ_EINVAL_NBITS);
    for (int st = 0; st >= -9; --st)
        CHECK(hqq_strerror(st) != nullptr && strlen(hqq_strerror(st)) > 0);
    free(W);
    free(pk);
    free(sc);
    free(ze);
}

// The certificate the launches carry: 0 < thr < every iteration's shrink
// threshold beta_k^(-1/(2-p)) (W_e = 0 below it), thr_m = 2048 thr; none
// (0) where the exponent 1 - (p - 1) is not positive.
static void test_certificate()
{
    uint16_t *W = (uint16_t *)aligned(64 * 128 * 2);
    uint32_t *pk = (uint32_t *)aligned(1 << 14);
    float *sc = (float *)aligned(1 << 14), *ze = (float *)aligned(1 << 14);
    const float ps[] = {0.7f, 0.3f, 1.0f, 1.5f, 2.5f};
    const float b0s[] = {10.f, 1000.f, 0.1f};
    for (float p : ps)
        for (float b0 : b0s) {
            g_solve.clear();
            g_seg.clear();
            CHECK(hqq_quantize(W, 64, 128, 4, 64, 1, 20, p, b0, 1.01f, pk, sc, ze, nullptr) == HQQ_OK);
            CHECK(g_solve.size() == 1);
            if (g_solve.empty())
                continue;
            const hqq::SolveArgs &a = g_solve[0];
            CHECK(a.pm1 == p - 1.0f && a.beta0 == b0 && a.kappa == 1.01f && a.iters == 20);
            const double ex = 1.0 - (double)(p - 1.0f);
            if (ex > 0.01) {
                CHECK(a.thr > 0.0f && a.thr_m == a.thr * 2048.0f);
                float b = b0;
                for (int k = 0; k < 20; ++k) {
                    const double tau = pow((double)b, -1.0 / ex);
                    CHECK((double)a.thr < tau);
                    b = b * 1.01f;
                }
            } else {
                CHECK(a.thr == 0.0f && a.thr_m == 0.0f);
            }
        }
    g_solve.clear();
    g_seg.clear();
    CHECK(hqq_quantize(W, 64, 128, 4, 64, 1, 0, 0.7f, 10.f, 1.01f, pk, sc, ze, nullptr) == HQQ_OK);
    CHECK(g_solve.size() == 1 && g_solve[0].thr == 0.0f);
    free(W);
    free(pk);
    free(sc);
    free(ze);
}

// Batched launches: 100 tensors of mixed shapes, every format and axis, small
// and large (the automatic mapping changes at seg_max_items groups per
// launch), with the mapping automatic or forced each way.
static void test_batches()
{
    const int fmts[][3] = {{4, 64, 1}, {3, 64, 0}, {2, 16, 1}, {1, 16, 0}, {8, 128, 1}, {4, 32, 1}, {2, 64, 1}, {1, 32, 1}, {1, 64, 1}};
    for (const char *force : {(const char *)nullptr, "lane", "seg", "seg16"}) {
        if (force)
            setenv("HQQ_SOLVE_MAPPING", force, 1);
        else
            unsetenv("HQQ_SOLVE_MAPPING");
        unsigned seed = 12345;
        auto rnd = [&](int m) { seed = seed * 1103515245u + 12345u; return (int)((seed >> 8) % (unsigned)m); };
        for (const auto &f : fmts)
            for (int64_t scale : {(int64_t)1, (int64_t)40}) {
                std::vector<hqq_tensor> ts;
                std::vector<void *> mem;
                for (int i = 0; i < 100; ++i) {
                    const int64_t lines = 1 + rnd(3000) * scale, other = (int64_t)f[1] * (1 + rnd(40));
                    const int64_t rows = f[2] == 1 ? lines : other, cols = f[2] == 1 ? other : lines;
                    // pointers are only recorded, never dereferenced: one small
                    // aligned block stands in for every buffer
                    void *p = aligned(256);
                    mem.push_back(p);
                    ts.push_back(hqq_tensor{(const uint16_t *)p, rows, cols, (uint32_t *)p, (float *)p, (float *)p});
                }
                g_solve.clear();
                g_seg.clear();
                CHECK(hqq_quantize_batch(ts.data(), (int)ts.size(), f[0], f[1], f[2], 20, 0.7f, 10.f, 1.01f,
                                         nullptr) == HQQ_OK);
                CHECK(g_solve.size() >= 3);
                // launches as even as kMaxBatch allows: 100 tensors -> 34, 33, 33
                // (more launches only where a launch's workgroups would overflow)
                for (const hqq::SolveArgs &a : g_solve)
                    CHECK(a.n <= 34);
                check_launches(ts, f[0], f[1], f[2]);
                for (void *p : mem)
                    free(p);
            }
    }
    unsetenv("HQQ_SOLVE_MAPPING");
}

// Streamed solve: the copies cover every row of every tensor exactly once,
// land inside the staging half of their chunk, and each chunk's launch reads
// what was copied; events are balanced.
static void test_streamed()
{
    const int fmts[][3] = {{4, 64, 1}, {3, 64, 0}, {2, 16, 0}, {8, 32, 1}};
    unsigned seed = 777;
    auto rnd = [&](int m) { seed = seed * 1103515245u + 12345u; return (int)((seed >> 8) % (unsigned)m); };
    for (const auto &f : fmts)
        for (int trial = 0; trial < 4; ++trial) {
            const int n = 1 + rnd(8);
            std::vector<hqq_host_tensor> ts;
            std::vector<uint16_t *> host;
            int64_t unit_rows = f[2] == 1 ? 16 : hqq::lcm_c(f[1], hqq::codes_per_word(f[0])) * 16;
            int64_t max_row_bytes = 0;
            for (int i = 0; i < n; ++i) {
                const int64_t rows = f[2] == 1 ? 1 + rnd(700) : (int64_t)hqq::lcm_c(f[1], hqq::codes_per_word(f[0])) * (1 + rnd(6));
                const int64_t cols = f[2] == 1 ? (int64_t)f[1] * (1 + rnd(12)) : 8 * (1 + rnd(40));
                uint16_t *h = (uint16_t *)aligned(rows * cols * 2);
                for (int64_t k = 0; k < rows * cols; ++k)
                    h[k] = (uint16_t)k;
                host.push_back(h);
                max_row_bytes = max_row_bytes > cols * 2 ? max_row_bytes : cols * 2;
                ts.push_back(hqq_host_tensor{h, rows, cols, (uint32_t *)aligned(256), (float *)aligned(256),
                                             (float *)aligned(256)});
            }
            const int64_t staging_bytes = 2 * (unit_rows * max_row_bytes + 256 * (1 + rnd(64)));
            char *staging = (char *)aligned(staging_bytes);
            g_copies.clear();
            g_solve.clear();
            g_seg.clear();
            g_event_log.clear();
            g_events = 0;
            g_events_live = 0;
            const int st = hqq_quantize_streamed(ts.data(), n, f[0], f[1], f[2], 20, 0.7f, 10.f, 1.01f, staging,
                                                 staging_bytes, (void *)1, (void *)2);
            CHECK(st == HQQ_OK);
            CHECK(g_events_live == 0);
            const int64_t half = (staging_bytes / 2) / 256 * 256;
            // every copy inside one half of the staging buffer
            for (const Copy &c : g_copies) {
                const int64_t off = c.dst - staging;
                CHECK(off >= 0 && off + (int64_t)c.bytes <= 2 * half);
                CHECK((off < half) == (off + (int64_t)c.bytes <= half));
            }
            // every row of every tensor copied exactly once
            for (int i = 0; i < n; ++i) {
                const int64_t total = ts[i].rows * ts[i].cols * 2;
                std::vector<int> seen((size_t)total, 0);
                for (const Copy &c : g_copies) {
                    const char *b = (const char *)host[i];
                    if (c.src >= b && c.src < b + total) {
                        CHECK(c.src + c.bytes <= b + total);
                        for (size_t k = 0; k < c.bytes; ++k)
                            ++seen[(size_t)(c.src - b) + k];
                    }
                }
                bool once = true;
                for (int v : seen)
                    once = once && v == 1;
                CHECK(once);
            }
            // each launched row block reads staging memory inside one half
            for (const hqq::SolveArgs &a : g_solve)
                for (int j = 0; j < a.n; ++j) {
                    const int64_t off = (const char *)a.t[j].W - staging;
                    const int64_t bytes = a.t[j].rows * a.t[j].cols * 2;
                    CHECK(off >= 0 && off + bytes <= 2 * half);
                }
            for (uint16_t *h : host)
                free(h);
            for (auto &t : ts) {
                free(t.packed);
                free(t.scale);
                free(t.zero);
            }
            free(staging);
        }
    // a staging buffer too small for one block unit (here one 2 KiB row in a
    // 512-byte half) is rejected up front
    static uint16_t h[64 * 1024];
    hqq_host_tensor t{h, 64, 1024, (uint32_t *)aligned(256), (float *)aligned(256), (float *)aligned(256)};
    char *small = (char *)aligned(1024);
    g_copies.clear();
    CHECK(hqq_quantize_streamed(&t, 1, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, small, 1024, nullptr, nullptr) ==
          HQQ_EINVAL_SHAPE);
    CHECK(g_copies.empty());
    free(t.packed);
    free(t.scale);
    free(t.zero);
    free(small);
}

// The no-allocation streamed entry point: the static array's address is
// looked up once and its events created once (five, never released); the
// copies of two calls in a row (the second smaller) land inside one half of
// the array and cover every row once; a row block larger than half the array
// is refused with HQQ_ESCRATCH before anything is enqueued.
static void test_streamed_static()
{
    g_events = 0;
    g_events_live = 0;
    g_symbol_lookups = 0;
    const int64_t half = (HQQ_STATIC_STAGING_BYTES / 2) / 256 * 256;
    for (int call = 0; call < 2; ++call) {
        const int64_t rows = call == 0 ? 5000 : 700, cols = 4096;
        uint16_t *h = (uint16_t *)aligned(rows * cols * 2);
        hqq_host_tensor t{h, rows, cols, (uint32_t *)aligned(256), (float *)aligned(256), (float *)aligned(256)};
        g_copies.clear();
        g_solve.clear();
        g_seg.clear();
        CHECK(hqq_quantize_streamed_static(&t, 1, 4, 64, 1, 20, 0.7f, 10.f, 1.01f, (void *)1, (void *)2) ==
              HQQ_OK);
        CHECK(g_symbol_lookups == 1 && g_events == 5 && g_events_live == 5);
        int64_t total = 0;
        for (const Copy &c : g_copies) {
            const int64_t off = c.dst - (const char *)g_symbol;
            CHECK(off >= 0 && off + (int64_t)c.bytes <= 2 * half);
            CHECK((off < half) == (off + (int64_t)c.bytes <= half));
            total += (int64_t)c.bytes;
        }
        CHECK(total == rows * cols * 2);
        CHECK(!g_solve.empty());
        free(h);
        free(t.packed);
        free(t.scale);
        free(t.zero);
    }
    // a 3-bit axis-0 row block (320 rows) of 65536 columns is 40 MiB
    uint16_t dummy[8];
    hqq_host_tensor big{dummy, 320, 65536, (uint32_t *)aligned(256), (float *)aligned(256), (float *)aligned(256)};
    g_copies.clear();
    g_solve.clear();
    CHECK(hqq_quantize_streamed_static(&big, 1, 3, 64, 0, 20, 0.7f, 10.f, 1.01f, (void *)1, (void *)2) ==
          HQQ_ESCRATCH);
    CHECK(g_copies.empty() && g_solve.empty() && g_events == 5);
    CHECK(strcmp(hqq_strerror(HQQ_ESCRATCH), "unknown status") != 0);
    free(big.packed);
    free(big.scale);
    free(big.zero);
}

// The linear layer's route: dequantize + GEMM per weight where the workspace
// holds the largest W_hat and M >= 2048 (or HQQ_LINEAR_PATH=gemm), the fused
// launch otherwise (also when hipBLASLt has no algorithm); W_hat at the
// workspace's start, the GEMM's workspace after it (256-byte rounded).  A
// batch of three weights here, so the one-weight threshold does not apply.
static void test_linear_routes()
{
    const int64_t K = 4096;
    const int64_t Ns[3] = {4096, 11008, 1024};
    uint16_t *X = (uint16_t *)aligned(256);
    char *work = (char *)aligned(1 << 20);
    std::vector<hqq_linear_weight> w;
    std::vector<void *> mem{X, work};
    for (int i = 0; i < 3; ++i) {
        void *p = aligned(256);
        mem.push_back(p);
        w.push_back(hqq_linear_weight{(const uint32_t *)p, (const float *)p, (const float *)p, Ns[i],
                                      (uint16_t *)aligned(256)});
        mem.push_back(w.back().Y);
    }
    const int64_t what = (11008 * K * 2 + 255) / 256 * 256;
    const int64_t big = what + (32 << 20);   // bytes claimed (the stubs never touch them)
    struct Case {
        const char *env;
        int64_t M, bytes;
        bool gemm_ok;
        bool want_gemm;
    } cases[] = {
        {nullptr, 2048, big, true, true},    {nullptr, 2047, big, true, false},
        {nullptr, 1024, big, true, false},   {nullptr, 2048, what, true, true},
        {nullptr, 2048, what - 256, true, false}, {nullptr, 2048, 0, true, false},
        {"fused", 2048, big, true, false},   {"gemm", 1, big, true, true},
        {"gemm", 64, what - 1, true, false}, {nullptr, 4096, big, false, false},
    };
    for (const Case &c : cases) {
        if (c.env)
            setenv("HQQ_LINEAR_PATH", c.env, 1);
        else
            unsetenv("HQQ_LINEAR_PATH");
        g_gemm_ok = c.gemm_ok;
        g_lin.clear();
        CHECK(hqq_linear_batch_ws(X, c.M, K, w.data(), 3, 4, 64, HQQ_DTYPE_FP16, c.bytes ? work : nullptr, c.bytes,
                                  nullptr) == HQQ_OK);
        if (c.want_gemm) {
            CHECK(g_lin.size() == 6);
            for (size_t i = 0; i + 1 < g_lin.size() && i < 6; i += 2) {
                const int j = (int)(i / 2);
                CHECK(g_lin[i].kind == 'd' && g_lin[i].a == w[j].packed && g_lin[i].b == work &&
                      g_lin[i].M == Ns[j] && g_lin[i].N == 4 && g_lin[i].K == 1 &&
                      (int64_t)g_lin[i].ws == hqq_packed_words(Ns[j], K, 4, 1));
                CHECK(g_lin[i + 1].kind == 'g' && g_lin[i + 1].a == w[j].Y && g_lin[i + 1].b == work &&
                      g_lin[i + 1].M == c.M && g_lin[i + 1].N == Ns[j] && g_lin[i + 1].K == K &&
                      (int64_t)g_lin[i + 1].ws == c.bytes - what);
            }
        } else {
            CHECK(g_lin.size() == 1 && g_lin[0].kind == 'f' && g_lin[0].N == 3);
        }
    }
    unsetenv("HQQ_LINEAR_PATH");
    g_gemm_ok = true;
    for (void *p : mem)
        free(p);
}

int main()
{
    test_linear_routes();
    test_validation();
    test_certificate();
    test_batches();
    test_streamed();
    test_streamed_static();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("abi host checks passed\n");
    return 0;
}
