// Host-side argument checks of every entry point of include/spec_verify.h,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// code (tests/test_abi_sanitized.py builds and runs it).  Every call here
// returns from its checks before anything is enqueued: the pointers are a
// fake, 16-byte aligned address that nothing dereferences, so no GPU is
// needed.  The workspace-size calls are also swept over the largest sizes
// the checks admit, where an overflowing product in the size arithmetic
// would be undefined behaviour the sanitizer stops on.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "spec_verify.h"

namespace {

int failures = 0;
int checks = 0;

void expect(int got, int want, const char *what, int line) {
    ++checks;
    if (got != want) {
        ++failures;
        fprintf(stderr, "line %d: %s returned %d (%s), expected %d (%s)\n", line, what, got,
                spec_verify_status_string(got), want, spec_verify_status_string(want));
    }
}

void expect_true(bool ok, const char *what, int line) {
    ++checks;
    if (!ok) {
        ++failures;
        fprintf(stderr, "line %d: %s is false\n", line, what);
    }
}

#define EXPECT(call, want) expect((call), (want), #call, __LINE__)
#define EXPECT_TRUE(cond) expect_true((cond), #cond, __LINE__)

char *const A = reinterpret_cast<char *>(uintptr_t(1) << 20);  // fake aligned address
float *const F = reinterpret_cast<float *>(A);
int32_t *const I = reinterpret_cast<int32_t *>(A);
const float kInf = INFINITY;
const float kNan = NAN;

struct Attn {
    const void *q = A, *k = A, *v = A, *kc = A, *vc = A;
    const int32_t *tau = I;
    void *out = A;
    int dtype = SV_BF16, batch = 1, block = 8, prefix = 32, hq = 4, hkv = 4, d = 64;
    double theta = 1e4;
    float scale = 0.f;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_attn(q, k, v, kc, vc, tau, out, dtype, batch, block, prefix, hq, hkv, d, theta, scale,
                                ws, wb, nullptr);
    }
};

struct Copies {
    const void *q = A, *k = A, *v = A, *kc = A, *vc = A;
    void *out = A;
    int dtype = SV_BF16, batch = 1, block = 32, copies = 9, prefix = 64, hq = 4, hkv = 4, d = 128;
    double theta = 1e6;
    float scale = 0.f;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_attn_copies(q, k, v, kc, vc, out, dtype, batch, block, copies, prefix, hq, hkv, d, theta,
                                       scale, ws, wb, nullptr);
    }
};

struct Paged {
    const void *q = A, *k = A, *v = A, *kp = A, *vp = A;
    const int32_t *table = I, *lens = I, *tau = I;
    void *out = A;
    int dtype = SV_BF16, batch = 2, block = 32, copies = 0, max_prefix = 2048, page = 64, max_pages = 33,
        n_pages = 66, hq = 32, hkv = 8, d = 128;
    double theta = 1e6;
    float scale = 0.f;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_attn_paged(q, k, v, kp, vp, table, lens, tau, out, dtype, batch, block, copies,
                                      max_prefix, page, max_pages, n_pages, hq, hkv, d, theta, scale, ws, wb,
                                      nullptr);
    }
};

struct Accept {
    const float *l = F, *p = F;
    const int32_t *x = I, *tau = I;
    const float *u = F;
    int batch = 2, block = 8, gamma = 8;
    int64_t vocab = 512;
    int32_t *len = I, *tok = I;
    float *alpha = F;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_accept(l, p, x, tau, u, batch, block, gamma, vocab, len, tok, alpha, ws, wb, nullptr);
    }
    int temperature(float T) const {
        return spec_verify_accept_temperature(l, p, x, tau, u, batch, block, gamma, vocab, T, len, tok, alpha, ws,
                                              wb, nullptr);
    }
    int noalloc() const {
        return spec_verify_accept_noalloc(l, p, x, tau, u, batch, block, gamma, vocab, len, tok, alpha, nullptr);
    }
};

struct Coupled {
    const float *l = F, *g = F;
    const int32_t *x = I, *tau = I;
    int batch = 2, block = 8, gamma = 8;
    int64_t vocab = 512;
    float T = 1.f;
    int32_t *len = I, *tok = I, *tt = I;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_accept_coupled(l, g, x, tau, batch, block, gamma, vocab, T, len, tok, tt, ws, wb,
                                          nullptr);
    }
};

struct Route {
    const float *p = F;
    const int32_t *tau = I;
    int batch = 2, block = 8, gamma = 8;
    int64_t vocab = 512;
    int est = SV_ROUTE_ENTROPY;
    double param = 1.0;
    float *kh = F, *ah = F;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_route(p, tau, batch, block, gamma, vocab, est, param, kh, ah, ws, wb, nullptr);
    }
};

struct Tree {
    const float *l = F, *g = F;
    const int32_t *par = I, *pos = I, *tok = I, *tp = I;
    int batch = 4, nodes = 9;
    int64_t vocab = 151936;
    float T = 1.f;
    int32_t *len = I, *path = I, *cp = I, *ct = I, *tt = I;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_tree(l, g, par, pos, tok, tp, batch, nodes, vocab, T, len, path, cp, ct, tt, ws, wb,
                                nullptr);
    }
};

struct States {
    const float *l = F, *g = F;
    const int32_t *par = I, *st = I;
    int batch = 32, nodes = 9, block = 32;
    int64_t vocab = 151936;
    float T = 1.f, thr = 1.f;
    int32_t *len = I, *path = I, *ns = I, *cm = I;
    float *cf = F;
    void *ws = A;
    size_t wb = size_t(1) << 30;
    int call() const {
        return spec_verify_tree_states(l, g, par, st, batch, nodes, block, vocab, T, thr, len, path, ns, cm, cf, ws,
                                       wb, nullptr);
    }
};

struct Append {
    const void *k = A, *v = A;
    int stride = 64;
    const int32_t *na = I;
    void *kp = A, *vp = A;
    const int32_t *table = I;
    int32_t *lens = I, *status = I;
    int dtype = SV_BF16, batch = 4, page = 64, max_pages = 33, n_pages = 132, hkv = 8, d = 128;
    double theta = 1e6;
    int call() const {
        return spec_verify_kv_append(k, v, stride, na, kp, vp, table, lens, status, dtype, batch, page, max_pages,
                                     n_pages, hkv, d, theta, nullptr);
    }
};

template <class T, class F>
T with(T base, F f) {
    f(base);
    return base;
}

void test_status_strings() {
    EXPECT_TRUE(spec_verify_abi_version() == SPEC_VERIFY_ABI_VERSION);
    for (int s = 0; s >= -8; --s) EXPECT_TRUE(spec_verify_status_string(s) != nullptr);
    EXPECT_TRUE(spec_verify_status_string(-99) != nullptr);
    EXPECT_TRUE(spec_verify_status_string(1 << 30) != nullptr);
}

void test_rope() {
    EXPECT(spec_verify_rope(nullptr, A, A, A, SV_BF16, 1, 8, 4, 4, 64, 32, 1e4, nullptr), SV_E_NULL);
    EXPECT(spec_verify_rope(A, A, A, A, SV_BF16, 1, 8, 4, 4, 64, 32, 0.0, nullptr), SV_E_SHAPE);
    EXPECT(spec_verify_rope(A, A, A, A, SV_BF16, 1, 8, 4, 4, 64, 32, (double)kNan, nullptr), SV_E_SHAPE);
    EXPECT(spec_verify_rope(A, A, A, A, SV_BF16, 1, 8, 4, 4, 80, 32, 1e4, nullptr), SV_E_UNSUPPORTED);
    EXPECT(spec_verify_rope(A, A, A + 2, A, SV_BF16, 1, 8, 4, 4, 64, 32, 1e4, nullptr), SV_E_ALIGN);
    EXPECT(spec_verify_rope(A, A, A, A, SV_BF16, 1 << 30, 64, 4, 4, 64, 32, 1e4, nullptr), SV_E_SHAPE);
}

void test_attn() {
    const Attn a;
    EXPECT(with(a, [](Attn &x) { x.q = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(a, [](Attn &x) { x.kc = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(a, [](Attn &x) { x.d = 96; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(a, [](Attn &x) { x.dtype = 7; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(a, [](Attn &x) { x.hq = 6; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.block = 65; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.block = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.prefix = -1; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.theta = (double)kInf; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.scale = kNan; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.q = A + 8; }).call(), SV_E_ALIGN);
    EXPECT(with(a, [](Attn &x) { x.dtype = SV_F32, x.ws = nullptr; }).call(), SV_E_WORKSPACE);
    EXPECT(with(a, [](Attn &x) { x.dtype = SV_F32, x.wb = 16; }).call(), SV_E_WORKSPACE);
    EXPECT(with(a, [](Attn &x) { x.dtype = SV_F32, x.ws = A + 4; }).call(), SV_E_ALIGN);
    EXPECT(with(a, [](Attn &x) { x.batch = 4, x.prefix = 16384, x.block = 32, x.hq = 32, x.hkv = 8, x.d = 128,
                                 x.ws = nullptr; }).call(),
           SV_E_WORKSPACE);
    // beyond the 32-bit index ranges
    EXPECT(with(a, [](Attn &x) { x.batch = 1 << 24, x.block = 64, x.hq = 64, x.hkv = 8; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Attn &x) { x.prefix = 0x7fffffff; }).call(), SV_E_SHAPE);
}

void test_copies() {
    const Copies c;
    EXPECT(with(c, [](Copies &x) { x.prefix = 2048, x.wb = 0; }).call(), SV_E_WORKSPACE);
    EXPECT(with(c, [](Copies &x) { x.q = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(c, [](Copies &x) { x.kc = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(c, [](Copies &x) { x.dtype = SV_F32; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(c, [](Copies &x) { x.copies = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(c, [](Copies &x) { x.copies = 33; }).call(), SV_E_SHAPE);
    EXPECT(with(c, [](Copies &x) { x.block = 65, x.copies = 2; }).call(), SV_E_SHAPE);
    EXPECT(with(c, [](Copies &x) { x.copies = 0x7fffffff; }).call(), SV_E_SHAPE);
    EXPECT(with(c, [](Copies &x) { x.out = A + 8; }).call(), SV_E_ALIGN);
}

void test_paged() {
    const Paged p;
    EXPECT(with(p, [](Paged &x) { x.dtype = SV_F32; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(p, [](Paged &x) { x.page = 96; }).call(), SV_E_SHAPE);
    EXPECT(with(p, [](Paged &x) { x.max_pages = 31; }).call(), SV_E_SHAPE);
    EXPECT(with(p, [](Paged &x) { x.n_pages = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(p, [](Paged &x) { x.copies = -1; }).call(), SV_E_SHAPE);
    EXPECT(with(p, [](Paged &x) { x.table = nullptr, x.page = 1000; }).call(), SV_E_SHAPE);
    EXPECT(with(p, [](Paged &x) { x.max_pages = 0x7fffffff, x.page = 0x7fffffc0; }).call(), SV_E_SHAPE);
    EXPECT(with(p, [](Paged &x) { x.tau = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(p, [](Paged &x) { x.tau = nullptr, x.copies = 9, x.wb = 0; }).call(), SV_E_WORKSPACE);
    EXPECT(with(p, [](Paged &x) { x.kp = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(p, [](Paged &x) { x.out = A + 4; }).call(), SV_E_ALIGN);
    EXPECT(with(p, [](Paged &x) { x.wb = 0; }).call(), SV_E_WORKSPACE);
}

void test_accept() {
    const Accept a;
    EXPECT(with(a, [](Accept &x) { x.l = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(a, [](Accept &x) { x.len = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(a, [](Accept &x) { x.gamma = 9; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.gamma = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.vocab = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.vocab = INT64_MAX; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.block = 65; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.u = F + 1; }).call(), SV_E_ALIGN);
    EXPECT(with(a, [](Accept &x) { x.ws = nullptr; }).call(), SV_E_WORKSPACE);
    EXPECT(with(a, [](Accept &x) { x.wb = 8; }).call(), SV_E_WORKSPACE);
    EXPECT(with(a, [](Accept &x) { x.batch = 1 << 21, x.block = 64, x.vocab = 4; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.batch = 1 << 14, x.block = 64, x.vocab = 1 << 21; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.batch = 0x7fffffff, x.block = 64; }).call(), SV_E_SHAPE);
    for (float T : {0.f, -1.f, kInf, kNan, 1e-45f}) EXPECT(a.temperature(T), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.ws = nullptr; }).temperature(0.7f), SV_E_WORKSPACE);
    EXPECT(with(a, [](Accept &x) { x.l = nullptr; }).temperature(0.7f), SV_E_NULL);
    // the allocation-free call: the same checks, and sizes beyond its buffer
    // refused before any device is touched
    EXPECT(with(a, [](Accept &x) { x.l = nullptr; }).noalloc(), SV_E_NULL);
    EXPECT(with(a, [](Accept &x) { x.gamma = 9; }).noalloc(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.vocab = (1 << 21) + 1; }).noalloc(), SV_E_SHAPE);
    EXPECT(with(a, [](Accept &x) { x.alpha = F + 2; }).noalloc(), SV_E_ALIGN);
    EXPECT(with(a, [](Accept &x) { x.batch = 1 << 12, x.block = 64, x.gamma = 64, x.vocab = 1 << 14; }).noalloc(),
           SV_E_SCRATCH);
}

void test_coupled() {
    const Coupled c;
    EXPECT(with(c, [](Coupled &x) { x.l = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(c, [](Coupled &x) { x.g = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(c, [](Coupled &x) { x.g = nullptr, x.T = 0.f, x.ws = nullptr; }).call(), SV_E_WORKSPACE);
    for (float T : {-1.f, kInf, kNan, 1e-45f}) EXPECT(with(c, [T](Coupled &x) { x.T = T; }).call(), SV_E_SHAPE);
    EXPECT(with(c, [](Coupled &x) { x.gamma = 9; }).call(), SV_E_SHAPE);
    EXPECT(with(c, [](Coupled &x) { x.g = F + 1; }).call(), SV_E_ALIGN);
    EXPECT(with(c, [](Coupled &x) { x.tt = I + 1; }).call(), SV_E_ALIGN);
    EXPECT(with(c, [](Coupled &x) { x.wb = 4; }).call(), SV_E_WORKSPACE);
    EXPECT(with(c, [](Coupled &x) { x.batch = 1 << 21, x.block = 64, x.vocab = 4; }).call(), SV_E_SHAPE);
}

void test_route() {
    const Route r;
    EXPECT(with(r, [](Route &x) { x.p = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(r, [](Route &x) { x.kh = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(r, [](Route &x) { x.est = 2; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(r, [](Route &x) { x.param = (double)kNan; }).call(), SV_E_SHAPE);
    EXPECT(with(r, [](Route &x) { x.gamma = 9; }).call(), SV_E_SHAPE);
    EXPECT(with(r, [](Route &x) { x.ah = F + 1; }).call(), SV_E_ALIGN);
    EXPECT(with(r, [](Route &x) { x.ws = nullptr; }).call(), SV_E_WORKSPACE);
}

void test_tree() {
    const Tree t;
    EXPECT(with(t, [](Tree &x) { x.nodes = 65; }).call(), SV_E_SHAPE);
    EXPECT(with(t, [](Tree &x) { x.nodes = 0; }).call(), SV_E_SHAPE);
    for (float T : {-1.f, kInf, kNan, 1e-45f}) EXPECT(with(t, [T](Tree &x) { x.T = T; }).call(), SV_E_SHAPE);
    EXPECT(with(t, [](Tree &x) { x.batch = 1 << 21, x.nodes = 64, x.vocab = 4; }).call(), SV_E_SHAPE);
    EXPECT(with(t, [](Tree &x) { x.g = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(t, [](Tree &x) { x.par = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(t, [](Tree &x) { x.l = F + 1; }).call(), SV_E_ALIGN);
    EXPECT(with(t, [](Tree &x) { x.wb = 0; }).call(), SV_E_WORKSPACE);
}

void test_states() {
    const States s;
    const size_t ws = spec_verify_tree_states_workspace_size(32, 9, 32, 151936);
    EXPECT_TRUE(ws >= size_t(32) * 9 * 32 * 24);
    EXPECT(with(s, [](States &x) { x.nodes = 65; }).call(), SV_E_SHAPE);
    EXPECT(with(s, [](States &x) { x.block = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(s, [](States &x) { x.block = 65; }).call(), SV_E_SHAPE);
    for (float T : {-1.f, kNan, kInf, 1e-45f}) EXPECT(with(s, [T](States &x) { x.T = T; }).call(), SV_E_SHAPE);
    EXPECT(with(s, [](States &x) { x.thr = kNan; }).call(), SV_E_SHAPE);
    EXPECT(with(s, [](States &x) { x.batch = (1 << 14) + 1, x.nodes = 64, x.block = 64, x.vocab = 4; }).call(),
           SV_E_SHAPE);
    EXPECT(with(s, [](States &x) { x.batch = 0x7fffffff, x.nodes = 64, x.block = 64; }).call(), SV_E_SHAPE);
    EXPECT(with(s, [](States &x) { x.g = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(s, [](States &x) { x.st = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(s, [](States &x) { x.ns = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(s, [](States &x) { x.l = F + 1; }).call(), SV_E_ALIGN);
    EXPECT(with(s, [](States &x) { x.g = F + 2; }).call(), SV_E_ALIGN);
    EXPECT(with(s, [ws](States &x) { x.wb = ws - 1; }).call(), SV_E_WORKSPACE);
    EXPECT(with(s, [ws](States &x) { x.ws = A + 4, x.wb = ws; }).call(), SV_E_ALIGN);
}

void test_commit_append() {
    EXPECT(spec_verify_check_tau(I, 4, 65, I, nullptr), SV_E_SHAPE);
    EXPECT(spec_verify_check_tau(nullptr, 4, 32, I, nullptr), SV_E_NULL);
    EXPECT(spec_verify_commit(I, I, 4, 32, 33, I, I, I, nullptr), SV_E_SHAPE);
    EXPECT(spec_verify_commit(I, I, 4, 65, 8, I, I, I, nullptr), SV_E_SHAPE);
    EXPECT(spec_verify_commit(I, I, 0x7fffffff, 64, 8, I, I, I, nullptr), SV_E_SHAPE);
    EXPECT(spec_verify_commit(nullptr, I, 4, 32, 8, I, I, I, nullptr), SV_E_NULL);
    const Append a;
    EXPECT(with(a, [](Append &x) { x.dtype = SV_F32; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(a, [](Append &x) { x.d = 96; }).call(), SV_E_UNSUPPORTED);
    EXPECT(with(a, [](Append &x) { x.stride = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Append &x) { x.max_pages = 0; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Append &x) { x.batch = 0x7fffffff, x.hkv = 64; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Append &x) { x.theta = (double)kNan; }).call(), SV_E_SHAPE);
    EXPECT(with(a, [](Append &x) { x.lens = nullptr; }).call(), SV_E_NULL);
    EXPECT(with(a, [](Append &x) { x.kp = A + 2; }).call(), SV_E_ALIGN);
}

// Every workspace-size call over the largest sizes its checks admit, and
// just beyond them.  A signed product that overflows in the size arithmetic
// stops the program under UBSan; every admitted size must come out nonzero
// where the call needs a workspace at all, and every refused one zero.
void test_workspace_extremes() {
    const int big_i[] = {1, 2, 63, 64, 65, 1 << 14, (1 << 14) + 1, 1 << 20, 1 << 26, 0x7fffffff};
    const int64_t vocabs[] = {1, 4, 16383, 16384, 151936, 1 << 21, (1 << 21) + 1, INT64_MAX};
    size_t sink = 0;
    for (int batch : big_i)
        for (int block : {1, 32, 64, 65})
            for (int64_t vocab : vocabs) {
                const bool rows_in = (int64_t)batch * block <= (int64_t(1) << 26) &&
                                     (vocab > (int64_t(1) << 40) ||
                                      (int64_t)batch * block * vocab <= (int64_t(1) << 40));
                const bool in = block <= 64 && vocab <= (1 << 21) && rows_in;
                const size_t a = spec_verify_accept_workspace_size(batch, block, block < 64 ? block : 64, vocab);
                const size_t c = spec_verify_accept_coupled_workspace_size(batch, block, 1, vocab);
                const size_t r = spec_verify_route_workspace_size(batch, block, 1, vocab);
                EXPECT_TRUE((a > 0) == in);
                EXPECT_TRUE((c > 0) == in);
                EXPECT_TRUE((r > 0) == in);
                const size_t t = spec_verify_tree_workspace_size(batch, block, vocab);
                EXPECT_TRUE((t > 0) == in);
                for (int nodes : {1, 9, 64, 65}) {
                    const bool srows = (int64_t)batch * nodes * block <= (int64_t(1) << 26) &&
                                       (int64_t)batch * nodes * block * (vocab < (1 << 22) ? vocab : 1) <=
                                           (int64_t(1) << 40);
                    const bool sin = nodes <= 64 && block <= 64 && vocab <= (1 << 21) && srows;
                    EXPECT_TRUE((spec_verify_tree_states_workspace_size(batch, nodes, block, vocab) > 0) == sin);
                }
                sink += a + c + r + t;
            }
    for (int dtype : {SV_F32, SV_BF16})
        for (int batch : big_i)
            for (int block : {1, 32, 64})
                for (int prefix : {0, 1, 2048, 1 << 20, (1 << 30) - 128, 0x7fffffff})
                    for (int hq : {1, 8, 64, 1 << 20})
                        for (int hkv : {1, 8})
                            for (int d : {64, 128}) {
                                sink += spec_verify_attn_workspace_size(dtype, batch, block, prefix, hq, hkv, d);
                                for (int copies : {1, 9, 32})
                                    sink += spec_verify_attn_copies_workspace_size(dtype, batch, block, copies,
                                                                                   prefix, hq, hkv, d);
                                for (int copies : {0, 9})
                                    sink += spec_verify_attn_paged_workspace_size(dtype, batch, block, copies,
                                                                                  prefix, hq, hkv, d);
                            }
    // the long-prefix workload splits its prompt: a bf16 workspace
    EXPECT_TRUE(spec_verify_attn_workspace_size(SV_BF16, 4, 32, 16384, 32, 8, 128) > 0);
    EXPECT_TRUE(spec_verify_attn_workspace_size(SV_BF16, 32, 32, 2048, 32, 8, 128) == 0);
    printf("workspace sweep: %zu bytes summed\n", sink);
}

}  // namespace

int main() {
    test_status_strings();
    test_rope();
    test_attn();
    test_copies();
    test_paged();
    test_accept();
    test_coupled();
    test_route();
    test_tree();
    test_states();
    test_commit_append();
    test_workspace_extremes();
    printf("%d checks, %d failures\n", checks, failures);
    return failures ? 1 : 0;
}
