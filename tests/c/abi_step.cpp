// abi_step.cpp -- a client of libspecverify.so that uses only the C ABI of
// include/spec_verify.h and the HIP runtime for memory and a stream: one
// verification step (spec_verify_attn with RoPE, then spec_verify_accept) on
// inputs read from binary files, outputs written back to files.  Test
// infrastructure: tests/test_gpu_c_client.py writes the inputs, runs this
// program and checks its outputs against the CPU oracle.
//
// usage: abi_step <dir>
//   <dir>/shape.txt: batch block gamma prefix n_qh n_kvh head_dim vocab theta
//   inputs:  q, k_new, v_new, k_cache, v_cache (.bin, bfloat16 bits), tau,
//            draft_tokens (int32), target_logits, draft_probs, uniforms (float32)
//   outputs: out (bfloat16 bits), accept_len, out_tokens (int32), alpha (float32)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "spec_verify.h"

namespace {

std::string g_dir;

bool read_file(const char *name, void *dst, size_t bytes) {
    const std::string path = g_dir + "/" + name;
    FILE *f = std::fopen(path.c_str(), "rb");
    if (!f) { std::fprintf(stderr, "cannot open %s\n", path.c_str()); return false; }
    const size_t got = std::fread(dst, 1, bytes, f);
    std::fclose(f);
    if (got != bytes) { std::fprintf(stderr, "%s: %zu of %zu bytes\n", path.c_str(), got, bytes); return false; }
    return true;
}

bool write_file(const char *name, const void *src, size_t bytes) {
    const std::string path = g_dir + "/" + name;
    FILE *f = std::fopen(path.c_str(), "wb");
    if (!f) { std::fprintf(stderr, "cannot create %s\n", path.c_str()); return false; }
    const size_t put = std::fwrite(src, 1, bytes, f);
    std::fclose(f);
    return put == bytes;
}

#define HIP_OK(x)                                                                        \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
            return 3;                                                                    \
        }                                                                                \
    } while (0)

#define SV_OK_OR_FAIL(x)                                                                 \
    do {                                                                                 \
        const int s_ = (x);                                                              \
        if (s_ != SV_OK) {                                                               \
            std::fprintf(stderr, "%s: %s\n", #x, spec_verify_status_string(s_));         \
            return 4;                                                                    \
        }                                                                                \
    } while (0)

struct Dev {  // one device buffer with its host copy
    std::vector<unsigned char> host;
    void *dev = nullptr;
};

}  // namespace

int main(int argc, char **argv) {
    if (argc != 2) { std::fprintf(stderr, "usage: abi_step <dir>\n"); return 2; }
    g_dir = argv[1];
    int batch, block, gamma, prefix, n_qh, n_kvh, head_dim;
    long long vocab;
    double theta;
    {
        const std::string path = g_dir + "/shape.txt";
        FILE *f = std::fopen(path.c_str(), "r");
        if (!f || std::fscanf(f, "%d %d %d %d %d %d %d %lld %lf", &batch, &block, &gamma, &prefix, &n_qh, &n_kvh,
                              &head_dim, &vocab, &theta) != 9) {
            std::fprintf(stderr, "bad %s\n", path.c_str());
            return 2;
        }
        std::fclose(f);
    }
    if (spec_verify_abi_version() != SPEC_VERIFY_ABI_VERSION) { std::fprintf(stderr, "ABI version mismatch\n"); return 2; }
    const size_t R = 2 * (size_t)block;
    const size_t n_q = (size_t)batch * R * n_qh * head_dim, n_kv = (size_t)batch * R * n_kvh * head_dim;
    const size_t n_cache = (size_t)batch * n_kvh * prefix * head_dim, n_slot = (size_t)batch * block;
    const size_t n_logit = n_slot * (size_t)vocab;
    struct Spec { const char *name; size_t bytes; bool input; };
    const Spec specs[] = {
        {"q.bin", n_q * 2, true},           {"k_new.bin", n_kv * 2, true},
        {"v_new.bin", n_kv * 2, true},      {"k_cache.bin", n_cache * 2, true},
        {"v_cache.bin", n_cache * 2, true}, {"tau.bin", n_slot * 4, true},
        {"draft_tokens.bin", n_slot * 4, true}, {"target_logits.bin", n_logit * 4, true},
        {"draft_probs.bin", n_logit * 4, true}, {"uniforms.bin", (size_t)batch * (gamma + 1) * 4, true},
        {"out.bin", n_q * 2, false},        {"accept_len.bin", (size_t)batch * 4, false},
        {"out_tokens.bin", n_slot * 4, false}, {"alpha.bin", (size_t)batch * gamma * 4, false},
    };
    constexpr int N = sizeof(specs) / sizeof(specs[0]);
    Dev buf[N];
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    for (int i = 0; i < N; ++i) {
        const size_t bytes = specs[i].bytes ? specs[i].bytes : 16;  // an empty cache still gets a valid pointer
        buf[i].host.assign(bytes, 0);
        if (specs[i].input && specs[i].bytes && !read_file(specs[i].name, buf[i].host.data(), specs[i].bytes)) return 2;
        HIP_OK(hipMalloc(&buf[i].dev, bytes));
        HIP_OK(hipMemcpyAsync(buf[i].dev, buf[i].host.data(), bytes, hipMemcpyHostToDevice, stream));
    }
    const size_t ws_attn = spec_verify_attn_workspace_size(SV_BF16, batch, block, prefix, n_qh, n_kvh, head_dim);
    const size_t ws_acc = spec_verify_accept_workspace_size(batch, block, gamma, vocab);
    if (ws_acc == 0) { std::fprintf(stderr, "accept workspace size 0: shape rejected\n"); return 2; }
    void *ws = nullptr;
    const size_t ws_bytes = ws_attn > ws_acc ? ws_attn : ws_acc;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    SV_OK_OR_FAIL(spec_verify_attn(buf[0].dev, buf[1].dev, buf[2].dev, buf[3].dev, buf[4].dev,
                                   (const int32_t *)buf[5].dev, buf[10].dev, SV_BF16, batch, block, prefix, n_qh,
                                   n_kvh, head_dim, theta, 0.0f, ws, ws_bytes, stream));
    SV_OK_OR_FAIL(spec_verify_accept((const float *)buf[7].dev, (const float *)buf[8].dev,
                                     (const int32_t *)buf[6].dev, (const int32_t *)buf[5].dev,
                                     (const float *)buf[9].dev, batch, block, gamma, vocab,
                                     (int32_t *)buf[11].dev, (int32_t *)buf[12].dev, (float *)buf[13].dev, ws,
                                     ws_bytes, stream));
    for (int i = 10; i < N; ++i)
        HIP_OK(hipMemcpyAsync(buf[i].host.data(), buf[i].dev, specs[i].bytes, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    for (int i = 10; i < N; ++i)
        if (!write_file(specs[i].name, buf[i].host.data(), specs[i].bytes)) return 2;
    for (int i = 0; i < N; ++i) HIP_OK(hipFree(buf[i].dev));
    HIP_OK(hipFree(ws));
    HIP_OK(hipStreamDestroy(stream));
    std::printf("abi_step: ok\n");
    return 0;
}
