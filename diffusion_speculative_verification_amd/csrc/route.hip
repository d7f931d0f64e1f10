// route.hip -- verify-routing estimator for gfx950 (MI355X).
//
// Method: "S2D2: Fast Decoding for Diffusion LLMs via Training-Free
// Self-Speculation", 方法步骤详情 (4), the routing decision: the expected
// accepted prefix length K = sum_k prod_{i<=k} alpha_i, with alpha_i
// estimated from the draft distribution by its margin (1[m_i >= threshold])
// or by its entropy (exp(-beta H~_i)).  Steps in draft order as in "SimSD:
// Simple Speculative Decoding in Diffusion Language Models", 关键设计 4.
//
// Two launches on the caller's stream:
//   route_partial_kernel  per (verified slot, vocab split): the two largest
//                         draft probabilities (three min/max per entry) and
//                         sum_v p_v log2 p_v (hardware log2, float32 within
//                         16 entries, float64 across), streaming the draft
//                         rows with 16-byte non-temporal loads.
//   route_scan_kernel     one wave per sequence: lane k merges slot k's
//                         partials into alpha_k; the alphas are placed in
//                         draft order through LDS, then an inclusive product
//                         scan and a sum give K.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct RoutePart {  // one (slot, vocab split)
    float p1, p2;   // largest and second largest probability
    double h2;      // sum p log2 p over the split (entries with p > 0)
};

typedef float rt_f4 __attribute__((ext_vector_type(4)));

// p log2 p with the hardware log2; entries below the smallest normal float
// (whose terms are below 1e-36) count as 0, which keeps denormal inputs away
// from the hardware log2
__device__ __forceinline__ float plog2p(float p) {
    return p >= 1.17549435e-38f ? p * __builtin_amdgcn_logf(p) : 0.f;
}

__device__ __forceinline__ void top2(float &p1, float &p2, float x) {
    p2 = fmaxf(p2, fminf(p1, x));
    p1 = fmaxf(p1, x);
}

template <bool VEC>
__global__ void __launch_bounds__(256) route_partial_kernel(const float *__restrict__ probs,
                                                            const int32_t *__restrict__ tau, RoutePart *parts,
                                                            int gamma, int64_t vocab, int n_vsplit) {
    __shared__ float red_p1[4], red_p2[4];
    __shared__ double red_h[4];
    const int row = blockIdx.x / n_vsplit, sp = blockIdx.x % n_vsplit;
    if (tau[row] > gamma) return;  // slot not verified in this call
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float p1 = -INFINITY, p2 = -INFINITY;
    double h = 0.0;
    if (VEC) {
        const int64_t n4 = vocab >> 2;
        const int64_t c0 = n4 * sp / n_vsplit, c1 = n4 * (sp + 1) / n_vsplit;
        const rt_f4 *src = reinterpret_cast<const rt_f4 *>(probs + (size_t)row * vocab);
        for (int64_t i = c0 + tid; i < c1; i += 256 * 4) {
            rt_f4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                x[u] = (i + 256 * u < c1) ? __builtin_nontemporal_load(src + i + 256 * u) : rt_f4{0.f, 0.f, 0.f, 0.f};
            float hs = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    top2(p1, p2, x[u][e]);
                    hs += plog2p(x[u][e]);
                }
            h += (double)hs;
        }
    } else {
        const int64_t c0 = vocab * sp / n_vsplit, c1 = vocab * (sp + 1) / n_vsplit;
        const float *pr = probs + (size_t)row * vocab;
        for (int64_t v = c0 + tid; v < c1; v += 256) {
            const float x = pr[v];
            top2(p1, p2, x);
            h += (double)plog2p(x);
        }
    }
    // padding entries of the vector path are zeros: they add nothing to the
    // sum and cannot displace a probability from the top two
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float q1 = __shfl_xor(p1, o), q2 = __shfl_xor(p2, o);
        p2 = fmaxf(fminf(p1, q1), fmaxf(p2, q2));
        p1 = fmaxf(p1, q1);
        h += __shfl_xor(h, o);
    }
    if (lane == 0) { red_p1[w] = p1; red_p2[w] = p2; red_h[w] = h; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < 4; ++k) {
            p2 = fmaxf(fminf(p1, red_p1[k]), fmaxf(p2, red_p2[k]));
            p1 = fmaxf(p1, red_p1[k]);
            h += red_h[k];
        }
        parts[(size_t)row * n_vsplit + sp] = RoutePart{p1, p2, h};
    }
}

// One wave per sequence; lane k takes slot k, then lane r takes draft step r+1.
__global__ void __launch_bounds__(64) route_scan_kernel(const int32_t *__restrict__ tau,
                                                        const RoutePart *__restrict__ parts, int block, int gamma,
                                                        int64_t vocab, int n_vsplit, int estimator, double param,
                                                        float *khat, float *alpha_hat) {
    __shared__ double a_step[64];
    const int lane = threadIdx.x, b = blockIdx.x;
    const bool in = lane < block;
    const size_t row = (size_t)b * block + (in ? lane : 0);
    const int t = in ? tau[row] : 0;
    const bool ver = in && t >= 1 && t <= gamma;
    a_step[lane] = 1.0;
    __syncthreads();
    if (ver) {
        float p1 = -INFINITY, p2 = -INFINITY;
        double h2 = 0.0;
        for (int i = 0; i < n_vsplit; ++i) {
            const RoutePart p = parts[row * n_vsplit + i];
            p2 = fmaxf(fminf(p1, p.p1), fmaxf(p2, p.p2));
            p1 = fmaxf(p1, p.p1);
            h2 += p.h2;
        }
        double a;
        if (estimator == 0) {
            const double m = (double)p1 - (double)fmaxf(p2, 0.f);  // exact in float64
            a = (m >= param) ? 1.0 : 0.0;
        } else {
            // -sum p ln p / ln V = -sum p log2 p / log2 V
            const double hn = vocab > 1 ? -h2 / log2((double)vocab) : 0.0;
            a = exp(-param * hn);
        }
        a_step[t - 1] = a;
    }
    __syncthreads();
    const double a = a_step[lane];  // draft step lane + 1 (1 past gamma)
    double prod = a;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double q = __shfl_up(prod, o);
        if (lane >= o) prod *= q;
    }
    double sum = lane < gamma ? prod : 0.0;
    sum = wave_sum(sum);
    if (alpha_hat && lane < gamma) alpha_hat[(size_t)b * gamma + lane] = (float)a;
    if (lane == 0) khat[b] = (float)sum;
}

// Vocabulary parts per verified row, as for the normaliser pass: about 2048
// workgroups, no part shorter than 32768 entries (128 verified rows at
// vocabulary 151936: 4 parts, 18.5 us per call against 20.3 us with 9).
RoutePlan route_plan(int batch, int block, int gamma, int64_t vocab) {
    RoutePlan p{};
    p.rows = batch * block;
    const long active = (long)batch * gamma;
    long vs = (2048 + active - 1) / active;
    long cap = vocab / 32768;
    if (cap < 1) cap = 1;
    if (vs > cap) vs = cap;
    if (vs < 1) vs = 1;
    p.n_vsplit = (int)vs;
    p.ws_total = align_up((size_t)p.rows * p.n_vsplit * sizeof(RoutePart));
    return p;
}

hipError_t launch_route(const RoutePlan &p, const float *probs, const int32_t *tau, int batch, int block,
                        int gamma, int64_t vocab, int estimator, double param, float *khat, float *alpha_hat,
                        void *ws, hipStream_t st) {
    RoutePart *parts = (RoutePart *)ws;
    const dim3 g1((unsigned)((size_t)p.rows * p.n_vsplit));
    if ((vocab & 3) == 0)
        hipLaunchKernelGGL(route_partial_kernel<true>, g1, dim3(256), 0, st, probs, tau, parts, gamma, vocab,
                           p.n_vsplit);
    else
        hipLaunchKernelGGL(route_partial_kernel<false>, g1, dim3(256), 0, st, probs, tau, parts, gamma, vocab,
                           p.n_vsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_scan_kernel, dim3(batch), dim3(64), 0, st, tau, parts, block, gamma, vocab,
                       p.n_vsplit, estimator, param, khat, alpha_hat);
    return hipGetLastError();
}

}  // namespace sv
