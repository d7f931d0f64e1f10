// coupled.hip -- shared-noise (Gumbel-coupled) and greedy verification for
// gfx950 (MI355X).
//
// Method: "SPOT: Enhancing Speculative Decoding for Diffusion Language Models
// via Commit-Order Prediction", 前置知识 "Gumbel-Max 技巧与随机耦合" (the argmax
// of log-probability plus Gumbel noise is a sample of the distribution; a
// noise table shared by draft and target couples the two samples) and
// 核心创新 / 方法步骤详情 (noise indexed by absolute output position; given the
// noise the target transition is deterministic; a step is accepted when the
// draft state equals the target's, otherwise the target's own result is
// committed; T = 0 is the greedy transition).  Draft order and slot layout as
// in "SimSD: Simple Speculative Decoding in Diffusion Language Models",
// 关键设计 1 and 4.
//
// Two launches on the caller's stream:
//   coupled_partial_kernel  vocab-parallel argmax of every verified slot's
//                           score fmaf(l, 1/T, g) in float32 (l alone when
//                           greedy): a streaming pass over the logits and the
//                           noise rows, 16-byte non-temporal loads (both are
//                           read once), 4 of each in flight per lane; per
//                           (slot, vocab split) the best score and its
//                           smallest index.
//   coupled_scan_kernel     one wave per sequence: lane k merges slot k's
//                           partials into the target's choice and compares it
//                           with the draft token; the first mismatch in draft
//                           order is a wave minimum over the mismatched steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct Best {   // best score of a vocab range and its smallest index
    float s;
    int32_t i;
};

// a beats b: higher score, or the same score at a smaller index
__device__ __forceinline__ bool better(float sa, int32_t ia, float sb, int32_t ib) {
    return sa > sb || (sa == sb && ia < ib);
}

typedef float cpl_f4 __attribute__((ext_vector_type(4)));

template <bool VEC, bool GREEDY>
__global__ void __launch_bounds__(256) coupled_partial_kernel(const float *__restrict__ logits,
                                                              const float *__restrict__ noise,
                                                              const int32_t *__restrict__ tau, Best *parts,
                                                              int gamma, int64_t vocab, int n_vsplit, float inv_t) {
    __shared__ float red_s[4];
    __shared__ int32_t red_i[4];
    const int row = blockIdx.x / n_vsplit, sp = blockIdx.x % n_vsplit;
    if (tau && tau[row] > gamma) return;  // slot not verified in this call (no tau: every row)
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float bs = -INFINITY;
    int32_t bi = INT32_MAX;
    auto take = [&](float l, float g, int64_t v) {
        const float sc = GREEDY ? l : fmaf(l, inv_t, g);
        if (better(sc, (int32_t)v, bs, bi)) { bs = sc; bi = (int32_t)v; }
    };
    if (VEC) {
        const int64_t n4 = vocab >> 2;
        const int64_t c0 = n4 * sp / n_vsplit, c1 = n4 * (sp + 1) / n_vsplit;
        const cpl_f4 *lsrc = reinterpret_cast<const cpl_f4 *>(logits + (size_t)row * vocab);
        const cpl_f4 *gsrc = GREEDY ? nullptr : reinterpret_cast<const cpl_f4 *>(noise + (size_t)row * vocab);
        // a lane visits its entries in ascending order (u, then the 4 lanes of
        // a vector), so a strict comparison keeps the smallest index of ties
        for (int64_t i = c0 + tid; i < c1; i += 256 * 4) {
            cpl_f4 l[4], g[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = i + 256 * u < c1;
                l[u] = ok ? __builtin_nontemporal_load(lsrc + i + 256 * u) : cpl_f4{0.f, 0.f, 0.f, 0.f};
                if (!GREEDY) g[u] = ok ? __builtin_nontemporal_load(gsrc + i + 256 * u) : cpl_f4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (i + 256 * u >= c1) break;
                const int64_t v = 4 * (i + 256 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (GREEDY) take(l[u][e], 0.f, v + e);
                    else take(l[u][e], g[u][e], v + e);
                }
            }
        }
    } else {
        const int64_t c0 = vocab * sp / n_vsplit, c1 = vocab * (sp + 1) / n_vsplit;
        const float *lr = logits + (size_t)row * vocab;
        const float *gr = GREEDY ? nullptr : noise + (size_t)row * vocab;
        for (int64_t v = c0 + tid; v < c1; v += 256) {
            if constexpr (GREEDY) take(lr[v], 0.f, v);
            else take(lr[v], gr[v], v);
        }
    }
    // workgroup merge
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float s2 = __shfl_xor(bs, o);
        const int32_t i2 = __shfl_xor(bi, o);
        if (better(s2, i2, bs, bi)) { bs = s2; bi = i2; }
    }
    if (lane == 0) { red_s[w] = bs; red_i[w] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < 4; ++k)
            if (better(red_s[k], red_i[k], bs, bi)) { bs = red_s[k]; bi = red_i[k]; }
        parts[(size_t)row * n_vsplit + sp] = Best{bs, bi};
    }
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

// One wave per sequence; lane k takes slot k (draft step tau(k)).
__global__ void __launch_bounds__(64) coupled_scan_kernel(const int32_t *__restrict__ tokens,
                                                          const int32_t *__restrict__ tau,
                                                          const Best *__restrict__ parts, int block, int gamma,
                                                          int n_vsplit, int32_t *accept_len, int32_t *out_tokens,
                                                          int32_t *target_tokens) {
    const int lane = threadIdx.x, b = blockIdx.x;
    const bool in = lane < block;
    const size_t row = (size_t)b * block + (in ? lane : 0);
    const int t = in ? tau[row] : 0;
    const int x = in ? tokens[row] : -1;
    const bool ver = in && t >= 1 && t <= gamma;  // slot verified at draft step t
    float bs = -INFINITY;
    int32_t bi = INT32_MAX;
    if (ver) {
#pragma unroll 4
        for (int i = 0; i < n_vsplit; ++i) {
            const Best p = parts[row * n_vsplit + i];
            if (better(p.s, p.i, bs, bi)) { bs = p.s; bi = p.i; }
        }
    }
    const int choice = ver ? bi : -1;  // the target's own token at this slot
    const int L = wave_min_i32((ver && x != choice) ? t - 1 : gamma);
    if (in) {
        out_tokens[row] = (t <= L) ? x : ((ver && t == L + 1) ? choice : -1);
        if (target_tokens) target_tokens[row] = choice;
    }
    if (lane == 0) accept_len[b] = L;
}

// Draft-tree verification ("SPOT", 核心方法 second step and 方法步骤详情 验证),
// one wave per sequence: lane n merges node n's partials into the target's
// own token at its next commit position; then, from the root, each step is
// one ballot over the nodes for the child whose (position, token) equals
// the target's own commit at the current node (the smallest such index).
// A walk has at most n_nodes - 1 edges, so the loop ends whatever the
// parent array holds; node 0 is the root and is never taken as a child.
__global__ void __launch_bounds__(64) tree_scan_kernel(const Best *__restrict__ parts, const int32_t *__restrict__ parent,
                                                       const int32_t *__restrict__ node_pos,
                                                       const int32_t *__restrict__ node_tok,
                                                       const int32_t *__restrict__ target_pos, int n_nodes,
                                                       int n_vsplit, int32_t *path_len, int32_t *path,
                                                       int32_t *commit_pos, int32_t *commit_tok, int32_t *target_tok) {
    const int lane = threadIdx.x, b = blockIdx.x;
    const bool in = lane < n_nodes;
    const size_t row = (size_t)b * n_nodes + (in ? lane : 0);
    const int par = in ? parent[row] : -2, pos = in ? node_pos[row] : -1, tok = in ? node_tok[row] : -1;
    const int tpos = in ? target_pos[row] : -1;
    float bs = -INFINITY;
    int32_t bi = INT32_MAX;
    if (in) {
#pragma unroll 4
        for (int i = 0; i < n_vsplit; ++i) {
            const Best p = parts[row * n_vsplit + i];
            if (better(p.s, p.i, bs, bi)) { bs = p.s; bi = p.i; }
        }
    }
    const int own = in ? bi : -1;  // the target's own token at this node's next commit
    if (in && target_tok) target_tok[row] = own;
    int cur = 0, L = 0;
    for (; L < n_nodes - 1; ++L) {
        const int cpos = __shfl(tpos, cur), ctok = __shfl(own, cur);
        const unsigned long long m = __ballot(in && lane > 0 && par == cur && pos == cpos && tok == ctok);
        if (!m) break;
        cur = __ffsll((long long)m) - 1;
        if (lane == 0) path[(size_t)b * n_nodes + L + 1] = cur;
    }
    if (in && lane > L) path[row] = -1;
    if (lane == 0) {
        path[(size_t)b * n_nodes] = 0;
        path_len[b] = L;
    }
    const int fpos = __shfl(tpos, cur), ftok = __shfl(own, cur);
    if (lane == 0) { commit_pos[b] = fpos; commit_tok[b] = ftok; }
}

hipError_t launch_tree(const CoupledPlan &p, const float *logits, const float *noise, const int32_t *parent,
                       const int32_t *node_pos, const int32_t *node_tok, const int32_t *target_pos, int batch,
                       int n_nodes, int64_t vocab, float inv_t, int32_t *path_len, int32_t *path, int32_t *commit_pos,
                       int32_t *commit_tok, int32_t *target_tok, void *ws, hipStream_t st) {
    Best *parts = (Best *)ws;
    const dim3 g1((unsigned)((size_t)p.rows * p.n_vsplit));
    const bool vec = (vocab & 3) == 0, greedy = !(inv_t > 0.f);
    const int32_t *no_tau = nullptr;
    if (vec && greedy)
        hipLaunchKernelGGL((coupled_partial_kernel<true, true>), g1, dim3(256), 0, st, logits, noise, no_tau, parts,
                           n_nodes, vocab, p.n_vsplit, inv_t);
    else if (vec)
        hipLaunchKernelGGL((coupled_partial_kernel<true, false>), g1, dim3(256), 0, st, logits, noise, no_tau, parts,
                           n_nodes, vocab, p.n_vsplit, inv_t);
    else if (greedy)
        hipLaunchKernelGGL((coupled_partial_kernel<false, true>), g1, dim3(256), 0, st, logits, noise, no_tau, parts,
                           n_nodes, vocab, p.n_vsplit, inv_t);
    else
        hipLaunchKernelGGL((coupled_partial_kernel<false, false>), g1, dim3(256), 0, st, logits, noise, no_tau, parts,
                           n_nodes, vocab, p.n_vsplit, inv_t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tree_scan_kernel, dim3(batch), dim3(64), 0, st, parts, parent, node_pos, node_tok, target_pos,
                       n_nodes, p.n_vsplit, path_len, path, commit_pos, commit_tok, target_tok);
    return hipGetLastError();
}

CoupledPlan coupled_plan(int batch, int block, int gamma, int64_t vocab) {
    CoupledPlan p{};
    p.rows = batch * block;
    const long active = (long)batch * gamma;
    long vs = (2048 + active - 1) / active;
    long cap = vocab / 16384;
    if (cap < 1) cap = 1;
    if (vs > cap) vs = cap;
    if (vs < 1) vs = 1;
    p.n_vsplit = (int)vs;
    p.ws_total = align_up((size_t)p.rows * p.n_vsplit * sizeof(Best));
    return p;
}

hipError_t launch_coupled(const CoupledPlan &p, const float *logits, const float *noise, const int32_t *tokens,
                          const int32_t *tau, int batch, int block, int gamma, int64_t vocab, float inv_t,
                          int32_t *accept_len, int32_t *out_tokens, int32_t *target_tokens, void *ws,
                          hipStream_t st) {
    Best *parts = (Best *)ws;
    const dim3 g1((unsigned)((size_t)p.rows * p.n_vsplit));
    const bool vec = (vocab & 3) == 0, greedy = !(inv_t > 0.f);
    if (vec && greedy)
        hipLaunchKernelGGL((coupled_partial_kernel<true, true>), g1, dim3(256), 0, st, logits, noise, tau, parts,
                           gamma, vocab, p.n_vsplit, inv_t);
    else if (vec)
        hipLaunchKernelGGL((coupled_partial_kernel<true, false>), g1, dim3(256), 0, st, logits, noise, tau, parts,
                           gamma, vocab, p.n_vsplit, inv_t);
    else if (greedy)
        hipLaunchKernelGGL((coupled_partial_kernel<false, true>), g1, dim3(256), 0, st, logits, noise, tau, parts,
                           gamma, vocab, p.n_vsplit, inv_t);
    else
        hipLaunchKernelGGL((coupled_partial_kernel<false, false>), g1, dim3(256), 0, st, logits, noise, tau, parts,
                           gamma, vocab, p.n_vsplit, inv_t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(coupled_scan_kernel, dim3(batch), dim3(64), 0, st, tokens, tau, parts, block, gamma,
                       p.n_vsplit, accept_len, out_tokens, target_tokens);
    return hipGetLastError();
}

}  // namespace sv
