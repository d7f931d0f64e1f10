// states.hip -- verification of a tree of block states for gfx950 (MI355X).
//
// Method: "SPOT: Enhancing Speculative Decoding for Diffusion Language Models
// via Commit-Order Prediction": 前置知识 "块扩散语言模型" (a decoding step
// commits the masked position of highest confidence), 前置知识 "动态阈值解码"
// (confidence c_s = max_v p_theta,s(v); every masked position above the
// threshold is committed, else the single highest), 核心方法 third step and
// 方法步骤详情 验证 (one forward over the root and every draft copy gives the
// target's own next transition at each state -- Phi_0 at T = 0, Phi_G for the
// fixed noise table at T > 0; edges whose child equals it are accepted, else
// the target's own result is committed) and 核心创新 (noise indexed by absolute
// output position, shared by all copies).
//
// Two launches on the caller's stream:
//   states_partial_kernel (or states_partial_noise_kernel, below)
//                          one streaming pass over the float32 logits of
//                          every masked slot of every copy (rows of decided
//                          slots are skipped): per (node, slot, vocab split)
//                          the max logit, the normaliser sum exp(l - max) in
//                          float64, and the argmax of the coupled score
//                          fmaf(l, 1/T, g) (l alone when greedy) with its
//                          smallest index (a lane takes the best score of
//                          each round of 16 entries first and looks for its
//                          index only when it beats the running best).
//                          16-byte non-temporal loads of the logits (read
//                          once), 4 in flight per lane; the noise rows are
//                          read with ordinary loads, because the copies of
//                          one slot read the same row.  At T > 0 on the
//                          16-byte path, states_partial_noise_kernel streams
//                          two copies of a slot per workgroup, so each noise
//                          load serves both.
//   states_walk_kernel     one workgroup per sequence: a wave per node turns
//                          its slots' partials into confidences (1 / sum, in
//                          float64) and applies the threshold rule with
//                          ballots (lane = slot); then each node is checked
//                          against its parent with the parent's commit
//                          applied, and wave 0 walks the tree from the root
//                          with one ballot per accepted edge.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct SPart {   // one (node, slot, vocab split)
    float m;     // max logit (-inf when every entry is -inf)
    float bs;    // best coupled score
    int32_t bi;  // its smallest index
    int32_t pad;
    double s;    // sum exp(l - m)
};

namespace {

typedef float st_f4 __attribute__((ext_vector_type(4)));

// a beats b: higher score, or the same score at a smaller index
__device__ __forceinline__ bool st_better(float sa, int32_t ia, float sb, int32_t ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// (m, s) pairs: the merged max and sum exp(l - max); -inf maxima carry s = 0
__device__ __forceinline__ void lse_merge(float &m, double &s, float m2, double s2) {
    if (m2 > m) {
        s = s * (double)__builtin_amdgcn_exp2f((m - m2) * kLog2e) + s2;
        m = m2;
    } else if (m2 != -INFINITY) {
        s += s2 * (double)__builtin_amdgcn_exp2f((m2 - m) * kLog2e);
    }
}

template <bool VEC, bool GREEDY>
__global__ void __launch_bounds__(256) states_partial_kernel(const float *__restrict__ logits,
                                                             const float *__restrict__ noise,
                                                             const int32_t *__restrict__ state, SPart *parts,
                                                             int n_nodes, int block, int64_t vocab, int n_vsplit,
                                                             long long n_tasks, float inv_t) {
    __shared__ float red_m[4], red_bs[4];
    __shared__ double red_s[4];
    __shared__ int32_t red_bi[4];
    // Workgroups go round-robin over the 8 XCDs (workgroup i to XCD i % 8).
    // Tasks come in groups of n_nodes -- the copies of one (slot, vocab
    // split), which read the same noise chunk -- and the groups are dealt
    // round-robin over the XCDs: the j-th workgroup an XCD receives takes
    // copy j % n_nodes of that XCD's (j / n_nodes)-th group, so a group's
    // copies run one after another on one XCD and share its L2, while every
    // XCD gets groups from every sequence (equal shares of the masked rows;
    // whole sequences per XCD left the XCDs up to 2x apart in work).
    const long long j = (long long)(blockIdx.x >> 3);
    const long long task = (8 * (j / n_nodes) + (blockIdx.x & 7)) * n_nodes + j % n_nodes;
    if (task >= n_tasks) return;
    const int n = (int)(task % n_nodes);
    long long t = task / n_nodes;
    const int sp = (int)(t % n_vsplit);
    t /= n_vsplit;
    const int s = (int)(t % block);
    const long long b = t / block;
    const size_t row = ((size_t)b * n_nodes + n) * block + s;
    if (state[row] >= 0) return;  // decided slot: no part in the transition
    const size_t nrow = (size_t)b * block + s;  // noise row of the slot's absolute position
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float m = -INFINITY, bs = -INFINITY;
    double sum = 0.0;
    int32_t bi = INT32_MAX;
    if (VEC) {
        const int64_t n4 = vocab >> 2;
        const int64_t c0 = n4 * sp / n_vsplit, c1 = n4 * (sp + 1) / n_vsplit;
        const st_f4 *lsrc = reinterpret_cast<const st_f4 *>(logits + row * vocab);
        const st_f4 *gsrc = GREEDY ? nullptr : reinterpret_cast<const st_f4 *>(noise + nrow * vocab);
        // a lane visits its entries in ascending index order (u, then the 4
        // entries of a vector)
        for (int64_t i = c0 + tid; i < c1; i += 256 * 4) {
            st_f4 x[4], g[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = i + 256 * u < c1;
                x[u] = ok ? __builtin_nontemporal_load(lsrc + i + 256 * u)
                          : st_f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                if (!GREEDY) g[u] = ok ? gsrc[i + 256 * u] : st_f4{0.f, 0.f, 0.f, 0.f};
            }
            float gm = m;
#pragma unroll
            for (int u = 0; u < 4; ++u) gm = fmaxf(gm, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
            if (gm > m) {
                if (m != -INFINITY) sum *= (double)__builtin_amdgcn_exp2f((m - gm) * kLog2e);
                m = gm;
            }
            const float mu = (m == -INFINITY) ? 0.f : m;
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) ps += __builtin_amdgcn_exp2f((x[u][e] - mu) * kLog2e);
            // the coupled argmax: the round's best score first, its first
            // index only when it beats the running best (entries ascend)
            st_f4 sc[4];
            float gs = -INFINITY;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sc[u][e] = GREEDY ? x[u][e] : fmaf(x[u][e], inv_t, g[u][e]);
                gs = fmaxf(gs, fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3])));
            }
            if (gs > bs) {
                int32_t idx = INT32_MAX;
#pragma unroll
                for (int u = 3; u >= 0; --u)
#pragma unroll
                    for (int e = 3; e >= 0; --e)
                        if (sc[u][e] == gs) idx = (int32_t)(4 * (i + 256 * u)) + e;
                bs = gs;
                bi = idx;
            }
            sum += (double)ps;
        }
    } else {
        const int64_t c0 = vocab * sp / n_vsplit, c1 = vocab * (sp + 1) / n_vsplit;
        const float *lr = logits + row * vocab;
        const float *gr = GREEDY ? nullptr : noise + nrow * vocab;
        for (int64_t v = c0 + tid; v < c1; v += 256) {
            const float x = lr[v];
            if (x > m) {
                if (m != -INFINITY) sum *= (double)__builtin_amdgcn_exp2f((m - x) * kLog2e);
                m = x;
            }
            sum += (double)__builtin_amdgcn_exp2f((x - ((m == -INFINITY) ? 0.f : m)) * kLog2e);
            const float sc = GREEDY ? x : fmaf(x, inv_t, gr[v]);
            if (st_better(sc, (int32_t)v, bs, bi)) { bs = sc; bi = (int32_t)v; }
        }
    }
    // workgroup merge
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o), bs2 = __shfl_xor(bs, o);
        const double s2 = __shfl_xor(sum, o);
        const int32_t bi2 = __shfl_xor(bi, o);
        lse_merge(m, sum, m2, s2);
        if (st_better(bs2, bi2, bs, bi)) { bs = bs2; bi = bi2; }
    }
    if (lane == 0) { red_m[w] = m; red_s[w] = sum; red_bs[w] = bs; red_bi[w] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < 4; ++k) {
            lse_merge(m, sum, red_m[k], red_s[k]);
            if (st_better(red_bs[k], red_bi[k], bs, bi)) { bs = red_bs[k]; bi = red_bi[k]; }
        }
        parts[row * n_vsplit + sp] = SPart{m, bs, bi, 0, sum};
    }
}

struct RowAcc {
    float m, bs;
    double sum;
    int32_t bi;
};

// One copy's running state in the shared-noise pass, and one round of 16
// entries of its row (as in states_partial_kernel's 16-byte path)
__device__ __forceinline__ void acc_round(RowAcc &A, const st_f4 (&x)[4], const st_f4 (&g)[4], float inv_t,
                                          int64_t i) {
    float gm = A.m;
#pragma unroll
    for (int u = 0; u < 4; ++u) gm = fmaxf(gm, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
    if (gm > A.m) {
        if (A.m != -INFINITY) A.sum *= (double)__builtin_amdgcn_exp2f((A.m - gm) * kLog2e);
        A.m = gm;
    }
    const float mu = (A.m == -INFINITY) ? 0.f : A.m;
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) ps += __builtin_amdgcn_exp2f((x[u][e] - mu) * kLog2e);
    st_f4 sc[4];
    float gs = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[u][e] = fmaf(x[u][e], inv_t, g[u][e]);
        gs = fmaxf(gs, fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3])));
    }
    if (gs > A.bs) {
        int32_t idx = INT32_MAX;
#pragma unroll
        for (int u = 3; u >= 0; --u)
#pragma unroll
            for (int e = 3; e >= 0; --e)
                if (sc[u][e] == gs) idx = (int32_t)(4 * (i + 256 * u)) + e;
        A.bs = gs;
        A.bi = idx;
    }
    A.sum += (double)ps;
}

__device__ __forceinline__ void acc_merge_write(RowAcc A, SPart *dst) {
    __shared__ float red_m[4], red_bs[4];
    __shared__ double red_s[4];
    __shared__ int32_t red_bi[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(A.m, o), bs2 = __shfl_xor(A.bs, o);
        const double s2 = __shfl_xor(A.sum, o);
        const int32_t bi2 = __shfl_xor(A.bi, o);
        lse_merge(A.m, A.sum, m2, s2);
        if (st_better(bs2, bi2, A.bs, A.bi)) { A.bs = bs2; A.bi = bi2; }
    }
    __syncthreads();
    if (lane == 0) { red_m[w] = A.m; red_s[w] = A.sum; red_bs[w] = A.bs; red_bi[w] = A.bi; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < 4; ++k) {
            lse_merge(A.m, A.sum, red_m[k], red_s[k]);
            if (st_better(red_bs[k], red_bi[k], A.bs, A.bi)) { A.bs = red_bs[k]; A.bi = red_bi[k]; }
        }
        *dst = SPart{A.m, A.bs, A.bi, 0, A.sum};
    }
}

// The shared-noise pass (T > 0, vocabulary a multiple of 4): NC copies of
// one (slot, vocab split) per workgroup, each 16-byte noise load serving all
// of them (two copies: 728 -> 682 us at the headline tree against one copy
// per workgroup; three tie with two, four lose occupancy).  Task groups and
// their XCD dealing as in states_partial_kernel, a group being the
// ceil(n_nodes / NC) workgroups of one (slot, vocab split).
template <int NC>
__global__ void __launch_bounds__(256) states_partial_noise_kernel(const float *__restrict__ logits,
                                                                   const float *__restrict__ noise,
                                                                   const int32_t *__restrict__ state, SPart *parts,
                                                                   int n_nodes, int block, int64_t vocab,
                                                                   int n_vsplit, long long n_tasks, float inv_t) {
    const int G = (n_nodes + NC - 1) / NC;
    const long long j = (long long)(blockIdx.x >> 3);
    const long long task = (8 * (j / G) + (blockIdx.x & 7)) * G + j % G;
    if (task >= n_tasks) return;
    const int k = (int)(task % G);
    long long t = task / G;
    const int sp = (int)(t % n_vsplit);
    t /= n_vsplit;
    const int s = (int)(t % block);
    const long long b = t / block;
    size_t row[NC];
    bool act[NC];
    bool any = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int n = NC * k + c;
        row[c] = ((size_t)b * n_nodes + (n < n_nodes ? n : NC * k)) * block + s;
        act[c] = n < n_nodes && state[row[c]] < 0;
        any |= act[c];
    }
    if (!any) return;
    const size_t nrow = (size_t)b * block + s;
    const int tid = threadIdx.x;
    RowAcc A[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) A[c] = RowAcc{-INFINITY, -INFINITY, 0.0, INT32_MAX};
    const int64_t n4 = vocab >> 2;
    const int64_t c0 = n4 * sp / n_vsplit, c1 = n4 * (sp + 1) / n_vsplit;
    const st_f4 *gsrc = reinterpret_cast<const st_f4 *>(noise + nrow * vocab);
    for (int64_t i = c0 + tid; i < c1; i += 256 * 4) {
        st_f4 x[NC][4], g[4];
        const st_f4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = i + 256 * u < c1;
            g[u] = ok ? gsrc[i + 256 * u] : st_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c)
                x[c][u] = (ok && act[c])
                    ? __builtin_nontemporal_load(reinterpret_cast<const st_f4 *>(logits + row[c] * vocab) + i + 256 * u)
                    : ninf;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (act[c]) acc_round(A[c], x[c], g, inv_t, i);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
        if (act[c]) acc_merge_write(A[c], parts + row[c] * n_vsplit + sp);
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
    return v;
}

constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kMaxStateCells = 64 * 64;  // n_nodes * block

// Every global load of a sequence's tree is issued before any of its values
// is used (one round trip of latency): the parents, and per node wave the
// states and vocab-split partials of its slots, the partials read whether or
// not the slot is masked (a decided slot's partial is never written, and its
// value is discarded).
__global__ void __launch_bounds__(kWalkThreads) states_walk_kernel(
    const SPart *__restrict__ parts, const int32_t *__restrict__ parent, const int32_t *__restrict__ state,
    int n_nodes, int block, int n_vsplit, double threshold, int32_t *path_len, int32_t *path, int32_t *next_state,
    int32_t *commit_out, float *conf_out) {
    __shared__ int32_t st[kMaxStateCells];   // every node's block
    __shared__ int32_t cm[kMaxStateCells];   // every node's commit (token or -1)
    __shared__ int32_t par[64];
    __shared__ uint8_t open[64], match[64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const size_t b = blockIdx.x;
    const bool in_slot = lane < block;
    if ((int)threadIdx.x < n_nodes) par[threadIdx.x] = parent[b * n_nodes + threadIdx.x];
    // 1. per node (one wave each): confidences and the threshold rule, lane = slot
    for (int n = w; n < n_nodes; n += kWalkWaves) {
        const size_t row = ((size_t)b * n_nodes + n) * block + (in_slot ? lane : 0);
        const int y = in_slot ? state[row] : 0;
        float m = -INFINITY, bs = -INFINITY;
        double sum = 0.0;
        int32_t bi = INT32_MAX;
#pragma unroll 4
        for (int i = 0; i < n_vsplit; ++i) {
            const SPart q = parts[row * n_vsplit + i];
            lse_merge(m, sum, q.m, q.s);
            if (st_better(q.bs, q.bi, bs, bi)) { bs = q.bs; bi = q.bi; }
        }
        const bool masked = in_slot && y < 0;
        const double c = masked ? (sum > 0.0 ? 1.0 / sum : 0.0) : -1.0;
        const int32_t x = (bi == INT32_MAX) ? 0 : bi;  // every entry -inf: the smallest index
        const unsigned long long any = __ballot(masked);
        unsigned long long take = __ballot(masked && c > threshold);
        if (take == 0 && any != 0) {
            const double top = wave_max_f64(c);
            const unsigned long long tops = __ballot(masked && c == top);
            take = tops & (~tops + 1);  // the smallest slot of highest confidence
        }
        const int32_t commit = ((take >> lane) & 1ull) ? x : -1;
        if (in_slot) {
            st[n * block + lane] = y;
            cm[n * block + lane] = commit;
            if (commit_out) commit_out[row] = commit;
            if (conf_out) conf_out[row] = (float)c;
        }
        if (lane == 0) open[n] = any != 0;
    }
    __syncthreads();
    // 2. per node: does it equal its parent with the parent's commit applied?
    for (int n = w; n < n_nodes; n += kWalkWaves) {
        const int p = (n > 0) ? par[n] : -1;
        const bool valid = p >= 0 && p < n;  // parents come before their children
        bool eq = true;
        if (valid && in_slot) {
            const int32_t c = cm[p * block + lane];
            eq = st[n * block + lane] == (c >= 0 ? c : st[p * block + lane]);
        }
        const bool all = __ballot(!eq) == 0;
        if (lane == 0) match[n] = valid && all;
    }
    __syncthreads();
    // 3. the walk from the root (wave 0, lane = node)
    if (w == 0) {
        const bool in_node = lane < n_nodes;
        const int pn = (in_node && lane > 0) ? par[lane] : -1;
        const bool ok = in_node && lane > 0 && match[lane];
        int cur = 0, len = 0;
        for (; len < n_nodes - 1; ++len) {
            if (!open[cur]) break;  // a finished block commits nothing more
            const unsigned long long kids = __ballot(ok && pn == cur);
            if (!kids) break;
            cur = __ffsll((long long)kids) - 1;
            if (lane == 0) path[b * n_nodes + len + 1] = cur;
        }
        if (in_node && lane > len) path[b * n_nodes + lane] = -1;
        if (lane == 0) {
            path[b * n_nodes] = 0;
            path_len[b] = len;
        }
        if (in_slot) {
            const int32_t c = cm[cur * block + lane];
            next_state[b * block + lane] = c >= 0 ? c : st[cur * block + lane];
        }
    }
}

}  // namespace

StatesPlan states_plan(int batch, int n_nodes, int block, int64_t vocab) {
    StatesPlan p{};
    p.rows = (long long)batch * n_nodes * block;
    long long vs = (16384 + p.rows - 1) / p.rows;  // about 8 workgroups per CU slot
    long long cap = vocab / 16384;
    if (cap < 1) cap = 1;
    if (vs > cap) vs = cap;
    if (vs < 1) vs = 1;
    p.n_vsplit = (int)vs;
    p.ws_total = align_up((size_t)p.rows * p.n_vsplit * sizeof(SPart));
    return p;
}

hipError_t launch_states(const StatesPlan &p, const float *logits, const float *noise, const int32_t *parent,
                         const int32_t *state, int batch, int n_nodes, int block, int64_t vocab, float inv_t,
                         float threshold, int32_t *path_len, int32_t *path, int32_t *next_state, int32_t *commit,
                         float *conf, void *ws, hipStream_t st) {
    SPart *parts = (SPart *)ws;
    const long long n_tasks = p.rows * p.n_vsplit;
    const long long unit = 8LL * n_nodes;  // whole groups for every XCD
    const dim3 g1((unsigned)((n_tasks + unit - 1) / unit * unit));
    const bool vec = (vocab & 3) == 0, greedy = !(inv_t > 0.f);
    if (vec && greedy)
        hipLaunchKernelGGL((states_partial_kernel<true, true>), g1, dim3(256), 0, st, logits, noise, state, parts,
                           n_nodes, block, vocab, p.n_vsplit, n_tasks, inv_t);
    else if (vec) {
        constexpr int NC = 2;  // copies per workgroup sharing the noise loads
        const long long gsz = (n_nodes + NC - 1) / NC, n_tasks2 = n_tasks / n_nodes * gsz, unit2 = 8 * gsz;
        const dim3 g2((unsigned)((n_tasks2 + unit2 - 1) / unit2 * unit2));
        hipLaunchKernelGGL(states_partial_noise_kernel<NC>, g2, dim3(256), 0, st, logits, noise, state, parts,
                           n_nodes, block, vocab, p.n_vsplit, n_tasks2, inv_t);
    }
    else if (greedy)
        hipLaunchKernelGGL((states_partial_kernel<false, true>), g1, dim3(256), 0, st, logits, noise, state, parts,
                           n_nodes, block, vocab, p.n_vsplit, n_tasks, inv_t);
    else
        hipLaunchKernelGGL((states_partial_kernel<false, false>), g1, dim3(256), 0, st, logits, noise, state, parts,
                           n_nodes, block, vocab, p.n_vsplit, n_tasks, inv_t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(states_walk_kernel, dim3(batch), dim3(kWalkThreads), 0, st, parts, parent, state, n_nodes,
                       block, p.n_vsplit, (double)threshold, path_len, path, next_state, commit, conf);
    return hipGetLastError();
}

}  // namespace sv
