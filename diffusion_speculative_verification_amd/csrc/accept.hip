// accept.hip -- verification epilogue for gfx950 (MI355X).
//
// Method: "SimSD: Simple Speculative Decoding in Diffusion Language Models",
// 关键设计 4 (alpha_r = min(1, p_theta/p_phi) along the draft order, longest
// accepted prefix, in-place resample at the first rejection) and "S2D2: Fast
// Decoding for Diffusion LLMs via Training-Free Self-Speculation", 前置知识
// "推测解码" and 方法步骤 (5) (residual (P_target - P_draft)^+).
//
// Four launches on the caller's stream:
//   lse_partial_kernel  vocab-parallel softmax normaliser of every verified
//                       slot: a streaming pass over the float32 target logits
//                       (16-byte coalesced loads, 4 in flight per lane), per
//                       lane running (max, sum) with the sum kept in float64,
//                       merged per workgroup into one (m, s) partial per
//                       (slot, vocab split).  This pass moves almost all the
//                       bytes of the epilogue.
//   accept_scan_kernel  one wave per sequence: lane r merges the partials of
//                       the slot of draft step r+1, forms alpha in float64,
//                       the first rejection is found with one ballot; writes
//                       accept_len, alpha and the draft part of out_tokens.
//   residual_sums_kernel  (sequence, vocab chunk) workgroups form the residual
//                       and target mass of their chunk at the rejected slot;
//   residual_pick_kernel  one workgroup per sequence picks the chunk holding
//                       u * Z and rescans it for the token.  (Two launches:
//                       the kernel boundary orders the chunk sums; a
//                       last-workgroup handoff would need a device-scope
//                       release per workgroup, which writes back the L2.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct Part {   // normaliser partial of one (slot, vocab split)
    float m;    // max logit
    float pad;
    double s;   // sum exp(l - m)
};

struct ResInfo {  // rejected slot of one sequence
    int slot;     // -1: every step accepted, nothing to resample
    float m;      // merged max logit of that slot
    double s;     // merged sum exp(l - m)
};

template <bool VEC>
__global__ void __launch_bounds__(256) lse_partial_kernel(const float *__restrict__ logits,
                                                          const int32_t *__restrict__ tau, Part *parts,
                                                          int block, int gamma, int64_t vocab, int n_vsplit) {
    __shared__ float red_m[4];
    __shared__ double red_s[4];
    const int row = blockIdx.x / n_vsplit, sp = blockIdx.x % n_vsplit;
    if (tau[row] > gamma) return;  // slot not verified in this call
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float m = -INFINITY;
    double s = 0.0;
    if (VEC) {
        const int64_t n4 = vocab >> 2;
        const int64_t c0 = n4 * sp / n_vsplit, c1 = n4 * (sp + 1) / n_vsplit;
        const float4 *src = reinterpret_cast<const float4 *>(logits + (size_t)row * vocab);
        for (int64_t i = c0 + tid; i < c1; i += 256 * 4) {
            float4 x[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ok[u] = i + 256 * u < c1;
                x[u] = ok[u] ? src[i + 256 * u] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            }
            float gm = m;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                gm = fmaxf(gm, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
            if (gm > m) {
                if (m != -INFINITY) s *= (double)__builtin_amdgcn_exp2f((m - gm) * kLog2e);
                m = gm;
            }
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ps += __builtin_amdgcn_exp2f((x[u].x - m) * kLog2e);
                ps += __builtin_amdgcn_exp2f((x[u].y - m) * kLog2e);
                ps += __builtin_amdgcn_exp2f((x[u].z - m) * kLog2e);
                ps += __builtin_amdgcn_exp2f((x[u].w - m) * kLog2e);
            }
            s += (double)ps;
        }
    } else {
        const int64_t c0 = vocab * sp / n_vsplit, c1 = vocab * (sp + 1) / n_vsplit;
        const float *src = logits + (size_t)row * vocab;
        for (int64_t i = c0 + tid; i < c1; i += 256) {
            const float x = src[i];
            if (x > m) {
                if (m != -INFINITY) s *= (double)__builtin_amdgcn_exp2f((m - x) * kLog2e);
                m = x;
            }
            s += (double)__builtin_amdgcn_exp2f((x - m) * kLog2e);
        }
    }
    // workgroup merge
    const float M = wave_max(m);
    double sc = (m == -INFINITY) ? 0.0 : s * exp((double)m - (double)M);
    sc = wave_sum(sc);
    if (lane == 0) { red_m[w] = M; red_s[w] = sc; }
    __syncthreads();
    if (tid == 0) {
        float MM = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
        double SS = 0.0;
        for (int k = 0; k < 4; ++k)
            if (red_m[k] != -INFINITY) SS += red_s[k] * exp((double)red_m[k] - (double)MM);
        Part p;
        p.m = MM;
        p.pad = 0.f;
        p.s = SS;
        parts[(size_t)row * n_vsplit + sp] = p;
    }
}

__global__ void __launch_bounds__(64) accept_scan_kernel(
    const float *__restrict__ logits, const float *__restrict__ probs, const int32_t *__restrict__ tokens,
    const int32_t *__restrict__ tau, const float *__restrict__ u, const Part *__restrict__ parts,
    int block, int gamma, int64_t vocab, int n_vsplit, int32_t *accept_len, int32_t *out_tokens,
    float *alpha_out, ResInfo *res) {
    __shared__ int inv_s[64];
    __shared__ int tau_s[64];
    const int b = blockIdx.x, lane = threadIdx.x;
    inv_s[lane] = 0;  // tau is a permutation by contract; keep slot indices in range regardless
    __syncthreads();
    if (lane < block) {
        const int t = tau[(size_t)b * block + lane];
        tau_s[lane] = t;
        if (t >= 1 && t <= block) inv_s[t - 1] = lane;
    }
    __syncthreads();
    bool rejected = false;
    float M = 0.f;
    double S = 1.0;
    if (lane < gamma) {
        const int k = inv_s[lane];
        const size_t row = (size_t)b * block + k;
        M = -INFINITY;
        for (int i = 0; i < n_vsplit; ++i) M = fmaxf(M, parts[row * n_vsplit + i].m);
        S = 0.0;
        for (int i = 0; i < n_vsplit; ++i) {
            const Part p = parts[row * n_vsplit + i];
            if (p.m != -INFINITY) S += p.s * exp((double)p.m - (double)M);
        }
        const int x = tokens[row];
        double a = 0.0;  // out-of-range draft token: rejected
        if (x >= 0 && x < vocab) {
            const double pt = exp((double)logits[row * vocab + x] - (double)M) / S;
            const double pd = (double)probs[row * vocab + x];
            a = (pd > 0.0) ? fmin(1.0, pt / pd) : 1.0;
        }
        rejected = !((double)u[(size_t)b * (gamma + 1) + lane] < a);
        if (alpha_out) alpha_out[(size_t)b * gamma + lane] = (float)a;
    }
    const unsigned long long rej = __ballot(rejected);
    const int L = rej ? (__ffsll((long long)rej) - 1) : gamma;
    if (lane < block)
        out_tokens[(size_t)b * block + lane] = (tau_s[lane] <= L) ? tokens[(size_t)b * block + lane] : -1;
    if (lane == 0) {
        accept_len[b] = L;
        if (L == gamma) {
            ResInfo r;
            r.slot = -1;
            r.m = 0.f;
            r.s = 0.0;
            res[b] = r;
        }
    }
    if (L < gamma && lane == L) {
        ResInfo r;
        r.slot = inv_s[L];
        r.m = M;
        r.s = S;
        res[b] = r;
    }
}

// Mass of one vocab entry at the rejected slot: p_theta(v) (float32 exp of
// the logit against the merged max, scaled by the float64 reciprocal of the
// merged normaliser) and the residual max(0, p_theta(v) - p_phi(v)) formed in
// float64.
__device__ __forceinline__ void masses(float l, float pd, float m, double inv_s, double &r, double &pt) {
    pt = (double)__builtin_amdgcn_exp2f((l - m) * kLog2e) * inv_s;
    const double d = pt - (double)pd;
    r = d > 0.0 ? d : 0.0;
}

// Exclusive prefix sum over the 256 threads of a workgroup (thread order).
__device__ __forceinline__ double block_exclusive_scan(double v, double *wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    double inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    double base = 0.0;
    for (int k = 0; k < w; ++k) base += wave_tot[k];
    return base + inc - v;
}

constexpr int kResChunk = 2048;       // vocab entries per residual workgroup
constexpr int kResRun = kResChunk / 256;  // contiguous entries per thread in the pick scan
constexpr int kMaxChunks = 1024;          // vocab <= kResChunk * kMaxChunks = 2^21

// Residual pass 1: one workgroup per (sequence, vocab chunk) writes the
// residual and target mass of its chunk at the rejected slot.
template <bool VEC>
__global__ void __launch_bounds__(256) residual_sums_kernel(const float *__restrict__ logits,
                                                            const float *__restrict__ probs,
                                                            const ResInfo *__restrict__ res, double2 *chunk_sums,
                                                            int block, int64_t vocab, int n_chunk) {
    __shared__ double red_a[4], red_b[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x / n_chunk, c = blockIdx.x % n_chunk;
    const ResInfo ri = res[b];
    if (ri.slot < 0) return;
    const size_t row = (size_t)b * block + ri.slot;
    const float *lr = logits + row * vocab;
    const float *pr = probs + row * vocab;
    const double inv_s = 1.0 / ri.s;
    const int64_t v0 = (int64_t)c * kResChunk;
    const int n = (int)min((int64_t)kResChunk, vocab - v0);
    double ra = 0.0, pa = 0.0;
    if (VEC) {
        const float4 *l4 = reinterpret_cast<const float4 *>(lr + v0);
        const float4 *p4 = reinterpret_cast<const float4 *>(pr + v0);
        for (int i = tid; i < (n >> 2); i += 256) {
            const float4 a = l4[i], q = p4[i];
            double r, pt;
            masses(a.x, q.x, ri.m, inv_s, r, pt); ra += r; pa += pt;
            masses(a.y, q.y, ri.m, inv_s, r, pt); ra += r; pa += pt;
            masses(a.z, q.z, ri.m, inv_s, r, pt); ra += r; pa += pt;
            masses(a.w, q.w, ri.m, inv_s, r, pt); ra += r; pa += pt;
        }
    } else {
        for (int i = tid; i < n; i += 256) {
            double r, pt;
            masses(lr[v0 + i], pr[v0 + i], ri.m, inv_s, r, pt);
            ra += r;
            pa += pt;
        }
    }
    ra = wave_sum(ra);
    pa = wave_sum(pa);
    if (lane == 0) { red_a[w] = ra; red_b[w] = pa; }
    __syncthreads();
    if (tid == 0)
        chunk_sums[(size_t)b * n_chunk + c] =
            make_double2(red_a[0] + red_a[1] + red_a[2] + red_a[3], red_b[0] + red_b[1] + red_b[2] + red_b[3]);
}

// Residual pass 2: one workgroup per sequence picks the chunk whose running
// sum (ascending token order) crosses u * Z, then the token inside it.
__global__ void __launch_bounds__(256) residual_pick_kernel(const float *__restrict__ logits,
                                                            const float *__restrict__ probs,
                                                            const float *__restrict__ u,
                                                            const ResInfo *__restrict__ res,
                                                            const double2 *__restrict__ chunk_sums,
                                                            int32_t *out_tokens, int block, int gamma, int64_t vocab,
                                                            int n_chunk) {
    __shared__ double mass_s[256 * (kResRun + 1)];  // skewed: thread t's run starts at t * (kResRun + 1)
    __shared__ double csum_r[kMaxChunks], csum_t[kMaxChunks];
    __shared__ double wave_tot[4];
    __shared__ int sel_chunk, sel_use_t;
    __shared__ double sel_base, sel_thr;
    __shared__ int pick_first, pick_last;
    const int tid = threadIdx.x, b = blockIdx.x;
    const ResInfo ri = res[b];
    if (ri.slot < 0) return;
    const size_t row = (size_t)b * block + ri.slot;
    const float *lr = logits + row * vocab;
    const float *pr = probs + row * vocab;
    const double inv_s = 1.0 / ri.s;
    for (int k = tid; k < n_chunk; k += 256) {
        const double2 cs = chunk_sums[(size_t)b * n_chunk + k];
        csum_r[k] = cs.x;
        csum_t[k] = cs.y;
    }
    __syncthreads();
    if (tid == 0) {
        double Z = 0.0, T = 0.0;
        for (int k = 0; k < n_chunk; ++k) { Z += csum_r[k]; T += csum_t[k]; }
        const int use_t = !(Z > 0.0);
        const double *add_s = use_t ? csum_t : csum_r;
        const double tot = use_t ? T : Z;
        const double thr = (double)u[(size_t)b * (gamma + 1) + gamma] * tot;
        double run = 0.0, last_base = 0.0, base = 0.0;
        int pick = -1, last_pos = 0;
        for (int k = 0; k < n_chunk; ++k) {
            const double add = add_s[k];
            if (add > 0.0) { last_pos = k; last_base = run; }
            if (pick < 0 && run + add > thr) { pick = k; base = run; }
            run += add;
        }
        if (pick < 0) { pick = last_pos; base = last_base; }
        sel_chunk = pick;
        sel_base = base;
        sel_thr = thr;
        sel_use_t = use_t;
        pick_first = 0x7fffffff;
        pick_last = -1;
    }
    __syncthreads();
    // masses of the chosen chunk into LDS (coalesced), per-thread contiguous
    // runs, exclusive prefix over threads, walk the run that crosses u * Z
    const int cc = sel_chunk;
    const bool use_t = sel_use_t;
    const int64_t v0 = (int64_t)cc * kResChunk;
    const int n = (int)min((int64_t)kResChunk, vocab - v0);
    for (int i = tid; i < kResChunk; i += 256) {
        double mass = 0.0;
        if (i < n) {
            double r, pt;
            masses(lr[v0 + i], pr[v0 + i], ri.m, inv_s, r, pt);
            mass = use_t ? pt : r;
        }
        mass_s[(i / kResRun) * (kResRun + 1) + (i % kResRun)] = mass;
    }
    __syncthreads();
    const double *run_s = mass_s + tid * (kResRun + 1);
    double mine = 0.0;
    int lastpos = -1;
    for (int k = 0; k < kResRun; ++k) {
        mine += run_s[k];
        if (run_s[k] > 0.0) lastpos = tid * kResRun + k;
    }
    if (lastpos >= 0) atomicMax(&pick_last, lastpos);
    double run = sel_base + block_exclusive_scan(mine, wave_tot);
    if (run + mine > sel_thr) {
        for (int k = 0; k < kResRun; ++k) {
            run += run_s[k];
            if (run > sel_thr) { atomicMin(&pick_first, tid * kResRun + k); break; }
        }
    }
    __syncthreads();
    if (tid == 0) {
        const int loc = (pick_first != 0x7fffffff) ? pick_first : (pick_last >= 0 ? pick_last : 0);
        out_tokens[(size_t)b * block + ri.slot] = (int32_t)(v0 + loc);
    }
}

AcceptPlan accept_plan(int batch, int block, int gamma, int64_t vocab) {
    AcceptPlan p{};
    p.rows = batch * block;
    const long active = (long)batch * gamma;
    long vs = (2048 + active - 1) / active;
    long cap = vocab / 16384;
    if (cap < 1) cap = 1;
    if (vs > cap) vs = cap;
    if (vs < 1) vs = 1;
    p.n_vsplit = (int)vs;
    p.chunk = kResChunk;
    p.n_chunk = (int)((vocab + p.chunk - 1) / p.chunk);
    p.off_part = 0;
    p.off_res = p.off_part + align_up((size_t)p.rows * p.n_vsplit * sizeof(Part));
    p.off_chunk = p.off_res + align_up((size_t)batch * sizeof(ResInfo));
    p.ws_total = p.off_chunk + align_up((size_t)batch * p.n_chunk * sizeof(double2));
    return p;
}

hipError_t launch_accept(const AcceptPlan &p, const float *logits, const float *probs,
                         const int32_t *tokens, const int32_t *tau, const float *u, int batch,
                         int block, int gamma, int64_t vocab, int32_t *accept_len,
                         int32_t *out_tokens, float *alpha, void *ws, hipStream_t st) {
    char *base = (char *)ws;
    Part *parts = (Part *)(base + p.off_part);
    ResInfo *res = (ResInfo *)(base + p.off_res);
    double2 *chunks = (double2 *)(base + p.off_chunk);
    const unsigned g1 = (unsigned)((size_t)p.rows * p.n_vsplit);
    if ((vocab & 3) == 0)
        hipLaunchKernelGGL(lse_partial_kernel<true>, dim3(g1), dim3(256), 0, st, logits, tau, parts, block, gamma,
                           vocab, p.n_vsplit);
    else
        hipLaunchKernelGGL(lse_partial_kernel<false>, dim3(g1), dim3(256), 0, st, logits, tau, parts, block,
                           gamma, vocab, p.n_vsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_scan_kernel, dim3(batch), dim3(64), 0, st, logits, probs, tokens, tau, u, parts,
                       block, gamma, vocab, p.n_vsplit, accept_len, out_tokens, alpha, res);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g3((unsigned)((size_t)batch * p.n_chunk));
    if ((vocab & 3) == 0)
        hipLaunchKernelGGL(residual_sums_kernel<true>, g3, dim3(256), 0, st, logits, probs, res, chunks, block, vocab,
                           p.n_chunk);
    else
        hipLaunchKernelGGL(residual_sums_kernel<false>, g3, dim3(256), 0, st, logits, probs, res, chunks, block,
                           vocab, p.n_chunk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(residual_pick_kernel, dim3(batch), dim3(256), 0, st, logits, probs, u, res, chunks, out_tokens,
                       block, gamma, vocab, p.n_chunk);
    return hipGetLastError();
}

}  // namespace sv
