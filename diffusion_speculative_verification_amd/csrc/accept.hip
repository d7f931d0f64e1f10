// accept.hip -- verification epilogue for gfx950 (MI355X).
//
// Method: "SimSD: Simple Speculative Decoding in Diffusion Language Models",
// 关键设计 4 (alpha_r = min(1, p_theta/p_phi) along the draft order, longest
// accepted prefix, in-place resample at the first rejection) and "S2D2: Fast
// Decoding for Diffusion LLMs via Training-Free Self-Speculation", 前置知识
// "推测解码" and 方法步骤 (5) (residual (P_target - P_draft)^+).
//
// Three launches on the caller's stream:
//   lse_partial_kernel   vocab-parallel softmax normaliser of every verified
//                        slot: a streaming pass over the float32 target
//                        logits (16-byte coalesced non-temporal loads -- the
//                        logits are read once -- 4 in flight per lane),
//                        per-lane running (max, sum) with the sum kept
//                        in float64, merged per workgroup into one (m, s)
//                        partial per (slot, vocab split).  This pass moves
//                        almost all the bytes of the epilogue.
//   accept_resid_kernel  one workgroup per (sequence, vocab chunk): wave 0
//                        runs the acceptance scan of the sequence (lane r
//                        merges the partials of the slot of draft step r+1,
//                        alpha in float64, first rejection by one ballot);
//                        chunk 0 writes accept_len, alpha and the draft part
//                        of out_tokens; every workgroup then forms the
//                        residual and target mass of its chunk at the
//                        rejected slot.
//   residual_pick_kernel one workgroup per sequence: block scans over the
//                        chunk sums find the chunk holding u * Z, a second
//                        scan inside it finds the token.
// The kernel boundaries order the hand-offs: a last-workgroup hand-off
// inside one kernel would need a device-scope release per workgroup, which on
// this GPU writes back the L2.
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

// float4 as a clang vector type, for the non-temporal load builtin
typedef float nt_f4 __attribute__((ext_vector_type(4)));

constexpr int kResChunk = 2048;           // vocab entries per residual workgroup
constexpr int kResRun = kResChunk / 256;  // contiguous entries per thread in the pick scan
constexpr int kMaxChunks = 1024;          // vocab <= kResChunk * kMaxChunks = 2^21

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
                if (ok[u]) {
                    const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4 *>(src + i + 256 * u));
                    x[u] = make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    x[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                }
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
// Contains a workgroup barrier; wave_tot is 4 doubles of LDS.
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
    __syncthreads();  // wave_tot may be reused by the caller
    return base + inc - v;
}

// Acceptance scan of one sequence, run by one wave (SimSD 关键设计 4): lane r
// merges the normaliser partials of the slot verified at draft step r+1,
// forms alpha in float64 and tests u[r] < alpha; one ballot gives the first
// rejection.  Returns L (number of leading accepts); *slot/*m_out/*s_out
// describe the rejected slot (slot -1 when L == gamma).
__device__ __forceinline__ int acceptance_scan(const float *__restrict__ logits, const float *__restrict__ probs,
                                               const int32_t *__restrict__ tokens, const float *__restrict__ u,
                                               const Part *__restrict__ parts, const int *inv_s, int b, int block,
                                               int gamma, int64_t vocab, int n_vsplit, double *alpha_lane,
                                               int *slot, float *m_out, double *s_out) {
    const int lane = threadIdx.x & 63;
    bool rejected = false;
    float M = 0.f;
    double S = 1.0, a = 0.0;
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
        if (x >= 0 && x < vocab) {  // an out-of-range draft token is rejected (alpha = 0)
            const double pt = exp((double)logits[row * vocab + x] - (double)M) / S;
            const double pd = (double)probs[row * vocab + x];
            a = (pd > 0.0) ? fmin(1.0, pt / pd) : 1.0;
        }
        rejected = !((double)u[(size_t)b * (gamma + 1) + lane] < a);
    }
    *alpha_lane = a;
    const unsigned long long rej = __ballot(rejected);
    const int L = rej ? (__ffsll((long long)rej) - 1) : gamma;
    const int src = L < gamma ? L : 0;
    *slot = L < gamma ? inv_s[L] : -1;
    *m_out = __shfl(M, src);
    *s_out = __shfl(S, src);
    return L;
}

// Acceptance + residual mass, one workgroup per (sequence, vocab chunk).
// Every workgroup of a sequence repeats the (small) acceptance scan; chunk 0
// writes accept_len, alpha, the draft part of out_tokens and the rejected
// slot's normaliser for the pick kernel.  If a step was rejected, each
// workgroup then forms the residual and target mass of its vocab chunk at
// the rejected slot.
template <bool VEC>
__global__ void __launch_bounds__(256) accept_resid_kernel(
    const float *__restrict__ logits, const float *__restrict__ probs, const int32_t *__restrict__ tokens,
    const int32_t *__restrict__ tau, const float *__restrict__ u, const Part *__restrict__ parts, int block,
    int gamma, int64_t vocab, int n_vsplit, int n_chunk, int32_t *accept_len, int32_t *out_tokens,
    float *alpha_out, ResInfo *res, double2 *chunk_sums) {
    __shared__ int inv_s[64];
    __shared__ int tau_s[64];
    __shared__ int slot_s;
    __shared__ float m_s;
    __shared__ double s_s;
    __shared__ double red_a[4], red_b[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x / n_chunk, c = blockIdx.x % n_chunk;
    if (tid < 64) inv_s[tid] = 0;  // tau is a permutation by contract; keep slot indices in range regardless
    __syncthreads();
    if (tid < block) {
        const int t = tau[(size_t)b * block + tid];
        tau_s[tid] = t;
        if (t >= 1 && t <= block) inv_s[t - 1] = tid;
    }
    __syncthreads();
    if (w == 0) {
        double a, S;
        int slot;
        float M;
        const int L = acceptance_scan(logits, probs, tokens, u, parts, inv_s, b, block, gamma, vocab, n_vsplit, &a,
                                      &slot, &M, &S);
        if (c == 0) {
            if (lane < gamma && alpha_out) alpha_out[(size_t)b * gamma + lane] = (float)a;
            if (lane < block)
                out_tokens[(size_t)b * block + lane] = (tau_s[lane] <= L) ? tokens[(size_t)b * block + lane] : -1;
            if (lane == 0) {
                accept_len[b] = L;
                ResInfo r;
                r.slot = slot;
                r.m = M;
                r.s = S;
                res[b] = r;
            }
        }
        if (lane == 0) { slot_s = slot; m_s = M; s_s = S; }
    }
    __syncthreads();
    const int slot = slot_s;
    if (slot < 0) return;
    const float M = m_s;
    const double inv_sum = 1.0 / s_s;
    const size_t row = (size_t)b * block + slot;
    const float *lr = logits + row * vocab;
    const float *pr = probs + row * vocab;
    const int64_t v0 = (int64_t)c * kResChunk;
    const int n = (int)min((int64_t)kResChunk, vocab - v0);
    double ra = 0.0, pa = 0.0;
    if (VEC) {
        const float4 *l4 = reinterpret_cast<const float4 *>(lr + v0);
        const float4 *p4 = reinterpret_cast<const float4 *>(pr + v0);
        for (int i = tid; i < (n >> 2); i += 256) {
            const float4 x = l4[i], q = p4[i];
            double r, pt;
            masses(x.x, q.x, M, inv_sum, r, pt); ra += r; pa += pt;
            masses(x.y, q.y, M, inv_sum, r, pt); ra += r; pa += pt;
            masses(x.z, q.z, M, inv_sum, r, pt); ra += r; pa += pt;
            masses(x.w, q.w, M, inv_sum, r, pt); ra += r; pa += pt;
        }
    } else {
        for (int i = tid; i < n; i += 256) {
            double r, pt;
            masses(lr[v0 + i], pr[v0 + i], M, inv_sum, r, pt);
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

// Residual pick: one workgroup per sequence finds the chunk whose running sum
// (ascending token order) crosses u * Z, then the token inside it.  Z is the
// residual mass; when it is zero the target distribution is sampled instead.
// If rounding leaves no crossing, the last entry with positive mass is taken.
__global__ void __launch_bounds__(256) residual_pick_kernel(const float *__restrict__ logits,
                                                            const float *__restrict__ probs,
                                                            const float *__restrict__ u,
                                                            const ResInfo *__restrict__ res,
                                                            const double2 *__restrict__ chunk_sums,
                                                            int32_t *out_tokens, int block, int gamma, int64_t vocab,
                                                            int n_chunk) {
    constexpr int CPT = kMaxChunks / 256;  // chunks per thread
    __shared__ double wave_tot[4];
    __shared__ double tot_s[2];
    __shared__ int sel_chunk;
    __shared__ double sel_base;
    __shared__ int pick_first, pick_last, last_chunk;
    const int tid = threadIdx.x, b = blockIdx.x;
    const ResInfo ri = res[b];
    if (ri.slot < 0) return;
    // thread t owns chunks [t * CPT, t * CPT + CPT)
    double cr[CPT], ct[CPT], my_r = 0.0, my_t = 0.0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int ch = tid * CPT + k;
        const double2 v = ch < n_chunk ? chunk_sums[(size_t)b * n_chunk + ch] : make_double2(0.0, 0.0);
        cr[k] = v.x;
        ct[k] = v.y;
        my_r += v.x;
        my_t += v.y;
    }
    if (tid == 0) { pick_first = 0x7fffffff; pick_last = -1; last_chunk = -1; sel_chunk = 0x7fffffff; sel_base = 0.0; }
    const double ex_r = block_exclusive_scan(my_r, wave_tot);
    const double ex_t = block_exclusive_scan(my_t, wave_tot);
    if (tid == 255) { tot_s[0] = ex_r + my_r; tot_s[1] = ex_t + my_t; }
    __syncthreads();
    const bool use_t = !(tot_s[0] > 0.0);
    const double tot = use_t ? tot_s[1] : tot_s[0];
    const double thr = (double)u[(size_t)b * (gamma + 1) + gamma] * tot;
    // each thread proposes the first of its chunks where the running sum
    // crosses u * Z; the smallest proposal wins and its owner publishes the
    // running sum before it
    int last = -1, cand = 0x7fffffff;
    double last_base = 0.0, cand_base = 0.0;
    {
        double run = use_t ? ex_t : ex_r;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const double add = use_t ? ct[k] : cr[k];
            if (add > 0.0) { last = tid * CPT + k; last_base = run; }
            if (cand == 0x7fffffff && run <= thr && run + add > thr) { cand = tid * CPT + k; cand_base = run; }
            run += add;
        }
        if (cand != 0x7fffffff) atomicMin(&sel_chunk, cand);
        if (last >= 0) atomicMax(&last_chunk, last);
    }
    __syncthreads();
    if (sel_chunk == 0x7fffffff) {  // rounding left no crossing: the last chunk with mass
        if (last >= 0 && last == last_chunk) { sel_chunk = last; sel_base = last_base; }
    } else if (cand == sel_chunk) {
        sel_base = cand_base;
    }
    __syncthreads();
    // the chosen chunk: thread t takes kResRun contiguous entries
    const int cc = (sel_chunk == 0x7fffffff) ? 0 : sel_chunk;
    const double base = sel_base;
    const int64_t v0 = (int64_t)cc * kResChunk;
    const int n = (int)min((int64_t)kResChunk, vocab - v0);
    const size_t row = (size_t)b * block + ri.slot;
    const float *lr = logits + row * vocab + v0;
    const float *pr = probs + row * vocab + v0;
    const double inv_sum = 1.0 / ri.s;
    double mass[kResRun], mine = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int k = 0; k < kResRun; ++k) {
        const int i = tid * kResRun + k;
        double r = 0.0, pt = 0.0;
        if (i < n) masses(lr[i], pr[i], ri.m, inv_sum, r, pt);
        mass[k] = use_t ? pt : r;
        mine += mass[k];
        if (mass[k] > 0.0) lastpos = i;
    }
    if (lastpos >= 0) atomicMax(&pick_last, lastpos);
    double run = base + block_exclusive_scan(mine, wave_tot);
    if (run <= thr && run + mine > thr) {
#pragma unroll
        for (int k = 0; k < kResRun; ++k) {
            run += mass[k];
            if (run > thr) { atomicMin(&pick_first, tid * kResRun + k); break; }
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
    const dim3 g2((unsigned)((size_t)batch * p.n_chunk));
    if ((vocab & 3) == 0)
        hipLaunchKernelGGL(accept_resid_kernel<true>, g2, dim3(256), 0, st, logits, probs, tokens, tau, u, parts, block,
                           gamma, vocab, p.n_vsplit, p.n_chunk, accept_len, out_tokens, alpha, res, chunks);
    else
        hipLaunchKernelGGL(accept_resid_kernel<false>, g2, dim3(256), 0, st, logits, probs, tokens, tau, u, parts,
                           block, gamma, vocab, p.n_vsplit, p.n_chunk, accept_len, out_tokens, alpha, res, chunks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(residual_pick_kernel, dim3(batch), dim3(256), 0, st, logits, probs, u, res, chunks, out_tokens,
                       block, gamma, vocab, p.n_chunk);
    return hipGetLastError();
}

}  // namespace sv
