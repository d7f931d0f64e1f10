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
//                        logits are read once -- 8 in flight per lane),
//                        per-lane running (max, sum) with the sum kept
//                        in float64, merged per workgroup into one (m, s)
//                        partial per (slot, vocab split).  The first split of
//                        each slot also gathers the target logit and draft
//                        probability of the slot's draft token, issued
//                        beside its first stream loads.  This pass moves
//                        almost all the bytes of the epilogue.
//   accept_resid_kernel  one workgroup per (sequence, vocab chunk): wave 0
//                        runs the acceptance scan of the sequence with lane k
//                        on slot k (every operand it needs is loaded in one
//                        round trip: labels, tokens, uniforms, partials,
//                        gathers); alpha in float64, the first rejection in
//                        draft order is a wave minimum over the rejected
//                        steps.  Chunk 0 writes accept_len, alpha and the
//                        draft part of out_tokens; every workgroup then forms
//                        the residual and target mass of its chunk at the
//                        rejected slot.
//   residual_pick_kernel one workgroup per sequence: block scans over the
//                        chunk sums find the chunk holding u * Z, a second
//                        scan inside it finds the token.
// At temperature T every target logit is tempered as it is loaded: l * (1/T),
// the product rounded to float32 (1/T rounded to float32 once, on the host);
// T = 1 multiplies by 1.0f and leaves every value unchanged.
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

struct Gath {  // draft token of one slot, gathered during the normaliser pass
    float l;    // target logit of the draft token
    float p;    // draft probability of the draft token
    int ok;     // 0: the draft token lies outside [0, vocab)
    int pad;
};

struct ResInfo {  // rejected slot of one sequence
    int slot;     // -1: every step accepted, nothing to resample
    float m;      // merged max logit of that slot
    double s;     // merged sum exp(l - m)
};

// float4 as a clang vector type, for the non-temporal load builtin
typedef float nt_f4 __attribute__((ext_vector_type(4)));

constexpr int kResChunk = 4096;             // vocab entries per residual workgroup
constexpr int kPickChunk = kResChunk / 2;   // vocab entries per published chunk sum
constexpr int kPickRun = kPickChunk / 256;  // contiguous entries per thread in the pick scan
constexpr int kMaxChunks = 1024;            // vocab <= kPickChunk * kMaxChunks = 2^21

// temper(x): x * inv_t rounded to float32 in the tempered instantiation,
// x itself at T = 1 (where the product is the identity).
template <bool TEMP>
__device__ __forceinline__ float temper(float x, float inv_t) {
    return TEMP ? __fmul_rn(x, inv_t) : x;
}

template <bool VEC, bool TEMP>
__global__ void __launch_bounds__(256) lse_partial_kernel(const float *__restrict__ logits,
                                                          const float *__restrict__ probs,
                                                          const int32_t *__restrict__ tokens,
                                                          const int32_t *__restrict__ tau, Part *parts, Gath *gath,
                                                          int block, int gamma, int64_t vocab, int n_vsplit,
                                                          float inv_t) {
    __shared__ float red_m[4];
    __shared__ double red_s[4];
    const int row = blockIdx.x / n_vsplit, sp = blockIdx.x % n_vsplit;
    const bool gatherer = sp == 0 && threadIdx.x == 0;
    const int t = tau[row];
    const int x = gatherer ? tokens[row] : -1;
    if (t > gamma) return;  // slot not verified in this call
    // the draft-token gather; its loads travel with the first stream loads
    Gath g{0.f, 0.f, 0, 0};
    if (gatherer && x >= 0 && x < vocab) {
        g.l = temper<TEMP>(logits[(size_t)row * vocab + x], inv_t);
        g.p = probs[(size_t)row * vocab + x];
        g.ok = 1;
    }
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float m = -INFINITY;
    double s = 0.0;
    if (VEC) {
        const int64_t n4 = vocab >> 2;
        const int64_t c0 = n4 * sp / n_vsplit, c1 = n4 * (sp + 1) / n_vsplit;
        const float4 *src = reinterpret_cast<const float4 *>(logits + (size_t)row * vocab);
        // 8 loads in flight per lane: the small and long-prompt workloads
        // (few slots) are bound by dependent load rounds, which this halves
        constexpr int U = 8;
        for (int64_t i = c0 + tid; i < c1; i += 256 * U) {
            float4 x[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ok[u] = i + 256 * u < c1;
                if (ok[u]) {
                    const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4 *>(src + i + 256 * u));
                    x[u] = make_float4(temper<TEMP>(v[0], inv_t), temper<TEMP>(v[1], inv_t),
                                       temper<TEMP>(v[2], inv_t), temper<TEMP>(v[3], inv_t));
                } else {
                    x[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                }
            }
            float gm = m;
#pragma unroll
            for (int u = 0; u < U; ++u)
                gm = fmaxf(gm, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
            if (gm > m) {
                if (m != -INFINITY) s *= (double)__builtin_amdgcn_exp2f((m - gm) * kLog2e);
                m = gm;
            }
            // while every entry so far is -inf (masked logits), m is -inf
            // and so are the entries of this round: subtracting 0 instead
            // keeps exp(-inf - m) at 0 rather than NaN
            const float mu = (m == -INFINITY) ? 0.f : m;
            // float32 partial sums of 16 terms each, added in float64
            float ps[U / 4] = {};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ps[u / 4] += __builtin_amdgcn_exp2f((x[u].x - mu) * kLog2e);
                ps[u / 4] += __builtin_amdgcn_exp2f((x[u].y - mu) * kLog2e);
                ps[u / 4] += __builtin_amdgcn_exp2f((x[u].z - mu) * kLog2e);
                ps[u / 4] += __builtin_amdgcn_exp2f((x[u].w - mu) * kLog2e);
            }
#pragma unroll
            for (int k = 0; k < U / 4; ++k) s += (double)ps[k];
        }
    } else {
        const int64_t c0 = vocab * sp / n_vsplit, c1 = vocab * (sp + 1) / n_vsplit;
        const float *src = logits + (size_t)row * vocab;
        for (int64_t i = c0 + tid; i < c1; i += 256) {
            const float x = temper<TEMP>(src[i], inv_t);
            if (x > m) {
                if (m != -INFINITY) s *= (double)__builtin_amdgcn_exp2f((m - x) * kLog2e);
                m = x;
            }
            s += (double)__builtin_amdgcn_exp2f((x - ((m == -INFINITY) ? 0.f : m)) * kLog2e);
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
        if (sp == 0) gath[row] = g;
    }
}

// Mass of one vocab entry at the rejected slot: p_theta(v) (float32 exp of
// the tempered logit against the merged max, scaled by the float64
// reciprocal of the merged normaliser) and the residual max(0, p_theta(v) -
// p_phi(v)) formed in float64.
__device__ __forceinline__ void masses(float l, float pd, float m, double inv_s, float inv_t, double &r,
                                       double &pt) {
    pt = (double)__builtin_amdgcn_exp2f((__fmul_rn(l, inv_t) - m) * kLog2e) * inv_s;
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

// The same for a pair of sums at once (both components scanned in the same
// order, so each equals block_exclusive_scan of that component alone).
__device__ __forceinline__ double2 block_exclusive_scan2(double2 v, double2 *wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    double2 inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double tx = __shfl_up(inc.x, o), ty = __shfl_up(inc.y, o);
        if (lane >= o) { inc.x += tx; inc.y += ty; }
    }
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    double bx = 0.0, by = 0.0;
    for (int k = 0; k < w; ++k) { bx += wave_tot[k].x; by += wave_tot[k].y; }
    __syncthreads();  // wave_tot may be reused by the caller
    return make_double2(bx + inc.x - v.x, by + inc.y - v.y);
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

// Acceptance scan of one sequence, run by one wave (SimSD 关键设计 4).  Lane
// k takes slot k: it merges the slot's normaliser partials (max first, then
// the rescaled sums, float64), forms alpha = min(1, p_theta(x)/p_phi(x)) of
// its draft token in float64 and tests the uniform of its draft step
// tau(k).  The first rejection in draft order is the smallest rejected step.
// Returns L (number of leading accepts); *slot/*m_out/*s_out describe the
// rejected slot (slot -1 when L == gamma).  *alpha_lane, *step and *token
// are lane k's alpha, label and draft token.
__device__ __forceinline__ int acceptance_scan(const int32_t *__restrict__ tokens, const int32_t *__restrict__ tau,
                                               const float *__restrict__ u, const Part *__restrict__ parts,
                                               const Gath *__restrict__ gath, int b, int block, int gamma,
                                               int n_vsplit, double *alpha_lane, int *step, int *token, int *slot,
                                               float *m_out, double *s_out) {
    const int lane = threadIdx.x & 63;
    const bool in = lane < block;
    const size_t row = (size_t)b * block + (in ? lane : 0);
    // one round trip: every load below is independent of the others
    const int t = in ? tau[row] : 0;
    const int x = in ? tokens[row] : -1;
    const float ul = lane < gamma ? u[(size_t)b * (gamma + 1) + lane] : 1.f;
    const Gath g = in ? gath[row] : Gath{0.f, 0.f, 0, 0};
    float M = -INFINITY;
    double S = 0.0;
    if (in) {
#pragma unroll 4
        for (int i = 0; i < n_vsplit; ++i) M = fmaxf(M, parts[row * n_vsplit + i].m);
#pragma unroll 4
        for (int i = 0; i < n_vsplit; ++i) {
            const Part p = parts[row * n_vsplit + i];
            if (p.m != -INFINITY) S += p.s * exp((double)p.m - (double)M);
        }
    }
    const bool ver = in && t >= 1 && t <= gamma;  // slot verified at draft step t
    double a = 0.0;
    if (ver && g.ok) {  // an out-of-range draft token is rejected (alpha = 0)
        const double pt = exp((double)g.l - (double)M) / S;
        const double pd = (double)g.p;
        // a row without a finite logit has no target distribution: its
        // NaN ratio survives the clamp (fmin would turn it into 1) and the
        // test u < alpha below rejects the step
        a = (pd > 0.0) ? pt / pd : 1.0;
        if (a > 1.0) a = 1.0;
    }
    const float ur = __shfl(ul, ver ? t - 1 : 0);  // uniform of draft step t
    const bool rejected = ver && !((double)ur < a);
    const int L = wave_min_int(rejected ? t - 1 : gamma);
    const unsigned long long at = __ballot(rejected && t - 1 == L);
    const int src = at ? (__ffsll((long long)at) - 1) : 0;
    *slot = L < gamma ? src : -1;
    *m_out = __shfl(M, src);
    *s_out = __shfl(S, src);
    *alpha_lane = a;
    *step = t;
    *token = x;
    return L;
}

// Acceptance + residual mass, one workgroup per (sequence, vocab chunk of
// kResChunk entries); the masses are published per half chunk.
// Every workgroup of a sequence repeats the (small) acceptance scan; chunk 0
// writes accept_len, alpha, the draft part of out_tokens and the rejected
// slot's normaliser for the pick kernel.  If a step was rejected, each
// workgroup then forms the residual and target mass of its vocab chunk at
// the rejected slot.
template <bool VEC>
__global__ void __launch_bounds__(256) accept_resid_kernel(
    const float *__restrict__ logits, const float *__restrict__ probs, const int32_t *__restrict__ tokens,
    const int32_t *__restrict__ tau, const float *__restrict__ u, const Part *__restrict__ parts,
    const Gath *__restrict__ gath, int block, int gamma, int64_t vocab, int n_vsplit, int n_chunk, int n_pick,
    float inv_t, int32_t *accept_len, int32_t *out_tokens, float *alpha_out, ResInfo *res, double2 *chunk_sums) {
    __shared__ int slot_s;
    __shared__ float m_s;
    __shared__ double s_s;
    __shared__ double red_a[2][4], red_b[2][4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x / n_chunk, c = blockIdx.x % n_chunk;
    if (w == 0) {
        double a, S;
        int slot, t, x;
        float M;
        const int L = acceptance_scan(tokens, tau, u, parts, gath, b, block, gamma, n_vsplit, &a, &t, &x, &slot,
                                      &M, &S);
        if (c == 0) {
            if (lane < block) {
                if (alpha_out && t >= 1 && t <= gamma) alpha_out[(size_t)b * gamma + t - 1] = (float)a;
                out_tokens[(size_t)b * block + lane] = (t <= L) ? x : -1;
            }
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
    // sums per half chunk (kPickChunk entries each): h = 0 first half, 1 second
    double ra[2] = {0.0, 0.0}, pa[2] = {0.0, 0.0};
    if (VEC) {
        // all loads of the chunk in flight before any use; float4 k of a
        // thread lies in half k / 2
        constexpr int U = kResChunk / 1024;
        const int n4 = n >> 2;
        const float4 *l4 = reinterpret_cast<const float4 *>(lr + v0);
        const float4 *p4 = reinterpret_cast<const float4 *>(pr + v0);
        float4 xl[U], xp[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int i = tid + 256 * k;
            xl[k] = i < n4 ? l4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            xp[k] = i < n4 ? p4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (tid + 256 * k >= n4) continue;
            const int h = k / (U / 2);
            double r, pt;
            masses(xl[k].x, xp[k].x, M, inv_sum, inv_t, r, pt); ra[h] += r; pa[h] += pt;
            masses(xl[k].y, xp[k].y, M, inv_sum, inv_t, r, pt); ra[h] += r; pa[h] += pt;
            masses(xl[k].z, xp[k].z, M, inv_sum, inv_t, r, pt); ra[h] += r; pa[h] += pt;
            masses(xl[k].w, xp[k].w, M, inv_sum, inv_t, r, pt); ra[h] += r; pa[h] += pt;
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll 4
            for (int i = h * kPickChunk + tid; i < min(n, (h + 1) * kPickChunk); i += 256) {
                double r, pt;
                masses(lr[v0 + i], pr[v0 + i], M, inv_sum, inv_t, r, pt);
                ra[h] += r;
                pa[h] += pt;
            }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ra[h] = wave_sum(ra[h]);
        pa[h] = wave_sum(pa[h]);
        if (lane == 0) { red_a[h][w] = ra[h]; red_b[h][w] = pa[h]; }
    }
    __syncthreads();
    if (tid < 2 && 2 * c + tid < n_pick)
        chunk_sums[(size_t)b * n_pick + 2 * c + tid] =
            make_double2(red_a[tid][0] + red_a[tid][1] + red_a[tid][2] + red_a[tid][3],
                         red_b[tid][0] + red_b[tid][1] + red_b[tid][2] + red_b[tid][3]);
}

// Residual pick: one workgroup per sequence finds the chunk whose running sum
// (ascending token order) crosses u * Z, then the token inside it.  Z is the
// residual mass; when it is zero the target distribution is sampled instead.
// If rounding leaves no crossing, the last entry with positive mass is taken.
// VEC (vocab a multiple of 4): the chunk's entries arrive as 16-byte loads.
template <bool VEC>
__global__ void __launch_bounds__(256) residual_pick_kernel(const float *__restrict__ logits,
                                                            const float *__restrict__ probs,
                                                            const float *__restrict__ u,
                                                            const ResInfo *__restrict__ res,
                                                            const double2 *__restrict__ chunk_sums,
                                                            int32_t *out_tokens, int block, int gamma, int64_t vocab,
                                                            int n_chunk, float inv_t) {
    constexpr int CPT = kMaxChunks / 256;  // chunks per thread
    __shared__ double wave_tot[4];
    __shared__ double2 wave_tot2[4];
    __shared__ double tot_s[2];
    __shared__ int sel_chunk;
    __shared__ double sel_base;
    __shared__ int pick_first, pick_last, last_chunk;
    const int tid = threadIdx.x, b = blockIdx.x;
    // thread t owns chunks [t * CPT, t * CPT + CPT); the chunk sums are loaded
    // beside the sequence's ResInfo (workspace memory, read before the
    // early exit so both loads share one round trip)
    double2 v[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int ch = tid * CPT + k;
        v[k] = ch < n_chunk ? chunk_sums[(size_t)b * n_chunk + ch] : make_double2(0.0, 0.0);
    }
    const ResInfo ri = res[b];
    if (ri.slot < 0) return;
    double cr[CPT], ct[CPT], my_r = 0.0, my_t = 0.0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        cr[k] = v[k].x;
        ct[k] = v[k].y;
        my_r += v[k].x;
        my_t += v[k].y;
    }
    if (tid == 0) { pick_first = 0x7fffffff; pick_last = -1; last_chunk = -1; sel_chunk = 0x7fffffff; sel_base = 0.0; }
    const double2 ex = block_exclusive_scan2(make_double2(my_r, my_t), wave_tot2);
    const double ex_r = ex.x, ex_t = ex.y;
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
    // the chosen chunk: thread t takes kPickRun contiguous entries
    const int cc = (sel_chunk == 0x7fffffff) ? 0 : sel_chunk;
    const double base = sel_base;
    const int64_t v0 = (int64_t)cc * kPickChunk;
    const int n = (int)min((int64_t)kPickChunk, vocab - v0);
    const size_t row = (size_t)b * block + ri.slot;
    const float *lr = logits + row * vocab + v0;
    const float *pr = probs + row * vocab + v0;
    const double inv_sum = 1.0 / ri.s;
    float xl[kPickRun], xp[kPickRun];
    if (VEC) {
        // n and the chunk start are multiples of 4: whole float4 or nothing
        static_assert(kPickRun % 4 == 0, "float4 runs");
#pragma unroll
        for (int q = 0; q < kPickRun / 4; ++q) {  // every load in flight before any use
            const int i = tid * kPickRun + 4 * q;
            const float4 a4 = i < n ? *reinterpret_cast<const float4 *>(lr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 p4 = i < n ? *reinterpret_cast<const float4 *>(pr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
            xl[4 * q] = a4.x; xl[4 * q + 1] = a4.y; xl[4 * q + 2] = a4.z; xl[4 * q + 3] = a4.w;
            xp[4 * q] = p4.x; xp[4 * q + 1] = p4.y; xp[4 * q + 2] = p4.z; xp[4 * q + 3] = p4.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kPickRun; ++k) {  // every load in flight before any use
            const int i = tid * kPickRun + k;
            xl[k] = i < n ? lr[i] : 0.f;
            xp[k] = i < n ? pr[i] : 0.f;
        }
    }
    double mass[kPickRun], mine = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int k = 0; k < kPickRun; ++k) {
        const int i = tid * kPickRun + k;
        double r = 0.0, pt = 0.0;
        if (i < n) masses(xl[k], xp[k], ri.m, inv_sum, inv_t, r, pt);
        mass[k] = use_t ? pt : r;
        mine += mass[k];
        if (mass[k] > 0.0) lastpos = i;
    }
    if (lastpos >= 0) atomicMax(&pick_last, lastpos);
    double run = base + block_exclusive_scan(mine, wave_tot);
    if (run <= thr && run + mine > thr) {
#pragma unroll
        for (int k = 0; k < kPickRun; ++k) {
            run += mass[k];
            if (run > thr) { atomicMin(&pick_first, tid * kPickRun + k); break; }
        }
    }
    __syncthreads();
    if (tid == 0) {
        const int loc = (pick_first != 0x7fffffff) ? pick_first : (pick_last >= 0 ? pick_last : 0);
        out_tokens[(size_t)b * block + ri.slot] = (int32_t)(v0 + loc);
    }
}

// Vocabulary parts per verified row: enough for about 2048 workgroups, but
// no part shorter than 32768 entries (at vocabulary 151936: at most 4
// parts; with 9 parts of 16384 the 128-row workloads ran their accept call
// ~2 us slower, 31.5 vs 29.4 us and 29.9 vs 27.9 us, the headline equal).
AcceptPlan accept_plan(int batch, int block, int gamma, int64_t vocab) {
    AcceptPlan p{};
    p.rows = batch * block;
    const long active = (long)batch * gamma;
    long vs = (2048 + active - 1) / active;
    long cap = vocab / 32768;
    if (cap < 1) cap = 1;
    if (vs > cap) vs = cap;
    if (vs < 1) vs = 1;
    p.n_vsplit = (int)vs;
    p.chunk = kResChunk;
    p.n_chunk = (int)((vocab + p.chunk - 1) / p.chunk);
    p.n_pick = (int)((vocab + kPickChunk - 1) / kPickChunk);
    p.off_part = 0;
    p.off_gath = p.off_part + align_up((size_t)p.rows * p.n_vsplit * sizeof(Part));
    p.off_res = p.off_gath + align_up((size_t)p.rows * sizeof(Gath));
    p.off_chunk = p.off_res + align_up((size_t)batch * sizeof(ResInfo));
    p.ws_total = p.off_chunk + align_up((size_t)batch * p.n_pick * sizeof(double2));
    return p;
}

hipError_t launch_accept(const AcceptPlan &p, const float *logits, const float *probs,
                         const int32_t *tokens, const int32_t *tau, const float *u, int batch,
                         int block, int gamma, int64_t vocab, float inv_t, int32_t *accept_len,
                         int32_t *out_tokens, float *alpha, void *ws, hipStream_t st) {
    char *base = (char *)ws;
    Part *parts = (Part *)(base + p.off_part);
    Gath *gath = (Gath *)(base + p.off_gath);
    ResInfo *res = (ResInfo *)(base + p.off_res);
    double2 *chunks = (double2 *)(base + p.off_chunk);
    const unsigned g1 = (unsigned)((size_t)p.rows * p.n_vsplit);
    const bool vec = (vocab & 3) == 0, temp = inv_t != 1.0f;
    if (vec && !temp)
        hipLaunchKernelGGL((lse_partial_kernel<true, false>), dim3(g1), dim3(256), 0, st, logits, probs, tokens, tau,
                           parts, gath, block, gamma, vocab, p.n_vsplit, inv_t);
    else if (vec)
        hipLaunchKernelGGL((lse_partial_kernel<true, true>), dim3(g1), dim3(256), 0, st, logits, probs, tokens, tau,
                           parts, gath, block, gamma, vocab, p.n_vsplit, inv_t);
    else if (!temp)
        hipLaunchKernelGGL((lse_partial_kernel<false, false>), dim3(g1), dim3(256), 0, st, logits, probs, tokens,
                           tau, parts, gath, block, gamma, vocab, p.n_vsplit, inv_t);
    else
        hipLaunchKernelGGL((lse_partial_kernel<false, true>), dim3(g1), dim3(256), 0, st, logits, probs, tokens,
                           tau, parts, gath, block, gamma, vocab, p.n_vsplit, inv_t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((size_t)batch * p.n_chunk));
    if ((vocab & 3) == 0)
        hipLaunchKernelGGL(accept_resid_kernel<true>, g2, dim3(256), 0, st, logits, probs, tokens, tau, u, parts, gath,
                           block, gamma, vocab, p.n_vsplit, p.n_chunk, p.n_pick, inv_t, accept_len, out_tokens, alpha,
                           res, chunks);
    else
        hipLaunchKernelGGL(accept_resid_kernel<false>, g2, dim3(256), 0, st, logits, probs, tokens, tau, u, parts,
                           gath, block, gamma, vocab, p.n_vsplit, p.n_chunk, p.n_pick, inv_t, accept_len, out_tokens,
                           alpha, res, chunks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((vocab & 3) == 0)
        hipLaunchKernelGGL(residual_pick_kernel<true>, dim3(batch), dim3(256), 0, st, logits, probs, u, res, chunks,
                           out_tokens, block, gamma, vocab, p.n_pick, inv_t);
    else
        hipLaunchKernelGGL(residual_pick_kernel<false>, dim3(batch), dim3(256), 0, st, logits, probs, u, res, chunks,
                           out_tokens, block, gamma, vocab, p.n_pick, inv_t);
    return hipGetLastError();
}

}  // namespace sv
