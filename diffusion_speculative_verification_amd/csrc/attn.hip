// attn.hip -- copy-aligned RoPE and temporal-causal masked GQA attention of
// the 2B response rows for gfx950 (MI355X).
//
// Method: "SimSD: Simple Speculative Decoding in Diffusion Language Models",
// 关键设计 1 (paired layout [prompt | D | D~]), 关键设计 2 (mask A_ij from step
// labels tau), 关键设计 3 (D~_k reuses D_k's RoPE position).
//
// bf16 kernel (attn_bf16_kernel), one workgroup = 4 waves = 256 query rows of
// one kv head (all n_qh/n_kvh query heads of the GQA group share the K/V tile
// read, so every K/V byte of a (sequence, kv head) leaves HBM once per row
// block), looping over 64-key tiles of [prompt | D | D~]:
//   - K tile staged row-major in LDS, V tile staged transposed ([dim][key])
//     so both MFMA operands are contiguous LDS reads; double-buffered, the
//     next tile's global loads are in flight during the current tile's math;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on MFMA rows, queries
//     on columns): each lane then owns one query's scores, so the row
//     max/sum need one cross-lane exchange (lane ^ 32) per tile;
//   - the mask is evaluated in registers from tau only on tiles that reach
//     the response keys; prompt tiles take the unmasked path;
//   - online softmax in the log2 domain, P rounded to bf16 and fed straight
//     from the S^T accumulators as the B operand of O^T = V^T P^T (same
//     lane ownership, no shuffle); O is rescaled only when some lane's
//     running max moved;
//   - RoPE of Q and of the response keys is applied on load from a cos/sin
//     table built in LDS (angles formed in float64).
// Long prefixes with few (sequence, kv head) units are split over
// workgroups (flash-decoding style) and merged by attn_combine_kernel.
//
// float32 path: rope_kernel into the workspace, then attn_f32_kernel (one
// workgroup per response row and query head, float32 throughout).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

// ------------------------------------------------------------------ RoPE
template <typename T>
__device__ __forceinline__ float ld_elem(const T *p, size_t i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
template <typename T>
__device__ __forceinline__ void st_elem(T *p, size_t i, float v);
template <>
__device__ __forceinline__ void st_elem<float>(float *p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st_elem<uint16_t>(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }

// One thread per (row, head, pair i).  Rows r of both tensors sit at
// position prefix + (r mod block).
template <typename T>
__global__ void __launch_bounds__(256) rope_kernel(const T *__restrict__ q_in, const T *__restrict__ k_in,
                                                   T *q_out, T *k_out, int batch, int block, int n_qh,
                                                   int n_kvh, int d, int prefix, double log2_theta) {
    const int half = d >> 1;
    const int R = 2 * block, H = n_qh + n_kvh;
    const size_t total = (size_t)batch * R * H * half;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(idx % half);
        const size_t rh = idx / half;
        const int hh = (int)(rh % H);
        const size_t row = rh / H;  // b * R + r
        const int r = (int)(row % R);
        const T *src;
        T *dst;
        size_t off;
        if (hh < n_qh) { src = q_in; dst = q_out; off = (row * n_qh + hh) * d; }
        else { src = k_in; dst = k_out; off = (row * n_kvh + (hh - n_qh)) * d; }
        const float2 cs = rope_cs((double)prefix + (double)(r % block), rope_inv_freq(i, d, log2_theta));
        const float x1 = ld_elem(src, off + i), x2 = ld_elem(src, off + i + half);
        st_elem(dst, off + i, x1 * cs.x - x2 * cs.y);
        st_elem(dst, off + i + half, x1 * cs.y + x2 * cs.x);
    }
}

// ------------------------------------------------------- bf16 MFMA kernel
template <int D>
struct BfCfg {
    static constexpr int NS = D / 16;         // 16-dim k-steps of S^T
    static constexpr int NDB = D / 32;        // 32-dim blocks of O^T
    static constexpr int KROW = D + 8;        // K tile row stride (bf16), 16 B pad
    static constexpr int VROW = 34;           // V^T tile row stride (dwords): 64 keys + 2 pad dwords
    static constexpr int NKI = D / 64;        // K load items per thread (2 chunks each)
    static constexpr int NVI = D / 64;        // V load items per thread (2 keys each)
};

struct BfArgs {
    const uint16_t *q, *k_new, *v_new, *k_cache, *v_cache;
    const int32_t *tau;
    uint16_t *out;
    float *ws_o;    // split partials [split][batch][2B][Hq][D]
    float2 *ws_ml;  // [split][batch][2B][Hq] (running max in log2 units, sum)
    int batch, block, prefix, n_qh, n_kvh, n_rb, n_split, tiles_per_split, n_tiles;
    int use_rope;
    double log2_theta;
    float scale_log2;  // softmax scale * log2(e)
};

template <int D>
__device__ __forceinline__ const uint16_t *key_row(const BfArgs &a, const uint16_t *cache,
                                                   const uint16_t *fresh, int b, int kvh, int j) {
    const int R = 2 * a.block;
    if (j < a.prefix) return cache + (((size_t)b * a.n_kvh + kvh) * a.prefix + j) * D;
    if (j < a.prefix + R) return fresh + (((size_t)b * R + (j - a.prefix)) * a.n_kvh + kvh) * D;
    return nullptr;
}

__device__ __forceinline__ uint16_t u4_elem(const uint4 &v, int e) {
    const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
    return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

template <int D>
__global__ void __launch_bounds__(256, 1) attn_bf16_kernel(BfArgs a) {
    using C = BfCfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kTileKeys][C::KROW];
    __shared__ __attribute__((aligned(16))) uint32_t vt_lds[2][D][C::VROW];
    __shared__ __attribute__((aligned(16))) float2 cs_lds[64 * (D / 2)];
    __shared__ double invf_lds[D / 2];
    __shared__ int tau_lds[64];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int B = a.block, R2 = 2 * B, g = a.n_qh / a.n_kvh, R = g * R2;
    const int P = a.prefix, Nk = P + R2;

    // workgroup -> (b, kvh, rb, split); consecutive logical ids land on one
    // XCD when the grid divides by 8, so row blocks / splits of one kv head
    // share that XCD's L2.
    const int nblk = gridDim.x;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int split = bid % a.n_split;
    int rest = bid / a.n_split;
    const int rb = rest % a.n_rb;
    rest /= a.n_rb;
    const int kvh = rest % a.n_kvh;
    const int b = rest / a.n_kvh;
    const int t0 = split * a.tiles_per_split;
    const int t1 = min(a.n_tiles, t0 + a.tiles_per_split);

    if (tid < B) tau_lds[tid] = a.tau[(size_t)b * B + tid];

    // ---- global -> register staging of one K/V tile
    uint4 kreg[C::NKI][2], vreg[C::NVI][2];
    auto issue_loads = [&](int t) {
        const int base = t * kTileKeys;
#pragma unroll
        for (int s = 0; s < C::NKI; ++s) {
            const int it = tid + 256 * s, key = it / (D / 16), cp = it % (D / 16);
            const uint16_t *src = key_row<D>(a, a.k_cache, a.k_new, b, kvh, base + key);
            if (src) {
                kreg[s][0] = *reinterpret_cast<const uint4 *>(src + 8 * cp);
                kreg[s][1] = *reinterpret_cast<const uint4 *>(src + 8 * cp + D / 2);
            } else {
                kreg[s][0] = make_uint4(0, 0, 0, 0);
                kreg[s][1] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int s = 0; s < C::NVI; ++s) {
            const int c = (lane & 7) + 8 * s, kp = w * 8 + (lane >> 3);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint16_t *src = key_row<D>(a, a.v_cache, a.v_new, b, kvh, base + 2 * kp + u);
                vreg[s][u] = src ? *reinterpret_cast<const uint4 *>(src + 8 * c) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto write_lds = [&](int buf, int t) {
        const int base = t * kTileKeys;
#pragma unroll
        for (int s = 0; s < C::NKI; ++s) {
            const int it = tid + 256 * s, key = it / (D / 16), cp = it % (D / 16);
            const int j = base + key;
            uint4 lo = kreg[s][0], hi = kreg[s][1];
            if (a.use_rope && j >= P && j < Nk) {
                const int pr = (j - P) % B;
                uint32_t lw[4], hw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float y1[2], y2[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = 2 * e2 + u;
                        const float2 cs = cs_lds[pr * (D / 2) + 8 * cp + e];
                        const float x1 = bf16_to_f32(u4_elem(lo, e)), x2 = bf16_to_f32(u4_elem(hi, e));
                        y1[u] = x1 * cs.x - x2 * cs.y;
                        y2[u] = x1 * cs.y + x2 * cs.x;
                    }
                    lw[e2] = pack_bf16x2(y1[0], y1[1]);
                    hw[e2] = pack_bf16x2(y2[0], y2[1]);
                }
                lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            }
            *reinterpret_cast<uint4 *>(&k_lds[buf][key][8 * cp]) = lo;
            *reinterpret_cast<uint4 *>(&k_lds[buf][key][8 * cp + D / 2]) = hi;
        }
#pragma unroll
        for (int s = 0; s < C::NVI; ++s) {
            const int c = (lane & 7) + 8 * s, kp = w * 8 + (lane >> 3);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vt_lds[buf][8 * c + e][kp] =
                    (uint32_t)u4_elem(vreg[s][0], e) | ((uint32_t)u4_elem(vreg[s][1], e) << 16);
        }
    };

    if (t0 < t1) issue_loads(t0);

    // ---- RoPE cos/sin table for positions P + 0..B-1 (float64 angles)
    if (a.use_rope) {
        if (tid < D / 2) invf_lds[tid] = rope_inv_freq(tid, D, a.log2_theta);
        __syncthreads();
        for (int idx = tid; idx < B * (D / 2); idx += 256) {
            const int pr = idx / (D / 2), i = idx % (D / 2);
            cs_lds[idx] = rope_cs((double)P + (double)pr, invf_lds[i]);
        }
    }
    __syncthreads();

    // ---- per-lane query rows (two 32-row blocks per wave)
    int qhead[2], rrow[2], t_row[2];
    bool rvalid[2], r_is_d[2];
    bf16x8 qop[2][C::NS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int rho = rb * kRowsPerBlock + w * kRowsPerWave + qb * 32 + l32;
        rvalid[qb] = rho < R;
        const int rr = rvalid[qb] ? rho : 0;
        const int r = rr % R2;
        qhead[qb] = kvh * g + rr / R2;
        rrow[qb] = r;
        r_is_d[qb] = r < B;
        t_row[qb] = tau_lds[r % B];
        const uint16_t *qp = a.q + (((size_t)b * R2 + r) * a.n_qh + qhead[qb]) * D + 8 * h;
        uint4 raw[C::NS];
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
            raw[s] = rvalid[qb] ? *reinterpret_cast<const uint4 *>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
        if (a.use_rope) {
            const int pr = r % B;
#pragma unroll
            for (int s = 0; s < C::NS / 2; ++s) {
                uint32_t lw[4], hw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float y1[2], y2[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = 2 * e2 + u;
                        const float2 cs = cs_lds[pr * (D / 2) + 16 * s + 8 * h + e];
                        const float x1 = bf16_to_f32(u4_elem(raw[s], e));
                        const float x2 = bf16_to_f32(u4_elem(raw[s + C::NS / 2], e));
                        y1[u] = x1 * cs.x - x2 * cs.y;
                        y2[u] = x1 * cs.y + x2 * cs.x;
                    }
                    lw[e2] = pack_bf16x2(y1[0], y1[1]);
                    hw[e2] = pack_bf16x2(y2[0], y2[1]);
                }
                raw[s] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                raw[s + C::NS / 2] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            }
        }
#pragma unroll
        for (int s = 0; s < C::NS; ++s) qop[qb][s] = __builtin_bit_cast(bf16x8, raw[s]);
    }
    const bool wave_active = (rb * kRowsPerBlock + w * kRowsPerWave) < R;

    f32x16 oacc[2][C::NDB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int x = 0; x < 16; ++x) oacc[qb][db][x] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    if (t0 < t1) write_lds(0, t0);
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        if (t + 1 < t1) issue_loads(t + 1);
        if (wave_active) {
            const int base = t * kTileKeys;
            // ---- S^T = K Q^T (keys x queries), 2 key blocks x 2 query blocks
            f32x16 sacc[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int x = 0; x < 16; ++x) sacc[qb][kb][x] = 0.f;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&k_lds[buf][kb * 32 + l32][16 * s + 8 * h]);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[qb][s], sacc[qb][kb], 0, 0, 0);
                }
            }
            // ---- temporal-causal mask, only where response / padding keys occur
            if (base + kTileKeys > P) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int x = 0; x < 16; ++x) {
                        const int j = base + kb * 32 + 8 * (x >> 2) + 4 * h + (x & 3);
                        if (j >= P) {
                            bool key_ok = false, key_d = false;
                            int tk = 0;
                            if (j < Nk) {
                                const int c = j - P;
                                key_d = c < B;
                                tk = tau_lds[c % B];
                                key_ok = true;
                            }
#pragma unroll
                            for (int qb = 0; qb < 2; ++qb)
                                if (!key_ok || !visible(t_row[qb], r_is_d[qb], tk, key_d))
                                    sacc[qb][kb][x] = -INFINITY;
                        }
                    }
                }
            }
            // ---- online softmax (log2 domain); each lane owns one query
            bf16x8 pop[2][4];
            bool rescale = false;
            float alpha[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[qb][kb][x]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[qb], mx * a.scale_log2);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
                rescale |= (alpha[qb] != 1.f);
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub) {
                        bf16x8 pv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][8 * sub + e], a.scale_log2, -m_use));
                            const __bf16 pb = (__bf16)p;
                            ls += (float)pb;
                            pv[e] = pb;
                        }
                        pop[qb][2 * kb + sub] = pv;
                    }
                }
                l_run[qb] = l_run[qb] * alpha[qb] + ls;
                m_run[qb] = m_new;
            }
            if (__any(rescale)) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                        for (int x = 0; x < 16; ++x) oacc[qb][db][x] *= alpha[qb];
            }
            // ---- O^T += V^T P^T: k-step s covers tile keys 16s..16s+15; lane
            // half h supplies keys 16s+4h+{0..3} and 16s+8+4h+{0..3}
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const uint32_t *vrow = &vt_lds[buf][db * 32 + l32][0];
                    const uint2 v0 = *reinterpret_cast<const uint2 *>(vrow + 8 * s + 2 * h);
                    const uint2 v1 = *reinterpret_cast<const uint2 *>(vrow + 8 * s + 4 + 2 * h);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pop[qb][s], oacc[qb][db], 0, 0, 0);
                }
            }
        }
        if (t + 1 < t1) write_lds(buf ^ 1, t + 1);
        __syncthreads();
    }

    if (!wave_active) return;
    // ---- epilogue: lane owns query (qb, l32); O^T rows dim = db*32 + 8*jj + 4*h + i
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
        if (!rvalid[qb]) continue;
        const size_t row = ((size_t)b * R2 + rrow[qb]) * a.n_qh + qhead[qb];
        if (a.n_split == 1) {
            const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
            uint16_t *op = a.out + row * D + 4 * h;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const f32x16 &o = oacc[qb][db];
                    uint2 pk;
                    pk.x = pack_bf16x2(o[4 * jj + 0] * inv, o[4 * jj + 1] * inv);
                    pk.y = pack_bf16x2(o[4 * jj + 2] * inv, o[4 * jj + 3] * inv);
                    *reinterpret_cast<uint2 *>(op + db * 32 + 8 * jj) = pk;
                }
        } else {
            const size_t prow = (size_t)split * a.batch * R2 * a.n_qh + row;
            float *op = a.ws_o + prow * D + 4 * h;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const f32x16 &o = oacc[qb][db];
                    *reinterpret_cast<float4 *>(op + db * 32 + 8 * jj) =
                        make_float4(o[4 * jj + 0], o[4 * jj + 1], o[4 * jj + 2], o[4 * jj + 3]);
                }
            if (h == 0) a.ws_ml[prow] = make_float2(m_run[qb], l_tot);
        }
    }
}

// Merge prefix splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename T>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float *__restrict__ ws_o,
                                                           const float2 *__restrict__ ws_ml, T *out,
                                                           int n_split, size_t rows_total, int n_qh, int d) {
    const size_t row0 = (size_t)blockIdx.x * n_qh;  // one (b, r): all heads
    for (int idx = threadIdx.x; idx < n_qh * d; idx += blockDim.x) {
        const int hh = idx / d, e = idx % d;
        const size_t row = row0 + hh;
        float M = -INFINITY;
        for (int s = 0; s < n_split; ++s) M = fmaxf(M, ws_ml[s * rows_total + row].x);
        float num = 0.f, den = 0.f;
        for (int s = 0; s < n_split; ++s) {
            const float2 ml = ws_ml[s * rows_total + row];
            const float f = (ml.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
            den += f * ml.y;
            num += f * ws_o[(s * rows_total + row) * d + e];
        }
        st_elem(out, row * d + e, den > 0.f ? num / den : 0.f);
    }
}

// ------------------------------------------------------------ float32 path
// One workgroup per (sequence, response row, query head); threads stride
// over keys with a per-thread online softmax, then a workgroup merge.
template <int D>
__global__ void __launch_bounds__(256) attn_f32_kernel(const float *__restrict__ q, const float *__restrict__ k_new,
                                                       const float *__restrict__ v_new, const float *__restrict__ k_cache,
                                                       const float *__restrict__ v_cache, const int32_t *__restrict__ tau,
                                                       float *out, int block, int prefix, int n_qh, int n_kvh, float scale) {
    __shared__ float q_s[D];
    __shared__ int tau_s[64];
    __shared__ float red_m[4];
    __shared__ float red_o[4][D + 1];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int R2 = 2 * block, P = prefix, Nk = P + R2;
    const int hq = blockIdx.x % n_qh;
    const int r = (blockIdx.x / n_qh) % R2;
    const int b = blockIdx.x / (n_qh * R2);
    const int kvh = hq / (n_qh / n_kvh);
    const size_t qrow = ((size_t)b * R2 + r) * n_qh + hq;
    for (int e = tid; e < D; e += 256) q_s[e] = q[qrow * D + e];
    if (tid < block) tau_s[tid] = tau[(size_t)b * block + tid];
    __syncthreads();
    const bool row_d = r < block;
    const int t_row = tau_s[r % block];
    float m = -INFINITY, l = 0.f, o[D];
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = 0.f;
    for (int j = tid; j < Nk; j += 256) {
        const float *kp, *vp;
        if (j < P) {
            kp = k_cache + (((size_t)b * n_kvh + kvh) * P + j) * D;
            vp = v_cache + (((size_t)b * n_kvh + kvh) * P + j) * D;
        } else {
            const int c = j - P;
            if (!visible(t_row, row_d, tau_s[c % block], c < block)) continue;
            kp = k_new + (((size_t)b * R2 + c) * n_kvh + kvh) * D;
            vp = v_new + (((size_t)b * R2 + c) * n_kvh + kvh) * D;
        }
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = fmaf(q_s[e], kp[e], s);
        s *= scale;
        const float mn = fmaxf(m, s);
        const float corr = expf(m - mn), p = expf(s - mn);
        l = l * corr + p;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = o[e] * corr + p * vp[e];
        m = mn;
    }
    // workgroup merge of (m, l, o)
    float M = wave_max(m);
    if (lane == 0) red_m[w] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    const float f = (m == -INFINITY) ? 0.f : expf(m - M);
    l *= f;
    for (int o2 = 32; o2 > 0; o2 >>= 1) l += __shfl_xor(l, o2);
#pragma unroll
    for (int e = 0; e < D; ++e) {
        float v = o[e] * f;
        for (int o2 = 32; o2 > 0; o2 >>= 1) v += __shfl_xor(v, o2);
        o[e] = v;
    }
    if (lane == 0) {
#pragma unroll
        for (int e = 0; e < D; ++e) red_o[w][e] = o[e];
        red_o[w][D] = l;
    }
    __syncthreads();
    for (int e = tid; e < D; e += 256) {
        const float ltot = red_o[0][D] + red_o[1][D] + red_o[2][D] + red_o[3][D];
        const float v = red_o[0][e] + red_o[1][e] + red_o[2][e] + red_o[3][e];
        out[qrow * D + e] = v / ltot;
    }
}

// ------------------------------------------------------------- host side
AttnPlan attn_plan(const AttnShape &s) {
    AttnPlan p{};
    const int g = s.n_qh / s.n_kvh;
    p.rows = g * 2 * s.block;
    p.n_rb = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int nk = s.prefix + 2 * s.block;
    p.n_tiles = (nk + kTileKeys - 1) / kTileKeys;
    p.n_split = 1;
    p.tiles_per_split = p.n_tiles;
    if (s.dtype == 1) {
        // aim for about one workgroup per compute unit (256 CUs)
        const long units = (long)s.batch * s.n_kvh * p.n_rb;
        if (units < 256 && p.n_tiles >= 4) {
            int want = (int)((256 + units - 1) / units);
            want = want < p.n_tiles / 2 ? want : p.n_tiles / 2;
            if (want > 1) {
                p.tiles_per_split = (p.n_tiles + want - 1) / want;
                p.n_split = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
            }
        }
        if (p.n_split > 1) {
            const size_t rows = (size_t)p.n_split * s.batch * 2 * s.block * s.n_qh;
            p.ws_partial_o = align_up(rows * s.head_dim * sizeof(float));
            p.ws_partial_ml = align_up(rows * sizeof(float2));
        }
    } else {
        const size_t rq = (size_t)s.batch * 2 * s.block * s.n_qh * s.head_dim;
        const size_t rk = (size_t)s.batch * 2 * s.block * s.n_kvh * s.head_dim;
        p.ws_rope = align_up(rq * sizeof(float)) + align_up(rk * sizeof(float));
    }
    p.ws_total = p.ws_partial_o + p.ws_partial_ml + p.ws_rope;
    return p;
}

hipError_t launch_rope(const void *q_in, const void *k_in, void *q_out, void *k_out, int dtype,
                       int batch, int block, int n_qh, int n_kvh, int head_dim, int prefix,
                       double theta, hipStream_t st) {
    const size_t total = (size_t)batch * 2 * block * (n_qh + n_kvh) * (head_dim / 2);
    size_t grid = (total + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (grid == 0) return hipSuccess;
    const double l2t = log2(theta);
    if (dtype == 1)
        hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, st,
                           (const uint16_t *)q_in, (const uint16_t *)k_in, (uint16_t *)q_out,
                           (uint16_t *)k_out, batch, block, n_qh, n_kvh, head_dim, prefix, l2t);
    else
        hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)grid), dim3(256), 0, st,
                           (const float *)q_in, (const float *)k_in, (float *)q_out, (float *)k_out,
                           batch, block, n_qh, n_kvh, head_dim, prefix, l2t);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnShape &s, const AttnPlan &p, const void *q, const void *k_new,
                       const void *v_new, const void *k_cache, const void *v_cache,
                       const int32_t *tau, void *out, double theta, float scale, void *ws,
                       hipStream_t st) {
    const int R2 = 2 * s.block;
    if (s.dtype == 1) {
        BfArgs a{};
        a.q = (const uint16_t *)q;
        a.k_new = (const uint16_t *)k_new;
        a.v_new = (const uint16_t *)v_new;
        a.k_cache = (const uint16_t *)k_cache;
        a.v_cache = (const uint16_t *)v_cache;
        a.tau = tau;
        a.out = (uint16_t *)out;
        a.ws_o = p.n_split > 1 ? (float *)ws : nullptr;
        a.ws_ml = p.n_split > 1 ? (float2 *)((char *)ws + p.ws_partial_o) : nullptr;
        a.batch = s.batch;
        a.block = s.block;
        a.prefix = s.prefix;
        a.n_qh = s.n_qh;
        a.n_kvh = s.n_kvh;
        a.n_rb = p.n_rb;
        a.n_split = p.n_split;
        a.tiles_per_split = p.tiles_per_split;
        a.n_tiles = p.n_tiles;
        a.use_rope = theta > 0 ? 1 : 0;
        a.log2_theta = theta > 0 ? log2(theta) : 0.0;
        a.scale_log2 = scale * kLog2e;
        const unsigned grid = (unsigned)((size_t)s.batch * s.n_kvh * p.n_rb * p.n_split);
        if (s.head_dim == 128)
            hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.n_split == 1) return e;
        const size_t rows_total = (size_t)s.batch * R2 * s.n_qh;
        hipLaunchKernelGGL(attn_combine_kernel<uint16_t>, dim3((unsigned)((size_t)s.batch * R2)), dim3(256), 0,
                           st, (const float *)a.ws_o, (const float2 *)a.ws_ml, (uint16_t *)out, p.n_split,
                           rows_total, s.n_qh, s.head_dim);
        return hipGetLastError();
    }
    // float32: rotate into the workspace (if asked), then attend
    const float *qq = (const float *)q, *kk = (const float *)k_new;
    if (theta > 0) {
        const size_t rq = (size_t)s.batch * R2 * s.n_qh * s.head_dim;
        float *qr = (float *)ws;
        float *kr = (float *)((char *)ws + align_up(rq * sizeof(float)));
        hipError_t e = launch_rope(q, k_new, qr, kr, 0, s.batch, s.block, s.n_qh, s.n_kvh, s.head_dim,
                                   s.prefix, theta, st);
        if (e != hipSuccess) return e;
        qq = qr;
        kk = kr;
    }
    const unsigned grid = (unsigned)((size_t)s.batch * R2 * s.n_qh);
    if (s.head_dim == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(256), 0, st, qq, kk, (const float *)v_new,
                           (const float *)k_cache, (const float *)v_cache, tau, (float *)out, s.block, s.prefix,
                           s.n_qh, s.n_kvh, scale);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(256), 0, st, qq, kk, (const float *)v_new,
                           (const float *)k_cache, (const float *)v_cache, tau, (float *)out, s.block, s.prefix,
                           s.n_qh, s.n_kvh, scale);
    return hipGetLastError();
}

}  // namespace sv
