// commit.hip -- the commit step after verification and the prompt-cache
// append, for gfx950 (MI355X).
//
// Method: "SimSD: Simple Speculative Decoding in Diffusion Language Models",
// 关键设计 4 (the accepted prefix is kept and the first rejected position is
// resampled in place; a block with fewer undecoded positions than the draft
// length is finished by ordinary target denoising) and 损失函数 / 训练策略 (the
// prompt's K/V are cached); the block-diffusion prior of "SPOT: Enhancing
// Speculative Decoding for Diffusion Language Models via Commit-Order
// Prediction", 前置知识 (a finished block joins the cached prefix).
//
// Launches on the caller's stream:
//   commit_kernel       one wave per sequence: lane k writes slot k's
//                       committed token into the block; the masked slots left
//                       are a ballot count; lane 0 writes R, the state and the
//                       rows to append.
//   append_rows_kernel  one workgroup per (sequence, kv head): each lane
//                       moves one 16-byte chunk of a key row's lower half and
//                       the matching chunk of its upper half (rotated at the
//                       row's new position when RoPE is on) and value chunks,
//                       into the row's page.
//   append_lens_kernel  then advances each sequence's prompt length (a
//                       separate launch: every row workgroup of a sequence
//                       reads the old length).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

__global__ void __launch_bounds__(64) commit_kernel(const int32_t *__restrict__ out_tokens, int32_t *block_tokens,
                                                    int block, int gamma, int32_t *remaining, int32_t *state,
                                                    int32_t *n_append) {
    const int lane = threadIdx.x, b = blockIdx.x;
    const bool in = lane < block;
    const size_t i = (size_t)b * block + (in ? lane : 0);
    int t = 0;
    if (in) {
        const int o = out_tokens[i];
        t = block_tokens[i];
        if (o >= 0) {
            t = o;
            block_tokens[i] = o;
        }
    }
    const int R = __popcll(__ballot(in && t < 0));
    if (lane == 0) {
        remaining[b] = R;
        state[b] = (R == 0) ? 2 : (R < gamma ? 1 : 0);
        n_append[b] = (R == 0) ? block : 0;
    }
}

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// append status of a sequence: 0 appended (or nothing to append), 1 would
// pass the capacity (nothing written), 2 n_append outside [0, src_stride],
// 3 a page the rows would land in has an id outside [0, n_pages) (nothing
// written: writing there could overwrite another sequence's page).  table is
// the sequence's block-table row (NULL: contiguous cache); every workgroup
// of the sequence and the length update read the same entries, so they agree.
__device__ __forceinline__ int append_status(int n, int P, int src_stride, long long capacity,
                                             const int32_t *table, int page_size, int n_pages) {
    if (n < 0 || n > src_stride || P < 0) return 2;
    if ((long long)P + n > capacity) return 1;
    if (table && n > 0) {
        for (int pg = P / page_size; pg <= (P + n - 1) / page_size; ++pg) {
            const int id = table[pg];
            if (id < 0 || id >= n_pages) return 3;
        }
    }
    return 0;
}

template <int D>
__global__ void __launch_bounds__(256) append_rows_kernel(const uint16_t *__restrict__ k_rows,
                                                          const uint16_t *__restrict__ v_rows,
                                                          const int32_t *__restrict__ n_append,
                                                          const int32_t *__restrict__ prefix_lens,
                                                          const int32_t *__restrict__ block_table, uint16_t *k_pages,
                                                          uint16_t *v_pages, int src_stride, int n_kvh,
                                                          int page_size, int max_pages, int n_pages,
                                                          long long capacity, int use_rope, double log2_theta) {
    constexpr int HC = D / 16;  // 16-byte chunks in half a row
    constexpr int NC = D / 8;   // 16-byte chunks in a row
    const int b = blockIdx.x / n_kvh, kvh = blockIdx.x % n_kvh;
    const int n = n_append[b], P = prefix_lens[b];
    const int32_t *table = block_table ? block_table + (size_t)b * max_pages : nullptr;
    if (append_status(n, P, src_stride, capacity, table, page_size, n_pages) != 0 || n == 0) return;
    auto dst_off = [&](int p) -> size_t {  // element offset of cache row p of (b, kvh)
        if (table) {  // every page id in range: checked by append_status
            const int pg = table[p / page_size];
            return (((size_t)pg * n_kvh + kvh) * page_size + p % page_size) * D;
        }
        return (((size_t)b * n_kvh + kvh) * page_size + p) * D;
    };
    // keys: one (row, chunk pair) per item, the pair = dims 8c..8c+7 and
    // D/2 + 8c .. D/2 + 8c + 7, rotated together (rotate-half pairs)
    for (int it = threadIdx.x; it < n * HC; it += blockDim.x) {
        const int i = it / HC, c = it % HC, p = P + i;
        const uint16_t *src = k_rows + (((size_t)b * src_stride + i) * n_kvh + kvh) * D;
        u16x8 lo = *reinterpret_cast<const u16x8 *>(src + 8 * c);
        u16x8 hi = *reinterpret_cast<const u16x8 *>(src + D / 2 + 8 * c);
        if (use_rope) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 cs = rope_cs((double)p, rope_inv_freq(8 * c + e, D, log2_theta));
                const float x1 = bf16_to_f32(lo[e]), x2 = bf16_to_f32(hi[e]);
                lo[e] = f32_to_bf16(x1 * cs.x - x2 * cs.y);
                hi[e] = f32_to_bf16(x1 * cs.y + x2 * cs.x);
            }
        }
        uint16_t *dst = k_pages + dst_off(p);
        *reinterpret_cast<u16x8 *>(dst + 8 * c) = lo;
        *reinterpret_cast<u16x8 *>(dst + D / 2 + 8 * c) = hi;
    }
    // values: plain 16-byte chunk copies
    for (int it = threadIdx.x; it < n * NC; it += blockDim.x) {
        const int i = it / NC, c = it % NC;
        const uint16_t *src = v_rows + (((size_t)b * src_stride + i) * n_kvh + kvh) * D;
        *reinterpret_cast<u16x8 *>(v_pages + dst_off(P + i) + 8 * c) = *reinterpret_cast<const u16x8 *>(src + 8 * c);
    }
}

__global__ void __launch_bounds__(256) append_lens_kernel(const int32_t *__restrict__ n_append, int32_t *prefix_lens,
                                                          int32_t *status, const int32_t *__restrict__ block_table,
                                                          int batch, int src_stride, long long capacity,
                                                          int page_size, int max_pages, int n_pages) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int n = n_append[b], P = prefix_lens[b];
    const int s = append_status(n, P, src_stride, capacity,
                                block_table ? block_table + (size_t)b * max_pages : nullptr, page_size, n_pages);
    if (s == 0) prefix_lens[b] = P + n;
    if (status) status[b] = s;
}

// One wave per sequence: bad[b] = 0 when tau[b] is a permutation of
// 1..block, else 1 (each label in range, and together they cover every
// label: the OR of one bit per lane is full).
__global__ void __launch_bounds__(64) check_tau_kernel(const int32_t *__restrict__ tau, int block, int32_t *bad) {
    const int lane = threadIdx.x, b = blockIdx.x;
    const bool in = lane < block;
    const int t = in ? tau[(size_t)b * block + lane] : 1;
    const bool ok = t >= 1 && t <= block;
    unsigned long long bits = (in && ok) ? (1ull << (t - 1)) : 0ull;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bits |= __shfl_xor(bits, o);
    const unsigned long long full = block == 64 ? ~0ull : ((1ull << block) - 1);
    const bool all_ok = __ballot(in && !ok) == 0ull;
    if (lane == 0) bad[b] = (all_ok && bits == full) ? 0 : 1;
}

hipError_t launch_check_tau(const int32_t *tau, int batch, int block, int32_t *bad, hipStream_t st) {
    hipLaunchKernelGGL(check_tau_kernel, dim3(batch), dim3(64), 0, st, tau, block, bad);
    return hipGetLastError();
}

hipError_t launch_commit(const int32_t *out_tokens, int32_t *block_tokens, int batch, int block, int gamma,
                         int32_t *remaining, int32_t *state, int32_t *n_append, hipStream_t st) {
    hipLaunchKernelGGL(commit_kernel, dim3(batch), dim3(64), 0, st, out_tokens, block_tokens, block, gamma,
                       remaining, state, n_append);
    return hipGetLastError();
}

hipError_t launch_append(const void *k_rows, const void *v_rows, int src_stride, const int32_t *n_append,
                         void *k_pages, void *v_pages, const int32_t *block_table, int32_t *prefix_lens,
                         int32_t *status, int batch, int page_size, int max_pages, int n_pages, int n_kvh,
                         int head_dim, double theta, hipStream_t st) {
    const long long capacity = block_table ? (long long)max_pages * page_size : page_size;
    const int use_rope = theta > 0 ? 1 : 0;
    const double l2t = theta > 0 ? log2(theta) : 0.0;
    const dim3 g((unsigned)(batch * n_kvh));
    if (head_dim == 128)
        hipLaunchKernelGGL(append_rows_kernel<128>, g, dim3(256), 0, st, (const uint16_t *)k_rows,
                           (const uint16_t *)v_rows, n_append, prefix_lens, block_table, (uint16_t *)k_pages,
                           (uint16_t *)v_pages, src_stride, n_kvh, page_size, max_pages, n_pages, capacity, use_rope,
                           l2t);
    else
        hipLaunchKernelGGL(append_rows_kernel<64>, g, dim3(256), 0, st, (const uint16_t *)k_rows,
                           (const uint16_t *)v_rows, n_append, prefix_lens, block_table, (uint16_t *)k_pages,
                           (uint16_t *)v_pages, src_stride, n_kvh, page_size, max_pages, n_pages, capacity, use_rope,
                           l2t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(append_lens_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, st, n_append,
                       prefix_lens, status, block_table, batch, src_stride, capacity, page_size, max_pages,
                       n_pages);
    return hipGetLastError();
}

}  // namespace sv
