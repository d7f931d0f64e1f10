// attn.hip -- copy-aligned RoPE and temporal-causal masked GQA attention of
// the 2B response rows for gfx950 (MI355X).
//
// Method: "SimSD: Simple Speculative Decoding in Diffusion Language Models",
// 关键设计 1 (paired layout [prompt | D | D~]), 关键设计 2 (mask A_ij from step
// labels tau), 关键设计 3 (D~_k reuses D_k's RoPE position).  The same bf16
// kernel, with a compile-time mask rule, runs the multi-copy layout of "SPOT:
// Enhancing Speculative Decoding for Diffusion Language Models via
// Commit-Order Prediction" (核心方法, third step: C copies of the block, each
// bidirectional over its own keys, the prompt shared), and reads the prompt
// cache either contiguously or through a page table with per-sequence
// prompt lengths.
//
// bf16 kernel (attn_bf16_kernel): one workgroup = NW waves x 32 query rows
// of one kv head (NW = 8 when the kv head has more than 128 rows, else 4;
// the n_qh/n_kvh query heads of a GQA group are rows of the same workgroup,
// so they share every K/V tile; row blocks and prefix splits of one kv head
// are placed on one XCD so that they meet its K/V in that XCD's L2).  One
// workgroup per CU (about 130 KB of LDS), looping over 64-key tiles of
// [prompt | D | D~]:
//   - a 3-stage LDS ring of (K, V) tiles, filled by direct global->LDS loads
//     (global_load_lds_dwordx4) two tiles ahead of the math; a prompt tile's
//     loads use a scalar tile base plus a loop-invariant lane offset and go
//     out between the S MFMAs; both tiles are row-major with 16-byte chunks
//     XOR-swizzled for the 64-bank LDS;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on MFMA rows, queries
//     on columns): each lane then owns one query's scores, so the row
//     max/sum need one cross-lane exchange (lane ^ 32) per tile; in the
//     8-wave kernel the K operand reads run four MFMAs ahead;
//   - the mask is evaluated in registers, only on tiles that reach the
//     response keys (prompt tiles take the unmasked path): each row holds a
//     64-key window of its key visibility built from the step labels, one
//     bit test per score;
//   - online softmax in the log2 domain, P rounded to bf16 and fed straight
//     from the S^T accumulators as the B operand of O^T = V^T P^T (same lane
//     ownership, no shuffle); V^T comes from the row-major V tile through
//     the transposing LDS read ds_read_b64_tr_b16; O is rescaled only when
//     the running max moves by more than 8 (log2 units);
//   - RoPE of Q is applied on load and that of the response keys in place in
//     the K tile, from a cos/sin table built in LDS (angles formed and
//     reduced in float64, hardware sine/cosine on the reduced revolutions).
// Long prefixes with few (sequence, kv head) units are split over
// workgroups (flash-decoding style) and merged by attn_combine_kernel.
//
// float32 path: rope_kernel into the workspace, then attn_f32_kernel (one
// workgroup per response row and query head, float32 throughout).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

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
// LDS tile layout: 64 rows (keys) x D bf16, rows of D*2 bytes, 16-byte
// chunks XOR-swizzled per row so that both the S^T operand reads and the
// transposed V reads are bank-conflict free.  The LDS serves 256 bytes (64
// banks of 4 bytes) per cycle: 16 lanes of a 16-byte read, 32 lanes of an
// 8-byte read.
// K tiles (IS_V = false): the 16 lanes served together read 16 consecutive
// rows at one logical chunk, so the swizzle gives those rows 16 distinct
// bank groups: chunk ^ (row & 15) for D = 128 (one row = one 256-byte bank
// line), chunk ^ ((row >> 1) & 7) for D = 64 (two rows per bank line).
// V tiles (IS_V = true): the 32 lanes served together read 4 consecutive
// rows x 4 logical chunks (8 bytes per lane), so the 4 rows must map that
// chunk quad to disjoint bank groups: chunk ^ ((row & 3) << 2) for D = 128;
// for D = 64 chunk ^ ((row & 3) << 1) keeps the 2 rows of a bank line apart.
template <int D, bool IS_V>
struct Tile {
    static constexpr int NCH = D / 8;             // 16-byte chunks per row
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int BYTES = kTileKeys * ROW_BYTES;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;  // rows one wave-wide 16 B/lane load fills
    static constexpr int LOADS = kTileKeys / ROWS_PER_LOAD;  // wave loads per tile and tensor
    __device__ static __forceinline__ int swz(int row) {
        if (IS_V) return D == 128 ? ((row & 3) << 2) : ((row & 3) << 1);
        return D == 128 ? (row & 15) : ((row >> 1) & 7);
    }
    __device__ static __forceinline__ int off(int row, int chunk) {  // byte offset of a logical chunk
        return row * ROW_BYTES + ((chunk ^ swz(row)) << 4);
    }
};

struct BfArgs {
    const uint16_t *q, *k_new, *v_new, *k_cache, *v_cache;
    const int32_t *tau;
    uint16_t *out;
    uint16_t *ws_o;  // split partials [split][batch][n_resp][Hq][D], unnormalised, bf16 (RNE)
    float2 *ws_ml;  // [split][batch][n_resp][Hq] (running max in log2 units, sum)
    int batch, block, prefix, n_qh, n_kvh, n_rb, n_split, tiles_per_split;
    int n_resp;  // response rows (and keys) per sequence: 2B, or copies * block
    // prompt cache: row j of (sequence b, kv head) lives in page
    // block_table[b][j / page_size] at row j % page_size, pages laid out
    // [page][kv head][page_size][D]; without a table the page is b and
    // page_size is the row stride of a contiguous [batch][kv head][stride][D]
    // cache.  prefix_lens (optional) gives each sequence its own prompt
    // length; `prefix` is then the longest.
    const int32_t *prefix_lens, *block_table;
    int page_size, max_pages, n_pages;
    int use_rope;
    double log2_theta;
    float scale_log2;  // softmax scale * log2(e)
};

// A wave-uniform read of a table the kernel never writes, through the
// constant address space, so that it is a scalar load (waited on by lgkmcnt):
// a vector load here would make the compiler wait on vmcnt, which also counts
// the direct tile loads in flight.
__device__ __forceinline__ int32_t uniform_ld(const int32_t *p, size_t i) {
    return *((const __attribute__((address_space(4))) int32_t *)(uintptr_t)p + i);
}

// Element offset of prompt row j of (b, kvh) in the cache.  Called with
// wave-uniform arguments only.  Page ids outside [0, n_pages) are clamped (a
// bad table gives wrong rows, never an access outside the pages).
template <int D>
__device__ __forceinline__ size_t cache_off(const BfArgs &a, int b, int kvh, int j) {
    if (a.block_table) {
        int pg = uniform_ld(a.block_table, (size_t)b * a.max_pages + j / a.page_size);
        pg = min(max(pg, 0), a.n_pages - 1);
        return (((size_t)pg * a.n_kvh + kvh) * a.page_size + j % a.page_size) * D;
    }
    return (((size_t)b * a.n_kvh + kvh) * a.page_size + j) * D;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define SV_LDS __attribute__((address_space(3)))

__device__ __forceinline__ uint16_t u4_elem(const uint4 &v, int e) {
    const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
    return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}


// Wave-wide direct global -> LDS copy of one tile of one tensor: load i of
// wave w fills rows [r0, r0 + ROWS_PER_LOAD) with r0 = (w + NW * i) *
// ROWS_PER_LOAD; lane l writes physical chunk l % NCH of its row and
// therefore fetches the logical chunk that the swizzle places there.
// One wave-wide direct global->LDS load: lane l's 16 bytes at `src` land at
// LDS address lds_dst + 16 * l, with the non-temporal hint when NT.  With one
// row block per kv head each K/V tile is read once and streamed (NT); with
// several (the multi-copy layout, wide GQA groups) the row blocks of a kv
// head read the same prompt tiles at about the same time on one XCD, and
// plain loads let the later ones hit in L2.  Issued as inline assembly so that the
// compiler's wait insertion does not treat later LDS reads of other ring
// stages as dependent on it: every wait on these loads is explicit
// (wait_vmcnt), and no compiler-visible global load is issued while tile
// loads are in flight inside the tile loop.
template <bool NT>
__device__ __forceinline__ void direct_load16(const void *src, char *lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(SV_LDS char *)lds_dst);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     :
                     : "s"(m0), "v"(src)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(m0), "v"(src)
                     : "memory", "m0");
}

// The same load with a uniform 64-bit base in scalar registers plus this
// lane's 32-bit byte offset (the scalar-base address form), and the LDS
// destination given as a wave-uniform address: no per-load vector address
// arithmetic.
template <bool NT>
__device__ __forceinline__ void direct_load16_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(m0), "v"(voff), "s"(sbase)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0), "v"(voff), "s"(sbase)
                     : "memory", "m0");
}

// Loop-invariant parts of this wave's tile loads: for load i, this lane's
// byte offset inside a prompt tile of K and of V (row and swizzled chunk),
// and the LDS byte offset of the rows it fills (wave-uniform).
template <int D, int NW>
struct LoadOffs {
    static constexpr int N = Tile<D, false>::LOADS / NW;
    uint32_t k[N], v[N], lds[N];
};

template <int D, int NW>
__device__ __forceinline__ LoadOffs<D, NW> load_offsets(int w, int lane) {
    using TK = Tile<D, false>;
    using TV = Tile<D, true>;
    LoadOffs<D, NW> o;
#pragma unroll
    for (int i = 0; i < LoadOffs<D, NW>::N; ++i) {
        const int r0 = (w + NW * i) * TK::ROWS_PER_LOAD;
        const int row = r0 + lane / TK::NCH, pc = lane % TK::NCH;
        o.k[i] = (uint32_t)((row * D + (pc ^ TK::swz(row)) * 8) * 2);
        o.v[i] = (uint32_t)((row * D + (pc ^ TV::swz(row)) * 8) * 2);
        o.lds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(r0 * TK::ROW_BYTES));
    }
    return o;
}

// Tiles that lie wholly inside the prompt take the fast path: a tile's rows
// are contiguous in one page (pages hold whole tiles; a contiguous cache is
// one page), so the source is a uniform tile base plus this lane's
// row/chunk offset.  Other tiles pick per row between the prompt (the same
// page: all prompt rows a tile holds lie in the page of its first row) and
// the response keys; keys at or past `jend` (the end of this workgroup's
// key range) read the row jend - 1 instead: such rows are never used, and
// re-reading one row keeps them in cache.
template <int D, int NW, bool IS_V, bool NT>
__device__ __forceinline__ void load_tile(const BfArgs &a, const uint16_t *cache, const uint16_t *fresh,
                                          int b, int kvh, int base, int jend, char *lds_tile, int w, int lane) {
    using T = Tile<D, IS_V>;
    const int P = a.prefix, R = a.n_resp;
    const bool fast = base + kTileKeys <= P;  // uniform
    // first row this tile reads (a tile past the end reads row jend - 1 only)
    const int jref = min(base, jend - 1);
    const uint16_t *tile = (jref < P) ? cache + cache_off<D>(a, b, kvh, jref) : cache;  // row jref
#pragma unroll
    for (int i = 0; i < T::LOADS / NW; ++i) {
        const int r0 = (w + NW * i) * T::ROWS_PER_LOAD;
        const int row = r0 + lane / T::NCH, pc = lane % T::NCH;
        const int q = pc ^ T::swz(row);
        const uint16_t *src;
        if (fast) {
            src = tile + row * D + q * 8;
        } else {
            const int j = min(base + row, jend - 1);
            src = (j < P ? tile + (size_t)(j - jref) * D
                         : fresh + (((size_t)b * R + (j - P)) * a.n_kvh + kvh) * D) + q * 8;
        }
        direct_load16<NT>(src, lds_tile + r0 * T::ROW_BYTES);
    }
}

// s_waitcnt vmcnt(N) through the builtin, so that the compiler's own wait
// insertion knows about it (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the tile ring, with release/acquire ordering of
// LDS only (the fences name the local address space): this wave's LDS
// accesses complete (lgkmcnt) before it arrives, and the compiler may not
// move LDS accesses across it.  Unlike __syncthreads() it does not order
// global memory, so the direct global->LDS loads of later tiles stay in
// flight across it; each wave waits for its own loads of the current tile
// (wait_vmcnt) before arriving, which makes that tile visible to all.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D, int QB>
struct RowState {  // per-lane attention state of its QB query rows
    f32x16 oacc[QB][D / 32];
    float m_run[QB], l_run[QB];
};

// Rotate the 8-dim chunk pair (lo: dims 8c.., hi: dims 8c + D/2 ..) of one
// row with cos/sin entries cs[0..7] (copy-aligned RoPE, rotate-half pairs).
__device__ __forceinline__ void rotate_pair(uint4 &lo, uint4 &hi, const float2 *__restrict__ cs) {
    uint32_t lw[4], hw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        float y1[2], y2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * e2 + u;
            const float2 c = cs[e];
            const float x1 = bf16_to_f32(u4_elem(lo, e)), x2 = bf16_to_f32(u4_elem(hi, e));
            y1[u] = x1 * c.x - x2 * c.y;
            y2[u] = x1 * c.y + x2 * c.x;
        }
        lw[e2] = pack_bf16x2(y1[0], y1[1]);
        hw[e2] = pack_bf16x2(y2[0], y2[1]);
    }
    lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
}

// Row stride (in float2 entries) of the cos/sin table in LDS: one entry per
// rotate-half pair plus one of padding, so that the 32 lanes of a wave half,
// which read the same pair index at 32 different positions, hit distinct
// banks.
template <int D>
constexpr int kCsStride = D / 2 + 1;

// (1.0, 1.0) in bf16
constexpr bf16x2_t kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// Key tiles a workgroup visits, in order: tile i of its list is tile
// map(i) of [prompt | response keys].  The paired layout visits every tile;
// in the multi-copy layout a workgroup visits the tiles holding prompt keys
// and then only those holding its own copies' keys.
template <int MASK>
struct TileMap {
    int n_prompt;  // tiles holding prompt keys (the list is the identity below it)
    int shift;     // response tiles skipped after them
    __device__ __forceinline__ int operator()(int i) const {
        if constexpr (MASK == 0) return i;
        else return i < n_prompt ? i : i + shift;
    }
};

// Row rho of a kv head's rows -> (response row, query head within the GQA
// group).  Paired layout: head-major, (head, row).  Multi-copy layout:
// (copy, head, position), so that the rows of a workgroup, and of a wave,
// belong to consecutive copies.
template <int MASK>
__device__ __forceinline__ int2 map_row(int rho, int R2, int B, int g) {
    if constexpr (MASK == 0) {
        return make_int2(rho % R2, rho / R2);
    } else {
        const int c = rho / (g * B), rem = rho % (g * B);
        return make_int2(c * B + rem % B, rem / B);
    }
}

template <int QB>
struct RowInfo {
    // paired layout: the row's label threshold, the step label of its slot
    // plus one for a D row (clamped to 0 .. B + 1); a D key is visible to the
    // row iff its label is below the threshold, a D~ key iff it is not.
    // Copies: the row's copy.
    int lab[QB];
    int c_lo, c_hi;  // copies: the range of copies this wave's rows belong to
};

// Bits of a 64-key window of a row's keys: bit j is the visibility of response
// key off + j.  m0 / m1 hold the visibility of response keys 0..63 / 64..127;
// keys before the first response key are prompt keys (visible), keys from 128
// on are padding (hidden).  off lies in -63 .. 131.
__device__ __forceinline__ uint64_t key_window(int off, uint64_t m0, uint64_t m1) {
    const int q = off >> 6, r = off & 63;  // q in -1 .. 2
    const uint64_t lo = q < 0 ? ~0ull : q == 0 ? m0 : q == 1 ? m1 : 0ull;
    const uint64_t hi = q < 0 ? m0 : q == 0 ? m1 : 0ull;
    return r == 0 ? lo : ((lo >> r) | (hi << (64 - r)));
}

// the n lowest bits, n in 0 .. 64
__device__ __forceinline__ uint64_t low_bits(int n) { return n >= 64 ? ~0ull : (1ull << n) - 1; }

// max of x over lanes l and l ^ 32.  The 8-wave kernel exchanges the two
// 32-lane halves with v_permlane32_swap, a VALU op (no LDS round trip queued
// behind the tile reads; each lane ends with its own value and its peer's);
// the 4-wave kernel keeps the LDS permute, which measured faster there.
template <int NW>
__device__ __forceinline__ float pair_max(float x) {
    if constexpr (NW == 8) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    } else {
        return fmaxf(x, __shfl_xor(x, 32));
    }
}

// Loop-invariant LDS byte offsets of this lane's MFMA operand reads.  The
// K swizzle depends on row & 15 and the V swizzle on row & 3 only, and each
// read family below moves in steps of 16 (K: 32) rows, so the swizzled chunk
// is fixed per lane:
//   S^T operand (K, row kb*32 + l32, chunk 2s + h):  k[s] + kb * 32 * ROW_BYTES
//   V^T operand (V, rows 16s + 4h + j/4 (+ 8), dims 32db + v_dim_lo):
//                                          v[db] + 16 * s * ROW_BYTES (+ 8 * ROW_BYTES)
template <int D>
struct LdsOffs {
    int k[D / 16];
    uint32_t v[D / 32];  // absolute LDS addresses in V stage 0 (see vbase_opaque)
};

// Per-lane V read bases hold the absolute LDS address of V stage 0 and are
// hidden from constant folding, so that each transposing read of any stage
// is this base plus an immediate offset below 64 KB (the DS offset field);
// without this the compiler re-forms every V address (one VALU op per read)
// because the stages lie above 64 KB.
__device__ __forceinline__ uint32_t vbase_opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int D>
__device__ __forceinline__ LdsOffs<D> lds_offsets(int lane, const char *v_stage0) {
    using TK = Tile<D, false>;
    using T = Tile<D, true>;
    const int h = lane >> 5, l32 = lane & 31, gq = lane >> 4, jl = lane & 15;
    LdsOffs<D> o;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) o.k[s] = TK::off(l32, 2 * s + h);
    const int v_dim_lo = 16 * (gq & 1) + 4 * (jl & 3);
    const int k0 = 4 * h + (jl >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int dim = 32 * db + v_dim_lo;
        o.v[db] = vbase_opaque((uint32_t)(uintptr_t)(const SV_LDS char *)v_stage0 + T::off(k0, dim >> 3) +
                               ((dim & 7) << 1));
    }
    return o;
}

// One ring step.  Tile `it` sits in (kt, vt); the stage consumed in the
// previous step, (kn, vn), is refilled with tile it + 2.  All LDS regions are
// __restrict__ parameters of this inlined function, which lets the compiler
// prove that the refill in flight never aliases this step's reads.  Each
// lane owns QB query rows (one per 32-row MFMA block); every K and V operand
// read from LDS feeds QB MFMAs.
template <int D, int NW, int QB, int MASK, bool NT>
__device__ __forceinline__ void tile_step(const BfArgs &a, int b, int kvh, int t0, int nt, int it, bool wave_active,
                                          const RowInfo<QB> &ri, const LdsOffs<D> &lo_, const bf16x8 (*qop)[D / 16],
                                          RowState<D, QB> &st, char *__restrict__ kt, char *__restrict__ vt,
                                          char *__restrict__ kn, char *__restrict__ vn,
                                          const float2 *__restrict__ cs, const uint64_t *__restrict__ below,
                                          const char *v_stage0, const LoadOffs<D, NW> &ldo, size_t unit_off,
                                          const TileMap<MASK> &tm, int jend) {
    using T = Tile<D, false>;
    constexpr int NS = D / 16, NDB = D / 32, NTH = 64 * NW;
    constexpr int LPT = 2 * (T::LOADS / NW);  // direct loads per wave per tile (K and V)
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5;
    const int B = a.block, P = a.prefix, Nk = P + a.n_resp;
    const int base = tm(t0 + it) * kTileKeys;
    // the LPT most recent loads are the refill issued one step ago (tile
    // it + 1); everything older, tile it included, has landed
    wait_vmcnt<LPT>();
    ring_barrier();
    // ---- RoPE of response keys, in place in the K tile
    if (a.use_rope && base + kTileKeys > P) {
        for (int idx = tid; idx < kTileKeys * (T::NCH / 2); idx += NTH) {
            const int row = idx / (T::NCH / 2), cp = idx % (T::NCH / 2);
            const int j = base + row;
            if (j < P || j >= Nk) continue;
            uint4 *plo = reinterpret_cast<uint4 *>(kt + T::off(row, cp));
            uint4 *phi = reinterpret_cast<uint4 *>(kt + T::off(row, cp + T::NCH / 2));
            uint4 lo = *plo, hi = *phi;
            rotate_pair(lo, hi, cs + ((j - P) % B) * kCsStride<D> + 8 * cp);
            *plo = lo;
            *phi = hi;
        }
        ring_barrier();
    }
    // ---- refill the stage consumed in the previous step with tile it + 2
    // (issued on every step, so the number of loads in flight is the same on
    // every path).  A prompt tile's loads take the scalar-base form; an
    // active wave issues them between its S MFMAs below, one every few
    // k-steps, so that their issue overlaps matrix work instead of queueing
    // behind the other waves' loads right after the barrier.
    constexpr int NL = LoadOffs<D, NW>::N;  // loads per tensor
    constexpr bool kNt = NT;                // see direct_load16
    const int nb = tm(t0 + it + 2) * kTileKeys;
    const bool prompt_refill = nb + kTileKeys <= P;  // uniform
    // element offset of the refill tile (contiguous cache: this unit's base
    // plus the tile's rows, without the general page arithmetic)
    size_t nb_off = 0;
    if (prompt_refill) nb_off = a.block_table ? cache_off<D>(a, b, kvh, nb) : unit_off + (size_t)nb * D;
    const uint16_t *kb_src = a.k_cache + nb_off, *vb_src = a.v_cache + nb_off;
    const uint32_t kn_lds = (uint32_t)(uintptr_t)(SV_LDS char *)kn, vn_lds = (uint32_t)(uintptr_t)(SV_LDS char *)vn;
    auto refill = [&](int i) {  // load i of 2 * NL: K loads first, then V
        if (i < NL) direct_load16_s<kNt>(kb_src, ldo.k[i], kn_lds + ldo.lds[i]);
        else direct_load16_s<kNt>(vb_src, ldo.v[i - NL], vn_lds + ldo.lds[i - NL]);
    };
    if (!prompt_refill) {
        load_tile<D, NW, false, kNt>(a, a.k_cache, a.k_new, b, kvh, nb, jend, kn, w, lane);
        load_tile<D, NW, true, kNt>(a, a.v_cache, a.v_new, b, kvh, nb, jend, vn, w, lane);
    } else if (!wave_active) {
#pragma unroll
        for (int i = 0; i < 2 * NL; ++i) refill(i);
    }
    if (!wave_active) return;

    // ---- copies: a tile of response keys none of whose copies has a row in
    // this wave is wholly masked for it and leaves its state unchanged (all
    // its probabilities are 0, the running max stays), so the wave skips it.
    // Tiles holding prompt keys are always live.
    if constexpr (MASK == 1) {
        const int c0 = base - P;  // first response key of the tile
        if (c0 >= 0 && !(c0 < a.n_resp && c0 / B <= ri.c_hi &&
                         min(c0 + kTileKeys - 1, a.n_resp - 1) / B >= ri.c_lo))
            return;
    }
    // ---- S^T = K Q^T (keys x queries): 2 key blocks of 32 per query block
    f32x16 sacc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) sacc[qb][kb][x] = 0.f;
    constexpr int KSTEP = NS / NL;  // S MFMAs between two refill loads
    // refill load i goes out after S MFMA i * KSTEP + 1 of the 2 * NS: all
    // 2 * NL of them only when KSTEP divides evenly and is at least 2
    static_assert(NS % NL == 0 && KSTEP >= 2, "every refill load must be issued between the S MFMAs");
    auto s_phase = [&](auto with_refill) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (with_refill && (2 * s + kb) % KSTEP == 1) refill((2 * s + kb) / KSTEP);
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kt + lo_.k[s] + kb * 32 * T::ROW_BYTES);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[qb][s], sacc[qb][kb], 0, 0, 0);
            }
        }
        if constexpr (NW == 8 && QB == 1) {
            // each K operand read issued four MFMAs ahead of its use (masks:
            // 0x100 LDS reads, 0x008 MFMAs)
            constexpr int kAhead = 4;
            __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
            for (int i = 0; i < 2 * NS - kAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
        }
    };
    // The 8-wave kernel picks the version with or without refill loads once,
    // so that each is a single basic block over which the reads above can be
    // scheduled ahead; the 4-wave kernel, faster with the plain loop by
    // measurement, tests the condition at each load.
    if constexpr (NW == 8) {
        if (prompt_refill)
            s_phase(std::true_type{});
        else
            s_phase(std::false_type{});
    } else {
        s_phase(prompt_refill);
    }
    // ---- temporal-causal mask, only where response / padding keys occur.
    // This lane's 32 scores belong to response keys off + j (negative: prompt
    // keys), j = 32 kb + 8 (x >> 2) + (x & 3) < 64, so one 64-bit window of
    // the row's key visibility covers them.
    if (base + kTileKeys > P) {
        const int off = base - P + 4 * h;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            uint64_t win;
            if constexpr (MASK == 0) {
                // response keys 0..B-1 are D keys, B..2B-1 their D~ keys
                const uint64_t dk = below[ri.lab[qb]];
                const uint64_t mk = ~dk & low_bits(B);
                win = key_window(off, B == 64 ? dk : (dk | (mk << B)), B == 64 ? mk : (mk >> (64 - B)));
            } else {
                // copies: the prompt keys and the keys of the row's own copy
                const int k0 = ri.lab[qb] * B - off;
                win = low_bits(min(max(-off, 0), 64)) |
                      (low_bits(min(max(k0 + B, 0), 64)) & ~low_bits(min(max(k0, 0), 64)));
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int j = 32 * kb + 8 * (x >> 2) + (x & 3);
                    sacc[qb][kb][x] = ((win >> j) & 1) ? sacc[qb][kb][x] : -INFINITY;
                }
        }
    }
    // ---- the V^T operands of the first PV k-step, read before the softmax so
    // that their LDS latency passes under it (layout: see the PV product)
    const uint32_t vt_off = (uint32_t)(vt - v_stage0);  // 0, 1 or 2 tile sizes
    auto vt_operand = [&](int s, int db) {
        const uint32_t o0 = lo_.v[db] + vt_off + 16 * s * T::ROW_BYTES;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SV_LDS v4i16 *)(uintptr_t)o0);
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SV_LDS v4i16 *)(uintptr_t)(o0 + 8 * T::ROW_BYTES));
        const v4i16 cat[2] = {lo, hi};
        return __builtin_bit_cast(bf16x8, cat);
    };
    bf16x8 va0[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) va0[db] = vt_operand(0, db);
    // ---- online softmax (log2 domain); each lane owns its queries' scores
    bf16x8 pop[QB][4];
    bool rescale = false;
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[qb][kb][x]);
        mx = pair_max<NW>(mx);
        // lazy rescale: the running max moves only when the tile max exceeds
        // it by more than 8 (log2 units); otherwise P = 2^(s - m_run) <= 2^8
        // and the accumulators keep their scale (exact after normalisation)
        const float m_tile = mx * a.scale_log2;
        const float m_new = (m_tile > st.m_run[qb] + 8.f) ? m_tile : st.m_run[qb];
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha[qb] = __builtin_amdgcn_exp2f(st.m_run[qb] - m_use);
        rescale |= alpha[qb] != 1.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x)
                sacc[qb][kb][x] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][x], a.scale_log2, -m_use));
        // P rounded to bf16 is what the PV product uses; the row sum adds the
        // same rounded values, two per dot2 against (1, 1)
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const f32x16 &pp = sacc[qb][kb];
                uint32_t pw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pw[e] = pack_bf16x2(pp[8 * sub + 2 * e], pp[8 * sub + 2 * e + 1]);
                    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[e]), kOnesBf16x2, ls, false);
                }
                pop[qb][2 * kb + sub] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            }
        st.l_run[qb] = st.l_run[qb] * alpha[qb] + ls;
        st.m_run[qb] = m_new;
    }
    if (__any(rescale)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) st.oacc[qb][db][x] *= alpha[qb];
    }
    // ---- O^T += V^T P^T: k-step s covers tile keys 16s..16s+15; lane half h
    // supplies keys 16s+4h+{0..3} and 16s+8+4h+{0..3}.  V^T comes from the
    // row-major V tile through the transposing LDS read: in 16-lane group gq,
    // lane j = 4k + c reads row key(k) at dims dim0 + 4c, and lane i receives
    // the four keys of dim dim0 + i.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const bf16x8 va = s == 0 ? va0[db] : vt_operand(s, db);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                st.oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pop[qb][s], st.oacc[qb][db], 0, 0, 0);
        }
    }
}

// Prologue: start the first tile's direct loads, build the RoPE table while
// they and the query loads are in flight, then the label-threshold table
// (which needs tau), rotate this lane's query rows, and only then start the second
// tile.  The compiler cannot see the direct loads, so its wait for the query
// registers is a full vmcnt(0): issuing the second tile after that wait
// keeps it out of the chip-wide burst that every workgroup waits on before
// its first tile.  LDS regions are __restrict__ parameters (see tile_step).
template <int D, int NW, int QB, int MASK, bool NT>
__device__ __forceinline__ void prologue(const BfArgs &a, int b, int kvh, int t0, const TileMap<MASK> &tm, int jend,
                                         int tau_v,
                                         uint4 (*raw)[D / 16], const bool *rvalid, const int *pos_idx,
                                         bf16x8 (*qop)[D / 16], char *__restrict__ k0, char *__restrict__ v0,
                                         char *__restrict__ k1, char *__restrict__ v1, float2 *__restrict__ cs,
                                         double *__restrict__ invf, uint64_t *__restrict__ below) {
    constexpr int NS = D / 16, NTH = 64 * NW;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5;
    const int B = a.block, P = a.prefix;
    // the first tile (every split has at least one)
    constexpr bool kNt = NT;
    load_tile<D, NW, false, kNt>(a, a.k_cache, a.k_new, b, kvh, tm(t0) * kTileKeys, jend, k0, w, lane);
    load_tile<D, NW, true, kNt>(a, a.v_cache, a.v_new, b, kvh, tm(t0) * kTileKeys, jend, v0, w, lane);
    // RoPE cos/sin table for positions P + 0..B-1 (float64 angles)
    if (a.use_rope) {
        if (tid < D / 2) invf[tid] = rope_inv_freq(tid, D, a.log2_theta);
        ring_barrier();
        for (int idx = tid; idx < B * (D / 2); idx += NTH) {
            const int pr = idx / (D / 2), i = idx % (D / 2);
            cs[pr * kCsStride<D> + i] = rope_cs((double)P + (double)pr, invf[i]);
        }
    }
    if constexpr (MASK == 0) {
        // below[t]: the slots whose step label is below t, one bit per slot
        // (lane k < B of every wave holds the label of slot k)
        for (int t = w; t <= B + 1; t += NW) {
            const uint64_t bits = __ballot(lane < B && tau_v < t);
            if (lane == 0) below[t] = bits;
        }
    }
    ring_barrier();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if (a.use_rope) {
#pragma unroll
            for (int s = 0; s < NS / 2; ++s)
                rotate_pair(raw[qb][s], raw[qb][s + NS / 2], cs + pos_idx[qb] * kCsStride<D> + 16 * s + 8 * h);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qop[qb][s] = __builtin_bit_cast(bf16x8, rvalid[qb] ? raw[qb][s] : make_uint4(0, 0, 0, 0));
    }
    // the second tile (a tile past the end reads clamped rows and is never
    // consumed)
    load_tile<D, NW, false, kNt>(a, a.k_cache, a.k_new, b, kvh, tm(t0 + 1) * kTileKeys, jend, k1, w, lane);
    load_tile<D, NW, true, kNt>(a, a.v_cache, a.v_new, b, kvh, tm(t0 + 1) * kTileKeys, jend, v1, w, lane);
}

// NW waves x QB x 32 query rows per workgroup; 3-deep LDS ring of K/V tiles
// fed by direct global->LDS loads.
template <int D, int NW, int QB, int MASK, bool NT>
__global__ void __launch_bounds__(64 * NW, 1) attn_bf16_kernel(BfArgs a) {
    using T = Tile<D, false>;
    constexpr int NS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int ROWS_W = 32 * QB;
    constexpr int ROWS_B = ROWS_W * NW;
    // one LDS array per ring stage and tensor
    __shared__ __attribute__((aligned(1024))) char k_st0[T::BYTES], k_st1[T::BYTES], k_st2[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char v_st0[T::BYTES], v_st1[T::BYTES], v_st2[T::BYTES];
    __shared__ __attribute__((aligned(16))) float2 cs_lds[kMaxBlock * kCsStride<D>];
    __shared__ double invf_lds[D / 2];
    __shared__ uint64_t below_lds[MASK == 0 ? kMaxBlock + 2 : 1];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int B = a.block, R2 = a.n_resp, g = a.n_qh / a.n_kvh, R = g * R2;

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
    // this sequence's prompt length, and the key tiles of this workgroup
    if (a.prefix_lens) a.prefix = min(max(uniform_ld(a.prefix_lens, b), 0), a.prefix);
    int n_tiles;
    TileMap<MASK> tm{0, 0};
    if constexpr (MASK == 0) {
        n_tiles = (a.prefix + R2 + kTileKeys - 1) / kTileKeys;
    } else {
        // copies cl .. ch hold this workgroup's rows; their keys lie in
        // tiles ra .. rz
        const int cl = (rb * ROWS_B) / (g * B), ch = (min(R, (rb + 1) * ROWS_B) - 1) / (g * B);
        const int n_p = (a.prefix + kTileKeys - 1) / kTileKeys;
        const int ra = max(n_p, (a.prefix + cl * B) / kTileKeys);
        const int rz = (a.prefix + (ch + 1) * B - 1) / kTileKeys;
        tm = TileMap<MASK>{n_p, ra - n_p};
        n_tiles = n_p + max(0, rz - ra + 1);
    }
    const int t0 = split * a.tiles_per_split;
    const int t1 = min(n_tiles, t0 + a.tiles_per_split);
    const int nt = t1 - t0;
    if (nt <= 0) {
        // a split past this sequence's keys: an empty partial (the merge
        // skips it without reading its output rows)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int rho = rb * ROWS_B + w * ROWS_W + qb * 32 + l32;
            if (rho < R && h == 0) {
                const int2 rh = map_row<MASK>(rho, R2, B, g);
                const size_t row = ((size_t)b * R2 + rh.x) * a.n_qh + kvh * g + rh.y;
                a.ws_ml[(size_t)split * a.batch * R2 * a.n_qh + row] = make_float2(-INFINITY, 0.f);
            }
        }
        return;
    }

    // ---- tau (lane k of every wave holds tau[k]) and this lane's query rows:
    // their loads go out before the tiles' so that waiting for them does not
    // drain the tile loads
    const int tau_v = MASK == 0 ? a.tau[(size_t)b * B + min(lane, B - 1)] : 0;
    bool rvalid[QB];
    int rrow[QB], qhead[QB], pos_idx[QB];
    uint4 raw[QB][NS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int rho = rb * ROWS_B + w * ROWS_W + qb * 32 + l32;
        rvalid[qb] = rho < R;
        const int2 rh = map_row<MASK>(rvalid[qb] ? rho : 0, R2, B, g);
        rrow[qb] = rh.x;
        qhead[qb] = kvh * g + rh.y;
        pos_idx[qb] = rrow[qb] % B;
        const uint16_t *qp = a.q + (((size_t)b * R2 + rrow[qb]) * a.n_qh + qhead[qb]) * D + 8 * h;
#pragma unroll
        for (int s = 0; s < NS; ++s) raw[qb][s] = *reinterpret_cast<const uint4 *>(qp + 16 * s);  // valid row
    }
    const int jend = min(a.prefix + R2, (tm(t1 - 1) + 1) * kTileKeys);  // end of this workgroup's keys
    bf16x8 qop[QB][NS];
    prologue<D, NW, QB, MASK, NT>(a, b, kvh, t0, tm, jend, tau_v, raw, rvalid, pos_idx, qop, k_st0, v_st0, k_st1, v_st1, cs_lds,
                        invf_lds, below_lds);
    RowInfo<QB> ri;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if constexpr (MASK == 0)
            ri.lab[qb] = min(max(__shfl(tau_v, pos_idx[qb]), 0), B) + (rrow[qb] < B ? 1 : 0);
        else
            ri.lab[qb] = rrow[qb] / B;  // the row's copy
    }
    ri.c_lo = 0;
    ri.c_hi = R2 / B - 1;
    if constexpr (MASK == 1) {
        // rows rho0 .. rho1 of this wave belong to copies rho0 / (g B) ..
        // rho1 / (g B) (rows are copy-major)
        const int rho0 = __builtin_amdgcn_readfirstlane(rb * ROWS_B + w * ROWS_W);
        const int rho1 = min(rho0 + ROWS_W, R) - 1;
        if (rho0 < R) {
            ri.c_lo = rho0 / (g * B);
            ri.c_hi = rho1 / (g * B);
        }
    }
    const LdsOffs<D> offs = lds_offsets<D>(lane, v_st0);
    const LoadOffs<D, NW> ldo = load_offsets<D, NW>(w, lane);
    const size_t unit_off = ((size_t)b * a.n_kvh + kvh) * a.page_size * D;  // contiguous cache only
    const bool wave_active = (rb * ROWS_B + w * ROWS_W) < R;

    RowState<D, QB> st;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int x = 0; x < 16; ++x) st.oacc[qb][db][x] = 0.f;
        st.m_run[qb] = -INFINITY;
        st.l_run[qb] = 0.f;
    }

    for (int it = 0; it < nt; it += 3) {
        tile_step<D, NW, QB, MASK, NT>(a, b, kvh, t0, nt, it, wave_active, ri, offs, qop, st, k_st0, v_st0, k_st2, v_st2,
                             cs_lds, below_lds, v_st0, ldo, unit_off, tm, jend);
        if (it + 1 < nt)
            tile_step<D, NW, QB, MASK, NT>(a, b, kvh, t0, nt, it + 1, wave_active, ri, offs, qop, st, k_st1, v_st1, k_st0,
                                 v_st0, cs_lds, below_lds, v_st0, ldo, unit_off, tm, jend);
        if (it + 2 < nt)
            tile_step<D, NW, QB, MASK, NT>(a, b, kvh, t0, nt, it + 2, wave_active, ri, offs, qop, st, k_st2, v_st2, k_st1,
                                 v_st1, cs_lds, below_lds, v_st0, ldo, unit_off, tm, jend);
    }
    wait_vmcnt<0>();  // no direct load may still target this workgroup's LDS when it exits

    if (!wave_active) return;
    // ---- epilogue: lane owns query l32 of each block; O^T rows dim = db*32 + 8*jj + 4*h + i
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32);
        if (!rvalid[qb]) continue;
        const size_t row = ((size_t)b * R2 + rrow[qb]) * a.n_qh + qhead[qb];
        if (a.n_split == 1) {
            const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
            uint16_t *op = a.out + row * D + 4 * h;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const f32x16 &o = st.oacc[qb][db];
                    uint2 pk;
                    pk.x = pack_bf16x2(o[4 * jj + 0] * inv, o[4 * jj + 1] * inv);
                    pk.y = pack_bf16x2(o[4 * jj + 2] * inv, o[4 * jj + 3] * inv);
                    *reinterpret_cast<uint2 *>(op + db * 32 + 8 * jj) = pk;
                }
        } else {
            const size_t prow = (size_t)split * a.batch * R2 * a.n_qh + row;
            // the merge weights are non-negative and sum to one over the
            // splits, so rounding each partial to bf16 adds at most one
            // bf16 rounding (2^-9 relative) to the merged row
            uint16_t *op = a.ws_o + prow * D + 4 * h;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const f32x16 &o = st.oacc[qb][db];
                    uint2 pk;
                    pk.x = pack_bf16x2(o[4 * jj + 0], o[4 * jj + 1]);
                    pk.y = pack_bf16x2(o[4 * jj + 2], o[4 * jj + 3]);
                    *reinterpret_cast<uint2 *>(op + db * 32 + 8 * jj) = pk;
                }
            if (h == 0) a.ws_ml[prow] = make_float2(st.m_run[qb], l_tot);
        }
    }
}

// Merge prefix splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per (row, head, 4 dims): the split partials of one row are
// independent loads (unrolled, so many are in flight), and the 32 threads of
// a row read the same (m, l) entries as one broadcast.
template <typename T>
__global__ void __launch_bounds__(256) attn_combine_kernel(const uint16_t *__restrict__ ws_o,
                                                           const float2 *__restrict__ ws_ml, T *out,
                                                           int n_split, size_t rows_total, int d) {
    const int d4 = d >> 2;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows_total * d4) return;
    const size_t row = gid / d4;
    const int e = (int)(gid % d4) * 4;
    float M = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, ws_ml[s * rows_total + row].x);
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
#pragma unroll 8
    for (int s = 0; s < n_split; ++s) {
        const float2 ml = ws_ml[s * rows_total + row];
        if (ml.x == -INFINITY) continue;  // no visible key in this split (or an empty split)
        const uint2 pk = *reinterpret_cast<const uint2 *>(ws_o + (s * rows_total + row) * d + e);
        const float4 o = make_float4(__uint_as_float(pk.x << 16), __uint_as_float(pk.x & 0xFFFF0000u),
                                     __uint_as_float(pk.y << 16), __uint_as_float(pk.y & 0xFFFF0000u));
        const float f = __builtin_amdgcn_exp2f(ml.x - M);
        den += f * ml.y;
        num.x += f * o.x;
        num.y += f * o.y;
        num.z += f * o.z;
        num.w += f * o.w;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    st_elem(out, row * d + e + 0, num.x * inv);
    st_elem(out, row * d + e + 1, num.y * inv);
    st_elem(out, row * d + e + 2, num.z * inv);
    st_elem(out, row * d + e + 3, num.w * inv);
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
    p.rows = g * s.n_resp;
    // 32 query rows per wave; 8 waves when a kv head has more than 128 rows
    p.qb = 1;
    p.nw = p.rows > 128 ? 8 : 4;
    p.n_rb = (p.rows + 32 * p.qb * p.nw - 1) / (32 * p.qb * p.nw);
    const int nk = s.prefix + s.n_resp;
    p.n_tiles = (nk + kTileKeys - 1) / kTileKeys;
    p.n_split = 1;
    p.tiles_per_split = p.n_tiles;
    if (s.dtype == 1) {
        // aim for about one workgroup per compute unit (256 CUs) -- unless
        // a workgroup would stream only a few tiles anyway, where the merge
        // launch and the partials cost more than the idle compute units: 64
        // units of 5 tiles (a 256-key prompt) take 19.1 us unsplit and 20.5
        // split, of 7 tiles 22.0 and 20.2 us
        const long units = (long)s.batch * s.n_kvh * p.n_rb;
        if (units < 256 && p.n_tiles > 6) {
            int want = (int)((256 + units - 1) / units);
            want = want < p.n_tiles / 2 ? want : p.n_tiles / 2;
            if (want > 1) {
                p.tiles_per_split = (p.n_tiles + want - 1) / want;
                p.n_split = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
            }
        }
        if (p.n_split > 1) {
            const size_t rows = (size_t)p.n_split * s.batch * s.n_resp * s.n_qh;
            p.ws_partial_o = align_up(rows * s.head_dim * sizeof(uint16_t));
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

template <int MASK, bool NT>
void launch_bf16(int head_dim, int nw, unsigned grid, dim3 blk, hipStream_t st, const BfArgs &a) {
    if (head_dim == 128 && nw == 8) hipLaunchKernelGGL((attn_bf16_kernel<128, 8, 1, MASK, NT>), dim3(grid), blk, 0, st, a);
    else if (head_dim == 128) hipLaunchKernelGGL((attn_bf16_kernel<128, 4, 1, MASK, NT>), dim3(grid), blk, 0, st, a);
    else if (nw == 8) hipLaunchKernelGGL((attn_bf16_kernel<64, 8, 1, MASK, NT>), dim3(grid), blk, 0, st, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, 4, 1, MASK, NT>), dim3(grid), blk, 0, st, a);
}

hipError_t launch_attn(const AttnShape &s, const AttnPlan &p, const void *q, const void *k_new,
                       const void *v_new, const void *k_cache, const void *v_cache,
                       const int32_t *tau, void *out, double theta, float scale, void *ws,
                       hipStream_t st, const CacheView &cv) {
    const int R2 = s.n_resp;
    if (s.dtype == 1) {
        BfArgs a{};
        a.q = (const uint16_t *)q;
        a.k_new = (const uint16_t *)k_new;
        a.v_new = (const uint16_t *)v_new;
        a.k_cache = (const uint16_t *)k_cache;
        a.v_cache = (const uint16_t *)v_cache;
        a.tau = tau;
        a.out = (uint16_t *)out;
        a.ws_o = p.n_split > 1 ? (uint16_t *)ws : nullptr;
        a.ws_ml = p.n_split > 1 ? (float2 *)((char *)ws + p.ws_partial_o) : nullptr;
        a.batch = s.batch;
        a.block = s.block;
        a.prefix = s.prefix;
        a.n_qh = s.n_qh;
        a.n_kvh = s.n_kvh;
        a.n_rb = p.n_rb;
        a.n_split = p.n_split;
        a.tiles_per_split = p.tiles_per_split;
        a.n_resp = s.n_resp;
        a.prefix_lens = cv.prefix_lens;
        a.block_table = cv.block_table;
        a.page_size = cv.page_size > 0 ? cv.page_size : s.prefix;
        a.max_pages = cv.max_pages;
        a.n_pages = cv.n_pages;
        a.use_rope = theta > 0 ? 1 : 0;
        a.log2_theta = theta > 0 ? log2(theta) : 0.0;
        a.scale_log2 = scale * kLog2e;
        const unsigned grid = (unsigned)((size_t)s.batch * s.n_kvh * p.n_rb * p.n_split);
        const dim3 blk(64 * p.nw);
        // non-temporal tile loads when each kv head's K/V is read by one
        // row block only; with several row blocks the later ones find the
        // prompt tiles in L2
        const bool nt = p.n_rb == 1;
        if (s.mask == 0) {
            if (nt) launch_bf16<0, true>(s.head_dim, p.nw, grid, blk, st, a);
            else launch_bf16<0, false>(s.head_dim, p.nw, grid, blk, st, a);
        } else {
            if (nt) launch_bf16<1, true>(s.head_dim, p.nw, grid, blk, st, a);
            else launch_bf16<1, false>(s.head_dim, p.nw, grid, blk, st, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.n_split == 1) return e;
        const size_t rows_total = (size_t)s.batch * R2 * s.n_qh;
        const size_t threads = rows_total * (size_t)(s.head_dim / 4);
        hipLaunchKernelGGL(attn_combine_kernel<uint16_t>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           st, (const uint16_t *)a.ws_o, (const float2 *)a.ws_ml, (uint16_t *)out, p.n_split,
                           rows_total, s.head_dim);
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
