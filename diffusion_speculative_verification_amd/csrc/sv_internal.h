// sv_internal.h -- host-side plans and launchers shared by the translation
// units of libspecverify.so (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kTileKeys = 64;        // keys per attention tile
constexpr int kMaxBlock = 64;        // largest block size B
constexpr int kMaxResp = 1024;       // largest number of response rows (copies * block)
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct AttnShape {
    int dtype, batch, block, prefix, n_qh, n_kvh, head_dim;
    int n_resp;  // response rows per sequence: 2 * block (paired layout) or copies * block
    int mask;    // 0: temporal mask from tau; 1: copies, each bidirectional over its own block
};

struct AttnPlan {
    int rows;            // rows per kv head = (n_qh / n_kvh) * n_resp
    int nw;              // waves per workgroup
    int qb;              // 32-row query blocks per wave
    int n_rb;            // row blocks of 32 * qb * nw rows per kv head
    int n_tiles;         // key tiles over prefix + n_resp keys (the longest prompt)
    int n_split;         // prefix splits (1 = no combine pass)
    int tiles_per_split;
    size_t ws_partial_o;   // bytes of split partial outputs (bf16)
    size_t ws_partial_ml;  // bytes of split (max, sum) pairs
    size_t ws_rope;        // bytes of rotated q/k copies (float32 path)
    size_t ws_total;
};

AttnPlan attn_plan(const AttnShape &s);

hipError_t launch_rope(const void *q_in, const void *k_in, void *q_out, void *k_out, int dtype,
                       int batch, int block, int n_qh, int n_kvh, int head_dim, int prefix,
                       double theta, hipStream_t st);

// Addressing of the prompt K/V cache.  Default: contiguous
// [batch][n_kvh][prefix][d], every sequence with `prefix` prompt keys.  With
// a block table: pages [n_pages][n_kvh][page_size][d] (page_size a multiple
// of 64), row j of sequence b in page block_table[b * max_pages + j /
// page_size].  Without a table and page_size > 0: contiguous with row stride
// page_size.  prefix_lens: per-sequence prompt lengths (<= prefix).
struct CacheView {
    const int32_t *prefix_lens = nullptr, *block_table = nullptr;
    int page_size = 0, max_pages = 0, n_pages = 0;
};

hipError_t launch_attn(const AttnShape &s, const AttnPlan &p, const void *q, const void *k_new,
                       const void *v_new, const void *k_cache, const void *v_cache,
                       const int32_t *tau, void *out, double theta, float scale, void *ws,
                       hipStream_t st, const CacheView &cv = CacheView());

struct AcceptPlan {
    int rows;        // batch * block logits rows
    int n_vsplit;    // vocab splits of the normaliser pass
    int64_t chunk;   // vocab elements per residual workgroup
    int n_chunk;     // residual workgroups per sequence
    int n_pick;      // published residual sums per sequence (half chunks)
    size_t off_part, off_gath, off_res, off_chunk, ws_total;
};

AcceptPlan accept_plan(int batch, int block, int gamma, int64_t vocab);

hipError_t launch_accept(const AcceptPlan &p, const float *logits, const float *probs,
                         const int32_t *tokens, const int32_t *tau, const float *u, int batch,
                         int block, int gamma, int64_t vocab, float inv_t, int32_t *accept_len,
                         int32_t *out_tokens, float *alpha, void *ws, hipStream_t st);

struct CoupledPlan {
    int rows;        // batch * block logits rows
    int n_vsplit;    // vocab splits of the streaming argmax
    size_t ws_total;
};

CoupledPlan coupled_plan(int batch, int block, int gamma, int64_t vocab);

hipError_t launch_coupled(const CoupledPlan &p, const float *logits, const float *noise, const int32_t *tokens,
                          const int32_t *tau, int batch, int block, int gamma, int64_t vocab, float inv_t,
                          int32_t *accept_len, int32_t *out_tokens, int32_t *target_tokens, void *ws,
                          hipStream_t st);

struct RoutePlan {
    int rows;        // batch * block draft rows
    int n_vsplit;    // vocab splits of the streaming reduction
    size_t ws_total;
};

RoutePlan route_plan(int batch, int block, int gamma, int64_t vocab);

hipError_t launch_route(const RoutePlan &p, const float *probs, const int32_t *tau, int batch, int block,
                        int gamma, int64_t vocab, int estimator, double param, float *khat, float *alpha_hat,
                        void *ws, hipStream_t st);

hipError_t launch_tree(const CoupledPlan &p, const float *logits, const float *noise, const int32_t *parent,
                       const int32_t *node_pos, const int32_t *node_tok, const int32_t *target_pos, int batch,
                       int n_nodes, int64_t vocab, float inv_t, int32_t *path_len, int32_t *path, int32_t *commit_pos,
                       int32_t *commit_tok, int32_t *target_tok, void *ws, hipStream_t st);

struct StatesPlan {
    long long rows;  // batch * n_nodes * block logits rows
    int n_vsplit;    // vocab splits of the streaming pass
    size_t ws_total;
};

StatesPlan states_plan(int batch, int n_nodes, int block, int64_t vocab);

hipError_t launch_states(const StatesPlan &p, const float *logits, const float *noise, const int32_t *parent,
                         const int32_t *state, int batch, int n_nodes, int block, int64_t vocab, float inv_t,
                         float threshold, int32_t *path_len, int32_t *path, int32_t *next_state, int32_t *commit,
                         float *conf, void *ws, hipStream_t st);

hipError_t launch_check_tau(const int32_t *tau, int batch, int block, int32_t *bad, hipStream_t st);

hipError_t launch_commit(const int32_t *out_tokens, int32_t *block_tokens, int batch, int block, int gamma,
                         int32_t *remaining, int32_t *state, int32_t *n_append, hipStream_t st);

hipError_t launch_append(const void *k_rows, const void *v_rows, int src_stride, const int32_t *n_append,
                         void *k_pages, void *v_pages, const int32_t *block_table, int32_t *prefix_lens,
                         int32_t *status, int batch, int page_size, int max_pages, int n_pages, int n_kvh,
                         int head_dim, double theta, hipStream_t st);

}  // namespace sv
