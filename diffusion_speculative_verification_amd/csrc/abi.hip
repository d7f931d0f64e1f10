// abi.hip -- extern "C" entry points of libspecverify.so: host-side argument
// checks, workspace sizing and launches on the caller's stream.  No entry
// point allocates, synchronises or keeps state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/spec_verify.h"
#include "sv_internal.h"

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_heads(int dtype, int batch, int block, int n_qh, int n_kvh, int head_dim, int prefix) {
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_E_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return SV_E_UNSUPPORTED;
    if (batch < 1 || block < 1 || block > 64 || n_qh < 1 || n_kvh < 1 || prefix < 0) return SV_E_SHAPE;
    if (n_qh % n_kvh) return SV_E_SHAPE;
    // index arithmetic of the kernels stays within 32-bit grid sizes
    if ((long long)batch * 2 * block * n_qh > (1ll << 30)) return SV_E_SHAPE;
    if ((long long)prefix + 2 * block > (1ll << 30)) return SV_E_SHAPE;
    return SV_OK;
}

int map_launch(hipError_t e) { return e == hipSuccess ? SV_OK : SV_E_LAUNCH; }

// the vocabulary-streaming calls: batch x rows (slots or nodes) x vocab
// within the kernels' index ranges (grids of rows x vocab splits stay below
// 2^31 workgroups)
bool rows_ok(int batch, int rows, int64_t vocab) {
    return (long long)batch * rows <= (1ll << 26) && (long long)batch * rows * vocab <= (1ll << 40);
}

}  // namespace

extern "C" {

int spec_verify_abi_version(void) { return SPEC_VERIFY_ABI_VERSION; }

const char *spec_verify_status_string(int status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_E_NULL: return "a required pointer is NULL";
        case SV_E_SHAPE: return "a size is out of range or inconsistent";
        case SV_E_UNSUPPORTED: return "unsupported dtype or head_dim";
        case SV_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case SV_E_WORKSPACE: return "workspace missing or too small";
        case SV_E_LAUNCH: return "kernel launch failed";
        case SV_E_INVALID_TAU: return "tau is not a permutation of 1..block";
        case SV_E_SCRATCH:
            return "the sizes need more scratch than the library's static buffer holds "
                   "(SPEC_VERIFY_SCRATCH_BYTES); use the call that takes a workspace";
        default: return "unknown status";
    }
}

int spec_verify_rope(const void *q_in, const void *k_in, void *q_out, void *k_out, int dtype, int batch,
                     int block, int n_qh, int n_kvh, int head_dim, int prefix_len, double theta,
                     void *stream) {
    int rc = check_heads(dtype, batch, block, n_qh, n_kvh, head_dim, prefix_len);
    if (rc) return rc;
    if (!q_in || !k_in || !q_out || !k_out) return SV_E_NULL;
    if (!(theta > 0) || !isfinite(theta)) return SV_E_SHAPE;
    if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out)) return SV_E_ALIGN;
    return map_launch(sv::launch_rope(q_in, k_in, q_out, k_out, dtype, batch, block, n_qh, n_kvh, head_dim,
                                      prefix_len, theta, (hipStream_t)stream));
}

size_t spec_verify_attn_workspace_size(int dtype, int batch, int block, int prefix_len, int n_qh, int n_kvh,
                                       int head_dim) {
    if (check_heads(dtype, batch, block, n_qh, n_kvh, head_dim, prefix_len)) return 0;
    sv::AttnShape s{dtype, batch, block, prefix_len, n_qh, n_kvh, head_dim, 2 * block, 0};
    return sv::attn_plan(s).ws_total;
}

int spec_verify_attn(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                     const void *v_cache, const int32_t *tau, void *out, int dtype, int batch, int block,
                     int prefix_len, int n_qh, int n_kvh, int head_dim, double rope_theta,
                     float softmax_scale, void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_heads(dtype, batch, block, n_qh, n_kvh, head_dim, prefix_len);
    if (rc) return rc;
    if (!q || !k_new || !v_new || !tau || !out) return SV_E_NULL;
    if (prefix_len > 0 && (!k_cache || !v_cache)) return SV_E_NULL;
    if (!isfinite(rope_theta) || !isfinite(softmax_scale)) return SV_E_SHAPE;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) || !aligned16(tau))
        return SV_E_ALIGN;
    if (prefix_len > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) return SV_E_ALIGN;
    sv::AttnShape s{dtype, batch, block, prefix_len, n_qh, n_kvh, head_dim, 2 * block, 0};
    const sv::AttnPlan p = sv::attn_plan(s);
    const bool need_ws = (dtype == SV_BF16) ? p.n_split > 1 : rope_theta > 0;
    if (need_ws && (!workspace || workspace_bytes < p.ws_total)) return SV_E_WORKSPACE;
    if (need_ws && !aligned16(workspace)) return SV_E_ALIGN;
    const float scale = softmax_scale > 0 ? softmax_scale : (float)(1.0 / sqrt((double)head_dim));
    return map_launch(sv::launch_attn(s, p, q, k_new, v_new, k_cache, v_cache, tau, out, rope_theta, scale,
                                      workspace, (hipStream_t)stream));
}

namespace {
int check_copies(int dtype, int batch, int block, int n_copies, int n_qh, int n_kvh, int head_dim, int prefix) {
    if (dtype != SV_BF16) return SV_E_UNSUPPORTED;
    int rc = check_heads(dtype, batch, block, n_qh, n_kvh, head_dim, prefix);
    if (rc) return rc;
    if (n_copies < 1 || (long long)n_copies * block > sv::kMaxResp) return SV_E_SHAPE;
    if ((long long)batch * n_copies * block * n_qh > (1ll << 30)) return SV_E_SHAPE;
    if ((long long)prefix + (long long)n_copies * block > (1ll << 30)) return SV_E_SHAPE;
    return SV_OK;
}
}  // namespace

size_t spec_verify_attn_copies_workspace_size(int dtype, int batch, int block, int n_copies, int prefix_len,
                                              int n_qh, int n_kvh, int head_dim) {
    if (check_copies(dtype, batch, block, n_copies, n_qh, n_kvh, head_dim, prefix_len)) return 0;
    sv::AttnShape s{dtype, batch, block, prefix_len, n_qh, n_kvh, head_dim, n_copies * block, 1};
    return sv::attn_plan(s).ws_total;
}

int spec_verify_attn_copies(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                            const void *v_cache, void *out, int dtype, int batch, int block, int n_copies,
                            int prefix_len, int n_qh, int n_kvh, int head_dim, double rope_theta,
                            float softmax_scale, void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_copies(dtype, batch, block, n_copies, n_qh, n_kvh, head_dim, prefix_len);
    if (rc) return rc;
    if (!q || !k_new || !v_new || !out) return SV_E_NULL;
    if (prefix_len > 0 && (!k_cache || !v_cache)) return SV_E_NULL;
    if (!isfinite(rope_theta) || !isfinite(softmax_scale)) return SV_E_SHAPE;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return SV_E_ALIGN;
    if (prefix_len > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) return SV_E_ALIGN;
    sv::AttnShape s{dtype, batch, block, prefix_len, n_qh, n_kvh, head_dim, n_copies * block, 1};
    const sv::AttnPlan p = sv::attn_plan(s);
    if (p.n_split > 1 && (!workspace || workspace_bytes < p.ws_total)) return SV_E_WORKSPACE;
    if (p.n_split > 1 && !aligned16(workspace)) return SV_E_ALIGN;
    const float scale = softmax_scale > 0 ? softmax_scale : (float)(1.0 / sqrt((double)head_dim));
    return map_launch(sv::launch_attn(s, p, q, k_new, v_new, k_cache, v_cache, nullptr, out, rope_theta, scale,
                                      workspace, (hipStream_t)stream));
}

namespace {
// the response layout of the paged call: n_copies == 0 is the paired layout
int check_paged(int dtype, int batch, int block, int n_copies, int n_qh, int n_kvh, int head_dim, int max_prefix) {
    if (dtype != SV_BF16) return SV_E_UNSUPPORTED;
    if (n_copies < 0) return SV_E_SHAPE;
    return n_copies == 0 ? check_heads(dtype, batch, block, n_qh, n_kvh, head_dim, max_prefix)
                         : check_copies(dtype, batch, block, n_copies, n_qh, n_kvh, head_dim, max_prefix);
}

sv::AttnShape paged_shape(int dtype, int batch, int block, int n_copies, int max_prefix, int n_qh, int n_kvh,
                          int head_dim) {
    return sv::AttnShape{dtype, batch, block, max_prefix, n_qh, n_kvh, head_dim,
                         n_copies == 0 ? 2 * block : n_copies * block, n_copies == 0 ? 0 : 1};
}
}  // namespace

size_t spec_verify_attn_paged_workspace_size(int dtype, int batch, int block, int n_copies, int max_prefix,
                                             int n_qh, int n_kvh, int head_dim) {
    if (check_paged(dtype, batch, block, n_copies, n_qh, n_kvh, head_dim, max_prefix)) return 0;
    return sv::attn_plan(paged_shape(dtype, batch, block, n_copies, max_prefix, n_qh, n_kvh, head_dim)).ws_total;
}

int spec_verify_attn_paged(const void *q, const void *k_new, const void *v_new, const void *k_pages,
                           const void *v_pages, const int32_t *block_table, const int32_t *prefix_lens,
                           const int32_t *tau, void *out, int dtype, int batch, int block, int n_copies,
                           int max_prefix, int page_size, int max_pages, int n_pages, int n_qh, int n_kvh,
                           int head_dim, double rope_theta, float softmax_scale, void *workspace,
                           size_t workspace_bytes, void *stream) {
    int rc = check_paged(dtype, batch, block, n_copies, n_qh, n_kvh, head_dim, max_prefix);
    if (rc) return rc;
    if (block_table) {
        if (page_size < 64 || page_size % 64 != 0 || max_pages < 1 || n_pages < 1) return SV_E_SHAPE;
        if ((long long)max_pages * page_size < max_prefix) return SV_E_SHAPE;
        if ((long long)batch * max_pages > (1ll << 31) - 1) return SV_E_SHAPE;
    } else {
        if (page_size == 0) page_size = max_prefix;
        if (page_size < max_prefix) return SV_E_SHAPE;
    }
    if (!q || !k_new || !v_new || !out || (n_copies == 0 && !tau)) return SV_E_NULL;
    if (max_prefix > 0 && (!k_pages || !v_pages)) return SV_E_NULL;
    if (!isfinite(rope_theta) || !isfinite(softmax_scale)) return SV_E_SHAPE;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return SV_E_ALIGN;
    if (max_prefix > 0 && (!aligned16(k_pages) || !aligned16(v_pages))) return SV_E_ALIGN;
    const sv::AttnShape s = paged_shape(dtype, batch, block, n_copies, max_prefix, n_qh, n_kvh, head_dim);
    const sv::AttnPlan p = sv::attn_plan(s);
    if (p.n_split > 1 && (!workspace || workspace_bytes < p.ws_total)) return SV_E_WORKSPACE;
    if (p.n_split > 1 && !aligned16(workspace)) return SV_E_ALIGN;
    sv::CacheView cv;
    cv.prefix_lens = prefix_lens;
    cv.block_table = block_table;
    cv.page_size = page_size;
    cv.max_pages = block_table ? max_pages : 0;
    cv.n_pages = block_table ? n_pages : 0;
    const float scale = softmax_scale > 0 ? softmax_scale : (float)(1.0 / sqrt((double)head_dim));
    return map_launch(sv::launch_attn(s, p, q, k_new, v_new, k_pages, v_pages, n_copies == 0 ? tau : nullptr, out,
                                      rope_theta, scale, workspace, (hipStream_t)stream, cv));
}

int spec_verify_check_tau(const int32_t *tau, int batch, int block, int32_t *bad, void *stream) {
    if (batch < 1 || block < 1 || block > 64) return SV_E_SHAPE;
    if (!tau || !bad) return SV_E_NULL;
    return map_launch(sv::launch_check_tau(tau, batch, block, bad, (hipStream_t)stream));
}

int spec_verify_commit(const int32_t *out_tokens, int32_t *block_tokens, int batch, int block, int gamma,
                       int32_t *remaining, int32_t *state, int32_t *n_append, void *stream) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block) return SV_E_SHAPE;
    if ((long long)batch * block > (1ll << 31) - 1) return SV_E_SHAPE;
    if (!out_tokens || !block_tokens || !remaining || !state || !n_append) return SV_E_NULL;
    return map_launch(sv::launch_commit(out_tokens, block_tokens, batch, block, gamma, remaining, state, n_append,
                                        (hipStream_t)stream));
}

int spec_verify_kv_append(const void *k_rows, const void *v_rows, int src_stride, const int32_t *n_append,
                          void *k_pages, void *v_pages, const int32_t *block_table, int32_t *prefix_lens,
                          int32_t *status, int dtype, int batch, int page_size, int max_pages, int n_pages,
                          int n_kvh, int head_dim, double rope_theta, void *stream) {
    if (dtype != SV_BF16) return SV_E_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return SV_E_UNSUPPORTED;
    if (batch < 1 || src_stride < 1 || n_kvh < 1 || page_size < 1) return SV_E_SHAPE;
    if ((long long)batch * n_kvh > (1ll << 31) - 1) return SV_E_SHAPE;
    if (block_table && (max_pages < 1 || n_pages < 1)) return SV_E_SHAPE;
    if (!isfinite(rope_theta)) return SV_E_SHAPE;
    if (!k_rows || !v_rows || !n_append || !k_pages || !v_pages || !prefix_lens) return SV_E_NULL;
    if (!aligned16(k_rows) || !aligned16(v_rows) || !aligned16(k_pages) || !aligned16(v_pages)) return SV_E_ALIGN;
    return map_launch(sv::launch_append(k_rows, v_rows, src_stride, n_append, k_pages, v_pages, block_table,
                                        prefix_lens, status, batch, page_size, block_table ? max_pages : 1,
                                        block_table ? n_pages : batch, n_kvh, head_dim, rope_theta,
                                        (hipStream_t)stream));
}

size_t spec_verify_accept_workspace_size(int batch, int block, int gamma, int64_t vocab) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21) || !rows_ok(batch, block, vocab))
        return 0;
    return sv::accept_plan(batch, block, gamma, vocab).ws_total;
}

namespace {
int accept_impl(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                const int32_t *tau, const float *uniforms, int batch, int block, int gamma, int64_t vocab,
                float inv_t, int32_t *accept_len, int32_t *out_tokens, float *alpha, void *workspace,
                size_t workspace_bytes, void *stream) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21))
        return SV_E_SHAPE;
    if (!rows_ok(batch, block, vocab)) return SV_E_SHAPE;
    if (!target_logits || !draft_probs || !draft_tokens || !tau || !uniforms || !accept_len || !out_tokens)
        return SV_E_NULL;
    if (!aligned16(target_logits) || !aligned16(draft_probs) || !aligned16(draft_tokens) || !aligned16(tau) ||
        !aligned16(uniforms) || !aligned16(accept_len) || !aligned16(out_tokens) || (alpha && !aligned16(alpha)))
        return SV_E_ALIGN;
    const sv::AcceptPlan p = sv::accept_plan(batch, block, gamma, vocab);
    if (!workspace || workspace_bytes < p.ws_total) return SV_E_WORKSPACE;
    if (!aligned16(workspace)) return SV_E_ALIGN;
    return map_launch(sv::launch_accept(p, target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block,
                                        gamma, vocab, inv_t, accept_len, out_tokens, alpha, workspace,
                                        (hipStream_t)stream));
}
}  // namespace

int spec_verify_accept(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                       const int32_t *tau, const float *uniforms, int batch, int block, int gamma,
                       int64_t vocab, int32_t *accept_len, int32_t *out_tokens, float *alpha, void *workspace,
                       size_t workspace_bytes, void *stream) {
    return accept_impl(target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block, gamma, vocab, 1.0f,
                       accept_len, out_tokens, alpha, workspace, workspace_bytes, stream);
}

int spec_verify_accept_temperature(const float *target_logits, const float *draft_probs,
                                   const int32_t *draft_tokens, const int32_t *tau, const float *uniforms, int batch,
                                   int block, int gamma, int64_t vocab, float temperature, int32_t *accept_len,
                                   int32_t *out_tokens, float *alpha, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (!(temperature > 0.f) || !isfinite(temperature)) return SV_E_SHAPE;
    // 1/T rounded to float32 once, here: the kernels and the definition use
    // the same reciprocal
    const float inv_t = 1.0f / temperature;
    if (!isfinite(inv_t)) return SV_E_SHAPE;
    return accept_impl(target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block, gamma, vocab, inv_t,
                       accept_len, out_tokens, alpha, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free verification epilogue.  Its scratch memory (the normaliser
// partials, draft-token gathers, rejected-slot records and residual chunk
// sums that spec_verify_accept keeps in the caller's workspace) is this
// file-scope device array: every GPU the library runs on holds its own copy
// from first use until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is taken
// once per device with hipGetSymbolAddress and only that address is passed
// to the kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[SPEC_VERIFY_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];  // device address of `scratch` per device, NULL until taken

// Device address of the current device's `scratch`, taken on the first call
// on that device (with the device current); NULL if it cannot be obtained.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int spec_verify_accept_noalloc(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                               const int32_t *tau, const float *uniforms, int batch, int block, int gamma,
                               int64_t vocab, int32_t *accept_len, int32_t *out_tokens, float *alpha, void *stream) {
    // the same host checks as spec_verify_accept, before anything else
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21))
        return SV_E_SHAPE;
    if (!rows_ok(batch, block, vocab)) return SV_E_SHAPE;
    if (!target_logits || !draft_probs || !draft_tokens || !tau || !uniforms || !accept_len || !out_tokens)
        return SV_E_NULL;
    if (!aligned16(target_logits) || !aligned16(draft_probs) || !aligned16(draft_tokens) || !aligned16(tau) ||
        !aligned16(uniforms) || !aligned16(accept_len) || !aligned16(out_tokens) || (alpha && !aligned16(alpha)))
        return SV_E_ALIGN;
    const sv::AcceptPlan p = sv::accept_plan(batch, block, gamma, vocab);
    if (p.ws_total > (size_t)SPEC_VERIFY_SCRATCH_BYTES) return SV_E_SCRATCH;
    void *ws = device_scratch();
    if (!ws) return SV_E_LAUNCH;
    // every scratch entry a kernel reads is written earlier in the same call
    // (the workspace variant gets uninitialised memory too): nothing to clear
    return map_launch(sv::launch_accept(p, target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block,
                                        gamma, vocab, 1.0f, accept_len, out_tokens, alpha, ws, (hipStream_t)stream));
}

size_t spec_verify_accept_coupled_workspace_size(int batch, int block, int gamma, int64_t vocab) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21) || !rows_ok(batch, block, vocab))
        return 0;
    return sv::coupled_plan(batch, block, gamma, vocab).ws_total;
}

int spec_verify_accept_coupled(const float *target_logits, const float *gumbel, const int32_t *draft_tokens,
                               const int32_t *tau, int batch, int block, int gamma, int64_t vocab,
                               float temperature, int32_t *accept_len, int32_t *out_tokens,
                               int32_t *target_tokens, void *workspace, size_t workspace_bytes, void *stream) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21))
        return SV_E_SHAPE;
    if (!rows_ok(batch, block, vocab)) return SV_E_SHAPE;
    if (!(temperature >= 0.f) || !isfinite(temperature)) return SV_E_SHAPE;
    if (!target_logits || !draft_tokens || !tau || !accept_len || !out_tokens) return SV_E_NULL;
    if (temperature > 0.f && !gumbel) return SV_E_NULL;
    if (!aligned16(target_logits) || (gumbel && !aligned16(gumbel)) || !aligned16(draft_tokens) ||
        !aligned16(tau) || !aligned16(accept_len) || !aligned16(out_tokens) ||
        (target_tokens && !aligned16(target_tokens)))
        return SV_E_ALIGN;
    const sv::CoupledPlan p = sv::coupled_plan(batch, block, gamma, vocab);
    if (!workspace || workspace_bytes < p.ws_total) return SV_E_WORKSPACE;
    if (!aligned16(workspace)) return SV_E_ALIGN;
    // 1/T rounded to float32 once, here: the kernels and the definition use
    // the same reciprocal
    const float inv_t = temperature > 0.f ? 1.0f / temperature : 0.f;
    if (temperature > 0.f && !isfinite(inv_t)) return SV_E_SHAPE;
    return map_launch(sv::launch_coupled(p, target_logits, temperature > 0.f ? gumbel : nullptr, draft_tokens,
                                         tau, batch, block, gamma, vocab, inv_t, accept_len, out_tokens,
                                         target_tokens, workspace, (hipStream_t)stream));
}

size_t spec_verify_tree_workspace_size(int batch, int n_nodes, int64_t vocab) {
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || vocab < 1 || vocab > (1ll << 21) ||
        !rows_ok(batch, n_nodes, vocab))
        return 0;
    return sv::coupled_plan(batch, n_nodes, n_nodes, vocab).ws_total;
}

int spec_verify_tree(const float *target_logits, const float *gumbel, const int32_t *parent, const int32_t *node_pos,
                     const int32_t *node_tok, const int32_t *target_pos, int batch, int n_nodes, int64_t vocab,
                     float temperature, int32_t *path_len, int32_t *path, int32_t *commit_pos, int32_t *commit_tok,
                     int32_t *target_tok, void *workspace, size_t workspace_bytes, void *stream) {
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || vocab < 1 || vocab > (1ll << 21)) return SV_E_SHAPE;
    if (!rows_ok(batch, n_nodes, vocab)) return SV_E_SHAPE;
    if (!(temperature >= 0.f) || !isfinite(temperature)) return SV_E_SHAPE;
    if (!target_logits || !parent || !node_pos || !node_tok || !target_pos || !path_len || !path || !commit_pos ||
        !commit_tok)
        return SV_E_NULL;
    if (temperature > 0.f && !gumbel) return SV_E_NULL;
    if (!aligned16(target_logits) || (gumbel && !aligned16(gumbel))) return SV_E_ALIGN;
    const sv::CoupledPlan p = sv::coupled_plan(batch, n_nodes, n_nodes, vocab);
    if (!workspace || workspace_bytes < p.ws_total) return SV_E_WORKSPACE;
    if (!aligned16(workspace)) return SV_E_ALIGN;
    const float inv_t = temperature > 0.f ? 1.0f / temperature : 0.f;
    if (temperature > 0.f && !isfinite(inv_t)) return SV_E_SHAPE;
    return map_launch(sv::launch_tree(p, target_logits, temperature > 0.f ? gumbel : nullptr, parent, node_pos,
                                      node_tok, target_pos, batch, n_nodes, vocab, inv_t, path_len, path, commit_pos,
                                      commit_tok, target_tok, workspace, (hipStream_t)stream));
}

size_t spec_verify_tree_states_workspace_size(int batch, int n_nodes, int block, int64_t vocab) {
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || block < 1 || block > 64 || vocab < 1 || vocab > (1ll << 21) ||
        !rows_ok(batch, n_nodes * block, vocab))
        return 0;
    return sv::states_plan(batch, n_nodes, block, vocab).ws_total;
}

int spec_verify_tree_states(const float *target_logits, const float *gumbel, const int32_t *parent,
                            const int32_t *state, int batch, int n_nodes, int block, int64_t vocab, float temperature,
                            float threshold, int32_t *path_len, int32_t *path, int32_t *next_state, int32_t *commit,
                            float *confidence, void *workspace, size_t workspace_bytes, void *stream) {
    if (batch < 1 || n_nodes < 1 || n_nodes > 64 || block < 1 || block > 64 || vocab < 1 || vocab > (1ll << 21))
        return SV_E_SHAPE;
    if (!rows_ok(batch, n_nodes * block, vocab)) return SV_E_SHAPE;
    if (!(temperature >= 0.f) || !isfinite(temperature) || isnan(threshold)) return SV_E_SHAPE;
    if (!target_logits || !parent || !state || !path_len || !path || !next_state) return SV_E_NULL;
    if (temperature > 0.f && !gumbel) return SV_E_NULL;
    if (!aligned16(target_logits) || (gumbel && !aligned16(gumbel))) return SV_E_ALIGN;
    const sv::StatesPlan p = sv::states_plan(batch, n_nodes, block, vocab);
    if (!workspace || workspace_bytes < p.ws_total) return SV_E_WORKSPACE;
    if (!aligned16(workspace)) return SV_E_ALIGN;
    const float inv_t = temperature > 0.f ? 1.0f / temperature : 0.f;
    if (temperature > 0.f && !isfinite(inv_t)) return SV_E_SHAPE;
    return map_launch(sv::launch_states(p, target_logits, temperature > 0.f ? gumbel : nullptr, parent, state, batch,
                                        n_nodes, block, vocab, inv_t, threshold, path_len, path, next_state, commit,
                                        confidence, workspace, (hipStream_t)stream));
}

size_t spec_verify_route_workspace_size(int batch, int block, int gamma, int64_t vocab) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21) || !rows_ok(batch, block, vocab))
        return 0;
    return sv::route_plan(batch, block, gamma, vocab).ws_total;
}

int spec_verify_route(const float *draft_probs, const int32_t *tau, int batch, int block, int gamma,
                      int64_t vocab, int estimator, double param, float *khat, float *alpha_hat, void *workspace,
                      size_t workspace_bytes, void *stream) {
    if (batch < 1 || block < 1 || block > 64 || gamma < 1 || gamma > block || vocab < 1 ||
        vocab > (1ll << 21))
        return SV_E_SHAPE;
    if (!rows_ok(batch, block, vocab)) return SV_E_SHAPE;
    if (estimator != SV_ROUTE_MARGIN && estimator != SV_ROUTE_ENTROPY) return SV_E_UNSUPPORTED;
    if (!isfinite(param)) return SV_E_SHAPE;
    if (!draft_probs || !tau || !khat) return SV_E_NULL;
    if (!aligned16(draft_probs) || !aligned16(tau) || !aligned16(khat) || (alpha_hat && !aligned16(alpha_hat)))
        return SV_E_ALIGN;
    const sv::RoutePlan p = sv::route_plan(batch, block, gamma, vocab);
    if (!workspace || workspace_bytes < p.ws_total) return SV_E_WORKSPACE;
    if (!aligned16(workspace)) return SV_E_ALIGN;
    return map_launch(sv::launch_route(p, draft_probs, tau, batch, block, gamma, vocab, estimator, param, khat,
                                       alpha_hat, workspace, (hipStream_t)stream));
}

}  // extern "C"
