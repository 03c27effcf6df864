// gdn_api.hip -- the C ABI declared in include/gdn.h: argument checks, then
// launches on the caller's stream.  Nothing here allocates, synchronises or
// keeps state between calls.
//
// Shapes are refused loudly rather than run wrongly (the CPU page's account of
// a hard-coded head width that silently corrupted memory ends with the engine
// refusing unsupported head sizes outright).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates dims and fills the kernel geometry.
gdn_status check_dims(const gdn_dims* d, gdn::Geo& g) {
    if (!d)
        return GDN_ERR_NULL;
    if (d->act_dtype != GDN_F32 && d->act_dtype != GDN_BF16)
        return GDN_ERR_DTYPE;
    if (d->batch < 1 || d->num_k_heads < 1 || d->num_v_heads < 1 || d->num_v_heads % d->num_k_heads != 0 ||
        d->head_k_dim != d->head_v_dim || (d->head_k_dim != 32 && d->head_k_dim != 128) || d->conv_width != 4)
        return GDN_ERR_SHAPE;
    const int64_t C = 2ll * d->num_k_heads * d->head_k_dim + static_cast<int64_t>(d->num_v_heads) * d->head_v_dim;
    // Kernel index arithmetic keeps per-sequence channel and head offsets in 32 bits.
    if (C > (1ll << 24) || static_cast<int64_t>(d->batch) * d->num_v_heads > (1ll << 24))
        return GDN_ERR_SHAPE;
    g.B = d->batch;
    g.Hk = d->num_k_heads;
    g.Hv = d->num_v_heads;
    g.D = d->head_k_dim;
    g.C = static_cast<int>(C);
    g.bf16 = d->act_dtype == GDN_BF16;
    return GDN_OK;
}

gdn_status ptrs_ok(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p)
            return GDN_ERR_NULL;
    for (const void* p : ps)
        if (!aligned16(p))
            return GDN_ERR_ALIGN;
    return GDN_OK;
}

gdn_status launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ws_optional: the UT-form calls accept a NULL workspace (the one-launch form).
gdn_status tree_verify_args(const gdn_dims* d, gdn::Geo& g, std::initializer_list<const void*> ptrs, int32_t n_nodes,
                            const int32_t* tree_status, const void* workspace, size_t workspace_bytes,
                            bool ws_optional = false) {
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && (g.B > GDN_MAX_TREE_BATCH || g.Hv / g.Hk > 64))
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok(ptrs);
    if (st == GDN_OK && tree_status && !aligned16(tree_status))
        st = GDN_ERR_ALIGN;
    if (st == GDN_OK && (n_nodes < 1 || n_nodes > GDN_MAX_TREE_NODES))
        st = GDN_ERR_TREE;
    if (st != GDN_OK)
        return st;
    if (ws_optional && !workspace)
        return GDN_OK;
    if (!workspace || workspace_bytes < gdn::tree_ws_bytes(g.B, n_nodes, g.Hk, g.Hv, g.D))
        return GDN_ERR_WORKSPACE;
    return aligned16(workspace) ? GDN_OK : GDN_ERR_ALIGN;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "unsupported or inconsistent shape";
        case GDN_ERR_DTYPE: return "unsupported activation dtype";
        case GDN_ERR_ALIGN: return "pointer not 16-byte aligned";
        case GDN_ERR_TREE: return "malformed draft tree or path";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "HIP launch failed";
        case GDN_ERR_ALIAS: return "buffers that must be distinct overlap";
        case GDN_ERR_SIGNATURE: return "snapshot of another layer shape or format";
        case GDN_ERR_INDEX: return "sequence index out of range or repeated";
        case GDN_ERR_SELF_CHECK: return "self-check: verify or commit rows differ from decode";
        default: return "unknown status";
    }
}

size_t gdn_conv_channels(const gdn_dims* d) {
    gdn::Geo g;
    return check_dims(d, g) == GDN_OK ? static_cast<size_t>(g.C) : 0;
}

size_t gdn_state_bytes(const gdn_dims* d) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK)
        return 0;
    return static_cast<size_t>(g.B) * g.Hv * g.D * g.D * sizeof(float);
}

size_t gdn_conv_tail_bytes(const gdn_dims* d) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK)
        return 0;
    return static_cast<size_t>(g.B) * g.C * 4 * (g.bf16 ? 2 : 4);
}

gdn_status gdn_conv_update(const gdn_dims* d, const void* x, void* conv_tail, const void* conv_w, float* y,
                           void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK)
        st = ptrs_ok({x, conv_tail, conv_w, y});
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_conv_update(g, x, conv_tail, conv_w, y, as_stream(stream)));
}

gdn_status gdn_decode_step(const gdn_dims* d, float* state, const float* y, const float* a, const float* b,
                           float* o, void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK)
        st = ptrs_ok({state, y, a, b, o});
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_decode(g, state, y, a, b, o, as_stream(stream)));
}

gdn_status gdn_decode_token(const gdn_dims* d, float* state, const void* conv_tail_in, void* conv_tail_out,
                            const void* conv_w, const void* x, const float* a, const float* b, float* o,
                            void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK)
        st = ptrs_ok({state, conv_tail_in, conv_tail_out, conv_w, x, a, b, o});
    if (st != GDN_OK)
        return st;
    const size_t tail_bytes = static_cast<size_t>(g.B) * g.C * 4 * (g.bf16 ? 2 : 4);
    const uintptr_t ti = reinterpret_cast<uintptr_t>(conv_tail_in), to = reinterpret_cast<uintptr_t>(conv_tail_out);
    if (ti < to + tail_bytes && to < ti + tail_bytes)
        return GDN_ERR_ALIAS;
    return launched(gdn::launch_token(g, state, conv_tail_in, conv_tail_out, conv_w, x, a, b, o, as_stream(stream)));
}

gdn_status gdn_kda_decode_step(const gdn_dims* d, float* state, const float* y, const float* a, const float* b,
                               float* o, void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK)
        st = ptrs_ok({state, y, a, b, o});
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_kda_decode(g, state, y, a, b, o, as_stream(stream)));
}

gdn_status gdn_kda_decode_token(const gdn_dims* d, float* state, const void* conv_tail_in, void* conv_tail_out,
                                const void* conv_w, const void* x, const float* a, const float* b, float* o,
                                void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK)
        st = ptrs_ok({state, conv_tail_in, conv_tail_out, conv_w, x, a, b, o});
    if (st != GDN_OK)
        return st;
    const size_t tail_bytes = static_cast<size_t>(g.B) * g.C * 4 * (g.bf16 ? 2 : 4);
    const uintptr_t ti = reinterpret_cast<uintptr_t>(conv_tail_in), to = reinterpret_cast<uintptr_t>(conv_tail_out);
    if (ti < to + tail_bytes && to < ti + tail_bytes)
        return GDN_ERR_ALIAS;
    return launched(
        gdn::launch_kda_token(g, state, conv_tail_in, conv_tail_out, conv_w, x, a, b, o, as_stream(stream)));
}

gdn_status gdn_tree_tables(int32_t n_nodes, const int32_t* parent, int32_t* depth, int32_t* order,
                           int32_t* tree_status, void* stream) {
    if (n_nodes < 1 || n_nodes > GDN_MAX_TREE_NODES)
        return GDN_ERR_TREE;
    const gdn_status st = ptrs_ok({parent, depth, order, tree_status});
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_tree_tables(n_nodes, parent, depth, order, tree_status, as_stream(stream)));
}

size_t gdn_tree_workspace_bytes(const gdn_dims* d, int32_t n_nodes) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK || n_nodes < 1 || n_nodes > GDN_MAX_TREE_NODES)
        return 0;
    return gdn::tree_ws_bytes(g.B, n_nodes, g.Hk, g.Hv, g.D);
}

gdn_status gdn_tree_verify(const gdn_dims* d, const float* state_ckpt, const void* conv_tail, const void* conv_w,
                           int32_t n_nodes, const int32_t* parent, const void* x, const float* a, const float* b,
                           float* o, int32_t* tree_status, void* workspace, size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    const gdn_status st = tree_verify_args(d, g, {state_ckpt, conv_tail, conv_w, parent, x, a, b, o}, n_nodes,
                                           tree_status, workspace, workspace_bytes);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_tree_verify(g, state_ckpt, conv_tail, conv_w, n_nodes, parent, x, a, b, o,
                                            tree_status, workspace, as_stream(stream)));
}

gdn_status gdn_tree_verify_ut(const gdn_dims* d, const float* state_ckpt, const void* conv_tail, const void* conv_w,
                              int32_t n_nodes, const int32_t* parent, const void* x, const float* a, const float* b,
                              float* o, int32_t* tree_status, void* workspace, size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    const gdn_status st = tree_verify_args(d, g, {state_ckpt, conv_tail, conv_w, parent, x, a, b, o}, n_nodes,
                                           tree_status, workspace, workspace_bytes, true);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_tree_verify_ut(g, state_ckpt, conv_tail, conv_w, n_nodes, parent, x, a, b, o,
                                               tree_status, workspace, as_stream(stream)));
}

gdn_status gdn_commit_path(const gdn_dims* d, float* state, void* conv_tail, const void* conv_w, int32_t n_nodes,
                           const int32_t* parent, const void* x, const float* a, const float* b, int32_t path_len,
                           const int32_t* path, float* o, int32_t* tree_status, void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && (g.B > GDN_MAX_TREE_BATCH || g.Hv / g.Hk > 64))
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok({state, conv_tail, conv_w, parent, x, a, b, path});
    if (st == GDN_OK && ((o && !aligned16(o)) || (tree_status && !aligned16(tree_status))))
        st = GDN_ERR_ALIGN;
    if (st == GDN_OK && (n_nodes < 1 || n_nodes > GDN_MAX_TREE_NODES || path_len < 1 ||
                         path_len > GDN_MAX_TREE_DEPTH || path_len > n_nodes))
        st = GDN_ERR_TREE;
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_commit(g, state, conv_tail, conv_w, n_nodes, parent, x, a, b, path_len, path, o,
                                       tree_status, nullptr, as_stream(stream)));
}

gdn_status gdn_commit_path_prepared(const gdn_dims* d, float* state, void* conv_tail, int32_t n_nodes,
                                    const int32_t* parent, const void* x, int32_t path_len, const int32_t* path,
                                    float* o, int32_t* tree_status, const void* workspace, size_t workspace_bytes,
                                    void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && (g.B > GDN_MAX_TREE_BATCH || g.Hv / g.Hk > 64))
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok({state, conv_tail, parent, x, path});
    if (st == GDN_OK && ((o && !aligned16(o)) || (tree_status && !aligned16(tree_status))))
        st = GDN_ERR_ALIGN;
    if (st == GDN_OK && (n_nodes < 1 || n_nodes > GDN_MAX_TREE_NODES || path_len < 1 ||
                         path_len > GDN_MAX_TREE_DEPTH || path_len > n_nodes))
        st = GDN_ERR_TREE;
    if (st != GDN_OK)
        return st;
    if (!workspace || workspace_bytes < gdn::tree_ws_bytes(g.B, n_nodes, g.Hk, g.Hv, g.D))
        return GDN_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return GDN_ERR_ALIGN;
    return launched(gdn::launch_commit(g, state, conv_tail, nullptr, n_nodes, parent, x, nullptr, nullptr, path_len,
                                       path, o, tree_status, const_cast<void*>(workspace), as_stream(stream)));
}

size_t gdn_block_workspace_bytes(const gdn_dims* d, int32_t k) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK || k < 1 || k > GDN_MAX_TREE_NODES)
        return 0;
    return gdn::tree_ws_bytes(g.B, k, g.Hk, g.Hv, g.D);
}

}  // extern "C"

namespace {

gdn_status block_args(const gdn_dims* d, gdn::Geo& g, std::initializer_list<const void*> ptrs, int32_t k,
                      const void* o, const int32_t* status, const void* workspace, size_t workspace_bytes,
                      bool ws_optional = false) {
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && (g.B > GDN_MAX_TREE_BATCH || g.Hv / g.Hk > 64))
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok(ptrs);
    if (st == GDN_OK && ((o && !aligned16(o)) || (status && !aligned16(status))))
        st = GDN_ERR_ALIGN;
    if (st == GDN_OK && (k < 1 || k > GDN_MAX_TREE_NODES))
        st = GDN_ERR_SHAPE;
    if (st != GDN_OK)
        return st;
    if (ws_optional && !workspace)
        return GDN_OK;
    if (!workspace || workspace_bytes < gdn::tree_ws_bytes(g.B, k, g.Hk, g.Hv, g.D))
        return GDN_ERR_WORKSPACE;
    return aligned16(workspace) ? GDN_OK : GDN_ERR_ALIGN;
}

}  // namespace

extern "C" {

gdn_status gdn_block_verify(const gdn_dims* d, const float* state_ckpt, const void* conv_tail, const void* conv_w,
                            int32_t k, const void* x, const float* a, const float* b, float* o, void* workspace,
                            size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    const gdn_status st = block_args(d, g, {state_ckpt, conv_tail, conv_w, x, a, b, o}, k, o, nullptr, workspace,
                                     workspace_bytes);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_block(g, false, const_cast<float*>(state_ckpt), const_cast<void*>(conv_tail),
                                      conv_w, k, x, a, b, nullptr, o, nullptr, workspace, false,
                                      as_stream(stream)));
}

gdn_status gdn_block_verify_ut(const gdn_dims* d, const float* state_ckpt, const void* conv_tail, const void* conv_w,
                               int32_t k, const void* x, const float* a, const float* b, float* o, void* workspace,
                               size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    const gdn_status st = block_args(d, g, {state_ckpt, conv_tail, conv_w, x, a, b, o}, k, o, nullptr, workspace,
                                     workspace_bytes, true);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_tree_verify_ut(g, state_ckpt, conv_tail, conv_w, k, nullptr, x, a, b, o, nullptr,
                                               workspace, as_stream(stream)));
}

gdn_status gdn_block_commit(const gdn_dims* d, float* state, void* conv_tail, const void* conv_w, int32_t k,
                            const void* x, const float* a, const float* b, const int32_t* accepted, float* o,
                            int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    const gdn_status st = block_args(d, g, {state, conv_tail, conv_w, x, a, b, accepted}, k, o, status, workspace,
                                     workspace_bytes);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_block(g, true, state, conv_tail, conv_w, k, x, a, b, accepted, o, status, workspace,
                                      false, as_stream(stream)));
}

gdn_status gdn_block_commit_prepared(const gdn_dims* d, float* state, void* conv_tail, int32_t k, const void* x,
                                     const int32_t* accepted, float* o, int32_t* status, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    const gdn_status st = block_args(d, g, {state, conv_tail, x, accepted}, k, o, status, workspace, workspace_bytes);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_block(g, true, state, conv_tail, nullptr, k, x, nullptr, nullptr, accepted, o, status,
                                      workspace, true, as_stream(stream)));
}

uint64_t gdn_state_signature(const gdn_dims* d) {
    gdn::Geo g;
    return check_dims(d, g) == GDN_OK ? gdn::state_signature(g) : 0;
}

size_t gdn_snapshot_bytes(const gdn_dims* d, int32_t count) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK || count < 1 || count > GDN_MAX_TREE_BATCH)
        return 0;
    return gdn::snapshot_bytes(g, count);
}

}  // extern "C"

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

gdn_status snapshot_args(const gdn_dims* d, gdn::Geo& g, const void* state, const void* tail, int32_t count,
                         const int32_t* seqs, const void* blob, size_t blob_bytes, const int32_t* status) {
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && g.B > GDN_MAX_TREE_BATCH)
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok({state, tail, seqs, blob, status});
    if (st == GDN_OK && (reinterpret_cast<uintptr_t>(blob) & 255u))
        st = GDN_ERR_ALIGN;
    if (st == GDN_OK && (count < 1 || count > GDN_MAX_TREE_BATCH))
        st = GDN_ERR_SHAPE;
    if (st != GDN_OK)
        return st;
    const size_t need = gdn::snapshot_bytes(g, count);
    if (blob_bytes < need)
        return GDN_ERR_WORKSPACE;
    const size_t sb = static_cast<size_t>(g.B) * g.Hv * g.D * g.D * 4;
    const size_t tb = static_cast<size_t>(g.B) * g.C * 4 * (g.bf16 ? 2 : 4);
    if (overlaps(blob, need, state, sb) || overlaps(blob, need, tail, tb))
        return GDN_ERR_ALIAS;
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_snapshot(const gdn_dims* d, const float* state, const void* conv_tail, int32_t count,
                        const int32_t* seqs, void* blob, size_t blob_bytes, int32_t* status, void* stream) {
    gdn::Geo g;
    const gdn_status st = snapshot_args(d, g, state, conv_tail, count, seqs, blob, blob_bytes, status);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_snapshot(g, false, const_cast<float*>(state), const_cast<void*>(conv_tail), count,
                                         seqs, blob, status, as_stream(stream)));
}

gdn_status gdn_restore(const gdn_dims* d, float* state, void* conv_tail, int32_t count, const int32_t* seqs,
                       const void* blob, size_t blob_bytes, int32_t* status, void* stream) {
    gdn::Geo g;
    const gdn_status st = snapshot_args(d, g, state, conv_tail, count, seqs, blob, blob_bytes, status);
    if (st != GDN_OK)
        return st;
    return launched(gdn::launch_snapshot(g, true, state, conv_tail, count, seqs, const_cast<void*>(blob), status,
                                         as_stream(stream)));
}

size_t gdn_prefill_workspace_bytes(const gdn_dims* d, int32_t T) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK || T < 1)
        return 0;
    return gdn::prefill_workspace_bytes(g, T);
}

gdn_status gdn_prefill_chunked(const gdn_dims* d, float* state, void* conv_tail, const void* conv_w, int32_t T,
                               const void* x, const float* a, const float* b, float* o, void* workspace,
                               size_t workspace_bytes, void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK)
        st = ptrs_ok({state, conv_tail, conv_w, x, a, b, o});
    if (st == GDN_OK && (T < 1 || g.D != 128 || g.Hv / g.Hk > 8))
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK && static_cast<int64_t>(g.B) * T * g.C >= (1ll << 40))
        st = GDN_ERR_SHAPE;
    if (st != GDN_OK)
        return st;
    const size_t need = gdn::prefill_workspace_bytes(g, T);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return GDN_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace))
        return GDN_ERR_ALIGN;
    return launched(gdn::launch_prefill(g, state, conv_tail, conv_w, T, x, a, b, o, workspace, as_stream(stream)));
}

size_t gdn_self_check_workspace_bytes(const gdn_dims* d) {
    gdn::Geo g;
    if (check_dims(d, g) != GDN_OK || g.Hv / g.Hk > 64)
        return 0;
    return gdn::self_check_ws_bytes(g);
}

gdn_status gdn_self_check(const gdn_dims* d, uint32_t seed, int32_t flags, void* workspace, size_t workspace_bytes,
                          int32_t* result, void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && g.Hv / g.Hk > 64)
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok({result});
    if (st == GDN_OK && (flags & ~GDN_SELF_CHECK_PERTURB))
        st = GDN_ERR_SHAPE;
    if (st != GDN_OK)
        return st;
    if (!workspace || workspace_bytes < gdn::self_check_ws_bytes(g))
        return GDN_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return GDN_ERR_ALIGN;
    return launched(gdn::launch_self_check(g, workspace, seed, flags & GDN_SELF_CHECK_PERTURB, result,
                                           as_stream(stream)));
}

gdn_status gdn_tree_verify_ut_noalloc(const gdn_dims* d, const float* state_ckpt, const void* conv_tail,
                                      const void* conv_w, int32_t n_nodes, const int32_t* parent, const void* x,
                                      const float* a, const float* b, float* o, int32_t* tree_status, void* stream) {
    gdn::Geo g;
    gdn_status st = check_dims(d, g);
    if (st == GDN_OK && (g.B > GDN_MAX_TREE_BATCH || g.Hv / g.Hk > 64))
        st = GDN_ERR_SHAPE;
    if (st == GDN_OK)
        st = ptrs_ok({state_ckpt, conv_tail, conv_w, parent, x, a, b, o});
    if (st == GDN_OK && tree_status && !aligned16(tree_status))
        st = GDN_ERR_ALIGN;
    if (st == GDN_OK && (n_nodes < 1 || n_nodes > GDN_MAX_TREE_NODES))
        st = GDN_ERR_TREE;
    if (st != GDN_OK)
        return st;
    if (gdn::tree_ws_bytes(g.B, n_nodes, g.Hk, g.Hv, g.D) > GDN_NOALLOC_SCRATCH_BYTES)
        return GDN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (gdn::noalloc_scratch(&ws) != hipSuccess)
        return GDN_ERR_HIP;
    return launched(gdn::launch_tree_verify_ut(g, state_ckpt, conv_tail, conv_w, n_nodes, parent, x, a, b, o,
                                               tree_status, ws, as_stream(stream)));
}

}  // extern "C"
