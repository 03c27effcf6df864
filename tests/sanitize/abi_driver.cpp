// abi_driver.cpp -- calls every entry point of include/gdn.h with arguments the
// host checks refuse (null, misaligned or overlapping pointers, bad dims,
// sizes out of range, short workspaces) and every size query, in a host build
// of the library with AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing
// reaches a device: each refused call returns before any HIP call.  Test
// infrastructure: tests/test_sanitizers.py builds and runs it.
// Exit status 0: every call returned the status expected of it.
#include <cstdint>
#include <cstdio>

#include "gdn.h"

namespace {
int failures = 0;
void expect(const char* what, int got, int want) {
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}
void expect_size(const char* what, size_t got, bool nonzero) {
    if ((got != 0) != nonzero) {
        std::fprintf(stderr, "%s: size %zu\n", what, got);
        ++failures;
    }
}
}  // namespace

int main() {
    gdn_dims good{1, 16, 48, 128, 128, 4, GDN_BF16};
    gdn_dims tiny{3, 4, 4, 32, 32, 4, GDN_F32};
    gdn_dims bad_w = good, bad_d = good, bad_g = good, bad_t = good, big = good, wide{1, 1, 128, 32, 32, 4, GDN_BF16};
    bad_w.conv_width = 3;
    bad_d.head_k_dim = 64;
    bad_g.num_v_heads = 47;
    bad_t.act_dtype = 7;
    big.batch = 65536;
    void* f = reinterpret_cast<void*>(0x1000);           // never dereferenced
    void* g = reinterpret_cast<void*>(0x200000);
    void* mis = reinterpret_cast<void*>(0x1004);
    float* ff = static_cast<float*>(f);
    float* fg = static_cast<float*>(g);
    int32_t* fi = static_cast<int32_t*>(f);

    for (const gdn_dims* d : {&good, &tiny}) {
        expect_size("channels", gdn_conv_channels(d), true);
        expect_size("state", gdn_state_bytes(d), true);
        expect_size("tail", gdn_conv_tail_bytes(d), true);
        expect_size("tree ws", gdn_tree_workspace_bytes(d, 32), true);
        expect_size("block ws", gdn_block_workspace_bytes(d, 17), true);
        expect_size("prefill ws", gdn_prefill_workspace_bytes(d, 4097), d == &good);
        expect_size("snapshot", gdn_snapshot_bytes(d, 3), true);
        expect_size("self-check ws", gdn_self_check_workspace_bytes(d), true);
    }
    for (const gdn_dims* d : {&bad_w, &bad_d, &bad_g, &bad_t}) {
        expect_size("bad channels", gdn_conv_channels(d), false);
        expect_size("bad tree ws", gdn_tree_workspace_bytes(d, 32), false);
        expect("bad conv", gdn_conv_update(d, f, f, f, ff, nullptr), d == &bad_t ? GDN_ERR_DTYPE : GDN_ERR_SHAPE);
    }
    expect_size("tree ws 33 nodes", gdn_tree_workspace_bytes(&good, 33), false);
    expect("abi", gdn_abi_version(), GDN_ABI_VERSION);
    for (int s = -1; s < 13; ++s)
        if (!gdn_status_str(s))
            ++failures;

    expect("conv null", gdn_conv_update(&good, nullptr, f, f, ff, nullptr), GDN_ERR_NULL);
    expect("conv misaligned", gdn_conv_update(&good, mis, f, f, ff, nullptr), GDN_ERR_ALIGN);
    expect("step null", gdn_decode_step(&good, ff, ff, ff, ff, nullptr, nullptr), GDN_ERR_NULL);
    expect("kda step null", gdn_kda_decode_step(&good, ff, nullptr, ff, ff, ff, nullptr), GDN_ERR_NULL);
    expect("token alias", gdn_decode_token(&good, ff, f, f, f, f, ff, ff, ff, nullptr), GDN_ERR_ALIAS);
    expect("kda token alias", gdn_kda_decode_token(&good, ff, f, f, f, f, ff, ff, ff, nullptr), GDN_ERR_ALIAS);
    expect("kda token dims", gdn_kda_decode_token(&bad_d, ff, f, g, f, f, ff, ff, ff, nullptr), GDN_ERR_SHAPE);

    expect("tables n", gdn_tree_tables(33, fi, fi, fi, fi, nullptr), GDN_ERR_TREE);
    expect("tables null", gdn_tree_tables(4, nullptr, fi, fi, fi, nullptr), GDN_ERR_NULL);
    for (int n : {0, 33}) {
        expect("verify n", gdn_tree_verify(&good, ff, f, f, n, fi, f, ff, ff, ff, nullptr, f, 1u << 30, nullptr),
               GDN_ERR_TREE);
        expect("verify ut n", gdn_tree_verify_ut(&good, ff, f, f, n, fi, f, ff, ff, ff, nullptr, nullptr, 0, nullptr),
               GDN_ERR_TREE);
        expect("block n", gdn_block_verify(&good, ff, f, f, n, f, ff, ff, ff, f, 1u << 30, nullptr), GDN_ERR_SHAPE);
        expect("block ut n", gdn_block_verify_ut(&good, ff, f, f, n, f, ff, ff, ff, nullptr, 0, nullptr),
               GDN_ERR_SHAPE);
    }
    expect("verify ws", gdn_tree_verify(&good, ff, f, f, 4, fi, f, ff, ff, ff, nullptr, f, 1024, nullptr),
           GDN_ERR_WORKSPACE);
    expect("verify ws null", gdn_tree_verify(&good, ff, f, f, 4, fi, f, ff, ff, ff, nullptr, nullptr, 0, nullptr),
           GDN_ERR_WORKSPACE);
    expect("verify ut short ws", gdn_tree_verify_ut(&good, ff, f, f, 4, fi, f, ff, ff, ff, nullptr, f, 1024, nullptr),
           GDN_ERR_WORKSPACE);
    expect("verify ut batch", gdn_tree_verify_ut(&big, ff, f, f, 4, fi, f, ff, ff, ff, nullptr, nullptr, 0, nullptr),
           GDN_ERR_SHAPE);
    expect("verify ut heads", gdn_tree_verify_ut(&wide, ff, f, f, 4, fi, f, ff, ff, ff, nullptr, nullptr, 0, nullptr),
           GDN_ERR_SHAPE);
    expect("verify ut status", gdn_tree_verify_ut(&good, ff, f, f, 4, fi, f, ff, ff, ff, static_cast<int32_t*>(mis),
                                                  nullptr, 0, nullptr), GDN_ERR_ALIGN);
    gdn_dims thirteen = good;
    thirteen.batch = 13;
    expect("noalloc size", gdn_tree_verify_ut_noalloc(&thirteen, ff, f, f, 32, fi, f, ff, ff, ff, nullptr, nullptr),
           GDN_ERR_WORKSPACE);
    expect("commit null", gdn_commit_path(&good, ff, f, f, 4, fi, f, ff, ff, 2, nullptr, nullptr, nullptr, nullptr),
           GDN_ERR_NULL);
    expect("commit len", gdn_commit_path(&good, ff, f, f, 4, fi, f, ff, ff, 9, fi, nullptr, nullptr, nullptr),
           GDN_ERR_TREE);
    expect("prepared ws", gdn_commit_path_prepared(&good, ff, f, 4, fi, f, 2, fi, nullptr, nullptr, f, 16, nullptr),
           GDN_ERR_WORKSPACE);
    expect("block commit ws", gdn_block_commit(&good, ff, f, f, 4, f, ff, ff, fi, nullptr, nullptr, f, 16, nullptr),
           GDN_ERR_WORKSPACE);
    expect("block prepared ws",
           gdn_block_commit_prepared(&good, ff, f, 4, f, fi, nullptr, nullptr, nullptr, 0, nullptr),
           GDN_ERR_WORKSPACE);
    expect("prefill T", gdn_prefill_chunked(&good, ff, f, f, 0, f, ff, ff, ff, f, 1u << 30, nullptr), GDN_ERR_SHAPE);
    expect("prefill shape", gdn_prefill_chunked(&tiny, ff, f, f, 64, f, ff, ff, ff, f, 1u << 30, nullptr),
           GDN_ERR_SHAPE);
    expect("prefill ws", gdn_prefill_chunked(&good, ff, f, f, 64, f, ff, ff, ff, f, 64, nullptr), GDN_ERR_WORKSPACE);
    expect("snapshot count", gdn_snapshot(&good, ff, f, 0, fi, f, 1u << 30, fi, nullptr), GDN_ERR_SHAPE);
    expect("snapshot blob", gdn_snapshot(&good, ff, f, 1, fi, f, 16, fi, nullptr), GDN_ERR_WORKSPACE);
    expect("restore null", gdn_restore(&good, nullptr, f, 1, fi, f, 1u << 30, fi, nullptr), GDN_ERR_NULL);
    expect("self-check ws", gdn_self_check(&good, 1, 0, f, 16, fi, nullptr), GDN_ERR_WORKSPACE);
    expect("self-check flags", gdn_self_check(&good, 1, 8, f, 1u << 30, fi, nullptr), GDN_ERR_SHAPE);
    (void)fg;
    (void)gdn_state_signature(&good);
    (void)gdn_state_signature(&bad_d);
    if (failures) {
        std::fprintf(stderr, "%d unexpected results\n", failures);
        return 1;
    }
    std::printf("abi driver: every call refused as expected\n");
    return 0;
}
