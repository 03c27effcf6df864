"""The C-ABI library, on the CPU: it loads, exports every function include/gdn.h
declares, and refuses bad arguments before it touches a device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "gated_deltanet_decode_amd", "libgdn.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built (python -m gated_deltanet_decode_amd.build)")
    return C.CDLL(LIB)


def test_header_declares_the_five_calls():
    names = declared_functions()
    for f in ("gdn_conv_update", "gdn_decode_step", "gdn_tree_verify", "gdn_commit_path", "gdn_prefill_chunked",
              "gdn_decode_token"):
        assert f in names


def test_library_exports_every_declared_function(lib):
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, f"not exported: {missing}"


class Dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("batch", "num_k_heads", "num_v_heads", "head_k_dim",
                                         "head_v_dim", "conv_width", "act_dtype")]


GOOD = dict(batch=1, num_k_heads=16, num_v_heads=48, head_k_dim=128, head_v_dim=128, conv_width=4, act_dtype=1)


def mk(**kw):
    d = dict(GOOD)
    d.update(kw)
    return Dims(**d)


def test_prefill_workspace_stops_growing_at_one_segment(lib):
    """The binding's PREFILL_SEGMENT is the library's: the prefill workspace holds
    one segment, so it grows with T (in 64-token chunks) up to it and no further."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_gdn_consts", os.path.join(ROOT, "gated_deltanet_decode_amd",
                                                                               "__init__.py"))
    src = open(spec.origin).read()
    seg = int(re.search(r"^PREFILL_SEGMENT = (\d+)", src, re.M).group(1))
    lib.gdn_prefill_workspace_bytes.restype = C.c_size_t
    lib.gdn_prefill_workspace_bytes.argtypes = [C.POINTER(Dims), C.c_int32]
    d = mk()
    ws = lambda T: lib.gdn_prefill_workspace_bytes(C.byref(d), T)
    assert ws(64) < ws(seg - 64) < ws(seg) == ws(seg + 64) == ws(8 * seg)


def test_tree_workspace_is_bounded(lib):
    lib.gdn_tree_workspace_bytes.restype = C.c_size_t
    d = mk()
    sizes = [lib.gdn_tree_workspace_bytes(C.byref(d), n) for n in (1, 16, 32)]
    assert 0 < sizes[0] < sizes[1] < sizes[2] < 2 * 1024 * 1024
    assert lib.gdn_tree_workspace_bytes(C.byref(d), 33) == 0


def test_size_queries_match_the_pages(lib):
    """The 27B-class layer: 3.15 MB of fp32 state and an 80 KB bf16 conv tail per
    sequence ("Architecture" section 8.1 table), 151 MB over 48 layers (8.2)."""
    for f in ("gdn_state_bytes", "gdn_conv_tail_bytes", "gdn_conv_channels"):
        getattr(lib, f).restype = C.c_size_t
    d = mk()
    assert lib.gdn_conv_channels(C.byref(d)) == 10240
    assert lib.gdn_state_bytes(C.byref(d)) == 48 * 128 * 128 * 4 == 3_145_728
    assert lib.gdn_conv_tail_bytes(C.byref(d)) == 4 * 10240 * 2 == 81_920
    assert 48 * lib.gdn_state_bytes(C.byref(d)) == 150_994_944  # the pages' 151 MB
    assert lib.gdn_state_bytes(C.byref(mk(batch=64))) == 64 * 3_145_728
    assert lib.gdn_state_bytes(C.byref(mk(head_k_dim=64, head_v_dim=64))) == 0


@pytest.mark.parametrize("bad,status", [
    (dict(head_k_dim=64, head_v_dim=64), 2), (dict(head_v_dim=32), 2), (dict(num_v_heads=40), 2),
    (dict(conv_width=3), 2), (dict(batch=0), 2), (dict(act_dtype=7), 3),
])
def test_bad_dims_are_refused_before_launch(lib, bad, status):
    """Non-null, aligned fake pointers: the call must return before using them."""
    fake = C.c_void_p(0x1000)
    d = mk(**bad)
    assert lib.gdn_decode_step(C.byref(d), fake, fake, fake, fake, fake, None) == status
    assert lib.gdn_conv_update(C.byref(d), fake, fake, fake, fake, None) == status


def test_null_and_misaligned_pointers_are_refused(lib):
    d = mk()
    fake = C.c_void_p(0x1000)
    odd = C.c_void_p(0x1004)
    assert lib.gdn_decode_step(C.byref(d), None, fake, fake, fake, fake, None) == 1
    assert lib.gdn_decode_step(C.byref(d), odd, fake, fake, fake, fake, None) == 4
    assert lib.gdn_decode_step(None, fake, fake, fake, fake, fake, None) == 1


def test_tree_sizes_are_refused_before_launch(lib):
    P = C.c_void_p
    lib.gdn_tree_verify.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, P, P, C.c_size_t, P]
    lib.gdn_commit_path.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, C.c_int32, P, P, P, P]
    fake = C.c_void_p(0x1000)
    d = mk()
    args = [fake] * 3
    # n_nodes out of range
    for n in (0, 33):
        assert lib.gdn_tree_verify(C.byref(d), *args, n, fake, fake, fake, fake, fake, None, fake, 1 << 30, None) == 5
    # at most GDN_MAX_TREE_BATCH sequences per call
    big = mk(batch=65536)
    assert lib.gdn_tree_verify(C.byref(big), *args, 4, fake, fake, fake, fake, fake, None, fake, 1 << 40, None) == 2
    assert lib.gdn_commit_path(C.byref(big), *args, 4, fake, fake, fake, fake, 1, fake, None, None, None) == 2
    # the workspace holds every sequence's nodes: one sized for a single tree is short for two
    lib.gdn_tree_workspace_bytes.restype = C.c_size_t
    lib.gdn_tree_workspace_bytes.argtypes = [C.POINTER(Dims), C.c_int32]
    d2 = mk(batch=2)
    one, two = lib.gdn_tree_workspace_bytes(C.byref(d), 4), lib.gdn_tree_workspace_bytes(C.byref(d2), 4)
    assert two > one > 0
    assert lib.gdn_tree_verify(C.byref(d2), *args, 4, fake, fake, fake, fake, fake, None, fake, one, None) == 6
    # a missing or short workspace is refused before launch
    assert lib.gdn_tree_verify(C.byref(d), *args, 4, fake, fake, fake, fake, fake, None, None, 0, None) == 6
    assert lib.gdn_tree_verify(C.byref(d), *args, 4, fake, fake, fake, fake, fake, None, fake, 1024, None) == 6
    # path longer than the depth limit, than the tree, or empty
    for n, L in ((32, 9), (4, 5), (4, 0)):
        assert lib.gdn_commit_path(C.byref(d), *args, n, fake, fake, fake, fake, L, fake, None, None, None) == 5
    assert lib.gdn_tree_tables(0, fake, fake, fake, fake, None) == 5


def test_fused_token_refuses_overlapping_tails(lib):
    P = C.c_void_p
    lib.gdn_decode_token.argtypes = [C.POINTER(Dims)] + [P] * 9
    d = mk()
    fake = P(0x1000)
    tail_bytes = 4 * 10240 * 2
    # same buffer, and a partial overlap
    assert lib.gdn_decode_token(C.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, None) == 8
    assert lib.gdn_decode_token(C.byref(d), fake, fake, P(0x1000 + tail_bytes - 16), fake, fake, fake, fake, fake,
                                None) == 8
    # bad dims are still refused first
    assert lib.gdn_decode_token(C.byref(mk(conv_width=3)), fake, fake, P(0x1000000), fake, fake, fake, fake, fake,
                                None) == 2


def test_status_strings(lib):
    lib.gdn_status_str.restype = C.c_char_p
    for s in range(12):
        assert lib.gdn_status_str(s) and lib.gdn_status_str(s) != b"unknown status"
    assert lib.gdn_status_str(12) == b"unknown status"
    assert lib.gdn_abi_version() == 1


def fnv1a64(data: bytes) -> int:
    h = 0xCBF29CE484222325
    for byte in data:
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def test_fnv1a64_reference_vectors():
    """The published FNV-1a 64-bit test vectors, so the check below pins the definition."""
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_state_signature_is_the_documented_hash(lib):
    """gdn_state_signature is FNV-1a 64 of the section text the header documents: names,
    shapes and dtypes of the two sections; the batch size does not enter it."""
    lib.gdn_state_signature.restype = C.c_uint64
    lib.gdn_state_signature.argtypes = [C.POINTER(Dims)]
    cases = [mk(), mk(batch=64), mk(act_dtype=0), mk(num_k_heads=4, num_v_heads=4, head_k_dim=32, head_v_dim=32),
             mk(num_k_heads=8)]
    sigs = []
    for d in cases:
        Cc = 2 * d.num_k_heads * d.head_k_dim + d.num_v_heads * d.head_v_dim
        text = (f"gdn-state-v1;state:f32[{d.num_v_heads},{d.head_v_dim},{d.head_k_dim}];"
                f"conv_tail:{'bf16' if d.act_dtype == 1 else 'f32'}[{Cc},4]")
        assert lib.gdn_state_signature(C.byref(d)) == fnv1a64(text.encode())
        sigs.append(lib.gdn_state_signature(C.byref(d)))
    assert sigs[0] == sigs[1]                      # batch is not part of it
    assert len({sigs[0], sigs[2], sigs[3], sigs[4]}) == 4
    assert lib.gdn_state_signature(C.byref(mk(conv_width=3))) == 0


def test_snapshot_sizes_and_refusals(lib):
    P = C.c_void_p
    lib.gdn_snapshot_bytes.restype = C.c_size_t
    lib.gdn_snapshot_bytes.argtypes = [C.POINTER(Dims), C.c_int32]
    for f in (lib.gdn_snapshot, lib.gdn_restore):
        f.argtypes = [C.POINTER(Dims), P, P, C.c_int32, P, P, C.c_size_t, P, P]
    d = mk(batch=4)
    per = 48 * 128 * 128 * 4 + 10240 * 4 * 2
    assert lib.gdn_snapshot_bytes(C.byref(d), 3) == 256 + 3 * per
    assert lib.gdn_snapshot_bytes(C.byref(d), 0) == 0
    assert lib.gdn_snapshot_bytes(C.byref(d), 65536) == 0
    need = 256 + 2 * per
    S, T, Q, ST = P(0x10000000), P(0x20000000), P(0x30000000), P(0x30000100)
    blob = P(0x40000000)
    for f in (lib.gdn_snapshot, lib.gdn_restore):
        assert f(C.byref(d), S, T, 2, Q, blob, need, None, None) == 1          # status is required
        assert f(C.byref(d), S, T, 2, Q, P(0x40000010), need, ST, None) == 4   # blob not 256-byte aligned
        assert f(C.byref(d), S, T, 2, Q, blob, need - 16, ST, None) == 6       # blob too small
        assert f(C.byref(d), S, T, 0, Q, blob, need, ST, None) == 2            # count out of range
        assert f(C.byref(d), S, T, 2, Q, P(0x10000000 + 4096), need, ST, None) == 8   # blob inside the state
        assert f(C.byref(mk(batch=65536)), S, T, 2, Q, blob, need, ST, None) == 2


def test_tree_and_block_calls_refuse_more_than_64_value_heads_per_qk_head(lib):
    P = C.c_void_p
    fake = P(0x1000)
    d = mk(num_k_heads=1, num_v_heads=128, head_k_dim=32, head_v_dim=32)
    lib.gdn_tree_verify.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, P, P, C.c_size_t, P]
    lib.gdn_block_verify.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, C.c_size_t, P]
    assert lib.gdn_tree_verify(C.byref(d), fake, fake, fake, 4, fake, fake, fake, fake, fake, None, fake, 1 << 30,
                               None) == 2
    assert lib.gdn_block_verify(C.byref(d), fake, fake, fake, 4, fake, fake, fake, fake, fake, 1 << 30, None) == 2


def test_ut_form_calls_refuse_what_the_exact_calls_refuse(lib):
    """gdn_tree_verify_ut and gdn_block_verify_ut share the exact calls' argument checks:
    node counts, batch limit, workspace size, heads per q/k head, null pointers."""
    P = C.c_void_p
    fake = P(0x1000)
    lib.gdn_tree_verify_ut.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, P, P, C.c_size_t, P]
    lib.gdn_block_verify_ut.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, C.c_size_t, P]
    d = mk()
    for n in (0, 33):
        assert lib.gdn_tree_verify_ut(C.byref(d), fake, fake, fake, n, fake, fake, fake, fake, fake, None, fake,
                                      1 << 30, None) == 5
        assert lib.gdn_block_verify_ut(C.byref(d), fake, fake, fake, n, fake, fake, fake, fake, fake, 1 << 30,
                                       None) == 2
    big = mk(batch=65536)
    assert lib.gdn_tree_verify_ut(C.byref(big), fake, fake, fake, 4, fake, fake, fake, fake, fake, None, fake,
                                  1 << 40, None) == 2
    assert lib.gdn_tree_verify_ut(C.byref(d), fake, fake, fake, 4, fake, fake, fake, fake, fake, None, fake, 1024,
                                  None) == 6
    assert lib.gdn_block_verify_ut(C.byref(d), fake, fake, fake, 4, fake, fake, fake, fake, fake, 1024, None) == 6
    assert lib.gdn_tree_verify_ut(C.byref(d), None, fake, fake, 4, fake, fake, fake, fake, fake, None, fake, 1 << 30,
                                  None) == 1
    wide = mk(num_k_heads=1, num_v_heads=128, head_k_dim=32, head_v_dim=32)
    assert lib.gdn_tree_verify_ut(C.byref(wide), fake, fake, fake, 4, fake, fake, fake, fake, fake, None, fake,
                                  1 << 30, None) == 2
    assert lib.gdn_block_verify_ut(C.byref(wide), fake, fake, fake, 4, fake, fake, fake, fake, fake, 1 << 30,
                                   None) == 2


def test_prepared_commit_refuses_a_missing_or_short_workspace(lib):
    P = C.c_void_p
    fake = P(0x1000)
    lib.gdn_commit_path_prepared.argtypes = [C.POINTER(Dims), P, P, C.c_int32, P, P, C.c_int32, P, P, P, P,
                                             C.c_size_t, P]
    lib.gdn_tree_workspace_bytes.restype = C.c_size_t
    lib.gdn_tree_workspace_bytes.argtypes = [C.POINTER(Dims), C.c_int32]
    d = mk()
    need = lib.gdn_tree_workspace_bytes(C.byref(d), 8)
    assert lib.gdn_commit_path_prepared(C.byref(d), fake, fake, 8, fake, fake, 3, fake, None, None, None, 0,
                                        None) == 6
    assert lib.gdn_commit_path_prepared(C.byref(d), fake, fake, 8, fake, fake, 3, fake, None, None, fake, need - 1,
                                        None) == 6
    for n, L in ((32, 9), (4, 5), (4, 0), (0, 1)):
        assert lib.gdn_commit_path_prepared(C.byref(d), fake, fake, n, fake, fake, L, fake, None, None, fake, need,
                                            None) == 5
    assert lib.gdn_commit_path_prepared(C.byref(d), None, fake, 8, fake, fake, 3, fake, None, None, fake, need,
                                        None) == 1


def test_prepared_block_commit_refuses_what_block_commit_refuses(lib):
    P = C.c_void_p
    fake = P(0x1000)
    lib.gdn_block_commit_prepared.argtypes = [C.POINTER(Dims), P, P, C.c_int32, P, P, P, P, P, C.c_size_t, P]
    d = mk()
    for k in (0, 33):
        assert lib.gdn_block_commit_prepared(C.byref(d), fake, fake, k, fake, fake, None, None, fake, 1 << 30,
                                             None) == 2
    assert lib.gdn_block_commit_prepared(C.byref(d), fake, fake, 4, fake, fake, None, None, fake, 1024, None) == 6
    assert lib.gdn_block_commit_prepared(C.byref(d), fake, fake, 4, None, fake, None, None, fake, 1 << 30, None) == 1


def test_self_check_refusals(lib):
    """gdn_self_check refuses bad dims, a null or misaligned result word, unknown flags and a
    short workspace before anything is queued (fake pointers are never touched)."""
    lib.gdn_self_check_workspace_bytes.restype = C.c_size_t
    lib.gdn_self_check.argtypes = [C.POINTER(Dims), C.c_uint32, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p,
                                   C.c_void_p]
    d = mk()
    need = lib.gdn_self_check_workspace_bytes(C.byref(d))
    # 32 replayed states of 3.15 MB dominate; the rest is a few MB
    assert 32 * 3_145_728 < need < 160 * 1024 * 1024
    assert lib.gdn_self_check_workspace_bytes(C.byref(mk(head_k_dim=64, head_v_dim=64))) == 0
    ws, res = 1 << 20, 1 << 12   # non-null, aligned fake addresses
    call = lambda dd, flags=0, w=ws, n=need, r=res: lib.gdn_self_check(C.byref(dd), 7, flags, w, n, r, None)
    assert call(mk(num_v_heads=40)) == 2
    assert call(mk(act_dtype=9)) == 3
    assert call(d, r=None) == 1
    assert call(d, r=res + 4) == 4
    assert call(d, flags=2) == 2
    assert call(d, w=None) == 6
    assert call(d, n=need - 1) == 6
    assert call(d, w=ws + 8) == 4


def test_tree_verify_ut_noalloc_refusals(lib):
    """The no-workspace tree verify refuses bad dims, null pointers, bad node counts and a
    batch whose operands exceed its fixed scratch before any device call."""
    P = C.c_void_p
    lib.gdn_tree_verify_ut_noalloc.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, P, P]
    lib.gdn_tree_workspace_bytes.restype = C.c_size_t
    f = P(1 << 20)
    call = lambda d, n=32, o=f: lib.gdn_tree_verify_ut_noalloc(C.byref(d), f, f, f, n, f, f, f, f, o, None, None)
    assert call(mk(num_v_heads=40)) == 2
    assert call(mk(), o=None) == 1
    assert call(mk(), n=0) == 5 and call(mk(), n=33) == 5
    scratch = 16 << 20
    assert lib.gdn_tree_workspace_bytes(C.byref(mk(batch=12)), 32) <= scratch
    assert lib.gdn_tree_workspace_bytes(C.byref(mk(batch=13)), 32) > scratch
    assert call(mk(batch=13)) == 6


def test_prefill_refusals(lib):
    """gdn_prefill_chunked refuses, before any launch: an empty or negative prompt, head
    widths other than 128, more than eight value heads per q/k head (GDN_ERR_SHAPE), a
    missing or short workspace (GDN_ERR_WORKSPACE), a misaligned one (GDN_ERR_ALIGN) and
    a NULL operand (GDN_ERR_NULL)."""
    P = C.c_void_p
    fake = P(0x1000)
    lib.gdn_prefill_chunked.restype = C.c_int
    lib.gdn_prefill_chunked.argtypes = [C.POINTER(Dims), P, P, P, C.c_int32, P, P, P, P, P, C.c_size_t, P]
    lib.gdn_prefill_workspace_bytes.restype = C.c_size_t
    lib.gdn_prefill_workspace_bytes.argtypes = [C.POINTER(Dims), C.c_int32]
    d = mk()
    T = 100
    need = lib.gdn_prefill_workspace_bytes(C.byref(d), T)
    assert need > 0
    call = lambda dd, t, ws, nbytes, state=fake: lib.gdn_prefill_chunked(
        C.byref(dd), state, fake, fake, t, fake, fake, fake, fake, ws, nbytes, None)
    for t in (0, -1):
        assert lib.gdn_prefill_workspace_bytes(C.byref(d), t) == 0
        assert call(d, t, fake, need) == 2
    narrow = mk(num_k_heads=4, num_v_heads=4, head_k_dim=32, head_v_dim=32)
    assert lib.gdn_prefill_workspace_bytes(C.byref(narrow), T) == 0
    assert call(narrow, T, fake, need) == 2
    assert call(mk(num_k_heads=1, num_v_heads=16), T, fake, need) == 2   # 16 value heads per q/k head
    assert call(d, T, None, 0) == 6
    assert call(d, T, fake, need - 1) == 6
    assert call(d, T, P(0x1008), need) == 4
    assert call(d, T, fake, need, state=None) == 1
