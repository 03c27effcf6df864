"""Python binding of libgdn, the HIP library of the Gated DeltaNet recurrent
mixer for MI355X (gfx950).  The C ABI is include/gdn.h; this module only
marshals torch tensors (device memory) and streams into those calls and
checks that each tensor has the size, dtype and device the call expects, so
that a mistake in Python raises here instead of reaching a kernel.

Every computation runs in the HIP library.  If libgdn.so is missing this
module raises on import: there is no other path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "GdnError", "Dims", "dims", "conv_channels", "state_bytes", "conv_tail_bytes",
    "prefill_workspace_bytes", "tree_workspace_bytes", "block_workspace_bytes", "snapshot_bytes",
    "conv_update", "decode_step", "decode_token", "kda_decode_step", "kda_decode_token", "tree_verify",
    "tree_verify_ut", "commit_path",
    "commit_path_prepared",
    "tree_tables", "block_verify", "block_verify_ut", "block_commit", "block_commit_prepared", "state_signature", "snapshot", "restore", "prefill_chunked",
    "self_check_workspace_bytes", "self_check", "SELF_CHECK_PERTURB", "tree_verify_ut_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "LIB_PATH", "MAX_TREE_NODES", "MAX_TREE_DEPTH", "PREFILL_CHUNK", "PREFILL_SEGMENT", "F32", "BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
MAX_TREE_NODES = 32
MAX_TREE_DEPTH = 8
PREFILL_CHUNK = 64
PREFILL_SEGMENT = 4096   # tokens per group of prefill launches; the workspace stops growing here
F32, BF16 = 0, 1
SELF_CHECK_PERTURB = 1
NOALLOC_SCRATCH_BYTES = 16 << 20
_STATUS_TREE = 5

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python gated_deltanet_decode_amd/build.py`")

_lib = C.CDLL(LIB_PATH)


class Dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("batch", "num_k_heads", "num_v_heads", "head_k_dim",
                                         "head_v_dim", "conv_width", "act_dtype")]

    @property
    def C(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def act_torch(self):
        return torch.bfloat16 if self.act_dtype == BF16 else torch.float32


def dims(batch, num_k_heads, num_v_heads, head_k_dim, head_v_dim, conv_width=4, act="bf16") -> Dims:
    return Dims(batch, num_k_heads, num_v_heads, head_k_dim, head_v_dim, conv_width,
                BF16 if act in ("bf16", BF16, torch.bfloat16) else F32)


_P = C.c_void_p
_D = C.POINTER(Dims)
_I = C.c_int32
_sig = {
    "gdn_abi_version": ([], C.c_int),
    "gdn_status_str": ([C.c_int], C.c_char_p),
    "gdn_conv_channels": ([_D], C.c_size_t),
    "gdn_state_bytes": ([_D], C.c_size_t),
    "gdn_conv_tail_bytes": ([_D], C.c_size_t),
    "gdn_prefill_workspace_bytes": ([_D, _I], C.c_size_t),
    "gdn_conv_update": ([_D, _P, _P, _P, _P, _P], C.c_int),
    "gdn_decode_step": ([_D, _P, _P, _P, _P, _P, _P], C.c_int),
    "gdn_decode_token": ([_D, _P, _P, _P, _P, _P, _P, _P, _P, _P], C.c_int),
    "gdn_kda_decode_step": ([_D, _P, _P, _P, _P, _P, _P], C.c_int),
    "gdn_kda_decode_token": ([_D, _P, _P, _P, _P, _P, _P, _P, _P, _P], C.c_int),
    "gdn_tree_workspace_bytes": ([_D, _I], C.c_size_t),
    "gdn_tree_verify": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_tree_verify_ut": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_commit_path": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P], C.c_int),
    "gdn_block_commit_prepared": ([_D, _P, _P, _I, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_commit_path_prepared": ([_D, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_tree_tables": ([_I, _P, _P, _P, _P, _P], C.c_int),
    "gdn_prefill_chunked": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_block_workspace_bytes": ([_D, _I], C.c_size_t),
    "gdn_block_verify": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_block_verify_ut": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_block_commit": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "gdn_state_signature": ([_D], C.c_uint64),
    "gdn_snapshot_bytes": ([_D, _I], C.c_size_t),
    "gdn_snapshot": ([_D, _P, _P, _I, _P, _P, C.c_size_t, _P, _P], C.c_int),
    "gdn_restore": ([_D, _P, _P, _I, _P, _P, C.c_size_t, _P, _P], C.c_int),
    "gdn_self_check_workspace_bytes": ([_D], C.c_size_t),
    "gdn_self_check": ([_D, C.c_uint32, _I, _P, C.c_size_t, _P, _P], C.c_int),
    "gdn_tree_verify_ut_noalloc": ([_D, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P], C.c_int),
}
for _name, (_args, _res) in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class GdnError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {_lib.gdn_status_str(status).decode()} (status {status})")
        self.status = status


def _check(status: int, call: str) -> None:
    if status != 0:
        raise GdnError(status, call)


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _t(t: torch.Tensor, name: str, dtype, numel: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _opt(t, name, dtype, numel):
    return None if t is None else _t(t, name, dtype, numel)


def conv_channels(d: Dims) -> int:
    return _lib.gdn_conv_channels(C.byref(d))


def state_bytes(d: Dims) -> int:
    return _lib.gdn_state_bytes(C.byref(d))


def conv_tail_bytes(d: Dims) -> int:
    return _lib.gdn_conv_tail_bytes(C.byref(d))


def prefill_workspace_bytes(d: Dims, T: int) -> int:
    return _lib.gdn_prefill_workspace_bytes(C.byref(d), T)


def conv_update(d: Dims, x, tail, w, y, stream=None) -> None:
    B, Cc = d.batch, d.C
    _check(_lib.gdn_conv_update(C.byref(d), _t(x, "x", d.act_torch, B * Cc),
                                _t(tail, "conv_tail", d.act_torch, B * Cc * 4),
                                _t(w, "conv_w", d.act_torch, Cc * 4),
                                _t(y, "y", torch.float32, B * Cc), _stream(stream)), "gdn_conv_update")


def decode_step(d: Dims, state, y, a, b, o, stream=None) -> None:
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    _check(_lib.gdn_decode_step(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                _t(y, "y", torch.float32, B * Cc), _t(a, "a", torch.float32, B * Hv),
                                _t(b, "b", torch.float32, B * Hv), _t(o, "o", torch.float32, B * Hv * dv),
                                _stream(stream)), "gdn_decode_step")


def decode_token(d: Dims, state, tail_in, tail_out, w, x, a, b, o, stream=None) -> None:
    """conv_update + decode_step in one launch; the tail goes from tail_in to tail_out."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    _check(_lib.gdn_decode_token(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                 _t(tail_in, "conv_tail_in", d.act_torch, B * Cc * 4),
                                 _t(tail_out, "conv_tail_out", d.act_torch, B * Cc * 4),
                                 _t(w, "conv_w", d.act_torch, Cc * 4), _t(x, "x", d.act_torch, B * Cc),
                                 _t(a, "a", torch.float32, B * Hv), _t(b, "b", torch.float32, B * Hv),
                                 _t(o, "o", torch.float32, B * Hv * dv), _stream(stream)), "gdn_decode_token")


def kda_decode_step(d: Dims, state, y, a, b, o, stream=None) -> None:
    """decode_step with the per-channel forget gate: a is [B][Hv][dk]."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    _check(_lib.gdn_kda_decode_step(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                    _t(y, "y", torch.float32, B * Cc), _t(a, "a", torch.float32, B * Hv * dk),
                                    _t(b, "b", torch.float32, B * Hv), _t(o, "o", torch.float32, B * Hv * dv),
                                    _stream(stream)), "gdn_kda_decode_step")


def kda_decode_token(d: Dims, state, tail_in, tail_out, w, x, a, b, o, stream=None) -> None:
    """decode_token with the per-channel forget gate: a is [B][Hv][dk]."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    _check(_lib.gdn_kda_decode_token(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                     _t(tail_in, "conv_tail_in", d.act_torch, B * Cc * 4),
                                     _t(tail_out, "conv_tail_out", d.act_torch, B * Cc * 4),
                                     _t(w, "conv_w", d.act_torch, Cc * 4), _t(x, "x", d.act_torch, B * Cc),
                                     _t(a, "a", torch.float32, B * Hv * dk), _t(b, "b", torch.float32, B * Hv),
                                     _t(o, "o", torch.float32, B * Hv * dv), _stream(stream)),
           "gdn_kda_decode_token")


def tree_workspace_bytes(d: Dims, n_nodes: int) -> int:
    return _lib.gdn_tree_workspace_bytes(C.byref(d), n_nodes)


def tree_verify(d: Dims, state, tail, w, parent, x, a, b, o, status=None, workspace=None, stream=None) -> None:
    """One tree of n nodes per sequence: parent [B][n]; workspace: a device byte tensor of at
    least tree_workspace_bytes(d, n) bytes; status [B] or None."""
    _tree_verify("gdn_tree_verify", d, state, tail, w, parent, x, a, b, o, status, workspace, stream)


def tree_verify_ut(d: Dims, state, tail, w, parent, x, a, b, o, status=None, workspace=None, stream=None) -> None:
    """tree_verify in the UT form (one read of each checkpoint, MFMA products); outputs equal
    decode's to rounding rather than bit for bit.  workspace None: one launch that prepares
    nothing for commit_path_prepared; with a workspace, as tree_verify."""
    _tree_verify("gdn_tree_verify_ut", d, state, tail, w, parent, x, a, b, o, status, workspace, stream,
                 optional=True)


def _tree_verify(name, d, state, tail, w, parent, x, a, b, o, status, workspace, stream, optional=False) -> None:
    B = d.batch
    if parent.numel() % B:
        raise ValueError("parent must be [B][n_nodes]")
    n = parent.numel() // B
    Hv, dk, dv, Cc = d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    if workspace is None and optional:
        ws_ptr, ws_bytes = None, 0
    else:
        ws_ptr, ws_bytes = _blob(workspace, tree_workspace_bytes(d, n), "workspace")
    _check(getattr(_lib, name)(C.byref(d), _t(state, "state_ckpt", torch.float32, B * Hv * dv * dk),
                               _t(tail, "conv_tail", d.act_torch, B * Cc * 4), _t(w, "conv_w", d.act_torch, Cc * 4),
                               n, _t(parent, "parent", torch.int32, B * n), _t(x, "x", d.act_torch, B * n * Cc),
                               _t(a, "a", torch.float32, B * n * Hv), _t(b, "b", torch.float32, B * n * Hv),
                               _t(o, "o", torch.float32, B * n * Hv * dv), _opt(status, "tree_status", torch.int32, B),
                               ws_ptr, ws_bytes, _stream(stream)), name)


def commit_path(d: Dims, state, tail, w, parent, x, a, b, path, o=None, status=None, stream=None) -> None:
    """path [B][L]: each row root first, -1 after its end; o [B][L][Hv][dv] or None; status [B] or None."""
    B = d.batch
    if parent.numel() % B or path.numel() % B:
        raise ValueError("parent must be [B][n_nodes] and path [B][path_len]")
    n, L = parent.numel() // B, path.numel() // B
    Hv, dk, dv, Cc = d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    _check(_lib.gdn_commit_path(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                _t(tail, "conv_tail", d.act_torch, B * Cc * 4), _t(w, "conv_w", d.act_torch, Cc * 4),
                                n, _t(parent, "parent", torch.int32, B * n), _t(x, "x", d.act_torch, B * n * Cc),
                                _t(a, "a", torch.float32, B * n * Hv), _t(b, "b", torch.float32, B * n * Hv),
                                L, _t(path, "path", torch.int32, B * L), _opt(o, "o", torch.float32, B * L * Hv * dv),
                                _opt(status, "tree_status", torch.int32, B), _stream(stream)), "gdn_commit_path")


def commit_path_prepared(d: Dims, state, tail, parent, x, path, workspace, o=None, status=None,
                         stream=None) -> None:
    """commit_path for the trees just verified with `workspace` (tree_verify or
    tree_verify_ut on the same inputs): the path's operands are read from it."""
    B = d.batch
    if parent.numel() % B or path.numel() % B:
        raise ValueError("parent must be [B][n_nodes] and path [B][path_len]")
    n, L = parent.numel() // B, path.numel() // B
    Hv, dk, dv, Cc = d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    if workspace is None or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("commit_path_prepared needs the verify's contiguous device workspace tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.gdn_commit_path_prepared(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                         _t(tail, "conv_tail", d.act_torch, B * Cc * 4), n,
                                         _t(parent, "parent", torch.int32, B * n), _t(x, "x", d.act_torch, B * n * Cc),
                                         L, _t(path, "path", torch.int32, B * L),
                                         _opt(o, "o", torch.float32, B * L * Hv * dv),
                                         _opt(status, "tree_status", torch.int32, B), workspace.data_ptr(), ws_bytes,
                                         _stream(stream)), "gdn_commit_path_prepared")


def tree_tables(parent, depth, order, status, stream=None) -> None:
    n = parent.numel()
    _check(_lib.gdn_tree_tables(n, _t(parent, "parent", torch.int32, n), _t(depth, "depth", torch.int32, n),
                                _t(order, "order", torch.int32, n), _t(status, "tree_status", torch.int32, 1),
                                _stream(stream)), "gdn_tree_tables")


def block_workspace_bytes(d: Dims, k: int) -> int:
    return _lib.gdn_block_workspace_bytes(C.byref(d), k)


def _block_common(d, x, workspace, optional=False):
    B, Cc = d.batch, d.C
    if x.numel() % (B * Cc):
        raise ValueError("x must be [B][k][C]")
    k = x.numel() // (B * Cc)
    if workspace is None and optional:
        return k, None, 0
    ptr, nbytes = _blob(workspace, block_workspace_bytes(d, k), "workspace")
    return k, ptr, nbytes


def block_verify(d: Dims, state, tail, w, x, a, b, o, workspace, stream=None) -> None:
    """A block of k tokens per sequence: x [B][k][C], a, b [B][k][Hv], o [B][k][Hv][dv]."""
    _block_verify("gdn_block_verify", d, state, tail, w, x, a, b, o, workspace, stream)


def block_verify_ut(d: Dims, state, tail, w, x, a, b, o, workspace=None, stream=None) -> None:
    """block_verify in the UT form; outputs equal decode's to rounding.  workspace None: one
    launch that prepares nothing for block_commit_prepared."""
    _block_verify("gdn_block_verify_ut", d, state, tail, w, x, a, b, o, workspace, stream, optional=True)


def _block_verify(name, d, state, tail, w, x, a, b, o, workspace, stream, optional=False) -> None:
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    k, ptr, nbytes = _block_common(d, x, workspace, optional)
    _check(getattr(_lib, name)(C.byref(d), _t(state, "state_ckpt", torch.float32, B * Hv * dv * dk),
                               _t(tail, "conv_tail", d.act_torch, B * Cc * 4), _t(w, "conv_w", d.act_torch, Cc * 4),
                               k, _t(x, "x", d.act_torch, B * k * Cc), _t(a, "a", torch.float32, B * k * Hv),
                               _t(b, "b", torch.float32, B * k * Hv), _t(o, "o", torch.float32, B * k * Hv * dv),
                               ptr, nbytes, _stream(stream)), name)


def block_commit(d: Dims, state, tail, w, x, a, b, accepted, o=None, status=None, workspace=None,
                 stream=None) -> None:
    """Advance each sequence by its first accepted[seq] (int32 [B], device) block tokens."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    k, ptr, nbytes = _block_common(d, x, workspace)
    _check(_lib.gdn_block_commit(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                 _t(tail, "conv_tail", d.act_torch, B * Cc * 4), _t(w, "conv_w", d.act_torch, Cc * 4),
                                 k, _t(x, "x", d.act_torch, B * k * Cc), _t(a, "a", torch.float32, B * k * Hv),
                                 _t(b, "b", torch.float32, B * k * Hv), _t(accepted, "accepted", torch.int32, B),
                                 _opt(o, "o", torch.float32, B * k * Hv * dv), _opt(status, "status", torch.int32, B),
                                 ptr, nbytes, _stream(stream)), "gdn_block_commit")


def block_commit_prepared(d: Dims, state, tail, x, accepted, workspace, o=None, status=None, stream=None) -> None:
    """block_commit for the blocks just verified with `workspace` (block_verify or
    block_verify_ut on the same inputs): the operands are read from it."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    k, ptr, nbytes = _block_common(d, x, workspace)
    _check(_lib.gdn_block_commit_prepared(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                          _t(tail, "conv_tail", d.act_torch, B * Cc * 4), k,
                                          _t(x, "x", d.act_torch, B * k * Cc), _t(accepted, "accepted", torch.int32, B),
                                          _opt(o, "o", torch.float32, B * k * Hv * dv),
                                          _opt(status, "status", torch.int32, B), ptr, nbytes, _stream(stream)),
           "gdn_block_commit_prepared")


def state_signature(d: Dims) -> int:
    return _lib.gdn_state_signature(C.byref(d))


def snapshot_bytes(d: Dims, count: int) -> int:
    return _lib.gdn_snapshot_bytes(C.byref(d), count)


def _blob(blob, need, name):
    if not isinstance(blob, torch.Tensor) or blob.device.type != "cuda" or not blob.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    nbytes = blob.numel() * blob.element_size()
    if nbytes < need:
        raise ValueError(f"{name} of {nbytes} bytes, need {need}")
    return blob.data_ptr(), nbytes


def snapshot(d: Dims, state, tail, seqs, blob, status, stream=None) -> None:
    """Copy sequences seqs [count] (int32, device) of (state, tail) into blob (device bytes of at
    least snapshot_bytes(d, count)); status [1] int32 (device) receives the outcome."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    n = seqs.numel()
    ptr, nbytes = _blob(blob, snapshot_bytes(d, n), "blob")
    _check(_lib.gdn_snapshot(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                             _t(tail, "conv_tail", d.act_torch, B * Cc * 4), n, _t(seqs, "seqs", torch.int32, n),
                             ptr, nbytes, _t(status, "status", torch.int32, 1), _stream(stream)), "gdn_snapshot")


def restore(d: Dims, state, tail, seqs, blob, status, stream=None) -> None:
    """Copy blob slots 0..count-1 into sequences seqs [count] (distinct) of (state, tail)."""
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    n = seqs.numel()
    ptr, nbytes = _blob(blob, snapshot_bytes(d, n), "blob")
    _check(_lib.gdn_restore(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                            _t(tail, "conv_tail", d.act_torch, B * Cc * 4), n, _t(seqs, "seqs", torch.int32, n),
                            ptr, nbytes, _t(status, "status", torch.int32, 1), _stream(stream)), "gdn_restore")


def prefill_chunked(d: Dims, state, tail, w, x, a, b, o, workspace=None, stream=None) -> None:
    B, Hv, dk, dv, Cc = d.batch, d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    if x.numel() % (B * Cc):
        raise ValueError("x must be [B][T][C]")
    T = x.numel() // (B * Cc)
    need = prefill_workspace_bytes(d, T)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace of {ws_bytes} bytes, need {need}")
    _check(_lib.gdn_prefill_chunked(C.byref(d), _t(state, "state", torch.float32, B * Hv * dv * dk),
                                    _t(tail, "conv_tail", d.act_torch, B * Cc * 4),
                                    _t(w, "conv_w", d.act_torch, Cc * 4), T, _t(x, "x", d.act_torch, B * T * Cc),
                                    _t(a, "a", torch.float32, B * T * Hv), _t(b, "b", torch.float32, B * T * Hv),
                                    _t(o, "o", torch.float32, B * T * Hv * dv), ws_ptr, ws_bytes, _stream(stream)),
           "gdn_prefill_chunked")


def self_check_workspace_bytes(d: Dims) -> int:
    return _lib.gdn_self_check_workspace_bytes(C.byref(d))


def self_check(d: Dims, result, workspace, seed: int = 0x5EED, flags: int = 0, stream=None) -> None:
    """Queue the load-time self-check for d's layer shape; result [4] int32 (device) receives
    the verdict: result[0] == 0 when verify and commit rows equal decode's bit for bit."""
    ptr, nbytes = _blob(workspace, self_check_workspace_bytes(d), "workspace")
    _check(_lib.gdn_self_check(C.byref(d), seed & 0xFFFFFFFF, flags, ptr, nbytes,
                               _t(result, "result", torch.int32, 4), _stream(stream)), "gdn_self_check")


def tree_verify_ut_noalloc(d: Dims, state, tail, w, parent, x, a, b, o, status=None, stream=None) -> None:
    """tree_verify_ut with no workspace argument: the library's per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES) holds the prepared operands; calls on one GPU must not overlap."""
    B = d.batch
    if parent.numel() % B:
        raise ValueError("parent must be [B][n_nodes]")
    n = parent.numel() // B
    Hv, dk, dv, Cc = d.num_v_heads, d.head_k_dim, d.head_v_dim, d.C
    _check(_lib.gdn_tree_verify_ut_noalloc(C.byref(d), _t(state, "state_ckpt", torch.float32, B * Hv * dv * dk),
                                           _t(tail, "conv_tail", d.act_torch, B * Cc * 4),
                                           _t(w, "conv_w", d.act_torch, Cc * 4), n,
                                           _t(parent, "parent", torch.int32, B * n),
                                           _t(x, "x", d.act_torch, B * n * Cc), _t(a, "a", torch.float32, B * n * Hv),
                                           _t(b, "b", torch.float32, B * n * Hv),
                                           _t(o, "o", torch.float32, B * n * Hv * dv),
                                           _opt(status, "tree_status", torch.int32, B), _stream(stream)),
           "gdn_tree_verify_ut_noalloc")
