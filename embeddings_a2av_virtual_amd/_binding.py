"""ctypes binding of ``liba2av.so`` (the C ABI in ``include/a2av.h``).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the stream to the C entry
point of the same name, and raises :class:`A2avError` for a nonzero host
return code. All computation runs in the library's HIP kernels; if the library
is missing the first call raises, there is no fallback.

torch is used for device memory and streams only. The stream defaults to
torch's current stream on the tensors' device.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "A2avError", "lib", "LIB_PATH",
    "OK", "EARG", "EHIP", "MAX_W", "MAX_SPLIT", "MAX_EXPERTS",
    "ST_BAD_SPLIT", "ST_SEND_OVERRUN", "ST_RECV_OVERFLOW", "ST_BAD_EXPERT", "ST_BAD_OFFSETS",
    "ST_BAD_PERM",
    "a2av_abi_version", "a2av_strerror", "a2av_exchange_splits", "a2av_offsets", "a2av_copy",
    "a2av_all_to_all_vdev",
    "moe_pack_workspace_bytes", "moe_pack", "moe_unpack", "moe_combine",
    "moe_regroup_workspace_bytes", "moe_regroup", "moe_dispatch_grouped_workspace_bytes",
    "moe_dispatch_grouped", "moe_combine_grouped_workspace_bytes", "moe_combine_grouped",
    "moe_pack_dispatch_workspace_bytes", "moe_pack_dispatch", "moe_unpack_return_workspace_bytes",
    "moe_unpack_return", "moe_combine_return_workspace_bytes", "moe_combine_return",
    "keys_bucketize_workspace_bytes",
    "keys_bucketize", "keys_exchange_workspace_bytes", "keys_exchange",
    "keys_exchange_noalloc", "NOALLOC_SCRATCH_BYTES", "a2av_device_copy",
    "a2av_device_read", "a2av_device_fill", "SINK_WORDS",
    "MAX_TABLES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liba2av.so")

OK, EARG, EHIP = 0, -1, -2
MAX_W = 64
MAX_SPLIT = 1 << 40
MAX_EXPERTS = 4096
MAX_TABLES = 4096
NOALLOC_SCRATCH_BYTES = 1 << 20
SINK_WORDS = 4096
ST_BAD_SPLIT = 1
ST_SEND_OVERRUN = 2
ST_RECV_OVERFLOW = 4
ST_BAD_EXPERT = 8
ST_BAD_OFFSETS = 16
ST_BAD_PERM = 32

_lib = None


class A2avError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code}: {a2av_strerror(code)}")
        self.code = code


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m embeddings_a2av_virtual_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        vpp = ctypes.POINTER(ctypes.c_void_p)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.a2av_abi_version.argtypes = []
        L.a2av_abi_version.restype = i32
        L.a2av_strerror.argtypes = [i32]
        L.a2av_strerror.restype = ctypes.c_char_p
        L.a2av_exchange_splits.argtypes = [i32, vp, vp, vp, vp]
        L.a2av_offsets.argtypes = [i32, vp, vp, vp, vp, vp, vp]
        L.a2av_copy.argtypes = [i32, sz, vpp, i64p, vpp, i64p, vp, vp, vp, vp, vp]
        L.a2av_all_to_all_vdev.argtypes = [i32, sz, vpp, i64p, vpp, i64p, vp, vp, vp, vp, vp, vp]
        L.moe_pack_workspace_bytes.argtypes = [i32, i64, i32, i32]
        L.moe_pack_workspace_bytes.restype = sz
        L.moe_pack.argtypes = [i32, i64, i32, i32, sz, vpp, vpp, vpp, vpp, vp, vp, vp, sz, vp, vp]
        L.moe_unpack.argtypes = [i32, i64, i32, sz, vpp, vpp, vpp, vp, vp]
        L.moe_combine.argtypes = [i32, i64, i32, i64, vpp, vpp, vpp, vpp, vp, vp]
        L.moe_regroup_workspace_bytes.argtypes = [i32, i32]
        L.moe_regroup_workspace_bytes.restype = sz
        L.moe_regroup.argtypes = [i32, i32, sz, vp, vpp, i64p, vpp, i64p, vp, i32, vp, sz, vp, vp]
        L.moe_dispatch_grouped_workspace_bytes.argtypes = [i32, i32]
        L.moe_dispatch_grouped_workspace_bytes.restype = sz
        L.moe_dispatch_grouped.argtypes = [i32, i32, sz, vp, vpp, i64p, vpp, i64p, vp, i32, vp, sz,
                                           vp, vp]
        L.moe_combine_grouped_workspace_bytes.argtypes = [i32, i64, i32, i32]
        L.moe_combine_grouped_workspace_bytes.restype = sz
        L.moe_combine_grouped.argtypes = [i32, i64, i32, i32, i64, vp, vpp, vpp, vpp, i64p, vpp,
                                          vpp, vp, sz, vp, vp]
        L.moe_pack_dispatch_workspace_bytes.argtypes = [i32, i64, i32, i32]
        L.moe_pack_dispatch_workspace_bytes.restype = sz
        L.moe_pack_dispatch.argtypes = [i32, i64, i32, i32, sz, vpp, vpp, vpp, i64p, vpp, vp, vp,
                                        vp, i32, vp, sz, vp, vp]
        L.moe_unpack_return_workspace_bytes.argtypes = [i32, i32]
        L.moe_unpack_return_workspace_bytes.restype = sz
        L.moe_unpack_return.argtypes = [i32, i64, i32, i32, sz, vp, vpp, vpp, vpp, i64p, vpp, i32,
                                        vp, sz, vp, vp]
        L.moe_combine_return_workspace_bytes.argtypes = [i32, i64, i32, i32]
        L.moe_combine_return_workspace_bytes.restype = sz
        L.moe_combine_return.argtypes = [i32, i64, i32, i32, i64, vp, vpp, vpp, vpp, i64p, vpp, vpp,
                                         i32, vp, sz, vp, vp]
        L.keys_bucketize_workspace_bytes.argtypes = [i32, i32]
        L.keys_bucketize_workspace_bytes.restype = sz
        L.keys_bucketize.argtypes = [i32, i32, i64, vpp, vpp, i64p, vpp, vpp, vp, vp, vp, sz, vp,
                                     vp]
        L.keys_exchange_workspace_bytes.argtypes = [i32, i32]
        L.keys_exchange_workspace_bytes.restype = sz
        L.keys_exchange.argtypes = [i32, i32, i64, vpp, vpp, i64p, vpp, i64p, vpp, i64p, vp, vp, vp,
                                    vp, sz, vp, vp]
        L.keys_exchange_noalloc.argtypes = [i32, i32, i64, vpp, vpp, i64p, vpp, i64p, vpp, i64p,
                                            vp, vp, vp, vp, vp]
        L.a2av_device_copy.argtypes = [vp, vp, sz, vp]
        L.a2av_device_read.argtypes = [vp, sz, vp, vp]
        L.a2av_device_fill.argtypes = [vp, sz, ctypes.c_uint32, i32, vp]
        for f in ("a2av_exchange_splits", "a2av_offsets", "a2av_copy", "a2av_all_to_all_vdev",
                  "moe_pack", "moe_unpack", "moe_combine", "moe_regroup", "moe_dispatch_grouped",
                  "moe_combine_grouped", "moe_pack_dispatch", "moe_unpack_return",
                  "moe_combine_return",
                  "keys_bucketize", "keys_exchange", "keys_exchange_noalloc",
                  "a2av_device_copy", "a2av_device_read", "a2av_device_fill"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling helpers
def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream, like: torch.Tensor) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr_array(tensors, name):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else _dev(t, f"{name}[{i}]")
    return arr


def _i64_array(vals):
    arr = (ctypes.c_int64 * len(vals))()
    for i, v in enumerate(vals):
        arr[i] = int(v)
    return arr


def _check(fn, rc):
    if rc != OK:
        raise A2avError(fn, rc)


# ------------------------------------------------------------------ entry points
def a2av_abi_version() -> int:
    return lib().a2av_abi_version()


def a2av_strerror(code: int) -> str:
    return lib().a2av_strerror(int(code)).decode()


def a2av_exchange_splits(S, O, status, stream=None):
    """O[d][s] = S[s][d]; S, O: int64 [W, W] on the GPU; status: int32 [1]."""
    W = S.shape[0]
    _check("a2av_exchange_splits",
           lib().a2av_exchange_splits(W, _dev(S, "S"), _dev(O, "O"), _dev(status, "status"),
                                      _stream(stream, S)))


def a2av_offsets(S, O, send_off, recv_off, status, stream=None):
    """Exclusive scans of the rows of S and O into [W, W+1] int64 offsets."""
    W = S.shape[0]
    _check("a2av_offsets",
           lib().a2av_offsets(W, _dev(S, "S"), _dev(O, "O"), _dev(send_off, "send_off"),
                              _dev(recv_off, "recv_off"), _dev(status, "status"),
                              _stream(stream, S)))


def a2av_copy(row_bytes, ins, in_rows, outs, out_cap_rows, S, send_off, recv_off, status,
              stream=None):
    """Payload step. ``ins``/``outs``: W GPU tensors (any dtype, contiguous);
    ``in_rows``/``out_cap_rows``: W host integers (rows each buffer holds)."""
    W = len(ins)
    if len(outs) != W or len(in_rows) != W or len(out_cap_rows) != W:
        raise ValueError("ins, outs, in_rows and out_cap_rows need W entries each")
    _check("a2av_copy",
           lib().a2av_copy(W, int(row_bytes), _ptr_array(ins, "ins"), _i64_array(in_rows),
                           _ptr_array(outs, "outs"), _i64_array(out_cap_rows), _dev(S, "S"),
                           _dev(send_off, "send_off"), _dev(recv_off, "recv_off"),
                           _dev(status, "status"), _stream(stream, S)))


def a2av_all_to_all_vdev(row_bytes, ins, in_rows, outs, out_cap_rows, S, O, send_off, recv_off,
                         status, stream=None):
    """Exchange, offsets and payload in one call (one launch for W <= 16)."""
    W = len(ins)
    if len(outs) != W or len(in_rows) != W or len(out_cap_rows) != W:
        raise ValueError("ins, outs, in_rows and out_cap_rows need W entries each")
    _check("a2av_all_to_all_vdev",
           lib().a2av_all_to_all_vdev(W, int(row_bytes), _ptr_array(ins, "ins"),
                                      _i64_array(in_rows), _ptr_array(outs, "outs"),
                                      _i64_array(out_cap_rows), _dev(S, "S"), _dev(O, "O"),
                                      _dev(send_off, "send_off"), _dev(recv_off, "recv_off"),
                                      _dev(status, "status"), _stream(stream, S)))


def moe_pack_workspace_bytes(W, T, k, E) -> int:
    return int(lib().moe_pack_workspace_bytes(int(W), int(T), int(k), int(E)))


def moe_pack(W, T, k, E, row_bytes, tokens, ids, send, perm, S, expert_counts, workspace,
             status, stream=None):
    """Stable pack of every rank's routing slots by expert id (see a2av.h)."""
    _check("moe_pack",
           lib().moe_pack(int(W), int(T), int(k), int(E), int(row_bytes),
                          _ptr_array(tokens, "tokens"), _ptr_array(ids, "ids"),
                          _ptr_array(send, "send"), _ptr_array(perm, "perm"), _dev(S, "S"),
                          _dev(expert_counts, "expert_counts"), _dev(workspace, "workspace"),
                          workspace.numel() * workspace.element_size(), _dev(status, "status"),
                          _stream(stream, S)))


def moe_unpack(W, T, k, row_bytes, back, perm, out, status, stream=None):
    """out[r][q] = back[r][perm[r][q]] for every rank r."""
    _check("moe_unpack",
           lib().moe_unpack(int(W), int(T), int(k), int(row_bytes), _ptr_array(back, "back"),
                            _ptr_array(perm, "perm"), _ptr_array(out, "out"),
                            _dev(status, "status"), _stream(stream, status)))


def moe_combine(W, T, k, H, back, perm, weights, out, status, stream=None):
    """Gate-weighted combine: out[r][t] = bf16(fma chain over j of
    weights[r][t][j] * back[r][perm[r][t*k+j]]), in slot order."""
    _check("moe_combine",
           lib().moe_combine(int(W), int(T), int(k), int(H), _ptr_array(back, "back"),
                             _ptr_array(perm, "perm"), _ptr_array(weights, "weights"),
                             _ptr_array(out, "out"), _dev(status, "status"),
                             _stream(stream, status)))


def moe_regroup_workspace_bytes(W, E) -> int:
    return int(lib().moe_regroup_workspace_bytes(int(W), int(E)))


def moe_regroup(W, E, row_bytes, counts, ins, in_rows, outs, out_cap_rows, expert_offsets,
                direction, workspace, status, stream=None):
    """Per-rank regroup between (source, expert) and (expert, source) row order."""
    if len(ins) != W or len(outs) != W or len(in_rows) != W or len(out_cap_rows) != W:
        raise ValueError("ins, outs, in_rows and out_cap_rows need W entries each")
    _check("moe_regroup",
           lib().moe_regroup(int(W), int(E), int(row_bytes), _dev(counts, "counts"),
                             _ptr_array(ins, "ins"), _i64_array(in_rows), _ptr_array(outs, "outs"),
                             _i64_array(out_cap_rows), _dev(expert_offsets, "expert_offsets"),
                             int(direction), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(),
                             _dev(status, "status"), _stream(stream, status)))


def moe_dispatch_grouped_workspace_bytes(W, E) -> int:
    return int(lib().moe_dispatch_grouped_workspace_bytes(int(W), int(E)))


def moe_dispatch_grouped(W, E, row_bytes, counts, ins, in_rows, outs, out_cap_rows,
                         expert_offsets, direction, workspace, status, stream=None):
    """Dispatch a2av + expert regroup in one copy (direction 0), or its inverse (1)."""
    if len(ins) != W or len(outs) != W or len(in_rows) != W or len(out_cap_rows) != W:
        raise ValueError("ins, outs, in_rows and out_cap_rows need W entries each")
    _check("moe_dispatch_grouped",
           lib().moe_dispatch_grouped(int(W), int(E), int(row_bytes), _dev(counts, "counts"),
                                      _ptr_array(ins, "ins"), _i64_array(in_rows),
                                      _ptr_array(outs, "outs"), _i64_array(out_cap_rows),
                                      _dev(expert_offsets, "expert_offsets"), int(direction),
                                      _dev(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _dev(status, "status"), _stream(stream, status)))


def moe_combine_grouped_workspace_bytes(W, T, k, E) -> int:
    return int(lib().moe_combine_grouped_workspace_bytes(int(W), int(T), int(k), int(E)))


def moe_combine_grouped(W, T, k, E, H, counts, ids, perm, expert_side, exp_rows, weights, out,
                        workspace, status, stream=None):
    """The return trip and the weighted combine in one pass, reading every
    slot's row on its owner's expert side."""
    _check("moe_combine_grouped",
           lib().moe_combine_grouped(int(W), int(T), int(k), int(E), int(H),
                                     _dev(counts, "counts"), _ptr_array(ids, "ids"),
                                     _ptr_array(perm, "perm"),
                                     _ptr_array(expert_side, "expert_side"),
                                     _i64_array(exp_rows), _ptr_array(weights, "weights"),
                                     _ptr_array(out, "out"), _dev(workspace, "workspace"),
                                     workspace.numel() * workspace.element_size(),
                                     _dev(status, "status"), _stream(stream, status)))


def moe_pack_dispatch_workspace_bytes(W, T, k, E) -> int:
    return int(lib().moe_pack_dispatch_workspace_bytes(int(W), int(T), int(k), int(E)))


def moe_pack_dispatch(W, T, k, E, row_bytes, tokens, ids, recv, recv_cap_rows, perm, S,
                      expert_counts, block_offsets, layout, workspace, status, stream=None):
    """moe_pack and the dispatch in one step: every slot's token row written
    straight into its owner's receive buffer (layout 0: source-major, as the
    a2av delivers; 1: expert-major, as the grouped dispatch delivers)."""
    if (len(tokens) != W or len(ids) != W or len(recv) != W or len(recv_cap_rows) != W
            or len(perm) != W):
        raise ValueError("tokens, ids, recv, recv_cap_rows and perm need W entries each")
    _check("moe_pack_dispatch",
           lib().moe_pack_dispatch(int(W), int(T), int(k), int(E), int(row_bytes),
                                   _ptr_array(tokens, "tokens"), _ptr_array(ids, "ids"),
                                   _ptr_array(recv, "recv"), _i64_array(recv_cap_rows),
                                   _ptr_array(perm, "perm"), _dev(S, "S"),
                                   _dev(expert_counts, "expert_counts"),
                                   _dev(block_offsets, "block_offsets"), int(layout),
                                   _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(),
                                   _dev(status, "status"), _stream(stream, status)))


def moe_unpack_return_workspace_bytes(W, E) -> int:
    return int(lib().moe_unpack_return_workspace_bytes(int(W), int(E)))


def moe_unpack_return(W, T, k, E, row_bytes, expert_counts, ids, perm, recv, recv_rows, out,
                      layout, workspace, status, stream=None):
    """The inverse of moe_pack_dispatch: every slot's row read back from its
    owner's receive buffer."""
    if len(ids) != W or len(perm) != W or len(recv) != W or len(recv_rows) != W or len(out) != W:
        raise ValueError("ids, perm, recv, recv_rows and out need W entries each")
    _check("moe_unpack_return",
           lib().moe_unpack_return(int(W), int(T), int(k), int(E), int(row_bytes),
                                   _dev(expert_counts, "expert_counts"), _ptr_array(ids, "ids"),
                                   _ptr_array(perm, "perm"), _ptr_array(recv, "recv"),
                                   _i64_array(recv_rows), _ptr_array(out, "out"), int(layout),
                                   _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(),
                                   _dev(status, "status"), _stream(stream, status)))


def moe_combine_return_workspace_bytes(W, T, k, E) -> int:
    return int(lib().moe_combine_return_workspace_bytes(int(W), int(T), int(k), int(E)))


def moe_combine_return(W, T, k, E, H, expert_counts, ids, perm, recv, recv_rows, weights, out,
                       layout, workspace, status, stream=None):
    """The return trip and the gate-weighted combine in one pass, reading
    every slot's row where moe_pack_dispatch left it."""
    if (len(ids) != W or len(perm) != W or len(recv) != W or len(recv_rows) != W
            or len(weights) != W or len(out) != W):
        raise ValueError("ids, perm, recv, recv_rows, weights and out need W entries each")
    _check("moe_combine_return",
           lib().moe_combine_return(int(W), int(T), int(k), int(E), int(H),
                                    _dev(expert_counts, "expert_counts"), _ptr_array(ids, "ids"),
                                    _ptr_array(perm, "perm"), _ptr_array(recv, "recv"),
                                    _i64_array(recv_rows), _ptr_array(weights, "weights"),
                                    _ptr_array(out, "out"), int(layout),
                                    _dev(workspace, "workspace"),
                                    workspace.numel() * workspace.element_size(),
                                    _dev(status, "status"), _stream(stream, status)))


def keys_bucketize_workspace_bytes(W, n_tables) -> int:
    return int(lib().keys_bucketize_workspace_bytes(int(W), int(n_tables)))


def keys_bucketize(W, n_tables, batch, lengths, keys, n_keys, lengths_out, keys_out, split_keys,
                   split_lengths, workspace, status, stream=None):
    """Owner-order bucketing of every rank's jagged keys (table t -> rank t mod W)."""
    if len(lengths) != W or len(keys) != W or len(n_keys) != W:
        raise ValueError("lengths, keys and n_keys need W entries each")
    _check("keys_bucketize",
           lib().keys_bucketize(int(W), int(n_tables), int(batch), _ptr_array(lengths, "lengths"),
                                _ptr_array(keys, "keys"), _i64_array(n_keys),
                                _ptr_array(lengths_out, "lengths_out"),
                                _ptr_array(keys_out, "keys_out"), _dev(split_keys, "split_keys"),
                                _dev(split_lengths, "split_lengths"), _dev(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(),
                                _dev(status, "status"), _stream(stream, status)))


def keys_exchange_workspace_bytes(W, n_tables) -> int:
    return int(lib().keys_exchange_workspace_bytes(int(W), int(n_tables)))


def keys_exchange(W, n_tables, batch, lengths, keys, n_keys, lengths_out, lengths_cap, keys_out,
                  keys_cap, split_keys, split_lengths, recv_off_keys, workspace, status,
                  stream=None):
    """Bucketing and both exchanges of one batch's keys in one call."""
    if any(len(x) != W for x in (lengths, keys, n_keys, lengths_out, lengths_cap, keys_out,
                                 keys_cap)):
        raise ValueError("every per-rank list needs W entries")
    _check("keys_exchange",
           lib().keys_exchange(int(W), int(n_tables), int(batch), _ptr_array(lengths, "lengths"),
                               _ptr_array(keys, "keys"), _i64_array(n_keys),
                               _ptr_array(lengths_out, "lengths_out"), _i64_array(lengths_cap),
                               _ptr_array(keys_out, "keys_out"), _i64_array(keys_cap),
                               _dev(split_keys, "split_keys"), _dev(split_lengths, "split_lengths"),
                               _dev(recv_off_keys, "recv_off_keys"), _dev(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(),
                               _dev(status, "status"), _stream(stream, status)))


def keys_exchange_noalloc(W, n_tables, batch, lengths, keys, n_keys, lengths_out, lengths_cap,
                          keys_out, keys_cap, split_keys, split_lengths, recv_off_keys, status,
                          stream=None):
    """keys_exchange with the library's fixed per-GPU scratch instead of a
    workspace (allocates nothing)."""
    if any(len(x) != W for x in (lengths, keys, n_keys, lengths_out, lengths_cap, keys_out,
                                 keys_cap)):
        raise ValueError("every per-rank list needs W entries")
    _check("keys_exchange_noalloc",
           lib().keys_exchange_noalloc(int(W), int(n_tables), int(batch),
                                       _ptr_array(lengths, "lengths"), _ptr_array(keys, "keys"),
                                       _i64_array(n_keys), _ptr_array(lengths_out, "lengths_out"),
                                       _i64_array(lengths_cap), _ptr_array(keys_out, "keys_out"),
                                       _i64_array(keys_cap), _dev(split_keys, "split_keys"),
                                       _dev(split_lengths, "split_lengths"),
                                       _dev(recv_off_keys, "recv_off_keys"),
                                       _dev(status, "status"), _stream(stream, status)))


def a2av_device_copy(dst, src, nbytes, stream=None):
    """Plain contiguous copy of nbytes from src to dst (bandwidth ceiling)."""
    _check("a2av_device_copy",
           lib().a2av_device_copy(_dev(dst, "dst"), _dev(src, "src"), int(nbytes),
                                  _stream(stream, dst)))


def a2av_device_read(src, nbytes, sink, stream=None):
    """Read nbytes of src once (read-only bandwidth ceiling); each wave XORs
    the fold of what it read into one word of sink (SINK_WORDS int64)."""
    if sink.numel() * sink.element_size() < SINK_WORDS * 8:
        raise ValueError("sink needs SINK_WORDS int64 words")
    _check("a2av_device_read",
           lib().a2av_device_read(_dev(src, "src"), int(nbytes), _dev(sink, "sink"),
                                  _stream(stream, src)))


def a2av_device_fill(dst, nbytes, pattern, nontemporal=True, stream=None):
    """Write the 32-bit pattern over nbytes of dst (write-only bandwidth ceiling)."""
    _check("a2av_device_fill",
           lib().a2av_device_fill(_dev(dst, "dst"), int(nbytes), int(pattern) & 0xFFFFFFFF,
                                  1 if nontemporal else 0, _stream(stream, dst)))
