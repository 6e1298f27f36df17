"""The C ABI library loads, exports every symbol its header declares, and
rejects bad host arguments before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "a2av.h")


def declared_functions(path):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    return sorted(set(re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", text)))


@pytest.fixture(scope="module")
def L():
    from embeddings_a2av_virtual_amd import _binding
    return _binding.lib()


def test_header_declares_the_boundary():
    names = declared_functions(HEADER)
    for must in ("a2av_exchange_splits", "a2av_offsets", "a2av_copy", "moe_pack", "moe_unpack",
                 "moe_pack_workspace_bytes", "a2av_abi_version", "a2av_strerror",
                 "moe_combine", "moe_regroup", "moe_regroup_workspace_bytes", "keys_bucketize",
                 "keys_bucketize_workspace_bytes", "keys_exchange", "keys_exchange_workspace_bytes",
                 "moe_dispatch_grouped", "moe_dispatch_grouped_workspace_bytes",
                 "moe_combine_grouped", "moe_combine_grouped_workspace_bytes",
                 "moe_pack_dispatch", "moe_pack_dispatch_workspace_bytes", "moe_unpack_return",
                 "moe_unpack_return_workspace_bytes", "moe_combine_return",
                 "moe_combine_return_workspace_bytes"):
        assert must in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions(HEADER):
        assert hasattr(L, name), f"{name} declared in a2av.h but not exported"


def test_only_declared_symbols_are_exported():
    import subprocess
    from embeddings_a2av_virtual_amd._binding import LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.split()[1] in ("T", "W")}
    exported = {n for n in exported if not n.startswith("_")}
    assert exported == set(declared_functions(HEADER))


def test_version_and_strerror(L):
    from embeddings_a2av_virtual_amd import _binding as B
    assert B.a2av_abi_version() == 1
    for code in (0, -1, -2, 1, 2, 4, 8, 16, 32, 12345):
        assert isinstance(B.a2av_strerror(code), str) and B.a2av_strerror(code)


def test_host_argument_errors(L):
    """Checks that return A2AV_EARG before any HIP call is made."""
    EARG = -1
    vp = ctypes.c_void_p
    assert L.a2av_exchange_splits(0, vp(8), vp(8), vp(8), None) == EARG
    assert L.a2av_exchange_splits(65, vp(8), vp(8), vp(8), None) == EARG
    assert L.a2av_exchange_splits(4, None, vp(8), vp(8), None) == EARG
    assert L.a2av_offsets(4, vp(8), vp(8), None, vp(8), vp(8), None) == EARG
    arr = (ctypes.c_void_p * 4)(8, 8, 8, 8)
    rows = (ctypes.c_int64 * 4)(1, 1, 1, 1)
    neg = (ctypes.c_int64 * 4)(1, -1, 1, 1)
    # row_bytes 0, negative rows, rows * row_bytes overflowing, null buffers with rows
    assert L.a2av_copy(4, 0, arr, rows, arr, rows, vp(8), vp(8), vp(8), vp(8), None) == EARG
    assert L.a2av_copy(4, 8, arr, neg, arr, rows, vp(8), vp(8), vp(8), vp(8), None) == EARG
    big = (ctypes.c_int64 * 4)(1, 1 << 62, 1, 1)
    assert L.a2av_copy(4, 8, arr, big, arr, rows, vp(8), vp(8), vp(8), vp(8), None) == EARG
    nul = (ctypes.c_void_p * 4)(8, None, 8, 8)
    assert L.a2av_copy(4, 8, nul, rows, arr, rows, vp(8), vp(8), vp(8), vp(8), None) == EARG
    # MoE size rules: E % W, E above the maximum, T*k past 2^31, small workspace
    assert L.moe_pack_workspace_bytes(8, 8192, 8, 256) > 0
    assert L.moe_pack_workspace_bytes(3, 10, 2, 8) == 0
    assert L.moe_pack_workspace_bytes(1, 10, 2, 4097) == 0
    assert L.moe_pack_workspace_bytes(1, 1 << 29, 8, 8) == 0
    ptrs = (ctypes.c_void_p * 2)(8, 8)
    ws = L.moe_pack_workspace_bytes(2, 10, 2, 8)
    assert L.moe_pack(2, 10, 2, 8, 16, ptrs, ptrs, ptrs, ptrs, vp(8), vp(8), vp(8), ws - 1,
                      vp(8), None) == EARG
    assert L.moe_unpack(2, 10, 0, 16, ptrs, ptrs, ptrs, vp(8), None) == EARG
    # combine: k = 0, H = 0, a null buffer for a rank with tokens
    assert L.moe_combine(2, 10, 0, 16, ptrs, ptrs, ptrs, ptrs, vp(8), None) == EARG
    assert L.moe_combine(2, 10, 2, 0, ptrs, ptrs, ptrs, ptrs, vp(8), None) == EARG
    assert L.moe_combine(2, 10, 2, 16, nul, ptrs, ptrs, ptrs, vp(8), None) == EARG
    # regroup: E % W, bad direction, small workspace, negative rows
    two = (ctypes.c_int64 * 2)(4, 4)
    wsr = L.moe_regroup_workspace_bytes(2, 8)
    assert wsr > 0 and L.moe_regroup_workspace_bytes(3, 8) == 0
    assert L.moe_regroup(3, 8, 16, vp(8), arr, rows, arr, rows, vp(8), 0, vp(8), 1 << 20,
                         vp(8), None) == EARG
    assert L.moe_regroup(2, 8, 16, vp(8), ptrs, two, ptrs, two, vp(8), 2, vp(8), wsr,
                         vp(8), None) == EARG
    assert L.moe_regroup(2, 8, 16, vp(8), ptrs, two, ptrs, two, vp(8), 0, vp(8), wsr - 1,
                         vp(8), None) == EARG
    negr = (ctypes.c_int64 * 2)(4, -4)
    assert L.moe_regroup(2, 8, 16, vp(8), ptrs, negr, ptrs, two, vp(8), 0, vp(8), wsr,
                         vp(8), None) == EARG
    # bucketize: too many tables, negative batch, small workspace, negative key count
    wsb = L.keys_bucketize_workspace_bytes(2, 26)
    assert wsb > 0 and L.keys_bucketize_workspace_bytes(2, 4097) == 0
    assert L.keys_bucketize(2, 26, -1, ptrs, ptrs, two, ptrs, ptrs, vp(8), vp(8), vp(8), wsb,
                            vp(8), None) == EARG
    assert L.keys_bucketize(2, 26, 8, ptrs, ptrs, two, ptrs, ptrs, vp(8), vp(8), vp(8), wsb - 1,
                            vp(8), None) == EARG
    assert L.keys_bucketize(2, 26, 8, ptrs, ptrs, negr, ptrs, ptrs, vp(8), vp(8), vp(8), wsb,
                            vp(8), None) == EARG
    # grouped dispatch: E % W, bad direction, small workspace
    wsg = L.moe_dispatch_grouped_workspace_bytes(2, 8)
    assert wsg > 0 and L.moe_dispatch_grouped_workspace_bytes(3, 8) == 0
    assert L.moe_dispatch_grouped(2, 8, 16, vp(8), ptrs, two, ptrs, two, vp(8), 3, vp(8), wsg,
                                  vp(8), None) == EARG
    assert L.moe_dispatch_grouped(2, 8, 16, vp(8), ptrs, two, ptrs, two, vp(8), 0, vp(8), wsg - 1,
                                  vp(8), None) == EARG
    # grouped combine: small workspace, E % W, H = 0
    wsc = L.moe_combine_grouped_workspace_bytes(2, 10, 2, 8)
    assert wsc > 0 and L.moe_combine_grouped_workspace_bytes(3, 10, 2, 8) == 0
    assert L.moe_combine_grouped(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, two, ptrs, ptrs, vp(8),
                                 wsc - 1, vp(8), None) == EARG
    assert L.moe_combine_grouped(2, 10, 2, 8, 0, vp(8), ptrs, ptrs, ptrs, two, ptrs, ptrs, vp(8),
                                 wsc, vp(8), None) == EARG
    # pack + dispatch: bad layout, k above 64, small workspace, negative capacity
    wsp = L.moe_pack_dispatch_workspace_bytes(2, 10, 2, 8)
    assert wsp > L.moe_pack_workspace_bytes(2, 10, 2, 8)
    assert L.moe_pack_dispatch_workspace_bytes(3, 10, 2, 8) == 0
    assert L.moe_pack_dispatch(2, 10, 2, 8, 16, ptrs, ptrs, ptrs, two, ptrs, vp(8), vp(8), vp(8),
                               2, vp(8), wsp, vp(8), None) == EARG
    assert L.moe_pack_dispatch(2, 10, 65, 8, 16, ptrs, ptrs, ptrs, two, ptrs, vp(8), vp(8), vp(8),
                               0, vp(8), L.moe_pack_dispatch_workspace_bytes(2, 10, 65, 8),
                               vp(8), None) == EARG
    assert L.moe_pack_dispatch(2, 10, 2, 8, 16, ptrs, ptrs, ptrs, two, ptrs, vp(8), vp(8), vp(8),
                               0, vp(8), wsp - 1, vp(8), None) == EARG
    assert L.moe_pack_dispatch(2, 10, 2, 8, 16, ptrs, ptrs, ptrs, negr, ptrs, vp(8), vp(8), vp(8),
                               0, vp(8), wsp, vp(8), None) == EARG
    # its inverse: bad layout, small workspace, negative receive rows, E % W
    wsu = L.moe_unpack_return_workspace_bytes(2, 8)
    assert wsu > 0 and L.moe_unpack_return_workspace_bytes(3, 8) == 0
    assert L.moe_unpack_return(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, two, ptrs, 5, vp(8), wsu,
                               vp(8), None) == EARG
    assert L.moe_unpack_return(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, two, ptrs, 1, vp(8),
                               wsu - 1, vp(8), None) == EARG
    assert L.moe_unpack_return(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, negr, ptrs, 0, vp(8), wsu,
                               vp(8), None) == EARG
    assert L.moe_unpack_return(3, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, two, ptrs, 0, vp(8), wsu,
                               vp(8), None) == EARG
    # combine at the owners: bad layout, H = 0, small workspace, negative rows
    wcr = L.moe_combine_return_workspace_bytes(2, 10, 2, 8)
    assert wcr > 0 and L.moe_combine_return_workspace_bytes(3, 10, 2, 8) == 0
    assert L.moe_combine_return(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, two, ptrs, ptrs, 2,
                                vp(8), wcr, vp(8), None) == EARG
    assert L.moe_combine_return(2, 10, 2, 8, 0, vp(8), ptrs, ptrs, ptrs, two, ptrs, ptrs, 0,
                                vp(8), wcr, vp(8), None) == EARG
    assert L.moe_combine_return(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, two, ptrs, ptrs, 1,
                                vp(8), wcr - 1, vp(8), None) == EARG
    assert L.moe_combine_return(2, 10, 2, 8, 16, vp(8), ptrs, ptrs, ptrs, negr, ptrs, ptrs, 0,
                                vp(8), wcr, vp(8), None) == EARG
    # fused exchange: small workspace, negative capacity, too many tables
    wsx = L.keys_exchange_workspace_bytes(2, 26)
    assert wsx > 0 and L.keys_exchange_workspace_bytes(2, 4097) == 0
    assert L.keys_exchange(2, 26, 8, ptrs, ptrs, two, ptrs, two, ptrs, two, vp(8), vp(8), vp(8),
                           vp(8), wsx - 1, vp(8), None) == EARG
    assert L.keys_exchange(2, 26, 8, ptrs, ptrs, two, ptrs, negr, ptrs, two, vp(8), vp(8), vp(8),
                           vp(8), wsx, vp(8), None) == EARG
    # the no-allocation exchange: sizes whose scratch exceeds its fixed array,
    # then the exchange's own checks, all before any device call
    from embeddings_a2av_virtual_amd import _binding as B
    p64 = (ctypes.c_void_p * 64)(*([8] * 64))
    z64 = (ctypes.c_int64 * 64)(*([0] * 64))
    assert L.keys_exchange_workspace_bytes(64, 4096) > B.NOALLOC_SCRATCH_BYTES
    assert L.keys_exchange_workspace_bytes(8, 26) <= B.NOALLOC_SCRATCH_BYTES
    assert L.keys_exchange_noalloc(64, 4096, 1, p64, p64, z64, p64, z64, p64, z64, vp(8), vp(8),
                                   vp(8), vp(8), None) == EARG
    assert L.keys_exchange_noalloc(2, 4097, 8, ptrs, ptrs, two, ptrs, two, ptrs, two, vp(8),
                                   vp(8), vp(8), vp(8), None) == EARG
    assert L.keys_exchange_noalloc(2, 26, 8, ptrs, ptrs, two, ptrs, negr, ptrs, two, vp(8),
                                   vp(8), vp(8), vp(8), None) == EARG
    assert L.keys_exchange_noalloc(2, 26, -1, ptrs, ptrs, two, ptrs, two, ptrs, two, vp(8),
                                   vp(8), vp(8), vp(8), None) == EARG
    assert L.keys_exchange_noalloc(2, 26, 8, ptrs, ptrs, two, ptrs, two, ptrs, two, vp(8),
                                   vp(8), vp(8), None, None) == EARG
    # one-direction ceilings: sizes and bases that are not 16-byte multiples, null buffers
    assert L.a2av_device_read(vp(16), 24, vp(16), None) == EARG
    assert L.a2av_device_read(vp(20), 32, vp(16), None) == EARG
    assert L.a2av_device_read(vp(16), 32, None, None) == EARG
    assert L.a2av_device_fill(vp(16), 8, 1, 1, None) == EARG
    assert L.a2av_device_fill(vp(24), 32, 1, 0, None) == EARG
    assert L.a2av_device_fill(None, 32, 1, 0, None) == EARG
    assert L.a2av_device_read(None, 0, None, None) == 0 and L.a2av_device_fill(None, 0, 1, 0, None) == 0


def test_workspace_formula(L):
    # one int32 counter per (rank, expert, segment of 1024 slots), 256-byte rounded
    assert L.moe_pack_workspace_bytes(8, 8192, 8, 256) == 8 * 256 * 64 * 4
    assert L.moe_pack_workspace_bytes(2, 0, 2, 8) == 256
