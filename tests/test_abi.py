"""Host-side checks of the C ABI (CPU only: no kernel is launched).

Every call here fails validation before any launch, so it runs without a GPU: the library
loads, exports every symbol include/gla.h declares, returns the documented status codes, and
computes workspace sizes.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    m = pytest.importorskip("linear_recurrent_sequence_gla_amd")
    if not os.path.exists(m.lib_path):
        pytest.skip("library not built")
    return m.lib()


def header_symbols():
    src = open(os.path.join(ROOT, "include", "gla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|int|size_t)\s+(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    import linear_recurrent_sequence_gla_amd as m
    syms = header_symbols()
    assert len(syms) >= 12, syms
    for s in syms:
        assert hasattr(lib, s), f"{s} declared in gla.h but not exported"
    assert set(syms) == set(m.EXPORTED_SYMBOLS), (set(syms) ^ set(m.EXPORTED_SYMBOLS))


def test_version_and_status_strings(lib):
    assert lib.gla_abi_version() >= 1
    for code in range(9):
        s = lib.gla_status_str(code).decode()
        assert s.startswith("GLA_"), s
    assert lib.gla_status_str(99).decode() == "unknown status"


NOP = [None] * 7


def fwd(lib, B=1, H=1, L=64, Dk=16, Dv=16, C=16, dt=1, ptrs=None, ws=None, wsb=0):
    p = ptrs if ptrs is not None else NOP
    return lib.gla_fwd(*p, B, H, L, Dk, Dv, C, dt, ws, wsb, None)


def test_dtype_shape_unsupported(lib):
    assert fwd(lib, dt=5) == 3                        # GLA_ERR_DTYPE
    assert fwd(lib, L=0) == 2                         # GLA_ERR_SHAPE
    assert fwd(lib, B=0) == 2
    assert fwd(lib, C=48) == 4                        # GLA_ERR_UNSUPPORTED
    assert fwd(lib, Dk=24) == 4
    assert fwd(lib, Dk=512) == 4
    assert fwd(lib, Dv=520) == 4
    # chunk sizes whose tiles exceed a CU's LDS run at a smaller chunk (the result does not
    # depend on C): accepted, so these calls get as far as their NULL pointers
    assert fwd(lib, Dk=256, C=128) == 1               # bf16: runs at C = 64
    assert fwd(lib, Dk=128, C=128, dt=0) == 1         # fp32: runs at C = 64
    assert lib.gla_fwd_workspace_bytes(1, 1, 64, 64, 16, 128, 0) > 0        # fp32 forward fits
    assert lib.gla_bwd_workspace_bytes(1, 1, 64, 64, 16, 128, 0) == lib.gla_bwd_workspace_bytes(1, 1, 64, 64, 16, 64, 0)
    assert lib.gla_saved_bytes(1, 1, 300, 256, 64, 128, 1) == lib.gla_saved_bytes(1, 1, 300, 256, 64, 64, 1) > 0
    assert lib.gla_fwd_workspace_bytes(1, 1, 300, 256, 64, 128, 1) == lib.gla_fwd_workspace_bytes(1, 1, 300, 256, 64, 64, 1)
    assert fwd(lib, B=70000) == 4                     # grid limit


def test_null_workspace_alias(lib):
    a = ctypes.c_void_p(0x10000000)
    b = ctypes.c_void_p(0x20000000)
    assert fwd(lib) == 1                              # NULL pointers
    ptrs = [a, ctypes.c_void_p(0x11000000), ctypes.c_void_p(0x12000000), ctypes.c_void_p(0x13000000), None, b, None]
    need = lib.gla_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 1)
    assert need > 0
    assert fwd(lib, ptrs=ptrs, ws=None, wsb=0) == 5   # no workspace
    assert fwd(lib, ptrs=ptrs, ws=ctypes.c_void_p(0x30000000), wsb=need - 1) == 5
    alias = list(ptrs)
    alias[5] = ctypes.c_void_p(0x10000000 + 64)       # o overlaps q
    assert fwd(lib, ptrs=alias, ws=ctypes.c_void_p(0x30000000), wsb=need) == 6
    wsalias = ctypes.c_void_p(0x20000000 + 32)        # workspace overlaps o
    assert fwd(lib, ptrs=ptrs, ws=wsalias, wsb=need) == 6
    mis = list(ptrs)
    mis[0] = ctypes.c_void_p(0x10000000 + 2)          # misaligned q
    assert fwd(lib, ptrs=mis, ws=ctypes.c_void_p(0x30000000), wsb=need) == 4


def test_workspace_sizes(lib):
    # forward: Qs, KdT (C x Dk each, bf16), A (C x C), Gamma (fp32) per chunk, 256-byte
    # aligned, then the chunk-start states (Dk x Dv bf16 per chunk)
    B, H, L, Dk, Dv, C = 8, 4, 2048, 128, 256, 64
    N = L // C
    expect = 2 * (B * H * N * C * Dk * 2) + B * H * N * C * C * 2 + B * H * N * Dk * 4 + B * H * N * Dk * Dv * 2
    assert lib.gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, 1) == expect
    assert lib.gla_bwd_workspace_bytes(B, H, L, Dk, Dv, C, 1) > expect
    assert lib.gla_fwd_workspace_bytes(1, 1, 64, 16, 16, 48, 1) == 0
    assert lib.gla_bwd_launch_count(B, H, L, Dk, Dv, C, 1) == 4
    assert lib.gla_bwd_launch_count(4, 4, 4096, 256, 512, 64, 1) == 5
    # the forward's kernel phases: 3, or 2 where the walk and the outputs run as one kernel,
    # which depends on the device's compute units (none here: 3)
    assert lib.gla_fwd_launch_count(B, H, L, Dk, Dv, C, 1, 0) in (2, 3)
    assert lib.gla_fwd_launch_count(B, H, L, Dk, Dv, C, 1, 1) in (2, 3)
    assert lib.gla_fwd_launch_count(1, 1, 64, 16, 16, 64, 0, 0) == 3     # fp32: never fused
    assert lib.gla_fwd_launch_count(1, 1, 64, 16, 16, 48, 1, 0) == 0     # unsupported chunk size


def test_forward_workspace_keeps_room_for_a_segmented_walk(lib):
    # few, long sequences: room for up to 8 walk segments (two fp32 [BH][8][Dk][Dv] carry
    # buffers and the per-chunk decay prefixes); many sequences: none
    B, H, L, Dk, Dv, C = 1, 4, 20480, 128, 256, 64
    N = L // C
    ops = 2 * (B * H * N * C * Dk * 2) + B * H * N * C * C * 2 + B * H * N * Dk * 4
    states = B * H * N * Dk * Dv * 2
    seg = (2 * B * H * 8 * Dk * Dv + B * H * N * Dk + B * H * 8 * Dk) * 4
    assert lib.gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, 1) == ops + states + seg
    # no segmentation scratch at 32 sequences, so the forward workspace is the saved layout
    assert lib.gla_fwd_workspace_bytes(8, 4, 2048, 128, 256, 64, 1) == lib.gla_saved_bytes(8, 4, 2048, 128, 256, 64, 1)


def test_saved_path_sizes_and_validation(lib):
    # saved = the chunk operands (Qs, KdT, A, Gam) + chunk-start states; its workspace = dH
    B, H, L, Dk, Dv, C = 8, 4, 2048, 128, 256, 64
    N = L // C
    ops = 2 * (B * H * N * C * Dk * 2) + B * H * N * C * C * 2 + B * H * N * Dk * 4
    states = B * H * N * Dk * Dv * 2
    assert lib.gla_saved_bytes(B, H, L, Dk, Dv, C, 1) == ops + states
    assert lib.gla_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, C, 1) == states
    assert lib.gla_saved_bytes(1, 1, 64, 16, 16, 48, 1) == 0          # unsupported C
    assert lib.gla_saved_bytes(1, 1, 64, 256, 64, 128, 1) > 0         # runs at C = 64
    q, k, v, g, o = (ctypes.c_void_p(0x10000000 + i * 0x1000000) for i in range(5))
    need = lib.gla_saved_bytes(1, 1, 64, 16, 16, 16, 1)
    assert lib.gla_fwd_save(q, k, v, g, None, o, None, 1, 1, 64, 16, 16, 16, 1, None, 0, None, None, 0) == 5
    assert lib.gla_fwd_save(q, k, v, g, None, o, None, 1, 1, 64, 16, 16, 16, 1,
                            ctypes.c_void_p(0x30000000), need - 1, None, None, 0) == 5
    assert lib.gla_fwd_save(q, k, v, g, None, o, None, 1, 1, 64, 16, 16, 16, 1,
                            ctypes.c_void_p(0x10000000 + 256), need, None, None, 0) == 6   # saved overlaps q
    assert lib.gla_fwd_save(None, k, v, g, None, o, None, 1, 1, 64, 16, 16, 16, 1,
                            ctypes.c_void_p(0x30000000), need, None, None, 0) == 1
    ev = (ctypes.c_void_p * 2)()
    assert lib.gla_fwd_save(q, k, v, g, None, o, None, 1, 1, 64, 16, 16, 16, 1,
                            ctypes.c_void_p(0x30000000), need, None, ev, 2) == 1            # too few events
    d = [ctypes.c_void_p(0x40000000 + i * 0x1000000) for i in range(5)]
    wsb = lib.gla_bwd_saved_workspace_bytes(1, 1, 64, 16, 16, 16, 1)
    args = [q, k, v, g, None, o, None, d[0], d[1], d[2], d[3], None, 1, 1, 64, 16, 16, 16, 1]
    assert lib.gla_bwd_saved(*args, ctypes.c_void_p(0x30000000), need, None, 0, None, None, 0) == 5
    assert lib.gla_bwd_saved(*args, ctypes.c_void_p(0x30000000), need, d[4], wsb - 1, None, None, 0) == 5
    assert lib.gla_bwd_saved(*args, ctypes.c_void_p(0x30000000), need,
                             ctypes.c_void_p(0x30000000 + 512), wsb, None, None, 0) == 6     # workspace in saved
    assert lib.gla_bwd_saved(*args, d[0], need, d[4], wsb, None, None, 0) == 6               # saved is dq


def test_gsa_saved_path_sizes_and_validation(lib):
    # saved = the backward's share of gsa_bwd's workspace; gsa_bwd_saved's workspace = the rest
    B, H, L, Dk, Dv, m, C = 8, 4, 2048, 128, 128, 64, 64
    sv = lib.gsa_saved_bytes(B, H, L, Dk, Dv, m, C, 1)
    gw = lib.gsa_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, m, C, 1)
    assert sv > lib.gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, C, 1) > 0
    assert sv + gw == lib.gsa_bwd_workspace_bytes(B, H, L, Dk, Dv, m, C, 1)
    assert lib.gsa_saved_bytes(1, 1, 64, 16, 16, 16, 48, 1) == 0       # unsupported C
    # chunk sizes beyond the GSA tiles run at a smaller chunk: C = 128 at 64, and the backward
    # with more than 64 slots at 32
    assert lib.gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, 128, 1) == lib.gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, 64, 1)
    assert lib.gsa_saved_bytes(B, H, L, Dk, Dv, 128, 64, 1) == lib.gsa_saved_bytes(B, H, L, Dk, Dv, 128, 32, 1) > 0
    assert lib.gsa_saved_bytes(B, H, L, Dk, Dv, 128, 128, 0) == 0        # fp32, 128 slots: no backward
    q, k, v, g, o = (ctypes.c_void_p(0x10000000 + i * 0x1000000) for i in range(5))
    need = lib.gsa_saved_bytes(1, 1, 64, 16, 16, 16, 16, 1)
    base = [q, k, v, g, None, None, o, None, None, 1, 1, 64, 16, 16, 16, 16, 1, 0]
    assert lib.gsa_fwd_save(*base, None, 0, None) == 5
    assert lib.gsa_fwd_save(*base, ctypes.c_void_p(0x30000000), need - 1, None) == 5
    assert lib.gsa_fwd_save(*base, ctypes.c_void_p(0x10000000 + 256), need, None) == 6    # saved overlaps q
    assert lib.gsa_fwd_save(*base[:-1], 9, ctypes.c_void_p(0x30000000), need, None) == 4  # bad read-out
    d = [ctypes.c_void_p(0x40000000 + i * 0x1000000) for i in range(5)]
    wsb = lib.gsa_bwd_saved_workspace_bytes(1, 1, 64, 16, 16, 16, 16, 1)
    args = [q, k, v, g, None, None, o, None, None, d[0], d[1], d[2], d[3], None, None,
            1, 1, 64, 16, 16, 16, 16, 1, 0]
    assert lib.gsa_bwd_saved(*args, None, need, d[4], wsb, None) == 1
    assert lib.gsa_bwd_saved(*args, ctypes.c_void_p(0x30000000), need - 1, d[4], wsb, None) == 5
    assert lib.gsa_bwd_saved(*args, ctypes.c_void_p(0x30000000), need, d[4], wsb - 1, None) == 5
    assert lib.gsa_bwd_saved(*args, ctypes.c_void_p(0x30000000), need,
                             ctypes.c_void_p(0x30000000 + 512), wsb, None) == 6            # workspace in saved
    assert lib.gsa_bwd_saved(*args, d[0], need, d[4], wsb, None) == 6                     # saved is dq


def test_decode_validation(lib):
    assert lib.gla_decode_step(*[None] * 6, 1, 1, 16, 16, 7, None) == 3
    assert lib.gla_decode_step(*[None] * 6, 1, 1, 16, 16, 1, None) == 1
    assert lib.gla_decode_step(*[None] * 6, 1, 1, 20, 16, 1, None) == 4
    p = [ctypes.c_void_p(0x10000000 + i * 0x1000000) for i in range(6)]
    p[5] = ctypes.c_void_p(0x10000000 + 16)             # o overlaps q
    assert lib.gla_decode_step(*p, 1, 1, 16, 16, 1, None) == 6


def test_gsa_decode_validation(lib):
    N = [None] * 7
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 16, 7, 0, None) == 3            # dtype
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 0, 1, 0, None) == 2             # m < 1
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 16, 1, 0, None) == 1            # null pointers
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 20, 1, 0, None) == 4            # m not a multiple of 16
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 272, 1, 0, None) == 4           # m > 256
    assert lib.gsa_decode_step(*N, 1, 1, 272, 16, 16, 1, 0, None) == 4           # Dk > 256
    assert lib.gsa_decode_step(*N, 1, 1, 16, 528, 16, 1, 0, None) == 4          # Dv > 512
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 16, 1, 5, None) == 4          # act not a gsa_act
    assert lib.gsa_decode_step(*N, 1, 1, 16, 16, 16, 1, -1, None) == 4
    p = [ctypes.c_void_p(0x10000000 + i * 0x1000000) for i in range(7)]
    assert lib.gsa_decode_step(*p[:6], ctypes.c_void_p(0x10000000 + 2), 1, 1, 16, 16, 16, 1, 0, None) == 4  # misaligned
    q = list(p)
    q[6] = ctypes.c_void_p(0x10000000 + 16)                                  # o overlaps q
    assert lib.gsa_decode_step(*q, 1, 1, 16, 16, 16, 1, 0, None) == 6
    q = list(p)
    q[5] = ctypes.c_void_p(0x10000000 + 0x4000000 + 512)                     # hv overlaps hk
    assert lib.gsa_decode_step(*q, 1, 1, 16, 16, 16, 1, 0, None) == 6
    q = list(p)
    q[4] = ctypes.c_void_p(0x10000000 + 0x2000000)                           # hk is v
    assert lib.gsa_decode_step(*q, 1, 1, 16, 16, 16, 1, 0, None) == 6


def test_profiled_needs_events(lib):
    assert lib.gla_fwd_profiled(*NOP, 1, 1, 64, 16, 16, 16, 1, None, 0, None, None, 0) == 1


def test_binding_fails_loudly_without_library(monkeypatch):
    import linear_recurrent_sequence_gla_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "lib_path", "/nonexistent/libgla_amd.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        m.lib()


def test_gsa_read_out_validation(lib):
    """An act outside gsa_act is rejected before the pointers are looked at; every valid act
    gets as far as the null-pointer check."""
    for act, want in ((-1, 4), (5, 4), (0, 1), (1, 1), (2, 1), (3, 1), (4, 1)):
        assert lib.gsa_fwd(*[None] * 9, 1, 1, 64, 16, 16, 16, 16, 1, act, None, 0, None) == want
        assert lib.gsa_bwd(*[None] * 15, 1, 1, 64, 16, 16, 16, 16, 1, act, None, 0, None) == want


def test_msgla_validation(lib):
    """Group arrays are checked before anything else is looked at."""
    I = lambda *xs: (ctypes.c_int * len(xs))(*xs)
    N = [None] * 8
    args = lambda n, sc, hd: (*N, 1, 4, 64, 64, 64, 64, 1, n, sc, hd, None, 0, None)
    assert lib.msgla_fwd(*args(3, I(1, 2, 4), I(2, 1, 1))) == 1                 # valid groups, null tensors
    assert lib.msgla_fwd(*args(0, I(1), I(4))) == 4                             # no group
    assert lib.msgla_fwd(*args(9, I(*[1] * 9), I(*[1] * 9))) == 4               # more than 8 groups
    assert lib.msgla_fwd(*args(2, I(1, 2), I(2, 1))) == 2                       # heads sum to 3, not 4
    assert lib.msgla_fwd(*args(2, I(1, 2), I(3, 2))) == 2                       # heads sum to 5
    assert lib.msgla_fwd(*args(2, I(0, 2), I(2, 2))) == 2                       # scale 0
    assert lib.msgla_fwd(*args(2, I(1, 70000), I(2, 2))) == 4                   # scale too large
    assert lib.msgla_fwd(*N, 1, 4, 64, 64, 64, 64, 1, 1, None, I(4), None, 0, None) == 1
    assert lib.msgla_fwd_workspace_bytes(1, 4, 64, 64, 64, 64, 1, 2, I(1, 2), I(2, 1)) == 0
    assert lib.msgla_fwd_workspace_bytes(1, 4, 64, 64, 64, 64, 1, 2, I(1, 2), I(2, 2)) > 0


def test_noalloc_validation(lib):
    """gla_fwd_noalloc validates like gla_fwd and refuses sizes beyond its fixed scratch before
    touching the device."""
    assert lib.gla_fwd_noalloc_max_workspace_bytes() == 64 << 20
    assert lib.gla_fwd_noalloc(*NOP, 1, 1, 64, 16, 16, 16, 5, None) == 3          # GLA_ERR_DTYPE
    assert lib.gla_fwd_noalloc(*NOP, 1, 1, 0, 16, 16, 16, 1, None) == 2           # GLA_ERR_SHAPE
    assert lib.gla_fwd_noalloc(*NOP, 1, 1, 64, 16, 16, 48, 1, None) == 4          # GLA_ERR_UNSUPPORTED
    # the 340M-layer batch needs a ~110 MB forward workspace
    assert lib.gla_fwd_workspace_bytes(8, 4, 2048, 128, 256, 64, 1) > (64 << 20)
    assert lib.gla_fwd_noalloc(*NOP, 8, 4, 2048, 128, 256, 64, 1, None) == 8      # GLA_ERR_SCRATCH
    assert lib.gla_status_str(8).decode().startswith("GLA_ERR_SCRATCH")
