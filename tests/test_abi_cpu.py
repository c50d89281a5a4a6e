"""The C-ABI library on the CPU: it loads, exports every symbol include/kda.h
declares, and rejects bad arguments with the documented status before any
HIP call (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_89_amd as kda
from gated_delta_rule_89_amd import _lib

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(HERE, "..", "include", "kda.h")

OK, NULL, SHAPE, DTYPE, UNSUP, SEQ, ALIAS, ALIGN, WS, HIP = range(10)
F32, BF16 = 0, 1
P = ctypes.c_void_p


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_exports_match_header():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(kda.lib, n), n


def header_enum(name):
    """{member: value} of `typedef enum name { ... }` in kda.h."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum %s\s*\{(.*?)\}" % name, src, flags=re.S).group(1)
    return {m: int(v) for m, v in re.findall(r"(KDA_[A-Z0-9_]+)\s*=\s*(\d+)", body)}


def test_binding_constants_match_header():
    variants = header_enum("kda_variant")
    assert {("KDA_VARIANT_" + k.upper()): v for k, v in _lib.VARIANTS.items()} == variants
    status = header_enum("kda_status")
    assert sorted(status.values()) == list(range(10))
    assert (OK, NULL, SHAPE, DTYPE, UNSUP, SEQ, ALIAS, ALIGN, WS, HIP) == tuple(
        status["KDA_" + n] for n in ("OK", "ERR_NULL", "ERR_SHAPE", "ERR_DTYPE", "ERR_UNSUPPORTED",
                                     "ERR_SEQLENS", "ERR_ALIAS", "ERR_ALIGN", "ERR_WORKSPACE", "ERR_HIP"))
    assert header_enum("kda_dtype") == {"KDA_F32": F32, "KDA_BF16": BF16}


def test_abi_version_and_status_strings():
    assert kda.abi_version() == 1
    for code in range(10):
        s = kda.status_str(code)
        assert isinstance(s, str) and s
    assert kda.status_str(0) == "ok"


# Fake device addresses: never dereferenced, every call below fails validation.
BASE = 0x7F0000000000
MB = 1 << 20


def addr(i, off=0):
    return P(BASE + i * 64 * MB + off)


def chunk(q=None, k=None, v=None, g=None, beta=None, h0=None, cu=None, cu_host=None,
          B=1, T=64, H=2, dk=16, dv=16, N=1, ind=F32, outd=F32, o=None, fin=None, ws=None,
          ws_bytes=0, variant=0):
    q = addr(0) if q is None else q
    k = addr(1) if k is None else k
    v = addr(2) if v is None else v
    g = addr(3) if g is None else g
    beta = addr(4) if beta is None else beta
    o = addr(5) if o is None else o
    return kda.lib.kda_chunk_fwd(q, k, v, g, beta, 0.25, h0, cu, cu_host, B, T, H, dk, dv, N,
                                 ind, outd, o, fin, ws, ws_bytes, variant, None)


def host_cu(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr, ctypes.cast(arr, P)


def test_chunk_validation():
    assert chunk(ind=7) == DTYPE
    assert chunk(outd=2) == DTYPE
    assert chunk(T=-1) == SHAPE
    assert chunk(dk=48) == UNSUP
    assert chunk(dv=256) == UNSUP
    assert chunk(variant=9) == UNSUP
    assert chunk(N=2) == SHAPE                       # N != B without cu_seqlens
    assert chunk(q=P(0)) == NULL
    assert chunk(o=P(0)) == NULL
    assert chunk(q=addr(0, 2)) == ALIGN
    assert chunk(beta=addr(4, 2)) == ALIGN
    assert chunk(fin=addr(7, 8), h0=addr(6)) == ALIGN
    # cu_seqlens: device and host copies go together; B = 1; 0 = c0 <= ... <= cN = T
    _, c = host_cu([0, 30, 64])
    assert chunk(cu=addr(8), N=2) == NULL
    assert chunk(cu_host=c, N=2) == NULL
    assert chunk(cu=addr(8), cu_host=c, N=2, B=2) == SHAPE
    keep, bad = host_cu([0, 40, 30, 64])
    assert chunk(cu=addr(8), cu_host=bad, N=3) == SEQ
    keep2, bad2 = host_cu([0, 30, 63])
    assert chunk(cu=addr(8), cu_host=bad2, N=2) == SEQ
    keep3, bad3 = host_cu([1, 30, 64])
    assert chunk(cu=addr(8), cu_host=bad3, N=2) == SEQ
    # AUTO takes the fp32 chunked kernel for these fp32 d = 16 inputs: it needs
    # the item list, checked before the aliasing
    assert chunk() == WS
    assert chunk(variant=5, ws=addr(9), ws_bytes=64) == WS
    # aliasing (the recurrent variant needs no workspace): o over q; final
    # over q; final partially over the initial state; workspace over o
    assert chunk(o=addr(0), variant=1) == ALIAS
    assert chunk(fin=addr(1), variant=1) == ALIAS
    assert chunk(h0=addr(6), fin=addr(6, 1024), variant=1) == ALIAS
    assert chunk(o=addr(7), fin=addr(7, 4096), variant=1) == ALIAS
    assert chunk(o=addr(7), ws=addr(7, 256), ws_bytes=256) == ALIAS


def test_workspace_size_rejects_bad_arguments():
    ws = kda.lib.kda_chunk_fwd_workspace_size
    assert ws(1, -1, 1, 128, 128, 1, None, BF16, 0) == 0
    assert ws(1, 64, 1, 100, 128, 1, None, BF16, 0) == 0
    assert ws(1, 64, 1, 128, 128, 1, None, 5, 0) == 0
    assert ws(1, 64, 1, 128, 128, 1, None, BF16, 7) == 0
    keep, bad = host_cu([0, 40, 30])
    assert ws(1, 30, 1, 128, 128, 2, bad, BF16, 2) == 0     # non-monotone lengths
    assert ws(2, 64, 1, 128, 128, 1, None, BF16, 0) == 0    # N != B without lengths


def test_workspace_size_grows_with_segments():
    """The segment scan needs map and staged-state space; the plain chunked
    path only an item list; the recurrent path nothing."""
    ws = kda.lib.kda_chunk_fwd_workspace_size
    keep, cu = host_cu([0, 100000, 100100])
    plain = ws(1, 100100, 4, 128, 128, 2, cu, BF16, 2)
    scan = ws(1, 100100, 4, 128, 128, 2, cu, BF16, 3)
    assert 0 < plain < 4096 and scan > 4 * 128 * 128 * 4
    assert ws(1, 100100, 4, 128, 128, 2, cu, BF16, 1) == 0
    assert ws(1, 100100, 4, 128, 128, 2, cu, BF16, 4) == plain     # CHUNK64: item list only
    assert ws(1, 100100, 4, 128, 128, 2, cu, BF16, 5) == plain     # CHUNK8: item list only
    assert ws(1, 100100, 4, 16, 64, 2, cu, F32, 0) == plain        # AUTO on fp32: CHUNK8


def decode(q=None, k=None, v=None, g=None, beta=None, state=None, N=4, H=2, dk=16, dv=16,
           ind=F32, outd=F32, o=None):
    q = addr(0) if q is None else q
    k = addr(1) if k is None else k
    v = addr(2) if v is None else v
    g = addr(3) if g is None else g
    beta = addr(4) if beta is None else beta
    state = addr(5) if state is None else state
    o = addr(6) if o is None else o
    return kda.lib.kda_decode_step(q, k, v, g, beta, 0.25, state, N, H, dk, dv, ind, outd, o, None)


def test_decode_validation():
    assert decode(ind=3) == DTYPE
    assert decode(N=-1) == SHAPE
    assert decode(dk=7) == UNSUP
    assert decode(state=P(0)) == NULL
    assert decode(g=P(0)) == NULL
    assert decode(q=addr(0, 4)) == ALIGN
    assert decode(o=addr(5)) == ALIAS                 # o over the state
    assert decode(state=addr(2)) == ALIAS             # state over v
    assert decode(N=0) == OK                          # no-op, nothing launched


def steps(q=None, k=None, v=None, g=None, beta=None, state=None, N=4, T=5, H=2, dk=16, dv=16,
          ind=F32, outd=F32, o=None):
    q = addr(0) if q is None else q
    k = addr(1) if k is None else k
    v = addr(2) if v is None else v
    g = addr(3) if g is None else g
    beta = addr(4) if beta is None else beta
    state = addr(5) if state is None else state
    o = addr(6) if o is None else o
    return kda.lib.kda_fused_recurrent_fwd(q, k, v, g, beta, 0.25, state, N, T, H, dk, dv,
                                           ind, outd, o, None)


def test_fused_recurrent_validation():
    assert steps(outd=9) == DTYPE
    assert steps(T=-1) == SHAPE
    assert steps(dv=24) == UNSUP
    assert steps(T=_lib.FUSED_RECURRENT_MAX_T + 1) == UNSUP   # long runs belong to kda_chunk_fwd
    assert steps(beta=P(0)) == NULL
    assert steps(v=addr(2, 8)) == ALIGN
    assert steps(beta=addr(4, 1)) == ALIGN
    # o spans N*T*H*dv*4 bytes: one ending inside q's range overlaps it
    assert steps(o=addr(0, 64)) == ALIAS
    assert steps(state=addr(6, 4 * 5 * 2 * 16 * 4 - 16)) == ALIAS   # state starts inside o
    assert steps(T=0) == OK and steps(N=0) == OK                      # no-ops


def chunk_snap(interval=64, snaps=None, T=128, B=1, N=1, H=2, dk=16, dv=16, o=None, fin=None,
               ws=None, ws_bytes=0, variant=1):
    snaps = addr(9) if snaps is None else snaps
    o = addr(5) if o is None else o
    return kda.lib.kda_chunk_fwd_snapshots(addr(0), addr(1), addr(2), addr(3), addr(4), 0.25, None,
                                           None, None, B, T, H, dk, dv, N, F32, F32, o, fin,
                                           interval, snaps, ws, ws_bytes, variant, None)


def test_snapshot_validation():
    assert chunk_snap(interval=0) == SHAPE
    assert chunk_snap(interval=-64) == SHAPE
    assert chunk_snap(interval=96) == UNSUP            # not a multiple of 64
    assert chunk_snap(snaps=P(0)) == NULL              # two snapshots requested, no buffer
    assert chunk_snap(snaps=addr(9, 4)) == ALIGN
    assert chunk_snap(snaps=addr(0, 256), ws=addr(10), ws_bytes=4096) == ALIAS    # over q
    assert chunk_snap(snaps=addr(5, 1024), ws=addr(10), ws_bytes=4096) == ALIAS   # over o
    assert chunk_snap(snaps=addr(10, 512), ws=addr(10), ws_bytes=4096) == ALIAS   # over the workspace
    # the recurrent variant needs no workspace of its own; snapshots need the row table
    assert chunk_snap() == WS
    wsz = kda.lib.kda_chunk_fwd_snapshots_workspace_size
    assert wsz(1, 128, 2, 16, 16, 1, None, F32, 1, 64) == 256
    assert wsz(1, 63, 2, 16, 16, 1, None, F32, 1, 64) == 0      # shorter than the interval
    assert wsz(1, 128, 2, 16, 16, 1, None, F32, 1, 100) == 0    # rejected interval
    keep, cu = host_cu([0, 100000, 100100])
    plain = kda.lib.kda_chunk_fwd_workspace_size(1, 100100, 4, 128, 128, 2, cu, BF16, 3)
    assert wsz(1, 100100, 4, 128, 128, 2, cu, BF16, 3, 4096) == ((plain + 255) // 256) * 256 + 256


def chunk_gated(gate=None, weight=None, eps=1e-6, o=None, ws=None, ws_bytes=0, variant=1,
                T=64, H=2, dk=16, dv=16):
    gate = addr(11) if gate is None else gate
    weight = addr(12) if weight is None else weight
    o = addr(5) if o is None else o
    return kda.lib.kda_chunk_fwd_gated(addr(0), addr(1), addr(2), addr(3), addr(4), 0.25, None, None,
                                       None, 1, T, H, dk, dv, 1, F32, F32, gate, weight, eps, o,
                                       None, ws, ws_bytes, variant, None)


def test_gated_validation():
    assert chunk_gated(gate=P(0)) == NULL
    assert chunk_gated(weight=P(0)) == NULL
    assert chunk_gated(eps=-1e-6) == SHAPE
    assert chunk_gated(eps=float("nan")) == SHAPE
    assert chunk_gated(eps=float("inf")) == SHAPE
    assert chunk_gated(gate=addr(11, 4)) == ALIGN
    assert chunk_gated(weight=addr(12, 8)) == ALIGN
    assert chunk_gated(gate=addr(5, 64)) == ALIAS      # the gate inside o
    assert chunk_gated(weight=addr(5, 128)) == ALIAS   # the weight inside o
    assert chunk_gated(T=0) == OK                      # no token: nothing to do


def fgate(z=None, w=None, b=None, u=None, M=100, r=128, H=2, dk=128, ind=BF16, g=None, beta=None):
    z = addr(0) if z is None else z
    w = addr(1) if w is None else w
    u = addr(2) if u is None else u
    g = addr(3) if g is None else g
    beta = addr(4) if beta is None else beta
    return kda.lib.kda_fused_gate(z, w, b, u, M, r, H, dk, ind, g, beta, None)


def test_fused_gate_validation():
    assert fgate(ind=5) == DTYPE
    assert fgate(M=-1) == SHAPE and fgate(H=65536) == SHAPE
    assert fgate(ind=F32) == UNSUP and fgate(dk=64) == UNSUP and fgate(r=100) == UNSUP
    assert fgate(u=P(0)) == NULL and fgate(g=P(0)) == NULL
    assert fgate(b=P(BASE + 2)) == ALIGN and fgate(w=addr(1, 8)) == ALIGN
    assert fgate(g=addr(0, 512)) == ALIAS                 # g over z
    assert fgate(beta=addr(3, 1024)) == ALIAS             # beta inside g
    assert fgate(M=0) == OK


def test_noalloc_rejects_workspace_beyond_its_array():
    """kda_chunk_fwd_noalloc checks the workspace size on the host before any
    HIP call: an explicit segment scan over one long sequence needs more than
    the library's array and is refused (fake pointers, nothing launched)."""
    T, H = 1 << 20, 32
    need = kda.workspace_size(1, T, H, 128, 128, 1, variant="chunk_scan")
    assert need > _lib.NOALLOC_MAX_WORKSPACE
    rc = kda.lib.kda_chunk_fwd_noalloc(addr(0), addr(1), addr(2), addr(3), addr(4), 0.1, None, None,
                                       None, 1, T, H, 128, 128, 1, BF16, F32, addr(5), addr(6),
                                       3, None)
    assert rc == WS
