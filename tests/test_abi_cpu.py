"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

from linear_attention_sequence_03_amd import gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gdr.LIBRARY_PATH),
                                reason="libgdr.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(gdr.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(gdr.LIBRARY_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    assert gdr.gdr_status_string(0) == "GDR_OK"
    assert gdr.gdr_status_string(1) == "GDR_ERR_INVALID_ARG"
    assert gdr.gdr_status_string(2) == "GDR_ERR_UNSUPPORTED"
    assert gdr.gdr_status_string(3) == "GDR_ERR_HIP"
    assert gdr.gdr_status_string(99) == "GDR_UNKNOWN_STATUS"


# ----- raw calls with fake (never dereferenced) device addresses -------------
BASE = 1 << 40
MB = 1 << 24


def _addr(i):
    return ctypes.c_void_p(BASE + i * MB)


def _chunk(lib, q=0, k=1, v=2, la=3, be=4, s0=None, o=6, st=7, ws=8, B=1, T=128, H=2, dk=64,
           dv=64, chunk=64, io=0, gate=0, wsbytes=1 << 22):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_chunk_fwd(p(q), p(k), p(v), p(la), p(be), p(s0), p(o), p(st),
                             B, T, H, dk, dv, chunk, io, gate, p(ws), wsbytes, None)


def _chunk_noalloc(lib, q=0, k=1, v=2, la=3, be=4, o=6, st=7, B=1, T=128, H=2, dk=64, dv=64,
                   chunk=64, io=0, gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_chunk_fwd_noalloc(p(q), p(k), p(v), p(la), p(be), None, p(o), p(st),
                                     B, T, H, dk, dv, chunk, io, gate, None)


def _decode(lib, q=0, k=1, v=2, la=3, be=4, si=5, so=6, o=7, B=2, H=2, dk=64, dv=64, io=0,
            gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_decode_step(p(q), p(k), p(v), p(la), p(be), p(si), p(so), p(o),
                               B, H, dk, dv, io, gate, None)


@pytest.fixture(scope="module")
def lib():
    return gdr.load_library()


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(la=None), 1), (dict(ws=None), 1),
    (dict(B=0), 1), (dict(H=-1), 1), (dict(T=-1), 1), (dict(dk=0), 1),
    (dict(dk=96, dv=96), 2), (dict(dk=64, dv=128), 2), (dict(dk=256, dv=256), 2),
    (dict(chunk=48), 2), (dict(chunk=128), 2), (dict(chunk=0), 1),
    (dict(io=7), 1), (dict(gate=5), 1), (dict(wsbytes=16), 1),
    (dict(q=ctypes.c_void_p(BASE + 8)), 1),            # misaligned
    (dict(o=ctypes.c_void_p(BASE + 4 * 1024)), 1),      # o inside q
    (dict(st=ctypes.c_void_p(BASE + 3 * MB + 64)), 1),  # S_T inside log_alpha
    (dict(ws=ctypes.c_void_p(BASE + 6 * MB + 256)), 1), # workspace inside o
    # a chunk's row offsets would pass 2^31 bytes: refused before any launch
    (dict(H=70000, dk=128, dv=128, io=1, T=64), 2),
    (dict(H=140000, dk=64, dv=64, io=0, T=64, wsbytes=1 << 62), 2),
])
def test_chunk_fwd_rejects(lib, kw, code):
    assert _chunk(lib, **kw) == code
    assert lib.gdr_last_error()  # a message was left


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(B=0), 1), (dict(chunk=48), 2), (dict(dk=96, dv=96), 2),
    (dict(o=ctypes.c_void_p(BASE + 4 * 1024)), 1),      # o inside q
    # workspace beyond the fixed scratch: KDA bf16 d = 128, 1024 chunk blocks of
    # 74496 bytes (76.3 MB > 64 MiB); refused before the scratch is looked up
    (dict(B=1, T=4096, H=16, dk=128, dv=128, io=1, gate=1), 2),
    # fp32 scalar d = 64, chunk 64: 2048 blocks, far past the scratch
    (dict(B=8, T=16384, H=16), 2),
])
def test_chunk_fwd_noalloc_rejects(lib, kw, code):
    assert _chunk_noalloc(lib, **kw) == code
    assert lib.gdr_last_error()


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GDR_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdr.GDR_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(si=None), 1), (dict(so=None), 1), (dict(o=None), 1),
    (dict(B=0), 1), (dict(dk=32, dv=32), 2), (dict(dk=128, dv=64), 2), (dict(io=2), 1),
    (dict(so=ctypes.c_void_p(BASE + 5 * MB + 1024)), 1),   # partial overlap with S_in
    (dict(o=ctypes.c_void_p(BASE + 6 * MB + 64)), 1),      # o inside S_out
    (dict(v=ctypes.c_void_p(BASE + 2 * MB + 4)), 1),       # misaligned
])
def test_decode_step_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def _chunk_pro(lib, flags, q=0, k=1, v=2, la=3, be=4, o=6, st=7, ws=8, B=1, T=128, H=2, dk=64,
               dv=64, chunk=64, io=1, gate=0, wsbytes=1 << 22):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_chunk_fwd_prologue(p(q), p(k), p(v), p(la), p(be), None, p(o), p(st),
                                      B, T, H, dk, dv, chunk, io, gate, p(ws), wsbytes, flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(flags=8), 1), (dict(flags=1 << 31), 1),              # unknown flags
    # staged calls (fp32 io, scalar chunk 16 / 32) need the prologue workspace
    (dict(flags=1, io=0, wsbytes=4096), 1), (dict(flags=7, chunk=32, wsbytes=4096), 1),
    (dict(flags=4, chunk=16, ws=None), 1),
    (dict(flags=1, q=None), 1),                                 # the plain checks still run
])
def test_chunk_fwd_prologue_rejects(lib, kw, code):
    assert _chunk_pro(lib, **kw) == code
    assert lib.gdr_last_error()


def test_prologue_workspace_size():
    F32, BF16, SC, CH = gdr.GDR_F32, gdr.GDR_BF16, gdr.GDR_GATE_SCALAR, gdr.GDR_GATE_CHANNEL
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, T, H, d = 2, 100, 3, 64
    rows = B * T * H
    # fused calls: the plain size whatever the flags
    for io, gate, c in ((BF16, SC, 64), (BF16, CH, 16), (BF16, CH, 64)):
        plain = gdr.gdr_chunk_fwd_workspace_size(B, T, H, d, d, c, io, gate)
        for f in (0, 1, 2, 4, 7):
            assert gdr.gdr_chunk_fwd_prologue_workspace_size(B, T, H, d, d, c, io, gate, f) == plain
    # staged calls: plain + the mapped tensors, each 256-byte aligned
    for io, gate, c, es in ((F32, SC, 64, 4), (F32, CH, 32, 4), (BF16, SC, 16, 2)):
        plain = gdr.gdr_chunk_fwd_workspace_size(B, T, H, d, d, c, io, gate)
        la = rows * (d if gate == CH else 1) * 4
        want = {0: plain, 1: al(plain) + 2 * al(rows * d * es), 2: al(plain) + al(rows * 4),
                4: al(plain) + al(la), 7: al(plain) + 2 * al(rows * d * es) + al(rows * 4) + al(la)}
        for f, w in want.items():
            assert gdr.gdr_chunk_fwd_prologue_workspace_size(B, T, H, d, d, c, io, gate, f) == w, (io, c, f)
    with pytest.raises(gdr.GdrError):
        gdr.gdr_chunk_fwd_prologue_workspace_size(B, T, H, d, d, 64, F32, SC, 8)
    # T = 0 stages nothing
    assert gdr.gdr_chunk_fwd_prologue_workspace_size(B, 0, H, d, d, 64, F32, SC, 7) == 0


def test_decode_step_prologue_rejects(lib):
    p = _addr
    args = [p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), 2, 2, 64, 64, 0, 0]
    assert lib.gdr_decode_step_prologue(*args, 8, None) == 1        # unknown flag
    args[0] = None
    assert lib.gdr_decode_step_prologue(*args, 1, None) == 1        # plain checks still run


def test_workspace_size():
    # bf16 scalar gate with 64-token chunks runs as one kernel: no workspace
    for d in (64, 128):
        assert gdr.gdr_chunk_fwd_workspace_size(4, 4096, 16, d, d, 64, gdr.GDR_BF16,
                                                gdr.GDR_GATE_SCALAR) == 0
    # two-kernel path, per (b,h,chunk): scalar gate = T + P (C*C each) + two
    # decay vectors (2C floats), 256-aligned; bf16 adds a 16-byte flag slot
    # and the residual of T (C*C)
    n = gdr.gdr_chunk_fwd_workspace_size(4, 4096, 16, 128, 128, 32, gdr.GDR_BF16,
                                         gdr.GDR_GATE_SCALAR)
    blk = (2 * 32 * 32 * 2 + 2 * 32 * 4 + 16 + 32 * 32 * 2 + 255) // 256 * 256
    assert n == 4 * 16 * 128 * blk
    n = gdr.gdr_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, gdr.GDR_BF16, gdr.GDR_GATE_CHANNEL)
    assert n == (2 * 64 * 64 * 2 + 3 * 64 * 128 * 2 + 128 * 4 + 16 + 64 * 64 * 2 + 255) // 256 * 256
    # channel gate: three gate-scaled [C, dk] operands and dk floats instead
    n = gdr.gdr_chunk_fwd_workspace_size(1, 100, 1, 64, 64, 32, gdr.GDR_F32,
                                         gdr.GDR_GATE_CHANNEL)
    blk = (2 * 32 * 32 * 4 + 3 * 32 * 64 * 4 + 64 * 4 + 255) // 256 * 256
    assert n == 4 * blk
    assert gdr.gdr_chunk_fwd_workspace_size(1, 0, 1, 64, 64, 16, 0, 0) == 0
    with pytest.raises(gdr.GdrError) as e:
        gdr.gdr_chunk_fwd_workspace_size(1, 10, 1, 96, 96, 16, 0, 0)
    assert e.value.status == gdr.GDR_ERR_UNSUPPORTED


def test_binding_type_checks_before_calling():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(TypeError):
        gdr.gdr_chunk_fwd(q.double(), q, q, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1))
    with pytest.raises(ValueError):
        gdr.gdr_chunk_fwd(q, q, q, torch.zeros(1, 4, 2), torch.zeros(1, 4, 1))
    # the tree commit takes its sizes from k, which must be contiguous like every other tensor
    kt = torch.zeros(1, 4, 1, 128)[..., ::2]
    with pytest.raises(ValueError, match="k must be contiguous"):
        gdr.gdr_decode_tree_commit(kt, torch.zeros(1, 4, 1), torch.zeros(1, 4, dtype=torch.int32),
                                   torch.zeros(1, 4, 1, 64), torch.zeros(1, dtype=torch.int32),
                                   torch.zeros(1, 1, 64, 64))


# ----- channel-wise write rates (FG2) ----------------------------------------
def _fg2_chunk(lib, q=0, k=1, v=2, la=3, bk=4, bv=None, s0=None, o=6, st=7, ws=8, B=1, T=128, H=2,
               dk=64, dv=64, chunk=64, io=0, gate=1, wsbytes=1 << 23):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_fg2_chunk_fwd(p(q), p(k), p(v), p(la), p(bk), p(bv), p(s0), p(o), p(st),
                                 B, T, H, dk, dv, chunk, io, gate, p(ws), wsbytes, None)


def _fg2_decode(lib, q=0, k=1, v=2, la=3, bk=4, bv=None, si=5, so=6, o=7, B=2, H=2, dk=64, dv=64,
                io=0, gate=1):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_fg2_decode_step(p(q), p(k), p(v), p(la), p(bk), p(bv), p(si), p(so), p(o),
                                   B, H, dk, dv, io, gate, None)


@pytest.mark.parametrize("kw,code", [
    (dict(bk=None), 1), (dict(q=None), 1), (dict(ws=None), 1), (dict(wsbytes=1024), 1),
    (dict(dk=64, dv=128), 2), (dict(chunk=8), 2), (dict(gate=3), 1),
    (dict(bk=ctypes.c_void_p(BASE + 4 * MB + 4)), 1),     # misaligned
    (dict(o=ctypes.c_void_p(BASE + 4 * MB + 4096)), 1),   # o inside beta_k
    (dict(bv=ctypes.c_void_p(BASE + 6 * MB)), 1),         # beta_v is o
    (dict(H=70000, dk=128, dv=128, T=64, wsbytes=1 << 62), 2),   # row offsets past 2^31 bytes
])
def test_fg2_chunk_fwd_rejects(lib, kw, code):
    assert _fg2_chunk(lib, **kw) == code
    assert lib.gdr_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(bk=None), 1), (dict(so=None), 1), (dict(dk=128, dv=64), 2),
    (dict(o=ctypes.c_void_p(BASE + 4 * MB)), 1),          # o is beta_k
    (dict(bv=ctypes.c_void_p(BASE + 9 * MB + 8)), 1),     # misaligned beta_v
])
def test_fg2_decode_step_rejects(lib, kw, code):
    assert _fg2_decode(lib, **kw) == code


def test_fg2_workspace_size():
    """The FG2 workspace is the chunk path's plus the scaled k and v of the
    whole call and one unit rate per token, each 256-byte aligned."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for io, es in ((gdr.GDR_F32, 4), (gdr.GDR_BF16, 2)):
        for gate in (gdr.GDR_GATE_SCALAR, gdr.GDR_GATE_CHANNEL):
            B, T, H, d, C = 2, 100, 3, 64, 32
            inner = gdr.gdr_chunk_fwd_workspace_size(B, T, H, d, d, C, io, gate)
            ntok = B * T * H
            want = al(inner) + 2 * al(ntok * d * es) + al(ntok * 4)
            assert gdr.gdr_fg2_chunk_fwd_workspace_size(B, T, H, d, d, C, io, gate) == want
    assert gdr.gdr_fg2_chunk_fwd_workspace_size(1, 0, 1, 64, 64, 16, 0, 1) == 0


# ----- several tokens per call ------------------------------------------------
def _multi(lib, q=0, k=1, v=2, la=3, be=4, si=5, so=6, acc=9, o=7, B=2, Td=4, H=2, dk=64, dv=64,
           io=0, gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_decode_multi(p(q), p(k), p(v), p(la), p(be), p(si), p(so), p(acc), p(o),
                                B, Td, H, dk, dv, io, gate, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(si=None), 1), (dict(Td=0), 2), (dict(Td=65), 2),
    (dict(dk=128, dv=64), 2), (dict(gate=4), 1),
    (dict(acc=ctypes.c_void_p(BASE + 9 * MB + 2)), 1),     # misaligned accepted
    (dict(so=ctypes.c_void_p(BASE + 5 * MB + 4096)), 1),   # partial overlap with S_in
    (dict(o=ctypes.c_void_p(BASE + 9 * MB)), 1),           # o is accepted
    (dict(o=ctypes.c_void_p(BASE + 1 * MB)), 1),           # o is k
])
def test_decode_multi_rejects(lib, kw, code):
    assert _multi(lib, **kw) == code
    assert lib.gdr_last_error()


def test_decode_multi_nothing_requested_is_ok(lib):
    assert _multi(lib, so=None, o=None) == 0


# ----- decoupled erase / write gates -----------------------------------------
def _gdn2(lib, q=0, k=1, v=2, la=3, eb=4, ww=5, s0=None, o=6, st=7, B=1, T=64, H=2, dk=64, dv=64,
          io=0, gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_gdn2_fwd(p(q), p(k), p(v), p(la), p(eb), p(ww), p(s0), p(o), p(st),
                            B, T, H, dk, dv, io, gate, None)


@pytest.mark.parametrize("kw,code", [
    (dict(eb=None), 1), (dict(ww=None), 1), (dict(o=None), 1), (dict(T=-1), 1),
    (dict(dk=64, dv=128), 2), (dict(io=5), 1),
    (dict(ww=ctypes.c_void_p(BASE + 5 * MB + 8)), 1),     # misaligned
    (dict(o=ctypes.c_void_p(BASE + 4 * MB + 1024)), 1),   # o inside erase
])
def test_gdn2_rejects(lib, kw, code):
    assert _gdn2(lib, **kw) == code
    assert lib.gdr_last_error()


def _gdn2c(lib, q=0, k=1, v=2, la=3, eb=4, ww=5, s0=None, o=6, st=7, ws=8, wsb=1 << 24, B=1, T=64,
           H=2, dk=64, dv=64, chunk=64, io=1, gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_gdn2_chunk_fwd(p(q), p(k), p(v), p(la), p(eb), p(ww), p(s0), p(o), p(st),
                                  B, T, H, dk, dv, chunk, io, gate, p(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(eb=None), 1), (dict(ww=None), 1), (dict(o=None), 1), (dict(T=-1), 1),
    (dict(io=0), 2), (dict(chunk=32), 2), (dict(chunk=0), 1), (dict(dk=64, dv=128), 2),
    (dict(ws=None), 1), (dict(wsb=100), 1),
    (dict(ww=ctypes.c_void_p(BASE + 5 * MB + 8)), 1),     # misaligned
    (dict(o=ctypes.c_void_p(BASE + 4 * MB + 1024)), 1),   # o inside erase
    (dict(ws=ctypes.c_void_p(BASE + 6 * MB)), 1),         # workspace over o
])
def test_gdn2_chunk_rejects(lib, kw, code):
    assert _gdn2c(lib, **kw) == code
    assert lib.gdr_last_error()


def test_gdn2_chunk_workspace_size():
    """One block per (b, h, 64-token chunk): four bf16 [64][d] tiles, one bf16
    [64][64] tile and d fp32 decay factors, rounded up to 256 bytes."""
    for d in (64, 128):
        blk = -(-(4 * 64 * d * 2 + 64 * 64 * 2 + 4 * d) // 256) * 256
        for B, T, H in [(1, 1, 1), (2, 130, 3), (2, 8192, 32)]:
            want = B * H * (-(-T // 64)) * blk
            assert gdr.gdr_gdn2_chunk_fwd_workspace_size(B, T, H, d, d, 64, 1, 1) == want
    assert gdr.gdr_gdn2_chunk_fwd_workspace_size(1, 0, 1, 64, 64, 64, 1, 0) == 0
    with pytest.raises(gdr.GdrError):
        gdr.gdr_gdn2_chunk_fwd_workspace_size(1, 64, 1, 64, 64, 64, 0, 0)   # fp32 io


def _tree(lib, q=0, k=1, v=2, la=3, be=4, si=5, par=6, o=7, D=8, B=2, Td=5, H=2, dk=64, dv=64, io=0, gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_decode_tree(p(q), p(k), p(v), p(la), p(be), p(si), p(par), p(o), p(D),
                               B, Td, H, dk, dv, io, gate, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Td=0), 2), (dict(Td=65), 2), (dict(q=None), 1), (dict(par=None), 1), (dict(si=None), 1),
    (dict(dk=96, dv=96), 2), (dict(io=3), 1),
    (dict(par=ctypes.c_void_p(BASE + 6 * MB + 2)), 1),     # parent not 4-byte aligned
    (dict(o=ctypes.c_void_p(BASE + 1024)), 1),              # o inside q
    (dict(D=ctypes.c_void_p(BASE + 6 * MB + 16)), 1),       # D overlaps parent
    (dict(o=ctypes.c_void_p(BASE + 7 * MB + 8)), 1),        # o misaligned
])
def test_decode_tree_rejects(lib, kw, code):
    assert _tree(lib, **kw) == code
    assert lib.gdr_last_error()


def test_decode_tree_nothing_requested_is_ok(lib):
    assert _tree(lib, o=None, D=None) == 0


def _tree_commit(lib, k=1, la=3, par=6, D=8, acc=9, si=5, so=10, B=2, Td=5, H=2, dk=64, dv=64, io=0,
                 gate=0):
    p = lambda i: None if i is None else (_addr(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_decode_tree_commit(p(k), p(la), p(par), p(D), p(acc), p(si), p(so),
                                      B, Td, H, dk, dv, io, gate, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Td=65), 2), (dict(acc=None), 1), (dict(D=None), 1), (dict(so=None), 1),
    (dict(so=ctypes.c_void_p(BASE + 5 * MB + 4096)), 1),    # S_out partially overlaps S_in
    (dict(so=ctypes.c_void_p(BASE + 8 * MB)), 1),           # S_out is D
    (dict(acc=ctypes.c_void_p(BASE + 9 * MB + 1)), 1),      # accepted misaligned
])
def test_decode_tree_commit_rejects(lib, kw, code):
    assert _tree_commit(lib, **kw) == code
    assert lib.gdr_last_error()
