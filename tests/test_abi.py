"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, sizes workspaces, and rejects bad arguments on the host
before any HIP call (each call below fails validation, so nothing launches)."""
import ctypes

import pytest

from kv_cached_decode_amd import binding as kb

FAKE = 0x10000        # 16-byte aligned non-null stand-in; never dereferenced
MIS = 0x10008         # misaligned stand-in


@pytest.fixture(scope="module")
def lib():
    return kb.lib()


def test_header_declares_the_five_calls_and_helpers():
    names = kb.declared_functions()
    for n in ("kv_append", "kv_reorder", "decode_attn_self", "decode_step_self", "decode_attn_cross",
              "verify_accept", "kvd_attn_workspace_bytes", "kvd_verify_workspace_bytes",
              "kvd_status_string"):
        assert n in names
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol(lib):
    for n in kb.declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(-9, 1):
        s = kb.status_string(code)
        assert s and s != "unknown status"
    assert kb.status_string(-99) == "unknown status"


def _cache(B=1, H=20, S=448, D=64, dtype=kb.F16, k=FAKE, v=FAKE):
    return kb.KvdCache(k, v, B, H, S, D, dtype)


def test_kv_append_validation(lib):
    c = _cache()
    f = lib.kv_append
    assert f(None, FAKE, FAKE, 0, 1, 0.0, None) == -1
    assert f(ctypes.byref(_cache(k=None)), FAKE, FAKE, 0, 1, 0.0, None) == -1
    assert f(ctypes.byref(c), None, FAKE, 0, 1, 0.0, None) == -1
    assert f(ctypes.byref(_cache(dtype=7)), FAKE, FAKE, 0, 1, 0.0, None) == -3
    assert f(ctypes.byref(_cache(D=128)), FAKE, FAKE, 0, 1, 0.0, None) == -2
    assert f(ctypes.byref(c), FAKE, FAKE, 0, 0, 0.0, None) == -2          # T < 1
    assert f(ctypes.byref(c), FAKE, FAKE, -1, 1, 0.0, None) == -2         # pos < 0
    assert f(ctypes.byref(c), FAKE, FAKE, 0, 1, -1.0, None) == -2         # rope base < 0
    assert f(ctypes.byref(c), FAKE, FAKE, 448, 1, 0.0, None) == -4        # capacity
    assert f(ctypes.byref(c), FAKE, FAKE, 440, 9, 0.0, None) == -4
    assert f(ctypes.byref(c), MIS, FAKE, 0, 1, 0.0, None) == -7
    assert f(ctypes.byref(_cache(k=MIS)), FAKE, FAKE, 0, 1, 0.0, None) == -7


def test_beam_step_validation(lib):
    big = 1 << 30
    src = _cache(B=5)
    dst = _cache(B=5, k=0x1000000, v=0x2000000)   # storage 5*20*448*128 B = 5.7 MB apart
    far = _cache(B=5, k=0x4000000, v=0x5000000)
    f = lib.decode_step_self_beams

    def call(q=FAKE, kn=FAKE, vn=FAKE, Hq=20, N=1, s=src, d=dst, par=FAKE, L=100, ws_bytes=big,
             st=None):
        return f(q, kn, vn, Hq, N, ctypes.byref(s), ctypes.byref(d), par, L, 0.125, 0.0, FAKE,
                 FAKE, ws_bytes, st, None)
    assert f(FAKE, FAKE, FAKE, 20, 1, None, ctypes.byref(dst), FAKE, 100, 0.125, 0.0, FAKE, FAKE,
             big, None, None) == -1
    assert call(par=None) == -1
    assert call(kn=None) == -1
    assert call(q=None) == -1
    assert call(d=_cache(B=5, k=0x1000000, v=0x2000000, dtype=kb.BF16)) == -3   # dtypes differ
    assert call(d=_cache(B=4, k=0x1000000, v=0x2000000)) == -2                 # B differs
    assert call(d=_cache(B=5, S=447, k=0x1000000, v=0x2000000)) == -2          # S_max differs
    assert call(N=17) == -2
    assert call(d=src) == -2                                                   # same storage
    assert call(s=dst, d=_cache(B=5, k=0x1000000 + 5 * 20 * 448 * 128 - 16, v=0x6000000)) == -2
    assert call(s=far, d=_cache(B=5, k=0x6000000, v=0x4000000 + 4096)) == -2  # dst.v inside src.k
    assert call(par=FAKE + 2) == -7
    assert call(st=FAKE + 1) == -7
    assert call(L=0) == -4
    assert call(L=449) == -4
    assert call(N=5, L=4) == -4
    assert call(Hq=21) == -2
    assert call(L=448, ws_bytes=0) == -6      # 5 x 20 heads of 448 rows: split keys


def test_ragged_validation(lib):
    c = ctypes.byref(_cache(B=4))
    big = 1 << 30
    a = lib.kv_append_ragged
    assert a(c, FAKE, FAKE, None, 5, 0.0, None, None) == -1
    assert a(c, FAKE, FAKE, FAKE, 0, 0.0, None, None) == -2              # T < 1
    assert a(c, FAKE, FAKE, FAKE, 449, 0.0, None, None) == -4            # T > S_max
    assert a(c, FAKE, FAKE, FAKE + 2, 5, 0.0, None, None) == -7          # pos misaligned
    assert a(c, FAKE, FAKE, FAKE, 5, 0.0, FAKE + 1, None) == -7          # dev_status misaligned
    s = lib.decode_attn_self_ragged
    assert s(FAKE, 20, 5, c, None, 448, 0.125, 0.0, FAKE, FAKE, big, None, None) == -1
    assert s(FAKE, 20, 5, c, FAKE, 449, 0.125, 0.0, FAKE, FAKE, big, None, None) == -4
    assert s(FAKE, 20, 5, c, FAKE, 4, 0.125, 0.0, FAKE, FAKE, big, None, None) == -4
    assert s(FAKE, 20, 5, c, FAKE + 2, 448, 0.125, 0.0, FAKE, FAKE, big, None, None) == -7
    assert s(FAKE, 20, 5, c, FAKE, 448, 0.125, 0.0, FAKE, FAKE, big, FAKE + 2, None) == -7
    t = lib.decode_step_self_ragged
    assert t(FAKE, FAKE, None, 20, 5, c, FAKE, 448, 0.125, 0.0, FAKE, FAKE, big, None, None) == -1
    assert t(FAKE, FAKE, FAKE, 20, 5, c, None, 448, 0.125, 0.0, FAKE, FAKE, big, None, None) == -1
    assert t(FAKE, FAKE, FAKE, 20, 17, c, FAKE, 448, 0.125, 0.0, FAKE, FAKE, big, None, None) == -2
    assert t(FAKE, FAKE, FAKE, 20, 5, c, FAKE, 3, 0.125, 0.0, FAKE, FAKE, big, None, None) == -4
    assert t(FAKE, MIS, FAKE, 20, 5, c, FAKE, 448, 0.125, 0.0, FAKE, FAKE, big, None, None) == -7


def test_kv_reorder_validation(lib):
    f = lib.kv_reorder
    assert f(ctypes.byref(_cache(B=5)), None, 10, None, None) == -1
    assert f(ctypes.byref(_cache(B=17)), FAKE, 10, None, None) == -2      # too many beams
    assert f(ctypes.byref(_cache(B=5)), FAKE, -1, None, None) == -2
    assert f(ctypes.byref(_cache(B=5)), FAKE, 449, None, None) == -4
    assert f(ctypes.byref(_cache(B=5)), FAKE + 2, 10, None, None) == -7


def test_decode_attn_validation(lib):
    c = _cache()
    ws = FAKE
    s = lib.decode_attn_self
    assert s(None, 20, 1, ctypes.byref(c), 10, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -1
    assert s(FAKE, 20, 1, ctypes.byref(c), 10, 0.125, 0.0, None, ws, 1 << 30, None) == -1
    assert s(FAKE, 20, 0, ctypes.byref(c), 10, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -2
    assert s(FAKE, 30, 1, ctypes.byref(c), 10, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -2  # Hq % H
    assert s(FAKE, 20, 1, ctypes.byref(c), 449, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -4
    assert s(FAKE, 20, 5, ctypes.byref(c), 4, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -4   # len < N
    assert s(FAKE, 20, 1, ctypes.byref(c), 10, float("nan"), 0.0, FAKE, ws, 1 << 30, None) == -2
    assert s(MIS, 20, 1, ctypes.byref(c), 10, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -7
    # a long cache needs split partials: no or too small a workspace is refused
    long_c = _cache(S=1500)
    assert s(FAKE, 20, 1, ctypes.byref(long_c), 1500, 0.125, 0.0, FAKE, None, 0, None) == -6
    assert s(FAKE, 20, 1, ctypes.byref(long_c), 1500, 0.125, 0.0, FAKE, ws, 64, None) == -6
    st = lib.decode_step_self
    assert st(FAKE, None, FAKE, 20, 1, ctypes.byref(c), 10, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -1
    assert st(FAKE, FAKE, FAKE, 20, 1, ctypes.byref(c), 449, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -4
    assert st(FAKE, FAKE, MIS, 20, 1, ctypes.byref(c), 10, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -7
    assert st(FAKE, FAKE, MIS, 20, 40, ctypes.byref(c), 100, 0.125, 0.0, FAKE, ws, 1 << 30, None) == -7
    x = lib.decode_attn_cross
    xc = _cache(B=1, S=1500)
    assert x(FAKE, 5, 20, 1, ctypes.byref(xc), 1501, 0.125, FAKE, ws, 1 << 30, None) == -4
    assert x(FAKE, 5, 20, 1, ctypes.byref(_cache(B=2, S=1500)), 1500, 0.125, FAKE, ws, 1 << 30, None) == -2
    assert x(FAKE, 5, 20, 1, ctypes.byref(xc), 0, 0.125, FAKE, ws, 1 << 30, None) == -2
    assert x(FAKE, 1, 20, 1, ctypes.byref(xc), 1500, 0.125, FAKE, None, 0, None) == -6


def test_verify_accept_validation(lib):
    f = lib.verify_accept
    big = 1 << 30
    assert f(None, 0, 1, 5, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 0, 1, 5, 51865, None, 5, None, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 9, 1, 5, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 0, 1, 7, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -5
    assert f(FAKE, 0, 1, 4, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -5
    assert f(FAKE, 0, 1, 5, 0, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -2
    assert f(FAKE, 0, 1, 5, 51865, FAKE, 5, None, FAKE, FAKE, None, 0, None) == -6
    assert f(FAKE, 0, 1, 5, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, 100, None) == -6
    assert f(FAKE + 2, 0, 1, 5, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -7  # f32
    assert f(FAKE + 1, 1, 1, 5, 51865, FAKE, 5, None, FAKE, FAKE, FAKE, big, None) == -7  # f16


def test_verify_accept_masked_validation(lib):
    f = lib.verify_accept_masked
    big = 1 << 30
    ok = [FAKE, 0, 1, 5, 51865, FAKE, 5, FAKE, FAKE, None, FAKE, FAKE, FAKE, big, None]

    def call(**kw):
        args = list(ok)
        names = ["logits", "dt", "B", "R", "V", "draft", "N", "sup", "first", "am", "acc", "nxt",
                 "ws", "wsb", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)
    assert call(logits=None) == -1
    assert call(draft=None) == -1                   # drafts needed when N > 0
    assert call(draft=None, N=0, R=1, ws=None) == -6   # N = 0 takes no drafts (stops at the workspace)
    assert call(N=0, R=2) == -5 and call(N=0, R=0) == -5
    assert call(V=(1 << 20) + 1) == -2 and call(N=64, R=64) == -2
    assert call(sup=FAKE + 2) == -7 and call(first=FAKE + 1) == -7
    assert call(ws=None) == -6
    assert lib.verify_accept(FAKE, 0, 1, 5, (1 << 20) + 1, FAKE, 5, None, FAKE, FAKE, FAKE, big,
                             None) == -2


def test_workspace_sizes(lib):
    # a 1500-key cache is split, a 40-key one is not (the counter block only)
    assert kb.attn_workspace_bytes(1, 20, 1, 1500) > 16384
    assert kb.attn_workspace_bytes(1, 20, 1, 40) == 0
    assert kb.attn_workspace_bytes(1, 20, 1, 1500) >= kb.attn_workspace_bytes(1, 20, 1, 448)
    assert kb.attn_workspace_bytes(0, 20, 1, 448) == 0
    assert kb.verify_workspace_bytes(1, 5, 51865) > 16384
    assert kb.verify_workspace_bytes(1, 0, 10) == 0


def test_read_probe_validation(lib):
    f = lib.kvd_read_probe
    assert f(None, None, 16, FAKE, None) == -1
    assert f(FAKE, None, 16, None, None) == -1
    assert f(FAKE, None, 0, FAKE, None) == -2
    assert f(FAKE, None, 24, FAKE, None) == -2            # not a multiple of 16
    assert f(MIS, None, 16, FAKE, None) == -7
    assert f(FAKE, MIS, 16, FAKE, None) == -7
    assert f(FAKE, None, 16, FAKE + 2, None) == -7


def test_beam_select_validation(lib):
    f = lib.beam_select
    ws_need = kb.beam_workspace_bytes(1, 5, 51865)
    assert ws_need > 16384
    ok = [FAKE, kb.F32, 1, 5, 51865, FAKE, 50256] + [FAKE] * 6 + [FAKE, ws_need, None]

    def call(**kw):
        args = list(ok)
        names = ["logits", "dt", "B", "K", "V", "sums", "eot", "parent", "token", "score", "fc", "fp",
                 "fs", "ws", "wsb", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)
    assert call(logits=None) == -1
    assert call(fs=None) == -1
    assert call(dt=9) == -3
    assert call(K=0) == -2 and call(K=17) == -2 and call(V=5) == -2 and call(B=0) == -2
    assert call(K=16, V=61441) == -2              # 31 chunks x 17 entries exceed the 512 merged per beam
    assert call(K=1, V=524289) == -2               # 257 chunks x 2 entries
    assert call(ws=None) == -6 and call(wsb=ws_need - 4) == -6
    assert call(logits=FAKE + 2) == -7 and call(logits=FAKE + 1, dt=kb.F16) == -7
    assert call(parent=FAKE + 2) == -7


def test_read_probe_ex_validation(lib):
    f = lib.kvd_read_probe_ex
    assert f(None, None, 16, FAKE, 4, 0, None) == -1
    assert f(FAKE, None, 16, None, 4, 0, None) == -1
    for u in (0, 3, 5, 32, -1):                       # loads in flight: 1, 2, 4, 8 or 16
        assert f(FAKE, None, 16, FAKE, u, 0, None) == -2
    assert f(FAKE, None, 16, FAKE, 4, 65536, None) == -2      # grid limit
    assert f(FAKE, None, 24, FAKE, 4, 0, None) == -2          # not a multiple of 16
    assert f(MIS, None, 16, FAKE, 4, 0, None) == -7


def test_plan_override_validation_and_reset(lib):
    f = lib.kvd_set_plan_override
    assert f(2, 0, 0) == -2
    assert f(-2, 0, 0) == -2
    assert f(-1, 17, 0) == -2
    assert f(-1, 0, -5) == -2
    # one query head over 1500 keys: 12 splits of 128 keys as planned, 24 of 64
    # on 2 waves when forced (the query's maximum over dtypes and plans grows)
    base = kb.attn_workspace_bytes(1, 1, 1, 1500)
    with kb.plan_override(waves=2, chunk=64):         # more splits: more partials
        forced = kb.attn_workspace_bytes(1, 1, 1, 1500)
    assert forced > base
    assert kb.attn_workspace_bytes(1, 1, 1, 1500) == base     # restored on exit
    assert f(-1, 0, 0) == 0
