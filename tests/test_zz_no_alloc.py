"""decode_step_self_static (its split merge in the library's static device
array, no workspace argument) against decode_step_self with a caller's
workspace, through the C ABI: the same cache bits and the same output bits,
on calls in a row whose shapes shrink, and a refusal for a shape whose merge
does not fit the array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from kv_cached_decode_amd import binding as kb
from _util import TORCH_DTYPE, bits, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _inputs(dtype, B, Hq, Hkv, N, L, seed):
    g = np.random.default_rng(seed)
    k_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
    v_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    return k_all, v_all, q


def _both(dtype, B, Hq, Hkv, N, L, rope, seed):
    """The same step through both entry points, each on its own cache that
    holds the same rows [0, L - N) before the call."""
    say(f"case: static step {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} L={L} rope={rope}")
    k_all, v_all, q = _inputs(dtype, B, Hq, Hkv, N, L, seed)
    old, new = slice(0, L - N), slice(L - N, L)
    caches = []
    for _ in range(2):
        c = kb.Cache(B, Hkv, L + 2, TORCH_DTYPE[dtype])
        if L > N:
            kb.kv_append(c, to_dev(k_all[:, :, old], dtype), to_dev(v_all[:, :, old], dtype), 0, rope)
        caches.append(c)
    qd, kn, vn = to_dev(q, dtype), to_dev(k_all[:, :, new], dtype), to_dev(v_all[:, :, new], dtype)
    ws = kb.workspace(kb.attn_workspace_bytes(B, Hq, N, L))
    ref = kb.decode_step_self(qd, kn, vn, caches[0], L, 0.125, rope_base=rope, ws=ws)
    got = kb.decode_step_self_static(qd, kn, vn, caches[1], L, 0.125, rope_base=rope)
    torch.cuda.synchronize()
    for name in ("k", "v"):
        a = from_dev(getattr(caches[0], name), dtype)
        b = from_dev(getattr(caches[1], name), dtype)
        assert np.array_equal(bits(a), bits(b)), name
    assert torch.equal(ref, got)
    return kb.attn_workspace_bytes(B, Hq, N, L)


def test_static_step_equals_workspace_step_on_shrinking_calls():
    cap = kb.static_scratch_bytes()
    # the largest first: GQA decode at 1024 with rotary keys (split merge of
    # 24 tiles), then a Whisper-shaped step at a shorter length, then a
    # 5-draft block and a tiny unsplit one
    need1 = _both("bf16", 8, 9, 3, 1, 1024, 10000.0, 1)
    need2 = _both("f16", 1, 20, 20, 1, 300, 0.0, 2)
    need3 = _both("f16", 1, 20, 20, 5, 448, 0.0, 3)
    need4 = _both("bf16", 2, 9, 3, 1, 40, 10000.0, 4)
    say(f"workspace the shapes need: {need1}, {need2}, {need3}, {need4} of {cap}")
    assert need1 > need2 > 0 and need1 <= cap


def test_static_step_repeated_calls_share_the_array():
    # the counters the merge uses are back at zero after each call, so the
    # same call again (on fresh caches) gives the same bits
    _both("f16", 1, 20, 20, 1, 448, 0.0, 5)
    _both("f16", 1, 20, 20, 1, 448, 0.0, 5)


def test_static_step_refuses_a_shape_beyond_the_array():
    B, Hq, N, L = 16, 20, 16, 448
    assert kb.attn_workspace_bytes(B, Hq, N, L) > kb.static_scratch_bytes()
    c = kb.Cache(B, 20, L, torch.float16)
    q = torch.zeros((B, Hq, N, 64), dtype=torch.float16, device="cuda")
    kn = torch.zeros((B, 20, N, 64), dtype=torch.float16, device="cuda")
    out = torch.empty((B, Hq, N, 64), dtype=torch.float32, device="cuda")
    before = c.k.clone()
    st = kb.lib().decode_step_self_static(q.data_ptr(), kn.data_ptr(), kn.data_ptr(), Hq, N,
                                          ctypes.byref(c.desc()), L, 0.125, 0.0, out.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == -9
    assert torch.equal(c.k, before)   # nothing ran
