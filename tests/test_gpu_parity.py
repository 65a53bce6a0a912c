"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: cache append (plain copy), beam reorder, argmax, accepted length and
corrected token. Attention outputs: max |err| <= 1e-5 with fp32 storage and
<= 2e-3 with fp16/bf16 storage (fp32 accumulation on the GPU, fp64 in the
oracle, both reading the same stored bits). Rotated keys are bit-exact too:
kernel and oracle both rotate in fp64 (the same pow-derived angles, each side
with its own cos / sin) and round once to the storage type.
"""
import numpy as np
import pytest
import torch

import oracle as O
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import inputs as I
from _util import TOL, TORCH_DTYPE, bits, from_dev, max_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _ws(nbytes=64 << 20):
    return kb.workspace(nbytes)


# ------------------------------------------------------------ tiny step ----

def test_tiny_step_fp32_against_recompute():
    w = I.TINY
    say("case: tiny fp32 step, self 32+1, cross 1500")
    k_all, v_all = I.self_kv(w, 0)                     # [1, 6, 33, 64]
    xk, xv = I.cross_kv(w, 0)
    q = I.queries(w, 0, 32)
    qx = I.queries(w, 0, 32, cross=True)
    cache = kb.Cache(1, 6, 33, torch.float32)
    xc = kb.Cache(1, 6, 1500, torch.float32)
    kb.kv_append(cache, to_dev(k_all[:, :, :32], "f32"), to_dev(v_all[:, :, :32], "f32"), 0)
    kb.kv_append(cache, to_dev(k_all[:, :, 32:], "f32"), to_dev(v_all[:, :, 32:], "f32"), 32)
    kb.kv_append(xc, to_dev(xk, "f32"), to_dev(xv, "f32"), 0)
    ws = _ws()
    o_self = kb.decode_attn_self(to_dev(q, "f32"), cache, 33, w.attn_scale, ws=ws)
    o_cross = kb.decode_attn_cross(to_dev(qx, "f32"), xc, 1500, w.attn_scale, ws=ws)
    torch.cuda.synchronize()

    oc = O.ConcatCache(1, 6, 64, "f32")
    oc.append(k_all[:, :, :32], v_all[:, :, :32])
    oc.append(k_all[:, :, 32:], v_all[:, :, 32:])
    ox = O.ConcatCache(1, 6, 64, "f32")
    ox.set_once(xk, xv)
    assert np.array_equal(bits(from_dev(cache.k, "f32")), bits(oc.k))
    assert np.array_equal(bits(from_dev(cache.v, "f32")), bits(oc.v))
    assert np.array_equal(bits(from_dev(xc.k, "f32")), bits(xk))
    ref_self = O.attend_self(q, oc, w.attn_scale)
    # the last row of a full causal recomputation over all 33 tokens
    full = O.full_causal_attention(np.concatenate([np.zeros((6, 32, 64)), O.widen(q, "f32")[0]], 1),
                                   O.widen(k_all, "f32")[0], O.widen(v_all, "f32")[0],
                                   w.attn_scale)[:, 32]
    assert np.max(np.abs(ref_self[0, :, 0] - full)) < 1e-12
    e_self = max_err(o_self, ref_self)
    e_cross = max_err(o_cross, O.attend_cross(qx, ox, w.attn_scale))
    say(f"tiny: self max|err| {e_self:.2e}, cross {e_cross:.2e}")
    assert e_self <= TOL["f32"] and e_cross <= TOL["f32"]


# ------------------------------------------------- whisper greedy shape ----

@pytest.mark.parametrize("layer", [0, 31])
def test_whisper_greedy_sweep_lengths(layer):
    """Full large-v2 layer shape (20 heads, 1500 frames, self cache to 448):
    tokens appended one per step, attention checked at sampled lengths that
    include split boundaries."""
    w = I.WHISPER_GREEDY
    say(f"case: whisper greedy layer {layer}")
    k_all, v_all = I.self_kv(w, layer)
    xk, xv = I.cross_kv(w, layer)
    cache = kb.Cache(1, 20, 448, torch.float16)
    xc = kb.Cache(1, 20, 1500, torch.float16)
    kb.kv_append(xc, to_dev(xk, "f16"), to_dev(xv, "f16"), 0)
    ox = O.ConcatCache(1, 20, 64, "f16")
    ox.set_once(xk, xv)
    oc = O.ConcatCache(1, 20, 64, "f16")
    kd, vd = to_dev(k_all, "f16"), to_dev(v_all, "f16")
    ws = _ws()
    check = {1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 257, 384, 447, 448}
    worst = 0.0
    for L in range(1, 449):
        kb.kv_append(cache, kd[:, :, L - 1:L].contiguous(), vd[:, :, L - 1:L].contiguous(), L - 1)
        oc.append(k_all[:, :, L - 1:L], v_all[:, :, L - 1:L])
        if L not in check:
            continue
        q = I.queries(w, layer, L)
        qx = I.queries(w, layer, L, cross=True)
        o_self = kb.decode_attn_self(to_dev(q, "f16"), cache, L, w.attn_scale, ws=ws)
        o_cross = kb.decode_attn_cross(to_dev(qx, "f16"), xc, 1500, w.attn_scale, ws=ws)
        e1 = max_err(o_self, O.attend_self(q, oc, w.attn_scale))
        e2 = max_err(o_cross, O.attend_cross(qx, ox, w.attn_scale))
        worst = max(worst, e1, e2)
        assert e1 <= TOL["f16"] and e2 <= TOL["f16"], (L, e1, e2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(from_dev(cache.k, "f16")), bits(oc.k))
    assert np.array_equal(bits(from_dev(cache.v, "f16")), bits(oc.v))
    say(f"whisper layer {layer}: worst max|err| {worst:.2e}")


# Plans forced through the library's testing hook (kvd_set_plan_override),
# so that split boundaries and the narrow (1-, 2-wave) and wide (8-wave)
# workgroups are covered at lengths the default plan runs otherwise.
# Blocks of queries (N > 1, 16-bit storage) take the matrix-core kernel by
# default; "stream" runs them through the streaming kernel instead.
PLANS = {"default": {}, "chunk128": {"chunk": 128},
         "wide": {"waves": 8}, "wide_chunk512": {"waves": 8, "chunk": 512},
         "w8_chunk256": {"waves": 8, "chunk": 256},
         "w1": {"waves": 1}, "w2_chunk64": {"waves": 2, "chunk": 64},
         "stream": {"mfma": 0}, "stream_chunk128": {"mfma": 0, "chunk": 128}}


@pytest.fixture(params=list(PLANS))
def plan(request):
    with kb.plan_override(**PLANS[request.param]):
        yield request.param


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 5])
@pytest.mark.parametrize("L", [1, 2, 5, 64, 129, 130, 133, 257, 448, 1100])
def test_sentinel_mask(dtype, N, L, plan):
    """Query i's own key and the next key (one it must not see) both align
    with it; one-hot values name every key that got weight."""
    if L < N:
        pytest.skip("len < N")
    say(f"case: sentinel dtype={dtype} N={N} L={L} plan={plan}")
    g = np.random.default_rng(100 + L + N)
    H, D = 4, 64
    k = g.standard_normal((1, H, L, D)) * 0.05
    v = np.zeros((1, H, L, D))
    v[0, :, np.arange(L), np.arange(L) % D] = 1.0
    q = np.zeros((1, H, N, D))
    for i in range(N):
        q[0, :, i, 40 + i] = 1.0
        p = L - N + i
        k[0, :, p, 40 + i] = 120.0
        if p + 1 < L:
            k[0, :, p + 1, 40 + i] = 120.0
    ks, vs, qs = (O.narrow(a, dtype) for a in (k, v, q))
    cache = kb.Cache.wrap(to_dev(ks, dtype), to_dev(vs, dtype))
    out = kb.decode_attn_self(to_dev(qs, dtype), cache, L, 0.125, ws=_ws())
    oc = O.ConcatCache(1, H, D, dtype)
    oc.append(ks, vs)
    ref = O.attend_self(qs, oc, 0.125)
    got = out.cpu().numpy()
    for i in range(N):
        own = (L - N + i) % D
        assert np.all(got[0, :, i, own] > 0.99)
    assert max_err(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_large_scores_online_rescale(dtype, plan):
    """Scores with sd ~ 16: the running max changes often inside a split."""
    say(f"case: large scores {dtype} plan={plan}")
    g = np.random.default_rng(5)
    B, H, L, N = 2, 8, 700, 3
    k = O.narrow(g.standard_normal((B, H, L, 64)) * 4, dtype)
    v = O.narrow(g.standard_normal((B, H, L, 64)), dtype)
    q = O.narrow(g.standard_normal((B, H, N, 64)) * 4, dtype)
    cache = kb.Cache.wrap(to_dev(k, dtype), to_dev(v, dtype))
    out = kb.decode_attn_self(to_dev(q, dtype), cache, L, 0.125, ws=_ws())
    oc = O.ConcatCache(B, H, 64, dtype)
    oc.append(k, v)
    e = max_err(out, O.attend_self(q, oc, 0.125))
    say(f"large scores {dtype}: {e:.2e}")
    assert e <= TOL[dtype]


# ------------------------------------------------------- ragged batches ----
# Each batch row has its own length ([S] over a batch of sequences). Rows past
# a row's length hold large "poison" keys and values: reading any of them
# would move that row's output far outside the tolerance.

def _ragged_setup(dtype, group, N, lens, S_max, g):
    B, Hkv = len(lens), 2
    Hq = Hkv * group
    k = g.standard_normal((B, Hkv, S_max, 64)) * 0.5
    v = g.standard_normal((B, Hkv, S_max, 64))
    for b, L in enumerate(lens):
        k[b, :, L:] = g.standard_normal((Hkv, S_max - L, 64)) * 8.0
        v[b, :, L:] = 100.0
    q = g.standard_normal((B, Hq, N, 64))
    return tuple(O.narrow(a, dtype) for a in (k, v, q))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 5])
@pytest.mark.parametrize("group,rope", [(1, 0.0), (3, 1e4)])
def test_ragged_self_attention(dtype, N, group, rope, plan):
    say(f"case: ragged self {dtype} N={N} group={group} rope={rope} plan={plan}")
    g = np.random.default_rng([40, N, group, len(dtype)])
    S_max, len_max = 448, 448
    lens = [448, 441, 65, N]
    ks, vs, qs = _ragged_setup(dtype, group, N, lens, S_max, g)
    cache = kb.Cache.wrap(to_dev(ks, dtype), to_dev(vs, dtype))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = kb.decode_attn_self_ragged(to_dev(qs, dtype), cache, lt, len_max, 0.125, rope_base=rope,
                                     ws=_ws(), dev_status=st)
    rows = []
    for b, L in enumerate(lens):
        c = O.ConcatCache(1, ks.shape[1], 64, dtype)
        c.append(ks[b:b + 1, :, :L], vs[b:b + 1, :, :L])
        rows.append(c)
    e = max_err(out, O.attend_self_ragged(qs, rows, 0.125, rope_base=rope))
    assert e <= TOL[dtype], e
    assert int(st.item()) == 0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N", [1, 5, 16])
def test_ragged_step_self_equals_append_then_attend(dtype, N, plan):
    """The fused ragged step writes each row's N new rows at lens[b] - N
    (rotated for bf16) exactly as kv_append_ragged does, returns what
    decode_attn_self_ragged returns afterwards, and matches the oracle."""
    say(f"case: ragged step {dtype} N={N} plan={plan}")
    g = np.random.default_rng([41, N, len(dtype)])
    rope = 1e4 if dtype == "bf16" else 0.0
    S_max, len_max = 448, 448
    lens = [448, 300, N + 2, N]
    ks, vs, qs = _ragged_setup(dtype, 3 if dtype == "bf16" else 1, N, lens, S_max, g)
    kn = O.narrow(g.standard_normal((4, 2, N, 64)) * 0.5, dtype)
    vn = O.narrow(g.standard_normal((4, 2, N, 64)), dtype)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pt = torch.tensor([L - N for L in lens], dtype=torch.int32, device="cuda")
    fused = kb.Cache.wrap(to_dev(ks, dtype), to_dev(vs, dtype))
    split = kb.Cache.wrap(to_dev(ks, dtype), to_dev(vs, dtype))
    ws = _ws()
    out_f = kb.decode_step_self_ragged(to_dev(qs, dtype), to_dev(kn, dtype), to_dev(vn, dtype),
                                       fused, lt, len_max, 0.125, rope_base=rope, ws=ws)
    kb.kv_append_ragged(split, to_dev(kn, dtype), to_dev(vn, dtype), pt, rope_base=rope)
    out_s = kb.decode_attn_self_ragged(to_dev(qs, dtype), split, lt, len_max, 0.125,
                                       rope_base=rope, ws=ws)
    assert np.array_equal(bits(from_dev(fused.k, dtype)), bits(from_dev(split.k, dtype)))
    assert np.array_equal(bits(from_dev(fused.v, dtype)), bits(from_dev(split.v, dtype)))
    assert torch.equal(out_f, out_s)
    rows = []
    fk, fv = from_dev(fused.k, dtype), from_dev(fused.v, dtype)
    for b, L in enumerate(lens):
        c = O.ConcatCache(1, 2, 64, dtype)
        c.append(ks[b:b + 1, :, :L - N], vs[b:b + 1, :, :L - N])
        c.append(kn[b:b + 1], vn[b:b + 1], rope_base=rope)
        rows.append(c)
        assert _same_bits(fk[b:b + 1, :, :L], c.k, f"row {b} keys")
        assert _same_bits(fv[b:b + 1, :, :L], c.v, f"row {b} values")
    e = max_err(out_f, O.attend_self_ragged(qs, rows, 0.125, rope_base=rope))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_kv_append_ragged_bit_exact_and_skips_rows_outside(dtype):
    say(f"case: append ragged {dtype}")
    g = np.random.default_rng(42)
    B, H, S_max, T = 4, 3, 448, 5
    base_k = O.narrow(g.standard_normal((B, H, S_max, 64)), dtype)
    base_v = O.narrow(g.standard_normal((B, H, S_max, 64)), dtype)
    kn = O.narrow(g.standard_normal((B, H, T, 64)), dtype)
    vn = O.narrow(g.standard_normal((B, H, T, 64)), dtype)
    pos = [0, 100, 443, 444]                       # row 3 would end at 449 > S_max
    cache = kb.Cache.wrap(to_dev(base_k, dtype), to_dev(base_v, dtype))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kb.kv_append_ragged(cache, to_dev(kn, dtype), to_dev(vn, dtype),
                        torch.tensor(pos, dtype=torch.int32, device="cuda"), dev_status=st)
    want_k, want_v = base_k.copy(), base_v.copy()
    for b in range(3):
        want_k[b, :, pos[b]:pos[b] + T] = kn[b]
        want_v[b, :, pos[b]:pos[b] + T] = vn[b]
    assert np.array_equal(bits(from_dev(cache.k, dtype)), bits(want_k))
    assert np.array_equal(bits(from_dev(cache.v, dtype)), bits(want_v))
    assert int(st.item()) == -4


def test_ragged_lengths_outside_the_plan_are_clamped_and_flagged():
    say("case: ragged clamp")
    g = np.random.default_rng(43)
    N, len_max = 5, 448
    given = [500, 3, 100, 448]
    used = [448, 5, 100, 448]
    ks, vs, qs = _ragged_setup("f16", 1, N, used, 448, g)
    cache = kb.Cache.wrap(to_dev(ks, "f16"), to_dev(vs, "f16"))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kb.decode_attn_self_ragged(to_dev(qs, "f16"), cache,
                                     torch.tensor(given, dtype=torch.int32, device="cuda"),
                                     len_max, 0.125, ws=_ws(), dev_status=st)
    rows = []
    for b, L in enumerate(used):
        c = O.ConcatCache(1, 2, 64, "f16")
        c.append(ks[b:b + 1, :, :L], vs[b:b + 1, :, :L])
        rows.append(c)
    assert max_err(out, O.attend_self_ragged(qs, rows, 0.125)) <= TOL["f16"]
    assert int(st.item()) == -4


def test_ragged_speculative_loop_with_rollback():
    """Whisper self-attention shape, 4 sequences: every iteration appends 5
    drafts to each row at its own length (one fused launch), and each row then
    keeps its own number of them; the next iteration writes over the rest.
    Outputs match the oracle every iteration, and the kept cache rows match
    the oracle's cache bit for bit at the end."""
    say("case: ragged speculative loop")
    g = np.random.default_rng(44)
    B, H, N, S_max = 4, 20, 5, 448
    pos = [10, 57, 200, 390]
    cache = kb.Cache(B, H, S_max, torch.float16)
    rows = []
    for b in range(B):
        k0 = O.narrow(g.standard_normal((1, H, pos[b], 64)) * 0.5, "f16")
        v0 = O.narrow(g.standard_normal((1, H, pos[b], 64)), "f16")
        cache.k[b:b + 1, :, :pos[b]].copy_(to_dev(k0, "f16"))
        cache.v[b:b + 1, :, :pos[b]].copy_(to_dev(v0, "f16"))
        c = O.ConcatCache(1, H, 64, "f16")
        c.append(k0, v0)
        rows.append(c)
    ws = _ws()
    for it in range(8):
        lens = [p + N for p in pos]
        q = O.narrow(g.standard_normal((B, H, N, 64)), "f16")
        kn = O.narrow(g.standard_normal((B, H, N, 64)) * 0.5, "f16")
        vn = O.narrow(g.standard_normal((B, H, N, 64)), "f16")
        out = kb.decode_step_self_ragged(to_dev(q, "f16"), to_dev(kn, "f16"), to_dev(vn, "f16"),
                                         cache, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                         S_max, 0.125, ws=ws)
        for b in range(B):
            rows[b].append(kn[b:b + 1], vn[b:b + 1])
        e = max_err(out, O.attend_self_ragged(q, rows, 0.125))
        assert e <= TOL["f16"], (it, e)
        for b in range(B):
            keep = int(g.integers(0, N + 1))
            pos[b] = min(pos[b] + keep, S_max - N)
            rows[b].truncate(pos[b])
    got_k, got_v = from_dev(cache.k, "f16"), from_dev(cache.v, "f16")
    for b in range(B):
        assert np.array_equal(bits(got_k[b, :, :pos[b]]), bits(rows[b].k[0]))
        assert np.array_equal(bits(got_v[b, :, :pos[b]]), bits(rows[b].v[0]))


@pytest.mark.parametrize("dtype,rope", [("f16", 0.0), ("bf16", 1e4)])
@pytest.mark.parametrize("N", [80, 72, 100])
@pytest.mark.parametrize("ragged", [False, True])
def test_prefill_tiles_paired(dtype, rope, N, ragged):
    """Causal blocks on one 16-row tile per wave, each wave taking a tile and
    its complement (4 rows x 2 KV heads x 4 query heads: 20, 18 and 25 tiles
    per unit, the odd count leaving the middle tile alone)."""
    say(f"case: paired prefill {dtype} N={N} ragged={ragged}")
    g = np.random.default_rng([45, N, len(dtype), int(ragged)])
    B, Hq, Hkv, S = 4, 8, 2, 256
    lens = [N + 30, N + 30, N + 30, N + 30] if not ragged else [N + 30, N + 3, N + 100, N]
    k = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    v = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    cache = kb.Cache.wrap(to_dev(k, dtype), to_dev(v, dtype))
    ws = _ws()
    if ragged:
        out = kb.decode_attn_self_ragged(to_dev(q, dtype), cache,
                                         torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                         max(lens), 0.125, rope_base=rope, ws=ws)
    else:
        out = kb.decode_attn_self(to_dev(q, dtype), cache, lens[0], 0.125, rope_base=rope, ws=ws)
    rows = []
    for b, L in enumerate(lens):
        c = O.ConcatCache(1, Hkv, 64, dtype)
        c.append(k[b:b + 1, :, :L], v[b:b + 1, :, :L])
        rows.append(c)
    e = max_err(out, O.attend_self_ragged(q, rows, 0.125, rope_base=rope))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N", [96, 37])
def test_query_block_over_cross_cache(dtype, N):
    """A block of N queries per head over a 1500-frame cross cache (no mask):
    with 96 rows the matrix-core prefill plan (every row sees every frame, the
    last 64-key block ragged at 1500); with 37 the shared-tile plan."""
    say(f"case: query block over cross cache {dtype} N={N}")
    g = np.random.default_rng([46, N, len(dtype)])
    B, H, F = 1, 20, 1500
    xk = O.narrow(g.standard_normal((B, H, F, 64)) / 8, dtype)
    xv = O.narrow(g.standard_normal((B, H, F, 64)) / 8, dtype)
    q = O.narrow(g.standard_normal((B, H, N, 64)) / 8, dtype)
    xc = kb.Cache(B, H, F, TORCH_DTYPE[dtype])
    kb.kv_append(xc, to_dev(xk, dtype), to_dev(xv, dtype), 0)
    out = kb.decode_attn_cross(to_dev(q, dtype), xc, F, 0.125, ws=_ws())
    ox = O.ConcatCache(B, H, 64, dtype)
    ox.set_once(xk, xv)
    e = max_err(out, O.attend_cross(q, ox, 0.125))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("dtype,rope", [("f16", 0.0), ("bf16", 1e4), ("f16", 1e4)])
@pytest.mark.parametrize("N,L", [(200, 200), (130, 333), (64, 64)])
def test_prefill_blocks_mha(dtype, rope, N, L):
    """One query head per KV head (no grouping), N causal queries at the end
    of a cache of L rows: row blocks of 64 that end inside a sequence, cache
    lengths that are not a multiple of the 64-key staging block."""
    say(f"case: mha prefill {dtype} rope={rope} N={N} L={L}")
    g = np.random.default_rng([47, N, L, len(dtype), int(rope)])
    B, H, S = 2, 4, 352
    k = O.narrow(g.standard_normal((B, H, S, 64)), dtype)
    v = O.narrow(g.standard_normal((B, H, S, 64)), dtype)
    q = O.narrow(g.standard_normal((B, H, N, 64)), dtype)
    cache = kb.Cache.wrap(to_dev(k, dtype), to_dev(v, dtype))
    out = kb.decode_attn_self(to_dev(q, dtype), cache, L, 0.125, rope_base=rope, ws=_ws())
    oc = O.ConcatCache(B, H, 64, dtype)
    oc.append(k[:, :, :L], v[:, :, :L])
    e = max_err(out, O.attend_self(q, oc, 0.125, rope_base=rope))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("dtype,rope", [("f16", 0.0), ("bf16", 1e4), ("bf16", 0.0)])
@pytest.mark.parametrize("B,Hkv,group,N,L", [(2, 2, 3, 384, 384), (1, 4, 1, 256, 600), (3, 1, 2, 320, 330)])
def test_prefill_long_row_blocks(dtype, rope, B, Hkv, group, N, L):
    """Causal prefill with row blocks of 64 that tile the sequences and up to
    10 key blocks per row block: 384 queries from position 0, 256 queries
    after 344 cached rows, 320 queries after 10 rows; the same call twice
    gives the same bits."""
    say(f"case: prefill long row blocks {dtype} rope={rope} B={B} Hkv={Hkv} group={group} N={N} L={L}")
    g = np.random.default_rng([48, B, Hkv, group, N, L, len(dtype), int(rope)])
    Hq, S = Hkv * group, L + 8
    k = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    v = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    cache = kb.Cache.wrap(to_dev(k, dtype), to_dev(v, dtype))
    ws = _ws()
    out = kb.decode_attn_self(to_dev(q, dtype), cache, L, 0.125, rope_base=rope, ws=ws)
    again = kb.decode_attn_self(to_dev(q, dtype), cache, L, 0.125, rope_base=rope, ws=ws)
    assert torch.equal(out, again)
    oc = O.ConcatCache(B, Hkv, 64, dtype)
    oc.append(k[:, :, :L], v[:, :, :L])
    e = max_err(out, O.attend_self(q, oc, 0.125, rope_base=rope))
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("dtype,rope", [("f16", 0.0), ("bf16", 1e4)])
def test_prefill_per_cu_order_partial_round(dtype, rope):
    """A prefill grid whose units are a multiple of 8 (the per-CU workgroup
    order applies) with 40 row blocks per unit: per XCD one full round of 32
    workgroups and a reversed partial round of 8, so every (unit, row block)
    pair must still be taken exactly once (8 rows x 1 KV head x 20 query
    heads, 128 causal queries after 32 cached rows)."""
    say(f"case: prefill per-CU order, partial round {dtype} rope={rope}")
    g = np.random.default_rng([49, len(dtype), int(rope)])
    B, Hkv, group, N, L = 8, 1, 20, 128, 160
    Hq, S = Hkv * group, L
    k = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    v = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    cache = kb.Cache.wrap(to_dev(k, dtype), to_dev(v, dtype))
    out = kb.decode_attn_self(to_dev(q, dtype), cache, L, 0.125, rope_base=rope, ws=_ws())
    oc = O.ConcatCache(B, Hkv, 64, dtype)
    oc.append(k, v)
    e = max_err(out, O.attend_self(q, oc, 0.125, rope_base=rope))
    assert e <= TOL[dtype], e


# ------------------------------------------------------ speculative verify ----

@pytest.mark.parametrize("L_before", list(I.WHISPER_VERIFY.extra["L_before"]))
def test_verify_attention_n5(L_before, plan):
    """Five draft rows appended at once, causal among themselves, over the
    self cache and the cross cache (large-v2 layer shape)."""
    w = I.WHISPER_VERIFY
    say(f"case: verify attention L_before={L_before} plan={plan}")
    layer = 3
    L = L_before + 5
    k_all, v_all = I.self_kv(w, layer)
    xk, xv = I.cross_kv(w, layer)
    cache = kb.Cache(1, 20, 448, torch.float16)
    kb.kv_append(cache, to_dev(k_all[:, :, :L_before], "f16"), to_dev(v_all[:, :, :L_before], "f16"), 0)
    kb.kv_append(cache, to_dev(k_all[:, :, L_before:L], "f16"), to_dev(v_all[:, :, L_before:L], "f16"),
                 L_before)
    xc = kb.Cache(1, 20, 1500, torch.float16)
    kb.kv_append(xc, to_dev(xk, "f16"), to_dev(xv, "f16"), 0)
    q = I.queries(w, layer, L, N=5)
    qx = I.queries(w, layer, L, N=5, cross=True)
    ws = _ws()
    o_self = kb.decode_attn_self(to_dev(q, "f16"), cache, L, w.attn_scale, ws=ws)
    o_cross = kb.decode_attn_cross(to_dev(qx, "f16"), xc, 1500, w.attn_scale, ws=ws)
    oc = O.ConcatCache(1, 20, 64, "f16")
    oc.append(k_all[:, :, :L_before], v_all[:, :, :L_before])
    oc.append(k_all[:, :, L_before:L], v_all[:, :, L_before:L])
    ox = O.ConcatCache(1, 20, 64, "f16")
    ox.set_once(xk, xv)
    e1 = max_err(o_self, O.attend_self(q, oc, w.attn_scale))
    e2 = max_err(o_cross, O.attend_cross(qx, ox, w.attn_scale))
    say(f"verify L={L}: self {e1:.2e} cross {e2:.2e}")
    assert e1 <= TOL["f16"] and e2 <= TOL["f16"]


def _verify_gpu(logits, draft, dtype="f32"):
    lt = to_dev(logits if dtype == "f32" else O.narrow(logits.astype(np.float64), dtype), dtype)
    dt = torch.from_numpy(draft).to("cuda")
    B, R, _ = logits.shape
    am = torch.empty((B, R), dtype=torch.int32, device="cuda")
    acc, nxt, _ = kb.verify_accept(lt, dt, argmax_out=am)
    return acc.cpu().numpy(), nxt.cpu().numpy(), am.cpu().numpy()


def test_verify_accept_random_trials_bit_exact():
    """1000 trials at V = 51865 (7 in 8 with a planted argmax per row that the
    drafts copy with p = 0.75): argmax, accepted length and next token equal
    the oracle's; over the planted trials the accepted lengths follow
    P(n = k) = 0.75^k 0.25 for k < 5 and P(5) = 0.75^5 (chi-square, 5 degrees
    of freedom, below the 0.001 critical value 20.52)."""
    w = I.WHISPER_VERIFY
    trials = 1000
    say(f"case: verify_accept {trials} trials V=51865")
    hist = np.zeros(6, dtype=int)
    for t in range(trials):
        planted = t % 8 != 0
        logits, draft = I.verify_logits(w, t, plant=planted)
        acc, nxt, am = _verify_gpu(logits, draft)
        ram, racc, rnxt = O.verify_accept(logits, draft)
        assert np.array_equal(am, ram), t
        assert np.array_equal(acc, racc) and np.array_equal(nxt, rnxt), t
        if planted:
            hist[int(acc[0])] += 1
    p = w.extra["p_match"]
    probs = np.array([p ** k * (1 - p) for k in range(5)] + [p ** 5])
    expected = probs * hist.sum()
    chi2 = float(((hist - expected) ** 2 / expected).sum())
    say(f"accept histogram {hist.tolist()} expected {np.round(expected, 1).tolist()} chi2 {chi2:.2f}")
    assert chi2 < 20.52


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_verify_accept_edges(dtype):
    say(f"case: verify edges {dtype}")
    g = np.random.default_rng(21)
    B, N, V = 4, 5, 51865
    for R in (N, N + 1):
        logits = g.standard_normal((B, R, V)).astype(np.float32) * 2
        logits[0, 0, [4095, 4096, 9000]] = 30.0          # tie across workgroup slices
        logits[0, 1, :] = -np.inf                          # all -inf -> 0
        logits[0, 2, :5000] = -np.inf
        logits[1, 0, V - 1] = 31.0                         # last element
        logits[1, 1, :] = 0.5                              # all equal -> 0
        logits[2, 3, [17, 40000]] = 33.0
        ref_am = O.argmax_rows(O.widen(O.narrow(logits.astype(np.float64), dtype), dtype)
                               if dtype != "f32" else logits)
        draft = ref_am[:, :N].copy().astype(np.int32)
        draft[1, 2] = -5                                   # out of range never matches
        draft[2, 0] = V + 7
        draft[3, 4] = (draft[3, 4] + 1) % V                # mismatch at the last draft
        acc, nxt, am = _verify_gpu(logits, draft, dtype)
        racc = np.zeros(B, np.int32)
        rnxt = np.zeros(B, np.int32)
        for b in range(B):
            racc[b], rnxt[b] = O.accept(ref_am[b], draft[b])
        assert np.array_equal(am, ref_am)
        assert np.array_equal(acc, racc) and np.array_equal(nxt, rnxt)
        assert acc[0] == N and nxt[0] == (ref_am[0, N] if R == N + 1 else -1)


@pytest.mark.parametrize("V", [1, 7, 2048, 2049, 4096, 4097, 12289])
def test_verify_accept_small_vocab(V):
    say(f"case: verify V={V}")
    g = np.random.default_rng(V)
    logits = np.round(g.standard_normal((2, 3, V)) * 2).astype(np.float32)  # many ties
    draft = g.integers(0, V, (2, 3)).astype(np.int32)
    acc, nxt, am = _verify_gpu(logits, draft)
    ram, racc, rnxt = O.verify_accept(logits, draft)
    assert np.array_equal(am, ram) and np.array_equal(acc, racc) and np.array_equal(nxt, rnxt)


def _masked_gpu(logits, draft, sup, first, dtype="f32"):
    lt = to_dev(logits if dtype == "f32" else O.narrow(logits.astype(np.float64), dtype), dtype)
    B, R, V = logits.shape
    dt = torch.from_numpy(draft).to("cuda") if draft is not None and draft.shape[1] else None
    sp = kb.token_bitmap(np.flatnonzero(sup), V) if sup is not None else None
    sf = kb.token_bitmap(np.flatnonzero(first), V) if first is not None else None
    am = torch.empty((B, R), dtype=torch.int32, device="cuda")
    acc, nxt, _ = kb.verify_accept_masked(lt, dt, sp, sf, argmax_out=am)
    return acc.cpu().numpy(), nxt.cpu().numpy(), am.cpu().numpy()


def _masked_ref(logits, draft, sup, first, dtype="f32"):
    x = logits if dtype == "f32" else O.widen(O.narrow(logits.astype(np.float64), dtype), dtype)
    d = draft if draft is not None else np.zeros((logits.shape[0], 0), dtype=np.int32)
    return O.verify_accept_masked(x, d, sup, first)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("R_extra", [0, 1])
def test_verify_accept_masked_filters(dtype, R_extra):
    """SuppressTokens (30% of the vocabulary, every row) and SuppressBlank
    (blank and end-of-text, first row only) before the argmax, at the
    whisper-large-v2 vocabulary, drafts agreeing with the filtered argmax
    except where planted."""
    say(f"case: verify masked {dtype} R=N+{R_extra}")
    g = np.random.default_rng([25, R_extra, len(dtype)])
    B, N, V, blank, eot = 3, 5, 51865, 220, 50256
    R = N + R_extra
    logits = (g.standard_normal((B, R, V)) * 2).astype(np.float32)
    sup = g.random(V) < 0.3
    sup[[blank, eot]] = False
    first = np.zeros(V, dtype=bool)
    first[[blank, eot]] = True
    logits[:, :, blank] = 40.0                       # blank wins every row but the first
    logits[0, 0, eot] = 41.0                         # end-of-text would win (0, 0)
    top = np.flatnonzero(sup)[:3]
    logits[1, :, top] = 50.0                         # suppressed tokens would win row 1
    ram, _, _ = _masked_ref(logits, np.zeros((B, N), np.int32), sup, first, dtype)
    draft = ram[:, :N].astype(np.int32).copy()
    draft[2, 3] = top[0]                             # a draft the filter removed
    acc, nxt, am = _masked_gpu(logits, draft, sup, first, dtype)
    ram, racc, rnxt = _masked_ref(logits, draft, sup, first, dtype)
    assert np.array_equal(am, ram) and np.array_equal(acc, racc) and np.array_equal(nxt, rnxt)
    assert (am[:, 0] != blank).all() and (am[:, 1:] == blank).all() and acc[2] == 3


@pytest.mark.parametrize("B,V", [(4, 51865), (2, 7), (1, 2049), (1, 1 << 20)])
def test_verify_accept_masked_language_detection(B, V):
    """No drafts, one row: the argmax over an allowed token set (every other
    token suppressed), with ties among the allowed tokens and a suppressed
    global maximum; one batch row has every token suppressed (gives 0)."""
    say(f"case: masked argmax B={B} V={V}")
    g = np.random.default_rng([26, B, V])
    logits = (g.standard_normal((B, 1, V)) * 2).astype(np.float32)
    lang = np.sort(g.choice(V, size=min(V, 99), replace=False))
    sup = np.ones(V, dtype=bool)
    sup[lang] = False
    logits[0, 0, lang[:2]] = 60.0                    # tie: the lower token wins
    big = np.flatnonzero(sup)
    if big.size:
        logits[-1, 0, big[0]] = 70.0                 # suppressed, must not win
    acc, nxt, am = _masked_gpu(logits, None, sup, None)
    ram, racc, rnxt = _masked_ref(logits, None, sup, None)
    assert np.array_equal(am, ram) and np.array_equal(nxt, rnxt) and (acc == 0).all()
    assert nxt[0] == lang[0]
    acc, nxt, am = _masked_gpu(logits, None, np.ones(V, dtype=bool), None)
    assert (nxt == 0).all() and (am == 0).all()


def test_verify_accept_masked_without_bitmaps_equals_verify_accept():
    say("case: masked verify with no bitmaps")
    w = I.WHISPER_VERIFY
    for t in range(20):
        logits, draft = I.verify_logits(w, 1000 + t, plant=True)
        a = _verify_gpu(logits, draft)
        b = _masked_gpu(logits, draft, None, None)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


# ------------------------------------------------------------------ beam ----

def test_beam_reorder_and_attention():
    w = I.WHISPER_BEAM
    say("case: beam 5, 224 steps, two layers")
    layers = [0, 1]
    steps = 224
    ws = _ws()
    xcs, oxs, caches, ocs, kvs = [], [], [], [], []
    for l in layers:
        xk, xv = I.cross_kv(w, l)
        xc = kb.Cache(1, 20, 1500, torch.float16)
        kb.kv_append(xc, to_dev(xk, "f16"), to_dev(xv, "f16"), 0)
        ox = O.ConcatCache(1, 20, 64, "f16"); ox.set_once(xk, xv)
        xcs.append(xc); oxs.append(ox)
        caches.append(kb.Cache(5, 20, 448, torch.float16))
        ocs.append(O.ConcatCache(5, 20, 64, "f16"))
        k_all, v_all = I.self_kv(w, l)
        kvs.append((k_all, v_all, to_dev(k_all, "f16"), to_dev(v_all, "f16")))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    worst = 0.0
    for s in range(steps):
        par = I.parents(w, s)
        pd = torch.from_numpy(par).to("cuda")
        L = s + 1
        for li, l in enumerate(layers):
            k_all, v_all, kd, vd = kvs[li]
            if s > 0:
                kb.kv_reorder(caches[li], pd, s, status)
                ocs[li].reorder(par)
            kb.kv_append(caches[li], kd[:, :, s:s + 1].contiguous(), vd[:, :, s:s + 1].contiguous(), s)
            ocs[li].append(k_all[:, :, s:s + 1], v_all[:, :, s:s + 1])
            if s % 16 == 15 or s == steps - 1:
                q = I.queries(w, l, s)
                qx = I.queries(w, l, s, cross=True)
                o1 = kb.decode_attn_self(to_dev(q, "f16"), caches[li], L, w.attn_scale, ws=ws)
                o2 = kb.decode_attn_cross(to_dev(qx, "f16"), xcs[li], 1500, w.attn_scale, ws=ws)
                e1 = max_err(o1, O.attend_self(q, ocs[li], w.attn_scale))
                e2 = max_err(o2, O.attend_cross(qx, oxs[li], w.attn_scale))
                worst = max(worst, e1, e2)
                assert e1 <= TOL["f16"] and e2 <= TOL["f16"]
                kc = from_dev(caches[li].k, "f16")[:, :, :L]
                vc = from_dev(caches[li].v, "f16")[:, :, :L]
                assert np.array_equal(bits(kc), bits(ocs[li].k))
                assert np.array_equal(bits(vc), bits(ocs[li].v))
    assert int(status.item()) == 0
    say(f"beam: worst attention max|err| {worst:.2e}")


def test_reorder_duplicate_parents_and_bad_parent():
    say("case: reorder duplicates / invalid parent")
    g = np.random.default_rng(3)
    for dtype in ("f32", "f16", "bf16"):
        B, H, S, L = 7, 3, 40, 33
        k = O.narrow(g.standard_normal((B, H, S, 64)), dtype)
        v = O.narrow(g.standard_normal((B, H, S, 64)), dtype)
        cache = kb.Cache.wrap(to_dev(k, dtype), to_dev(v, dtype))
        par = np.array([3, 3, 0, 6, 6, 6, 1], dtype=np.int32)
        kb.kv_reorder(cache, torch.from_numpy(par).cuda(), L)
        ek = k.copy(); ek[:, :, :L] = O.reorder(k[:, :, :L], par)
        ev = v.copy(); ev[:, :, :L] = O.reorder(v[:, :, :L], par)
        assert np.array_equal(bits(from_dev(cache.k, dtype)), bits(ek))
        assert np.array_equal(bits(from_dev(cache.v, dtype)), bits(ev))
        # an invalid parent leaves its beam unchanged and is reported
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        before_k = from_dev(cache.k, dtype)
        bad = np.array([1, 0, 9, 3, -1, 5, 6], dtype=np.int32)
        kb.kv_reorder(cache, torch.from_numpy(bad).cuda(), L, status)
        after_k = from_dev(cache.k, dtype)
        assert int(status.item()) == -2
        assert np.array_equal(bits(after_k[2]), bits(before_k[2]))
        assert np.array_equal(bits(after_k[4]), bits(before_k[4]))
        assert np.array_equal(bits(after_k[0, :, :L]), bits(before_k[1, :, :L]))
        assert np.array_equal(bits(after_k[0, :, L:]), bits(before_k[0, :, L:]))


# ---------------------------------------------------------- GQA + RoPE ----

def _same_bits(gpu, ref, what):
    """Bit equality of two storage arrays, reporting how many elements differ."""
    gb, rb = bits(gpu), bits(ref)
    diff = int(np.count_nonzero(gb != rb))
    say(f"{what}: {diff} of {gb.size} elements differ")
    return diff == 0


@pytest.mark.parametrize("layer", [0, 29])
def test_gqa_prefill_then_decode_with_rope(layer):
    """B=8, 9 query / 3 KV heads, bf16, RoPE base 10000: prefill 512 tokens
    (one append, 512 causal queries), then decode to 1024 one token at a time."""
    w = I.GQA_PREFILL_DECODE
    say(f"case: gqa prefill+decode layer {layer}")
    P, S = 512, 1024
    k_all, v_all = I.self_kv(w, layer)                  # [8, 3, 1024, 64] bf16
    kd, vd = to_dev(k_all, "bf16"), to_dev(v_all, "bf16")
    cache = kb.Cache(8, 3, S, torch.bfloat16)
    oc = O.ConcatCache(8, 3, 64, "bf16")
    ws = _ws()
    # prefill
    kb.kv_append(cache, kd[:, :, :P].contiguous(), vd[:, :, :P].contiguous(), 0, rope_base=w.rope_base)
    oc.append(k_all[:, :, :P], v_all[:, :, :P], rope_base=w.rope_base)
    qp = I.queries(w, layer, 0, N=P)
    out = kb.decode_attn_self(to_dev(qp, "bf16"), cache, P, w.attn_scale, rope_base=w.rope_base, ws=ws)
    gk = from_dev(cache.k, "bf16")[:, :, :P]
    assert _same_bits(gk, oc.k, "prefill rotated keys")
    assert np.array_equal(from_dev(cache.v, "bf16")[:, :, :P], oc.v)
    # the oracle attends over its own rotated keys; the kernel over its own
    e = max_err(out, O.attend_self(qp, oc, w.attn_scale, rope_base=w.rope_base))
    say(f"prefill max|err| {e:.2e}")
    assert e <= TOL["bf16"]
    # decode
    check = {P + 1, 700, S}
    for L in range(P + 1, S + 1):
        kb.kv_append(cache, kd[:, :, L - 1:L].contiguous(), vd[:, :, L - 1:L].contiguous(), L - 1,
                     rope_base=w.rope_base)
        oc.append(k_all[:, :, L - 1:L], v_all[:, :, L - 1:L], rope_base=w.rope_base)
        if L in check:
            q = I.queries(w, layer, L)
            o = kb.decode_attn_self(to_dev(q, "bf16"), cache, L, w.attn_scale, rope_base=w.rope_base, ws=ws)
            e = max_err(o, O.attend_self(q, oc, w.attn_scale, rope_base=w.rope_base))
            say(f"decode L={L} max|err| {e:.2e}")
            assert e <= TOL["bf16"]
    assert _same_bits(from_dev(cache.k, "bf16"), oc.k, "rotated keys after decode to 1024")
    assert _same_bits(from_dev(cache.v, "bf16"), oc.v, "values after decode to 1024")


def test_cross_cache_per_row_and_shared_agree():
    """A cross cache shared by 3 rows gives what 3 identical per-row copies give."""
    say("case: cross shared vs per-row")
    g = np.random.default_rng(8)
    F = 1500
    xk = O.narrow(g.standard_normal((1, 6, F, 64)) / 8, "f16")
    xv = O.narrow(g.standard_normal((1, 6, F, 64)) / 8, "f16")
    q = O.narrow(g.standard_normal((3, 6, 2, 64)) / 8, "f16")
    shared = kb.Cache.wrap(to_dev(xk, "f16"), to_dev(xv, "f16"))
    per_row = kb.Cache.wrap(to_dev(np.repeat(xk, 3, 0), "f16"), to_dev(np.repeat(xv, 3, 0), "f16"))
    ws = _ws()
    a = kb.decode_attn_cross(to_dev(q, "f16"), shared, F, 0.125, ws=ws)
    b = kb.decode_attn_cross(to_dev(q, "f16"), per_row, F, 0.125, ws=ws)
    ox = O.ConcatCache(1, 6, 64, "f16"); ox.set_once(xk, xv)
    ref = O.attend_cross(q, ox, 0.125)
    assert max_err(a, ref) <= TOL["f16"] and max_err(b, ref) <= TOL["f16"]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,Hq,Hkv,N,F", [(3, 12, 4, 5, 1500), (7, 15, 5, 3, 300), (2, 14, 2, 11, 129)])
def test_cross_shared_grouped_rows(dtype, B, Hq, Hkv, N, F, plan):
    """Shared cross cache with grouped heads and several queries per row: the
    rows of a KV head are numbered (row, head in group, query), so both
    divisions of the row numbering (by N, by the group size) are non-trivial."""
    say(f"case: cross shared {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} F={F} plan={plan}")
    g = np.random.default_rng(B * 100 + N)
    xk = O.narrow(g.standard_normal((1, Hkv, F, 64)), dtype)
    xv = O.narrow(g.standard_normal((1, Hkv, F, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)) / 4, dtype)
    shared = kb.Cache.wrap(to_dev(xk, dtype), to_dev(xv, dtype))
    out = kb.decode_attn_cross(to_dev(q, dtype), shared, F, 0.125, ws=_ws())
    ox = O.ConcatCache(1, Hkv, 64, dtype)
    ox.set_once(xk, xv)
    assert max_err(out, O.attend_cross(q, ox, 0.125)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 5])
@pytest.mark.parametrize("F,waves,chunk", [
    (1500, 1, 192),   # 8 partials: the smallest merge load count, full
    (1100, 1, 128),   # 9: the next load count (16) with 7 partials unused
    (1500, 1, 96),    # 16
    (2100, 1, 128),   # 17: load count 32
    (1499, 2, 64),    # 24, ragged last split
    (1056, 1, 32),    # 33: load count 64
    (2048, 1, 32),    # 64: the most partials a merge takes
])
def test_cross_split_counts(dtype, N, F, waves, chunk):
    """Split counts on both sides of every load count of the merge (8, 16,
    32, 64 partials): the merge's max and sum run over the first 8, 16, 32
    or 64 lanes only, so each width is checked with every lane of it used
    and with lanes past the split count."""
    say(f"case: cross split counts {dtype} N={N} F={F} waves={waves} chunk={chunk}")
    g = np.random.default_rng(F + N)
    xk = O.narrow(g.standard_normal((1, 4, F, 64)), dtype)
    xv = O.narrow(g.standard_normal((1, 4, F, 64)), dtype)
    q = O.narrow(g.standard_normal((2, 4, N, 64)) / 4, dtype)
    shared = kb.Cache.wrap(to_dev(xk, dtype), to_dev(xv, dtype))
    with kb.plan_override(waves=waves, chunk=chunk):
        out = kb.decode_attn_cross(to_dev(q, dtype), shared, F, 0.125, ws=_ws())
    ox = O.ConcatCache(1, 4, 64, dtype)
    ox.set_once(xk, xv)
    assert max_err(out, O.attend_cross(q, ox, 0.125)) <= TOL[dtype]


# --------------------------------------------------- fused append + attend ----

@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,L,rope", [
    ("f16", 1, 20, 20, 1, 1, 0.0),          # first token
    ("f16", 1, 20, 20, 1, 300, 0.0),        # whisper decode step
    ("f16", 1, 20, 20, 5, 133, 0.0),        # verify block across a split boundary
    ("bf16", 8, 9, 3, 1, 700, 10000.0),     # GQA decode with rotary keys
    ("bf16", 8, 9, 3, 16, 530, 10000.0),    # largest fused block
    ("bf16", 2, 9, 3, 40, 100, 10000.0),    # long block: append then attend
    ("f32", 2, 4, 4, 3, 70, 10000.0),
])
def test_step_self_equals_append_then_attend(dtype, B, Hq, Hkv, N, L, rope, plan):
    """decode_step_self leaves the cache exactly as kv_append does and returns
    decode_attn_self's output, and both match the oracle."""
    say(f"case: step_self {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} L={L} rope={rope} plan={plan}")
    g = np.random.default_rng(L * 7 + N)
    S = L + 3
    k_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
    v_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    old, new = slice(0, L - N), slice(L - N, L)
    ws = _ws()
    c1 = kb.Cache(B, Hkv, S, TORCH_DTYPE[dtype])
    c2 = kb.Cache(B, Hkv, S, TORCH_DTYPE[dtype])
    if L > N:
        for c in (c1, c2):
            kb.kv_append(c, to_dev(k_all[:, :, old], dtype), to_dev(v_all[:, :, old], dtype), 0, rope)
    kb.kv_append(c1, to_dev(k_all[:, :, new], dtype), to_dev(v_all[:, :, new], dtype), L - N, rope)
    o1 = kb.decode_attn_self(to_dev(q, dtype), c1, L, 0.125, rope_base=rope, ws=ws)
    o2 = kb.decode_step_self(to_dev(q, dtype), to_dev(k_all[:, :, new], dtype),
                             to_dev(v_all[:, :, new], dtype), c2, L, 0.125, rope_base=rope, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(from_dev(c1.k, dtype)), bits(from_dev(c2.k, dtype)))
    assert np.array_equal(bits(from_dev(c1.v, dtype)), bits(from_dev(c2.v, dtype)))
    assert torch.equal(o1, o2)
    oc = O.ConcatCache(B, Hkv, 64, dtype)
    if L > N:
        oc.append(k_all[:, :, old], v_all[:, :, old], rope)
    oc.append(k_all[:, :, new], v_all[:, :, new], rope)
    assert _same_bits(from_dev(c2.k, dtype)[:, :, :L], oc.k, "appended keys")
    assert _same_bits(from_dev(c2.v, dtype)[:, :, :L], oc.v, "appended values")
    assert max_err(o2, O.attend_self(q, oc, 0.125, rope_base=rope)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,L", [
    ("f16", 1, 4, 4, 2, 33),      # new rows straddle two 32-key tiles
    ("f16", 2, 6, 2, 9, 95),      # grouped rows: early row tiles see only the first new rows
    ("f16", 1, 3, 3, 16, 16),     # every key new
    ("f16", 1, 5, 5, 16, 161),
    ("f32", 2, 4, 4, 7, 70),
    ("f32", 1, 2, 2, 16, 47),
])
@pytest.mark.parametrize("plan_name", ["stream", "w1", "w2_chunk64", "stream_chunk128"])
def test_step_self_streaming_new_rows(dtype, B, Hq, Hkv, N, L, plan_name):
    """Fused steps on the streaming kernel without rotation: the wave whose
    tile holds new rows takes them from k_new / v_new, row tile 0 writes them,
    and new rows past every query row of a row tile are copied after its key
    loop. The cache must hold exactly the appended rows (all N of them, with
    row tiles and splits cutting through the new rows and one-wave
    workgroups holding two tiles of them) and the output must match."""
    with kb.plan_override(**PLANS[plan_name]):
        say(f"case: streaming new rows {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} L={L} plan={plan_name}")
        g = np.random.default_rng([51, B, N, L, len(dtype)])
        k_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
        v_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
        q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
        old, new = slice(0, L - N), slice(L - N, L)
        c = kb.Cache(B, Hkv, L + 5, TORCH_DTYPE[dtype])
        if L > N:
            kb.kv_append(c, to_dev(k_all[:, :, old], dtype), to_dev(v_all[:, :, old], dtype), 0)
        out = kb.decode_step_self(to_dev(q, dtype), to_dev(k_all[:, :, new], dtype),
                                  to_dev(v_all[:, :, new], dtype), c, L, 0.125, ws=_ws())
        torch.cuda.synchronize()
        oc = O.ConcatCache(B, Hkv, 64, dtype)
        oc.append(k_all, v_all)
        assert _same_bits(from_dev(c.k, dtype)[:, :, :L], oc.k, "appended keys")
        assert _same_bits(from_dev(c.v, dtype)[:, :, :L], oc.v, "appended values")
        assert max_err(out, O.attend_self(q, oc, 0.125)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,L,rope", [
    ("bf16", 1, 9, 3, 1, 448, 10000.0),     # the rotary tile splits where the plain one does not
    ("bf16", 1, 9, 3, 1, 448, 0.0),
    ("f16", 1, 20, 20, 5, 448, 10000.0),
    ("f16", 4, 20, 20, 5, 300, 0.0),
    ("bf16", 2, 9, 3, 1, 1024, 10000.0),
    ("f32", 1, 4, 4, 1, 700, 10000.0),
])
def test_queried_workspace_suffices(dtype, B, Hq, Hkv, N, L, rope):
    """A workspace of exactly kvd_attn_workspace_bytes(B, Hq, N, len) serves
    decode_attn_self and decode_step_self at that length, rotary plans
    included, on the default plan."""
    say(f"case: exact workspace {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} L={L} rope={rope}")
    g = np.random.default_rng(L * 3 + N + B)
    k_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
    v_all = O.narrow(g.standard_normal((B, Hkv, L, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    old, new = slice(0, L - N), slice(L - N, L)
    nbytes = kb.attn_workspace_bytes(B, Hq, N, L)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    c1 = kb.Cache(B, Hkv, L, TORCH_DTYPE[dtype])
    c2 = kb.Cache(B, Hkv, L, TORCH_DTYPE[dtype])
    for c in (c1, c2):
        kb.kv_append(c, to_dev(k_all[:, :, old], dtype), to_dev(v_all[:, :, old], dtype), 0, rope)
    kb.kv_append(c1, to_dev(k_all[:, :, new], dtype), to_dev(v_all[:, :, new], dtype), L - N, rope)
    o1 = kb.decode_attn_self(to_dev(q, dtype), c1, L, 0.125, rope_base=rope, ws=ws)
    o2 = kb.decode_step_self(to_dev(q, dtype), to_dev(k_all[:, :, new], dtype),
                             to_dev(v_all[:, :, new], dtype), c2, L, 0.125, rope_base=rope, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    oc = O.ConcatCache(B, Hkv, 64, dtype)
    oc.append(k_all[:, :, old], v_all[:, :, old], rope)
    oc.append(k_all[:, :, new], v_all[:, :, new], rope)
    assert max_err(o1, O.attend_self(q, oc, 0.125, rope_base=rope)) <= TOL[dtype]


# ------------------------------------------ fused beam step (two caches) ----

@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,L,rope", [
    ("f16", 5, 20, 20, 1, 1, 0.0),          # first token: nothing to copy
    ("f16", 5, 20, 20, 1, 2, 0.0),
    ("f16", 5, 20, 20, 1, 300, 0.0),        # whisper beam step (split keys)
    ("f16", 5, 20, 20, 1, 448, 0.0),        # full cache
    ("bf16", 16, 20, 20, 1, 77, 0.0),       # 16 beams
    ("bf16", 4, 9, 3, 1, 700, 10000.0),     # grouped heads, rotary keys
    ("bf16", 3, 9, 3, 16, 530, 10000.0),    # largest fused block
    ("f16", 2, 8, 2, 5, 133, 0.0),          # draft block across a split boundary
    ("f32", 3, 4, 4, 3, 70, 10000.0),
    ("f32", 2, 4, 2, 1, 1100, 0.0),
])
def test_beam_step_equals_reorder_then_step(dtype, B, Hq, Hkv, N, L, rope, plan):
    """decode_step_self_beams(src -> dst) leaves dst exactly as a copy of
    src, kv_reorder and decode_step_self would (rows from L on untouched),
    leaves src as it was, returns the same output bit for bit on the same
    (streaming) plan, and matches the oracle."""
    say(f"case: beam step {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} L={L} rope={rope} plan={plan}")
    # the composition on the beam step's kernel (the streaming one)
    forced = dict(PLANS[plan], mfma=0)
    with kb.plan_override(**forced):
        _beam_step_case(dtype, B, Hq, Hkv, N, L, rope)


def _beam_step_case(dtype, B, Hq, Hkv, N, L, rope):
    g = np.random.default_rng(L * 11 + N + B)
    S = L + 5
    old, new = slice(0, L - N), slice(L - N, L)
    src_k = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    src_v = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    dst_k = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)   # stale rows of an older step
    dst_v = O.narrow(g.standard_normal((B, Hkv, S, 64)), dtype)
    k_new = O.narrow(g.standard_normal((B, Hkv, N, 64)), dtype)
    v_new = O.narrow(g.standard_normal((B, Hkv, N, 64)), dtype)
    q = O.narrow(g.standard_normal((B, Hq, N, 64)), dtype)
    par = g.integers(0, B, size=B).astype(np.int32)
    par[0] = B - 1
    pd = torch.from_numpy(par).cuda()
    src = kb.Cache.wrap(to_dev(src_k, dtype), to_dev(src_v, dtype))
    dst = kb.Cache.wrap(to_dev(dst_k, dtype), to_dev(dst_v, dtype))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_beam = kb.decode_step_self_beams(to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype),
                                       src, dst, pd, L, 0.125, rope_base=rope,
                                       dev_status=status)
    # the same step as reorder in place + fused step on a copy of src
    ref = kb.Cache.wrap(to_dev(src_k, dtype), to_dev(src_v, dtype))
    kb.kv_reorder(ref, pd, L - N)
    o_ref = kb.decode_step_self(to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype), ref,
                                L, 0.125, rope_base=rope)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    gk, gv = from_dev(dst.k, dtype), from_dev(dst.v, dtype)
    rk, rv = from_dev(ref.k, dtype), from_dev(ref.v, dtype)
    assert np.array_equal(bits(gk[:, :, :L]), bits(rk[:, :, :L]))
    assert np.array_equal(bits(gv[:, :, :L]), bits(rv[:, :, :L]))
    assert np.array_equal(bits(gk[:, :, L:]), bits(dst_k[:, :, L:]))     # rows past L untouched
    assert np.array_equal(bits(gv[:, :, L:]), bits(dst_v[:, :, L:]))
    assert np.array_equal(bits(from_dev(src.k, dtype)), bits(src_k))     # src only read
    assert np.array_equal(bits(from_dev(src.v, dtype)), bits(src_v))
    assert torch.equal(o_beam, o_ref)
    # the oracle: the parents' rows, then the append, then attention
    oc = O.ConcatCache(B, Hkv, 64, dtype)
    if L > N:
        oc.set_once(O.reorder(src_k[:, :, old], par), O.reorder(src_v[:, :, old], par))
    oc.append(k_new, v_new, rope)
    assert np.array_equal(bits(gk[:, :, old]), bits(oc.k[:, :, old]))   # copied rows
    assert np.array_equal(bits(gv[:, :, :L]), bits(oc.v))
    assert _same_bits(gk[:, :, new], oc.k[:, :, new], "new keys")
    assert max_err(o_beam, O.attend_self(q, oc, 0.125, rope_base=rope)) <= TOL[dtype]


def test_beam_step_bad_parent_reads_own_rows():
    say("case: beam step with parents outside [0, B)")
    dtype, B, H, S, L = "f16", 4, 20, 64, 40
    g = np.random.default_rng(5)
    src_k = O.narrow(g.standard_normal((B, H, S, 64)), dtype)
    src_v = O.narrow(g.standard_normal((B, H, S, 64)), dtype)
    k_new = O.narrow(g.standard_normal((B, H, 1, 64)), dtype)
    v_new = O.narrow(g.standard_normal((B, H, 1, 64)), dtype)
    q = O.narrow(g.standard_normal((B, H, 1, 64)), dtype)
    par = np.array([2, -1, 4, 0], dtype=np.int32)
    src = kb.Cache.wrap(to_dev(src_k, dtype), to_dev(src_v, dtype))
    dst = kb.Cache(B, H, S, torch.float16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kb.decode_step_self_beams(to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype),
                                    src, dst, torch.from_numpy(par).cuda(), L, 0.125,
                                    dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == -2
    eff = np.array([2, 1, 2, 0], dtype=np.int32)   # invalid parents: the beam's own rows
    oc = O.ConcatCache(B, H, 64, dtype)
    oc.set_once(O.reorder(src_k[:, :, :L - 1], eff), O.reorder(src_v[:, :, :L - 1], eff))
    oc.append(k_new, v_new)
    assert np.array_equal(bits(from_dev(dst.k, dtype)[:, :, :L]), bits(oc.k))
    assert np.array_equal(bits(from_dev(dst.v, dtype)[:, :, :L]), bits(oc.v))
    assert max_err(out, O.attend_self(q, oc, 0.125)) <= TOL[dtype]


def test_beam_step_ping_pong_whisper():
    """Beam search over 96 steps of two whisper layers (5 beams, 20 heads,
    fp16) with the caches used in turn: at each step the parents of the
    step's beams are read from one cache and written into the other with the
    new row. Caches and attention are checked against the oracle's reorder +
    append + attention along the way."""
    w = I.WHISPER_BEAM
    say("case: beam step ping-pong, 5 beams, 96 steps, two layers")
    steps = 96
    ws = _ws()
    worst = 0.0
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in (0, 1):
        pair = [kb.Cache(5, 20, 448, torch.float16), kb.Cache(5, 20, 448, torch.float16)]
        oc = O.ConcatCache(5, 20, 64, "f16")
        k_all, v_all = I.self_kv(w, l)
        kd, vd = to_dev(k_all, "f16"), to_dev(v_all, "f16")
        for s in range(steps):
            par = I.parents(w, s) if s > 0 else np.arange(5, dtype=np.int32)
            src, dst = pair[s % 2], pair[(s + 1) % 2]
            q = I.queries(w, l, s)
            o = kb.decode_step_self_beams(to_dev(q, "f16"), kd[:, :, s:s + 1].contiguous(),
                                          vd[:, :, s:s + 1].contiguous(), src, dst,
                                          torch.from_numpy(par).cuda(), s + 1, w.attn_scale,
                                          ws=ws, dev_status=status)
            if s > 0:
                oc.reorder(par)
            oc.append(k_all[:, :, s:s + 1], v_all[:, :, s:s + 1])
            if s % 8 == 7 or s < 3:
                e = max_err(o, O.attend_self(q, oc, w.attn_scale))
                worst = max(worst, e)
                assert e <= TOL["f16"], (l, s, e)
                assert np.array_equal(bits(from_dev(dst.k, "f16")[:, :, :s + 1]), bits(oc.k))
                assert np.array_equal(bits(from_dev(dst.v, "f16")[:, :, :s + 1]), bits(oc.v))
    assert int(status.item()) == 0
    say(f"beam ping-pong: worst max|err| {worst:.2e}")


def test_read_probe_reads_every_vector():
    """kvd_read_probe: a buffer whose only nonzero 16-byte vector folds to the
    probe's marker makes it store that word; an all-zero buffer stores nothing."""
    say("case: read probe")
    magic = 0x9E3779B9 - (1 << 32)   # as int32
    for n_vec, hot in ((1, 0), (4096 * 1024 + 7, 4096 * 1024 + 3), (100003, 77777)):
        buf = torch.zeros(n_vec * 4, dtype=torch.int32, device="cuda")
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        kb.read_probe(buf, None, n_vec * 16, sink)
        torch.cuda.synchronize()
        assert int(sink[0]) == 0
        buf[hot * 4] = magic
        kb.read_probe(buf, None, n_vec * 16, sink)
        torch.cuda.synchronize()
        assert int(sink[0]) == magic
        # the same vector in the second buffer
        other = torch.zeros_like(buf)
        sink.zero_()
        kb.read_probe(other, buf, n_vec * 16, sink)
        torch.cuda.synchronize()
        assert int(sink[0]) == magic


# ---------------------------------------------------------------------------
# Beam-search candidate scoring
# ---------------------------------------------------------------------------

def _beam_check(logits_stored, dtype, sums, eot, res, tol=1e-4):
    """Token choices must equal the oracle's wherever the oracle's candidate
    order has no near-tie (gap <= tol, where fp32 and fp64 may order
    differently); scores within tol."""
    ref = O.beam_select(O.widen(logits_stored, dtype), sums.astype(np.float64), eot)
    parent, token, score = (from_dev(res[k], None) for k in ("parent", "token", "score"))
    fc, fp, fs = (from_dev(res[k], None) for k in ("finished_count", "finished_parent", "finished_score"))
    B, K, _ = logits_stored.shape
    lp = O.log_softmax_rows(O.widen(logits_stored, dtype))
    for b in range(B):
        cands = []
        for j in range(K):
            top = np.lexsort((np.arange(lp.shape[-1]), -lp[b, j]))[:K + 1]
            cands += [sums[b, j] + lp[b, j, t] for t in top]
        walked = np.sort(np.array(cands))[::-1][:K + ref[3][b] + 1]   # the walk and the next one
        gaps = -np.diff(walked)
        # equal scores are ordered alike on both sides; gaps within fp32
        # rounding may not be
        tight = bool(np.any((gaps > 0) & (gaps <= tol)))
        if not tight:
            assert parent[b].tolist() == ref[0][b].tolist(), (b, parent[b], ref[0][b])
            assert token[b].tolist() == ref[1][b].tolist()
            assert fc[b] == ref[3][b] and fp[b, :fc[b]].tolist() == ref[4][b, :fc[b]].tolist()
            assert (fp[b, fc[b]:] == -1).all() and np.isnan(fs[b, fc[b]:]).all()
        for i in range(K):   # every chosen next beam is a real candidate with its score
            j, t = int(parent[b, i]), int(token[b, i])
            assert t != eot and abs(score[b, i] - (sums[b, j] + lp[b, j, t])) <= tol
        np.testing.assert_allclose(np.sort(score[b]), np.sort(ref[2][b]), rtol=0, atol=tol)
    return ref


@pytest.mark.parametrize("step", range(8))
def test_beam_select_whisper_shape(step):
    """5 beams over the 51865-token vocabulary, fp32 logits ~ N(0, 4)."""
    w = I.WHISPER_BEAM
    say(f"case: beam select step {step}")
    logits, sums = I.beam_logits(w, step)
    eot = 50256
    if step % 2:   # end-of-text the best candidate of the best-scoring beam
        j = int(np.argmax(sums[0]))
        logits[0, j, eot] = logits[0, j].max() + 3.0
    res = kb.beam_select(to_dev(logits, "f32"), torch.from_numpy(sums).cuda(), eot)
    torch.cuda.synchronize()
    ref = _beam_check(logits, "f32", sums, eot, res)
    if step % 2:
        assert ref[3][0] >= 1


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B,K,V", [(3, 1, 17), (2, 4, 4097), (1, 16, 20000), (2, 3, 4), (4, 8, 12289)])
def test_beam_select_shapes(dtype, B, K, V):
    say(f"case: beam select {dtype} B={B} K={K} V={V}")
    g = np.random.default_rng([21, B, K, V])
    logits = I.to_storage(g.standard_normal((B, K, V), dtype=np.float32) * 2, dtype)
    sums = (-g.random((B, K)) * 3).astype(np.float32)
    eot = V - 1
    res = kb.beam_select(to_dev(logits, dtype), torch.from_numpy(sums).cuda(), eot)
    torch.cuda.synchronize()
    _beam_check(logits, dtype, sums, eot, res)


@pytest.mark.parametrize("B,K,V", [(1, 16, 61440), (1, 1, 524288)])
def test_beam_select_largest_vocabulary(B, K, V):
    """The largest vocabulary each beam width takes: every lane of the merge
    holds 8 chunk entries."""
    say(f"case: beam select limit B={B} K={K} V={V}")
    g = np.random.default_rng([23, K, V])
    logits = (g.standard_normal((B, K, V)) * 2).astype(np.float32)
    sums = (-g.random((B, K)) * 3).astype(np.float32)
    res = kb.beam_select(to_dev(logits, "f32"), torch.from_numpy(sums).cuda(), V - 1)
    torch.cuda.synchronize()
    _beam_check(logits, "f32", sums, V - 1, res)


@pytest.mark.parametrize("kind", ["ties", "masked"])
def test_beam_select_ties_and_masks(kind):
    """Equal logits and equal scores (integer logits, equal running scores:
    lower token, then lower beam first), and masked vocabulary (-inf over half
    the tokens and over a whole 2048-token chunk, with -0.0 and +0.0 tied)."""
    say(f"case: beam select {kind}")
    B, K, V = 2, 5, 9000
    g = np.random.default_rng([24, len(kind)])
    logits = (g.standard_normal((B, K, V)) * 2).astype(np.float32)
    sums = (-g.random((B, K)) * 3).astype(np.float32)
    if kind == "ties":
        logits = np.round(logits)
        sums[:] = -1.0
    else:
        logits[g.random(logits.shape) < 0.5] = -np.inf
        logits[:, :, 2048:4096] = -np.inf
        logits[:, :, 5000:5003] = [0.0, -0.0, 0.0]
        logits[:, :, 6000:6003] = logits.max() + 1
    eot = 6001
    res = kb.beam_select(to_dev(logits, "f32"), torch.from_numpy(sums).cuda(), eot)
    torch.cuda.synchronize()
    _beam_check(logits, "f32", sums, eot, res)


def test_beam_select_repeated_calls_share_workspace():
    """The workspace counters reset themselves: ten calls in a row on one
    workspace, alternating shapes."""
    say("case: beam select repeated")
    ws = kb.workspace(max(kb.beam_workspace_bytes(2, 5, 51865), kb.beam_workspace_bytes(3, 2, 999)))
    for i in range(10):
        B, K, V = (2, 5, 51865) if i % 2 == 0 else (3, 2, 999)
        g = np.random.default_rng([22, i])
        logits = (g.standard_normal((B, K, V)) * 2).astype(np.float32)
        sums = (-g.random((B, K))).astype(np.float32)
        res = kb.beam_select(to_dev(logits, "f32"), torch.from_numpy(sums).cuda(), 3, ws=ws)
        torch.cuda.synchronize()
        _beam_check(logits, "f32", sums, 3, res)
