"""The selection scheme of the beam-scoring kernel, restated in NumPy and
checked against the oracle on the CPU (no GPU, no HIP code): order keys,
the K + 1 best of each 2048-logit chunk, their merge per beam, and the walk
placed in parallel (a candidate's slot follows from how many candidates, and
how many end-of-text candidates, rank before it). Beam-search update steps of
"Whisper のデコーダー内部：Beam Search、Logit フィルター、KV キャッシュ"."""
import numpy as np
import pytest

import oracle as O

CHUNK = 2048
MAX_CAND = 16 * 17


def order_bits(v: np.ndarray) -> np.ndarray:
    """uint64 holding 32-bit unsigned integers ordered as the float32 values
    (-0.0 taken as +0.0)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, 0, u)
    neg = (u & 0x80000000) != 0
    return np.where(neg, (~u) & 0xFFFFFFFF, u | 0x80000000)


def order_value(k: int) -> float:
    b = (k & 0x7FFFFFFF) if (k & 0x80000000) else (~k & 0xFFFFFFFF)
    return float(np.uint32(b).view(np.float32))


def top_keys(keys: np.ndarray, n: int) -> list:
    ks = sorted((int(k) for k in keys if k), reverse=True)
    return (ks + [0] * n)[:n]


def scheme(logits: np.ndarray, sums: np.ndarray, eot: int):
    B, K, V = logits.shape
    KP = K + 1
    chunks = (V + CHUNK - 1) // CHUNK
    parent = np.zeros((B, K), int)
    token = np.zeros((B, K), int)
    score = np.zeros((B, K), np.float32)
    fin_count = np.zeros(B, int)
    fin_parent = np.full((B, K), -1)
    for b in range(B):
        cand = np.zeros(K * KP, dtype=np.uint64)
        eot_key = np.zeros(K, dtype=np.uint64)
        for j in range(K):
            recs = []
            for c in range(chunks):
                x = logits[b, j, c * CHUNK:(c + 1) * CHUNK].astype(np.float32)
                cm = np.float32(x.max())
                ref = np.float32(0) if cm == -np.inf else cm
                cs = np.float32(np.exp(x - ref, dtype=np.float32).sum(dtype=np.float32))
                idx = np.arange(c * CHUNK, c * CHUNK + len(x), dtype=np.uint64)
                keys = (order_bits(x) << np.uint64(32)) | (~idx & np.uint64(0xFFFFFFFF))
                recs.append((cm, cs, top_keys(keys, KP)))
            M = max(r[0] for r in recs)
            S = np.float32(sum(np.float32(r[1] * np.exp(np.float32(r[0] - M))) for r in recs))
            lse = np.float32(M + np.log(S))
            best = top_keys(np.array([k for r in recs for k in r[2]], dtype=np.uint64), KP)
            for r, k in enumerate(best):
                t = j * KP + r
                v = order_value(k >> 32)
                tok = (~k) & 0xFFFFFFFF
                s = np.float32(np.float32(sums[b, j]) + np.float32(np.float32(v) - lse))
                key = (int(order_bits(s)) << 32) | ((MAX_CAND - 1 - t) << 23) | tok
                cand[t] = np.uint64(key)
                if tok == eot:
                    eot_key[j] = np.uint64(key)
        for t in range(K * KP):
            me = cand[t]
            rank = int((cand > me).sum())
            eots = int((eot_key > me).sum())
            if rank - eots < K:
                tok = int(me) & 0x7FFFFF
                if tok == eot:
                    fin_parent[b, eots] = t // KP
                    fin_count[b] += 1
                else:
                    parent[b, rank - eots] = t // KP
                    token[b, rank - eots] = tok
                    score[b, rank - eots] = order_value(int(me) >> 32)
    return parent, token, score, fin_count, fin_parent


@pytest.mark.parametrize("case", range(12))
def test_beam_scheme_matches_oracle(case):
    rng = np.random.default_rng([31, case])
    B, K = 1 + case % 2, 1 + case % 5
    V = int(rng.integers(K + 1, 7000))
    kind = case % 4
    x = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    sums = (-rng.random((B, K)) * 3).astype(np.float32)
    if kind == 1:     # equal logits within rows, equal running scores
        x = np.round(x)
        sums[:] = -1.0
    elif kind == 2:   # masked vocabulary, -0.0 tied with +0.0
        x[rng.random(x.shape) < 0.5] = -np.inf
        x[..., :K + 1] = 0.0
        x[..., 1] = -0.0
    elif kind == 3:   # a whole chunk of -inf
        x[..., :min(V, CHUNK)] = -np.inf
        x[..., -K - 1:] = 1.0
    eot = int(rng.integers(0, V))
    if case % 3 == 0:
        x[:, :, eot] = x.max() + 1
    ref = O.beam_select(x.astype(np.float64), sums.astype(np.float64), eot)
    got = scheme(x, sums, eot)
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1], ref[1])
    np.testing.assert_allclose(got[2], ref[2], atol=1e-4, rtol=0)
    np.testing.assert_array_equal(got[3], ref[3])
    for b in range(B):
        np.testing.assert_array_equal(got[4][b, :got[3][b]], ref[4][b, :ref[3][b]])
