"""End-to-end speculative decoding on the device ("추측 디코딩으로 Whisper
추론 속도 2배 향상", "추측 디코딩이란?"): the emitted stream equals the main
model's greedy stream, token for token, with drafts accepted and rolled back
on the device; the caches hold every kept row at its position, and the last
verification pass attends exactly as the oracle does."""
import numpy as np
import pytest
import torch

import oracle as O
from kv_cached_decode_amd.specloop import SpecConfig, SpecLoop
from _util import TOL, max_err, say

pytestmark = pytest.mark.gpu

CFG = SpecConfig(main_layers=2, asst_layers=1, heads=4, s_max=128, frames=64, vocab=3000,
                 prompt=3, seed=11)


@pytest.fixture(scope="module")
def loop():
    return SpecLoop(CFG)


def _greedy_tokens(loop, start, count):
    am = O.argmax_rows(loop.LM.cpu().numpy().astype(np.float64))
    return [int(am[p]) for p in range(start, start + count)]


@pytest.mark.parametrize("graphs", [False, True])
def test_speculative_stream_equals_greedy(loop, graphs):
    say(f"case: speculative loop graphs={graphs}")
    if graphs:
        loop.capture()
    else:
        loop._graphs = {}
    n_it = loop.run()
    torch.cuda.synchronize()
    log, stream = loop.emitted()
    assert len(log) == n_it
    assert stream == _greedy_tokens(loop, CFG.prompt, len(stream))
    assert loop.tokens_emitted() == len(stream)
    P = log[:, 0].tolist()
    acc = log[:, 1].tolist()
    for i in range(1, len(P)):                       # P moves past every emitted token
        assert P[i] == P[i - 1] + acc[i - 1] + 1
    # drafts agree with the main model with probability 0.75: some accepted, some not
    assert 0 < sum(acc) < CFG.drafts * n_it
    # every kept row sits at its position: K / V of position p are table rows p
    L = P[-1] + loop.R
    for l in range(CFG.main_layers):
        assert torch.equal(loop.m_self[l].k[0, :, :L], loop.mk[l, :, :L])
        assert torch.equal(loop.m_self[l].v[0, :, :L], loop.mv[l, :, :L])
    # the last verification pass against the oracle
    for l in range(CFG.main_layers):
        c = O.ConcatCache(1, CFG.heads, 64, "f16")
        c.append(loop.mk[l, :, :L][None].cpu().numpy(), loop.mv[l, :, :L][None].cpu().numpy())
        q = loop.mq[l, :, P[-1]:L][None].cpu().numpy()
        assert max_err(loop.m_out[l], O.attend_self(q, c, 0.125)) <= TOL["f16"]


def test_greedy_loop_emits_the_same_stream(loop):
    say("case: greedy loop")
    loop.capture()
    n = loop.run_greedy(60)
    torch.cuda.synchronize()
    assert loop.greedy_stream() == _greedy_tokens(loop, CFG.prompt, n)


def test_full_large_v2_shape_stream_equals_greedy():
    """The same loop at the large-v2 shape (32-layer main model, 2-layer
    assistant, 20 heads, 448 positions, 1500 frames, vocab 51865), from
    captured graphs: the stream equals the greedy stream and the last
    verification pass of the first and last main layers matches the oracle."""
    cfg = SpecConfig()
    say("case: speculative loop at the large-v2 shape")
    big = SpecLoop(cfg)
    big.capture()
    n_it = big.run()
    torch.cuda.synchronize()
    log, stream = big.emitted()
    am = O.argmax_rows(big.LM.cpu().numpy().astype(np.float64))
    assert stream == [int(am[p]) for p in range(cfg.prompt, cfg.prompt + len(stream))]
    P = log[:, 0].tolist()
    acc = log[:, 1].tolist()
    say(f"{n_it} iterations, {len(stream)} tokens, mean accepted {np.mean(acc):.2f}")
    assert 0 < sum(acc) < cfg.drafts * n_it
    L = P[-1] + big.R
    for l in (0, cfg.main_layers - 1):
        assert torch.equal(big.m_self[l].k[0, :, :L], big.mk[l, :, :L])
        c = O.ConcatCache(1, cfg.heads, 64, "f16")
        c.append(big.mk[l, :, :L][None].cpu().numpy(), big.mv[l, :, :L][None].cpu().numpy())
        q = big.mq[l, :, P[-1]:L][None].cpu().numpy()
        assert max_err(big.m_out[l], O.attend_self(q, c, 0.125)) <= TOL["f16"]
