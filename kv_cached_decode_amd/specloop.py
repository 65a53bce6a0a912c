"""A device-resident speculative decoding loop built from the entry points
("추측 디코딩으로 Whisper 추론 속도 2배 향상", section "추측 디코딩이란?":
an assistant drafts N tokens one at a time, the main model scores all of them
in one pass, keeps them up to the first one that differs from its own choice
and puts its own token there).

The models are synthetic: the q / k / v rows (and cross queries) of the token
at position p come from seeded per-position tables, and so do the logits
(main: LM[p], assistant: LA[p], whose argmax agrees with LM's with a set
probability). What runs is the real decode path: per iteration the assistant
runs N + 1 single-token steps (decode_step_self_ragged + decode_attn_cross
per layer, then verify_accept_masked with no drafts as its greedy argmax) and
the main model one pass over N + 1 rows (the last emitted token and the N
drafts) followed by verify_accept. The position P of the last emitted token
lives on the device, every length derives from it, and one small update
P += accepted + 1 closes the iteration, so the two captured graphs replay
back to back with no host round trip; rolled-back cache rows are simply
written over by the next iteration.

Test and benchmark harness: it stages inputs with torch ops (gathers from
the tables) and calls only the C-ABI entry points for the decode work.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as kb


@dataclass
class SpecConfig:
    main_layers: int = 32
    asst_layers: int = 2
    heads: int = 20
    s_max: int = 448
    frames: int = 1500
    vocab: int = 51865
    drafts: int = 5
    prompt: int = 4          # tokens in both caches before the first iteration
    p_agree: float = 0.75    # P(argmax LA[p] == argmax LM[p])
    seed: int = 7


class SpecLoop:
    def __init__(self, cfg: SpecConfig, device: str = "cuda"):
        self.cfg = c = cfg
        g = torch.Generator(device=device).manual_seed(c.seed)
        rn = lambda *sh: (torch.randn(*sh, generator=g, device=device) / 8).half()
        H, D, N = c.heads, 64, c.drafts
        self.R = N + 1
        T = c.s_max + self.R
        self.T = T
        # per-position tables: main [layers, H, T, D] (a gather of R positions
        # is the [layers, H, R, D] operand itself), assistant [layers, T, H, D]
        # (one position of one layer is a contiguous [H, D] row)
        self.mq, self.mk, self.mv, self.mx = (rn(c.main_layers, H, T, D) for _ in range(4))
        self.aq, self.ak, self.av, self.ax = (rn(c.asst_layers, T, H, D) for _ in range(4))
        self.LM = torch.randn(T, c.vocab, generator=g, device=device) * 2
        greedy = self.LM.argmax(-1)
        LA = torch.randn(T, c.vocab, generator=g, device=device) * 2
        agree = torch.rand(T, generator=g, device=device) < c.p_agree
        shift = torch.randint(1, c.vocab, (T,), generator=g, device=device)
        pick = torch.where(agree, greedy, (greedy + shift) % c.vocab)
        LA[torch.arange(T, device=device), pick] = LA.max(-1).values + 1.0
        self.LA = LA
        # caches
        self.m_self = [kb.Cache(1, H, c.s_max, torch.float16, device) for _ in range(c.main_layers)]
        self.a_self = [kb.Cache(1, H, c.s_max, torch.float16, device) for _ in range(c.asst_layers)]
        self.m_cross, self.a_cross = [], []
        for lst, n in ((self.m_cross, c.main_layers), (self.a_cross, c.asst_layers)):
            for _ in range(n):
                x = kb.Cache(1, H, c.frames, torch.float16, device)
                x.k.copy_(rn(1, H, c.frames, D))
                x.v.copy_(rn(1, H, c.frames, D))
                lst.append(x)
        # device state and buffers
        self.P = torch.zeros(1, dtype=torch.int32, device=device)
        self.it = torch.zeros(1, dtype=torch.int64, device=device)
        self.draft = torch.zeros(1, N, dtype=torch.int32, device=device)
        self.acc = torch.zeros(1, dtype=torch.int32, device=device)
        self.nxt = torch.zeros(1, dtype=torch.int32, device=device)
        self.scratch = torch.zeros(2, dtype=torch.int32, device=device)
        self.ar = torch.arange(self.R, dtype=torch.int32, device=device)
        self.m_out = torch.empty(c.main_layers, 1, H, self.R, D, dtype=torch.float32, device=device)
        self.m_outx = torch.empty_like(self.m_out)
        self.a_out = torch.empty(c.asst_layers, 1, H, 1, D, dtype=torch.float32, device=device)
        self.a_outx = torch.empty_like(self.a_out)
        span = max(c.s_max, c.frames)
        self.ws = kb.workspace(max(kb.attn_workspace_bytes(1, H, self.R, span),
                                   kb.attn_workspace_bytes(1, H, 1, span),
                                   kb.verify_workspace_bytes(1, self.R, c.vocab)), device)
        self.max_iters = (c.s_max - self.R - c.prompt) // self.R + 1
        self.log = torch.zeros(self.max_iters, 3 + N, dtype=torch.int32, device=device)
        self.g_out = torch.empty(c.main_layers, 1, H, 1, D, dtype=torch.float32, device=device)
        self.g_outx = torch.empty_like(self.g_out)
        self.max_greedy = c.s_max - c.prompt
        self.glog = torch.zeros(self.max_greedy, dtype=torch.int32, device=device)
        self._graphs = {}

    # -- one iteration, as launched (and captured) ------------------------
    def _assistant(self):
        c = self.cfg
        rows = (self.P + self.ar).long()                      # positions P .. P + N
        lens = self.P + 1 + self.ar                           # after each step's append
        # every step's inputs in one gather per table: [layers, R, H, D], [R, V]
        q, k, v, x = (t.index_select(1, rows) for t in (self.aq, self.ak, self.av, self.ax))
        logits = self.LA.index_select(0, rows)
        for j in range(self.R):
            for l in range(c.asst_layers):
                one = lambda t: t[l, j].view(1, c.heads, 1, 64)
                kb.decode_step_self_ragged(one(q), one(k), one(v), self.a_self[l], lens[j:j + 1],
                                           c.s_max, 0.125, out=self.a_out[l], ws=self.ws)
                kb.decode_attn_cross(one(x), self.a_cross[l], c.frames, 0.125,
                                     out=self.a_outx[l], ws=self.ws)
            if j < c.drafts:   # greedy draft for position P + j + 1
                kb.verify_accept_masked(logits[j].view(1, 1, c.vocab), None,
                                        accept_len=self.scratch[0:1],
                                        next_token=self.draft[0, j:j + 1], ws=self.ws)

    def _main(self):
        c = self.cfg
        rows = (self.P + self.ar).long()                      # positions P .. P + N
        lens = self.P + self.R
        q, k, v, x = (t.index_select(2, rows) for t in (self.mq, self.mk, self.mv, self.mx))
        for l in range(c.main_layers):                        # [layers, H, R, D]
            kb.decode_step_self_ragged(q[l:l + 1], k[l:l + 1], v[l:l + 1], self.m_self[l], lens,
                                       c.s_max, 0.125, out=self.m_out[l], ws=self.ws)
            kb.decode_attn_cross(x[l:l + 1], self.m_cross[l], c.frames, 0.125,
                                 out=self.m_outx[l], ws=self.ws)
        logits = self.LM.index_select(0, rows).view(1, self.R, c.vocab)
        kb.verify_accept(logits, self.draft, ws=self.ws, accept_len=self.acc, next_token=self.nxt)
        # record (P, accepted, next, drafts) and move P past the emitted tokens
        entry = torch.cat([self.P, self.acc, self.nxt, self.draft[0]])
        self.log.index_copy_(0, self.it, entry.view(1, -1))
        self.it.add_(1)
        self.P.add_(self.acc + 1)

    def iteration(self):
        self._assistant()
        self._main()

    def greedy_iteration(self):
        """The main model alone, one token per pass: append + attend the token
        at P, argmax of LM[P] is the token at P + 1."""
        c = self.cfg
        rows = self.P.long()
        lens = self.P + 1
        q, k, v, x = (t.index_select(2, rows) for t in (self.mq, self.mk, self.mv, self.mx))
        for l in range(c.main_layers):                        # [layers, H, 1, D]
            kb.decode_step_self_ragged(q[l:l + 1], k[l:l + 1], v[l:l + 1], self.m_self[l], lens,
                                       c.s_max, 0.125, out=self.g_out[l], ws=self.ws)
            kb.decode_attn_cross(x[l:l + 1], self.m_cross[l], c.frames, 0.125,
                                 out=self.g_outx[l], ws=self.ws)
        logits = self.LM.index_select(0, rows).view(1, 1, c.vocab)
        kb.verify_accept_masked(logits, None, ws=self.ws, accept_len=self.scratch[0:1],
                                next_token=self.nxt)
        self.glog.index_copy_(0, self.it, self.nxt)
        self.it.add_(1)
        self.P.add_(1)

    # -- setup and runs ----------------------------------------------------
    def reset(self):
        """Both caches hold the prompt (positions [0, prompt)); P = prompt."""
        c = self.cfg
        p = c.prompt
        for l, cache in enumerate(self.m_self):
            kb.kv_append(cache, self.mk[l, :, :p].unsqueeze(0).contiguous(),
                         self.mv[l, :, :p].unsqueeze(0).contiguous(), 0)
        for l, cache in enumerate(self.a_self):
            kb.kv_append(cache, self.ak[l, :p].transpose(0, 1).unsqueeze(0).contiguous(),
                         self.av[l, :p].transpose(0, 1).unsqueeze(0).contiguous(), 0)
        self.P.fill_(p)
        self.it.zero_()
        self.log.zero_()
        self.glog.zero_()

    def capture(self):
        """Capture one speculative iteration and one greedy step as graphs
        (replayed with the device P)."""
        for name, fn in (("spec", self.iteration), ("greedy", self.greedy_iteration)):
            self.reset()
            stream = torch.cuda.Stream()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                fn()   # warm: plans, code objects
                self.reset()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    fn()
            torch.cuda.current_stream().wait_stream(stream)
            torch.cuda.synchronize()
            self._graphs[name] = g

    def replay(self, iters: int, greedy: bool = False):
        """`iters` captured iterations (or greedy steps) from the current
        state, back to back; the caller keeps them within max_iters /
        max_greedy of a reset."""
        g = self._graphs["greedy" if greedy else "spec"]
        for _ in range(iters):
            g.replay()

    def run(self, iters: int | None = None):
        """Reset, then `iters` speculative iterations back to back (default:
        as many as can never pass the cache capacity, N + 1 positions per
        iteration at most). Returns the number of iterations."""
        n = self.max_iters if iters is None else min(iters, self.max_iters)
        self.reset()
        for _ in range(n):
            if "spec" in self._graphs:
                self._graphs["spec"].replay()
            else:
                self.iteration()
        return n

    def run_greedy(self, steps: int | None = None):
        """Reset, then `steps` greedy steps back to back (one token each)."""
        n = self.max_greedy if steps is None else min(steps, self.max_greedy)
        self.reset()
        for _ in range(n):
            if "greedy" in self._graphs:
                self._graphs["greedy"].replay()
            else:
                self.greedy_iteration()
        return n

    def greedy_stream(self):
        return self.glog[: int(self.it.item())].cpu().tolist()

    def emitted(self):
        """Host copy of the log: per iteration (P, accepted n, next token,
        drafts), and the emitted stream: drafts[:n] + [next] each iteration."""
        log = self.log[: int(self.it.item())].cpu()
        stream = []
        for row in log.tolist():
            n = row[1]
            stream += row[3:3 + n] + [row[2]]
        return log, stream

    def tokens_emitted(self) -> int:
        return int(self.P.item()) - self.cfg.prompt
