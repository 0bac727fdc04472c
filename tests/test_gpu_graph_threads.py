"""The library under a captured HIP graph and from several host threads
(needs a GPU).

Every entry point (forward, split-KV forward, backward, FP8 forward, row
softmax) allocates nothing, keeps no state and only enqueues on the
caller's stream, so (a) a sequence of calls can be captured into a HIP graph
and replayed, and (b) host threads can call it at the same time on their own
streams. Both are checked against the same calls made eagerly, bit for bit:
the kernels are deterministic (no atomics, fixed reduction order).

The graph is replayed several times with eager work and synchronisations in
between, inputs are changed between replays (the graph reads them through
the same device addresses), and every replay is compared with an eager run
on the same inputs.
"""
import threading

import numpy as np
import pytest
import torch

from online_softmax_03_amd import attention as A
from online_softmax_03_amd import capi
from online_softmax_03_amd import softmax as S
from online_softmax_03_amd import workloads as W
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(seed, B=2, H=4, N=300, d=128):
    w = W.BY_NAME["bf16_causal_n8192_d128"].with_shape(B=B, H=H, N=N, d=d, seed=seed)
    x = W.generate(w)
    return {k: x[k].to(DEV) for k in ("q", "k", "v")}, w


class _Buffers:
    """Preallocated inputs and outputs of one fwd + split-KV fwd + bwd +
    FP8 fwd + row-softmax sequence (a graph may not allocate)."""

    def __init__(self, B=2, H=4, N=300, d=128):
        x, self.w = _inputs(1, B, H, N, d)
        self.q, self.k, self.v = x["q"].clone(), x["k"].clone(), x["v"].clone()
        shape, dt = self.q.shape, self.q.dtype
        self.o = torch.empty(shape, dtype=dt, device=DEV)
        self.lse = torch.empty(shape[:3], dtype=torch.float32, device=DEV)
        self.o2 = torch.empty_like(self.o)
        self.lse2 = torch.empty_like(self.lse)
        self.splits = 3
        self.ws = torch.empty(capi.fa_splitkv_workspace_bytes(B, H, N, d, self.splits), dtype=torch.uint8,
                              device=DEV)
        self.dout = W.generate_dout(self.w).to(DEV)
        self.grads = tuple(torch.empty(shape, dtype=dt, device=DEV) for _ in range(3))
        self.bws = torch.empty(capi.fa_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=DEV)
        self.w8 = W.FP8_BY_NAME["fp8_causal_n8192_d128"].with_shape(B=B, H=H, N=N, d=d, seed=1)
        x8 = W.generate(self.w8)
        self.q8, self.k8, self.v8 = (x8[n].to(DEV).clone() for n in ("q", "k", "v"))
        self.o8 = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        self.lse8 = torch.empty_like(self.lse)
        self.sx = torch.randn(64, 1000, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
        self.sy = torch.empty_like(self.sx)
        self.slse = torch.empty(64, dtype=torch.float32, device=DEV)

    def load(self, seed):
        x, _ = _inputs(seed, *self.q.shape)
        self.q.copy_(x["q"])
        self.k.copy_(x["k"])
        self.v.copy_(x["v"])
        x8 = W.generate(self.w8.with_shape(seed=seed))
        for dst, n in ((self.q8, "q"), (self.k8, "k"), (self.v8, "v")):
            dst.copy_(x8[n])

    def run(self):
        sc = self.w.scale
        A.attention_fwd(self.q, self.k, self.v, scale=sc, causal=True, out=self.o, lse=self.lse)
        A.attention_fwd(self.q, self.k, self.v, scale=sc, causal=True, out=self.o2, lse=self.lse2,
                        num_splits=self.splits, workspace=self.ws)
        A.attention_bwd(self.q, self.k, self.v, self.o, self.dout, self.lse, scale=sc, causal=True,
                        workspace=self.bws, out=self.grads)
        dq, dk, dv = self.w8.descale
        A.attention_fwd_fp8(self.q8, self.k8, self.v8, scale=self.w8.scale, descale_q=dq, descale_k=dk,
                            descale_v=dv, causal=True, out=self.o8, lse=self.lse8)
        S.softmax_rows(self.sx, out=self.sy, lse=self.slse)

    def outputs(self):
        return [t.detach().clone() for t in (self.o, self.lse, self.o2, self.lse2, *self.grads, self.o8, self.lse8,
                                             self.sy, self.slse)]


def test_graph_replays_match_eager():
    buf = _Buffers()
    # warm up on a side stream (as torch recommends before capture)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        buf.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        buf.run()
    torch.cuda.synchronize()
    for rep, seed in enumerate((11, 12, 11, 13)):
        buf.load(seed)
        g.replay()
        torch.cuda.synchronize()
        got = buf.outputs()
        # eager work between replays, on the same buffers
        for t in got[:2]:
            t.mul_(1.0)
        buf.run()
        torch.cuda.synchronize()
        want = buf.outputs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep} (inputs {seed}): output {i} differs from the eager run"
        log(f"  replay {rep} with inputs {seed}: identical to eager")


def test_concurrent_host_threads_on_own_streams():
    n = 4
    cases = [_inputs(100 + i, B=1, H=3, N=257 + 64 * i)[0] for i in range(n)]
    scale = 1.0 / np.sqrt(128)

    def call(x, out, lse, stream):
        with torch.cuda.stream(stream):
            A.attention_fwd(x["q"], x["k"], x["v"], scale=scale, causal=True, out=out, lse=lse)

    # serial reference
    ref = []
    for x in cases:
        o, l = A.attention_fwd(x["q"], x["k"], x["v"], scale=scale, causal=True)
        ref.append((o, l))
    torch.cuda.synchronize()
    outs = [(torch.full_like(o, float("nan")), torch.full_like(l, float("nan"))) for o, l in ref]
    streams = [torch.cuda.Stream() for _ in range(n)]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            for _ in range(5):
                call(cases[i], outs[i][0], outs[i][1], streams[i])
        except Exception as e:  # pragma: no cover - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(n):
        assert torch.equal(outs[i][0], ref[i][0]) and torch.equal(outs[i][1], ref[i][1]), f"thread {i} differs"
    log(f"  {n} threads x 5 calls on their own streams: identical to the serial results")
