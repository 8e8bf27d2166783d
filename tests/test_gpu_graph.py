"""The whole step -- lookup, every shard's forward, the combine, a shard's backward and
the lookup gradient -- on a stream other than the default one, and captured in a HIP
graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, never synchronises and launches only on the stream it is
given, so it can be captured: a launch on any other stream while the capture is open
would fail the capture.  Each replay runs on new input values copied into the captured
buffers and must reproduce, bit for bit, an eager run on the same values (the kernels
reduce in a fixed order), with eager work and synchronisations between the replays.  The
eager results are pinned to the oracle on the first inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import assert_loss_close, dev_bf16, dev_i64, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


class _Step:
    """Buffers of one step of the small-LM workload (N=4096, H=512, V=6400, T=2), all
    allocated up front; ``run`` enqueues the step on the current stream."""

    def __init__(self, vp, inp):
        import torch
        wl = inp.wl
        self.vp, self.wl = vp, wl
        self.T, self.N, self.H = wl.T, wl.N, wl.H
        self.rng = [vp.vp_shard_range(wl.V, wl.T, t) for t in range(wl.T)]
        self.x = dev_bf16(inp.x)
        self.w = dev_bf16(inp.w)
        self.y = dev_i64(inp.targets)
        self.ids = dev_i64(inp.ids)
        self.dout = torch.empty((wl.embed_N, wl.H), dtype=torch.bfloat16, device="cuda")
        f = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")  # noqa: E731
        self.m, self.s, self.zy = f(self.T, self.N), f(self.T, self.N), f(self.T, self.N)
        self.loss, self.lse, self.mean = f(self.N), f(self.N), f(1)
        vs = self.rng[0][1] - self.rng[0][0]
        self.dx, self.dw, self.dw_embed = f(self.N, self.H), f(vs, self.H), f(vs, self.H)
        self.emb = torch.empty((wl.embed_N, wl.H), dtype=torch.bfloat16, device="cuda")
        self.ws_f = vp.alloc_workspace(vp.vp_lmhead_ce_fwd_workspace(self.N, self.H, 0, vs), "cuda")
        self.ws_b = vp.alloc_workspace(vp.vp_lmhead_ce_bwd_workspace(self.N, self.H, 0, vs), "cuda")
        self.ws_e = vp.alloc_workspace(vp.vp_embed_bwd_workspace(wl.embed_N, self.H, 0, vs), "cuda")
        self.g = oracle.mean_scale(inp.targets)

    def outputs(self):
        return (self.emb, self.m, self.s, self.zy, self.loss, self.lse, self.mean, self.dx,
                self.dw, self.dw_embed)

    def run(self):
        vp, (a0, b0) = self.vp, self.rng[0]
        w0 = self.w[a0:b0]
        vp.vp_embed_fwd(self.ids, w0, a0, b0, out=self.emb)
        for t, (a, b) in enumerate(self.rng):
            vp.vp_lmhead_ce_fwd(self.x, self.w[a:b], self.y, a, b, self.m[t], self.s[t], self.zy[t],
                                workspace=self.ws_f)
        vp.vp_ce_combine(self.m, self.s, self.zy, self.y, loss=self.loss, lse=self.lse,
                         loss_mean=self.mean)
        vp.vp_lmhead_ce_bwd(self.x, w0, self.y, self.lse, a0, b0, self.g, dx=self.dx, dw=self.dw,
                            workspace=self.ws_b)
        vp.vp_embed_bwd(self.ids, self.dout, a0, b0, dw=self.dw_embed, workspace=self.ws_e)


def _load(step, seed):
    """New input values into the step's buffers (eager copies on the current stream)."""
    import torch
    r = np.random.default_rng(seed)
    wl = step.wl
    step.x.copy_(dev_bf16(vp_inputs.f32_to_bf16_bits(
        r.standard_normal((wl.N, wl.H)).astype(np.float32))))
    step.w.copy_(dev_bf16(vp_inputs.f32_to_bf16_bits(
        r.standard_normal((wl.V, wl.H)).astype(np.float32) * np.float32(0.05))))
    step.y.copy_(dev_i64(r.integers(0, wl.V, wl.N)))
    step.ids.copy_(dev_i64(r.integers(-10, wl.V + 10, wl.embed_N)))
    step.dout.copy_(dev_bf16(vp_inputs.f32_to_bf16_bits(
        r.standard_normal((wl.embed_N, wl.H)).astype(np.float32))))
    step.dw_embed.zero_()   # the lookup gradient adds into it
    torch.cuda.synchronize()


def _snapshot(step):
    return [t.detach().clone() for t in step.outputs()]


def _same(a, b, what):
    import torch
    for k, (u, v) in enumerate(zip(a, b)):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v), \
            f"{what}: output {k} differs"


def test_side_stream_and_graph_replays(vp):
    import torch
    inp = vp_inputs.make_inputs("small_lm")
    step = _Step(vp, inp)
    seeds = [101, 102, 103, 104]

    # eager on the default stream, then on a side stream: same bits
    _load(step, seeds[0])
    step.run()
    torch.cuda.synchronize()
    ref = _snapshot(step)
    side = torch.cuda.Stream()
    _load(step, seeds[0])
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    side.synchronize()
    _same(_snapshot(step), ref, "side stream")

    # the eager results on these inputs against the oracle (loss of every token)
    x = vp_inputs.bf16_bits_to_f64(step.x.view(torch.int16).cpu().numpy().view(np.uint16))
    w = vp_inputs.bf16_bits_to_f64(step.w.view(torch.int16).cpu().numpy().view(np.uint16))
    y = step.y.cpu().numpy()
    loss, lse, _ = oracle.dense_ce(oracle.logits(x, w), y)
    assert_loss_close(host(ref[4]), loss)

    # capture: warm up on the side stream, then record the step
    graph = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()

    for k, seed in enumerate(seeds[1:] + seeds[:1]):
        _load(step, seed)
        step.run()                       # eager reference on these inputs
        torch.cuda.synchronize()
        want = _snapshot(step)
        _load(step, seed)
        graph.replay()
        torch.cuda.synchronize()
        _same(_snapshot(step), want, f"replay {k} (inputs {seed})")
        log(f"  replay {k} (inputs {seed}): bit-identical to the eager step")


def test_explicit_stream_argument(vp):
    """Calls given ``stream=`` a side stream that is not the current one, with the wrappers
    allocating their own workspaces and outputs.  Those are allocated on the side stream, so
    the caching allocator cannot hand a freed workspace to work queued on the current stream
    while the side stream's kernels still use it: work on the current stream right after
    the calls (allocations of the same sizes, filled with garbage) must not change the
    results, which equal the eager ones bit for bit."""
    import torch
    inp = vp_inputs.make_inputs("small_lm")
    step = _Step(vp, inp)
    _load(step, 105)
    wl = step.wl
    a0, b0 = step.rng[0]
    w0 = step.w[a0:b0]
    # eager on the current stream, library-allocated workspaces
    m, s, zy = (torch.empty((step.T, step.N), device="cuda") for _ in range(3))
    for t, (a, b) in enumerate(step.rng):
        vp.vp_lmhead_ce_fwd(step.x, step.w[a:b], step.y, a, b, m[t], s[t], zy[t])
    loss, lse, mean = vp.vp_ce_combine(m, s, zy, step.y)
    dx, dw = vp.vp_lmhead_ce_bwd(step.x, w0, step.y, lse, a0, b0, step.g)
    dwe = vp.vp_embed_bwd(step.ids, step.dout, a0, b0)
    torch.cuda.synchronize()
    want = [t.clone() for t in (m, s, zy, loss, lse, mean, dx, dw, dwe)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    m2, s2, zy2 = (torch.empty((step.T, step.N), device="cuda") for _ in range(3))
    for t, (a, b) in enumerate(step.rng):
        vp.vp_lmhead_ce_fwd(step.x, step.w[a:b], step.y, a, b, m2[t], s2[t], zy2[t], stream=side)
    loss2, lse2, mean2 = vp.vp_ce_combine(m2, s2, zy2, step.y, stream=side)
    dx2, dw2 = vp.vp_lmhead_ce_bwd(step.x, w0, step.y, lse2, a0, b0, step.g, stream=side)
    dwe2 = vp.vp_embed_bwd(step.ids, step.dout, a0, b0, stream=side)
    # the current stream reuses whatever its pool holds, at the workspaces' sizes
    vs = b0 - a0
    junk = [torch.empty(vp.vp_lmhead_ce_bwd_workspace(step.N, step.H, a0, b0), dtype=torch.uint8,
                        device="cuda").fill_(0xFF),
            torch.empty(vp.vp_lmhead_ce_fwd_workspace(step.N, step.H, a0, b0), dtype=torch.uint8,
                        device="cuda").fill_(0xFF),
            torch.empty(vp.vp_embed_bwd_workspace(wl.embed_N, step.H, a0, b0), dtype=torch.uint8,
                        device="cuda").fill_(0xFF),
            torch.full((vs, step.H), float("nan"), device="cuda")]
    side.synchronize()
    torch.cuda.synchronize()
    got = (m2, s2, zy2, loss2, lse2, mean2, dx2, dw2, dwe2)
    for k, (u, v) in enumerate(zip(got, want)):
        assert torch.equal(u, v), f"output {k} differs with stream= a side stream"
    del junk
    log("  every output bit-identical with stream= a side stream")
