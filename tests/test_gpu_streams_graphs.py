"""The library's stream contract on the GPU: calls enqueue on the stream they
are given and keep no state between calls, so (i) the hot path run on two
streams at once gives each stream the same bits as running it alone, and
(ii) the whole step (AdaLN, RoPE on K, attention with Q rotated on load)
can be captured in a HIP graph (the library neither allocates nor
synchronises) and every replay gives the eager result bit for bit.

The graph is replayed several times with eager work and synchronisations
between the replays, and each replay is checked.  K is rotated in place, so
the captured step first copies the unrotated K into the working buffer with
an elementwise kernel (a multiply by one: no memset or memcpy node).
"""
import numpy as np
import pytest

from _helpers import bits, dev, say
from spatiotemporal_attention_vx_amd import binding, configs, inputs

pytestmark = pytest.mark.gpu


def _tensors(wl, seed):
    import torch
    x, sh, sc = inputs.adaln_inputs(wl, seed)
    q, k, v = inputs.attention_inputs(wl, seed)
    t = {n: dev(a) for n, a in (("x", x), ("sh", sh), ("sc", sc), ("q", q), ("k0", k), ("v", v))}
    t["k"] = torch.empty_like(t["k0"])
    t["y"] = torch.empty_like(t["x"])
    t["o"] = torch.empty_like(t["q"])
    t["lse"] = torch.empty((wl.batch, wl.heads, wl.n_tokens), device="cuda")
    return t


def _step(wl, t, stream):
    import torch
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    with torch.cuda.stream(stream):
        torch.mul(t["k0"], 1, out=t["k"])
        binding.adaln_modulate(t["x"], t["sh"], t["sc"], t["y"], wl.eps, stream=stream)
        binding.rope3d_apply(None, t["k"], desc, stream=stream)
        binding.flash_attn_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], 0.0, desc, stream=stream)


def _snapshot(t):
    return {n: bits(t[n]) for n in ("y", "k", "o", "lse")}


def _same(a, b, what):
    for n in a:
        assert np.array_equal(a[n], b[n]), f"{what}: {n} differs"


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_two_streams_at_once_match_each_alone(gpu_lib, name):
    import torch
    wl = configs.WORKLOADS[name]
    say(f"two streams {name}")
    ta, tb = _tensors(wl, 1), _tensors(wl, 2)
    s0 = torch.cuda.current_stream()
    _step(wl, ta, s0)
    torch.cuda.synchronize()
    alone_a = _snapshot(ta)
    _step(wl, tb, s0)
    torch.cuda.synchronize()
    alone_b = _snapshot(tb)
    for t in (ta, tb):
        for n in ("y", "k", "o", "lse"):
            t[n].fill_(float("nan"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    for _ in range(3):          # interleave the two streams' launches
        _step(wl, ta, sa)
        _step(wl, tb, sb)
    torch.cuda.synchronize()
    _same(_snapshot(ta), alone_a, "stream a")
    _same(_snapshot(tb), alone_b, "stream b")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_graph_replays_match_eager(gpu_lib, name):
    import torch
    wl = configs.WORKLOADS[name]
    say(f"graph capture {name}")
    t = _tensors(wl, 3)
    side = torch.cuda.Stream()
    # eager reference on the stream the graph is captured on
    _step(wl, t, side)
    torch.cuda.synchronize()
    eager = _snapshot(t)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _step(wl, t, side)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        for n in ("y", "k", "o", "lse"):
            t[n].fill_(float("nan"))
        scratch.mul_(1.5).add_(1.0)         # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_snapshot(t), eager, f"replay {r}")
    del graph
