"""GPU parity of vx_rope3d_apply against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from _helpers import ChunkCheck, bits, check, dev, host, say
from spatiotemporal_attention_vx_amd import binding, configs, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_workload(gpu_lib, name):
    import torch
    wl = configs.WORKLOADS[name]
    say(f"rope workload {name}: N={wl.n_tokens} H={wl.heads} d={wl.head_dim} {wl.dtype}")
    q, k, _ = inputs.attention_inputs(wl)
    tq, tk = dev(q), dev(k)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    binding.rope3d_apply(tq, tk, desc)
    torch.cuda.synchronize()
    # every token, in chunks that bound the host's fp64 copies
    for src, t, nm in ((q, tq, "q"), (k, tk, "k")):
        got_all = host(t)[0]
        acc = ChunkCheck(wl.dtype, f"rope {name} {nm}")
        for r0 in range(0, wl.n_tokens, 4096):
            rows = np.arange(r0, min(r0 + 4096, wl.n_tokens))
            x = inputs.values(src[0, rows]).astype(np.float64)
            acc.add(got_all[rows], oracle.rope3d_apply(x, wl.grid, wl.split, wl.theta,
                                                       wl.n_prefix, tokens=rows))
        acc.done()
        del got_all
    if wl.n_prefix:
        # text tokens are not touched at all
        np.testing.assert_array_equal(bits(tq)[0, :wl.n_prefix],
                                      q[0, :wl.n_prefix].view(np.int16))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(configs.SP_WORKLOADS))
def test_sp_share_workload(gpu_lib, name):
    """One GPU's share under sequence parallelism: all tokens of the grid with
    H/P heads (5 to 24), so a token row is narrow and each thread of a
    workgroup has only a few chunks; every token of Q and K against the
    oracle."""
    import torch
    wl = configs.SP_WORKLOADS[name]
    say(f"rope sp share {name}: N={wl.n_tokens} H={wl.heads} d={wl.head_dim}")
    q, k, _ = inputs.attention_inputs(wl)
    tq, tk = dev(q), dev(k)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    binding.rope3d_apply(tq, tk, desc)
    torch.cuda.synchronize()
    for src, t, nm in ((q, tq, "q"), (k, tk, "k")):
        got_all = host(t)[0]
        acc = ChunkCheck(wl.dtype, f"rope {name} {nm}")
        for r0 in range(0, wl.n_tokens, 8192):
            rows = np.arange(r0, min(r0 + 8192, wl.n_tokens))
            x = inputs.values(src[0, rows]).astype(np.float64)
            acc.add(got_all[rows], oracle.rope3d_apply(x, wl.grid, wl.split, wl.theta,
                                                       wl.n_prefix, tokens=rows))
        acc.done()


@pytest.mark.parametrize("dtype,grid,prefix,heads,d,batch,split", [
    ("f32", (1, 1, 1), 0, 1, 64, 1, (16, 24, 24)),
    ("f32", (2, 3, 5), 7, 3, 128, 2, (44, 42, 42)),
    ("bf16", (2, 3, 5), 7, 3, 128, 2, (44, 42, 42)),
    ("bf16", (3, 1, 4), 0, 5, 64, 1, (16, 24, 24)),
    ("bf16", (2, 2, 2), 1, 2, 8, 1, (2, 2, 4)),
    ("bf16", (2, 4, 3), 0, 1, 256, 3, (64, 96, 96)),
    ("bf16", (5, 2, 3), 3, 2, 96, 1, (0, 48, 48)),
    # wide token rows (8 or more chunks per thread of a 4-token workgroup): the
    # eight-deep load batches, with a ragged last workgroup, a prefix, batch 2
    ("bf16", (3, 5, 7), 2, 40, 128, 2, (44, 42, 42)),
    ("f32", (2, 3, 5), 3, 32, 128, 1, (44, 42, 42)),
])
def test_ragged(gpu_lib, dtype, grid, prefix, heads, d, batch, split):
    import torch
    n = prefix + grid[0] * grid[1] * grid[2]
    say(f"rope ragged {dtype} grid={grid} prefix={prefix} heads={heads} d={d} batch={batch}")
    g = np.random.default_rng(n * 31 + d)
    q = inputs.storage(g.standard_normal((batch, n, heads, d)).astype(np.float32), dtype)
    k = inputs.storage(g.standard_normal((batch, n, heads, d)).astype(np.float32), dtype)
    tq, tk = dev(q), dev(k)
    binding.rope3d_apply(tq, tk, binding.RopeDesc.of(grid, split, 10000.0, prefix))
    torch.cuda.synchronize()
    for src, t, nm in ((q, tq, "q"), (k, tk, "k")):
        got = host(t)
        for b in range(batch):
            ref = oracle.rope3d_apply(inputs.values(src[b]).astype(np.float64), grid, split,
                                      10000.0, prefix)
            check(got[b], ref, dtype, f"rope ragged {nm}[{b}]")


def test_single_tensor_calls_match_pair_call(gpu_lib):
    import torch
    say("rope q-only / k-only")
    wl = configs.WORKLOADS["small"]
    q, k, _ = inputs.attention_inputs(wl)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    tq, tk = dev(q), dev(k)
    binding.rope3d_apply(tq, tk, desc)
    tq1, tk1 = dev(q), dev(k)
    binding.rope3d_apply(tq1, None, desc)
    binding.rope3d_apply(None, tk1, desc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(tq1), bits(tq))
    np.testing.assert_array_equal(bits(tk1), bits(tk))


def test_f32_norm_preserved(gpu_lib):
    import torch
    say("rope f32 norm")
    wl = configs.WORKLOADS["tiny"]
    q, k, _ = inputs.attention_inputs(wl)
    tq = dev(q)
    binding.rope3d_apply(tq, None, binding.RopeDesc.of(wl.grid, wl.split, wl.theta))
    torch.cuda.synchronize()
    got = host(tq).astype(np.float64)
    x = inputs.values(q).astype(np.float64)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = got[..., 0::2] ** 2 + got[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=2e-6, atol=1e-6)
