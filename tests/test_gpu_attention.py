"""GPU parity of vx_flash_attn_fwd (and the RoPE + attention path) against
the fp64 oracle."""
import numpy as np
import pytest

import oracle
from _helpers import ChunkCheck, bits, check, dev, host, say
from spatiotemporal_attention_vx_amd import binding, configs, inputs

pytestmark = pytest.mark.gpu

# LSE bounds, max abs against the fp64 oracle, fixed (no term depends on the
# inputs).  bf16: half of the 2e-2 bound for bf16 results.  A call that asks
# for the LSE keeps Q exactly as stored and applies the softmax scale in fp32,
# so the LSE carries only fp32 rounding and the bf16 rounding of the weights
# in the row sum (at most 2^-9 relative, 2e-3 in the log); after RoPE the
# rotated Q and K are the path's own bf16 values while the oracle rotates in
# fp64, which moves a score by about 1.6e-3 (RMS, unit inputs) and the LSE by
# a weighted mean of those moves.
LSE_TOL = {"f32": 1e-5, "bf16": 1e-2}


def _rand(shape, dtype, seed):
    g = np.random.default_rng(seed)
    return inputs.storage(g.standard_normal(shape).astype(np.float32), dtype)


def _attn(q, k, v, with_lse=True, scale=0.0, rope_q=None):
    import torch
    tq, tk, tv = dev(q), dev(k), dev(v)
    o = torch.full_like(tq, float("nan"))
    b, n, h, _ = tq.shape
    lse = torch.full((b, h, n), float("nan"), device="cuda") if with_lse else None
    binding.flash_attn_fwd(tq, tk, tv, o, lse, scale, rope_q)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("with_lse", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,heads,d,batch", [
    (1, 1, 64, 1), (2, 2, 128, 1), (63, 1, 64, 1), (64, 3, 128, 1), (65, 2, 64, 2),
    (127, 1, 128, 1), (128, 2, 64, 1), (129, 3, 128, 1), (200, 2, 64, 2), (1000, 2, 128, 1),
    (4097, 1, 64, 1),
])
def test_ragged(gpu_lib, dtype, n, heads, d, batch, with_lse):
    """Both bf16 instruction streams: with the LSE (Q exact, scale in fp32)
    and without (scale folded into Q)."""
    say(f"attn ragged {dtype} n={n} heads={heads} d={d} batch={batch} lse={with_lse}")
    shape = (batch, n, heads, d)
    q, k, v = (_rand(shape, dtype, n * 7 + i) for i in range(3))
    o, lse = _attn(q, k, v, with_lse=with_lse)
    og = host(o)
    for b in range(batch):
        ref, rl = oracle.attention(inputs.values(q[b]), inputs.values(k[b]), inputs.values(v[b]))
        check(og[b], ref, dtype, f"o[{b}]")
        if with_lse:
            assert np.abs(lse.cpu().numpy()[b] - rl).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_explicit_scale(gpu_lib, dtype):
    say(f"attn explicit scale {dtype}")
    shape = (1, 300, 2, 128)
    q, k, v = (_rand(shape, dtype, 50 + i) for i in range(3))
    o, lse = _attn(q, k, v, scale=0.05)
    ref, rl = oracle.attention(inputs.values(q[0]), inputs.values(k[0]), inputs.values(v[0]),
                               scale=0.05)
    check(host(o)[0], ref, dtype, "o")
    assert np.abs(lse.cpu().numpy()[0] - rl).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_single_token_returns_v_exactly(gpu_lib, dtype, d):
    say(f"attn N=1 {dtype} d={d}")
    q, k, v = (_rand((2, 1, 3, d), dtype, 90 + i) for i in range(3))
    o, lse = _attn(q, k, v)
    np.testing.assert_array_equal(host(o), inputs.values(v))
    s = np.einsum("bnhd,bnhd->bhn", inputs.values(q).astype(np.float64),
                  inputs.values(k).astype(np.float64)) / np.sqrt(d)
    assert np.abs(lse.cpu().numpy() - s).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_equal_keys_give_mean_of_v(gpu_lib, dtype):
    say(f"attn equal keys {dtype}")
    n = 333
    q, k, v = (_rand((1, n, 2, 64), dtype, 120 + i) for i in range(3))
    k[:] = k[:, :1]
    o, _ = _attn(q, k, v, with_lse=False)
    mean = inputs.values(v).astype(np.float64).mean(axis=1, keepdims=True)
    check(host(o), np.broadcast_to(mean, o.shape), dtype, "o")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_fused_rope_q_matches_separate(gpu_lib, name):
    import torch
    wl = configs.WORKLOADS[name]
    say(f"attn fused rope_q {name}")
    q, k, v = inputs.attention_inputs(wl)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    tq, tk, tv = dev(q), dev(k), dev(v)
    binding.rope3d_apply(tq, tk, desc)
    o1 = torch.empty_like(tq)
    binding.flash_attn_fwd(tq, tk, tv, o1)
    tq0 = dev(q)
    o2 = torch.empty_like(tq)
    binding.flash_attn_fwd(tq0, tk, tv, o2, rope_q=desc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o2), bits(o1))
    np.testing.assert_array_equal(bits(tq0), q.view(np.int16 if q.dtype == np.uint16 else np.int32))


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_workload_rope_then_attention(gpu_lib, name):
    """The whole hot path at each workload's real size, in three forms:
    Q and K rotated by vx_rope3d_apply then attention with the LSE; K rotated
    and Q rotated on load, with the LSE (the same bits as the first: the same
    instruction stream and the same rotation); and the same without the LSE
    (the instruction stream the step runs).  The oracle checks all rows on
    the small workloads and 256 seeded rows (all heads, all keys) on the
    large ones."""
    import torch
    wl = configs.WORKLOADS[name]
    say(f"attn workload {name}: N={wl.n_tokens} H={wl.heads} d={wl.head_dim}")
    q, k, v = inputs.attention_inputs(wl)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    rows = inputs.sample_rows(wl)
    tq, tk, tv = dev(q), dev(k), dev(v)
    binding.rope3d_apply(None, tk, desc)
    o_fast = torch.empty_like(tq)
    binding.flash_attn_fwd(tq, tk, tv, o_fast, None, rope_q=desc)
    o_fused = torch.empty_like(tq)
    lse_fused = torch.empty((1, wl.heads, wl.n_tokens), device="cuda")
    binding.flash_attn_fwd(tq, tk, tv, o_fused, lse_fused, rope_q=desc)
    binding.rope3d_apply(tq, None, desc)
    o_sep = torch.empty_like(tq)
    lse = torch.empty_like(lse_fused)
    binding.flash_attn_fwd(tq, tk, tv, o_sep, lse, rope_q=None)
    torch.cuda.synchronize()
    del tq, tk, tv
    as_int = torch.int16 if wl.dtype == "bf16" else torch.int32
    assert torch.equal(o_sep.view(as_int), o_fused.view(as_int))
    assert torch.equal(lse.view(torch.int32), lse_fused.view(torch.int32))
    del o_fused, lse_fused
    og_sep, og_fast = host(o_sep)[0, rows], host(o_fast)[0, rows]
    lg = lse.cpu().numpy()[0][:, rows]
    del o_sep, o_fast, lse
    ref, rl = oracle.attention_rope(inputs.values(q[0]), inputs.values(k[0]), inputs.values(v[0]),
                                    wl.grid, wl.split, wl.theta, wl.n_prefix, rows=rows)
    check(og_sep, ref, wl.dtype, f"attn {name} (with LSE)")
    check(og_fast, ref, wl.dtype, f"attn {name} (without LSE)")
    say(f"  output rms {float(np.sqrt(np.mean(ref ** 2))):.3e} "
        f"(an all-zero output has rel L2 1.0)")
    lse_err = float(np.abs(lg - rl).max())
    say(f"  lse max abs {lse_err:.3e}")
    assert lse_err <= LSE_TOL[wl.dtype]


@pytest.mark.timeout(1200)
def test_mid_every_row(gpu_lib):
    """The mid workload (32,760 tokens, 40 heads x 128) with every query row
    of every head checked against all keys, K rotated by vx_rope3d_apply and
    Q on load: 22 TFLOP of fp64 work for the host oracle, one head at a time
    (a few seconds per head with 16 host threads).  VX_ORACLE_MID_HEADS=n
    checks only the first n heads."""
    import os
    import time
    import torch
    wl = configs.WORKLOADS["mid"]
    heads = list(range(int(os.environ.get("VX_ORACLE_MID_HEADS", wl.heads))))
    say(f"attn mid every row: N={wl.n_tokens}, heads {heads}")
    q, k, v = inputs.attention_inputs(wl)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix)
    tq, tk, tv = dev(q), dev(k), dev(v)
    binding.rope3d_apply(None, tk, desc)
    o = torch.empty_like(tq)
    lse = torch.empty((1, wl.heads, wl.n_tokens), device="cuda")
    binding.flash_attn_fwd(tq, tk, tv, o, lse, rope_q=desc)
    o_fast = torch.empty_like(tq)
    binding.flash_attn_fwd(tq, tk, tv, o_fast, None, rope_q=desc)
    torch.cuda.synchronize()
    og, og_fast, lg = host(o)[0], host(o_fast)[0], lse.cpu().numpy()[0]
    del tq, tk, tv, o, o_fast, lse
    acc = ChunkCheck(wl.dtype, "attn mid, every row (with LSE)")
    acc_fast = ChunkCheck(wl.dtype, "attn mid, every row (without LSE)")
    lse_err = 0.0
    t0 = time.perf_counter()
    for h in heads:
        sel = [h]
        ref, rl = oracle.attention_rope(inputs.values(q[0][:, sel]), inputs.values(k[0][:, sel]),
                                        inputs.values(v[0][:, sel]), wl.grid, wl.split, wl.theta,
                                        wl.n_prefix)
        acc.add(og[:, sel], ref)
        acc_fast.add(og_fast[:, sel], ref)
        lse_err = max(lse_err, float(np.abs(lg[sel] - rl).max()))
        say(f"  head {h}: done, {time.perf_counter() - t0:.1f} s of host oracle")
    acc.done()
    acc_fast.done()
    say(f"  lse max abs {lse_err:.3e}")
    assert lse_err <= LSE_TOL[wl.dtype]


def _aligned_scores(n, heads, d, pattern, seed):
    """Q and K rows close to one unit direction per head, so scores reach
    about 50-80 (natural units).  'rising': scores grow linearly along the
    keys, so the kernel raises its running maximum again and again (about
    every two key tiles).  'jump': the first half of the keys score near 0
    and the second half near the top, so the maximum is raised once, by a
    weight factor far below the float range."""
    g = np.random.default_rng(seed)
    q = np.empty((1, n, heads, d), np.float32)
    k = np.empty((1, n, heads, d), np.float32)
    v = g.standard_normal((1, n, heads, d)).astype(np.float32)
    for h in range(heads):
        u = g.standard_normal(d)
        u /= np.linalg.norm(u)
        a = 4.0 + 2.0 * g.random(n)
        if pattern == "rising":
            b = 12.0 * np.sqrt(d) * np.arange(n) / n
        else:
            b = np.where(np.arange(n) < n // 2, 0.0, 12.0 * np.sqrt(d))
        q[0, :, h] = a[:, None] * u + 0.05 * g.standard_normal((n, d))
        k[0, :, h] = b[:, None] * u + 0.05 * g.standard_normal((n, d))
    return (inputs.storage(x, "bf16") for x in (q, k, v))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("pattern", ["rising", "jump"])
def test_large_rising_scores(gpu_lib, d, pattern):
    """The lazy rescale under scores of 50-80: O to the usual bf16 tolerance
    from both instruction streams, and the LSE to the same fixed bound as
    everywhere else."""
    n, heads = 1500, 2
    say(f"attn large scores {pattern} d={d}")
    q, k, v = _aligned_scores(n, heads, d, pattern, 11 + d)
    o, lse = _attn(q, k, v)
    o_fast, _ = _attn(q, k, v, with_lse=False)
    qv, kv, vv = (inputs.values(x[0]).astype(np.float64) for x in (q, k, v))
    ref, rl = oracle.attention(qv, kv, vv)
    check(host(o)[0], ref, "bf16", f"o {pattern} (with LSE)")
    check(host(o_fast)[0], ref, "bf16", f"o {pattern} (without LSE)")
    err = np.abs(lse.cpu().numpy()[0] - rl)
    for h in range(heads):
        say(f"  head {h}: lse max abs {err[h].max():.3e}, max lse {rl[h].max():.1f}")
    assert err.max() <= LSE_TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_widest_rows_the_host_accepts(gpu_lib, d, dtype):
    """heads * head_dim = 2^22, the most the host accepts: a token row is 8 MiB,
    so a key tile is 0.5 or 1 GiB and its buffer resource is clamped near the
    2^31-byte limit (bf16); 130 tokens leave a ragged last tile.  Inputs are
    drawn on the GPU (N(0,1), in the dtype); sampled heads, all rows, against
    the oracle."""
    import torch
    heads, n = 2**22 // d, 130
    say(f"attn widest rows {dtype} d={d} heads={heads} n={n}")
    g = torch.Generator(device="cuda")
    g.manual_seed(11 + d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.randn((1, n, heads, d), device="cuda", generator=g).to(tdt)
               for _ in range(3))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, heads, n), float("nan"), device="cuda")
    binding.flash_attn_fwd(q, k, v, o, lse)
    torch.cuda.synchronize()
    picks = [0, 1, heads // 2 + 3, heads - 2, heads - 1]
    for h in picks:
        sl = lambda t: t[0, :, h:h + 1, :].float().cpu().numpy()
        ref, rl = oracle.attention(sl(q), sl(k), sl(v))
        check(sl(o), ref, dtype, f"o head {h}")
        assert np.abs(lse[0, h].cpu().numpy() - rl[0]).max() <= LSE_TOL[dtype]
    assert not torch.isnan(o).any().item()
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,heads,d,batch,rope", [
    (4096, 8, 128, 1, False), (3001, 4, 64, 2, False), (2000, 3, 128, 1, True),
    (1555, 2, 64, 1, True),
])
def test_f32_mfma_at_size(gpu_lib, n, heads, d, batch, rope):
    """fp32 attention (v_mfma_f32_32x32x2_f32 for both products) beyond the
    tiny workload: every row of every head against the oracle at the fp32
    bound, with ragged last tiles and, with RoPE, a text prefix and Q rotated
    on load (K rotated by vx_rope3d_apply)."""
    import torch
    say(f"attn f32 mfma n={n} heads={heads} d={d} batch={batch} rope={rope}")
    shape = (batch, n, heads, d)
    q, k, v = (_rand(shape, "f32", 7000 + n + i) for i in range(3))
    tq, tk, tv = dev(q), dev(k), dev(v)
    split = (16, 24, 24) if d == 64 else (44, 42, 42)
    prefix = 7
    grid = None
    if rope:
        nv = n - prefix
        grid = (1, 1, nv)
        for tt in range(2, 12):
            if nv % tt == 0:
                grid = (tt, 1, nv // tt)
                break
        desc = binding.RopeDesc.of(grid, split, 10000.0, prefix)
        binding.rope3d_apply(None, tk, desc)
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((batch, heads, n), float("nan"), device="cuda")
    binding.flash_attn_fwd(tq, tk, tv, o, lse, 0.0, desc if rope else None)
    torch.cuda.synchronize()
    og, lg = host(o), lse.cpu().numpy()
    for b in range(batch):
        if rope:
            ref, rl = oracle.attention_rope(inputs.values(q[b]), inputs.values(k[b]),
                                            inputs.values(v[b]), grid, split, 10000.0, prefix)
        else:
            ref, rl = oracle.attention(inputs.values(q[b]), inputs.values(k[b]),
                                       inputs.values(v[b]))
        check(og[b], ref, "f32", f"o[{b}]")
        assert np.abs(lg[b] - rl).max() <= LSE_TOL["f32"]
