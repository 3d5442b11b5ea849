"""GPU parity of attention with key padding (vx_flash_attn_fwd_masked)
against the fp64 oracle: per-sample padded key ranges anywhere in the
sequence, including ranges that start at key 0 and whole tiles."""
import numpy as np
import pytest

import oracle
from _helpers import bits, check, dev, host, say
from spatiotemporal_attention_vx_amd import binding, configs, inputs

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-5, "bf16": 1e-2}


def _rand(shape, dtype, seed):
    g = np.random.default_rng(seed)
    return inputs.storage(g.standard_normal(shape).astype(np.float32), dtype)


def _masked(tq, tk, tv, pads, rope_q=None, with_lse=True):
    """Without the LSE the bf16 kernel runs its other instruction stream
    (softmax scale folded into Q)."""
    import torch
    b, nq, h, _ = tq.shape
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((b, h, nq), float("nan"), device="cuda") if with_lse else None
    binding.flash_attn_fwd_masked(tq, tk, tv, o, pads, lse, 0.0, rope_q)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,pads", [
    (300, 1000, [(100, 226)]),                 # inside: partial, whole and partial tiles
    (300, 1000, [(0, 200)]),                   # from key 0: the key loop starts at tile 3
    (129, 777, [(0, 64)]),                     # exactly the first tile
    (129, 777, [(0, 700)]),                    # all but the last 77 keys
    (64, 500, [(450, 500)]),                   # a padded tail
    (64, 500, [(1, 500)]),                     # one valid key
    (200, 333, [(5, 5), (0, 300), (64, 128)]), # per sample: none, from 0, one tile
    (50, 65, [(64, 65), (0, 1)]),
])
def test_padded_ranges(gpu_lib, dtype, d, nq, nk, pads):
    import torch
    batch = len(pads)
    say(f"attn masked {dtype} d={d} nq={nq} nk={nk} pads={pads}")
    seed = nq * 13 + nk + d
    q = _rand((batch, nq, 2, d), dtype, seed)
    k = _rand((batch, nk, 2, d), dtype, seed + 1)
    v = _rand((batch, nk, 2, d), dtype, seed + 2)
    o, lse = _masked(dev(q), dev(k), dev(v), pads)
    o_fast, _ = _masked(dev(q), dev(k), dev(v), pads, with_lse=False)
    torch.cuda.synchronize()
    og, og_fast, lg = host(o), host(o_fast), lse.cpu().numpy()
    for b, (lo, hi) in enumerate(pads):
        ref, rl = oracle.attention_masked(inputs.values(q[b]), inputs.values(k[b]),
                                          inputs.values(v[b]), lo, hi)
        check(og[b], ref, dtype, f"o[{b}]")
        check(og_fast[b], ref, dtype, f"o[{b}] (without LSE)")
        assert np.abs(lg[b] - rl).max() <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_padded_tail_equals_shorter_key_set(gpu_lib, dtype, d):
    """Padding [len, n_kv) adds exact zeros: the same bits as attending over
    the first len keys."""
    import torch
    say(f"attn masked tail == kv {dtype} d={d}")
    nq, nk, ln = 257, 900, 613
    q = _rand((1, nq, 3, d), dtype, 11)
    k = _rand((1, nk, 3, d), dtype, 12)
    v = _rand((1, nk, 3, d), dtype, 13)
    tq, tk, tv = dev(q), dev(k), dev(v)
    o1, l1 = _masked(tq, tk, tv, [(ln, nk)])
    o2 = torch.empty_like(tq)
    l2 = torch.empty_like(l1)
    binding.flash_attn_fwd_kv(tq, tk[:, :ln].contiguous(), tv[:, :ln].contiguous(), o2, l2)
    o3, _ = _masked(tq, tk, tv, [(ln, nk)], with_lse=False)
    o4 = torch.empty_like(tq)
    binding.flash_attn_fwd_kv(tq, tk[:, :ln].contiguous(), tv[:, :ln].contiguous(), o4, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o1), bits(o2))
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
    np.testing.assert_array_equal(bits(o3), bits(o4))


def test_padded_values_are_never_read_into_the_result(gpu_lib):
    """Changing K and V inside the padded range leaves the output bits alone."""
    import torch
    say("attn masked: padded K/V do not matter")
    q, k, v = (_rand((1, 400, 2, 128), "bf16", 20 + i) for i in range(3))
    pads = [(0, 150)]
    o1, l1 = _masked(dev(q), dev(k), dev(v), pads)
    k2, v2 = k.copy(), v.copy()
    k2[:, :150] = inputs.storage(np.full((1, 150, 2, 128), 3.0, np.float32), "bf16")
    v2[:, :150] = inputs.storage(np.full((1, 150, 2, 128), -9.0, np.float32), "bf16")
    o2, l2 = _masked(dev(q), dev(k2), dev(v2), pads)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o1), bits(o2))
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())


@pytest.mark.timeout(1200)
def test_joint_text_video_with_padded_text(gpu_lib):
    """The CogVideoX1.5 grid (226 text + 11 x 48 x 85 video tokens, 48 heads
    x 64) with text padded after 100 tokens: keys 100..225 masked, K
    rotated by vx_rope3d_apply, Q inside the attention load; 256 seeded rows
    x every head x every key against the oracle."""
    import torch
    wl = configs.FAMILY_WORKLOADS["cogvx15"]
    lo, hi = 100, wl.n_prefix
    say(f"attn masked {wl.name}: N={wl.n_tokens} pad [{lo}, {hi})")
    q, k, v = inputs.attention_inputs(wl)
    desc = binding.RopeDesc.of(wl.grid, wl.split, wl.theta, wl.n_prefix, wl.pairing)
    tq, tk, tv = dev(q), dev(k), dev(v)
    binding.rope3d_apply(None, tk, desc)
    o, lse = _masked(tq, tk, tv, [(lo, hi)], rope_q=desc)
    o_fast, _ = _masked(tq, tk, tv, [(lo, hi)], rope_q=desc, with_lse=False)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(wl)
    og, lg = host(o)[0, rows], lse.cpu().numpy()[0][:, rows]
    og_fast = host(o_fast)[0, rows]
    del o, o_fast, lse, tq, tk, tv
    qv, kv, vv = (inputs.values(a[0]) for a in (q, k, v))
    qr = oracle.rope3d_apply(qv[rows], wl.grid, wl.split, wl.theta, wl.n_prefix, tokens=rows)
    kr = oracle.rope3d_apply(kv, wl.grid, wl.split, wl.theta, wl.n_prefix)
    ref, rl = oracle.attention_masked(qr, kr, vv, lo, hi)
    check(og, ref, wl.dtype, "attn masked cogvx15")
    check(og_fast, ref, wl.dtype, "attn masked cogvx15 (without LSE)")
    lse_err = float(np.abs(lg - rl).max())
    say(f"  lse max abs {lse_err:.3e}")
    assert lse_err <= LSE_TOL[wl.dtype]
