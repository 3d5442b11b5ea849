"""GPU parity of vx_adaln_modulate against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from _helpers import ChunkCheck, bits, check, dev, host, say
from spatiotemporal_attention_vx_amd import binding, configs, inputs

pytestmark = pytest.mark.gpu


def _run(x, sh, sc, eps, dtype):
    import torch
    tx, tsh, tsc = dev(x), dev(sh), dev(sc)
    y = torch.empty_like(tx)
    binding.adaln_modulate(tx, tsh, tsc, y, eps)
    torch.cuda.synchronize()
    return y


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_workload(gpu_lib, name):
    wl = configs.WORKLOADS[name]
    say(f"adaln workload {name}: rows={wl.n_tokens} hidden={wl.hidden} {wl.dtype}")
    x, sh, sc = inputs.adaln_inputs(wl)
    y = host(_run(x, sh, sc, wl.eps, wl.dtype))
    # every row, in chunks that bound the host's fp64 copies
    acc = ChunkCheck(wl.dtype, f"adaln {name}")
    for r0 in range(0, wl.n_tokens, 8192):
        sl = slice(r0, r0 + 8192)
        v = lambda a: inputs.values(a[sl]).astype(np.float64)
        acc.add(y[sl], oracle.adaln_modulate(v(x), v(sh), v(sc), wl.eps))
    acc.done()


@pytest.mark.parametrize("dtype,rows,hidden", [
    ("bf16", 1, 8), ("bf16", 3, 24), ("bf16", 5, 136), ("bf16", 6, 1000), ("bf16", 9, 3072),
    ("bf16", 2, 8192), ("f32", 1, 4), ("f32", 7, 12), ("f32", 5, 128), ("f32", 3, 1028),
    ("f32", 2, 4096), ("f32", 3, 4100), ("f32", 2, 5120), ("f32", 5, 6148), ("f32", 3, 8192),
])
def test_ragged(gpu_lib, dtype, rows, hidden):
    say(f"adaln ragged {dtype} rows={rows} hidden={hidden}")
    g = np.random.default_rng(rows * 10007 + hidden)
    mk = lambda s: inputs.storage((g.standard_normal((rows, hidden)) * s + 0.3).astype(np.float32),
                                  dtype)
    x, sh, sc = mk(1.0), mk(0.1), mk(0.1)
    y = host(_run(x, sh, sc, 1e-6, dtype))
    v = lambda a: inputs.values(a).astype(np.float64)
    check(y, oracle.adaln_modulate(v(x), v(sh), v(sc), 1e-6), dtype, "adaln ragged")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_row_gives_shift_exactly(gpu_lib, dtype):
    say(f"adaln constant rows {dtype}")
    g = np.random.default_rng(3)
    x = inputs.storage(np.full((4, 1024), 2.5, np.float32), dtype)
    sh = inputs.storage(g.normal(0, 0.1, (4, 1024)).astype(np.float32), dtype)
    sc = inputs.storage(g.normal(0, 0.1, (4, 1024)).astype(np.float32), dtype)
    y = host(_run(x, sh, sc, 1e-6, dtype))
    np.testing.assert_array_equal(y, inputs.values(sh))


def test_in_place_matches_out_of_place(gpu_lib):
    import torch
    say("adaln in place")
    wl = configs.WORKLOADS["small"]
    x, sh, sc = inputs.adaln_inputs(wl)
    y = _run(x, sh, sc, wl.eps, wl.dtype)
    tx, tsh, tsc = dev(x), dev(sh), dev(sc)
    binding.adaln_modulate(tx, tsh, tsc, tx, wl.eps)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(tx), bits(y))


def test_bf16_rounding_is_unbiased(gpu_lib):
    # Round-to-nearest-even leaves no systematic pull toward zero; truncation
    # would show a mean signed error of about -1/2 ulp.
    say("adaln rounding bias")
    wl = configs.WORKLOADS["small"]
    x, sh, sc = inputs.adaln_inputs(wl)
    y = host(_run(x, sh, sc, wl.eps, wl.dtype)).astype(np.float64)
    v = lambda a: inputs.values(a).astype(np.float64)
    ref = oracle.adaln_modulate(v(x), v(sh), v(sc), wl.eps)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(ref) + 1e-30)) - 7)
    bias = float(np.mean((y - ref) * np.sign(ref) / ulp))
    say(f"  mean signed error toward |ref|: {bias:+.4f} ulp")
    assert abs(bias) < 0.05
