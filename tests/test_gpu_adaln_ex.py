"""GPU parity of vx_adaln_modulate_ex: per-token and per-sample tables,
each of x, the tables and y in bf16 or f32, against the fp64 oracle."""
import itertools

import numpy as np
import pytest

import oracle
from _helpers import bits, check, dev, host, say
from spatiotemporal_attention_vx_amd import binding, configs, inputs

pytestmark = pytest.mark.gpu

DTYPES = list(itertools.product(["bf16", "f32"], repeat=3))     # (x, tables, y)


def _max_hidden(xd, md, yd):
    return 8192


def _group(xd, md, yd):
    return 4 if (xd, md, yd) == ("f32", "f32", "f32") else 8


def _run(x, sh, sc, y_dtype, eps=1e-6):
    import torch
    tx, tsh, tsc = dev(x), dev(sh), dev(sc)
    ty = torch.full(tx.shape, float("nan"),
                    dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32, device="cuda")
    binding.adaln_modulate_ex(tx, tsh, tsc, ty, eps)
    torch.cuda.synchronize()
    return ty


def _ref(x, sh, sc, per_sample, eps=1e-6):
    v = lambda a: inputs.values(a).astype(np.float64)
    if per_sample:
        return oracle.adaln_modulate_per_sample(v(x), v(sh)[:, 0, :], v(sc)[:, 0, :], eps)
    return oracle.adaln_modulate(v(x), v(sh), v(sc), eps)


SHAPES = [(2, 5, 8), (1, 7, 136), (3, 4, 1000), (2, 3, 5120), (1, 2, 8192), (2, 3, 12),
          (1, 3, 4096), (2, 3, 4100), (1, 2, 6144)]
# every dtype mix at every width it accepts (a multiple of 8, of 4 when all are
# f32; the host's rejection of the others is a CPU test of the C ABI)
LAYOUTS = [(xd, md, yd, b, n, hid) for (xd, md, yd) in DTYPES for (b, n, hid) in SHAPES
           if hid % _group(xd, md, yd) == 0 and hid <= _max_hidden(xd, md, yd)]


@pytest.mark.parametrize("xd,md,yd,batch,n,hidden", LAYOUTS)
@pytest.mark.parametrize("per_sample", [False, True])
def test_dtype_and_table_layouts(gpu_lib, xd, md, yd, per_sample, batch, n, hidden):
    say(f"adaln_ex x={xd} tables={md} y={yd} per_sample={per_sample} b={batch} n={n} d={hidden}")
    g = np.random.default_rng(batch * 7919 + n * 31 + hidden)
    mrows = 1 if per_sample else n
    x = inputs.storage((g.standard_normal((batch, n, hidden)) + 0.3).astype(np.float32), xd)
    sh = inputs.storage((g.standard_normal((batch, mrows, hidden)) * 0.1).astype(np.float32), md)
    sc = inputs.storage((g.standard_normal((batch, mrows, hidden)) * 0.1).astype(np.float32), md)
    y = host(_run(x, sh, sc, yd))
    check(y, _ref(x, sh, sc, per_sample), yd, "adaln_ex")


@pytest.mark.parametrize("dtype,n,hidden", [("bf16", 300, 5120), ("bf16", 41, 1000),
                                            ("f32", 33, 1028), ("f32", 20, 4096),
                                            ("f32", 17, 5120), ("f32", 9, 8192)])
def test_uniform_per_token_equals_vx_adaln_modulate(gpu_lib, dtype, n, hidden):
    import torch
    say(f"adaln_ex == adaln {dtype} n={n} d={hidden}")
    g = np.random.default_rng(n + hidden)
    mk = lambda s: inputs.storage((g.standard_normal((1, n, hidden)) * s).astype(np.float32), dtype)
    x, sh, sc = mk(1.0), mk(0.1), mk(0.1)
    y_ex = _run(x, sh, sc, dtype)
    tx = dev(x)
    y = torch.empty_like(tx)
    binding.adaln_modulate(tx[0], dev(sh)[0], dev(sc)[0], y[0])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y_ex), bits(y))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_in_place(gpu_lib, dtype):
    import torch
    say(f"adaln_ex in place {dtype}")
    g = np.random.default_rng(5)
    x = inputs.storage(g.standard_normal((2, 9, 1024)).astype(np.float32), dtype)
    sh = inputs.storage((g.standard_normal((2, 1, 1024)) * 0.1).astype(np.float32), "f32")
    sc = inputs.storage((g.standard_normal((2, 1, 1024)) * 0.1).astype(np.float32), "f32")
    y = _run(x, sh, sc, dtype)
    tx = dev(x)
    binding.adaln_modulate_ex(tx, dev(sh), dev(sc), tx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(tx), bits(y))


def test_per_sample_constant_rows_give_shift_exactly(gpu_lib):
    say("adaln_ex per-sample constant rows")
    g = np.random.default_rng(6)
    x = inputs.storage(np.full((3, 4, 512), -1.5, np.float32), "f32")
    sh = inputs.storage(g.normal(0, 0.1, (3, 1, 512)).astype(np.float32), "bf16")
    sc = inputs.storage(g.normal(0, 0.1, (3, 1, 512)).astype(np.float32), "bf16")
    y = host(_run(x, sh, sc, "f32"))
    np.testing.assert_array_equal(y, np.broadcast_to(inputs.values(sh), y.shape))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("xd,md,per_sample", [("bf16", "bf16", True), ("f32", "bf16", False),
                                              ("bf16", "f32", False), ("f32", "f32", False)])
def test_large_workload_variants(gpu_lib, xd, md, per_sample):
    """75,600 tokens x 5120 with bf16 output, as the bench step runs each
    variant; the oracle checks 2048 seeded rows."""
    wl = configs.WORKLOADS["large"]
    say(f"adaln_ex large x={xd} tables={md} per_sample={per_sample}")
    x, sh, sc = inputs.adaln_inputs_ex(wl, xd, md, per_sample)
    y = host(_run(x, sh, sc, "bf16", wl.eps))[0]
    rows = inputs.sample_rows(wl, count=2048)
    xs = x[:, rows]
    tabs = (sh, sc) if per_sample else (sh[:, rows], sc[:, rows])
    ref = _ref(xs, *tabs, per_sample, wl.eps)[0]
    check(y[rows], ref, "bf16", "adaln_ex large")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("per_sample", [False, True])
def test_large_workload_all_f32(gpu_lib, per_sample):
    """75,600 tokens x 5120 with x, the tables and y all fp32 (a DiT kept in
    fp32 end to end at the 14B models' width): 5120 = 64 lanes x 20 groups of
    4, so only x is held in registers and the tables are read in the output
    pass; the oracle checks 2048 seeded rows."""
    wl = configs.WORKLOADS["large"]
    say(f"adaln_ex large all f32 per_sample={per_sample}")
    x, sh, sc = inputs.adaln_inputs_ex(wl, "f32", "f32", per_sample)
    y = host(_run(x, sh, sc, "f32", wl.eps))[0]
    rows = inputs.sample_rows(wl, count=2048)
    tabs = (sh, sc) if per_sample else (sh[:, rows], sc[:, rows])
    ref = _ref(x[:, rows], *tabs, per_sample, wl.eps)[0]
    check(y[rows], ref, "f32", "adaln_ex large all f32")
