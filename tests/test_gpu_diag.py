"""The MFMA ceiling probe (a measurement aid bench.py times) does the MFMA
work it is credited with: each wave's accumulators sum to what the fp64
products of its operand fragments give.

Whatever the accumulator layout, the sum of all entries of A B is
sum_k (column sum of A)_k (row sum of B)_k.  For v_mfma_f32_32x32x16_bf16,
lane l supplies A[l % 32][8 (l // 32) + e] and B[8 (l // 32) + e][l % 32],
e = 0..7, so k = 8 (l // 32) + e in both operands.
"""
import numpy as np
import pytest

from spatiotemporal_attention_vx_amd import diag


def _wave_total(frags, iters):
    """frags: [16, 64, 8] float64 (A fragments 0-7, B fragments 8-15)."""
    tot = 0.0
    for i in range(8):
        a, b = frags[i], frags[8 + ((3 * i + 1) & 7)]
        col_a = a.reshape(2, 32, 8).sum(axis=1)     # [lane half, e] -> k
        row_b = b.reshape(2, 32, 8).sum(axis=1)
        tot += float((col_a * row_b).sum())
    return iters * tot


@pytest.mark.gpu
@pytest.mark.parametrize("iters", [0, 1, 3])
def test_mfma_loop_sums(iters):
    import torch
    wg = 3
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    ops = torch.randn(wg * diag.OPERAND_BYTES_PER_WORKGROUP // 2, device="cuda",
                      generator=g).to(torch.bfloat16)
    out = torch.full((wg * 512,), float("nan"), device="cuda")
    diag.mfma_loop(ops, out, wg, iters)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(wg * 8, 64).sum(axis=1)
    vals = ops.float().cpu().double().numpy().reshape(wg * 8, 16, 64, 8)
    for w in range(wg * 8):
        want = _wave_total(vals[w], iters)
        scale = iters * 8 * 512 * 16 + 1.0       # sum of |products| is about this size
        assert abs(got[w] - want) <= 1e-5 * scale, (w, got[w], want)


def test_mfma_loop_rejects_bad_arguments_without_launching():
    lib = diag.load()
    assert lib.vx_diag_mfma_bf16_loop(None, None, 1, 1, None) == 1
    assert lib.vx_diag_mfma_bf16_loop(0x10008, 0x20000, 1, 1, None) == 1   # misaligned operands
    assert lib.vx_diag_mfma_bf16_loop(0x10000, 0x20000, 0, 1, None) == 2
    assert lib.vx_diag_mfma_bf16_loop(0x10000, 0x20000, 1, -1, None) == 2
    assert lib.vx_diag_mfma_bf16_loop_flops(1024, 20000) == 1024 * 8 * 8 * 20000 * 32768.0
