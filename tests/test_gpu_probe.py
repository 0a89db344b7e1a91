"""GPU test of the matrix-core probe (ring_attn_mfma_probe) through the C ABI.

Its operands are small multiples of 1/128, so every product and partial sum
is exact in fp32: the test rebuilds the expected accumulators on the CPU from
the operand and accumulator lane layouts of v_mfma_f32_32x32x16_bf16 (lane l
supplies row l % 32 of A and column l % 32 of B, k = 8 (l / 32) .. + 8; its
accumulator element j is row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32),
which the step kernels rely on, and compares bit for bit."""
import numpy as np
import pytest

import ring_attention_blockwise_amd as ra

pytestmark = pytest.mark.gpu


def _operand(lane, i, mult):
    return ((mult * lane + i) & 7) / 128.0


def _expected_sink(iters):
    a = np.array([[_operand(l, i, 1) for i in range(8)] for l in range(64)])
    b = np.array([[_operand(l, i, 3) for i in range(8)] for l in range(64)])

    def product(x, y):  # A from lanes' x, B from lanes' y
        A = np.zeros((32, 16))
        B = np.zeros((16, 32))
        for l in range(64):
            A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = x[l]
            B[8 * (l // 32):8 * (l // 32) + 8, l % 32] = y[l]
        return iters * (A @ B)

    cab, cba = product(a, b), product(b, a)
    sink = np.zeros(64)
    for l in range(64):
        for j in range(16):
            r, c = 8 * (j // 4) + 4 * (l // 32) + j % 4, l % 32
            sink[l] += 2 * cab[r, c] + 2 * cba[r, c]
    return np.tile(sink, 4)  # four identical waves per workgroup


def test_mfma_probe_layout_and_stamps(gpu):
    import torch
    blocks, iters = 512, 256
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=gpu)
    stamps = torch.zeros(blocks * 4, dtype=torch.int64, device=gpu)
    ra.mfma_probe(blocks, iters, sink, stamps)
    torch.cuda.synchronize()
    want = np.tile(_expected_sink(iters), blocks).astype(np.float32)
    got = sink.cpu().numpy()
    assert np.array_equal(got, want)
    st = stamps.view(blocks, 4).cpu().numpy()
    assert (st[:, 1] > st[:, 0]).all() and (st[:, 3] >= st[:, 2]).all()


def test_mfma_probe_rejects_wrong_buffers(gpu):
    import torch
    sink = torch.empty(100, dtype=torch.float32, device=gpu)
    stamps = torch.zeros(4, dtype=torch.int64, device=gpu)
    with pytest.raises(ValueError):
        ra.mfma_probe(1, 1, sink, stamps)
