"""GPU checks of the two rate probes that give the roofline denominators: the
MFMA probe's accumulators end at their closed-form value with operands of
ones (16 per MFMA, 8 chains summed: 128 * iters) and at the fp64 value of
the header's formula with random operands (which also pins the MFMA operand
and accumulator lane layouts the formula states), and the read probe's
outputs XOR to the XOR of
every 32-bit word of its buffer (computed on the host), also for a size that
leaves a ragged tail of 16-byte words."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import metrics as M  # noqa: E402
from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"


@pytest.mark.parametrize("n_wg,iters", [(1, 1), (3, 7), (512, 64)])
def test_mfma_probe_exact(n_wg, iters):
    print(f"mfma probe n_wg={n_wg} iters={iters}", flush=True)
    sink = torch.full((n_wg * 256,), -1.0, dtype=torch.float32, device=DEV)
    fl = SA.sa_measure_mfma_peak(n_wg, iters, sink)
    torch.cuda.synchronize()
    assert fl == n_wg * 4 * 8 * iters * 32768
    assert bool((sink == 128.0 * iters).all())


@pytest.mark.parametrize("n_wg,iters", [(1, 1), (3, 7), (64, 40)])
def test_mfma_probe_random_operands(n_wg, iters):
    print(f"mfma probe random n_wg={n_wg} iters={iters}", flush=True)
    sink = torch.full((n_wg * 256,), float("nan"), dtype=torch.float32, device=DEV)
    fl = SA.sa_measure_mfma_peak(n_wg, iters, sink, operands=1)
    torch.cuda.synchronize()
    assert fl == n_wg * 4 * 8 * iters * 32768
    want, scale = M.mfma_probe_random_sink(n_wg, iters)
    got = sink.cpu().double().numpy()
    # fp32 accumulation: each of the iters additions and the 8-chain sum
    # rounds at most 2^-24 of the running magnitude
    assert np.all(np.abs(got - want) <= (iters + 8) * 2.0**-23 * scale + 1e-6)
    assert np.abs(want).max() > 1.0  # not a degenerate case


@pytest.mark.parametrize("n_words,n_wg", [(4, 1), (4 * 1001, 3), (1 << 22, 1024), ((1 << 22) + 4 * 37, 2048)])
def test_hbm_probe_reads_every_word(n_words, n_wg):
    print(f"hbm probe words={n_words} n_wg={n_wg}", flush=True)
    rng = np.random.default_rng(n_words + n_wg)
    host = rng.integers(-2**31, 2**31 - 1, size=n_words, dtype=np.int32)
    buf = torch.from_numpy(host).to(DEV)
    sink = torch.full((n_wg * 256,), 7, dtype=torch.int32, device=DEV)
    nb = SA.sa_measure_hbm_read(buf, n_wg, sink)
    torch.cuda.synchronize()
    assert nb == 4 * n_words
    assert np.bitwise_xor.reduce(sink.cpu().numpy()) == np.bitwise_xor.reduce(host)
