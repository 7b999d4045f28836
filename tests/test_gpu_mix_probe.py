"""The instruction-mix probe (sparse_attn_mix_probe): a diagnostic that runs
the attention stage's products and softmax step with nothing else in the
way.  Checked here: every wave runs and reports its cycles, the results stay
finite, and the cycles are at least what the products alone occupy on a
SIMD (W waves x 32 products of 32 clocks per stage; one
v_mfma_f32_32x32x16_bf16 is 32768 FLOP and a SIMD retires 1024 FLOP per
clock at the published peak; half of that is asserted, allowing for
uneven residency), so the work was not optimised away."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("waves,pingpong", [(1, False), (2, False), (3, False), (2, True)])
def test_mix_probe_runs(waves, pingpong):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 40
    n = cus * waves
    print(f"mix probe waves_per_simd={waves} pingpong={pingpong} cus={cus} iters={iters}", flush=True)
    cyc = torch.zeros(n * 4, dtype=torch.int64, device="cuda")
    sink = torch.full((n * 256,), float("nan"), dtype=torch.float32, device="cuda")
    sa.sparse_attn_mix_probe(waves, cus, iters, cyc, sink, pingpong=pingpong)
    torch.cuda.synchronize()
    c = cyc.cpu().numpy()
    s = sink.cpu().numpy()
    assert np.all(c > 0)
    assert np.all(np.isfinite(s))
    assert np.median(c) >= 0.5 * waves * iters * 32 * 32


def test_mix_probe_binding_checks_sizes():
    cyc = torch.zeros(7, dtype=torch.int64, device="cuda")
    sink = torch.zeros(256 * 4, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        sa.sparse_attn_mix_probe(1, 4, 10, cyc, sink)
