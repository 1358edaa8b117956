"""The measurement probes on the GPU.  gdn_mfma_peak_probe: back-to-back
independent products reach a plausible share of the published dense peaks
(bf16 2.5 PFLOP/s, fp32 157.3 TFLOP/s).  gdn_hbm_copy_probe: the copy is exact
(every byte of dst equals src, also for a buffer that ends mid-loop) and its
rate a plausible share of the 8 TB/s HBM peak."""
import pytest
import torch

import linear_attention_state_amd as gdn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,peak", [("bf16", 2500.0), ("f32", 157.3)])
def test_probe_rate_is_plausible(dtype, peak):
    rate = gdn.gdn_mfma_peak_probe(dtype, 2048)
    print("%s: %.1f TFLOP/s (%.3f of the published peak)" % (dtype, rate, rate / peak), flush=True)
    assert 0.3 * peak < rate < 1.1 * peak


@pytest.mark.parametrize("nbytes", [256 << 20, 16 * 1000003, 48])
def test_copy_probe_copies_exactly(nbytes):
    g = torch.Generator(device="cuda").manual_seed(11)
    src = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    rate = gdn.gdn_hbm_copy_probe(src, dst, reps=3)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    print("%d bytes: %.0f GB/s" % (nbytes, rate), flush=True)
    if nbytes >= (256 << 20):
        assert 0.3 * 8000 < rate < 1.05 * 8000
