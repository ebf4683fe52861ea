"""The matrix-core rate microbenchmark (mfa_debug_mfma_rate) that the
measurement sets beside the MFMA fractions: its flop count follows from the
launch shape, the rate it measures lies below the data-sheet dense peaks
(bf16 2.5 PFLOP/s, FP8 5.0 PFLOP/s) and within reach of them, and its
argument checks hold."""
import pytest
import torch

pytestmark = pytest.mark.gpu

PEAK_TFLOPS = {0: 2500.0, 1: 5000.0}


def test_mfma_rate_flops_and_range():
    import decode_attention_mfa_amd as m
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    for kind, k in ((0, 32), (1, 128)):
        iters = 1 << 13
        fl = m.mfa_debug_mfma_rate(kind, iters, sink)
        assert fl == 2 * ncu * 4 * iters * 8 * 2 * 16 * 16 * k
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            m.mfa_debug_mfma_rate(kind, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        tflops = 3 * fl / (e0.elapsed_time(e1) / 1e3) / 1e12
        print(f"kind {kind}: {tflops:.1f} TFLOP/s of {PEAK_TFLOPS[kind]}", flush=True)
        assert 0.3 * PEAK_TFLOPS[kind] <= tflops <= 1.05 * PEAK_TFLOPS[kind]
    assert sink.item() == 0.0


def test_mfma_rate_rejects_bad_arguments():
    import decode_attention_mfa_amd as m
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    for kind, iters in ((2, 16), (-1, 16), (0, 0), (1, (1 << 24) + 1)):
        with pytest.raises(m.MfaError):
            m.mfa_debug_mfma_rate(kind, iters, sink)
    with pytest.raises(m.MfaError):
        m.mfa_debug_mfma_rate(0, 16, None)
