"""Shape and reproducibility checks of the seeded synthetic workloads (CPU)."""
import numpy as np

from decode_attention_nvfp4_amd import workloads as W


def test_decode_workload_shapes_and_pages():
    for cfg, (B, Hq, Hkv) in {1: (1, 1, 1), 2: (8, 32, 8), 3: (1, 64, 8), 4: (128, 32, 8)}.items():
        w = W.decode_workload(cfg)
        assert (w.B, w.Hq, w.Hkv) == (B, Hq, Hkv)
        used = np.concatenate([w.page_table[b, :-(-(int(w.lens[b]) + 16) // 16)] for b in range(B)])
        assert np.array_equal(np.sort(used), np.arange(w.num_pages))   # every page once
    w4 = W.decode_workload(4)
    assert w4.lens.min() >= 1024 and w4.lens.max() <= 8192
    assert not np.array_equal(w4.page_table[0, :10], np.arange(10))   # permuted


def test_reproducible_and_bf16_exact():
    a = W.decode_workload(2)
    b = W.decode_workload(2)
    ka, va = a.kv(3)
    kb, vb = b.kv(3)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    assert np.all((ka.view(np.uint32) & 0xFFFF) == 0)          # bf16-representable
    assert np.array_equal(a.q(5), b.q(5)) and not np.array_equal(a.q(5), a.q(6))
    # four x20 outlier channels per KV head in K
    amp = np.abs(ka).mean(axis=0)
    for h in range(a.Hkv):
        top = set(np.argsort(amp[h])[-4:].tolist())
        assert top == set(a.outlier_channels[h].tolist())


def test_long_context_drift_is_per_token():
    w = W.decode_workload(3)
    w.lens = np.array([2048], np.int32)
    k, v = w.kv(0)
    rms = np.sqrt((k.astype(np.float64) ** 2).mean(axis=(1, 2)))
    assert rms.std() > 0.2            # log-normal per-token factor, sigma 0.5
    assert k.shape == (2048, 8, 128)


def test_prefill_workload_shapes():
    p = W.PrefillWorkload()
    assert p.total == 34816 and p.num_pages == 2176
    s = W.small_prefill(64, 32, 8, 2)
    k, v = s.prefix_kv()
    assert k.shape == (64, 2, 128)
    assert s.q().shape == (32, 8, 128)
