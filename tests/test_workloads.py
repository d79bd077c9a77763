"""The synthetic workload shapes (CPU only)."""
import numpy as np

from workloads import host_tensors, transformer_shard_sizes, workloads, zero_bucket_sizes


def test_workload_shapes():
    w = workloads()
    assert w["tiny"].sizes == (4096, 1000, 7) and w["tiny"].bytes_per_elem == 28
    b = w["bench201"]
    assert b.sizes == (20_971_520,) * 201 and b.numel == 4_215_275_520 and b.bytes_per_elem == 28
    s = w["shard30b"]
    decay, no_decay = transformer_shard_sizes()
    assert len(decay) == 48 * 7 + 1 and sum(decay) == 11_005_853_696
    assert no_decay == (4096,) * 48 and s.numel == 11_006_050_304 and s.bytes_per_elem == 26
    z = w["zero1e9"]
    assert len(z.sizes) == 2048 and z.numel == 1_000_000_000 and z.bytes_per_elem == 28
    assert min(z.sizes) >= 65536 and max(z.sizes) <= 2_097_152 and all(n % 64 == 0 for n in z.sizes)
    r = w["rem5e8"]
    assert r.numel == 500_000_000 and r.bytes_per_elem == 26 and min(r.sizes) > 0
    assert any(n % 4 for n in r.sizes)  # ragged tails present
    assert zero_bucket_sizes() == zero_bucket_sizes()  # seeded


def test_host_tensors_distributions():
    h = host_tensors([100000], g_dtype="bf16", p_kind="bf16_rem", p_out=True, seed=3)[0]
    assert h.p.dtype == np.uint16 and h.rem.dtype == np.int16 and h.g.dtype == np.uint16
    assert h.p_out.dtype == np.uint16 and not h.m.any() and not h.v.any()
    g = (h.g.astype(np.uint32) << 16).view(np.float32)
    assert 0.9e-3 < g.std() < 1.1e-3
    assert h.rem.min() < -30000 and h.rem.max() > 30000
    h2 = host_tensors([100000], seed=3)[0]
    assert 0.98 < h2.p.std() < 1.02 and h2.p.dtype == np.float32


def test_fp16_and_scaled_workloads():
    w = workloads()
    assert w["zero1e9_f16"].bytes_per_elem == 28 and w["zero1e9_f16"].sizes == w["zero1e9"].sizes
    s = w["scaled1e9"]
    assert s.bytes_per_elem == 16 and s.numel == 1_000_000_000 and s.p_kind == "f16_scaled"


def test_scaled_state_inputs_decode_to_the_drawn_values():
    """Scaled-state inputs: stored x 2^-k reproduces the drawn float32
    values to the state type's precision; zero moments carry scale 0."""
    h = host_tensors([50000], g_dtype="f16", p_kind="f16_scaled", p_out="f16", seed=5,
                     m_v_init="random")[0]
    h32 = host_tensors([50000], g_dtype="f32", seed=5, m_v_init="random")[0]
    assert h.p.dtype == np.float16 and h.m.dtype == np.float16 and h.g.dtype == np.float16
    assert h.p_out.dtype == np.float16 and h.scales.dtype == np.float32
    for stored, scale, x in ((h.p, h.scales[0], h32.p), (h.m, h.scales[1], h32.m),
                             (h.v, h.scales[2], h32.v)):
        back = stored.astype(np.float64) * float(scale)
        assert np.all(np.abs(back - x) <= 2.0 ** -11 * np.abs(x) + float(scale) * 2.0 ** -24)
        assert np.isfinite(stored).all()
    z = host_tensors([100], p_kind="bf16_scaled", seed=1)[0]
    assert z.scales[1] == 0 and z.scales[2] == 0 and z.p.dtype == np.uint16
