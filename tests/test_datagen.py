"""The seeded input generator: determinism, block streaming, bf16 encoding, distributions."""
import numpy as np
import pytest
import torch

import datagen


def test_same_seed_same_values_other_seed_other_values():
    wl = datagen.workload("tiny_f32")
    a = datagen.scan_inputs(wl, seed=0)
    b = datagen.scan_inputs(wl, seed=0)
    c = datagen.scan_inputs(wl, seed=1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], c["x"])


def test_token_ranges_regenerate_the_same_values():
    """Any token range equals the same slice of the whole sequence (block streams)."""
    wl = datagen.custom("stream", batch=2, seqlen=3 * datagen.TBLK + 17, dim=5, dstate=3, io="bf16")
    for t in ("x", "delta", "B", "C"):
        full = datagen.gen_seq(wl, t)
        for t0, t1 in [(0, 1), (5, datagen.TBLK + 3), (datagen.TBLK, 2 * datagen.TBLK),
                       (2 * datagen.TBLK + 100, wl.seqlen)]:
            np.testing.assert_array_equal(datagen.gen_seq(wl, t, t0, t1), full[:, t0:t1])
        np.testing.assert_array_equal(datagen.gen_seq(wl, t, batch_rows=[1]), full[1:2])


def test_threaded_generation_matches_serial():
    wl = datagen.custom("thr", batch=3, seqlen=5 * datagen.TBLK, dim=7, dstate=4)
    np.testing.assert_array_equal(datagen.gen_seq(wl, "delta", threads=1),
                                  datagen.gen_seq(wl, "delta", threads=8))


def test_bf16_rounding_is_round_to_nearest_even():
    """Compared with torch's float32 -> bfloat16 conversion (RNE) on random and tie values."""
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  3.0e38, 1e-40, 0.0, -0.0], dtype=np.float32)])
    ours = datagen.round_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = datagen.bf16_bits(ours)
    np.testing.assert_array_equal(datagen.bits_to_f32(bits), ours)
    with pytest.raises(ValueError):
        datagen.bf16_bits(np.array([1.0 + 2 ** -20], dtype=np.float32))


def test_bf16_workload_values_are_bf16_representable():
    wl = datagen.custom("b", batch=1, seqlen=300, dim=9, dstate=4, io="bf16")
    for t in ("x", "delta", "B", "C"):
        v = datagen.gen_seq(wl, t)
        assert not np.any(v.view(np.uint32) & 0xFFFF)


def test_distributions():
    wl = datagen.custom("dist", batch=2, seqlen=4096, dim=64, dstate=16)
    x = datagen.gen_seq(wl, "x")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    d = datagen.gen_seq(wl, "delta").astype(np.float64)
    assert d.min() > 0
    # per-channel median ~ the biased softplus: inside the [1e-3, 1e-1] step range
    med = np.median(d.reshape(-1, 64), axis=0)
    assert med.min() > 5e-4 and med.max() < 0.15
    bias = datagen.gen_dt_bias(wl)
    step = np.log1p(np.exp(bias))
    assert step.min() >= 1e-3 - 1e-12 and step.max() <= 1e-1 + 1e-12
    A = datagen.gen_A(wl)
    assert A.shape == (64, 16) and (A <= -0.5).all() and (A >= -4.0).all()
    As = datagen.gen_A(datagen.workload("mamba130m_f32"))
    np.testing.assert_array_equal(As[17], -np.arange(1, 17, dtype=np.float32))


def test_workload_table():
    w = datagen.WORKLOADS
    assert w["tiny_f32"].elements == 1 * 256 * 16
    assert w["mamba1p4b_bf16"].elements == 4 * 8192 * 4096
    assert w["long1m_bf16"].seqlen == 1 << 20
    assert w["decode_bf16"].mode == "step"


def test_step_streams():
    wl = datagen.custom("st", batch=4, seqlen=10, dim=6, dstate=3, io="bf16", mode="step")
    a = datagen.step_inputs(wl, 3)
    b = datagen.step_inputs(wl, 3)
    c = datagen.step_inputs(wl, 4)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
        assert a[k].shape[0] == 4
    assert not np.array_equal(a["x"], c["x"])


def test_parameter_arrays_are_contiguous():
    for name in ("tiny_f32", "mamba130m_f32"):
        wl = datagen.workload(name)
        for a in (datagen.gen_A(wl), datagen.gen_Dskip(wl)):
            assert a.flags["C_CONTIGUOUS"] and torch.from_numpy(a).is_contiguous()
