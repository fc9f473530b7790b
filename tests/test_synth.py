"""Checks of the seeded input generator (host side): the E4M3 encoder against
the oracle's decoder and torch's float8 cast, the quantised-row contract, the
N(0,1) approximation, the planted-row count and slice consistency."""
import numpy as np
import torch

import oracle
import synth
from synth.workloads import WORKLOADS, host_indexer, host_kv


def test_e4m3_encoder_round_trips_every_finite_code():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = oracle.e4m3(c)
        got = synth.e4m3_encode(v)
        if v == 0.0:
            assert got in (0x00, 0x80)
        else:
            assert got == c, (hex(c), v, hex(got))


def test_e4m3_encoder_matches_torch_cast():
    rs = np.random.default_rng(0)
    x = np.concatenate([rs.standard_normal(5000) * 100, rs.standard_normal(5000) * 0.01,
                        rs.uniform(-460, 460, 2000)]).astype(np.float32)
    # torch's float -> float8_e4m3fn cast rounds to nearest even and saturates only
    # when asked; clamp to the finite range first
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    got = np.array([synth.e4m3_encode(float(v)) for v in x], np.uint8)
    ref = ref.numpy()
    zero = (ref & 0x7F) == 0
    assert np.array_equal(got[~zero], ref[~zero])
    assert np.all((got[zero] & 0x7F) == 0)


def test_e4m3_encoder_ties_and_saturation():
    # 1 + 1/16 lies halfway between 1 (0x38) and 1.125 (0x39): even -> 0x38
    assert synth.e4m3_encode(1.0 + 1 / 16) == 0x38
    assert synth.e4m3_encode(1.125 + 1 / 16) == 0x3A  # halfway 1.125..1.25 -> even 1.25
    assert synth.e4m3_encode(1000.0) == 0x7E and synth.e4m3_encode(-1e9) == 0xFE
    assert synth.e4m3_encode(2.0 ** -10) == 0x00  # halfway 0..2^-9 -> even 0
    assert synth.e4m3_encode(3 * 2.0 ** -10) == 0x02  # halfway 2^-9..2^-8 -> even


def test_quantised_rows_contract():
    codes, scales = synth.host_fp8_rows(3, synth.T_IDX_KEY, 0, 64, 128, 0, 0, 2, 0, 64)
    assert codes.shape == (2, 64, 128) and scales.shape == (2, 64)
    dec = np.vectorize(oracle.e4m3)(codes)
    assert np.all(np.isfinite(dec))
    # every row uses the full range: its largest code decodes to +-448 (amax / scale)
    assert np.all(np.abs(dec).max(axis=-1) == 448.0)
    assert np.all(scales > 0)


def test_normal_approximation_moments():
    x = synth.host_bf16_rows(99, synth.T_KV, 0, 576, 0, 1, 0, 400)
    f = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy().ravel()
    assert abs(f.mean()) < 0.01 and abs(f.var() - 1.0) < 0.01
    assert f.min() >= -6.0 and f.max() < 6.0


def test_uniform_range():
    u = synth.host_uniform_rows(5, synth.T_IDX_W, 0, 32, 0, 4, 0, 500).ravel()
    assert u.min() >= 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 0.01


def test_planted_count_is_exact():
    for R in (131072, 1000, 4096 + 37):
        p = synth.host_planted(2, 0, 3, R, 100)
        assert int(p.sum()) == (R * 100 + 5000) // 10000


def test_planted_keys_are_shifted_and_score_high():
    w = WORKLOADS["decode128k"]
    L = 4096
    codes, scales = synth.host_fp8_rows(w.seed, synth.T_IDX_KEY, 0, L, 128, 100, 0, 1, 0, L)
    p = synth.host_planted(w.seed, 0, 0, L, 100).astype(bool)
    dec = np.vectorize(oracle.e4m3)(codes[0]) * scales[0][:, None]
    assert dec[p].mean() > 2.5 and abs(dec[~p].mean()) < 0.05


def test_slices_equal_full_block():
    w = WORKLOADS["tiny"]
    full = host_indexer(w, 1)
    part = host_indexer(w, 1, key_r0=100, key_nr=50)
    assert np.array_equal(full["k8"][:, 100:150], part["k8"])
    assert np.array_equal(full["k_scale"][:, 100:150], part["k_scale"])
    kv, _ = host_kv(w, 2)
    kv2, _ = host_kv(w, 2, r0=4000, nr=3)
    assert np.array_equal(kv[:, 4000:4003], kv2)


def test_workload_vis_len_and_schedules():
    assert np.all(WORKLOADS["decode128k"].vis_len() == 131072)
    v = WORKLOADS["prefill"].vis_len()
    assert v[0, 0] == 131072 - 4096 + 1 and v[0, -1] == 131072
    assert WORKLOADS["decode1m"].full_layers() == [0, 1] + list(range(2, 78, 4))
    assert len(WORKLOADS["decode1m"].full_layers()) == 21
    assert WORKLOADS["tiny"].full_layers() == [0]
    assert WORKLOADS["mtp1m"].full_layers() == [0]
