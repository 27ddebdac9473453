"""The input generator: bf16 rounding against torch, determinism, shapes."""
import numpy as np
import torch

from synth import inputs as si


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -1.00390625, 65504.0, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(si.f32_to_bf16_bits(x), ref)
    back = si.bf16_bits_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_shaped():
    dims, w, c = si.decode_config(0)
    dims2, w2, c2 = si.decode_config(0)
    for k in w:
        np.testing.assert_array_equal(w[k], w2[k])
    assert c["target_hidden"].shape == (132, 3, 256)
    assert c["kv_rows"] == 132 and c["cu_window"][-1] == 128
    assert w["w_fc"].shape == (256, 768) and w["w_lm"].shape == (4096, 256)
    # stream RMS close to 0.5 / 0.6 / 0.8
    rms = np.sqrt(np.mean(c["target_hidden"].astype(np.float64) ** 2, axis=(0, 2)))
    np.testing.assert_allclose(rms, [0.5, 0.6, 0.8], rtol=0.02)


def test_decode_c64_layout():
    dims, _, c = si.decode_config(2, with_weights=False)
    assert c["R"] == 64 and int(c["cu_window"][-1]) == 448
    assert np.all((c["kv_len"] >= 512) & (c["kv_len"] <= 4096))
    assert np.all((c["n_rej"] >= 0) & (c["n_rej"] <= 6))
    cap = c["kv_len"].astype(np.int64) + 14
    np.testing.assert_array_equal(c["kv_base"][1:], np.cumsum(cap)[:-1])
    kc = c["k_cache"].view(np.uint16)
    for r in (0, 31, 63):
        b, n = int(c["kv_base"][r]), int(c["kv_len"][r])
        assert np.all(kc[b + n:b + n + 14] == si.SENTINEL_BF16)
        assert not np.any(kc[b:b + n] == si.SENTINEL_BF16)
