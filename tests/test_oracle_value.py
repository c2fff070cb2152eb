"""Pins for the oracle's W_UV up-projection and gate (no GPU).

* a per-element brute force (explicit sums) on a small case;
* an identity weight returns the first 128 latent columns;
* heads are independent: permuting heads of latent and W_UV permutes the
  output heads;
* gate = 0 halves the projection exactly (sigmoid(0) = 1/2); a large gate
  leaves it, a large negative gate zeroes it;
* the gate column of (head h, value v) is 128 h + v.
"""

import numpy as np
import torch

from oracle import v_up_proj
from head_latent_attention_sparse_amd.workloads import bf16_bits


def bits(x):
    return bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand(shape, seed, std=1.0):
    return bits(np.random.default_rng(seed).standard_normal(shape) * std)


def test_brute_force_small():
    lat, w, gate = rand((2, 2, 512), 1), rand((2, 512, 128), 2, 0.05), rand((2, 256), 3)
    got = v_up_proj(lat, w, gate)
    x, ww, gg = f64(lat), f64(w), f64(gate)
    for t in range(2):
        for h in range(2):
            for v in range(0, 128, 9):
                s = 0.0
                for l in range(512):
                    s += x[t, h, l] * ww[h, l, v]
                s *= 1.0 / (1.0 + np.exp(-gg[t, 128 * h + v]))
                assert abs(got[t, h, v] - s) <= 1e-12 * (1 + abs(s))


def test_identity_weight():
    lat = rand((5, 3, 512), 4)
    w = np.zeros((3, 512, 128), np.float32)
    w[:, :128, :] = np.eye(128)
    np.testing.assert_array_equal(v_up_proj(lat, bits(w)), f64(lat)[:, :, :128])


def test_heads_are_independent():
    lat, w = rand((4, 5, 512), 5), rand((5, 512, 128), 6, 0.05)
    perm = np.array([3, 0, 4, 1, 2])
    np.testing.assert_allclose(v_up_proj(lat[:, perm], w[perm]), v_up_proj(lat, w)[:, perm], rtol=0, atol=1e-12)


def test_gate_values_and_columns():
    lat, w = rand((3, 2, 512), 7), rand((2, 512, 128), 8, 0.05)
    base = v_up_proj(lat, w)
    np.testing.assert_array_equal(v_up_proj(lat, w, bits(np.zeros((3, 256)))), base * 0.5)
    np.testing.assert_allclose(v_up_proj(lat, w, bits(np.full((3, 256), 60.0))), base, rtol=1e-20, atol=0)
    assert np.all(np.abs(v_up_proj(lat, w, bits(np.full((3, 256), -60.0)))) < 1e-20 * (1 + np.abs(base)))
    g = np.zeros((3, 256), np.float32)
    g[:, 128 + 5] = -60.0  # head 1, value 5 only
    out = v_up_proj(lat, w, bits(g))
    assert np.all(np.abs(out[:, 1, 5]) < 1e-20) and np.all(out[:, 0, 5] == base[:, 0, 5] * 0.5)
