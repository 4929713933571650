"""Pins of the oracle's fc fusion (S1) and LM head (S2).

Pins used: block-identity fc weights (concat order, no dropped tap), one-hot rows
(weight orientation), a closed form with constant inputs, the width contract
printed on the pages, and exact vocab-slice boundaries of the LM head.
"""
import json
import os

import numpy as np
import pytest

from oracle import reference as ref

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _bits(x):
    return ref.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fc_block_identity_selects_each_tap(dtype):
    g = np.random.default_rng(1)
    T, rows, H = 5, 3, 8
    taps32 = [g.standard_normal((rows, H)).astype(np.float32) for _ in range(T)]
    taps = taps32 if dtype == "f32" else [_bits(t) for t in taps32]
    for t in range(T):
        W = np.zeros((H, T * H), dtype=np.float32)
        W[:, t * H:(t + 1) * H] = np.eye(H, dtype=np.float32)
        Wst = W if dtype == "f32" else _bits(W)
        F = ref.fuse_fc(taps, Wst, dtype)
        want = ref.widen(taps[t], dtype).astype(np.float32)
        assert np.array_equal(F, want), f"tap {t} not at columns [{t}*H, {t + 1}*H)"


def test_fc_one_hot_row_returns_weight_column():
    g = np.random.default_rng(2)
    T, rows, H = 3, 4, 6
    W = g.standard_normal((H, T * H)).astype(np.float32)
    for t0 in range(T):
        for h in range(H):
            taps = [np.zeros((rows, H), np.float32) for _ in range(T)]
            taps[t0][2, h] = 1.0
            F = ref.fuse_fc(taps, W, "f32")
            assert np.array_equal(F[2], W[:, t0 * H + h])
            assert not F[[0, 1, 3]].any()


def test_fc_constant_closed_form():
    T, rows, H = 5, 2, 16
    c = [0.5, -1.0, 2.0, 0.25, 3.0]
    taps = [np.full((rows, H), c[t], np.float32) for t in range(T)]
    W = np.ones((H, T * H), np.float32)
    F = ref.fuse_fc(taps, W, "f32")
    assert np.all(F == np.float32(H * sum(c)))


def test_fc_width_contract_flashnext_shape():
    fig = GOLDEN["flashnext_fc"]
    H, T = fig["hidden"], fig["n_taps"]
    assert fig["fc_weight_shape"] == [H, T * H]
    W = np.zeros(fig["fc_weight_shape"], np.uint16)
    taps = [np.zeros((1, H), np.uint16) for _ in range(T)]
    F = ref.fuse_fc(taps, W, "bf16")
    assert F.shape == (1, H) and not F.any()
    with pytest.raises(ValueError):
        ref.fuse_fc(taps[:4], W, "bf16")  # 4 taps x 2560 != 12800


def test_fc_width_contract_qwen27b():
    fig = GOLDEN["qwen27b_fc"]
    H, T = fig["hidden"], fig["n_taps"]
    assert len(fig["target_layer_ids"]) == T
    W = np.broadcast_to(np.uint16(0), (H, T * H))
    taps = [np.zeros((1, H), np.uint16) for _ in range(T)]
    with pytest.raises(ValueError):
        ref.fuse_fc(taps, W[:, :(T - 1) * H], "bf16")
    with pytest.raises(ValueError):
        ref.fuse_fc(taps[:3], W, "bf16")


def test_lm_head_one_hot_and_slice_boundaries():
    g = np.random.default_rng(3)
    H = 4
    V = ref.LM_HEAD_SLICE + 37
    lm = g.standard_normal((V, H)).astype(np.float32)
    hid = np.zeros((1, H, H), np.float32)
    for h in range(H):
        hid[0, h, h] = 1.0
    Z = ref.lm_head(hid, lm, "f32")
    assert Z.shape == (1, H, V)
    for h in range(H):
        assert np.array_equal(Z[0, h], lm[:, h])


def test_lm_head_constant_closed_form_bf16():
    B, k, H, V = 2, 3, 32, 100
    lm32 = np.repeat(np.arange(V, dtype=np.float32)[:, None] / 8.0, H, axis=1)
    hid = np.ones((B, k, H), np.float32)
    Z = ref.lm_head(_bits(hid), _bits(lm32), "bf16")
    want = (np.arange(V) / 8.0 * H).astype(np.float32)
    assert np.array_equal(Z, np.broadcast_to(want, (B, k, V)))


def test_lm_head_zero_hidden():
    lm = np.random.default_rng(4).standard_normal((50, 8)).astype(np.float32)
    assert not ref.lm_head(np.zeros((2, 2, 8), np.float32), lm, "f32").any()


def test_non_finite_inputs_rejected():
    W = np.zeros((2, 4), np.float32)
    taps = [np.array([[np.nan, 0.0]], np.float32), np.zeros((1, 2), np.float32)]
    with pytest.raises(ValueError):
        ref.fuse_fc(taps, W, "f32")
