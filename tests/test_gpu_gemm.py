"""GPU parity of the weight-streaming GEMM (drafter fc and LM head) across the
shapes that select each kernel variant: the row-split workgroup kernel for
bf16 with 2 to 10 A row tiles (tap segments, ranges walked in several passes,
ragged M / N / K, split K), the register kernel that fp32 with more than 16
rows takes, the tiled kernel above 160 rows, and the fallbacks just outside
those shapes.  Compared with
the oracle's float64 products."""
import dataclasses

import pytest
import torch

import oracle
import workloads
from workloads import synth
from gpu_util import RING_CASES, REL_TOL, dev, host_bits, log, max_rel_err, ring_tiles

pytestmark = pytest.mark.gpu


def _w(name, cid, base, **kw):
    return dataclasses.replace(workloads.get(base), cid=cid, name=name, fake_layers=0,
                               tap_layers=tuple(range(kw["n_taps"])), **kw)


# fc rows = batch * (k + 1), LM-head rows = batch * k
SHAPES = {
    # fc M=144 (3 tiles / wave), LM M=128 (2 tiles / wave); 512-byte tap segments
    "m144_seg512": _w("m144_seg512", 40, "b16", batch=16, k=8, hidden=256, n_taps=3,
                      vocab=3001, rank=16),
    # fc M=120 on 1 KB segments; LM M=100 with a ragged last tile and a ragged K block
    "m100_ragged": _w("m100_ragged", 41, "b16", batch=20, k=5, hidden=512, n_taps=5,
                      vocab=5003, rank=8),
    # LM K = 640 bytes: one full and one partial K block
    "m100_k640": _w("m100_k640", 42, "b16", batch=20, k=5, hidden=320, n_taps=2,
                    vocab=4099, rank=8),
    # fc M=36 / LM M=30: one tile per wave, two waves idle on the MFMAs
    "m36_flashnext_like": _w("m36_flashnext_like", 43, "flashnext_b4", batch=6, k=5,
                             hidden=512, n_taps=5, vocab=7001, rank=8),
    # LM M=160: the largest workgroup shape; fc M=176 falls back
    "m160": _w("m160", 44, "b16", batch=16, k=10, hidden=128, n_taps=2, vocab=2048, rank=8),
    # ranges longer than the load ring, crossing K-block boundaries:
    # LM M=112 over 40000 rows x 4 K blocks; LM M=30 over 60000 rows x 2 K blocks
    "m112_v40k": _w("m112_v40k", 47, "b16", batch=16, k=7, hidden=1024, n_taps=2,
                    vocab=40000, rank=8),
    "m30_v60k": _w("m30_v60k", 48, "flashnext_b4", batch=6, k=5, hidden=512, n_taps=2,
                   vocab=60000, rank=8),
    # ranges walked in two passes: LM M=112 over 100003 rows (25 tiles per range);
    # fp32 LM M=40 over 40000 rows (the register kernel)
    "m112_v100k": _w("m112_v100k", 49, "b16", batch=16, k=7, hidden=256, n_taps=2,
                     vocab=100003, rank=8),
    "f32_m40_v40k": _w("f32_m40_v40k", 50, "tiny", batch=8, k=5, hidden=64, n_taps=2,
                       vocab=40000, rank=8),
    # fp32: fc M=42, LM M=35 (the register kernel)
    "f32_m42": _w("f32_m42", 45, "tiny", batch=7, k=5, hidden=128, n_taps=2, vocab=2999,
                  rank=8),
    # fp32: LM M=140 and fc M=160 (the register kernel)
    "f32_m140": _w("f32_m140", 46, "tiny", batch=20, k=7, hidden=64, n_taps=2, vocab=1500,
                   rank=8),
    # tiled kernel (M > 160): fc M=300 (ragged row tile, ragged 160-column tile, split K over
    # 3 taps); LM M=275 over V=4100 (26 column tiles, the last ragged)
    "tile_m300": _w("tile_m300", 51, "b16", batch=25, k=11, hidden=512, n_taps=3, vocab=4100,
                    rank=8),
    # tiled kernel: fc M=1040 on H=2560 x 5 taps (5 row tiles x 16 column tiles, split K);
    # LM M=1000 over V=2000; LM head with V % 4 != 0 falls back to the register kernel
    "tile_m1040": _w("tile_m1040", 52, "flashnext_b4", batch=40, k=25, hidden=2560, n_taps=5,
                     vocab=2000, rank=8),
    "tile_fallback_v": _w("tile_fallback_v", 53, "b16", batch=20, k=9, hidden=256, n_taps=2,
                          vocab=1003, rank=8),
    # the wide (256 x 320, eight-wave) tile: LM M=4000 over V=5000 (ragged last row and column
    # tiles); fc M=4400 on the narrow tile
    "tile_wide_m4000": _w("tile_wide_m4000", 54, "b16", batch=400, k=10, hidden=512, n_taps=2,
                          vocab=5000, rank=8),
    # narrow tile with split K: fc M=520 over 4 taps of 1024 (21 tiles x 4 splits)
    "tile_split_m520": _w("tile_split_m520", 55, "b16", batch=40, k=12, hidden=1024, n_taps=4,
                          vocab=3000, rank=8),
}


def _data(w):
    return synth.make_weights(w), synth.make_step(w, 0, noise=False)


@pytest.mark.parametrize("name", list(SHAPES))
def test_fc_parity(name):
    import block_draft_readout_amd as bdr
    w = SHAPES[name]
    W, s = _data(w)
    log(f"fc {w.describe()} rows={w.rows}")
    ref = oracle.fuse_fc(s["taps"], W["fc_w"], w.dtype)
    out = bdr.dflash_fuse_fc([dev(t) for t in s["taps"]], dev(W["fc_w"]))
    err = max_rel_err(oracle.widen(host_bits(out), w.dtype), ref)
    log(f"  max rel err {err:.3e}")
    assert err <= (4e-3 if w.dtype == "bf16" else REL_TOL["f32"])


@pytest.mark.parametrize("name", list(SHAPES))
def test_lm_head_parity(name):
    import block_draft_readout_amd as bdr
    w = SHAPES[name]
    W, s = _data(w)
    log(f"lm head {w.describe()} rows={w.batch * w.k}")
    ref = oracle.lm_head(s["draft_hidden"], W["lm_w"], w.dtype)
    got = bdr.dspark_lm_head(dev(s["draft_hidden"]), dev(W["lm_w"])).cpu().numpy()
    err = max_rel_err(got, ref)
    log(f"  max rel err {err:.3e}")
    assert err <= min(REL_TOL[w.dtype], 1e-3)


def test_lm_head_repeat_is_bitwise_identical():
    """Fixed reduction order: two launches give the same bits."""
    import block_draft_readout_amd as bdr
    w = SHAPES["m144_seg512"]
    W, s = _data(w)
    h, lw = dev(s["draft_hidden"]), dev(W["lm_w"])
    a = bdr.dspark_lm_head(h, lw).cpu().numpy()
    b = bdr.dspark_lm_head(h, lw).cpu().numpy()
    assert (a.view("u4") == b.view("u4")).all()


@pytest.mark.parametrize("hidden", [2560, 5120])
def test_prefill_fc_parity_on_sampled_rows(hidden):
    """The prefill-shaped fc (4096 rows, five taps) through the tiled kernel,
    every output column of 96 sampled rows against the oracle."""
    import block_draft_readout_amd as bdr
    import numpy as np
    rows, T = 4096, 5
    cid = 60 + hidden // 2560
    taps = [synth.store(synth.normal_f32((rows, hidden), (cid, 1, 0, t)), "bf16") for t in range(T)]
    fc_w = synth.store(synth.normal_f32((hidden, T * hidden), (cid, 0, 0, 0),
                                        (1.0 / (T * hidden)) ** 0.5), "bf16")
    log(f"prefill fc rows={rows} H={hidden} T={T}")
    out = bdr.dflash_fuse_fc([dev(t) for t in taps], dev(fc_w))
    got = host_bits(out)
    sample = np.unique(np.concatenate([np.arange(0, rows, 43), [rows - 1, 255, 256, 4095 - 160]]))
    ref = oracle.fuse_fc([t[sample] for t in taps], fc_w, "bf16")
    err = max_rel_err(oracle.widen(got[sample], "bf16"), ref)
    log(f"  {sample.size} rows, max rel err {err:.3e}")
    assert err <= 4e-3


@pytest.mark.parametrize("mt,ring", RING_CASES)
def test_row_split_every_ring_lm_head(mt, ring):
    """Every ring depth built, forced through the plan
    override on two row ranges: two passes per wave with empty slots in the
    second, a ragged last tile, a partial last K block (H = 392)."""
    import block_draft_readout_amd as bdr
    import numpy as np
    T = ring_tiles(mt, ring)
    M, N, H = 16 * mt - 3, 2 * 4 * T * 16 - 5, 392
    rng = np.random.default_rng(mt * 100 + ring)
    hid = synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    lm_w = synth.to_bf16_bits((rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32))
    bdr.set_row_split_override(ring, 2, 0)
    try:
        got = bdr.dspark_lm_head(dev(hid), dev(lm_w)).cpu().numpy()
    finally:
        bdr.set_row_split_override(0, 0, 0)
    err = max_rel_err(got, oracle.lm_head(hid, lm_w, "bf16"))
    log(f"ring {ring}, {mt} row tiles: LM head M={M} N={N} H={H} ({T} tiles a wave): "
        f"max rel err {err:.3e}")
    assert err <= 1e-3


@pytest.mark.parametrize("mt,ring", RING_CASES)
def test_row_split_every_ring_fc_split_k(mt, ring):
    """The same on the fc: one row range of two passes per wave, two tap
    segments, the K range split in two (fp32 partials, ordered reduction)."""
    import block_draft_readout_amd as bdr
    import numpy as np
    T = ring_tiles(mt, ring)
    H = (64 * T + 127) // 128 * 128
    rows = 16 * mt - 3
    rng = np.random.default_rng(mt * 1000 + ring)
    taps = [synth.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32)) for _ in range(2)]
    fc_w = synth.to_bf16_bits((rng.standard_normal((H, 2 * H)) / np.sqrt(2 * H)).astype(np.float32))
    bdr.set_row_split_override(ring, 1, 2)
    try:
        out = bdr.dflash_fuse_fc([dev(t) for t in taps], dev(fc_w))
        torch.cuda.synchronize()
    finally:
        bdr.set_row_split_override(0, 0, 0)
    err = max_rel_err(oracle.widen(host_bits(out), "bf16"), oracle.fuse_fc(taps, fc_w, "bf16"))
    log(f"ring {ring}, {mt} row tiles: fc rows={rows} H={H} split K: max rel err {err:.3e}")
    assert err <= 4e-3


@pytest.mark.parametrize("M,N,H", [(17, 1, 128), (160, 17, 128), (33, 3, 256), (100, 65, 8),
                                   (48, 300, 136)])
def test_row_split_edge_shapes(M, N, H):
    """Row-split kernel at the edges: workgroups whose waves own no rows, a
    partial last K block (H = 136, 8), row counts just above a tile."""
    import block_draft_readout_amd as bdr
    import numpy as np
    rng = np.random.default_rng(M * 1000 + N)
    hid = synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    lm_w = synth.to_bf16_bits((rng.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32))
    got = bdr.dspark_lm_head(dev(hid), dev(lm_w)).cpu().numpy()
    ref = oracle.lm_head(hid, lm_w, "bf16")
    err = max_rel_err(got, ref)
    log(f"row-split edge M={M} N={N} H={H}: max rel err {err:.3e}")
    assert err <= 1e-3
