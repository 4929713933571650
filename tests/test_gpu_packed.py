"""GPU parity of the packed weight layout.

The packing itself is compared bit for bit with a plain pad / reshape /
permute of the row-major matrix.  Every call that takes packed weights is
compared with the same call on the row-major weight: bit for bit where both
take the same plan (17 to 160 activation rows, and the LM head's 160-row slabs
above that, whose per-element reduction order is that of a 160-row call), and
with the oracle where the row-major layout takes another kernel (up to 16
rows, the fc above 160 rows).  Shapes are ragged (vocabularies off the 16-row
tile, hidden sizes off the 128-column block) and include the full-size LM head
and fc of the 16-sequence workloads."""
import numpy as np
import pytest
import torch

import oracle
from workloads import synth
from gpu_util import RING_CASES, check_draft, dev, host_bits, log, max_rel_err, ring_tiles

pytestmark = pytest.mark.gpu


def _bdr():
    import block_draft_readout_amd as bdr
    return bdr


def _reference_packing(w: torch.Tensor) -> torch.Tensor:
    """packed[c][t][i][g][r][e] = w[16 t + r][128 c + 32 i + 8 g + e], zero
    outside w, as uint8 bytes."""
    rows, cols = w.shape
    T, C = (rows + 15) // 16, (cols + 127) // 128
    p = torch.zeros((T * 16, C * 128), dtype=w.dtype, device=w.device)
    p[:rows, :cols] = w
    # [t][r][c][i][g][e] -> [c][t][i][g][r][e]
    return (p.view(T, 16, C, 4, 4, 8).permute(2, 0, 3, 4, 1, 5).contiguous().view(-1)
            .view(torch.uint8))


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    iv = torch.int32 if a.dtype == torch.float32 else torch.int16
    return bool((a.view(iv) == b.view(iv)).all())


def _randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)


@pytest.mark.parametrize("rows,cols", [(1, 8), (16, 128), (17, 136), (37, 392), (5003, 520),
                                       (151936, 5120), (5120, 25600)])
def test_pack_weight_layout(rows, cols):
    """The packed copy, bit for bit, ragged rows and columns included, up to the
    LM head and fc of the 16-sequence workloads."""
    bdr = _bdr()
    w = _randn_bf16((rows, cols), rows * 7 + cols)
    log(f"pack [{rows}, {cols}]")
    p = bdr.pack_weight(w)
    assert p.data.numel() == bdr.lib().bdr_packed_weight_bytes(rows, cols)
    assert torch.equal(p.data, _reference_packing(w))


@pytest.mark.parametrize("M", [1, 8, 16, 17, 100, 128, 160, 161, 330])
def test_lm_head_packed(M):
    """The LM head on packed weights (V = 5003, H = 392: a ragged last tile and a
    partial last 128-column block) against the oracle at every row count, and
    bit for bit against the row-major call where the plans agree."""
    bdr = _bdr()
    V, H = 5003, 392
    rng = np.random.default_rng(500 + M)
    hid = synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    lm_w = synth.to_bf16_bits((rng.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32))
    hd, wd = dev(hid), dev(lm_w)
    pw = bdr.pack_weight(wd)
    log(f"packed LM head M={M} V={V} H={H}")
    got = bdr.dspark_lm_head(hd, pw)
    err = max_rel_err(got.cpu().numpy(), oracle.lm_head(hid, lm_w, "bf16"))
    log(f"  max rel err {err:.3e}")
    assert err <= 1e-3
    if 16 < M <= 160:
        assert _bits_equal(got, bdr.dspark_lm_head(hd, wd))
    elif M > 160:
        for m0 in range(0, M - M % 160, 160):
            assert _bits_equal(got[m0:m0 + 160], bdr.dspark_lm_head(hd[m0:m0 + 160], wd))


@pytest.mark.parametrize("M,T,H", [(8, 2, 256), (17, 1, 160), (40, 3, 256), (144, 5, 512),
                                   (160, 2, 128), (200, 2, 256)])
def test_fc_packed(M, T, H):
    """The fc on packed weights (tap segments, split K) against the oracle, and
    bit for bit against the row-major call for 17 to 160 rows."""
    bdr = _bdr()
    rng = np.random.default_rng(600 + M * 10 + T)
    taps = [synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32)) for _ in range(T)]
    fc_w = synth.to_bf16_bits((rng.standard_normal((H, T * H)) / np.sqrt(T * H)).astype(np.float32))
    td, wd = [dev(t) for t in taps], dev(fc_w)
    log(f"packed fc rows={M} taps={T} H={H}")
    got = bdr.dflash_fuse_fc(td, bdr.pack_weight(wd))
    err = max_rel_err(oracle.widen(host_bits(got), "bf16"), oracle.fuse_fc(taps, fc_w, "bf16"))
    log(f"  max rel err {err:.3e}")
    assert err <= 4e-3
    if 16 < M <= 160:
        assert _bits_equal(got, bdr.dflash_fuse_fc(td, wd))


def test_packed_rejects_multi_tap_hidden_off_block():
    """A multi-tap fc with packed weights needs H % 128 == 0."""
    bdr = _bdr()
    H, T = 160, 2
    taps = [_randn_bf16((20, H), 1 + t) for t in range(T)]
    pw = bdr.pack_weight(_randn_bf16((H, T * H), 9))
    with pytest.raises(bdr.BdrError) as e:
        bdr.dflash_fuse_fc(taps, pw)
    assert e.value.code == bdr._abi.BDR_EUNSUPPORTED


@pytest.mark.parametrize("mt,ring", RING_CASES)
def test_packed_every_ring_lm_head(mt, ring):
    """Every ring depth forced through the plan override on two row ranges (two
    passes a wave, empty slots, ragged last tile, partial last block): packed
    and row-major weights give the same bits."""
    bdr = _bdr()
    T = ring_tiles(mt, ring)
    M, N, H = 16 * mt - 3, 2 * 4 * T * 16 - 5, 392
    hid = _randn_bf16((M, H), mt * 100 + ring)
    lm_w = _randn_bf16((N, H), mt * 100 + ring + 1, H ** -0.5)
    pw = bdr.pack_weight(lm_w)
    bdr.set_row_split_override(ring, 2, 0)
    try:
        got = bdr.dspark_lm_head(hid, pw)
        ref = bdr.dspark_lm_head(hid, lm_w)
        torch.cuda.synchronize()
    finally:
        bdr.set_row_split_override(0, 0, 0)
    log(f"packed ring {ring}, {mt} row tiles: LM head M={M} N={N} H={H}")
    assert _bits_equal(got, ref)


@pytest.mark.parametrize("mt,ring", RING_CASES)
def test_packed_every_ring_fc_split_k(mt, ring):
    """The same on a two-tap fc with its K range split in two."""
    bdr = _bdr()
    T = ring_tiles(mt, ring)
    H = (64 * T + 127) // 128 * 128
    rows = 16 * mt - 3
    taps = [_randn_bf16((rows, H), mt * 1000 + ring + t) for t in range(2)]
    fc_w = _randn_bf16((H, 2 * H), mt * 1000 + ring + 7, (2 * H) ** -0.5)
    pw = bdr.pack_weight(fc_w)
    bdr.set_row_split_override(ring, 1, 2)
    try:
        got = bdr.dflash_fuse_fc(taps, pw)
        ref = bdr.dflash_fuse_fc(taps, fc_w)
        torch.cuda.synchronize()
    finally:
        bdr.set_row_split_override(0, 0, 0)
    log(f"packed ring {ring}, {mt} row tiles: fc rows={rows} H={H} split K")
    assert _bits_equal(got, ref)


@pytest.mark.parametrize("lm_rows,fc_rows,H,T,V", [(32, 40, 512, 5, 30011), (128, 144, 5120, 5, 151936),
                                                   (32, 40, 2560, 5, 151936), (80, 96, 1024, 5, 60011),
                                                   (112, 128, 2048, 3, 90011)])
def test_fused_fc_lm_head_packed(lm_rows, fc_rows, H, T, V):
    """dflash_fuse_fc_lm_head with both weights packed gives the bits of the
    row-major call (one launch or two, as the plan decides), at small and mid
    shapes (five and seven LM row tiles: the register ring beside the fc) and at
    the 16- and 4-sequence sizes."""
    bdr = _bdr()
    taps = [_randn_bf16((fc_rows, H), 30 + t) for t in range(T)]
    fc_w = _randn_bf16((H, T * H), 40, (T * H) ** -0.5)
    hid = _randn_bf16((lm_rows, H), 41)
    lm_w = _randn_bf16((V, H), 42, H ** -0.5)
    log(f"packed fused fc + LM head: lm rows={lm_rows} fc rows={fc_rows} H={H} T={T} V={V}")
    f_p, z_p = bdr.dflash_fuse_fc_lm_head(taps, bdr.pack_weight(fc_w), hid, bdr.pack_weight(lm_w))
    f_r, z_r = bdr.dflash_fuse_fc_lm_head(taps, fc_w, hid, lm_w)
    assert _bits_equal(z_p, z_r)
    assert _bits_equal(f_p, f_r)
    with pytest.raises(ValueError):
        bdr.dflash_fuse_fc_lm_head(taps, fc_w, hid, bdr.pack_weight(lm_w))


@pytest.mark.parametrize("B,k,noalloc", [(4, 8, False), (16, 8, False), (16, 8, True), (1, 8, False)])
def test_draft_block_packed(B, k, noalloc):
    """The draft block with a packed LM head: tokens and logits equal the
    row-major call's for 17 to 160 rows; at B = 1 (8 rows, another LM-head
    kernel) the logits are within the oracle's bar and every draft position
    passes the oracle's rule."""
    bdr = _bdr()
    V, H, r = 20011, 512, 16
    rng = np.random.default_rng(700 + B * 10 + int(noalloc))
    hid = synth.to_bf16_bits(rng.standard_normal((B, k, H)).astype(np.float32))
    lm_w = synth.to_bf16_bits((rng.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32))
    w1 = synth.to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32))
    w2 = synth.to_bf16_bits((rng.standard_normal((V, r)) * 0.3).astype(np.float32))
    prev = rng.integers(0, V, B).astype(np.int32)
    hd, wd, w1d, w2d, pd = dev(hid), dev(lm_w), dev(w1), dev(w2), dev(prev)
    pw = bdr.pack_weight(wd)
    log(f"packed draft block B={B} k={k} V={V} noalloc={noalloc}")
    z_p = torch.empty((B, k, V), dtype=torch.float32, device="cuda")
    z_r = torch.empty_like(z_p)
    call = bdr.dspark_draft_block_noalloc if noalloc else bdr.dspark_draft_block
    d_p = call(hd, pw, w1d, w2d, pd, logits_out=z_p)
    d_r = call(hd, wd, w1d, w2d, pd, logits_out=z_r)
    if B * k > 16:
        assert _bits_equal(z_p, z_r)
        assert torch.equal(d_p, d_r)
    else:
        Z = oracle.lm_head(hid.reshape(B * k, H), lm_w, "bf16").reshape(B, k, V)
        assert max_rel_err(z_p.cpu().numpy(), Z) <= 1e-3
        check_draft(d_p.cpu().numpy(), z_p.cpu().numpy(), w1, w2, prev, "bf16")


def test_fc_rows_packed():
    """The gathered-row fc with packed weights gives the row-major call's bits."""
    bdr = _bdr()
    T, H, rows, max_rows = 3, 256, 64, 48
    taps = [_randn_bf16((rows, H), 80 + t) for t in range(T)]
    fc_w = _randn_bf16((H, T * H), 90, (T * H) ** -0.5)
    g = torch.Generator().manual_seed(5)
    idx = torch.randperm(rows, generator=g)[:max_rows].to(torch.int32).cuda()
    cnt = torch.tensor([37], dtype=torch.int32, device="cuda")
    log(f"packed gathered fc rows={rows} max_rows={max_rows} count=37")
    got = bdr.dflash_fuse_fc_rows(taps, bdr.pack_weight(fc_w), idx, cnt, max_rows)
    ref = bdr.dflash_fuse_fc_rows(taps, fc_w, idx, cnt, max_rows)
    assert _bits_equal(got, ref)


@pytest.mark.parametrize("M", [112, 128])
def test_full_size_lm_head_packed(M):
    """The 16-sequence LM head (V = 151936, H = 5120) at the bench's launch
    configuration: packed and row-major weights give the same bits; sampled
    rows against the oracle."""
    bdr = _bdr()
    V, H = 151936, 5120
    hid = _randn_bf16((M, H), 11 + M)
    lm_w = _randn_bf16((V, H), 12, H ** -0.5)
    log(f"full-size packed LM head M={M}")
    got = bdr.dspark_lm_head(hid, bdr.pack_weight(lm_w))
    ref = bdr.dspark_lm_head(hid, lm_w)
    assert _bits_equal(got, ref)
    rows = [0, M // 2, M - 1]
    vs = torch.arange(0, V, 997, device="cuda")
    want = oracle.lm_head(host_bits(hid[rows]), host_bits(lm_w[vs]), "bf16")
    assert max_rel_err(got[rows][:, vs].cpu().numpy(), want) <= 1e-3
