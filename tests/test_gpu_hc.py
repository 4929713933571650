"""GPU parity of the hyper-connection stream average (dflash_hc_average)
against oracle.hc: bit-exact on bf16 and fp32, stream-major and row-major
stream layouts, hc from 1 to 16, ragged rows, wide dynamic range and
subnormal-range means; then the fc on the averaged taps against the oracle's
fc of the oracle's averages."""
import numpy as np
import pytest

import oracle
from oracle import hc as ohc
from workloads import synth
from gpu_util import dev, host_bits, log, max_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_readout_amd as bdr
    bdr.lib()


def bdr():
    import block_draft_readout_amd as m
    return m


def _streams(rng, hc, rows, H, dtype, spread=0.0, scale=1.0):
    out = []
    for _ in range(hc):
        x = rng.standard_normal((rows, H)) * scale * np.exp(rng.uniform(-spread, spread, (rows, H)))
        out.append(synth.store(x.astype(np.float32), dtype))
    return out


def _captured(streams, layout):
    """Device [hc, rows, H] view of the streams in the given memory layout."""
    a = np.stack(streams)                                   # [hc, rows, H]
    if layout == "stream_major":
        return dev(a)
    t = dev(np.ascontiguousarray(a.transpose(1, 0, 2)))      # memory [rows, hc, H]
    return t.transpose(0, 1)                                 # view [hc, rows, H]


CASES = [("bf16", 1, 7, 64, "stream_major"), ("bf16", 2, 37, 2560, "stream_major"),
         ("bf16", 3, 16, 5120, "row_major"), ("bf16", 4, 9, 512, "row_major"),
         ("bf16", 5, 33, 136, "stream_major"), ("bf16", 16, 5, 1024, "row_major"),
         ("f32", 3, 11, 64, "stream_major"), ("f32", 8, 6, 2560, "row_major")]


@pytest.mark.parametrize("dtype,hc,rows,H,layout", CASES)
def test_hc_average_bit_exact(dtype, hc, rows, H, layout):
    rng = np.random.default_rng(hc * 100 + rows)
    T = 3
    taps = [_streams(rng, hc, rows, H, dtype, spread=6.0) for _ in range(T)]
    got = bdr().dflash_hc_average([_captured(s, layout) for s in taps])
    for t in range(T):
        ref = ohc.hc_average(taps[t], dtype)
        g = host_bits(got[t])
        same = g.view(np.uint32 if dtype == "f32" else np.uint16) == \
            ref.view(np.uint32 if dtype == "f32" else np.uint16)
        log(f"hc={hc} {dtype} rows={rows} H={H} {layout} tap {t}: {int(same.sum())}/{same.size} bit-exact")
        assert same.all()


def test_hc_average_subnormal_range_and_empty():
    rng = np.random.default_rng(7)
    streams = _streams(rng, 3, 8, 128, "bf16", spread=2.0, scale=2.0 ** -128)
    got = host_bits(bdr().dflash_hc_average([_captured(streams, "stream_major")])[0])
    ref = ohc.hc_average(streams, "bf16")
    assert np.array_equal(got, ref)
    empty = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    assert bdr().dflash_hc_average([empty])[0].shape == (0, 64)


def test_fc_on_averaged_taps():
    rng = np.random.default_rng(8)
    hc, rows, H, T = 4, 8, 2560, 5
    taps = [_streams(rng, hc, rows, H, "bf16") for _ in range(T)]
    fc_w = synth.store((rng.standard_normal((H, T * H)) / np.sqrt(T * H)).astype(np.float32), "bf16")
    avg = bdr().dflash_hc_average([_captured(s, "row_major") for s in taps])
    F = bdr().dflash_fuse_fc(avg, dev(fc_w))
    ref = oracle.fuse_fc([ohc.hc_average(s, "bf16") for s in taps], fc_w, "bf16")
    err = max_rel_err(oracle.widen(host_bits(F), "bf16"), ref)
    log(f"fc on hc-averaged taps: max rel err {err:.3e}")
    assert err <= 4e-3
