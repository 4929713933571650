"""The drafter fc and the LM head in one call (dflash_fuse_fc_lm_head): the
logits equal dspark_lm_head's bit for bit and the fc output is within the bf16
bar of the oracle, at the full sizes of the batched workloads (one launch
shared by both matrices) and on shapes that fall back to two launches."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from workloads import synth
from gpu_util import REL_TOL, dev, host_bits, log, max_rel_err, oracle_step, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bdr():
    import block_draft_readout_amd as m
    return m


@pytest.mark.parametrize("name", ["flashnext_b4", "b16", "adaptive_b16"])
def test_fc_lm_head_full_size(name):
    w = workloads.get(name)
    ref = oracle_step(name)
    W = weights(name)
    s = ref["step"]
    gW = {k: dev(W[k]) for k in ("fc_w", "lm_w")}
    taps = [dev(t) for t in s["taps"]]
    hid = dev(s["draft_hidden"])
    m = bdr()
    need = m.lib().dflash_fuse_fc_lm_head_workspace_bytes(w.rows, w.hidden, w.n_taps,
                                                           w.batch * w.k, w.vocab, m.BDR_BF16)
    F, Z = m.dflash_fuse_fc_lm_head(taps, gW["fc_w"], hid, gW["lm_w"])
    Zs = m.dspark_lm_head(hid, gW["lm_w"])
    torch.cuda.synchronize()
    errF = max_rel_err(oracle.widen(host_bits(F), w.dtype), ref["F"])
    log(f"{name}: workspace {need} B; fc rel err {errF:.2e}; logits equal the LM head's: "
        f"{bool(torch.equal(Z, Zs))}")
    assert torch.equal(Z, Zs)
    assert errF <= 4e-3
    # repeatable, and reusing the workspace
    ws = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    F2, Z2 = m.dflash_fuse_fc_lm_head(taps, gW["fc_w"], hid, gW["lm_w"], workspace=ws)
    F3, Z3 = m.dflash_fuse_fc_lm_head(taps, gW["fc_w"], hid, gW["lm_w"], workspace=ws)
    assert torch.equal(F2, F3) and torch.equal(Z2, Z3) and torch.equal(F, F2)


@pytest.mark.parametrize("B,k,H,T,V", [(2, 8, 256, 5, 5003), (3, 6, 512, 3, 20011),
                                       (9, 16, 128, 8, 4099), (1, 7, 256, 5, 3001)])
def test_fc_lm_head_shapes(B, k, H, T, V):
    """Row tiles from 2 to 10 (one launch), and B = 1 (two launches)."""
    g = np.random.default_rng(B * 100 + k)
    rows = B * (k + 1)
    taps = [synth.to_bf16_bits(g.standard_normal((rows, H)).astype(np.float32)) for _ in range(T)]
    fc_w = synth.to_bf16_bits((g.standard_normal((H, T * H)) / np.sqrt(T * H)).astype(np.float32))
    hid = synth.to_bf16_bits(g.standard_normal((B, k, H)).astype(np.float32))
    lm = synth.to_bf16_bits((g.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32))
    m = bdr()
    F, Z = m.dflash_fuse_fc_lm_head([dev(t) for t in taps], dev(fc_w), dev(hid), dev(lm))
    Zs = m.dspark_lm_head(dev(hid), dev(lm))
    torch.cuda.synchronize()
    errF = max_rel_err(oracle.widen(host_bits(F), "bf16"), oracle.fuse_fc(taps, fc_w, "bf16"))
    errZ = max_rel_err(Z.cpu().numpy(), oracle.lm_head(hid, lm, "bf16"))
    log(f"fc+lm B={B} k={k} H={H} T={T} V={V}: fc {errF:.2e} logits {errZ:.2e}")
    assert torch.equal(Z, Zs)
    assert errF <= 4e-3 and errZ <= 1e-3


def test_fc_lm_head_fp32_falls_back():
    w = workloads.get("tiny")
    W = synth.make_weights(w)
    s = synth.make_step(w, 0, noise=False)
    m = bdr()
    F, Z = m.dflash_fuse_fc_lm_head([dev(t) for t in s["taps"]], dev(W["fc_w"]),
                                    dev(s["draft_hidden"]), dev(W["lm_w"]))
    torch.cuda.synchronize()
    assert max_rel_err(F.cpu().numpy(), oracle.fuse_fc(s["taps"], W["fc_w"], "f32")) <= REL_TOL["f32"]
    assert max_rel_err(Z.cpu().numpy(), oracle.lm_head(s["draft_hidden"], W["lm_w"], "f32")) <= 1e-4
