"""dspark_draft_block_noalloc (the draft block with the chain's hand-off in the
library's static per-device scratch) against dspark_draft_block with a
workspace: tokens, logits and status identical, on two calls in a row, the
second with a smaller block (the scratch keeps the first call's contents), and
the size limit rejected before anything is launched."""
import numpy as np
import pytest

from workloads import synth
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def bdr():
    import block_draft_readout_amd as m
    return m


def _case(seed, B, k, V, H, r):
    g = np.random.default_rng(seed)
    hid = synth.to_bf16_bits(g.standard_normal((B, k, H)).astype(np.float32))
    lm = synth.to_bf16_bits((g.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32))
    w1 = synth.to_bf16_bits(g.standard_normal((V, r)).astype(np.float32))
    w2 = synth.to_bf16_bits((g.standard_normal((V, r)) * 0.3).astype(np.float32))
    prev = g.integers(0, V, B).astype(np.int32)
    return [dev(x) for x in (hid, lm, w1, w2, prev)]


def test_noalloc_draft_block_matches_the_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m = bdr()
    for seed, (B, k, V, H, r) in ((1, (16, 8, 151936, 256, 64)), (2, (3, 5, 20011, 128, 32))):
        log(f"no-alloc draft block B={B} k={k} V={V} H={H} r={r}")
        hid, lm, w1, w2, prev = _case(seed, B, k, V, H, r)
        lg_ref = torch.empty((B, k, V), dtype=torch.float32, device="cuda")
        st_ref = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        d_ref = m.dspark_draft_block(hid, lm, w1, w2, prev, logits_out=lg_ref, status=st_ref)
        lg = torch.full((B, k, V), float("nan"), dtype=torch.float32, device="cuda")
        d = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        m.dspark_draft_block_noalloc(hid, lm, w1, w2, prev, draft_tokens=d, logits_out=lg,
                                     status=st)
        torch.cuda.synchronize()
        assert torch.equal(d, d_ref)
        assert torch.equal(lg, lg_ref)
        assert int(st.item()) == 0 and int(st_ref.item()) == 0


def test_noalloc_rejects_blocks_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m = bdr()
    hid, lm, w1, w2, prev = _case(3, 64, 8, 4096, 64, 16)
    with pytest.raises(m.BdrError) as e:
        m.dspark_draft_block_noalloc(hid, lm, w1, w2, prev)
    assert e.value.code == m._abi.BDR_EUNSUPPORTED
