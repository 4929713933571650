"""Host-side checks of the C-ABI library: it loads without a GPU, exports every
symbol include/bdr.h declares, sizes workspaces, and rejects invalid arguments
with the documented codes before touching the device (no compute calls here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bdr.h")


@pytest.fixture(scope="module")
def L():
    from block_draft_readout_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from block_draft_readout_amd import build
        build.build()
    return _abi.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_header_declares_the_three_path_calls():
    names = _declared()
    for n in ("dflash_fuse_fc", "dspark_draft_block", "spec_verify_greedy"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_binding_declares_every_header_symbol():
    from block_draft_readout_amd import _abi
    assert sorted(_abi.SIGNATURES) == _declared()


def test_version(L):
    assert L.bdr_abi_version() == 11


def test_workspace_sizes(L):
    from block_draft_readout_amd import _abi
    a256 = lambda x: (x + 255) // 256 * 256
    # per-position keys [k][16 groups][B] | per-workgroup slots [k][256][B]
    # two words apart | tokens [k][B] one per 128-byte line (all uint64) | a
    # completion-counter block | an error block
    markov = lambda B, k: a256(8 * 16 * B * k) + a256(16 * 256 * B * k) + a256(128 * B * k) + 256 + 256
    assert L.dspark_markov_workspace_bytes(16, 8) == markov(16, 8)
    assert L.dspark_markov_workspace_bytes(1, 7) == markov(1, 7)
    V = 151936
    with_logits = L.dspark_draft_workspace_bytes(16, 8, V, 1)
    assert with_logits == markov(16, 8) + a256(16 * 8 * V * 4)
    assert L.dspark_draft_workspace_bytes(16, 8, V, 0) == markov(16, 8)
    v = L.spec_verify_workspace_bytes(16, 8, V)
    assert v > 0 and v % 256 == 0
    # fc: split-K partials only when K is split
    assert L.dflash_fuse_fc_workspace_bytes(8, 5120, 5, _abi.BDR_BF16) > 0
    assert L.dflash_fuse_fc_workspace_bytes(0, 5120, 5, _abi.BDR_BF16) == 0
    # invalid shapes size to 0
    assert L.dflash_fuse_fc_workspace_bytes(8, 5120, 9, _abi.BDR_BF16) == 0
    assert L.spec_verify_workspace_bytes(1, 17, V) == 0


def _rc(L, fn, *args):
    return getattr(L, fn)(*args)


def test_fc_argument_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)  # never dereferenced: every call below fails validation first
    taps = (C.c_void_p * 5)(*([4096] * 5))
    assert L.dflash_fuse_fc(None, 5, 8, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EINVAL
    assert L.dflash_fuse_fc(taps, 0, 8, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EINVAL
    assert L.dflash_fuse_fc(taps, 9, 8, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EUNSUPPORTED
    assert L.dflash_fuse_fc(taps, 5, -1, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EINVAL
    assert L.dflash_fuse_fc(taps, 5, 8, 0, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EINVAL
    assert L.dflash_fuse_fc(taps, 5, 8, 5120, 7, P, P, None, 0, None) == A.BDR_EINVAL
    assert L.dflash_fuse_fc(taps, 5, 8, 5121, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EUNSUPPORTED
    assert L.dflash_fuse_fc(taps, 5, 8, 5120, A.BDR_BF16, None, P, None, 0, None) == A.BDR_EINVAL
    assert L.dflash_fuse_fc(taps, 5, 8, 5120, A.BDR_BF16, C.c_void_p(4098), P, None, 0, None) == A.BDR_EINVAL
    bad = (C.c_void_p * 5)(4096, 4096, None, 4096, 4096)
    assert L.dflash_fuse_fc(bad, 5, 8, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EINVAL
    assert b"taps[2]" in L.bdr_last_error()
    # split-K workspace required
    assert L.dflash_fuse_fc(taps, 5, 8, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_EWORKSPACE
    assert L.dflash_fuse_fc(taps, 5, 8, 5120, A.BDR_BF16, P, P, C.c_void_p(4096), 16, None) == A.BDR_EWORKSPACE
    assert L.dflash_fuse_fc(taps, 5, 8, 5120, A.BDR_BF16, P, P, C.c_void_p(4096 + 16), 1 << 30, None) == A.BDR_EWORKSPACE
    # rows == 0 is a no-op that succeeds without touching the device
    assert L.dflash_fuse_fc(taps, 5, 0, 5120, A.BDR_BF16, P, P, None, 0, None) == A.BDR_OK


def test_lm_head_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    assert L.dspark_lm_head(P, 7, 5120, 0, A.BDR_BF16, P, P, None) == A.BDR_EINVAL
    assert L.dspark_lm_head(P, 7, 5120, 1 << 31, A.BDR_BF16, P, P, None) == A.BDR_EUNSUPPORTED
    assert L.dspark_lm_head(P, 7, 5124, 1000, A.BDR_BF16, P, P, None) == A.BDR_EUNSUPPORTED
    assert L.dspark_lm_head(None, 7, 5120, 1000, A.BDR_BF16, P, P, None) == A.BDR_EINVAL
    assert L.dspark_lm_head(P, 0, 5120, 1000, A.BDR_BF16, P, P, None) == A.BDR_OK


def test_fp8_workspace_and_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    taps = (C.c_void_p * 5)(*([4096] * 5))
    # split-K partials: of all rows (one pass, <= 160 rows) or of one 16-row slab
    ws = L.dflash_fuse_fc_fp8_workspace_bytes(8, 5120, 5)
    assert ws > 0 and ws % 256 == 0
    assert L.dflash_fuse_fc_fp8_workspace_bytes(128, 5120, 5) % 256 == 0
    assert (L.dflash_fuse_fc_fp8_workspace_bytes(400, 192, 3)
            == L.dflash_fuse_fc_fp8_workspace_bytes(16, 192, 3))
    assert L.dflash_fuse_fc_fp8_workspace_bytes(0, 5120, 5) == 0
    assert L.dflash_fuse_fc_fp8_workspace_bytes(8, 5120, 9) == 0
    assert L.dflash_fuse_fc_fp8_workspace_bytes(8, 5130, 5) == 0
    fc = L.dflash_fuse_fc_fp8
    assert fc(None, 5, 8, 5120, P, P, P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 0, 8, 5120, P, P, P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 9, 8, 5120, P, P, P, None, 0, None) == A.BDR_EUNSUPPORTED
    assert fc(taps, 5, 8, 5088, P, P, P, None, 0, None) == A.BDR_EUNSUPPORTED   # H % 64
    assert fc(taps, 5, -1, 5120, P, P, P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 5, 8, 5120, None, P, P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 5, 8, 5120, C.c_void_p(4104), P, P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 5, 8, 5120, P, None, P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 5, 8, 5120, P, C.c_void_p(4098), P, None, 0, None) == A.BDR_EINVAL
    assert fc(taps, 5, 8, 5120, P, P, P, None, 0, None) == A.BDR_EWORKSPACE
    assert fc(taps, 5, 0, 5120, P, P, P, None, 0, None) == A.BDR_OK
    lm = L.dspark_lm_head_fp8
    assert lm(P, 7, 5120, 0, P, P, P, None) == A.BDR_EINVAL
    assert lm(P, 7, 5120, 1 << 31, P, P, P, None) == A.BDR_EUNSUPPORTED
    assert lm(P, 7, 5100, 1000, P, P, P, None) == A.BDR_EUNSUPPORTED
    assert lm(None, 7, 5120, 1000, P, P, P, None) == A.BDR_EINVAL
    assert lm(P, 7, 5120, 1000, P, None, P, None) == A.BDR_EINVAL
    assert lm(P, 7, 5120, 1000, P, P, None, None) == A.BDR_EINVAL
    assert lm(P, 0, 5120, 1000, P, P, P, None) == A.BDR_OK
    rws = L.dflash_fuse_fc_rows_fp8_workspace_bytes(64, 5120, 5)
    assert rws > 5 * 64 * 5120 * 2 and rws % 256 == 0
    fr = L.dflash_fuse_fc_rows_fp8
    assert fr(taps, 5, 8, 5120, P, P, 64, P, P, P, None, 0, None) == A.BDR_EWORKSPACE
    assert fr(taps, 5, 8, 5120, None, P, 64, P, P, P, None, 0, None) == A.BDR_EINVAL
    assert fr(taps, 5, 8, 5100, P, P, 64, P, P, P, None, 0, None) == A.BDR_EUNSUPPORTED
    assert fr(taps, 5, 8, 5120, P, P, 0, P, P, P, None, 0, None) == A.BDR_OK


def test_hc_average_validation(L):
    from block_draft_readout_amd import _abi as A
    src = (C.c_void_p * 5)(*([4096] * 5))
    dst = (C.c_void_p * 5)(*([8192] * 5))
    f = L.dflash_hc_average
    ok = (8 * 5120, 5120)          # [hc, rows, H] strides for rows = 8
    assert f(src, 5, 4, 8, 5120, *ok, 7, dst, None) == A.BDR_EINVAL                 # dtype
    assert f(src, 0, 4, 8, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EINVAL
    assert f(src, 9, 4, 8, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EUNSUPPORTED
    assert f(src, 5, 0, 8, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EINVAL
    assert f(src, 5, 17, 8, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EUNSUPPORTED
    assert f(src, 5, 4, -1, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EINVAL
    assert f(src, 5, 4, 8, 5124, 8 * 5124, 5124, A.BDR_BF16, dst, None) == A.BDR_EUNSUPPORTED
    assert f(src, 5, 4, 8, 5120, 8 * 5120, 5112, A.BDR_BF16, dst, None) == A.BDR_EINVAL  # row stride < H
    assert f(src, 5, 4, 8, 5120, 8 * 5120 + 4, 5120, A.BDR_BF16, dst, None) == A.BDR_EINVAL
    assert f(None, 5, 4, 8, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EINVAL
    bad = (C.c_void_p * 5)(4096, 4096, 4100, 4096, 4096)
    assert f(bad, 5, 4, 8, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_EINVAL
    assert f(src, 5, 4, 0, 5120, *ok, A.BDR_BF16, dst, None) == A.BDR_OK


def test_markov_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    ws = C.c_void_p(4096)
    args = lambda B=16, k=8, V=1000, dt=A.BDR_BF16, w1=P, w2=P, r=64, prev=P, d=P, wp=ws, wn=4096, \
        st=None: L.dspark_markov_argmax(P, B, k, V, dt, w1, w2, r, prev, d, st, wp, wn, None)
    assert args(k=0) == A.BDR_EINVAL
    assert args(k=17) == A.BDR_EUNSUPPORTED
    assert args(r=129) == A.BDR_EUNSUPPORTED
    assert args(r=60) == A.BDR_EUNSUPPORTED          # not a multiple of 8 for bf16
    assert args(r=-1) == A.BDR_EINVAL
    assert args(w2=None) == A.BDR_EINVAL             # only one Markov matrix
    assert args(prev=None) == A.BDR_EINVAL
    assert args(B=-1) == A.BDR_EINVAL
    assert args(wp=None) == A.BDR_EWORKSPACE
    assert args(wn=8) == A.BDR_EWORKSPACE
    assert args(st=C.c_void_p(4098)) == A.BDR_EINVAL  # misaligned status word
    assert args(B=0) == A.BDR_OK


def test_draft_block_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    f = lambda **kw: L.dspark_draft_block(kw.get("h", P), kw.get("B", 16), kw.get("k", 8), 5120,
                                          kw.get("V", 151936), A.BDR_BF16, kw.get("lm", P), P, P,
                                          64, P, P, kw.get("lo", None), kw.get("st", None),
                                          kw.get("ws", P), kw.get("wn", 1024), None)
    assert f(h=None) == A.BDR_EINVAL
    assert f(lm=None) == A.BDR_EINVAL
    assert f(k=20) == A.BDR_EUNSUPPORTED
    assert f() == A.BDR_EWORKSPACE                   # logits need workspace when logits_out is NULL
    assert f(B=0) == A.BDR_OK


def test_verify_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    f = lambda **kw: L.spec_verify_greedy(kw.get("y", P), kw.get("dt", A.BDR_BF16), kw.get("B", 16),
                                          kw.get("k", 8), kw.get("V", 151936), kw.get("d", P),
                                          kw.get("c", None), 0.3, kw.get("bl", P), P, P, None,
                                          kw.get("acc", None), None, kw.get("ws", None),
                                          kw.get("wn", 0), None)
    assert f(y=None) == A.BDR_EINVAL
    assert f(dt=5) == A.BDR_EINVAL
    assert f(d=None) == A.BDR_EINVAL
    assert f(bl=None) == A.BDR_EINVAL
    assert f(acc=C.c_void_p(4100)) == A.BDR_EINVAL   # int64 counters must be 8-byte aligned
    assert f(k=0) == A.BDR_EINVAL
    assert f(V=0) == A.BDR_EINVAL
    assert f() == A.BDR_EWORKSPACE
    assert f(B=0) == A.BDR_OK


def test_sampling_workspace_sizes(L):
    a256 = lambda x: (x + 255) // 256 * 256
    markov = lambda B, k: a256(8 * 16 * B * k) + a256(16 * 256 * B * k) + a256(128 * B * k) + 256 + 256
    V = 151936
    # a greedy Markov workspace (the chain generates the draws' noise itself)
    assert L.dspark_markov_sample_workspace_bytes(1, 7, V) == markov(1, 7)
    assert L.dspark_markov_sample_workspace_bytes(16, 8, 1000) == markov(16, 8)
    assert L.dspark_markov_sample_workspace_bytes(1, 7, (1 << 21) + 1) == 0
    v = L.spec_verify_sample_workspace_bytes(16, 8, V)
    assert v > 0 and v % 256 == 0
    assert L.spec_verify_sample_workspace_bytes(1, 17, V) == 0


def test_sampling_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    ws = C.c_void_p(4096)
    m = lambda T=1.0, B=4, k=8, V=1000, r=64, x=P, prev=P, wp=ws, wn=4096: \
        L.dspark_markov_sample(P, B, k, V, A.BDR_BF16, P, P, r, prev, T, 7, P, x, None,
                               float("nan"), None, wp, wn, None)
    assert m(T=0.0) == A.BDR_EINVAL
    assert m(T=-1.0) == A.BDR_EINVAL
    assert m(T=float("nan")) == A.BDR_EINVAL
    assert m(T=float("inf")) == A.BDR_EINVAL
    assert m(T=1e-45) == A.BDR_EUNSUPPORTED           # 1 / T overflows
    assert m(x=None) == A.BDR_EINVAL                   # draft_logits are an output
    assert m(prev=None) == A.BDR_EINVAL
    assert m(k=17) == A.BDR_EUNSUPPORTED
    assert m(r=60) == A.BDR_EUNSUPPORTED
    assert m(wn=8) == A.BDR_EWORKSPACE
    assert m(B=0) == A.BDR_OK
    assert m(B=0, T=0.0) == A.BDR_EINVAL                # scalars are checked first
    v = lambda T=1.0, y=P, x=P, dt=A.BDR_BF16, B=4, wp=None, wn=0: \
        L.spec_verify_sample(y, dt, B, 8, 1000, P, x, None, 0.3, T, 7, P, P, P, None, None, wp, wn,
                             None)
    assert v(T=0.0) == A.BDR_EINVAL
    assert v(y=None) == A.BDR_EINVAL
    assert v(x=None) == A.BDR_EINVAL
    assert v(dt=3) == A.BDR_EINVAL
    assert v() == A.BDR_EWORKSPACE
    assert v(B=0) == A.BDR_OK
    n = lambda B=2, k=3, V=1000, sid=0, out=P: L.dspark_gumbel_noise(B, k, V, 1, sid, out, None)
    assert n(sid=-1) == A.BDR_EINVAL
    assert n(out=None) == A.BDR_EINVAL
    assert n(V=(1 << 21) + 1) == A.BDR_EUNSUPPORTED
    assert n(B=0) == A.BDR_OK


def test_loop_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    c = lambda B=4, k=7, nxt=P, acc=P, em=None: L.spec_commit(P, acc, P, None, B, k, nxt, em, None,
                                                              None, None, None, None)
    assert c(k=0) == A.BDR_EINVAL
    assert c(k=17) == A.BDR_EUNSUPPORTED
    assert c(B=-1) == A.BDR_EINVAL
    assert c(nxt=None) == A.BDR_EINVAL
    assert c(acc=None) == A.BDR_EINVAL
    assert c(em=C.c_void_p(4098)) == A.BDR_EINVAL        # int32 outputs 4-byte aligned
    assert c(B=0) == A.BDR_OK
    taps = (C.c_void_p * 2)(*([4096] * 2))
    f = lambda mr=8, rows=8, H=512, ri=P, rc=P, wn=0: L.dflash_fuse_fc_rows(
        taps, 2, rows, H, A.BDR_BF16, ri, rc, mr, P, P, None, wn, None)
    assert f(H=500) == A.BDR_EUNSUPPORTED
    assert f(ri=None) == A.BDR_EINVAL
    assert f(rc=None) == A.BDR_EINVAL
    assert f(mr=-1) == A.BDR_EINVAL
    assert f(mr=0) == A.BDR_OK
    need = L.dflash_fuse_fc_rows_workspace_bytes(8, 512, 2, A.BDR_BF16)
    a256 = lambda x: (x + 255) // 256 * 256
    assert need >= 2 * a256(8 * 512 * 2)
    assert f() == A.BDR_EWORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    from block_draft_readout_amd import _abi
    saved = _abi._lib
    try:
        _abi._lib = None
        with pytest.raises(ImportError):
            _abi.load(str(tmp_path / "missing.so"))
    finally:
        _abi._lib = saved


def test_row_split_override_drives_the_plan(L):
    """The plan override (host state only): invalid values are rejected, a
    forced K split resizes the fc's partial-sum workspace, and clearing it
    restores the planner's own plan."""
    from block_draft_readout_amd import _abi as A
    a256 = lambda x: (x + 255) // 256 * 256
    rows, H, T = 144, 5120, 5
    own = L.dflash_fuse_fc_workspace_bytes(rows, H, T, A.BDR_BF16)
    assert own > 0 and own % (rows * H * 4) == 0
    try:
        for bad in [(-1, 0, 0), (0, -1, 0), (0, 0, -1), (0, 1 << 21, 0), (0, 0, 257)]:
            assert L.bdr_set_row_split_override(*bad) == A.BDR_EINVAL, bad
        for ks in (2, 3, 16):
            assert L.bdr_set_row_split_override(0, 0, ks) == A.BDR_OK
            assert L.dflash_fuse_fc_workspace_bytes(rows, H, T, A.BDR_BF16) == a256(ks * rows * H * 4)
        # the fused fc + LM head is not planned as one launch meanwhile: its
        # workspace is the fc's alone
        fused = L.dflash_fuse_fc_lm_head_workspace_bytes(rows, H, T, 128, 151936, A.BDR_BF16)
        assert fused == a256(16 * rows * H * 4)
    finally:
        assert L.bdr_set_row_split_override(0, 0, 0) == A.BDR_OK
    assert L.dflash_fuse_fc_workspace_bytes(rows, H, T, A.BDR_BF16) == own


def test_packed_weight_bytes(L):
    """Bytes of the packed copy: ceil(rows / 16) tiles x ceil(cols / 128)
    blocks x 4096; 0 where the layout cannot hold the matrix."""
    assert L.bdr_packed_weight_bytes(151936, 5120) == 9496 * 40 * 4096
    assert L.bdr_packed_weight_bytes(5120, 25600) == 320 * 200 * 4096
    assert L.bdr_packed_weight_bytes(17, 136) == 2 * 2 * 4096
    assert L.bdr_packed_weight_bytes(1, 8) == 4096
    assert L.bdr_packed_weight_bytes(16, 12) == 0           # cols % 8
    assert L.bdr_packed_weight_bytes(0, 128) == 0
    assert L.bdr_packed_weight_bytes(16, -8) == 0
    assert L.bdr_packed_weight_bytes(1 << 20, 1 << 10) == 0  # 2^31 bytes
    assert L.bdr_packed_weight_bytes((1 << 20) - 16, 1 << 10) == (1 << 31) - 16 * 2048
    assert L.bdr_packed_weight_bytes(1 << 62, 1 << 40) == 0


def test_packed_weight_validation(L):
    from block_draft_readout_amd import _abi as A
    P = C.c_void_p(4096)
    Q = C.c_void_p(1 << 40)
    assert L.bdr_pack_weight(P, 16, 12, Q, None) == A.BDR_EUNSUPPORTED
    assert L.bdr_pack_weight(None, 16, 128, Q, None) == A.BDR_EINVAL
    assert L.bdr_pack_weight(P, 16, 128, None, None) == A.BDR_EINVAL
    assert L.bdr_pack_weight(P, 16, 128, C.c_void_p(4104), None) == A.BDR_EINVAL   # alignment
    assert L.bdr_pack_weight(P, 16, 128, C.c_void_p(4096 + 2048), None) == A.BDR_EINVAL
    assert b"overlaps" in L.bdr_last_error()


def test_packed_dtype_acceptance(L):
    """BDR_BF16_PACKED is taken by the GEMM calls (same workspace as bf16 where
    the plans agree, the 160-row slab's above) and refused, before the device,
    by the calls whose dtype describes something else."""
    from block_draft_readout_amd import _abi as A
    PK = A.BDR_BF16_PACKED
    assert L.dflash_fuse_fc_workspace_bytes(144, 5120, 5, PK) == \
        L.dflash_fuse_fc_workspace_bytes(144, 5120, 5, A.BDR_BF16)
    assert L.dflash_fuse_fc_workspace_bytes(400, 5120, 5, PK) == \
        L.dflash_fuse_fc_workspace_bytes(160, 5120, 5, A.BDR_BF16)
    assert L.dflash_fuse_fc_workspace_bytes(8, 5120, 5, PK) > 0
    assert L.dflash_fuse_fc_workspace_bytes(20, 160, 2, PK) == 0       # multi-tap H % 128
    assert L.dflash_fuse_fc_rows_workspace_bytes(144, 5120, 5, PK) == \
        L.dflash_fuse_fc_rows_workspace_bytes(144, 5120, 5, A.BDR_BF16)
    assert L.dflash_fuse_fc_lm_head_workspace_bytes(144, 5120, 5, 128, 151936, PK) == \
        L.dflash_fuse_fc_lm_head_workspace_bytes(144, 5120, 5, 128, 151936, A.BDR_BF16)
    P = C.c_void_p(4096)
    taps = (C.c_void_p * 2)(*([4096] * 2))
    assert L.dflash_fuse_fc(taps, 2, 20, 160, PK, P, P, None, 0, None) == A.BDR_EUNSUPPORTED
    assert b"128" in L.bdr_last_error()
    assert L.dspark_lm_head(P, 7, 5120, 1 << 20, PK, P, P, None) == A.BDR_EUNSUPPORTED  # 2^31 bytes
    assert L.dspark_lm_head(P, 0, 5120, 151936, PK, P, P, None) == A.BDR_OK
    # the Markov and verification dtypes describe their own operands
    assert L.dspark_markov_argmax(P, 1, 8, 1000, PK, P, P, 8, P, P, None, P, 1 << 20, None) == A.BDR_EINVAL
    assert L.spec_verify_greedy(P, PK, 16, 8, 151936, P, None, 0.3, P, P, P, None, None, None,
                                None, 0, None) == A.BDR_EINVAL
    hc = (C.c_void_p * 1)(4096)
    assert L.dflash_hc_average(hc, 1, 2, 8, 128, 1024, 128, PK, hc, None) == A.BDR_EINVAL
