"""GPU parity of the fp8-weight fc and LM head (E4M3 codes with one fp32 scale
per output row, bf16 activations) against oracle.fp8.

* one-hot activations make every logit a single product scale * e4m3(code):
  compared bit-exactly, this pins the on-device decode of all 254 finite codes
  (subnormals included), the byte order inside each 16-code read and the
  reduction-index permutation shared by both operands;
* random shapes cover ragged K blocks, tap segments that blocks straddle,
  slabs of 16 rows (M > 16), split K and ragged row ranges;
* the Qwen3.8-27B-shaped LM head and fc at full size (weights quantised with
  the synthetic E4M3 recipe): sampled vocabulary rows / all fc outputs, and the
  Markov-biased draft computed from the fp8 logits against the oracle's chain
  under the near-tie protocol.
"""
import functools
import time

import numpy as np
import pytest

import oracle
import workloads
from oracle import fp8
from workloads import synth
from gpu_util import RING_CASES, check_draft, dev, host_bits, log, max_rel_err, ring_tiles

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LM_TOL = 1e-3       # fp32 logits: fp32 sums vs float64 sums
FC_TOL = 4e-3       # bf16 output: half an ulp of bf16 on top


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_readout_amd as bdr
    bdr.lib()


def bdr():
    import block_draft_readout_amd as m
    return m


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01          # NaN codes -> the largest finite magnitude
    return c


def _bf16(rng, shape, scale=1.0):
    return synth.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_one_hot_rows_decode_every_code_exactly():
    rng = np.random.default_rng(1)
    H, V = 1088, 768                       # one full and one partial K block
    pos = np.array([0, 7, 8, 15, 16, 63, 64, 100, 511, 512, 1000, 1023, 1024, 1030, 1087, 777])
    vals = np.array([1.0, -1.0, 0.5, 2.0] * 4, dtype=np.float32)
    hid = np.zeros((16, H), dtype=np.float32)
    hid[np.arange(16), pos] = vals
    hid = synth.to_bf16_bits(hid)
    q = _codes(rng, (V, H))
    q[:254, pos[0]] = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    s = (2.0 ** rng.integers(-4, 5, size=V)).astype(np.float32)
    got = bdr().dspark_lm_head_fp8(dev(hid), dev(q), dev(s)).cpu().numpy()
    want = (vals[:, None].astype(np.float64) * fp8.decode_e4m3(q[:, pos]).T
            * s[None, :].astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, want)
    assert np.array_equal(got, fp8.lm_head_fp8(hid, q, s, "bf16"))


# rows <= 16: one-wave kernel; 16 < rows <= 160: workgroup kernel with 1..3 A
# tiles per wave (ragged K, long ranges, passes); K = 192 x 3 taps: slabs
LM_CASES = [(1, 64, 1000), (7, 5120, 4099), (16, 1088, 3001), (23, 320, 2000), (40, 2560, 1500),
            (112, 1024, 40000), (30, 512, 60000), (144, 2048, 3001), (160, 512, 5003),
            (112, 256, 100003)]


@pytest.mark.parametrize("M,H,V", LM_CASES)
def test_lm_head_fp8_parity(M, H, V):
    rng = np.random.default_rng(M * 7 + H)
    hid = _bf16(rng, (M, H))
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((V, H)).astype(np.float32) / np.sqrt(H))
    got = bdr().dspark_lm_head_fp8(dev(hid), dev(q), dev(s)).cpu().numpy()
    ref = fp8.lm_head_fp8(hid, q, s, "bf16")
    err = max_rel_err(got, ref)
    log(f"lm head fp8 M={M} H={H} V={V}: max rel err {err:.3e}")
    assert err <= LM_TOL


def test_lm_head_fp8_random_codes_wide_range():
    rng = np.random.default_rng(2)
    M, H, V = 9, 2048, 2500
    hid = _bf16(rng, (M, H))
    q = _codes(rng, (V, H))
    s = (rng.random(V) * 2 + 1e-3).astype(np.float32)
    got = bdr().dspark_lm_head_fp8(dev(hid), dev(q), dev(s)).cpu().numpy()
    err = max_rel_err(got, fp8.lm_head_fp8(hid, q, s, "bf16"))
    log(f"lm head fp8, random codes: max rel err {err:.3e}")
    assert err <= LM_TOL


@pytest.mark.parametrize("mt,ring", RING_CASES)
def test_lm_head_fp8_every_ring(mt, ring):
    """Every ring depth of the row-split kernel with fp8 weights, forced
    through the plan override on two row ranges: two passes per wave with empty
    slots in the second, a ragged last tile, a partial last K block (H = 448)."""
    T = ring_tiles(mt, ring)
    M, V, H = 16 * mt - 3, 2 * 4 * T * 16 - 5, 448
    rng = np.random.default_rng(mt * 100 + ring + 7)
    hid = _bf16(rng, (M, H))
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((V, H)).astype(np.float32) / np.sqrt(H))
    bdr().set_row_split_override(ring, 2, 0)
    try:
        got = bdr().dspark_lm_head_fp8(dev(hid), dev(q), dev(s)).cpu().numpy()
    finally:
        bdr().set_row_split_override(0, 0, 0)
    err = max_rel_err(got, fp8.lm_head_fp8(hid, q, s, "bf16"))
    log(f"ring {ring}, {mt} row tiles: fp8 LM head M={M} V={V} H={H}: max rel err {err:.3e}")
    assert err <= LM_TOL


@pytest.mark.parametrize("mt,ring", RING_CASES)
def test_fc_fp8_every_ring_split_k(mt, ring):
    """The same on the fp8 fc: one row range, two tap segments, K split in two."""
    T = ring_tiles(mt, ring)
    H = (64 * T + 127) // 128 * 128
    rows = 16 * mt - 3
    rng = np.random.default_rng(mt * 1000 + ring + 7)
    taps = [_bf16(rng, (rows, H)) for _ in range(2)]
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((H, 2 * H)).astype(np.float32)
                                    / np.sqrt(2 * H))
    bdr().set_row_split_override(ring, 1, 2)
    try:
        out = bdr().dflash_fuse_fc_fp8([dev(t) for t in taps], dev(q), dev(s))
        torch.cuda.synchronize()
    finally:
        bdr().set_row_split_override(0, 0, 0)
    err = max_rel_err(oracle.widen(host_bits(out), "bf16"), fp8.fuse_fc_fp8(taps, q, s, "bf16"))
    log(f"ring {ring}, {mt} row tiles: fp8 fc rows={rows} H={H} split K: max rel err {err:.3e}")
    assert err <= FC_TOL


@pytest.mark.parametrize("rows,ring", [(80, 5), (144, 3)])
def test_fc_fp8_register_ring_partial_block(rows, ring):
    """The fp8 fc's register ring (K-split plans with five or more row tiles)
    on one tap with H = 192: the second 128-code block is partial, so its codes
    past K are cut from the operand loads; K forced into two splits."""
    H = 192
    rng = np.random.default_rng(rows * 10 + ring)
    taps = [_bf16(rng, (rows, H))]
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((H, H)).astype(np.float32) / np.sqrt(H))
    bdr().set_row_split_override(ring, 1, 2)
    try:
        out = bdr().dflash_fuse_fc_fp8([dev(t) for t in taps], dev(q), dev(s))
        torch.cuda.synchronize()
    finally:
        bdr().set_row_split_override(0, 0, 0)
    err = max_rel_err(oracle.widen(host_bits(out), "bf16"), fp8.fuse_fc_fp8(taps, q, s, "bf16"))
    log(f"fp8 fc register ring, partial block: rows={rows} H={H} ring {ring}: max rel err {err:.3e}")
    assert err <= FC_TOL


FC_CASES = [(5, 64, 5), (9, 192, 3), (8, 2560, 5), (36, 2560, 5), (8, 5120, 5), (20, 1024, 2),
            (128, 5120, 5), (144, 256, 3), (20, 192, 3), (40, 64, 5), (176, 512, 2)]


@pytest.mark.parametrize("rows,H,T", FC_CASES)
def test_fc_fp8_parity(rows, H, T):
    rng = np.random.default_rng(rows * 13 + H + T)
    taps = [_bf16(rng, (rows, H)) for _ in range(T)]
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((H, T * H)).astype(np.float32)
                                    / np.sqrt(T * H))
    out = bdr().dflash_fuse_fc_fp8([dev(t) for t in taps], dev(q), dev(s))
    got = oracle.widen(host_bits(out), "bf16")
    ref = fp8.fuse_fc_fp8(taps, q, s, "bf16")
    err = max_rel_err(got, ref)
    ws = bdr().workspace_bytes("fc_fp8", rows=rows, hidden=H, n_taps=T)
    log(f"fc fp8 rows={rows} H={H} T={T} (workspace {ws} B): max rel err {err:.3e}")
    assert err <= FC_TOL


def test_fp8_repeat_is_bitwise_identical_and_empty_is_a_noop():
    rng = np.random.default_rng(3)
    taps = [_bf16(rng, (8, 512)) for _ in range(5)]
    q = _codes(rng, (512, 2560))
    s = np.ones(512, np.float32)
    tg = [dev(t) for t in taps]
    a = host_bits(bdr().dflash_fuse_fc_fp8(tg, dev(q), dev(s)))
    b = host_bits(bdr().dflash_fuse_fc_fp8(tg, dev(q), dev(s)))
    assert np.array_equal(a, b)
    empty = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    out = bdr().dflash_fuse_fc_fp8([empty] * 5, dev(q), dev(s))
    assert out.shape == (0, 512)


@functools.lru_cache(maxsize=1)
def _qwen_fp8():
    w = workloads.get("qwen27b_b1")
    t0 = time.time()
    W = synth.make_weights_fp8(w)
    log(f"qwen27b_b1 fp8 weights in {time.time() - t0:.1f}s")
    return w, W


def test_qwen27b_fp8_fc_full_size():
    w, W = _qwen_fp8()
    s = synth.make_step(w, 0, noise=False)
    out = bdr().dflash_fuse_fc_fp8([dev(t) for t in s["taps"]], dev(W["fc_q"]), dev(W["fc_scale"]))
    got = oracle.widen(host_bits(out), "bf16")
    ref = fp8.fuse_fc_fp8(s["taps"], W["fc_q"], W["fc_scale"], "bf16")
    err = max_rel_err(got, ref)
    log(f"qwen27b fc fp8 rows={w.rows}: max rel err {err:.3e}")
    assert err <= FC_TOL


def test_qwen27b_fp8_draft_block():
    """LM head (fp8) -> Markov-biased argmax on the device, against the oracle's
    fp8 logits: logits on every vocabulary row, every draft position checked
    against the oracle's rule (context = the GPU's previous token)."""
    w, W = _qwen_fp8()
    s = synth.make_step(w, 0, noise=False)
    t0 = time.time()
    Z = fp8.lm_head_fp8(s["draft_hidden"], W["lm_q"], W["lm_scale"], "bf16")
    log(f"qwen27b fp8 oracle logits in {time.time() - t0:.1f}s")
    Zg = bdr().dspark_lm_head_fp8(dev(s["draft_hidden"]), dev(W["lm_q"]), dev(W["lm_scale"]))
    d = bdr().dspark_markov_argmax(Zg, dev(W["w1"]), dev(W["w2"]), dev(s["prev0"]))
    err = max_rel_err(Zg.cpu().numpy(), Z)
    c = check_draft(d.cpu().numpy(), Z, W["w1"], W["w2"], s["prev0"], w.dtype)
    log(f"  logits max rel err {err:.3e}; draft {c}")
    assert err <= LM_TOL


def test_b16_fp8_full_size_sampled():
    """The 16-sequence workload at full size: LM head (112 rows, workgroup
    kernel) on sampled vocabulary rows, and the fc (128 rows) on every output."""
    w = workloads.get("b16")
    t0 = time.time()
    W = synth.make_weights_fp8(w)
    log(f"b16 fp8 weights in {time.time() - t0:.1f}s")
    s = synth.make_step(w, 0, noise=False)
    Zg = bdr().dspark_lm_head_fp8(dev(s["draft_hidden"]), dev(W["lm_q"]), dev(W["lm_scale"]))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(w.vocab, 6000, replace=False),
                                     np.arange(w.vocab - 40, w.vocab), np.arange(40)]))
    ref = fp8.lm_head_fp8(s["draft_hidden"], W["lm_q"][rows], W["lm_scale"][rows], "bf16")
    err = max_rel_err(Zg.cpu().numpy()[..., rows], ref)
    F = bdr().dflash_fuse_fc_fp8([dev(t) for t in s["taps"]], dev(W["fc_q"]), dev(W["fc_scale"]))
    errf = max_rel_err(oracle.widen(host_bits(F), "bf16"),
                       fp8.fuse_fc_fp8(s["taps"], W["fc_q"], W["fc_scale"], "bf16"))
    log(f"  LM head {rows.size} vocab rows: max rel err {err:.3e}; fc max rel err {errf:.3e}")
    assert err <= LM_TOL
    assert errf <= FC_TOL



def test_fc_rows_fp8_on_gathered_rows():
    rng = np.random.default_rng(6)
    T, rows, H = 5, 40, 512
    taps = [_bf16(rng, (rows, H)) for _ in range(T)]
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((H, T * H)).astype(np.float32) / np.sqrt(T * H))
    idx = np.sort(rng.choice(rows, size=13, replace=False)).astype(np.int32)
    row_index = np.full(rows, -3, dtype=np.int32)
    row_index[:idx.size] = idx
    count = np.array([idx.size], dtype=np.int32)
    out = bdr().dflash_fuse_fc_rows_fp8([dev(t) for t in taps], dev(q), dev(s), dev(row_index),
                                        dev(count))
    got = oracle.widen(host_bits(out), "bf16")
    ref = fp8.fuse_fc_fp8([t[idx] for t in taps], q, s, "bf16")
    err = max_rel_err(got[:idx.size], ref)
    log(f"fc rows fp8: {idx.size}/{rows} rows, max rel err {err:.3e}")
    assert err <= FC_TOL
    assert np.all(got[idx.size:] == 0)


def test_closed_loop_fp8_on_device():
    """Three block-steps chained on the device with fp8 weights (LM head, draft,
    verify, commit, fc on the accepted rows), following the GPU's own path:
    each step's draft checked position by position against the oracle's rule
    from the GPU's context, then verified and committed by the oracle, every
    row compared."""
    import dataclasses
    from oracle import loop
    w = dataclasses.replace(workloads.get("b16"), cid=96, name="loop_fp8", batch=3, hidden=256,
                            n_taps=3, k=5, vocab=4099, rank=16)
    W = synth.make_weights_fp8(w)
    steps = 3
    inputs = [synth.make_step(w, s) for s in range(steps)]
    g = {n: dev(W[n]) for n in ("fc_q", "fc_scale", "lm_q", "lm_scale", "w1", "w2")}
    prev = dev(inputs[0]["prev0"])
    prev_g = inputs[0]["prev0"].astype(np.int64)
    L = np.full(w.batch, w.k)
    n_near = 0
    for s in range(steps):
        inp = inputs[s]
        Z = fp8.lm_head_fp8(inp["draft_hidden"], W["lm_q"], W["lm_scale"], "bf16")
        d_ref, _ = oracle.semi_ar_argmax(Z, W["w1"], W["w2"], prev_g, "bf16")
        Y = synth.plant_targets(w, s, inp["noise"], d_ref)["target_logits"]
        Zg = bdr().dspark_lm_head_fp8(dev(inp["draft_hidden"]), g["lm_q"], g["lm_scale"])
        d = bdr().dspark_markov_argmax(Zg, g["w1"], g["w2"], prev)
        v = bdr().spec_verify_greedy(dev(Y), d, target_argmax=False)
        c = bdr().spec_commit(d, v["accepted"], v["bonus"], v["block_len"])
        F = bdr().dflash_fuse_fc_rows_fp8([dev(t) for t in inp["taps"]], g["fc_q"], g["fc_scale"],
                                          c["row_index"], c["row_count"])
        torch.cuda.synchronize()
        r = {n: host_bits(x) for n, x in dict(d=d, F=F, **c, **v).items()}
        n_near += check_draft(r["d"], Z, W["w1"], W["w2"], prev_g, "bf16")["other_side"]
        t_ref = oracle.target_argmax(Y, "bf16", L)
        a_ref, bonus_ref, _, _ = oracle.verify_greedy(r["d"], t_ref, L)
        c_ref = loop.commit_step(r["d"], a_ref, bonus_ref, L)
        assert np.array_equal(r["accepted"], a_ref) and np.array_equal(r["bonus"], bonus_ref), s
        for n in ("emitted", "next_prev", "row_offsets"):
            assert np.array_equal(r[n], c_ref[n]), (s, n)
        nr = int(r["row_count"][0])
        assert nr == c_ref["row_count"]
        F_ref = fp8.fuse_fc_fp8([t[c_ref["row_index"]] for t in inp["taps"]], W["fc_q"],
                                W["fc_scale"], "bf16")
        err = max_rel_err(oracle.widen(r["F"], "bf16")[:nr], F_ref)
        assert err <= FC_TOL, (s, err)
        prev = c["next_prev"]
        prev_g = c_ref["next_prev"]
    log(f"fp8 closed loop: every row compared at every step; near-tie positions taken the "
        f"other admissible way: {n_near}")


@pytest.mark.parametrize("M,N,H", [(17, 1, 128), (33, 3, 256), (160, 17, 64), (48, 300, 192)])
def test_fp8_row_split_edge_shapes(M, N, H):
    rng = np.random.default_rng(M * 1000 + N + 7)
    hid = _bf16(rng, (M, H))
    q, s = synth.quantize_e4m3_rows(rng.standard_normal((N, H)).astype(np.float32) / np.sqrt(H))
    got = bdr().dspark_lm_head_fp8(dev(hid), dev(q), dev(s)).cpu().numpy()
    err = max_rel_err(got, fp8.lm_head_fp8(hid, q, s, "bf16"))
    log(f"fp8 row-split edge M={M} N={N} H={H}: max rel err {err:.3e}")
    assert err <= LM_TOL
