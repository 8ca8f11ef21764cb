"""The seeded generator: reproducibility, distributions and routing invariants (CPU only)."""
import numpy as np

import synth


def test_splitmix_reference_values():
    # SplitMix64 seeded with 0 yields these first outputs (Vigna's reference code):
    # mix64(0 + 1*GAMMA), mix64(0 + 2*GAMMA), ...
    expect = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [synth._mix64_int(i * synth.GAMMA) for i in (1, 2, 3)]
    assert got == expect
    k = synth.key(7, 3, 5)
    h = synth.hashes(7, 3, 5, 10, 4)
    assert [int(v) for v in h] == [synth._mix64_int(k + (i + 1) * synth.GAMMA) for i in range(10, 14)]


def test_reproducible_and_seed_sensitive():
    a = synth.affine_weights(1001, 64, 256)
    b = synth.affine_weights(1001, 64, 256)
    c = synth.affine_weights(1002, 64, 256)
    assert synth.sha256(a.codes, a.scale, a.bias) == synth.sha256(b.codes, b.scale, b.bias)
    assert synth.sha256(a.codes) != synth.sha256(c.codes)
    # any element can be regenerated alone
    cb = synth.code_bytes(1001, synth.S_CODES, 0, 64 * 128)
    assert np.array_equal(synth.code_bytes(1001, synth.S_CODES, 0, 13, start_byte=37), cb[37:50])


def test_distributions():
    w = synth.affine_weights(1000, 512, 256)
    q = np.concatenate([(w.codes >> np.uint32(4 * j)) & np.uint32(15) for j in range(8)]).ravel()
    counts = np.bincount(q.astype(np.int64), minlength=16)
    assert counts.min() > 0.9 * q.size / 16 and counts.max() < 1.1 * q.size / 16
    s = synth.bf16_to_f32(w.scale)
    b = synth.bf16_to_f32(w.bias)
    # bounds of the draw, widened by half a bf16 ulp for the final rounding
    assert s.min() >= 0.01 - 2 ** -16 and s.max() <= 0.05 + 2 ** -14
    assert b.min() >= -0.4 - 2 ** -10 and b.max() <= 0.0
    x = synth.bf16_to_f32(synth.activations(1000, synth.S_X, 1, 1 << 16)).astype(np.float64)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    m = synth.expert_gate_up(1003, 5, n=64, d=256)
    assert m.e8m0.min() >= 118 and m.e8m0.max() <= 126
    assert set(np.unique(m.e8m0).tolist()) == set(range(118, 127))


def test_draw_experts():
    e = synth.draw_experts(1003, 16, 896, 0)
    assert len(set(e.tolist())) == 16 and e.min() >= 0 and e.max() < 896
    assert not np.array_equal(e, synth.draw_experts(1003, 16, 896, 1))


def test_rows_regenerate_alone():
    # any rows of an expert matrix regenerate bit for bit without the rest
    full = synth.expert_gate_up(1003, 17, n=96, d=256)
    rows = [0, 5, 31, 32, 95]
    part = synth.expert_gate_up_rows(1003, 17, rows, n=96, d=256)
    assert np.array_equal(part.codes, full.codes[rows]) and np.array_equal(part.e8m0, full.e8m0[rows])
    whole = synth.expert_gate_up(1003, 4)
    part = synth.expert_gate_up_rows(1003, 4, [0, 255, 256, 6143])
    assert np.array_equal(part.codes, whole.codes[[0, 255, 256, 6143]])
    assert np.array_equal(part.e8m0, whole.e8m0[[0, 255, 256, 6143]])
