"""The seeded input generator: published SplitMix64 outputs, determinism, and
the code ranges of each generated field."""
import hashlib

import numpy as np

from bit_quantized_moe_dequant_amd import synth


def test_splitmix64_published_outputs():
    # SplitMix64 from state 0: the first two outputs are 0xe220a8397b1dcdaf and
    # 0x6e789e6aa1b965f4 (Vigna's reference splitmix64.c).
    g = np.array([0x9E3779B97F4A7C15, (2 * 0x9E3779B97F4A7C15) % 2 ** 64], dtype=np.uint64)
    assert [hex(int(v)) for v in synth.mix64(g)] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4"]


def test_stream_bytes_are_deterministic_and_offsettable():
    a = synth.raw_bytes(5, 3, 0, 1000)
    b = synth.raw_bytes(5, 3, 0, 1000)
    assert a.tobytes() == b.tobytes()
    assert synth.raw_bytes(5, 3, 13, 100).tobytes() == a[13:113].tobytes()
    assert synth.raw_bytes(5, 4, 0, 1000).tobytes() != a.tobytes()
    assert hashlib.sha256(a.tobytes()).hexdigest() == hashlib.sha256(b.tobytes()).hexdigest()


def test_field_ranges():
    e8 = synth.field_bytes(1, 1, synth.FIELD_E8M0_119_123, 0, 5000)
    assert set(np.unique(e8).tolist()) == {119, 120, 121, 122, 123}
    e4 = synth.field_bytes(1, 2, synth.FIELD_E4M3_08_28, 0, 20000)
    assert e4.min() == 0x08 and e4.max() == 0x28 and len(np.unique(e4)) == 33
    f8 = synth.field_bytes(1, 3, synth.FIELD_E4M3_FINITE, 0, 100000)
    assert 0x7F not in f8 and 0xFF not in f8 and len(np.unique(f8)) == 254


def test_block_fields_take_d_from_table():
    tab = synth.d_table().view(np.float16).astype(np.float64)
    assert tab.min() >= 0.00099 and tab.max() <= 0.01001
    q = synth.field_bytes(2, 1, synth.FIELD_Q2K_BLOCK, 84 * 10, 84 * 50).reshape(50, 84)
    d = q[:, 80:82].copy().view(np.float16).astype(np.float64)
    dmin = q[:, 82:84].copy().view(np.float16).astype(np.float64)
    assert np.all((d >= 0.00099) & (d <= 0.01001)) and np.all((dmin >= 0.00099) & (dmin <= 0.01001))
    i = synth.field_bytes(2, 2, synth.FIELD_IQ2_BLOCK, 0, 66 * 50).reshape(50, 66)
    d = i[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert np.all((d >= 0.00099) & (d <= 0.01001))


def test_expert_source_sizes():
    for fmt in synth.FMT_NAMES:
        rows, cols = (256, 512)
        planes = synth.expert_source(0, 0, 0, fmt, rows, cols, 3)
        sizes = [nb for nb, _ in synth.source_planes(fmt, rows, cols)]
        assert [p.size for p in planes] == sizes


def test_standin_grid_is_distinct():
    g = synth.iq2_standin_grid()
    assert g.shape == (256, 8) and len({tuple(r) for r in g.tolist()}) == 256
    assert set(np.unique(g).tolist()) <= {5, 19, 41}


def test_routing_generators():
    ids, w = synth.uniform_routing(0, 64, 256, 6)
    assert ids.shape == (64, 6) and all(len(set(r)) == 6 for r in ids.tolist())
    assert np.allclose(w.sum(1), 1, atol=1e-6)
    seq, _ = synth.cold_routing_sequence(0, 100, 256, 6)
    for s in range(100 - 42):
        win = seq[s:s + 42].reshape(-1)
        if s % 42 == 0:
            assert len(set(win.tolist())) == 252
    tok = synth.zipf_token_ids(0, 2048)
    hid, hw = synth.hash_routing(0, tok, 256, 6)
    assert all(len(set(r)) == 6 for r in hid.tolist())
    first = {}
    for t in range(2048):
        first.setdefault(int(tok[t]), hid[t].tolist())
        assert hid[t].tolist() == first[int(tok[t])]
