"""The seeded generator: reproducible draws and well-formed page tables."""
import numpy as np

from int2_rotated_kv_oscar_amd import synth


def test_draws_are_reproducible_and_bf16():
    w = synth.WORKLOADS["tiny"]
    a, b = synth.decode_inputs(w), synth.decode_inputs(w)
    assert np.array_equal(a.k_rows, b.k_rows) and np.array_equal(a.q, b.q)
    assert np.array_equal(a.bt_q, b.bt_q)
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3.14159])
    # round-half-even to 8 significant bits
    assert synth.bf16_bits_to_f32(synth.to_bf16_bits(x)).tolist() == [1.0, 1.0, 1 + 2 ** -6, -2.5, 3.140625]


def test_outliers_and_query_spectrum():
    w = synth.WORKLOADS["tiny"]
    kc, vc = synth.outlier_channels(w)
    assert kc.shape == (1, 3) and vc.shape == (1, 2) and len(set(kc[0])) == 3
    a = synth.query_mixers(w)
    sv = np.linalg.svd(a[0], compute_uv=False)
    np.testing.assert_allclose(sv, 1.0 / np.arange(1, 65), rtol=1e-10)


def test_tables_cover_every_region_once():
    w = synth.WORKLOADS["qwen3-8b-b28-ragged"]
    w = synth.Workload(**{**w.__dict__, "batch": 3, "name": "small-ragged"})
    inp = synth.decode_inputs(w, seq_lens=np.array([1300, 1500, 1200]))
    # shared prefix pages are aliased, the rest distinct
    assert np.array_equal(inp.bt_q[:, :64], np.repeat(inp.bt_q[:1, :64], 3, 0))
    own = np.concatenate([inp.bt_q[b, 64:(L + 15) // 16] for b, L in enumerate(inp.seq_lens)])
    own = own[own >= 0]
    assert len(set(own.tolist())) == len(own)
    assert not set(own.tolist()) & set(inp.bt_q[0, :64].tolist())
    ms, mp, mr = synth.middle_rows(inp)
    hs, hp, hr = synth.bf16_rows(inp)
    for b, L in enumerate(inp.seq_lens):
        sink, mid, rec = synth.regions(int(L), 4, 128)
        assert (inp.bt_q[b, np.arange(mid[0], mid[1]) // 16] >= 0).all()
        assert (inp.bt_h[b, np.r_[0:4, rec[0]:rec[1]] // 16] >= 0).all()
    assert len(ms) == 1020 + (1300 - 128 - 1024) + (1500 - 128 - 1024) + (1200 - 128 - 1024)
    assert len(hs) == 4 + 3 * 128
    assert inp.bt_q.max() < inp.n_int2_pages and inp.bt_h.max() < inp.n_bf16_pages
