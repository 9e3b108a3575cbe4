"""GPU parity of the C ABI (HIP kernels on gfx950) against the CPU oracle.

Quantize-append: codes bit-exact except within 1e-5 of a rounding boundary
(<= 0.01 % of codes), f16 scale/zero bit-equal except within 1e-6 (relative)
of an f16 rounding midpoint.  Decode: rel-L2 <= 5e-3 and max-abs <= 2e-2
against the oracle's float64 output on the same pages.
"""
import numpy as np
import pytest
import torch

from int2_rotated_kv_oscar_amd import lib, synth
from oracle import cache as ocache
from oracle import layout as olayout
from oracle import rotation as orot

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _tiny(**kw):
    w = synth.WORKLOADS["tiny"]
    return synth.Workload(**{**w.__dict__, **kw}) if kw else w


@pytest.fixture(scope="module")
def tiny_rot():
    return gh.oracle_rotation(_tiny())


def _page_slot(inp, rows):
    ms, mp, _ = rows
    return inp.bt_q[ms, mp // 16].astype(np.int64), (mp % 16).astype(np.int64)


def test_library_loaded_from_tree():
    import os
    assert os.path.dirname(lib.LIB_PATH).endswith("int2_rotated_kv_oscar_amd")
    lib.load()
    maps = open("/proc/self/maps").read()
    assert lib.LIB_PATH in maps


def test_quantize_append_tiny(tiny_rot):
    w = _tiny()
    inp = synth.decode_inputs(w)
    gc = gh.alloc_cache(inp, tiny_rot)
    rows = synth.middle_rows(inp)
    print(f"[quantize_append tiny] rows={len(rows[0])}", flush=True)
    gh.gpu_fill(inp, tiny_rot, gc, rows)
    torch.cuda.synchronize()
    _, _, res, orows = gh.oracle_pools(inp, tiny_rot)
    page, slot = _page_slot(inp, orows)
    rep = gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, slot)
    print(rep)
    gh.assert_codes_ok(rep, "tiny")


@pytest.mark.parametrize("d,hkv,n_seq,chunk", [(128, 2, 3, 48), (64, 3, 2, 8200)])
def test_quantize_append_page_aligned_prefill(d, hkv, n_seq, chunk):
    # whole pages back to back (the direct-store path), shuffled page ids,
    # a ragged last page, and (d=64) enough rows for the multi-tile waves
    w = synth.Workload("prefill-test", 5, n_seq, 4 * hkv, hkv, d, 4, 128, 64, ("fixed", chunk, chunk), k_noise="t3")
    k, v, row_seq, row_pos = synth.prefill_rows(w, n_seq, chunk)
    pages_per = (chunk + 15) // 16
    perm = synth.rng_for(99, 7).permutation(n_seq * pages_per).astype(np.int32)
    bt_q = perm.reshape(n_seq, pages_per)
    cal = synth.calibration_set(w, n_rows=256)
    from oracle import rotation as orot
    rt = orot.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    rot = gh.Rotation(rt["r_k"].astype(np.float32).astype(np.float64), rt["r_v"].astype(np.float32).astype(np.float64),
                      float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"])))
    int2 = torch.zeros(n_seq * pages_per * lib.int2_page_bytes(d, hkv), dtype=torch.uint8, device=gh.DEV)
    cache = lib.make_cache(d, hkv, 4, 128, int2, None)
    print(f"[prefill d={d} rows={len(row_seq)}]", flush=True)
    lib.quantize_append(cache, gh.bits_to_dev_bf16(k), gh.bits_to_dev_bf16(v), gh.i32(row_seq), gh.i32(row_pos),
                        gh.i32(bt_q), torch.from_numpy(rot.r_k.astype(np.float32)).to(gh.DEV),
                        torch.from_numpy(rot.r_v.astype(np.float32)).to(gh.DEV), rot.tau_k, rot.tau_v)
    torch.cuda.synchronize()
    pool = olayout.Int2Pool(n_seq * pages_per, hkv, d)
    res = ocache.quantize_append(pool, k, v, row_seq, row_pos, bt_q, rot.r_k, rot.r_v, rot.tau_k, rot.tau_v,
                                 olayout.bf16_to_f64)
    page = bt_q[row_seq, row_pos // 16].astype(np.int64)
    rep = gh.compare_appended(int2.cpu().numpy(), w, n_seq * pages_per, res, page, (row_pos % 16).astype(np.int64))
    print(rep)
    gh.assert_codes_ok(rep, "prefill")


def test_quantize_append_large_inputs(tiny_rot):
    # rows holding values of magnitude 2^15 and above take the kernel's
    # per-row power-of-two prescale (f16 staging); rows beside them do not
    w = _tiny()
    inp = synth.decode_inputs(w)
    ms, mp, mr = synth.middle_rows(inp)
    k = inp.k_rows[mr].copy()
    v = inp.v_rows[mr].copy()
    big = np.array([40000.0, -1.0e6, 3.0e5, 65504.0])
    rng = np.random.default_rng(11)
    rows = rng.choice(len(ms), size=24, replace=False)
    for j, r in enumerate(rows):
        c = rng.integers(0, w.d, size=2)
        k[r, 0, c] = synth.to_bf16_bits(np.full(2, big[j % 4]))
        v[r, 0, c[::-1]] = synth.to_bf16_bits(np.full(2, -big[(j + 1) % 4]))
    gc = gh.alloc_cache(inp, tiny_rot)
    print("[quantize_append large inputs]", flush=True)
    lib.quantize_append(gc.cache, gh.bits_to_dev_bf16(k), gh.bits_to_dev_bf16(v), gh.i32(ms), gh.i32(mp), gc.bt_q,
                        gc.r_k, gc.r_v, tiny_rot.tau_k, tiny_rot.tau_v)
    torch.cuda.synchronize()
    pool = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d)
    res = ocache.quantize_append(pool, k, v, ms, mp, inp.bt_q, tiny_rot.r_k, tiny_rot.r_v, tiny_rot.tau_k,
                                 tiny_rot.tau_v, olayout.bf16_to_f64)
    page, slot = _page_slot(inp, (ms, mp, mr))
    rep = gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, slot)
    print(rep)
    gh.assert_codes_ok(rep, "large inputs")


def test_quantize_append_small_magnitude_rows(tiny_rot):
    # more than 64 rows (the matrix-core kernel) where some rows are scaled
    # down by powers of two (exact in bf16): their values fall below the f16
    # normal range, so the kernel must rescale them before its f16 staging;
    # the scale and zero of the smallest rows are f16 subnormals or zero
    w = _tiny()
    inp = synth.decode_inputs(w)
    ms, mp, mr = synth.middle_rows(inp)
    k = synth.bf16_bits_to_f32(inp.k_rows[mr]).astype(np.float64)
    v = synth.bf16_bits_to_f32(inp.v_rows[mr]).astype(np.float64)
    rng = np.random.default_rng(21)
    rows = rng.permutation(len(ms))
    exps = [-3, -5, -10, -14, -17, -20, -24, -30]
    for j, r in enumerate(rows[:8 * 20]):
        k[r] *= 2.0 ** exps[j % 8]
        v[r] *= 2.0 ** exps[(j + 3) % 8]
    kb, vb = synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    assert np.array_equal(synth.bf16_bits_to_f32(kb).astype(np.float64), k)  # the scaling was exact
    gc = gh.alloc_cache(inp, tiny_rot)
    print(f"[quantize_append small-magnitude rows] rows={len(ms)}", flush=True)
    lib.quantize_append(gc.cache, gh.bits_to_dev_bf16(kb), gh.bits_to_dev_bf16(vb), gh.i32(ms), gh.i32(mp), gc.bt_q,
                        gc.r_k, gc.r_v, tiny_rot.tau_k, tiny_rot.tau_v)
    torch.cuda.synchronize()
    pool = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d)
    res = ocache.quantize_append(pool, kb, vb, ms, mp, inp.bt_q, tiny_rot.r_k, tiny_rot.r_v, tiny_rot.tau_k,
                                 tiny_rot.tau_v, olayout.bf16_to_f64)
    page, slot = _page_slot(inp, (ms, mp, mr))
    rep = gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, slot)
    print(rep)
    gh.assert_codes_ok(rep, "small-magnitude rows")
    # the same rows through the few-row kernel (float32 products)
    sel = rows[:64]
    gc2 = gh.alloc_cache(inp, tiny_rot)
    lib.quantize_append(gc2.cache, gh.bits_to_dev_bf16(kb[sel]), gh.bits_to_dev_bf16(vb[sel]), gh.i32(ms[sel]),
                        gh.i32(mp[sel]), gc2.bt_q, gc2.r_k, gc2.r_v, tiny_rot.tau_k, tiny_rot.tau_v)
    torch.cuda.synchronize()
    res2 = ocache.quantize_append(olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d), kb[sel], vb[sel], ms[sel],
                                  mp[sel], inp.bt_q, tiny_rot.r_k, tiny_rot.r_v, tiny_rot.tau_k, tiny_rot.tau_v,
                                  olayout.bf16_to_f64)
    page2, slot2 = _page_slot(inp, (ms[sel], mp[sel], mr[sel]))
    rep2 = gh.compare_appended(gc2.int2.cpu().numpy(), w, inp.n_int2_pages, res2, page2, slot2)
    print(rep2)
    gh.assert_codes_ok(rep2, "small-magnitude rows, few-row kernel")


def test_quantize_append_scattered_single_rows(tiny_rot):
    # rows in random order: neighbouring slots of one page written by
    # different waves at once (the partial-word path)
    w = _tiny()
    inp = synth.decode_inputs(w)
    ms, mp, mr = synth.middle_rows(inp)
    perm = np.random.default_rng(5).permutation(len(ms))
    rows = (ms[perm], mp[perm], mr[perm])
    gc = gh.alloc_cache(inp, tiny_rot)
    gc.int2.random_(0, 256)  # stale bytes in the pool must be replaced, not OR-ed
    gh.gpu_fill(inp, tiny_rot, gc, rows)
    torch.cuda.synchronize()
    _, _, res, _ = gh.oracle_pools(inp, tiny_rot)
    # oracle record is in middle_rows order; compare in that order
    page = inp.bt_q[ms, mp // 16].astype(np.int64)
    rep = gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, (mp % 16).astype(np.int64))
    gh.assert_codes_ok(rep, "scattered")


@pytest.mark.parametrize("d,hkv,n_rows", [(64, 1, 1), (64, 3, 7), (128, 8, 28), (128, 2, 64), (128, 2, 65)])
def test_quantize_append_few_rows(d, hkv, n_rows):
    # a decode step's appends: a few rows in random order at scattered slots
    # of pages holding stale bytes (up to 64 rows take the few-row kernel,
    # 65 the matrix-core one); every other byte of the pool stays as it was
    n_seq, chunk = 4, 64
    w = synth.Workload("few-rows", 5, n_seq, 4 * hkv, hkv, d, 4, 128, 64, ("fixed", chunk, chunk), k_noise="t3")
    k, v, row_seq, row_pos = synth.prefill_rows(w, n_seq, chunk)
    rng = np.random.default_rng(1000 + n_rows)
    sel = rng.choice(len(row_seq), size=n_rows, replace=False)
    k, v, row_seq, row_pos = k[sel], v[sel], row_seq[sel], row_pos[sel]
    pages_per = chunk // 16
    n_pages = n_seq * pages_per
    bt_q = synth.rng_for(98, 7).permutation(n_pages).astype(np.int32).reshape(n_seq, pages_per)
    cal = synth.calibration_set(w, n_rows=256)
    from oracle import rotation as orot
    rt = orot.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    rot = gh.Rotation(rt["r_k"].astype(np.float32).astype(np.float64), rt["r_v"].astype(np.float32).astype(np.float64),
                      float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"])))
    stale = rng.integers(0, 256, size=n_pages * lib.int2_page_bytes(d, hkv), dtype=np.uint8)
    int2 = torch.from_numpy(stale.copy()).to(gh.DEV)
    cache = lib.make_cache(d, hkv, 4, 128, int2, None)
    print(f"[few rows d={d} hkv={hkv} rows={n_rows}]", flush=True)
    lib.quantize_append(cache, gh.bits_to_dev_bf16(k), gh.bits_to_dev_bf16(v), gh.i32(row_seq), gh.i32(row_pos),
                        gh.i32(bt_q), torch.from_numpy(rot.r_k.astype(np.float32)).to(gh.DEV),
                        torch.from_numpy(rot.r_v.astype(np.float32)).to(gh.DEV), rot.tau_k, rot.tau_v)
    torch.cuda.synchronize()
    got = int2.cpu().numpy()
    pool = olayout.Int2Pool(n_pages, hkv, d, stale.copy())
    res = ocache.quantize_append(pool, k, v, row_seq, row_pos, bt_q, rot.r_k, rot.r_v, rot.tau_k, rot.tau_v,
                                 olayout.bf16_to_f64)
    page = bt_q[row_seq, row_pos // 16].astype(np.int64)
    slot = (row_pos % 16).astype(np.int64)
    rep = gh.compare_appended(got, w, n_pages, res, page, slot)
    print(rep)
    gh.assert_codes_ok(rep, "few rows")
    # with the appended rows' fields cleared in both, the pools are identical
    cleared = []
    for data in (got.copy(), pool.data.copy()):
        pc = olayout.Int2Pool(n_pages, hkv, d, data)
        zc = np.zeros((n_rows, d), np.uint8)
        zs = np.zeros((n_rows, d // 32), np.float16)
        for h in range(hkv):
            pc.write(page, slot, h, zc, zc, zs, zs, zs, zs)
        cleared.append(pc.data)
    assert np.array_equal(cleared[0], cleared[1]), "bytes outside the appended rows changed"


@pytest.mark.parametrize("d,hkv,S,W", [(64, 1, 4, 32), (128, 2, 4, 128), (64, 2, 4, 0), (128, 1, 0, 16)])
def test_decode_step_update(d, hkv, S, W):
    # one decode step's cache update (new tokens to BF16, the tokens leaving
    # the recent windows to INT2, read from their BF16 slots) against the
    # oracle's, over lengths around the region edges, on stale pools
    lens = np.array([0, 1, 3, 4, 5, S + W, S + W + 1, S + W + 2, 77, 160, 161, 300, 47, 250, 299], np.int32)
    B, maxl = len(lens), int(lens.max())
    mp = (maxl + 15) // 16
    w = synth.Workload("step", 6, B, 4 * hkv, hkv, d, S, W, 64, ("fixed", maxl, maxl))
    k, v, _, _ = synth.prefill_rows(w, B, maxl)   # row b * maxl + position
    rng = np.random.default_rng(77 + d + W)
    bt_q = rng.permutation(B * mp).astype(np.int32).reshape(B, mp)
    bt_h = rng.permutation(B * mp).astype(np.int32).reshape(B, mp)
    cal = synth.calibration_set(w, n_rows=256)
    from oracle import rotation as orot
    rt = orot.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    f = lambda a: np.asarray(a, np.float32).astype(np.float64)  # noqa: E731
    rot = gh.Rotation(f(rt["r_k"]), f(rt["r_v"]), float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"])))
    # state the previous steps left: every earlier token's raw row in its BF16 slot
    int2_0 = rng.integers(0, 256, size=B * mp * lib.int2_page_bytes(d, hkv), dtype=np.uint8)
    bf_0 = olayout.Bf16Pool(B * mp, hkv, d, rng.integers(0, 65536, size=(B * mp, hkv, 32 * d), dtype=np.uint16))
    seq = np.repeat(np.arange(B), np.maximum(lens - 1, 0))
    pos = np.concatenate([np.arange(max(L - 1, 0)) for L in lens]).astype(np.int64)
    ocache.write_bf16(bf_0, k[seq * maxl + pos], v[seq * maxl + pos], seq, pos, bt_h)
    newrow = np.arange(B) * maxl + np.maximum(lens - 1, 0)
    k_new, v_new = k[newrow], v[newrow]
    # GPU
    int2 = torch.from_numpy(int2_0.copy()).to(gh.DEV)
    bf16 = torch.from_numpy(bf_0.data.copy().reshape(-1).view(np.int16)).to(gh.DEV)
    cache = lib.make_cache(d, hkv, S, W, int2, bf16)
    print(f"[step update d={d} hkv={hkv} S={S} W={W}]", flush=True)
    lib.decode_step_update(cache, gh.bits_to_dev_bf16(k_new), gh.bits_to_dev_bf16(v_new), gh.i32(lens), gh.i32(bt_q),
                           gh.i32(bt_h), torch.from_numpy(rot.r_k.astype(np.float32)).to(gh.DEV),
                           torch.from_numpy(rot.r_v.astype(np.float32)).to(gh.DEV), rot.tau_k, rot.tau_v)
    torch.cuda.synchronize()
    got_q = int2.cpu().numpy()
    got_h = bf16.cpu().numpy().view(np.uint16).reshape(B * mp, hkv, 32 * d)
    # oracle
    i2 = olayout.Int2Pool(B * mp, hkv, d, int2_0.copy())
    bf = olayout.Bf16Pool(B * mp, hkv, d, bf_0.data.copy())
    res, (sq, ps) = ocache.decode_step_update(i2, bf, k_new, v_new, lens, bt_q, bt_h, S, W, rot.r_k, rot.r_v,
                                              rot.tau_k, rot.tau_v, olayout.bf16_to_f64)
    assert np.array_equal(got_h, bf.data), "BF16 pool differs"
    page, slot = bt_q[sq, ps // 16].astype(np.int64), (ps % 16).astype(np.int64)
    assert len(sq) >= 7
    rep = gh.compare_appended(got_q, w, B * mp, res, page, slot)
    print(rep)
    gh.assert_codes_ok(rep, "step update")
    cleared = []
    for data in (got_q.copy(), i2.data.copy()):
        pc = olayout.Int2Pool(B * mp, hkv, d, data)
        zc = np.zeros((len(sq), d), np.uint8)
        zs = np.zeros((len(sq), d // 32), np.float16)
        for h in range(hkv):
            pc.write(page, slot, h, zc, zc, zs, zs, zs, zs)
        cleared.append(pc.data)
    assert np.array_equal(cleared[0], cleared[1]), "INT2 bytes outside the quantized rows changed"


@pytest.mark.parametrize("d,hq,hkv,n", [(128, 32, 8, 1000), (64, 4, 1, 2048), (128, 12, 1, 77)])
def test_calib_gram_matches_oracle_targets(d, hq, hkv, n):
    # GPU calibration targets (Q^T Q and O^T O over N G pooled rows) against
    # the oracle's on the same bf16 rows, within the float32 accumulation bound
    # of 256-row blocks (|err| <= 256 2^-24 sum|x_a||x_b| / (N G)); then the
    # rotation built from them, whose eigenvalues move by at most ||dC|| (Weyl)
    w = synth.Workload("calib", 6, 1, hq, hkv, d, 4, 32, n, ("fixed", 64, 64))
    cal = synth.calibration_set(w, n_rows=n)
    o = synth.bf16_bits_to_f32(synth.to_bf16_bits(np.random.default_rng(n).standard_normal(cal.q.shape) * 0.7))
    G = hq // hkv
    cq, cs = orot.calibration_targets(cal.q.astype(np.float64), cal.k.astype(np.float64), cal.v.astype(np.float64), G,
                                      oc=o.astype(np.float64))
    print(f"[calib gram d={d} hq={hq} hkv={hkv} n={n}]", flush=True)
    gq = lib.calib_gram(gh.bits_to_dev_bf16(synth.to_bf16_bits(cal.q)), hkv)
    go = lib.calib_gram(gh.bits_to_dev_bf16(synth.to_bf16_bits(o)), hkv)
    torch.cuda.synchronize()
    gq, go = gq.cpu().numpy(), go.cpu().numpy()
    for got, ref, x in ((gq, cq, cal.q), (go, cs, o)):
        ax = np.abs(x.astype(np.float64))
        for h in range(hkv):
            xa = ax[:, h * G:(h + 1) * G, :].reshape(-1, d)
            bound = 2.0 ** -16 * (xa.T @ xa) / xa.shape[0] + 1e-300
            err = np.abs(got[h] - ref[h])
            assert (err <= bound).all(), f"max err/bound {(err / bound).max():.3g}"
    rg = lib.build_rotation_from_targets(gq, go, cal.k, cal.v)
    ro = lib.build_rotation_from_targets(cq, cs, cal.k, cal.v)
    for key, dc in (("eig_k", gq - cq), ("eig_v", go - cs)):
        for h in range(hkv):
            assert np.abs(rg[key][h] - ro[key][h]).max() <= np.linalg.norm(dc[h]) + 1e-12


def test_decode_on_oracle_pages_tiny(tiny_rot):
    w = _tiny()
    inp = synth.decode_inputs(w)
    int2, bf, _, _ = gh.oracle_pools(inp, tiny_rot)
    gc = gh.alloc_cache(inp, tiny_rot, int2.data, bf.data)
    ref = gh.oracle_decode(inp, tiny_rot, int2, bf)
    for sp in (0, 8, 16):
        print(f"[decode tiny oracle pages] split_pages={sp}", flush=True)
        got = gh.gpu_decode(inp, gc, split_pages=sp)
        print(sp, gh.attention_errors(got, ref))
        gh.assert_attention_close(got, ref, f"split {sp}")


def test_end_to_end_tiny(tiny_rot):
    w = _tiny()
    inp = synth.decode_inputs(w)
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, gc)
    got = gh.gpu_decode(inp, gc)
    int2, bf, _, _ = gh.oracle_pools(inp, tiny_rot)
    ref = gh.oracle_decode(inp, tiny_rot, int2, bf)
    print(gh.attention_errors(got, ref))
    gh.assert_attention_close(got, ref, "end-to-end tiny")


@pytest.mark.parametrize("lens", [[1], [2], [17], [36], [37], [100], [512, 1, 300, 0, 37, 129]])
def test_decode_lengths_and_ragged_batch(tiny_rot, lens):
    w = _tiny(batch=len(lens))
    inp = synth.decode_inputs(w, seq_lens=np.array(lens))
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, gc)
    print(f"[decode lens={lens}]", flush=True)
    got = gh.gpu_decode(inp, gc)
    int2, bf, _, _ = gh.oracle_pools(inp, tiny_rot)
    ref = gh.oracle_decode(inp, tiny_rot, int2, bf)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(got[b] == 0)
        else:
            gh.assert_attention_close(got[b], ref[b], f"len {L}")


@pytest.mark.parametrize("hq,hkv,d,q_scale", [(4, 4, 64, 1.0), (16, 1, 128, 1.0), (12, 1, 128, 8.0),
                                              (8, 2, 128, 8.0), (3, 1, 64, 1.0), (8, 1, 64, 1.0),
                                              (6, 1, 128, 8.0), (5, 1, 64, 8.0), (16, 2, 128, 1.0)])
def test_decode_group_shapes(hq, hkv, d, q_scale):
    w = synth.Workload("shape", 6, 2, hq, hkv, d, 4, 32, 512, ("fixed", 700, 700), q_scale=q_scale)
    rot = gh.oracle_rotation(w, n_rows=512, q_scale=q_scale)
    inp = synth.decode_inputs(w, seq_lens=np.array([700, 333]), q_scale=q_scale)
    gc = gh.alloc_cache(inp, rot)
    gh.gpu_fill(inp, rot, gc)
    print(f"[decode shape hq={hq} hkv={hkv} d={d}]", flush=True)
    got = gh.gpu_decode(inp, gc, split_pages=8)
    int2, bf, res, rows = gh.oracle_pools(inp, rot)
    page, slot = _page_slot(inp, rows)
    gh.assert_codes_ok(gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, slot))
    ref = gh.oracle_decode(inp, rot, int2, bf)
    print(gh.attention_errors(got, ref))
    gh.assert_attention_close(got, ref, "shape")


@pytest.mark.parametrize("variant", [lib.ROTATION_HADAMARD, lib.ROTATION_IDENTITY])
@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (8, 2, 128)])
def test_comparison_rotations_end_to_end(variant, hq, hkv, d):
    # the pages' baselines (Hadamard-only, naive INT2) through the same
    # kernels: rotation from the host library (equal to the oracle's, pinned
    # on the CPU), cache written and decoded on the GPU, against the oracle
    w = synth.Workload("ablation", 6, 2, hq, hkv, d, 4, 32, 512, ("fixed", 600, 600))
    cal = synth.calibration_set(w, n_rows=512)
    rt = lib.build_fixed_rotation(variant, cal.k, cal.v)
    f = lambda a: np.asarray(a, np.float32).astype(np.float64)  # noqa: E731
    rot = gh.Rotation(f(rt["r_k"]), f(rt["r_v"]), float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"])))
    inp = synth.decode_inputs(w, seq_lens=np.array([600, 291]))
    gc = gh.alloc_cache(inp, rot)
    gh.gpu_fill(inp, rot, gc)
    print(f"[comparison rotation {variant} hq={hq} hkv={hkv} d={d}]", flush=True)
    got = gh.gpu_decode(inp, gc)
    int2, bf, res, rows = gh.oracle_pools(inp, rot)
    page, slot = _page_slot(inp, rows)
    gh.assert_codes_ok(gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, slot))
    ref = gh.oracle_decode(inp, rot, int2, bf)
    print(gh.attention_errors(got, ref))
    gh.assert_attention_close(got, ref, "comparison rotation")


@pytest.mark.parametrize("S,W", [(0, 0), (0, 16), (4, 0), (16, 48), (32, 0)])
def test_decode_region_layouts(S, W):
    # degenerate region layouts: no sink, no recent window, neither, a wide
    # sink; ragged lengths around page edges; automatic and fixed splits
    lens = np.array([1, 15, 16, 17, 33, 64, 65, 700, 333])
    w = synth.Workload("regions", 6, len(lens), 8, 2, 128, S, W, 512, ("fixed", 700, 700))
    rot = gh.oracle_rotation(w, n_rows=512)
    inp = synth.decode_inputs(w, seq_lens=lens)
    gc = gh.alloc_cache(inp, rot)
    gh.gpu_fill(inp, rot, gc)
    int2, bf, res, rows = gh.oracle_pools(inp, rot)
    page, slot = _page_slot(inp, rows)
    gh.assert_codes_ok(gh.compare_appended(gc.int2.cpu().numpy(), w, inp.n_int2_pages, res, page, slot))
    ref = gh.oracle_decode(inp, rot, int2, bf)
    for split in (0, 8):
        print(f"[decode regions S={S} W={W} split={split}]", flush=True)
        got = gh.gpu_decode(inp, gc, split_pages=split)
        print(gh.attention_errors(got, ref))
        gh.assert_attention_close(got, ref, f"regions S={S} W={W} split={split}")


@pytest.mark.parametrize("all_raw", [False, True])
def test_decode_on_recycled_pools(tiny_rot, all_raw):
    # pools holding random bytes and NaN/infinity patterns everywhere the fill
    # does not write: sink slots of the first INT2 page, the middle tokens of
    # BF16 pages, BF16 page tails, whole pages past each length; per-unit
    # items (fixed splits) and balanced slices (many units)
    lens = np.array([512, 1, 17, 36, 37, 100, 333, 479, 480, 481, 0, 250])
    kw = dict(batch=len(lens))
    if all_raw:
        kw.update(n_sink=100000, n_recent=0)
    w = _tiny(**kw)
    inp = synth.decode_inputs(w, seq_lens=lens, spare_pages=7)
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.fill_stale(gc, seed=int(all_raw))
    gh.gpu_fill(inp, tiny_rot, gc)
    if not all_raw:
        gh.check_fill(inp, tiny_rot, gc, "recycled pools fill")
    ref = gh.oracle_decode_gpu_pages(inp, tiny_rot, gc)
    for split in (0, 8, 16):
        print(f"[decode recycled pools all_raw={all_raw} split={split}]", flush=True)
        got = gh.gpu_decode(inp, gc, split_pages=split, all_raw=all_raw)
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(got[b] == 0)
            else:
                gh.assert_attention_close(got[b], ref[b], f"recycled pools split {split} len {L}")
    # stale bytes outside the regions must not change a single output bit
    clean = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, clean)
    for split in (0, 8):
        assert np.array_equal(gh.gpu_decode(inp, clean, split_pages=split, all_raw=all_raw),
                              gh.gpu_decode(inp, gc, split_pages=split, all_raw=all_raw)), "stale bytes changed the output"
    # many units: the balanced-slice kernel over the same stale pools
    lens2 = np.random.default_rng(31).integers(1, 600, size=70)
    w2 = _tiny(**{**kw, "batch": len(lens2)})
    inp2 = synth.decode_inputs(w2, seq_lens=lens2)
    gc2 = gh.alloc_cache(inp2, tiny_rot)
    gh.fill_stale(gc2, seed=2 + int(all_raw))
    gh.gpu_fill(inp2, tiny_rot, gc2)
    ref2 = gh.oracle_decode_gpu_pages(inp2, tiny_rot, gc2)
    print(f"[decode recycled pools, balanced slices all_raw={all_raw}]", flush=True)
    got2 = gh.gpu_decode(inp2, gc2, all_raw=all_raw)
    for b in range(len(lens2)):
        gh.assert_attention_close(got2[b], ref2[b], f"recycled pools balanced slices seq {b}")
    clean2 = gh.alloc_cache(inp2, tiny_rot)
    gh.gpu_fill(inp2, tiny_rot, clean2)
    assert np.array_equal(gh.gpu_decode(inp2, clean2, all_raw=all_raw), got2), "stale bytes changed the output"


@pytest.mark.parametrize("hq,hkv,d,L,split", [(4, 1, 64, 9000, 8), (8, 1, 128, 32100, 8), (4, 2, 128, 20000, 8)])
def test_decode_many_chunks_multipass_merge(hq, hkv, d, L, split):
    # more than 32 records per (sequence, KV head): 70 to 252 INT2 chunks, so
    # the merge runs several weight passes and value rounds (four column
    # slots per query for G = 4, two for G = 8), against the oracle
    w = synth.Workload("chunks", 6, 1, hq, hkv, d, 4, 128, 512, ("fixed", L, L))
    rot = gh.oracle_rotation(w, n_rows=512)
    inp = synth.decode_inputs(w)
    gc = gh.alloc_cache(inp, rot)
    gh.fill_stale(gc, seed=5)
    gh.gpu_fill(inp, rot, gc)
    gh.check_fill(inp, rot, gc, "many chunks fill")
    ref = gh.oracle_decode_gpu_pages(inp, rot, gc)
    n_items = 1 + (L + 15) // 16 // split
    print(f"[decode many chunks hq={hq} d={d} L={L} split={split}: about {n_items} records]", flush=True)
    got = gh.gpu_decode(inp, gc, split_pages=split)
    print(gh.attention_errors(got, ref))
    gh.assert_attention_close(got, ref, f"{n_items} chunks")
    auto = gh.gpu_decode(inp, gc)
    gh.assert_attention_close(auto, ref, "automatic split")


def test_invariances_tables_splits_determinism(tiny_rot):
    w = _tiny(batch=2)
    lens = np.array([512, 400])
    a = synth.decode_inputs(w, seq_lens=lens, shuffle=True)
    b = synth.decode_inputs(w, seq_lens=lens, shuffle=False)
    ga = gh.alloc_cache(a, tiny_rot); gh.gpu_fill(a, tiny_rot, ga)
    gb = gh.alloc_cache(b, tiny_rot); gh.gpu_fill(b, tiny_rot, gb)
    oa = gh.gpu_decode(a, ga, split_pages=8)
    ob = gh.gpu_decode(b, gb, split_pages=8)
    assert np.array_equal(oa, ob), "shuffled and identity block tables differ"
    assert np.array_equal(oa, gh.gpu_decode(a, ga, split_pages=8)), "not deterministic"
    o64 = gh.gpu_decode(a, ga, split_pages=64)
    # outputs are bf16: different chunkings may round to neighbouring values;
    # both must meet the oracle bound and stay close to each other
    rel, mx = gh.attention_errors(o64, oa)
    assert rel <= 2e-3 and mx <= 1e-2, (rel, mx)
    int2, bf, _, _ = gh.oracle_pools(a, tiny_rot)
    ref = gh.oracle_decode(a, tiny_rot, int2, bf)
    gh.assert_attention_close(o64, ref, "64-page chunks")
    gh.assert_attention_close(oa, ref, "8-page chunks")


def test_shared_prefix_pages_alias(tiny_rot):
    # three sequences name the same physical pages for their first 64 tokens;
    # the output equals a run of the same batch where each sequence owns a
    # copy of them (same lengths, so the same work split: bit-identical); each
    # sequence decoded alone (another work split) meets the oracle bar too
    w = _tiny(batch=3, shared_prefix=64)
    lens = np.array([300, 512, 222])
    inp = synth.decode_inputs(w, seq_lens=lens)
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, gc)
    got = gh.gpu_decode(inp, gc)
    int2, bf, _, _ = gh.oracle_pools(inp, tiny_rot)
    ref = gh.oracle_decode(inp, tiny_rot, int2, bf)
    gh.assert_attention_close(got, ref, "shared prefix")
    wp = _tiny(batch=3, shared_prefix=0)
    private = synth.DecodeInputs(wp, lens, inp.k_rows, inp.v_rows, inp.row_of, inp.q,
                                 *_private_tables(inp, range(3)))
    gp = gh.alloc_cache(private, tiny_rot)
    gh.gpu_fill(private, tiny_rot, gp)
    assert np.array_equal(gh.gpu_decode(private, gp), got), "aliased and private prefix pages differ"
    for b in range(3):
        wb = _tiny(batch=1, shared_prefix=0)
        single = synth.DecodeInputs(wb, lens[b:b + 1], inp.k_rows, inp.v_rows, [inp.row_of[b]], inp.q[b:b + 1],
                                    *_private_tables(inp, [b]))
        gs = gh.alloc_cache(single, tiny_rot)
        gh.gpu_fill(single, tiny_rot, gs)
        gh.assert_attention_close(gh.gpu_decode(single, gs), ref[b:b + 1], f"sequence {b} alone")


def _private_tables(inp, seqs):
    # identity-style tables: sequence i of seqs owns pages [i n, i n + n)
    seqs = list(seqs)
    n = int(max((int(inp.seq_lens[b]) + 15) // 16 for b in seqs))
    bt_q = np.full((len(seqs), n), -1, np.int32)
    bt_h = np.full((len(seqs), n), -1, np.int32)
    for i, b in enumerate(seqs):
        m = (int(inp.seq_lens[b]) + 15) // 16
        own = i * n + np.arange(m, dtype=np.int32)
        bt_q[i, :m] = np.where(inp.bt_q[b, :m] >= 0, own, -1)
        bt_h[i, :m] = np.where(inp.bt_h[b, :m] >= 0, own, -1)
    return bt_q, bt_h, len(seqs) * n, len(seqs) * n, n


def test_bf16_baseline_matches_plain_attention(tiny_rot):
    from oracle import attention as oatt
    w = _tiny(batch=2, n_sink=100000, n_recent=0)   # every token in BF16 pages
    lens = np.array([512, 77])
    inp = synth.decode_inputs(w, seq_lens=lens)
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, gc)
    got = gh.gpu_decode(inp, gc, all_raw=True)
    q = synth.bf16_bits_to_f32(inp.q).astype(np.float64)
    for b, L in enumerate(lens):
        k = olayout.bf16_to_f64(inp.k_rows[inp.row_of[b], 0]); v = olayout.bf16_to_f64(inp.v_rows[inp.row_of[b], 0])
        ref = oatt.softmax_attention(q[b], k, v, 1 / 8.0)
        gh.assert_attention_close(got[b], ref, "bf16 baseline")


def test_decode_balanced_slices_many_units(tiny_rot):
    # more (sequence, KV head) units than a quarter of the CUs: the kernel
    # that spreads all units' pages over one workgroup per CU, so workgroups
    # cross unit and page-kind boundaries (several segments each) and skip
    # the overhead positions; ragged lengths including empty and one-page
    # sequences, every sequence checked.  The cache is the one the GPU wrote
    # (its codes checked against the oracle's, whose f16 ties at a rounding
    # midpoint may legitimately round the other way and move that group's
    # codes), and the oracle decodes those very pages.
    from oracle import attention as oatt
    lens = np.random.default_rng(11).integers(1, 700, size=80)
    lens[[3, 40]] = 0
    lens[[5, 6, 7]] = [1, 16, 37]
    w = _tiny(batch=len(lens))
    inp = synth.decode_inputs(w, seq_lens=lens)
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, gc)
    print(f"[decode balanced slices] B={len(lens)}", flush=True)
    got = gh.gpu_decode(inp, gc)
    _, _, res, rows = gh.oracle_pools(inp, tiny_rot)
    page, slot = _page_slot(inp, rows)
    int2_bytes = gc.int2.cpu().numpy()
    gh.assert_codes_ok(gh.compare_appended(int2_bytes, w, inp.n_int2_pages, res, page, slot), "balanced slices fill")
    int2 = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d, int2_bytes)
    bf = olayout.Bf16Pool(inp.n_bf16_pages, w.n_kv_heads, w.d, gc.bf16.cpu().numpy().view(np.uint16))
    q = synth.bf16_bits_to_f32(inp.q).astype(np.float64)
    ref = oatt.decode_attention(q, int2, bf, inp.seq_lens, inp.bt_q, inp.bt_h, tiny_rot.r_k, tiny_rot.r_v,
                                w.n_sink, w.n_recent)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(got[b] == 0)
        else:
            gh.assert_attention_close(got[b], ref[b], f"seq {b} len {L}")


@pytest.mark.parametrize("d,hq,hkv,mode", [(128, 16, 1, "uniform"), (128, 12, 2, "skewed"), (64, 8, 2, "skewed")])
def test_decode_balanced_slices_groups_and_skew(d, hq, hkv, mode):
    # balanced slices with the largest query group (16: the biggest per-range
    # overhead), a group of 6 (two column slots), and a skewed batch (one
    # sequence far longer than the rest, so the slice width is set by how many
    # records a unit may leave rather than by the even share), every sequence
    # against the oracle over the pages the GPU wrote
    from oracle import attention as oatt
    rng = np.random.default_rng(13 + d + hq)
    if mode == "uniform":
        lens = rng.integers(1, 700, size=70)
    else:
        lens = rng.integers(1, 200, size=40)
        lens[7] = 20000
    w = synth.Workload("slices", 21, len(lens), hq, hkv, d, 4, 32, 512, ("fixed", 1, 1))
    rot = gh.oracle_rotation(w, n_rows=512)
    inp = synth.decode_inputs(w, seq_lens=lens)
    gc = gh.alloc_cache(inp, rot)
    gh.fill_stale(gc, seed=3)
    gh.gpu_fill(inp, rot, gc)
    print(f"[decode balanced slices d={d} hq={hq} hkv={hkv} {mode}] B={len(lens)} max={int(lens.max())}", flush=True)
    got = gh.gpu_decode(inp, gc)
    int2, bf = gh.gpu_pages(inp, gc)
    q = synth.bf16_bits_to_f32(inp.q).astype(np.float64)
    ref = oatt.decode_attention(q, int2, bf, inp.seq_lens, inp.bt_q, inp.bt_h, rot.r_k, rot.r_v, w.n_sink, w.n_recent)
    for b, L in enumerate(lens):
        gh.assert_attention_close(got[b], ref[b], f"seq {b} len {L}")


def test_bf16_baseline_balanced_slices(tiny_rot):
    from oracle import attention as oatt
    lens = np.random.default_rng(12).integers(1, 600, size=72)
    w = _tiny(batch=len(lens), n_sink=100000, n_recent=0)   # every token in BF16 pages
    inp = synth.decode_inputs(w, seq_lens=lens)
    gc = gh.alloc_cache(inp, tiny_rot)
    gh.gpu_fill(inp, tiny_rot, gc)
    print(f"[bf16 baseline balanced slices] B={len(lens)}", flush=True)
    got = gh.gpu_decode(inp, gc, all_raw=True)
    q = synth.bf16_bits_to_f32(inp.q).astype(np.float64)
    for b, L in enumerate(lens):
        k = olayout.bf16_to_f64(inp.k_rows[inp.row_of[b], 0]); v = olayout.bf16_to_f64(inp.v_rows[inp.row_of[b], 0])
        ref = oatt.softmax_attention(q[b], k, v, 1 / 8.0)
        gh.assert_attention_close(got[b], ref, f"bf16 baseline seq {b}")


def test_abi_rejects_bad_arguments_on_device():
    w = _tiny()
    with pytest.raises(lib.OscarError) as e:
        lib.decode_workspace_bytes(1, 1, 4, 96, 512)
    assert e.value.status == 2
    with pytest.raises(lib.OscarError) as e:
        lib.decode_workspace_bytes(1, 2, 3, 128, 512)
    assert e.value.status == 1
    ws = torch.zeros(4, dtype=torch.int32, device=gh.DEV)
    inp = synth.decode_inputs(w)
    rot = gh.Rotation(np.eye(64)[None], np.eye(64)[None], 1.0, 1.0)
    gc = gh.alloc_cache(inp, rot)
    q = gh.bits_to_dev_bf16(inp.q)
    out = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device=gh.DEV)
    with pytest.raises(lib.OscarError) as e:
        lib.paged_decode_attn(gc.cache, q, gh.i32(inp.seq_lens), 512, gc.bt_q, gc.bt_h, gc.r_k, gc.r_v, out, ws)
    assert e.value.status == 4
