"""GPU parity at the workloads' full sizes, checked on sampled outputs.

Every workload is run at its real shape (sequence count, context lengths,
head counts, shuffled and aliased block tables), in the launch configuration
the benchmark uses (automatic split).  The cache is written by the library's
own kernels; the oracle then

* re-quantizes a random sample of the appended rows (codes bit-exact up to the
  rounding-boundary exemption, f16 scale/zero up to the midpoint exemption),
* decodes sampled sequences from the very pages the GPU wrote (rel-L2 <= 5e-3,
  max-abs <= 2e-2 against its float64 output).

For the batched workloads only the sampled sequences' histories are drawn;
the others keep all-zero rows (their outputs are computed but not checked).
"""
import numpy as np
import pytest
import torch

from int2_rotated_kv_oscar_amd import synth
from oracle import cache as ocache
from oracle import layout as olayout

import gpu_helpers as gh

pytestmark = pytest.mark.gpu

CALIB_ROWS = 1024  # the rotation is an input of both sides; its calibration size does not matter here


def _run(name, sample_seqs, n_code_rows=2048, seed=0, splits=(0,), stale=False):
    w = synth.WORKLOADS[name]
    lens = synth.context_lengths(w)
    if sample_seqs == "all":
        sample_seqs = list(range(len(lens)))
    print(f"[fullsize {name}] B={len(lens)} max_len={int(lens.max())} sampled={sample_seqs}", flush=True)
    inp = synth.decode_inputs(w, draw_seqs=sample_seqs)
    rot = gh.oracle_rotation(w, n_rows=CALIB_ROWS)
    gc = gh.alloc_cache(inp, rot)
    if stale:  # recycled pages: random bytes and NaN/infinity patterns wherever the fill does not write
        gh.fill_stale(gc, seed=seed)
    rows = synth.middle_rows(inp)
    print(f"[fullsize {name}] quantize_append rows={len(rows[0])}", flush=True)
    gh.gpu_fill(inp, rot, gc, rows)
    torch.cuda.synchronize()

    # codes and scales of sampled appended rows (from the sampled sequences)
    ms, mp, mr = rows
    mine = np.nonzero(np.isin(ms, sample_seqs))[0]
    rng = np.random.default_rng(seed)
    sel = np.sort(rng.choice(mine, size=min(n_code_rows, len(mine)), replace=False))
    k, v = inp.k_rows[mr[sel]], inp.v_rows[mr[sel]]
    scratch = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d)
    res = ocache.quantize_append(scratch, k, v, ms[sel], mp[sel], inp.bt_q, rot.r_k, rot.r_v, rot.tau_k, rot.tau_v,
                                 olayout.bf16_to_f64)
    int2_bytes = gc.int2.cpu().numpy()
    page = inp.bt_q[ms[sel], mp[sel] // 16].astype(np.int64)
    rep = gh.compare_appended(int2_bytes, w, inp.n_int2_pages, res, page, (mp[sel] % 16).astype(np.int64))
    print(rep, flush=True)
    gh.assert_codes_ok(rep, name)

    # the bench step's append: every sequence's row leaving the recent window,
    # appended again (the few-row kernel for these counts), checked on the
    # sampled sequences
    lv = [(b, int(L) - 1 - w.n_recent) for b, L in enumerate(lens) if int(L) - 1 - w.n_recent >= w.n_sink]
    if lv:
        ls = np.array([b for b, _ in lv]); lp = np.array([t for _, t in lv])
        lr = np.array([inp.row_of[b][t] for b, t in lv])
        print(f"[fullsize {name}] leaving-row append rows={len(lv)}", flush=True)
        from int2_rotated_kv_oscar_amd import lib
        lib.quantize_append(gc.cache, gh.bits_to_dev_bf16(inp.k_rows[lr]), gh.bits_to_dev_bf16(inp.v_rows[lr]),
                            gh.i32(ls), gh.i32(lp), gc.bt_q, gc.r_k, gc.r_v, rot.tau_k, rot.tau_v)
        torch.cuda.synchronize()
        chk = np.nonzero(np.isin(ls, sample_seqs))[0]
        res2 = ocache.quantize_append(olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d), inp.k_rows[lr[chk]],
                                      inp.v_rows[lr[chk]], ls[chk], lp[chk], inp.bt_q, rot.r_k, rot.r_v, rot.tau_k,
                                      rot.tau_v, olayout.bf16_to_f64)
        int2_bytes = gc.int2.cpu().numpy()
        rep2 = gh.compare_appended(int2_bytes, w, inp.n_int2_pages, res2, inp.bt_q[ls[chk], lp[chk] // 16].astype(np.int64),
                                   (lp[chk] % 16).astype(np.int64))
        print(rep2, flush=True)
        gh.assert_codes_ok(rep2, name + " leaving rows")

    # decode (all sequences on the GPU), checked on the sampled ones, for
    # each work split (0: the automatic one the bench uses)
    int2 = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d, int2_bytes)
    bf = olayout.Bf16Pool(inp.n_bf16_pages, w.n_kv_heads, w.d, gc.bf16.cpu().numpy().view(np.uint16))
    from oracle import attention as oatt
    sb = np.asarray(sample_seqs)
    q = synth.bf16_bits_to_f32(inp.q[sb]).astype(np.float64)
    ref = oatt.decode_attention(q, int2, bf, inp.seq_lens[sb], inp.bt_q[sb], inp.bt_h[sb], rot.r_k, rot.r_v,
                                w.n_sink, w.n_recent)
    for split in splits:
        print(f"[fullsize {name}] decode split_pages={split}", flush=True)
        got = gh.gpu_decode(inp, gc, split_pages=split)
        assert np.isfinite(got).all()
        err = gh.attention_errors(got[sb], ref)
        print(f"[fullsize {name}] decode split_pages={split} errors {err}", flush=True)
        gh.assert_attention_close(got[sb], ref, f"{name} split_pages={split}")


def test_qwen3_8b_b1_32k_bench_config():
    _run("qwen3-8b-b1-32k", "all")


def test_qwen3_8b_b28_ragged_shared_prefix():
    # on recycled pools (stale bytes and NaN/infinity patterns outside the regions)
    _run("qwen3-8b-b28-ragged", [0, 13, 27], stale=True)


def test_qwen3_32b_b1_128k():
    # automatic split, then split-K over 64 (128 pages each) and 205 (40
    # pages each) INT2 context chunks with the log-sum-exp merge
    _run("qwen3-32b-b1-128k", "all", n_code_rows=1024, splits=(0, 128, 40))


def test_qwen3_32b_b4_128k():
    # automatic split, then 64 INT2 chunks (128 pages) per (sequence, KV head)
    _run("qwen3-32b-b4-128k", [2], n_code_rows=1024, splits=(0, 128))


def test_gqa96_b64_ragged():
    _run("gqa96-b64-ragged", [5, 40], stale=True)


def test_prefill_8x8192_rows_per_sequence():
    # the large-GQA layer's prefill: 8 sequences x 8192 rows, page-aligned chunks
    w = synth.WORKLOADS["gqa96-b64-ragged"]
    n_seq, chunk = 8, 8192
    print(f"[fullsize prefill] {n_seq} x {chunk} rows", flush=True)
    k, v, row_seq, row_pos = synth.prefill_rows(w, n_seq, chunk)
    pages_per = (chunk + 15) // 16
    bt_q = synth.rng_for(w.cfg_id, 7).permutation(n_seq * pages_per).astype(np.int32).reshape(n_seq, pages_per)
    rot = gh.oracle_rotation(w, n_rows=CALIB_ROWS)
    from int2_rotated_kv_oscar_amd import lib
    int2 = torch.zeros(n_seq * pages_per * lib.int2_page_bytes(w.d, w.n_kv_heads), dtype=torch.uint8, device=gh.DEV)
    cache = lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, int2, None)
    lib.quantize_append(cache, gh.bits_to_dev_bf16(k), gh.bits_to_dev_bf16(v), gh.i32(row_seq), gh.i32(row_pos),
                        gh.i32(bt_q), torch.from_numpy(rot.r_k.astype(np.float32)).to(gh.DEV),
                        torch.from_numpy(rot.r_v.astype(np.float32)).to(gh.DEV), rot.tau_k, rot.tau_v)
    torch.cuda.synchronize()
    sel = np.sort(np.random.default_rng(1).choice(len(row_seq), size=4096, replace=False))
    scratch = olayout.Int2Pool(n_seq * pages_per, w.n_kv_heads, w.d)
    res = ocache.quantize_append(scratch, k[sel], v[sel], row_seq[sel], row_pos[sel], bt_q, rot.r_k, rot.r_v,
                                 rot.tau_k, rot.tau_v, olayout.bf16_to_f64)
    page = bt_q[row_seq[sel], row_pos[sel] // 16].astype(np.int64)
    rep = gh.compare_appended(int2.cpu().numpy(), w, n_seq * pages_per, res, page, (row_pos[sel] % 16).astype(np.int64))
    print(rep, flush=True)
    gh.assert_codes_ok(rep, "prefill 8x8192")


def test_extend_prefix_hit_qwen3_8b_b28_ragged():
    # the bench's chunked-prefill launch: the 28-sequence Qwen3-8B cache
    # (ragged contexts, a 1024-token prefix aliased by every table) extended by
    # 512 new rows per sequence, written by the library's kernels on recycled
    # pools; the oracle checks sampled rows of two sequences over those pages
    w = synth.WORKLOADS["qwen3-8b-b28-ragged"]
    lens = synth.context_lengths(w)
    print(f"[fullsize extend] B={len(lens)} max cached={int(lens.max())} new=512", flush=True)
    ext = gh.extend_inputs(w, lens, [512] * len(lens), seed=0, draw_seqs=[0, 27])
    rot = gh.oracle_rotation(w, n_rows=CALIB_ROWS)
    gc = gh.alloc_cache(ext.cache, rot)
    gh.fill_stale(gc, seed=3)
    gh.gpu_fill(ext.cache, rot, gc)
    got = gh.gpu_extend(ext, gc, 2)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(7)
    rows = sorted(set(rng.choice(512, size=24, replace=False).tolist()) | {0, 511})
    sel = [r for r in rows] + [ext.cu[27] + r for r in rows]
    ref = gh.oracle_extend_gpu_pages(ext, rot, gc, 2, seqs=[0, 27], rows=set(sel))
    err = gh.attention_errors(got[sel], ref[sel])
    print(f"[fullsize extend] errors {err}", flush=True)
    gh.assert_attention_close(got[sel], ref[sel], "extend b28")


def test_int4_decode_qwen3_8b_b1_32k():
    # the INT4 variant of the bench's decode workload at full size
    w = synth.WORKLOADS["qwen3-8b-b1-32k"]
    inp = synth.decode_inputs(w)
    rot = gh.oracle_rotation(w, n_rows=CALIB_ROWS)
    gc = gh.alloc_cache(inp, rot, bits=4)
    print("[fullsize int4 decode] fill", flush=True)
    gh.gpu_fill(inp, rot, gc, bits=4)
    torch.cuda.synchronize()
    got = gh.gpu_decode_int4(inp, gc)
    ref = gh.oracle_decode_gpu_pages(inp, rot, gc, bits=4)
    err = gh.attention_errors(got, ref)
    print(f"[fullsize int4 decode] errors {err}", flush=True)
    gh.assert_attention_close(got, ref, "int4 decode 32k")


def test_int4_decode_qwen3_32b_b4_128k():
    # the INT4 decode at the 128k batch-4 shape (8 queries per KV head, stale
    # pools), checked on one sampled sequence
    w = synth.WORKLOADS["qwen3-32b-b4-128k"]
    seqs = [3]
    inp = synth.decode_inputs(w, draw_seqs=seqs)
    rot = gh.oracle_rotation(w, n_rows=CALIB_ROWS)
    gc = gh.alloc_cache(inp, rot, bits=4)
    gh.fill_stale(gc, seed=3)
    print("[fullsize int4 decode 128k b4] fill", flush=True)
    gh.gpu_fill(inp, rot, gc, bits=4)
    torch.cuda.synchronize()
    got = gh.gpu_decode_int4(inp, gc)
    assert np.isfinite(got).all()
    from oracle import attention as oatt
    pool, bf = gh.gpu_pages(inp, gc, bits=4)
    sb = np.asarray(seqs)
    q = synth.bf16_bits_to_f32(inp.q[sb]).astype(np.float64)
    ref = oatt.decode_attention(q, pool, bf, inp.seq_lens[sb], inp.bt_q[sb], inp.bt_h[sb], rot.r_k, rot.r_v,
                                w.n_sink, w.n_recent)
    err = gh.attention_errors(got[seqs], ref)
    print(f"[fullsize int4 decode 128k b4] errors {err}", flush=True)
    gh.assert_attention_close(got[seqs], ref, "int4 decode 128k b4")
