"""The fused decode step (oscar_decode_step): the step's cache update and the
decode attention in one launch.

Over several consecutive steps on a stale (recycled) pool, each step's pools
must hold exactly the bytes the two-launch sequence (oscar_decode_step_update,
then oscar_paged_decode_attn) writes, and each step's output must match the
oracle's decode over the pages the GPU wrote (rel-L2 <= 5e-3, max-abs <=
2e-2).  After the last step every middle token's codes and f16 scale/zero are
checked against the oracle's fill of the whole history, and every sink and
recent token's BF16 slot against its raw row, bit for bit.  At full size (the
benchmark's default Qwen3-8B 32k workload and the 128k batch-4 one, automatic
plan, stale pools) the same holds on sampled sequences, with the rows each step
wrote checked against the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

from int2_rotated_kv_oscar_amd import lib, synth
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import layout as olayout

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _full_tables(inp: synth.DecodeInputs, seed: int) -> synth.DecodeInputs:
    """Every logical page of every sequence mapped in both pools (the region
    of a position changes from step to step), each pool a seeded permutation;
    the pages of a shared prefix stay shared (every sequence maps them to
    sequence 0's pages, which the fill writes once)."""
    B, mp = inp.bt_q.shape
    rng = np.random.default_rng(seed)
    bt_q = rng.permutation(B * mp).astype(np.int32).reshape(B, mp)
    bt_h = rng.permutation(B * mp).astype(np.int32).reshape(B, mp)
    pre_pages = inp.w.shared_prefix // 16
    if pre_pages:
        bt_q[:, :pre_pages] = bt_q[0, :pre_pages]
        bt_h[:, :pre_pages] = bt_h[0, :pre_pages]
    return dataclasses.replace(inp, bt_q=bt_q, bt_h=bt_h, n_int2_pages=B * mp, n_bf16_pages=B * mp)


def _clone(gc: gh.GpuCache, w: synth.Workload) -> gh.GpuCache:
    int2, bf16 = gc.int2.clone(), gc.bf16.clone()
    cache = lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, int2, bf16)
    return dataclasses.replace(gc, int2=int2, bf16=bf16, cache=cache)


def _bf16_slots_exact(inp: synth.DecodeInputs, gc: gh.GpuCache):
    w = inp.w
    bf = olayout.Bf16Pool(inp.n_bf16_pages, w.n_kv_heads, w.d, gc.bf16.cpu().numpy().view(np.uint16))
    hs, hp, hr = synth.bf16_rows(inp)
    page = inp.bt_h[hs, hp // 16]
    for h in range(w.n_kv_heads):
        k, v = bf.read(page, hp % 16, h)
        assert np.array_equal(k, inp.k_rows[hr, h]), f"BF16 K slots differ (head {h})"
        assert np.array_equal(v, inp.v_rows[hr, h]), f"BF16 V slots differ (head {h})"


def _run_steps(w: synth.Workload, final_lens, n_steps: int, split_pages: int = 0, seed: int = 0):
    final_lens = np.asarray(final_lens, np.int32)
    grow = final_lens > 0                       # empty sequences stay empty
    inp_f = _full_tables(synth.decode_inputs(w, seq_lens=final_lens), 500 + seed)
    rot = gh.oracle_rotation(w, n_rows=512)
    lens0 = np.where(grow, final_lens - n_steps, 0).astype(np.int32)
    assert lens0.min() >= 0
    inp0 = dataclasses.replace(inp_f, seq_lens=lens0)
    fused = gh.alloc_cache(inp0, rot)
    gh.fill_stale(fused, seed)
    gh.gpu_fill(inp0, rot, fused)
    torch.cuda.synchronize()
    two = _clone(fused, w)
    B, hq, hkv, d = len(final_lens), w.n_q_heads, w.n_kv_heads, w.d
    mixers = synth.query_mixers(w)
    max_ws = lib.decode_workspace_bytes(B, hkv, hq, d, int(final_lens.max()), split_pages)
    ws_f = torch.empty((max_ws + 3) // 4, dtype=torch.int32, device=gh.DEV)
    ws_t = torch.empty_like(ws_f)
    lib.decode_workspace_init(ws_f)
    lib.decode_workspace_init(ws_t)
    for s in range(n_steps):
        lens = np.where(grow, lens0 + s + 1, 0).astype(np.int32)
        max_len = int(lens.max())
        newrow = np.array([inp_f.row_of[b][L - 1] if L else 0 for b, L in enumerate(lens)], np.int64)
        k_new = gh.bits_to_dev_bf16(inp_f.k_rows[newrow])
        v_new = gh.bits_to_dev_bf16(inp_f.v_rows[newrow])
        q_bits = synth.q_rows(synth.rng_for(w.cfg_id, 60 + s), B, w, mixers)
        q = gh.bits_to_dev_bf16(q_bits)
        sl = gh.i32(lens)
        out_f = torch.full((B, hq, d), float("nan"), dtype=torch.bfloat16, device=gh.DEV)
        out_t = torch.full_like(out_f, float("nan"))
        print(f"[decode step {s}] d={d} hq={hq} hkv={hkv} S={w.n_sink} W={w.n_recent} B={B} "
              f"split={split_pages} max_len={max_len}", flush=True)
        lib.decode_step(fused.cache, k_new, v_new, q, sl, max_len, fused.bt_q, fused.bt_h, fused.r_k, fused.r_v,
                        rot.tau_k, rot.tau_v, out_f, ws_f, split_pages=split_pages)
        lib.decode_step_update(two.cache, k_new, v_new, sl, two.bt_q, two.bt_h, two.r_k, two.r_v, rot.tau_k,
                               rot.tau_v)
        lib.paged_decode_attn(two.cache, q, sl, max_len, two.bt_q, two.bt_h, two.r_k, two.r_v, out_t, ws_t,
                              split_pages=split_pages)
        torch.cuda.synchronize()
        assert torch.equal(fused.int2, two.int2), f"step {s}: INT2 pool differs from the two-launch step"
        assert torch.equal(fused.bf16, two.bf16), f"step {s}: BF16 pool differs from the two-launch step"
        got = gh.dev_bf16_to_f64(out_f)
        inp_s = dataclasses.replace(inp_f, seq_lens=lens)
        ref = gh.oracle_decode(inp_s, rot, *gh.gpu_pages(inp_s, fused), q_bits=q_bits)
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(got[b] == 0)
            else:
                gh.assert_attention_close(got[b], ref[b], f"step {s} seq {b} len {L}")
    inp_end = dataclasses.replace(inp_f, seq_lens=np.where(grow, final_lens, 0).astype(np.int32))
    gh.check_fill(inp_end, rot, fused, "after the steps")
    _bf16_slots_exact(inp_end, fused)


def _wl(d, hq, hkv, S, W, B, cfg=41):
    return synth.Workload("step", cfg, B, hq, hkv, d, S, W, 512, ("fixed", 1, 1))


def test_decode_step_region_edges():
    # lengths that start at 0, below the sink, at the sink/recent edges, just
    # before and after a page boundary of the middle, and long enough for
    # several INT2 pages; 24 steps move the middle's end across pages
    S, W = 4, 32
    starts = np.array([0, 2, S, S + W - 3, S + W, S + W + 1, 47, 64 + S + W - 1, 300, 511], np.int32)
    _run_steps(_wl(64, 4, 1, S, W, len(starts)), starts + 24, 24)


@pytest.mark.parametrize("d,hq,hkv,S,W,split", [
    (128, 32, 8, 4, 128, 0),    # group of 4: four column slots per query
    (128, 16, 2, 4, 32, 0),     # group of 8: two column slots per query
    (64, 6, 1, 4, 16, 8),       # group of 6: two slots, the last four columns unused
    (128, 16, 1, 4, 64, 0),     # group of 16
    (64, 8, 2, 0, 16, 8),       # no sink; 8 INT2 pages per workgroup, the last middle page in one of several
    (64, 4, 1, 4, 0, 0),        # no recent window: the new token goes straight to INT2
    (128, 2, 2, 0, 0, 8),       # neither: every token quantized, 8 pages per workgroup
    (64, 4, 1, 1000, 16, 0),    # sink longer than every sequence: nothing quantized
])
def test_decode_step_shapes(d, hq, hkv, S, W, split):
    starts = np.array([0, 1, 15, 16, 17, 150, 333], np.int32)
    _run_steps(_wl(d, hq, hkv, S, W, len(starts), cfg=42 + d + S + W), starts + 18, 18, split_pages=split,
               seed=d + W)


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 16, 2), (128, 32, 2), (64, 16, 8)])
def test_decode_step_balanced_slices(d, hq, hkv):
    # many (sequence, KV head) units: the balanced-slice kernel, whose
    # workgroups cross units and page kinds (groups of 4, 8 and 16); 144 units
    # take the fused launch, 576 units (more than the CUs) the update kernel
    # and then the decode
    rng = np.random.default_rng(5)
    starts = rng.integers(0, 400, size=72).astype(np.int32)
    starts[:4] = [0, 35, 36, 37]
    lens = starts + 6
    lens[9] = 0   # an empty sequence in the batch
    _run_steps(_wl(d, hq, hkv, 4, 32, len(lens), cfg=47), lens, 6, seed=3)


def test_decode_step_long_items_first_item_takes_int2_pages():
    # 64 units of up to 20k tokens (group of 4) on 256 CUs: per-unit items of
    # 376 pages, item 0 holding the BF16 pages and the first 152 INT2 pages;
    # the ragged lengths give middles shorter than that first chunk, empty
    # middles, an empty sequence and partial last items
    lens = np.array([20000, 9000, 2500, 150, 0, 18, 16000, 5000], np.int32)
    _run_steps(_wl(128, 32, 8, 4, 128, len(lens), cfg=49), lens, 3, seed=7)


def test_decode_step_rejects_bad_arguments():
    w = _wl(64, 4, 1, 4, 32, 1)
    inp = _full_tables(synth.decode_inputs(w, seq_lens=np.array([40], np.int32)), 1)
    rot = gh.Rotation(np.eye(64)[None], np.eye(64)[None], 1.0, 1.0)
    gc = gh.alloc_cache(inp, rot)
    q = gh.bits_to_dev_bf16(inp.q)
    kv = torch.zeros(1, 1, 64, dtype=torch.bfloat16, device=gh.DEV)
    out = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device=gh.DEV)
    ws = torch.zeros((lib.decode_workspace_bytes(1, 1, 4, 64, 40) + 3) // 4, dtype=torch.int32, device=gh.DEV)
    lib.decode_workspace_init(ws)
    sl = gh.i32(inp.seq_lens)
    for tau in ((0.0, 1.0), (1.0, float("nan")), (float("inf"), 1.0)):
        with pytest.raises(lib.OscarError) as e:
            lib.decode_step(gc.cache, kv, kv, q, sl, 40, gc.bt_q, gc.bt_h, gc.r_k, gc.r_v, *tau, out, ws)
        assert e.value.status == 1
    with pytest.raises(lib.OscarError) as e:
        lib.decode_step(gc.cache, kv, kv, q, sl, 40, gc.bt_q, gc.bt_h, gc.r_k, gc.r_v, 1.0, 1.0, out, ws[:4])
    assert e.value.status == 4


def _run_full_size_steps(name: str, n_steps: int, check_seqs):
    """The benchmark's timed call (oscar_decode_step, automatic plan) at a
    workload's full size, on a stale pool: every step's pools equal the
    two-launch sequence's bytes, the sampled sequences' outputs match the
    oracle over the GPU's pages, and the rows the steps wrote (each new
    token's BF16 slot, each entering token's INT2 codes and f16 scale/zero)
    match their raw rows and the oracle's quantization."""
    w = synth.WORKLOADS[name]
    final = synth.context_lengths(w)
    sb = np.asarray(check_seqs)
    inp_f = _full_tables(synth.decode_inputs(w, seq_lens=final, draw_seqs=check_seqs), 900)
    rot = gh.oracle_rotation(w, n_rows=1024)
    lens0 = (final - n_steps).astype(np.int32)
    inp0 = dataclasses.replace(inp_f, seq_lens=lens0)
    print(f"[full-size step {name}] B={len(final)} max_len={int(final.max())} steps={n_steps} checked={list(sb)}",
          flush=True)
    fused = gh.alloc_cache(inp0, rot)
    gh.fill_stale(fused, 7)
    gh.gpu_fill(inp0, rot, fused)
    torch.cuda.synchronize()
    two = _clone(fused, w)
    B, hq, hkv, d = len(final), w.n_q_heads, w.n_kv_heads, w.d
    mixers = synth.query_mixers(w)
    ws_b = lib.decode_workspace_bytes(B, hkv, hq, d, int(final.max()))
    ws_f = torch.empty((ws_b + 3) // 4, dtype=torch.int32, device=gh.DEV)
    ws_t = torch.empty_like(ws_f)
    lib.decode_workspace_init(ws_f)
    lib.decode_workspace_init(ws_t)
    entered = []  # (sequence, position) of the tokens the steps moved into INT2
    for s in range(n_steps):
        lens = (lens0 + s + 1).astype(np.int32)
        max_len = int(lens.max())
        newrow = np.array([inp_f.row_of[b][L - 1] for b, L in enumerate(lens)], np.int64)
        k_new = gh.bits_to_dev_bf16(inp_f.k_rows[newrow])
        v_new = gh.bits_to_dev_bf16(inp_f.v_rows[newrow])
        q_bits = synth.q_rows(synth.rng_for(w.cfg_id, 70 + s), B, w, mixers)
        q = gh.bits_to_dev_bf16(q_bits)
        sl = gh.i32(lens)
        out_f = torch.full((B, hq, d), float("nan"), dtype=torch.bfloat16, device=gh.DEV)
        out_t = torch.full_like(out_f, float("nan"))
        print(f"[full-size step {name}] step {s} max_len={max_len}", flush=True)
        lib.decode_step(fused.cache, k_new, v_new, q, sl, max_len, fused.bt_q, fused.bt_h, fused.r_k, fused.r_v,
                        rot.tau_k, rot.tau_v, out_f, ws_f)
        lib.decode_step_update(two.cache, k_new, v_new, sl, two.bt_q, two.bt_h, two.r_k, two.r_v, rot.tau_k,
                               rot.tau_v)
        lib.paged_decode_attn(two.cache, q, sl, max_len, two.bt_q, two.bt_h, two.r_k, two.r_v, out_t, ws_t)
        torch.cuda.synchronize()
        assert torch.equal(fused.int2, two.int2), f"step {s}: INT2 pool differs from the two-launch step"
        assert torch.equal(fused.bf16, two.bf16), f"step {s}: BF16 pool differs from the two-launch step"
        got = gh.dev_bf16_to_f64(out_f)
        assert np.isfinite(got).all()
        inp_s = dataclasses.replace(inp_f, seq_lens=lens)
        int2, bf = gh.gpu_pages(inp_s, fused)
        qs = synth.bf16_bits_to_f32(q_bits[sb]).astype(np.float64)
        ref = oatt.decode_attention(qs, int2, bf, lens[sb], inp_f.bt_q[sb], inp_f.bt_h[sb], rot.r_k, rot.r_v,
                                    w.n_sink, w.n_recent)
        err = gh.attention_errors(got[sb], ref)
        print(f"[full-size step {name}] step {s} errors {err}", flush=True)
        gh.assert_attention_close(got[sb], ref, f"{name} step {s}")
        entered += [(int(b), int(lens[b]) - 1 - w.n_recent) for b in sb if int(lens[b]) - 1 - w.n_recent >= w.n_sink]
    # the entering tokens' codes and f16 scale/zero, against the oracle
    es = np.array([b for b, _ in entered]); ep = np.array([t for _, t in entered])
    er = np.array([inp_f.row_of[b][t] for b, t in entered])
    res = ocache.quantize_append(olayout.Int2Pool(inp_f.n_int2_pages, hkv, d), inp_f.k_rows[er], inp_f.v_rows[er],
                                 es, ep, inp_f.bt_q, rot.r_k, rot.r_v, rot.tau_k, rot.tau_v, olayout.bf16_to_f64)
    rep = gh.compare_appended(fused.int2.cpu().numpy(), w, inp_f.n_int2_pages, res,
                              inp_f.bt_q[es, ep // 16].astype(np.int64), (ep % 16).astype(np.int64))
    print(rep, flush=True)
    gh.assert_codes_ok(rep, f"{name} entering tokens")
    # the new tokens' BF16 slots hold their raw rows
    bfp = olayout.Bf16Pool(inp_f.n_bf16_pages, hkv, d, fused.bf16.cpu().numpy().view(np.uint16))
    for b in sb:
        for s in range(n_steps):
            t = int(lens0[b]) + s
            page = inp_f.bt_h[b, t // 16]
            for h in range(hkv):
                k, v = bfp.read(np.array([page]), np.array([t % 16]), h)
                r = inp_f.row_of[b][t]
                assert np.array_equal(k[0], inp_f.k_rows[r, h]) and np.array_equal(v[0], inp_f.v_rows[r, h]), \
                    f"BF16 slot of token {t} (sequence {b}, head {h})"


def test_decode_step_full_size_bench_config():
    # the benchmark's default workload: Qwen3-8B layer, one 32k sequence (one fused launch per step)
    _run_full_size_steps("qwen3-8b-b1-32k", 2, [0])


def test_decode_step_full_size_qwen3_32b_b4_128k():
    # four 128k sequences, 8 queries per KV head (one fused launch per step)
    _run_full_size_steps("qwen3-32b-b4-128k", 1, [1])


def test_decode_step_full_size_qwen3_8b_b28_ragged():
    # 28 ragged sequences with a shared prefix: balanced slices over 224
    # units, one fused launch per step
    _run_full_size_steps("qwen3-8b-b28-ragged", 2, [0, 13])
