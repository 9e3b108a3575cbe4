"""The decode entry point that allocates nothing (its arrival counters and
records in the library's built-in device scratch) against the workspace one,
through the C ABI: bit-identical outputs on the same work plan, on two calls
in a row (the second smaller), and the size limit rejected on the host."""
import numpy as np
import pytest
import torch

from int2_rotated_kv_oscar_amd import lib, synth  # noqa: F401

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _noalloc(inp, gc, split_pages=0):
    w = inp.w
    B = len(inp.seq_lens)
    q = gh.bits_to_dev_bf16(inp.q)
    out = torch.full((B, w.n_q_heads, w.d), float("nan"), dtype=torch.bfloat16, device=gh.DEV)
    lib.paged_decode_attn_noalloc(gc.cache, q, gh.i32(inp.seq_lens), inp.max_seq_len, gc.bt_q, gc.bt_h, gc.r_k,
                                  gc.r_v, out, split_pages=split_pages)
    torch.cuda.synchronize()
    return gh.dev_bf16_to_f64(out)


def test_noalloc_matches_workspace_decode_twice():
    # a ragged batch of 80 sequences (the balanced-slice kernel), then one
    # sequence (per-unit items); each equal to the workspace entry point's
    # output bit for bit, and both within the oracle's bar
    big_lens = np.random.default_rng(3).integers(1, 900, size=80)
    cases = [("tiny-b80", big_lens, 0), ("tiny-b1", np.array([700]), 8)]
    for name, lens, split in cases:
        w = synth.Workload(**{**synth.WORKLOADS["tiny"].__dict__, "batch": len(lens), "name": name,
                              "ctx": ("fixed", 900, 900)})
        rot = gh.oracle_rotation(w, n_rows=512)
        inp = synth.decode_inputs(w, seq_lens=lens)
        gc = gh.alloc_cache(inp, rot)
        gh.gpu_fill(inp, rot, gc)
        print(f"[noalloc {name}] B={len(lens)} split={split}", flush=True)
        got = _noalloc(inp, gc, split)
        ref_ws = gh.gpu_decode(inp, gc, split_pages=split)
        assert np.array_equal(got, ref_ws), f"{name}: no-alloc output differs from the workspace entry point"
        ref = gh.oracle_decode_gpu_pages(inp, rot, gc)
        for b in range(len(lens)):
            gh.assert_attention_close(got[b], ref[b], f"{name} seq {b}")


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 64 sequences x 8 KV heads at 1M tokens with 8-page items needs far more
    # records than the built-in 32 MiB: rejected on the host, nothing launched
    int2 = torch.zeros(lib.int2_page_bytes(128, 8), dtype=torch.uint8, device=gh.DEV)
    bf16 = torch.zeros(lib.bf16_page_bytes(128, 8) // 2, dtype=torch.int16, device=gh.DEV)
    q = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device=gh.DEV)
    out = torch.zeros_like(q)
    cache = lib.make_cache(128, 8, 4, 32, int2, bf16)
    bt = torch.zeros(64, 65536, dtype=torch.int32, device=gh.DEV)
    sl = torch.full((64,), 1 << 20, dtype=torch.int32, device=gh.DEV)
    rk = torch.zeros(8, 128, 128, dtype=torch.float32, device=gh.DEV)
    with pytest.raises(lib.OscarError) as e:
        lib.paged_decode_attn_noalloc(cache, q, sl, 1 << 20, bt, bt, rk, rk, out, split_pages=4096)
    assert e.value.status == 4
