"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
drive the C ABI through the binding, and compare against the oracle with the
acceptance rules (bit-exact codes up to the rounding-boundary exemption, f16
scale/zero equality up to the f16-midpoint exemption, attention rel-L2 and
max-abs bounds)."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from int2_rotated_kv_oscar_amd import lib, synth
from oracle import cache as ocache
from oracle import layout as olayout
from oracle import quant as oquant
from oracle import rotation as orot

DEV = "cuda:0"
BOUNDARY_EPS = 1e-5        # codes may differ where (y - z)/s is this close to k + 1/2
MIDPOINT_REL = 1e-6        # f16 scale/zero may differ this close to an f16 midpoint, relative to max|y| of the group
FLIP_BUDGET = 1e-4         # at most 0.01 % of codes may differ from the oracle's (all exempt)
# Groups whose f16 scale or zero rounds to the neighbouring f16 value (the
# oracle's float64 value lies within the 1e-6 window of a rounding midpoint).
# Agreement to 1e-6 of the group's magnitude, the acceptance bar, lets up to
# about 2 * 1e-6 / 2^-11 = 0.4 % of f16 values straddle a midpoint; the kernels'
# float32 values (about 2^-22 of the magnitude) move about 0.03 % of groups.
GROUP_BUDGET = 1e-3
GROUP_ALLOWANCE = 4  # any test may hold this many (a rare event counted over a few thousand groups)
ATT_REL_L2 = 5e-3
ATT_MAX_ABS = 2e-2


def bits_to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    b = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


@dataclasses.dataclass
class Rotation:
    r_k: np.ndarray   # float32-exact float64 [H_kv, d, d]
    r_v: np.ndarray
    tau_k: float      # float32-exact
    tau_v: float


def oracle_rotation(w: synth.Workload, n_rows: int | None = None, q_scale=None) -> Rotation:
    """Calibrate with the oracle, round once to float32 (what both sides get)."""
    cal = synth.calibration_set(w, n_rows=n_rows, q_scale=q_scale)
    rt = orot.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    f = lambda a: np.asarray(a, np.float32).astype(np.float64)  # noqa: E731
    return Rotation(f(rt["r_k"]), f(rt["r_v"]), float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"])))


@dataclasses.dataclass
class GpuCache:
    int2: torch.Tensor
    bf16: torch.Tensor
    cache: lib.OscarCache
    bt_q: torch.Tensor
    bt_h: torch.Tensor
    r_k: torch.Tensor
    r_v: torch.Tensor


def alloc_cache(inp: synth.DecodeInputs, rot: Rotation, int2_bytes: np.ndarray | None = None,
                bf16_bits: np.ndarray | None = None, bits: int = 2) -> GpuCache:
    """Device pools for a decode batch; with bits = 4 the quantized pool is INT4."""
    w = inp.w
    nb_q = lib.int2_page_bytes(w.d, w.n_kv_heads) if bits == 2 else lib.int4_page_bytes(w.d, w.n_kv_heads)
    nb_h = lib.bf16_page_bytes(w.d, w.n_kv_heads)
    if int2_bytes is None:
        int2 = torch.zeros(inp.n_int2_pages * nb_q, dtype=torch.uint8, device=DEV)
    else:
        int2 = torch.from_numpy(np.ascontiguousarray(int2_bytes).reshape(-1)).to(DEV)
    if bf16_bits is None:
        bf16 = torch.zeros(inp.n_bf16_pages * nb_h // 2, dtype=torch.int16, device=DEV)
    else:
        bf16 = torch.from_numpy(np.ascontiguousarray(bf16_bits).reshape(-1).view(np.int16)).to(DEV)
    cache = lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, int2, bf16, code_bits=bits)
    return GpuCache(int2, bf16, cache, i32(inp.bt_q), i32(inp.bt_h),
                    torch.from_numpy(rot.r_k.astype(np.float32)).to(DEV),
                    torch.from_numpy(rot.r_v.astype(np.float32)).to(DEV))


def fill_stale(gc: GpuCache, seed: int = 0):
    """Pools as paged serving leaves them (recycled pages): every 16-bit half
    random, a quarter of them f16/bf16 NaN or infinity bit patterns.  A fill
    afterwards rewrites only the slots of the regions; the decode must never
    let the rest reach its sums."""
    g = torch.Generator(device=DEV)
    g.manual_seed(1234 + seed)
    pats = torch.tensor([0x7E00, 0x7C00, 0xFC00, 0x7FC0, 0x7F80, 0xFF80, 0xFFFF, 0x7FFF], dtype=torch.int32,
                        device=DEV)
    for buf in (gc.int2, gc.bf16):
        h = buf.view(torch.int16)
        r = torch.randint(0, 65536, h.shape, generator=g, device=DEV, dtype=torch.int32)
        pick = torch.randint(0, 4 * len(pats), h.shape, generator=g, device=DEV, dtype=torch.int32)
        r = torch.where(pick < len(pats), pats[pick.clamp(max=len(pats) - 1)], r)
        h.copy_((r - 65536 * (r >= 32768).int()).to(torch.int16))
    torch.cuda.synchronize()


def gpu_fill(inp: synth.DecodeInputs, rot: Rotation, gc: GpuCache, rows=None, bits: int = 2):
    """Quantize-append every middle row and store every sink/recent row."""
    ms, mp, mr = synth.middle_rows(inp) if rows is None else rows
    if len(ms):
        (lib.quantize_append if bits == 2 else lib.quantize_append_int4)(gc.cache, bits_to_dev_bf16(inp.k_rows[mr]), bits_to_dev_bf16(inp.v_rows[mr]), i32(ms),
                            i32(mp), gc.bt_q, gc.r_k, gc.r_v, rot.tau_k, rot.tau_v)
    hs, hp, hr = synth.bf16_rows(inp)
    if len(hs):
        lib.write_bf16(gc.cache, bits_to_dev_bf16(inp.k_rows[hr]), bits_to_dev_bf16(inp.v_rows[hr]), i32(hs),
                       i32(hp), gc.bt_h)


def gpu_decode(inp: synth.DecodeInputs, gc: GpuCache, split_pages: int = 0, all_raw: bool = False,
               q_bits: np.ndarray | None = None, seq_lens=None) -> np.ndarray:
    w = inp.w
    lens = inp.seq_lens if seq_lens is None else np.asarray(seq_lens, np.int32)
    B = len(lens)
    max_len = int(lens.max()) if B else 0
    ws_bytes = lib.decode_workspace_bytes(B, w.n_kv_heads, w.n_q_heads, w.d, max_len, split_pages)
    ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.int32, device=DEV)
    lib.decode_workspace_init(ws)
    q = bits_to_dev_bf16(inp.q if q_bits is None else q_bits)
    out = torch.full((B, w.n_q_heads, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    sl = i32(lens)
    if all_raw:
        lib.paged_decode_attn_bf16(gc.cache, q, sl, max_len, gc.bt_h, out, ws, split_pages=split_pages)
    else:
        lib.paged_decode_attn(gc.cache, q, sl, max_len, gc.bt_q, gc.bt_h, gc.r_k, gc.r_v, out, ws,
                              split_pages=split_pages)
    torch.cuda.synchronize()
    return dev_bf16_to_f64(out)


def oracle_pools(inp: synth.DecodeInputs, rot: Rotation, bits: int = 2):
    return ocache.build_from_inputs(inp, rot.r_k, rot.r_v, rot.tau_k, rot.tau_v, bits)


def gpu_pages(inp: synth.DecodeInputs, gc: GpuCache, bits: int = 2):
    """The pools the GPU wrote, as oracle page images (read back)."""
    w = inp.w
    cls = olayout.Int2Pool if bits == 2 else olayout.Int4Pool
    return (cls(inp.n_int2_pages, w.n_kv_heads, w.d, gc.int2.cpu().numpy()),
            olayout.Bf16Pool(inp.n_bf16_pages, w.n_kv_heads, w.d, gc.bf16.cpu().numpy().view(np.uint16)))


def oracle_decode(inp: synth.DecodeInputs, rot: Rotation, int2: olayout.Int2Pool, bf: olayout.Bf16Pool,
                  q_bits=None, seq_lens=None) -> np.ndarray:
    from oracle import attention as oatt
    q = synth.bf16_bits_to_f32(inp.q if q_bits is None else q_bits).astype(np.float64)
    lens = inp.seq_lens if seq_lens is None else seq_lens
    return oatt.decode_attention(q, int2, bf, lens, inp.bt_q, inp.bt_h, rot.r_k, rot.r_v, inp.w.n_sink,
                                 inp.w.n_recent)


def oracle_decode_gpu_pages(inp: synth.DecodeInputs, rot: Rotation, gc: GpuCache, seq_lens=None,
                            bits: int = 2) -> np.ndarray:
    """The oracle's decode over the very pages the GPU wrote (read back), so a
    code or scale the GPU legitimately rounded the other way at an exempt
    boundary is decoded the same way on both sides."""
    pool, bf = gpu_pages(inp, gc, bits)
    return oracle_decode(inp, rot, pool, bf, seq_lens=seq_lens)


def check_fill(inp: synth.DecodeInputs, rot: Rotation, gc: GpuCache, what="", bits: int = 2):
    """Codes and scale/zero of every middle row the GPU fill wrote, against the oracle's fill."""
    _, _, res, (ms, mp, _) = oracle_pools(inp, rot, bits)
    page = inp.bt_q[ms, mp // 16].astype(np.int64)
    rep = compare_appended(gc.int2.cpu().numpy(), inp.w, inp.n_int2_pages, res, page, (mp % 16).astype(np.int64),
                           bits)
    assert_codes_ok(rep, what)
    return rep


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def attention_errors(got: np.ndarray, ref: np.ndarray):
    """(rel-L2, max-abs) of a bf16 output against the float64 reference.

    max-abs is taken beyond the half-ulp the bf16 output format itself
    rounds away (|out| reaches ~20 on outlier channels, where one bf16 ulp is
    0.125, more than the arithmetic tolerance)."""
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    if not diff.size:
        return rel, 0.0
    beyond = np.maximum(np.abs(diff) - 0.5 * bf16_ulp(got), 0.0)
    return rel, float(beyond.max())


def assert_attention_close(got, ref, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    rel, mx = attention_errors(got, ref)
    assert rel <= ATT_REL_L2 and mx <= ATT_MAX_ABS, f"{what}: rel-L2 {rel:.3g} max-abs {mx:.3g}"
    return rel, mx


@dataclasses.dataclass
class CodeReport:
    n_codes: int
    exempt_flips: int   # codes at a rounding boundary that differ (against the reference codes below)
    bad_codes: int      # codes that differ away from any exemption
    n_groups: int
    exempt_groups: int  # scale or zero one f16 step off, at an f16 rounding midpoint
    bad_groups: int     # scale or zero different away from a midpoint
    changed_codes: int = 0  # codes different from the oracle's own codes, for any (exempt) reason


def compare_appended(gpu_int2: np.ndarray, inp_w: synth.Workload, n_pages: int, res: ocache.AppendResult,
                     page: np.ndarray, slot: np.ndarray, bits: int = 2) -> CodeReport:
    """Codes and f16 scale/zero the GPU wrote for rows (page, slot) vs the
    oracle's record ``res`` of the same rows (INT2 or INT4 pages)."""
    top = (1 << bits) - 1
    pool = (olayout.Int2Pool if bits == 2 else olayout.Int4Pool)(n_pages, inp_w.n_kv_heads, inp_w.d, gpu_int2)
    n_codes = flips = bad = n_groups = ex_groups = bad_groups = changed = 0
    for h in range(inp_w.n_kv_heads):
        ck, cv, ks, kz, vs, vz = pool.read(page, slot, h)
        for codes, s16, z16, ref in ((ck, ks, kz, res.k[h]), (cv, vs, vz, res.v[h])):
            n, d = codes.shape
            ng = d // 32
            s_eq = s16.view(np.uint16) == ref.s16.view(np.uint16)
            z_eq = z16.view(np.uint16) == ref.z16.view(np.uint16)
            grp_ok = s_eq & z_eq
            # window: 1e-6 of the group's magnitude max|y| (a zero point near 0
            # is as uncertain in absolute terms as any other value of its group)
            gmax = np.abs(ref.y.reshape(n, ng, 32)).max(axis=2)
            near = (oquant.f16_midpoint_distance(ref.s) * np.abs(ref.s) <= MIDPOINT_REL * gmax) | \
                   (oquant.f16_midpoint_distance(ref.z) * np.abs(ref.z) <= MIDPOINT_REL * gmax)
            n_groups += grp_ok.size
            ex_groups += int((~grp_ok & near).sum())
            bad_groups += int((~grp_ok & ~near).sum())
            for (i, g) in list(zip(*np.nonzero(~grp_ok & ~near)))[:8]:
                yg = ref.y[i, 32 * g:32 * g + 32]
                print(f"  bad group h={h} row={i} g={g}: s64={ref.s[i, g]!r} z64={ref.z[i, g]!r} "
                      f"s16 gpu/ora={float(s16[i, g])!r}/{float(ref.s16[i, g])!r} "
                      f"z16 gpu/ora={float(z16[i, g])!r}/{float(ref.z16[i, g])!r} "
                      f"mid-dist s={oquant.f16_midpoint_distance(ref.s[i:i+1, g])[0]:.3g} "
                      f"z={oquant.f16_midpoint_distance(ref.z[i:i+1, g])[0]:.3g} "
                      f"sum|y|={np.abs(yg).sum():.4g} max|y|={np.abs(yg).max():.4g}", flush=True)
            # reference codes: the oracle's, or re-quantized with the GPU's s/z where those legitimately differ
            t = ref.t.reshape(n, ng, 32).copy()
            ref_codes = ref.codes.reshape(n, ng, 32).astype(np.int64)
            if (~grp_ok).any():
                sg = s16.astype(np.float64)[:, :, None]
                zg = z16.astype(np.float64)[:, :, None]
                with np.errstate(divide="ignore", invalid="ignore"):
                    t2 = np.where(sg != 0, (ref.y.reshape(n, ng, 32) - zg) / sg, np.nan)
                c2 = np.where(sg != 0, np.clip(np.rint(np.nan_to_num(t2)), 0, top), 0).astype(np.int64)
                sel = np.broadcast_to(~grp_ok[:, :, None], t.shape)
                t[sel] = t2[sel]
                ref_codes[sel] = c2[sel]
            mism = codes.reshape(n, ng, 32).astype(np.int64) != ref_codes
            changed += int((codes.reshape(-1).astype(np.int64) != ref.codes.reshape(-1).astype(np.int64)).sum())
            exempt = oquant.boundary_distance(t, bits) <= BOUNDARY_EPS
            n_codes += codes.size
            flips += int((mism & exempt).sum())
            bad += int((mism & ~exempt).sum())
    return CodeReport(n_codes, flips, bad, n_groups, ex_groups, bad_groups, changed)


def assert_codes_ok(rep: CodeReport, what=""):
    assert rep.bad_codes == 0, f"{what}: {rep.bad_codes} non-exempt code mismatches ({rep})"
    assert rep.bad_groups == 0, f"{what}: {rep.bad_groups} scale/zero mismatches away from f16 midpoints ({rep})"
    assert rep.exempt_flips <= FLIP_BUDGET * rep.n_codes, f"{what}: too many boundary flips ({rep})"
    assert rep.changed_codes <= FLIP_BUDGET * rep.n_codes, f"{what}: too many codes differ from the oracle's ({rep})"
    assert rep.exempt_groups <= max(GROUP_ALLOWANCE, GROUP_BUDGET * rep.n_groups), \
        f"{what}: too many scale/zero midpoint groups ({rep})"


# --------------------------------------------------------------- extend ---


@dataclasses.dataclass
class ExtendInputs:
    """A chunked-prefill batch: the cached prefixes (a decode batch of lengths
    P) and n new rows per sequence at positions P .. P + n - 1."""
    cache: synth.DecodeInputs
    cu: np.ndarray          # int32 [B + 1]
    q: np.ndarray           # bf16 bits [T, H_q, d]
    k_new: np.ndarray       # bf16 bits [T, H_kv, d]
    v_new: np.ndarray

    @property
    def max_new(self) -> int:
        return int(np.diff(self.cu).max()) if len(self.cu) > 1 else 0


def extend_inputs(w: synth.Workload, cache_lens, n_new, seed: int = 0, draw_seqs=None) -> ExtendInputs:
    cache = synth.decode_inputs(w, seq_lens=np.asarray(cache_lens, np.int32), draw_seqs=draw_seqs)
    cu = np.concatenate([[0], np.cumsum(np.asarray(n_new, np.int64))]).astype(np.int32)
    rng = synth.rng_for(w.cfg_id, 100 + seed)
    T = int(cu[-1])
    k, v = synth.kv_rows(rng, T, w)
    q = synth.q_rows(rng, T, w, synth.query_mixers(w))
    return ExtendInputs(cache, cu, q, k, v)


def gpu_extend(ext: ExtendInputs, gc: GpuCache, bits: int = 2, split_steps: int = 0) -> np.ndarray:
    w = ext.cache.w
    B = len(ext.cache.seq_lens)
    T = int(ext.cu[-1])
    max_cache = int(ext.cache.seq_lens.max()) if B else 0
    wsb = lib.extend_workspace_bytes(B, w.n_kv_heads, w.n_q_heads, w.d, w.n_sink, w.n_recent, max_cache,
                                     ext.max_new, split_steps)
    ws = torch.empty(max(1, (wsb + 3) // 4), dtype=torch.int32, device=DEV)
    out = torch.full((T, w.n_q_heads, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lib.paged_extend_attn(gc.cache, bits, bits_to_dev_bf16(ext.q), bits_to_dev_bf16(ext.k_new),
                          bits_to_dev_bf16(ext.v_new), i32(ext.cu), i32(ext.cache.seq_lens), max_cache, ext.max_new,
                          gc.bt_q, gc.bt_h, gc.r_k, gc.r_v, out, ws, split_steps=split_steps)
    torch.cuda.synchronize()
    return dev_bf16_to_f64(out)


def oracle_extend_gpu_pages(ext: ExtendInputs, rot: Rotation, gc: GpuCache, bits: int = 2, seqs=None,
                            rows=None) -> np.ndarray:
    """The oracle's extend attention over the pages the GPU wrote, for the
    sequences ``seqs`` (all by default) and, if given, only the global rows
    ``rows``; other rows stay zero."""
    from oracle import attention as oatt
    w = ext.cache.w
    pool, bf = gpu_pages(ext.cache, gc, bits)
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)  # noqa: E731
    out = np.zeros((int(ext.cu[-1]), w.n_q_heads, w.d))
    for b in (range(len(ext.cache.seq_lens)) if seqs is None else seqs):
        r0, r1 = int(ext.cu[b]), int(ext.cu[b + 1])
        out[r0:r1] = oatt.extend_attention(f(ext.q[r0:r1]), f(ext.k_new[r0:r1]), f(ext.v_new[r0:r1]), pool, bf,
                                           [0, r1 - r0], ext.cache.seq_lens[b:b + 1], ext.cache.bt_q[b:b + 1],
                                           ext.cache.bt_h[b:b + 1], rot.r_k, rot.r_v, w.n_sink, w.n_recent,
                                           rows=None if rows is None else {r - r0 for r in rows if r0 <= r < r1})
    return out


def gpu_decode_int4(inp: synth.DecodeInputs, gc: GpuCache, split_steps: int = 0) -> np.ndarray:
    w = inp.w
    B = len(inp.seq_lens)
    max_len = int(inp.seq_lens.max()) if B else 0
    wsb = lib.decode_int4_workspace_bytes(B, w.n_kv_heads, w.n_q_heads, w.d, w.n_sink, w.n_recent, max_len, split_steps)
    ws = torch.empty(max(1, (wsb + 3) // 4), dtype=torch.int32, device=DEV)
    out = torch.full((B, w.n_q_heads, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lib.paged_decode_attn_int4(gc.cache, bits_to_dev_bf16(inp.q), i32(inp.seq_lens), max_len, gc.bt_q, gc.bt_h, gc.r_k,
                               gc.r_v, out, ws, split_steps=split_steps)
    torch.cuda.synchronize()
    return dev_bf16_to_f64(out)
