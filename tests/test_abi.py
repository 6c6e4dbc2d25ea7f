"""Host-side checks of the C ABI (no GPU needed): every declared symbol is
exported, the cache geometry matches the documented layout and the storage
accounting, and invalid arguments are rejected before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_int4_amd.rq as rq
import oracle as O
from tests.layout_decode import Geom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rq.h")

FAKE = ctypes.c_void_p(1 << 20)        # 256-aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)
ODD = ctypes.c_void_p((1 << 20) + 2)      # not 4-byte aligned


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(rq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = rq.lib()
    for name in _declared():
        assert hasattr(L, name), name


DESCS = [
    rq.make_desc(1, 4, 1, 2, 256, 64),
    rq.make_desc(4, 4, 24, 16, 8192 + 256, 128),
    rq.make_desc(2, 32, 4, 55, 8192 + 256, 96),
    rq.make_desc(2, 4, 3, 5, 300, 128, mode=rq.MODE_DIRECT),
    rq.make_desc(3, 8, 2, 3, 77, 96, anchor_bits=2, residual_bits=4),
    rq.make_desc(1, 4, 2, 2, 100, 64, anchor_bits=4, residual_bits=4, rotation=rq.ROT_NONE),
]


@pytest.mark.parametrize("desc", DESCS, ids=lambda d: f"{d.head_dim}-{d.max_tokens}-{d.mode}")
def test_geometry_matches_documented_layout(desc):
    g = Geom.of(desc)
    assert rq.cache_bytes(desc) == g.total()
    rng = np.random.default_rng(0)
    for _ in range(40):
        kv = int(rng.integers(0, 2))
        b = int(rng.integers(0, desc.batch))
        layer = int(rng.integers(0, desc.layers))
        loop = int(rng.integers(0, desc.loops))
        head = int(rng.integers(0, desc.kv_heads))
        s = rq.cache_slot(desc, kv, b, layer, loop, head)
        off = g.slot_offset(kv, b, layer, loop, head)
        c, z = g.sub_sizes(loop)
        assert s.codes_offset == off and s.codes_offset % 256 == 0
        assert s.sz_offset == off + c
        assert s.alpha_offset == (g.alpha_offset(kv, b, layer, loop, head) if g.has_alpha(loop)
                                  else 2 ** 64 - 1)
        assert s.bits == g.bits(loop)
        assert s.code_bytes == desc.head_dim * s.bits // 8
        assert s.slot_bytes == g.slot_bytes(loop)


@pytest.mark.parametrize("desc", DESCS, ids=lambda d: f"{d.head_dim}-{d.max_tokens}-{d.mode}")
def test_cache_layout_addresses_every_slot(desc):
    """rq_cache_layout's strides and sub-plane offsets, through the formula
    the header states, give every slot rq_cache_slot gives."""
    lay = rq.cache_layout(desc)
    assert lay.total_bytes == rq.cache_bytes(desc)
    P = desc.loops_per_group
    assert lay.token_tile == (32 if desc.head_dim == 64 else 16)
    assert lay.sz_row_bytes == 2 * desc.head_dim // 16
    for kv in range(2):
        for b in range(desc.batch):
            for layer in range(desc.layers):
                for loop in range(desc.loops):
                    for h in range(desc.kv_heads):
                        k, j = divmod(loop, P)
                        kind = 0 if j == P - 1 else 1
                        base = (((kv * desc.batch + b) * desc.layers + layer) * lay.layer_bytes
                                + k * lay.group_bytes)
                        off = base + j * desc.kv_heads * lay.slot_bytes[1] + h * lay.slot_bytes[kind]
                        s = rq.cache_slot(desc, kv, b, layer, loop, h)
                        assert s.codes_offset == off
                        assert s.sz_offset == off + lay.sz_offset[kind]
                        want_alpha = (base + lay.alpha_offset + (j * desc.kv_heads + h)
                                      * lay.alpha_row_bytes) if (kind == 1 and lay.alpha_offset
                                                                 != 2 ** 64 - 1) else 2 ** 64 - 1
                        assert s.alpha_offset == want_alpha
                        assert s.slot_bytes == lay.slot_bytes[kind]
                        assert s.code_bytes == lay.code_row_bytes[kind]


@pytest.mark.parametrize("desc", [DESCS[0], DESCS[3], DESCS[4], DESCS[5],
                                  rq.make_desc(2, 8, 2, 3, 16, 128),
                                  rq.make_desc(1, 4, 1, 16, 16, 96, mode=rq.MODE_CHAINED)],
                         ids=lambda d: f"{d.head_dim}-{d.max_tokens}-{d.mode}-{d.kv_heads}")
def test_cache_planes_tile_the_buffer(desc):
    """Every codes, sz and alpha range of every slot lies inside the buffer
    and no two overlap; alpha rows are only 2 * max_tokens bytes apart, so a
    16-token paged block carries no per-row padding."""
    total = rq.cache_bytes(desc)
    lay = rq.cache_layout(desc)
    n = desc.max_tokens
    ranges = []
    for kv in range(2):
        for b in range(desc.batch):
            for layer in range(desc.layers):
                for loop in range(desc.loops):
                    for h in range(desc.kv_heads):
                        s = rq.cache_slot(desc, kv, b, layer, loop, h)
                        ranges.append((s.codes_offset, s.codes_offset + n * s.code_bytes))
                        ranges.append((s.sz_offset, s.sz_offset + n * lay.sz_row_bytes))
                        if s.alpha_offset != 2 ** 64 - 1:
                            assert s.alpha_offset % 2 == 0
                            ranges.append((s.alpha_offset, s.alpha_offset + 2 * n))
    ranges.sort()
    assert ranges[0][0] >= 0 and ranges[-1][1] <= total
    for (a0, a1), (b0, _) in zip(ranges, ranges[1:]):
        assert a1 <= b0
    if desc.mode != rq.MODE_DIRECT:
        assert lay.alpha_row_bytes == 2 * n


def test_cache_layout_rejects_bad_arguments():
    L = rq.lib()
    bad = rq.make_desc(1, 4, 1, 2, 256, 80)
    assert L.rq_cache_layout(ctypes.byref(bad), ctypes.byref(rq.Layout())) == 2
    good = rq.make_desc(1, 4, 1, 2, 256, 64)
    assert L.rq_cache_layout(ctypes.byref(good), None) == 1


@pytest.mark.parametrize("mode,ab,rb", [(0, 4, 2), (1, 4, 2), (0, 4, 4), (0, 2, 2), (2, 4, 2)])
@pytest.mark.parametrize("d", [64, 96, 128])
def test_cache_bytes_equal_accounting(mode, ab, rb, d):
    """With max_tokens a multiple of 256 nothing is padded, so the buffer holds
    exactly bits_per_element * elements / 8 bytes."""
    desc = rq.make_desc(2, 8, 3, 5, 512, d, anchor_bits=ab, residual_bits=rb, mode=mode)
    elements = 2 * 2 * 8 * 3 * 5 * 512 * d
    bits = O.bits_per_element(ab, rb, 16, d, 4, with_alpha=(mode != 1))
    assert rq.cache_bytes(desc) * 8 == bits * elements


def test_unsupported_descriptors():
    base = dict(batch=1, loops=4, layers=1, kv_heads=2, max_tokens=16, head_dim=64)
    assert rq.validate_desc(rq.make_desc(**base)) == 0
    assert rq.validate_desc(rq.make_desc(**base, mode=2)) == 0
    bad = [dict(head_dim=80), dict(head_dim=256), dict(group_size=32), dict(loops=6),
           dict(anchor_bits=3), dict(residual_bits=8), dict(mode=3), dict(alpha_mode=5),
           dict(rotation=2), dict(loops=128, loops_per_group=4),
           dict(mode=2, loops=8, loops_per_group=8), dict(mode=2, residual_bits=4),
           dict(max_tokens=60_000_000)]
    for kw in bad:
        args = {**base}
        extra = {k: v for k, v in kw.items() if k not in base}
        args.update({k: v for k, v in kw.items() if k in base})
        assert rq.validate_desc(rq.make_desc(**args, **extra)) == 2, kw
    for kw in [dict(batch=0), dict(max_tokens=0), dict(kv_heads=-1)]:
        args = {**base, **kw}
        assert rq.validate_desc(rq.make_desc(**args)) == 1, kw
    assert rq.lib().rq_validate_desc(None) == 1


def test_entry_points_reject_bad_arguments_before_launch():
    L = rq.lib()
    d = rq.make_desc(1, 4, 1, 2, 256, 64)
    D = ctypes.byref(d)
    ws = rq.decode_workspace_bytes(d, 2, 256)
    # quantize_append
    assert L.rq_quantize_append(D, FAKE, FAKE, 200, 100, FAKE, None) == 3
    assert L.rq_quantize_append(D, FAKE, FAKE, -1, 1, FAKE, None) == 1
    assert L.rq_quantize_append(D, None, FAKE, 0, 1, FAKE, None) == 1
    assert L.rq_quantize_append(D, FAKE, FAKE, 0, 1, None, None) == 1       # signs needed
    assert L.rq_quantize_append(D, MISALIGNED, FAKE, 0, 1, FAKE, None) == 5
    assert L.rq_quantize_append(D, FAKE, FAKE, 256, 0, FAKE, None) == 0      # empty append
    # reconstruct
    assert L.rq_reconstruct(D, FAKE, FAKE, 10, 300, 0, FAKE, None) == 3
    assert L.rq_reconstruct(D, FAKE, FAKE, 10, 5, 0, FAKE, None) == 1
    assert L.rq_reconstruct(D, FAKE, FAKE, 0, 4, 7, FAKE, None) == 1
    assert L.rq_reconstruct(D, FAKE, FAKE, 3, 3, 0, FAKE, None) == 0
    # decode attention
    f = ctypes.c_float(0.125)
    assert L.rq_decode_attention(D, FAKE, FAKE, 4, 0, FAKE, 2, 10, f, FAKE, ws, FAKE, None) == 1
    assert L.rq_decode_attention(D, FAKE, FAKE, 0, 1, FAKE, 2, 10, f, FAKE, ws, FAKE, None) == 1
    assert L.rq_decode_attention(D, FAKE, FAKE, 0, 0, FAKE, 3, 10, f, FAKE, ws, FAKE, None) == 2
    assert L.rq_decode_attention(D, FAKE, FAKE, 0, 0, FAKE, 2, 257, f, FAKE, ws, FAKE, None) == 3
    big = rq.make_desc(1, 4, 1, 2, 8192, 64)
    need = rq.decode_workspace_bytes(big, 2, 8192)
    assert need > 0
    assert L.rq_decode_attention(ctypes.byref(big), FAKE, FAKE, 0, 0, FAKE, 2, 8192, f, FAKE,
                                 need - 4, FAKE, None) == 4
    assert L.rq_decode_attention(ctypes.byref(big), FAKE, FAKE, 0, 0, FAKE, 2, 8192, f, None,
                                 need, FAKE, None) == 1
    assert L.rq_decode_attention(D, FAKE, FAKE, 0, 0, FAKE, 2, 256, f, MISALIGNED, ws, FAKE,
                                 None) == 5
    assert L.rq_decode_attention(D, FAKE, None, 0, 0, FAKE, 2, 256, f, FAKE, ws, FAKE, None) == 1
    assert L.rq_decode_attention(D, FAKE, FAKE, 0, 0, FAKE, 2, 256, ctypes.c_float(float("nan")),
                                 FAKE, ws, FAKE, None) == 1
    # ragged variants
    assert L.rq_quantize_append_ragged(D, FAKE, FAKE, None, 1, FAKE, None) == 1
    assert L.rq_quantize_append_ragged(D, FAKE, FAKE, FAKE, 300, FAKE, None) == 3
    assert L.rq_quantize_append_ragged(D, FAKE, FAKE, ODD, 1, FAKE, None) == 5
    assert L.rq_quantize_append_ragged(D, FAKE, FAKE, None, 0, FAKE, None) == 0
    assert L.rq_decode_attention_ragged(D, FAKE, FAKE, 0, 0, FAKE, 2, None, 10, f, FAKE, ws, FAKE,
                                        None) == 1
    assert L.rq_decode_attention_ragged(D, FAKE, FAKE, 0, 0, FAKE, 2, FAKE, 257, f, FAKE, ws, FAKE,
                                        None) == 3
    assert L.rq_decode_attention_ragged(D, FAKE, FAKE, 0, 0, FAKE, 2, ODD, 10, f, FAKE,
                                        ws, FAKE, None) == 5
    # BF16 baseline
    wb = rq.bf16_decode_workspace_bytes(d, 2, 256)
    assert L.rq_bf16_decode_attention(D, FAKE, FAKE, 0, 0, FAKE, 2, 300, f, FAKE, wb, FAKE,
                                      None) == 3
    wbig = rq.bf16_decode_workspace_bytes(big, 2, 8192)
    assert wbig > 0
    assert L.rq_bf16_decode_attention(ctypes.byref(big), FAKE, FAKE, 0, 0, FAKE, 2, 8192, f, FAKE,
                                      8, FAKE, None) == 4
    # probe
    assert L.rq_read_probe(FAKE, 12, FAKE, None) == 1
    assert L.rq_read_probe(MISALIGNED, 16, FAKE, None) == 5


def test_paged_entry_points_reject_bad_arguments_before_launch():
    L = rq.lib()
    f = ctypes.c_float(0.125)
    # block sizes: a power of two, at least one wave tile of the decode kernel
    for bt, d, ok in ((16, 64, False), (32, 64, True), (16, 128, True), (16, 96, True),
                      (48, 128, False), (8, 96, False), (1024, 128, True)):
        p = rq.make_desc(10, 4, 1, 2, bt, d)
        st = L.rq_paged_decode_attention(ctypes.byref(p), FAKE, FAKE, 0, 0, FAKE, 2, 3, FAKE, 8,
                                         FAKE, 8 * bt + 1, f, FAKE, 1 << 40, FAKE, None)
        assert st == (3 if ok else 2), (bt, d)
        st = L.rq_paged_quantize_append(ctypes.byref(p), FAKE, FAKE, 3, FAKE, 8, FAKE,
                                        8 * bt + 1, FAKE, None)
        assert st == (3 if ok else 2), (bt, d)
    # one block's K bytes over all layers must stay under 4 GiB (131072-token
    # blocks of 24 layers: about 11 GB)
    huge = rq.make_desc(2, 4, 24, 16, 1 << 17, 128)
    st = L.rq_paged_decode_attention(ctypes.byref(huge), FAKE, FAKE, 0, 0, FAKE, 16, 1, FAKE, 1,
                                     FAKE, 1 << 17, f, FAKE, 1 << 40, FAKE, None)
    assert st == 2
    assert L.rq_paged_quantize_append(ctypes.byref(huge), FAKE, FAKE, 1, FAKE, 1, FAKE, 1,
                                      FAKE, None) == 2
    pool = rq.make_desc(40, 4, 1, 2, 32, 64)
    P = ctypes.byref(pool)
    ws = rq.paged_decode_workspace_bytes(pool, 2, 3, 256)

    def dec(n_seqs=3, table=FAKE, max_blocks=8, lengths=FAKE, max_n=256, wsb=ws, work=FAKE):
        return L.rq_paged_decode_attention(P, FAKE, FAKE, 0, 0, FAKE, 2, n_seqs, table,
                                           max_blocks, lengths, max_n, f, work, wsb, FAKE, None)

    assert dec(table=None) == 1
    assert dec(n_seqs=0) == 1
    assert dec(max_blocks=0) == 1
    assert dec(lengths=None) == 1
    assert dec(table=ODD) == 5
    assert dec(max_n=257) == 3           # 8 blocks of 32 tokens
    assert dec(max_blocks=1 << 27) == 2  # capacity beyond 2^31 - 1 tokens
    assert dec(max_blocks=(1 << 25) + 1) == 2  # 32-token blocks: 2^30 + 32 tokens
    need = rq.paged_decode_workspace_bytes(pool, 2, 3, 8192)
    assert need > 0
    assert dec(max_blocks=256, max_n=8192, wsb=need - 4) == 4
    assert dec(max_blocks=1 << 25, max_n=8192, wsb=need - 4) == 4  # 2^30 tokens pass capacity
    assert dec(max_blocks=256, max_n=8192, wsb=need, work=None) == 1
    # the workspace is sized by the sequences, not by the pool's block count
    assert rq.paged_decode_workspace_bytes(pool, 2, 3, 8192) == \
        rq.decode_workspace_bytes(rq.make_desc(3, 4, 1, 2, 8192, 64), 2, 8192)

    def app(table=FAKE, positions=FAKE, t_new=1, n_seqs=3, max_blocks=8):
        return L.rq_paged_quantize_append(P, FAKE, FAKE, n_seqs, table, max_blocks, positions,
                                          t_new, FAKE, None)

    assert app(positions=None) == 1
    assert app(positions=None, t_new=0) == 0
    assert app(t_new=0) == 0
    assert app(table=None) == 1
    assert app(n_seqs=0) == 1
    assert app(t_new=257) == 3
    assert app(t_new=-1) == 1
    assert app(positions=ODD) == 5
    assert app(table=ODD) == 5


def test_workspace_bound_is_monotone():
    for d in DESCS:
        for hq in (d.kv_heads, 2 * d.kv_heads):
            prev = 0
            for n in [0, 1, 63, 64, 65, 500, 4096, 8192, 16384]:
                w = rq.decode_workspace_bytes(d, hq, n)
                assert w >= prev
                prev = w


def test_workspace_holds_one_round_of_splits():
    """The split planner fills its target of four-wave workgroups exactly and
    no more (512 at d = 64 and 128, 768 at d = 96): 110 rows at d = 96 take 6
    splits each, and 768 - 660 = 108 of them a seventh.  The workspace is the
    256 KiB counter block plus one partial state (m, l, accA[d], accR[d]) per
    row, head and the largest split count."""
    counters = (1 << 16) * 4
    huginn = rq.make_desc(2, 4, 1, 55, 8192, 96)          # 110 (row, head) pairs
    assert rq.decode_workspace_bytes(huginn, 55, 8192) == counters + 110 * 7 * (2 + 2 * 96) * 4
    ouro = rq.make_desc(4, 4, 1, 16, 8192, 128)            # 64 pairs: 8 splits
    assert rq.decode_workspace_bytes(ouro, 16, 8192) == counters + 64 * 8 * (2 + 2 * 128) * 4
    # short contexts: at most half the 64-token tiles, and no workspace for one split
    assert rq.decode_workspace_bytes(ouro, 16, 256) == counters + 64 * 2 * (2 + 2 * 128) * 4
    assert rq.decode_workspace_bytes(ouro, 16, 127) == 0


def test_workspace_covers_every_split_plan():
    """For every call a descriptor admits, the workspace bound holds the
    partial states of the split plan the call runs (the entry points refuse
    a plan past it rather than write beyond the buffer)."""
    counters = (1 << 16) * 4
    for d in (64, 96, 128):
        for batch, kvh, ratio in ((1, 1, 1), (1, 4, 1), (2, 55, 1), (3, 16, 1), (4, 16, 1),
                                  (16, 4, 4), (1, 2, 8), (9, 7, 2), (64, 16, 1)):
            for mode in (rq.MODE_RESIDUAL, rq.MODE_DIRECT, rq.MODE_CHAINED):
                desc = rq.make_desc(batch, 4, 1, kvh, 65536, d, mode=mode)
                hq = kvh * ratio
                for n in (0, 1, 100, 257, 1000, 4097, 8192, 30000, 65536):
                    ws = rq.decode_workspace_bytes(desc, hq, n)
                    for loop in range(4):
                        s = rq.decode_splits(desc, loop, hq, n)
                        assert s >= 1
                        if s > 1:
                            assert ws >= counters + batch * hq * s * (2 + 2 * d) * 4, \
                                (d, batch, kvh, ratio, mode, n, loop, s, ws)


def test_split_plan_fits_one_round():
    """The split count the library reports for a call (the largest of any
    row): eight-wave calls (d = 128, at most one residual plane, paged anchors
    aside) aim at 256 workgroups, four-wave ones at 512 (d = 96 calls at 768;
    110 rows: 6 splits, 7 for the 108 rows that fill the target),
    grouped-query calls count (row, KV head) pairs, and no split is shorter
    than two tiles."""
    huginn = rq.make_desc(2, 4, 1, 55, 8192, 96)          # 110 (row, head) pairs, four waves
    assert rq.decode_splits(huginn, 0, 55, 8192) == 7     # 768-workgroup target at d = 96
    assert rq.decode_splits(huginn, 3, 55, 8192) == 7     # the anchor loop too
    h64 = rq.make_desc(2, 4, 1, 64, 8192, 96)             # 128 rows divide 768: no seventh split
    assert rq.decode_splits(h64, 0, 64, 8192) == 6
    short = rq.make_desc(2, 4, 1, 55, 768, 96)            # 12 tiles of 64: at most 6 splits
    assert rq.decode_splits(short, 0, 55, 768) == 6
    ouro = rq.make_desc(4, 4, 1, 16, 8192, 128)            # 64 pairs, eight waves
    assert rq.decode_splits(ouro, 0, 16, 8192) == 4
    assert rq.decode_splits(ouro, 3, 16, 8192) == 4       # the anchor loop
    assert rq.decode_splits(ouro, 0, 16, 256) == 1        # two 128-token tiles: one split
    assert rq.decode_splits(ouro, 0, 16, 0) == 1
    chained = rq.make_desc(4, 4, 1, 16, 8192, 128, mode=rq.MODE_CHAINED)
    assert rq.decode_splits(chained, 0, 16, 8192) == 8    # three residual planes: four waves
    gqa = rq.make_desc(16, 4, 1, 4, 8192, 128)             # 64 (row, KV head) pairs, 4 heads each
    assert rq.decode_splits(gqa, 0, 16, 8192) == 4
    assert rq.decode_splits(ouro, 4, 16, 8192) == 0       # no such loop
    assert rq.decode_splits(ouro, 0, 12, 8192) == 0       # 12 query heads on 16 KV heads


def test_status_strings():
    for s in range(7):
        assert rq._status_string(s)
    assert rq._status_string(99) == "unknown status"
