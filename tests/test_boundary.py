"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any device
work (every call below fails validation, so nothing is ever launched and the
fake pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import vector_quantized_bit_amd as vq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "vqkv.h")

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE, HIP = range(6)
A = 0x100000          # a fake, 16-byte aligned device address (never touched)
MIS = 0x100004        # a fake misaligned address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vq.LIB_PATH):
        pytest.fail("libvqkv.so is not built (run python -m vector_quantized_bit_amd.build)")
    return vq.library()


def lay(k_bits=8, v_bits=8, hkv=2, cap=1000, head_dim=128, sub_dim=4):
    return vq.Layout(head_dim, sub_dim, k_bits, v_bits, hkv, cap)


def test_header_functions_are_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    raw = ctypes.CDLL(vq.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    for st in range(6):
        assert vq.status_string(st)
    assert vq.status_string(OK) == "ok"
    assert "unknown" in vq.status_string(99)


def attn(lib, layout, q=A, q_dtype=0, lam=A, cbk=A, cbv=A, ck=A, cv=A, batch=1, hq=4, n=100,
         splits=0, out=A, ws=A, ws_bytes=1 << 30):
    return lib.vq_decode_attention(ctypes.byref(layout) if layout is not None else None, q,
                                   q_dtype, lam, cbk, cbv, ck, cv, batch, hq, n, splits, out, ws,
                                   ws_bytes, None)


@pytest.mark.parametrize("kw,layout_kw,status,needle", [
    (dict(), dict(head_dim=64), UNSUPPORTED, "head_dim"),
    (dict(), dict(sub_dim=8), UNSUPPORTED, "sub_dim"),
    (dict(), dict(sub_dim=8, k_bits=12, v_bits=8), UNSUPPORTED, "sub_dim"),
    (dict(), dict(sub_dim=6), UNSUPPORTED, "sub_dim"),
    (dict(q=None), dict(sub_dim=8, k_bits=12, v_bits=12), INVALID, "q is NULL"),
    (dict(), dict(k_bits=10), UNSUPPORTED, "k_code_bits"),
    (dict(), dict(v_bits=12), UNSUPPORTED, "v_code_bits"),
    (dict(), dict(hkv=0), INVALID, "num_kv_heads"),
    (dict(), dict(cap=0), INVALID, "capacity"),
    (dict(hq=3), dict(), INVALID, "multiple"),
    (dict(hq=18), dict(), UNSUPPORTED, "group"),
    (dict(batch=0), dict(), INVALID, "batch"),
    (dict(n=0), dict(), INVALID, "context_len"),
    (dict(n=1001), dict(), CAPACITY, "capacity"),
    (dict(q_dtype=7), dict(), INVALID, "q_dtype"),
    (dict(splits=-1), dict(), INVALID, "num_splits"),
    (dict(q=None), dict(), INVALID, "q is NULL"),
    (dict(lam=MIS), dict(), INVALID, "lambda"),
    (dict(ck=None), dict(), INVALID, "codes_k"),
    (dict(cv=MIS), dict(), INVALID, "codes_v"),
    (dict(cbk=None), dict(), INVALID, "cb_k"),
    (dict(out=MIS), dict(), INVALID, "out"),
    (dict(ws=None), dict(), WORKSPACE, "workspace"),
    (dict(ws_bytes=16), dict(), WORKSPACE, "workspace"),
    (dict(ws=MIS), dict(), INVALID, "workspace"),
])
def test_decode_attention_validation(lib, kw, layout_kw, status, needle):
    st = attn(lib, lay(**layout_kw), **kw)
    assert st == status, vq._last_error()
    assert needle in vq._last_error()


def test_decode_attention_null_layout(lib):
    assert attn(lib, None) == INVALID


def test_workspace_query_matches_partials_layout(lib):
    layout = lay(hkv=8, cap=196608)
    s = lib.vq_decode_attention_default_splits(ctypes.byref(layout), 1, 32, 196608)
    assert s >= 1
    need = lib.vq_decode_attention_workspace_bytes(ctypes.byref(layout), 1, 32, 196608, 0)

    def a256(x):
        return (x + 255) // 256 * 256

    n = 1 * 32 * s
    assert need == 2 * a256(4 * n) + a256(4 * 128 * n)
    # explicit split requests are clamped so that no split is empty
    # (splits are whole sweeps of 512 tokens: 1100 tokens allow at most 3)
    one = lib.vq_decode_attention_workspace_bytes(ctypes.byref(layout), 1, 32, 1100, 10 ** 6)
    n = 32 * 3
    assert one == 2 * a256(4 * n) + a256(4 * 128 * n)
    assert lib.vq_decode_attention_workspace_bytes(None, 1, 32, 100, 0) == 0


def encode(lib, layout, k=A, v=A, dtype=0, lam=A, cbk=A, cbv=A, ck=A, cv=A, batch=1, cur=0, new=1):
    return lib.vq_encode_append(ctypes.byref(layout), k, v, dtype, lam, cbk, cbv, ck, cv, batch,
                                cur, new, None)


@pytest.mark.parametrize("kw,layout_kw,status", [
    (dict(cur=1000, new=1), dict(), CAPACITY),
    (dict(cur=990, new=11), dict(), CAPACITY),
    (dict(cur=-1), dict(), INVALID),
    (dict(new=-1), dict(), INVALID),
    (dict(batch=0), dict(), INVALID),
    (dict(dtype=3), dict(), INVALID),
    (dict(k=None), dict(), INVALID),
    (dict(cbv=MIS), dict(), INVALID),
    (dict(), dict(k_bits=4), UNSUPPORTED),
])
def test_encode_append_validation(lib, kw, layout_kw, status):
    assert encode(lib, lay(**layout_kw), **kw) == status, vq._last_error()


def test_encode_append_zero_tokens_is_a_no_op(lib):
    # validated, then returns before any device work
    assert encode(lib, lay(), new=0) == OK
    assert vq._last_error() == ""


def test_transform_query_validation(lib):
    layout = lay(hkv=2)
    f = lib.vq_transform_query
    assert f(ctypes.byref(layout), None, 0, A, 1, 4, A, None) == INVALID
    assert f(ctypes.byref(layout), A, 0, A, 1, 5, A, None) == INVALID
    assert f(ctypes.byref(layout), A, 2, A, 1, 4, A, None) == INVALID
    assert f(ctypes.byref(layout), A, 0, A, 1, 4, MIS, None) == INVALID


def test_fp16_attention_validation(lib):
    f = lib.vq_fp16_decode_attention
    big = 1 << 30
    assert f(A, A, A, 1, 4, 0, 10, 5, 0, A, A, big, None) == INVALID       # num_kv_heads
    assert f(A, A, A, 1, 4, 1, 10, 11, 0, A, A, big, None) == CAPACITY
    assert f(A, A, A, 1, 4, 1, 10, 0, 0, A, A, big, None) == INVALID
    assert f(A, A, A, 1, 36, 4, 10, 5, 0, A, A, big, None) == UNSUPPORTED  # G = 9
    assert f(None, A, A, 1, 4, 1, 10, 5, 0, A, A, big, None) == INVALID
    assert f(A, A, A, 1, 4, 1, 10, 5, 0, A, A, 8, None) == WORKSPACE
    need = lib.vq_fp16_attention_workspace_bytes(1, 4, 1, 10, 0)
    assert need > 0


def test_plan_splits_is_a_fixed_point(lib):
    layout = lay(hkv=8, cap=196608)
    plan = lib.vq_decode_attention_plan_splits
    default = plan(ctypes.byref(layout), 1, 32, 196608, 0)
    assert default == lib.vq_decode_attention_default_splits(ctypes.byref(layout), 1, 32, 196608)
    for req in (0, 1, 3, 7, 32, 100, 10 ** 6):
        s = plan(ctypes.byref(layout), 1, 32, 196608, req)
        assert 1 <= s <= 384          # 196608 tokens hold 384 sweeps of 512
        assert plan(ctypes.byref(layout), 1, 32, 196608, s) == s
    assert plan(ctypes.byref(layout), 1, 32, 1100, 10 ** 6) == 3
    assert plan(None, 1, 32, 100, 0) == 0
    assert plan(ctypes.byref(layout), 1, 32, 0, 0) == 0
    assert plan(ctypes.byref(layout), 1, 32, 100, -1) == 0


def test_split_plan_keeps_each_split_under_2gib_of_codes(lib):
    # a split's code rows are addressed through a 32-bit byte range: an
    # explicit request of one split over 100 M tokens of 48-byte rows is
    # raised (here to the merge's 512 partials, by the split-length cap)
    layout = lay(k_bits=12, hkv=1, cap=100_000_000)
    s = lib.vq_decode_attention_plan_splits(ctypes.byref(layout), 1, 4, 100_000_000, 1)
    assert s == 512
    assert (100_000_000 + s - 1) // s * 48 < 2 ** 31
    assert lib.vq_decode_attention_plan_splits(ctypes.byref(layout), 1, 4, 100_000_000, s) == s
    # the default plan is far below the bound
    d = lib.vq_decode_attention_plan_splits(ctypes.byref(layout), 1, 4, 100_000_000, 0)
    assert (100_000_000 + d - 1) // d * 48 < 2 ** 31


@pytest.mark.parametrize("n,req,expect", [
    (24576, 1, 1),            # one split of 24576 tokens is the longest allowed
    (24577, 1, 2),
    (65536, 1, 3),            # requests of fewer splits are raised to splits of <= 24576
    (196608, 1, 8),
    (196608, 0, 256),         # the default (256 workgroups) is unaffected
    (512 * 24576, 1, 512),
    (512 * 24576 + 32, 1, 512),   # beyond 512 x 24576 tokens the splits grow instead
])
def test_split_plan_caps_the_split_length(lib, n, req, expect):
    """Waves accumulate their tiles' value products in fp32; behind a dominant
    token the rounding of many small contributions grows with the tiles per
    wave, so the planner keeps splits at 24576 tokens or fewer while the 512
    splits the merge takes allow it."""
    layout = lay(hkv=1, cap=n)
    s = lib.vq_decode_attention_plan_splits(ctypes.byref(layout), 1, 4, n, req)
    assert s == expect
    per = -(-n // s)
    assert per <= 24576 or s == 512
    m = lib.vq_decode_step_num_partials(ctypes.byref(layout), 1, 4, n - 1, req)
    assert -(-(n - 1) // (m - 1)) <= 24576 or m - 1 == 512


def test_split_plans_near_the_int32_limit(lib):
    # contexts up to 2^31 - 1 tokens plan without overflow: every split count
    # is positive, within the 512 the merge takes, and keeps splits under
    # 2^31 bytes of 48-byte rows
    n = 2 ** 31 - 10
    for k_bits in (8, 12):
        layout = lay(k_bits=k_bits, hkv=8, cap=2 ** 31 - 1)
        for bsz, req in ((1, 0), (8, 0), (8, 1), (32, 0)):
            for f in (lib.vq_decode_step_num_partials, lib.vq_decode_step_window_num_partials):
                m = f(ctypes.byref(layout), bsz, 32, n, req)
                assert 2 <= m <= 513, (f, bsz, req, m)
                assert -(-n // (m - 1)) * 48 < 2 ** 31
            s = lib.vq_decode_attention_plan_splits(ctypes.byref(layout), bsz, 32, n, req)
            assert 1 <= s <= 512 and -(-n // s) * 48 < 2 ** 31


def test_plan_queries_with_huge_stream_counts(lib):
    # batch x KV heads beyond the int32 range: the plan queries stay defined
    # (one split), and a launch with such a shape is refused before any work
    layout = lay(hkv=8, cap=1000)
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 2 ** 30, 32, 999, 0) == 2
    assert lib.vq_decode_attention_plan_splits(ctypes.byref(layout), 2 ** 30, 32, 999, 0) == 1
    assert attn(lib, layout, batch=2 ** 30, hq=32, n=999) == INVALID


def partials(lib, layout, splits=1, n=100, pm=A, pl=A, po=A, **kw):
    args = dict(q=A, q_dtype=0, lam=A, cbk=A, cbv=A, ck=A, cv=A, batch=1, hq=4)
    args.update(kw)
    return lib.vq_decode_attention_partials(
        ctypes.byref(layout), args["q"], args["q_dtype"], args["lam"], args["cbk"], args["cbv"],
        args["ck"], args["cv"], args["batch"], args["hq"], n, splits, pm, pl, po, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(splits=2), INVALID, "planned"),        # 100 tokens allow one split only
    (dict(splits=-1), INVALID, "num_splits"),
    (dict(pm=None), INVALID, "part_m"),
    (dict(pl=MIS), INVALID, "part_l"),
    (dict(po=None), INVALID, "part_o"),
    (dict(n=0), INVALID, "context_len"),
    (dict(n=1001), CAPACITY, "capacity"),
    (dict(hq=3), INVALID, "multiple"),
    (dict(ck=None), INVALID, "codes_k"),
])
def test_partials_validation(lib, kw, status, needle):
    assert partials(lib, lay(hkv=2), **kw) == status, vq._last_error()
    assert needle in vq._last_error()


@pytest.mark.parametrize("args,status,needle", [
    ((0, 4, 2, A, A, A, A), INVALID, "batch"),
    ((1, 0, 2, A, A, A, A), INVALID, "num_q_heads"),
    ((1, 4, 0, A, A, A, A), INVALID, "num_partials"),
    ((1, 4, 513, A, A, A, A), INVALID, "num_partials"),
    ((1, 4, 2, None, A, A, A), INVALID, "part_m"),
    ((1, 4, 2, A, A, MIS, A), INVALID, "part_o"),
    ((1, 4, 2, A, A, A, None), INVALID, "out"),
])
def test_merge_validation(lib, args, status, needle):
    assert lib.vq_merge_partials(*args, None) == status, vq._last_error()
    assert needle in vq._last_error()


def step(lib, layout, cur=10, splits=0, kv_dtype=0, kn=A, vn=A, ws=A, ws_bytes=1 << 30, out=A,
         hq=4):
    return lib.vq_decode_step(ctypes.byref(layout), A, 0, kn, vn, kv_dtype, A, A, A, A, A, 1, hq,
                              cur, splits, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cur=1000), CAPACITY, "capacity"),        # slot 1000 of a 1000-slot cache
    (dict(cur=-1), INVALID, "cur_len"),
    (dict(kv_dtype=5), INVALID, "kv_dtype"),
    (dict(kn=None), INVALID, "k_new"),
    (dict(vn=MIS), INVALID, "v_new"),
    (dict(out=None), INVALID, "out"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=8), WORKSPACE, "workspace"),
    (dict(hq=3), INVALID, "multiple"),
])
def test_decode_step_validation(lib, kw, status, needle):
    assert step(lib, lay(hkv=2), **kw) == status, vq._last_error()
    assert needle in vq._last_error()


def step_noalloc(lib, layout, cur=10, splits=0, kv_dtype=0, kn=A, vn=A, out=A, hq=4, batch=1):
    return lib.vq_decode_step_noalloc(ctypes.byref(layout), A, 0, kn, vn, kv_dtype, A, A, A, A, A,
                                      batch, hq, cur, splits, out, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cur=1000), CAPACITY, "capacity"),
    (dict(cur=-1), INVALID, "cur_len"),
    (dict(kv_dtype=5), INVALID, "kv_dtype"),
    (dict(kn=None), INVALID, "k_new"),
    (dict(vn=MIS), INVALID, "v_new"),
    (dict(out=None), INVALID, "out"),
    (dict(hq=3), INVALID, "multiple"),
])
def test_decode_step_noalloc_validation(lib, kw, status, needle):
    assert step_noalloc(lib, lay(hkv=2), **kw) == status, vq._last_error()
    assert needle in vq._last_error()


def test_decode_step_noalloc_rejects_partials_beyond_its_buffer(lib):
    """256 sequences x 32 query heads need 8.5 MB of partials, more than the
    4 MiB static buffer: rejected on the host, before any device call."""
    layout = lay(hkv=8, cap=1001)
    need = lib.vq_decode_step_workspace_bytes(ctypes.byref(layout), 256, 32, 1000, 0)
    assert need > vq.NOALLOC_SCRATCH_BYTES
    assert step_noalloc(lib, layout, cur=1000, hq=32, batch=256) == WORKSPACE
    assert "static buffer" in vq._last_error()
    # the largest batch that fits is accepted by the same size rule
    per_seq = lib.vq_decode_step_workspace_bytes(ctypes.byref(layout), 1, 32, 1000, 0)
    assert per_seq <= vq.NOALLOC_SCRATCH_BYTES


def test_noalloc_buffer_size_matches_the_header(lib):
    text = open(HEADER).read()
    m = re.search(r"#define VQ_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == vq.NOALLOC_SCRATCH_BYTES


def test_decode_step_partials_validation(lib):
    f = lib.vq_decode_step_partials
    layout = lay(hkv=2)
    # 10 cached tokens allow one split: 2 partials, nothing else
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 1, 4, 10, 0) == 2
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 1, 4, 10, 5) == 2
    assert f(ctypes.byref(layout), A, 0, A, A, 0, A, A, A, A, A, 1, 4, 10, 3, A, A, A,
             None) == INVALID
    assert "planned" in vq._last_error()
    assert f(ctypes.byref(layout), A, 0, A, A, 0, A, A, A, A, A, 1, 4, 999, 2, A, None, A,
             None) == INVALID
    assert "part_l" in vq._last_error()


def test_decode_step_plan_folds_or_leaves_room_for_the_new_token(lib):
    layout = lay(hkv=8, cap=196609)
    n = lib.vq_decode_step_num_partials(ctypes.byref(layout), 1, 32, 196608, 0)
    assert n == 32                                   # 31 splits x 8 heads + 8 = 256 workgroups
    need = lib.vq_decode_step_workspace_bytes(ctypes.byref(layout), 1, 32, 196608, 0)

    def a256(x):
        return (x + 255) // 256 * 256

    assert need == 2 * a256(4 * 32 * n) + a256(4 * 128 * 32 * n)
    # the first token of a sequence: no cached tokens, one empty split
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 1, 32, 0, 0) == 2
    # 128 streams (16 sequences x 8 heads): two splits each fill the 256 CUs,
    # the new token folded into the last
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 16, 32, 32767, 0) == 3
    # 64 streams: four splits each, folded
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 8, 32, 65535, 0) == 5
    big = lay(k_bits=12, hkv=8, cap=65600)
    assert lib.vq_decode_step_num_partials(ctypes.byref(big), 8, 40, 65535, 0) == 5
    # 32 streams of short contexts do not fold: 4096 tokens give 8 sweeps of
    # 512 (beside 32 new-token workgroups)
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 4, 32, 4096, 0) == 8
    # an explicit split count is a fixed point, folded or not
    for bsz, cur, req in ((1, 196608, 7), (1, 196608, 32), (4, 4096, 3), (8, 65535, 4),
                          (16, 32767, 1)):
        m = lib.vq_decode_step_num_partials(ctypes.byref(layout), bsz, 32, cur, req)
        assert lib.vq_decode_step_num_partials(ctypes.byref(layout), bsz, 32, cur, m - 1) == m


def wstep(lib, layout, codes=10, wlen=0, wcap=128, splits=0, kv_dtype=0, kn=A, vn=A, wk=A, wv=A,
          ws=A, ws_bytes=1 << 30, out=A, hq=4):
    return lib.vq_decode_step_window(ctypes.byref(layout), A, 0, kn, vn, kv_dtype, A, A, A, A, A,
                                     wk, wv, wcap, 1, hq, codes, wlen, splits, out, ws, ws_bytes,
                                     None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(wlen=128), CAPACITY, "window full"),     # no free slot: flush first
    (dict(wlen=-1), INVALID, "win_len"),
    (dict(wcap=0), INVALID, "window capacity"),
    (dict(codes=1001), CAPACITY, "num_codes"),
    (dict(codes=-1), INVALID, "num_codes"),
    (dict(wk=None), INVALID, "win_k"),
    (dict(wv=MIS), INVALID, "win_v"),
    (dict(kn=None), INVALID, "k_new"),
    (dict(kv_dtype=7), INVALID, "kv_dtype"),
    (dict(out=None), INVALID, "out"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=8), WORKSPACE, "workspace"),
    (dict(hq=3), INVALID, "multiple"),
])
def test_decode_step_window_validation(lib, kw, status, needle):
    assert wstep(lib, lay(hkv=2), **kw) == status, vq._last_error()
    assert needle in vq._last_error()


def test_decode_step_window_plan(lib):
    layout = lay(hkv=8, cap=196608)
    np_ = lib.vq_decode_step_window_num_partials
    # coded tokens split as in a decode step, plus the window's partial
    assert np_(ctypes.byref(layout), 1, 32, 196608, 0) == \
        lib.vq_decode_step_num_partials(ctypes.byref(layout), 1, 32, 196608, 0) == 32
    # 64 streams: a decode step folds its new token and a window step its
    # window (four splits per stream over all 256 CUs, plus that partial)
    assert np_(ctypes.byref(layout), 8, 32, 65535, 0) == 5
    assert lib.vq_decode_step_num_partials(ctypes.byref(layout), 8, 32, 65535, 0) == 5
    # 32 streams: the window workgroups run beside 224 split workgroups
    assert np_(ctypes.byref(layout), 4, 32, 65535, 0) == 8
    # 128 streams: two splits per stream either way (folded window)
    assert np_(ctypes.byref(layout), 16, 32, 32767, 0) == 3
    # no coded tokens: the window workgroup alone, one partial
    assert np_(ctypes.byref(layout), 1, 32, 0, 0) == 1
    assert np_(ctypes.byref(layout), 1, 32, -1, 0) == 0
    need = lib.vq_decode_step_window_workspace_bytes(ctypes.byref(layout), 1, 32, 0, 0)
    assert need == 2 * 256 + 4 * 128 * 32          # m, l (256-byte aligned) and o of 32 heads
    # a window-only step with too small a workspace is refused before any launch
    small = lib.vq_decode_step_window_workspace_bytes(ctypes.byref(lay(hkv=2)), 1, 4, 0, 0)
    assert wstep(lib, lay(hkv=2), codes=0, ws_bytes=small - 1) == WORKSPACE


def test_flush_window_validation(lib):
    layout = lay(hkv=2, cap=1000)
    f = lib.vq_flush_window
    assert f(ctypes.byref(layout), A, A, A, A, A, A, A, 0, 1, 0, None) == INVALID
    assert "window capacity" in vq._last_error()
    assert f(ctypes.byref(layout), A, A, A, A, A, A, A, 128, 1, 900, None) == CAPACITY
    assert f(ctypes.byref(layout), None, A, A, A, A, A, A, 128, 1, 0, None) == INVALID
    assert f(ctypes.byref(layout), A, A, A, A, A, A, A, 128, 1, -1, None) == INVALID


# --- offline calibration -----------------------------------------------------------

@pytest.mark.parametrize("args,status,needle", [
    ((A, 2, 8, 100, A), INVALID, "kv_dtype"),
    ((A, 0, 0, 100, A), INVALID, "num_kv_heads"),
    ((A, 0, 65536, 100, A), INVALID, "num_kv_heads"),
    ((A, 1, 8, 0, A), INVALID, "num_tokens"),
    ((None, 0, 8, 100, A), INVALID, "keys is NULL"),
    ((MIS, 0, 8, 100, A), INVALID, "keys"),
    ((A, 0, 8, 100, None), INVALID, "lambda"),
    ((A, 0, 8, 100, MIS), INVALID, "lambda"),
])
def test_calibrate_lambda_validation(lib, args, status, needle):
    assert lib.vq_calibrate_lambda(*args, None) == status, vq._last_error()
    assert needle in vq._last_error()


@pytest.mark.parametrize("args,status,needle", [
    ((A, 0, None, 8, 100, A), INVALID, "lambda"),
    ((A, 0, A, 8, 100, MIS), INVALID, "keys_tilde"),
    ((A, 0, A, 8, -5, A), INVALID, "num_tokens"),
    ((A, 5, A, 8, 100, A), INVALID, "kv_dtype"),
])
def test_transform_keys_validation(lib, args, status, needle):
    assert lib.vq_transform_keys(*args, None) == status, vq._last_error()
    assert needle in vq._last_error()


def kmeans_call(lib, samples=A, sets=2, n=1000, bits=8, init=A, iters=3, cent=A, cb=A, asg=A,
                ws=A, ws_bytes=1 << 30, sub=4):
    return lib.vq_kmeans(samples, sets, n, sub, bits, init, iters, cent, cb, asg, ws, ws_bytes,
                         None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(sets=0), INVALID, "num_sets"),
    (dict(sets=65536), INVALID, "num_sets"),
    (dict(n=0), INVALID, "num_samples"),
    (dict(n=(1 << 28) + 1), INVALID, "num_samples"),
    (dict(bits=10), UNSUPPORTED, "code_bits"),
    (dict(sub=6), UNSUPPORTED, "sub_dim"),
    (dict(iters=-1), INVALID, "iters"),
    (dict(iters=10001), INVALID, "iters"),
    (dict(samples=None), INVALID, "samples"),
    (dict(init=MIS), INVALID, "init"),
    (dict(cent=None), INVALID, "centroids"),
    (dict(cb=MIS), INVALID, "codebook"),
    (dict(asg=MIS), INVALID, "assign"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=4096), WORKSPACE, "workspace"),
    (dict(ws=MIS), INVALID, "workspace"),
])
def test_kmeans_validation(lib, kw, status, needle):
    assert kmeans_call(lib, **kw) == status, vq._last_error()
    assert needle in vq._last_error()


def test_kmeans_workspace_layout(lib):
    def a256(x):
        return (x + 255) // 256 * 256

    for sets, n, sub, bits in ((1, 1, 4, 8), (8, 4194304, 4, 8), (3, 8193, 4, 12),
                               (8, 2097152, 8, 12), (2, 100, 8, 8)):
        ent, chunks = 1 << bits, -(-n // 8192)
        want = (a256(sets * n * 4) + a256(sets * chunks * ent * 4) + 2 * a256(sets * ent * 4) +
                a256(sets * n * 4 * sub))
        assert lib.vq_kmeans_workspace_bytes(sets, n, sub, bits) == want
    for bad in ((0, 10, 4, 8), (1, 0, 4, 8), (1, 10, 4, 9), (1, (1 << 28) + 1, 4, 8),
                (1, 10, 5, 8)):
        assert lib.vq_kmeans_workspace_bytes(*bad) == 0


def _visible_gpus(lib):
    n = ctypes.c_int(0)
    rc = lib.hipGetDeviceCount(ctypes.byref(n))
    return n.value if rc == 0 else 0


def test_runtime_errors_come_back_as_vq_err_hip(lib):
    """A call that passes validation but cannot launch reports VQ_ERR_HIP with
    the runtime's message.  Forced here by the missing device: this test runs
    only where the HIP runtime sees no GPU (it would otherwise launch kernels
    on the fake addresses)."""
    if _visible_gpus(lib) > 0:
        pytest.skip("a GPU is visible: the calls below would launch")
    assert lib.vq_merge_partials(1, 4, 2, A, A, A, A, None) == HIP
    assert "merge_partials launch" in vq._last_error()
    layout = lay(hkv=1, cap=100)
    assert lib.vq_transform_query(ctypes.byref(layout), A, 0, A, 1, 4, A, None) == HIP
    assert "device" in vq._last_error()
    assert attn(lib, layout, n=100) == HIP
    assert vq.status_string(HIP) == "HIP runtime error"
    # a later call that fails validation reports its own error, not the old one
    assert attn(lib, layout, n=0) == INVALID and "context_len" in vq._last_error()
