"""C ABI checks that need no GPU: the library loads, exports every entry point
include/dsa.h declares, sizes workspaces, and rejects bad arguments before it
touches the device (so on a machine without a GPU a fully valid call reports
DSA_ERR_NO_DEVICE and nothing else)."""
import ctypes
import os
import re

import pytest

import torch

import sparse_attention_amd as m

# A fully valid call with the fake pointers below would launch kernels on a
# real device, so those calls are made only where no GPU is present.
HAS_GPU = torch.cuda.is_available()

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dsa.h")

OK, INVALID, MISALIGNED, WS_SMALL, NO_DEVICE, HIP = range(6)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.library_path()):
        from sparse_attention_amd.build import build_library
        build_library()
    return m.load_library()


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DSA_API\s+[\w\s\*]+?\b(dsa_\w+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert header_symbols() == sorted(m.exported_symbols())


def test_library_exports_every_declared_symbol(lib):
    for name in header_symbols():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in m.STATUS_NAMES.items():
        assert lib.dsa_status_string(code).decode() == name
    assert lib.dsa_status_string(99).decode() == "DSA_ERR_UNKNOWN_STATUS"


def test_workspace_sizes(lib):
    assert m.dsa_topk_workspace_size(0, 10, 2048) == 0
    assert m.dsa_sparse_mla_workspace_size(1, 0) == 0
    assert m.dsa_decode_step_workspace_size(1, 1, 2049) == 0
    # rows of up to 65,536 positions (one workgroup per row) need no top-k
    # workspace; few rows of up to 262,144 positions hold a 16-byte record and
    # 4,096 candidate slots per 4,096-position chunk
    assert m.dsa_topk_workspace_size(300, 32768, 2048) == 0
    assert m.dsa_topk_workspace_size(64, 32768, 2048) == 0
    assert m.dsa_topk_workspace_size(16, 202752, 2048) == 16 * 50 * 16 + 16 * 50 * 4096 * 8
    a = m.dsa_topk_workspace_size(16, 300000, 2048)
    b = m.dsa_topk_workspace_size(32, 300000, 2048)
    assert 0 < a < b and a % 256 == 0
    # decode-step workspace holds the fp32 scores of every row
    d = m.dsa_decode_step_workspace_size(64, 32768, 2048)
    assert d >= 64 * 32768 * 4 + m.dsa_topk_workspace_size(64, 32768, 2048)
    d = m.dsa_decode_step_workspace_size(4, 300000, 2048)
    assert d >= 4 * 300000 * 4 + m.dsa_topk_workspace_size(4, 300000, 2048)
    # many rows need no split partials
    assert m.dsa_sparse_mla_workspace_size(8192, 2048) == 0
    assert m.dsa_sparse_mla_workspace_size(16, 2048) > 0


def _rows(R=4, maxv=100, vis=0x10000, base=0x20000, flags=0):
    return m._CRows(R, maxv, vis, base, flags)


def _call_topk(lib, rows, scores=0x1000, ld=100, k=2048, idx=0x3000, ws=0x100000, ws_bytes=1 << 30):
    return lib.dsa_topk_select(ctypes.byref(rows) if rows is not None else None, scores, ld, k, idx, ws, ws_bytes,
                               None)


@pytest.mark.parametrize("case, expect", [
    (dict(rows=None), INVALID),
    (dict(rows=_rows(R=0)), INVALID),
    (dict(rows=_rows(maxv=0)), INVALID),
    (dict(rows=_rows(maxv=(1 << 24) + 1)), INVALID),
    (dict(rows=_rows(vis=0)), INVALID),
    (dict(rows=_rows(base=0)), INVALID),
    (dict(rows=_rows(base=0x20004)), MISALIGNED),
    (dict(rows=_rows(flags=2)), INVALID),
    (dict(scores=0), INVALID),
    (dict(scores=0x1004), MISALIGNED),
    (dict(ld=99), INVALID),
    (dict(ld=102, rows=_rows(maxv=100)), MISALIGNED),
    (dict(k=0), INVALID),
    (dict(k=2049), INVALID),
    (dict(idx=0), INVALID),
    (dict(idx=0x3002), MISALIGNED),
    # rows longer than 65,536 positions need a workspace
    (dict(ws_bytes=16, rows=_rows(maxv=300000), ld=300000), WS_SMALL),
    (dict(ws=0, rows=_rows(maxv=300000), ld=300000), INVALID),
    (dict(ws=0x100010, rows=_rows(maxv=300000), ld=300000), MISALIGNED),
    (dict(ws=0, ws_bytes=0), NO_DEVICE),  # no workspace needed for short rows
    (dict(), NO_DEVICE),
])
def test_topk_validation(lib, case, expect):
    case = dict(case)
    rows = case.pop("rows", _rows())
    if expect == NO_DEVICE and HAS_GPU:  # noqa: SIM102
        pytest.skip("a GPU is present: a valid call would launch on fake pointers")
    status = _call_topk(lib, rows, **case)
    assert status == expect, lib.dsa_last_error_detail()
    assert lib.dsa_last_error_detail().decode() != ""


def test_indexer_validation(lib):
    r = _rows()
    f = lambda **kw: lib.dsa_indexer_scores(ctypes.byref(r), kw.get("q", 0x1000), kw.get("w", 0x2000),
                                            kw.get("k", 0x3000), kw.get("scale", 1.0), kw.get("s", 0x4000),
                                            kw.get("ld", 100), None)
    assert f(q=0) == INVALID
    assert f(q=0x1008) == MISALIGNED
    assert f(w=0x2004) == MISALIGNED
    assert f(k=0) == INVALID
    assert f(s=0x4008) == MISALIGNED
    assert f(scale=0.0) == INVALID
    assert f(scale=float("nan")) == INVALID
    assert f(scale=float("inf")) == INVALID
    assert f(scale=-1.0) == INVALID
    assert f(ld=96) == INVALID
    if not HAS_GPU:
        assert f() == NO_DEVICE


def test_attention_and_decode_step_validation(lib):
    r = _rows(R=16)
    ws_need = m.dsa_sparse_mla_workspace_size(16, 2048)
    f = lambda **kw: lib.dsa_sparse_mla_attn(ctypes.byref(r), kw.get("qa", 0x1000), kw.get("kv", 0x2000),
                                             kw.get("idx", 0x3000), kw.get("k", 2048), kw.get("scale", 0.0625),
                                             kw.get("out", 0x4000), kw.get("lse", None), kw.get("ws", 0x100000),
                                             kw.get("ws_bytes", ws_need), None)
    assert f(qa=0) == INVALID
    assert f(kv=0x2001) == MISALIGNED
    assert f(idx=0) == INVALID
    assert f(k=0) == INVALID
    assert f(scale=0.0) == INVALID
    assert f(out=0x4004) == MISALIGNED
    assert f(lse=0x5002) == MISALIGNED
    assert f(ws_bytes=ws_need - 1) == WS_SMALL
    if not HAS_GPU:
        assert f() == NO_DEVICE
    need = m.dsa_decode_step_workspace_size(16, 100, 2048)
    g = lambda **kw: lib.dsa_decode_step(ctypes.byref(r), 0x1000, 0x2000, 0x3000, kw.get("iscale", 1.0), 0x4000,
                                         0x5000, kw.get("scale", 0.0625), kw.get("k", 2048), 0x6000, 0x7000, None,
                                         0x100000, kw.get("ws_bytes", need), None)
    assert g(iscale=0.0) == INVALID
    assert g(scale=float("nan")) == INVALID
    assert g(k=4096) == INVALID
    assert g(ws_bytes=need - 256) == WS_SMALL
    if not HAS_GPU:
        assert g() == NO_DEVICE


def test_projection_validation(lib):
    f = lambda **kw: lib.dsa_absorb_queries(kw.get("R", 4), kw.get("qn", 0x1000), kw.get("qp", 0x2000),
                                            kw.get("w", 0x3000), kw.get("qa", 0x4000), None)
    assert f(R=0) == INVALID
    assert f(R=(1 << 24) + 1) == INVALID
    assert f(qn=0) == INVALID
    assert f(qp=0x2008) == MISALIGNED
    assert f(w=0) == INVALID
    assert f(qa=0x4002) == MISALIGNED
    if not HAS_GPU:
        assert f() == NO_DEVICE
    g = lambda **kw: lib.dsa_v_up_proj(kw.get("R", 4), kw.get("o", 0x1000), kw.get("w", 0x3000),
                                       kw.get("out", 0x4000), None)
    assert g(R=-1) == INVALID
    assert g(o=0x1004) == MISALIGNED
    assert g(w=0x3008) == MISALIGNED
    assert g(out=0) == INVALID
    if not HAS_GPU:
        assert g() == NO_DEVICE


def test_index_share_source_matches_printed_layer_pattern(lib, oracle_mod):
    """The native layer schedule against the pattern the pages print
    (tests/golden/index_share_layers.json) and against the oracle's spelled-out
    indexer_types array, for all 78 layers."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "index_share_layers.json")) as fh:
        g = json.load(fh)
    L, freq = g["num_layers"], g["index_topk_freq"]
    src = [lib.dsa_index_share_source(l, L, 3, freq) for l in range(L)]
    for a, b, kind, source in g["rows"]:
        for l in range(a, b + 1):
            assert src[l] == source, l
            assert (src[l] == l) == (kind == "full"), l
    assert sum(s == l for l, s in enumerate(src)) == g["full_layers"]
    assert sum(s != l for l, s in enumerate(src)) == g["shared_layers"]
    types = ["full" if s == l else "shared" for l, s in enumerate(src)]
    assert types == oracle_mod.GLM52_INDEXER_TYPES
    # every shared layer points at the latest full layer below it
    for l in range(L):
        fulls = [j for j in range(l + 1) if types[j] == "full"]
        assert src[l] == fulls[-1]
    assert m.dsa_index_share_source(77) == 74


def test_index_share_source_validation_and_other_periods(lib):
    f = lib.dsa_index_share_source
    assert f(-1, 78, 3, 4) == -1
    assert f(78, 78, 3, 4) == -1
    assert f(0, 0, 3, 4) == -1
    assert f(5, 78, 0, 4) == -1
    assert f(5, 78, 3, 0) == -1
    assert [f(l, 10, 1, 1) for l in range(10)] == list(range(10))        # freq 1: no sharing
    assert [f(l, 8, 1, 2) for l in range(8)] == [0, 0, 2, 2, 4, 4, 6, 6]  # one full, one shared
    with pytest.raises(m.DsaError):
        m.dsa_index_share_source(78)


def test_cache_write_workspace_and_validation(lib):
    assert lib.dsa_cache_write_workspace_size(0) == 0
    assert lib.dsa_cache_write_workspace_size((1 << 24) + 1) == 0
    # 64 tokens: one token tile, K split 24 ways; 8192 tokens: no split
    assert lib.dsa_cache_write_workspace_size(64) == 24 * 64 * 704 * 4
    assert lib.dsa_cache_write_workspace_size(8192) == 8192 * 704 * 4
    ws_ok = lib.dsa_cache_write_workspace_size(4)
    d = dict(N=4, x=0x1000, wk=0x2000, kg=0x3000, kb=0x3200, keps=1e-6, kva=0x4000, kvg=0x5000, kveps=1e-5,
             pos=0x6000, slots=0x7000, theta=1e6, kc=0x8000, lc=0x9000, ws=0x10000, wsb=ws_ok)

    def f(**kw):
        a = dict(d, **kw)
        return lib.dsa_cache_write(a["N"], a["x"], a["wk"], a["kg"], a["kb"], a["keps"], a["kva"], a["kvg"],
                                   a["kveps"], a["pos"], a["slots"], a["theta"], a["kc"], a["lc"], a["ws"], a["wsb"],
                                   None)
    assert f(N=0) == INVALID
    assert f(x=0) == INVALID
    assert f(wk=0x2004) == MISALIGNED
    assert f(kva=0) == INVALID
    assert f(kvg=0x5004) == MISALIGNED
    assert f(kg=0) == INVALID
    assert f(kb=0x3201) == MISALIGNED
    assert f(kg=0x3004) == MISALIGNED
    assert f(pos=0) == INVALID
    assert f(slots=0x7004) == MISALIGNED
    assert f(keps=-1.0) == INVALID
    assert f(kveps=float("nan")) == INVALID
    assert f(theta=0.0) == INVALID
    assert f(theta=float("inf")) == INVALID
    assert f(kc=0x8008) == MISALIGNED
    assert f(lc=0) == INVALID
    assert f(wsb=ws_ok - 1) == WS_SMALL
    assert f(ws=0x10010) == MISALIGNED
    if not HAS_GPU:
        assert f() == NO_DEVICE


# ---------------------------------------------------------------------------
# The binding checks every buffer's size against the call's dimensions before
# calling the library (the C ABI sees pointers only, so an undersized output
# would otherwise be written past its end).  CPU tensors suffice: the size
# checks run before any device or pointer check.

def _fake_rows(R=4, maxv=100):
    import types
    return types.SimpleNamespace(num_rows=R, max_visible=maxv, c=None)


def _t(n, dtype=torch.float32):
    return torch.zeros(int(n), dtype=dtype)


def _expect_size_error(fn, name):
    with pytest.raises(m.DsaError) as e:
        fn()
    assert e.value.status == INVALID and name in e.value.detail, e.value.detail


def test_binding_rejects_undersized_buffers(lib):
    R, maxv, k = 4, 100, 2048
    rows = _fake_rows(R, maxv)
    bf = torch.bfloat16
    good = dict(q_idx=_t(R * 32 * 128, bf), w=_t(R * 32), k_idx=_t(200 * 128, bf), q_abs=_t(R * 64 * 576, bf),
                kv=_t(200 * 576, bf), idx=_t(R * k, torch.int32), out=_t(R * 64 * 512), lse=_t(R * 64))

    def with_(**kw):
        d = dict(good)
        d.update(kw)
        return d

    def step(d):
        return lambda: m.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], 1.0, d["q_abs"], d["kv"], 0.0625, k,
                                         d["idx"], d["out"], d["lse"], None)

    _expect_size_error(step(with_(idx=_t(R * k - 1, torch.int32))), "indices")
    _expect_size_error(step(with_(out=_t(R * 64 * 512 - 4))), "out_latent")
    _expect_size_error(step(with_(lse=_t(R * 64 - 1))), "out_lse")
    _expect_size_error(step(with_(q_idx=_t(R * 32 * 128 - 8, bf))), "q_idx")
    _expect_size_error(step(with_(q_abs=_t((R - 1) * 64 * 576, bf))), "q_abs")
    _expect_size_error(step(with_(w=_t(R * 32 - 1))), "w")
    # the attention call and its paged form
    _expect_size_error(lambda: m.dsa_sparse_mla_attn(rows, good["q_abs"], good["kv"], _t(R * k - 1, torch.int32), k,
                                                     0.0625, good["out"], good["lse"]), "indices")
    _expect_size_error(lambda: m.dsa_sparse_mla_attn(rows, good["q_abs"], good["kv"], good["idx"], k, 0.0625,
                                                     _t(100), good["lse"]), "out_latent")
    _expect_size_error(lambda: m.dsa_sparse_mla_attn_paged(rows, None, good["q_abs"], good["kv"], good["idx"], k,
                                                           0.0625, good["out"], _t(3)), "out_lse")
    # scores: too few rows, a flat buffer, a stride below max_visible
    _expect_size_error(lambda: m.dsa_indexer_scores(rows, good["q_idx"], good["w"], good["k_idx"], 1.0,
                                                    _t((R - 1) * 100).view(R - 1, 100)), "scores")
    _expect_size_error(lambda: m.dsa_indexer_scores(rows, good["q_idx"], good["w"], good["k_idx"], 1.0,
                                                    _t(R * 100)), "scores")
    _expect_size_error(lambda: m.dsa_indexer_scores(rows, good["q_idx"], good["w"], good["k_idx"], 1.0,
                                                    _t(R * 96).view(R, 96)), "max_visible")
    _expect_size_error(lambda: m.dsa_topk_select(rows, _t(R * 100).view(R, 100), k, _t(R * k - 2, torch.int32),
                                                 None), "indices")
    _expect_size_error(lambda: m.dsa_indexer_scores_paged(rows, None, _t(8, bf), good["w"], good["k_idx"], 1.0,
                                                          _t(R * 100).view(R, 100)), "q_idx")
    _expect_size_error(lambda: m.dsa_decode_step_paged(rows, None, good["q_idx"], good["w"], good["k_idx"], 1.0,
                                                       good["q_abs"], good["kv"], 0.0625, k, good["idx"], _t(5),
                                                       None), "out_latent")
    # projections and the cache writer
    kvb = _t(64 * 448 * 512, bf)
    _expect_size_error(lambda: m.dsa_absorb_queries(_t(3 * 64 * 192, bf).view(3, 64, 192), _t(3 * 64 * 64, bf),
                                                    kvb, _t(2 * 64 * 576, bf)), "q_abs")
    _expect_size_error(lambda: m.dsa_absorb_queries(_t(3 * 64 * 192, bf).view(3, 64, 192), _t(3 * 64 * 64, bf),
                                                    _t(100, bf), _t(3 * 64 * 576, bf)), "kv_b_weight")
    _expect_size_error(lambda: m.dsa_v_up_proj(_t(2 * 64 * 512).view(2, 64, 512), kvb, _t(2 * 64 * 255)), "out")
    N = 3
    cw = dict(hidden=_t(N * 6144, bf).view(N, 6144), wk=_t(128 * 6144, bf), kg=_t(128), kb=_t(128),
              kva=_t(576 * 6144, bf), kvg=_t(512), pos=_t(N, torch.int32), slots=_t(N, torch.int64))

    def cwcall(**kw):
        d = dict(cw)
        d.update(kw)
        return lambda: m.dsa_cache_write(d["hidden"], d["wk"], d["kg"], d["kb"], 1e-6, d["kva"], d["kvg"], 1e-5,
                                         d["pos"], d["slots"], 1e6, _t(128, bf), _t(576, bf), None)

    _expect_size_error(cwcall(slots=_t(N - 1, torch.int64)), "slots")
    _expect_size_error(cwcall(kva=_t(575 * 6144, bf)), "kv_a_weight")
    _expect_size_error(cwcall(kvg=_t(511)), "kv_norm_weight")


def test_binding_passes_correctly_sized_buffers_on_to_the_device_checks(lib):
    """Buffers of exactly the needed size pass the size checks; the call then
    stops at the device-placement check (CPU tensors here)."""
    R, k = 4, 2048
    rows = _fake_rows(R, 100)
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="device tensor"):
        m.dsa_sparse_mla_attn(rows, _t(R * 64 * 576, bf), _t(576, bf), _t(R * k, torch.int32), k, 0.0625,
                              _t(R * 64 * 512).view(R, 64, 512), _t(R * 64))
    with pytest.raises(ValueError, match="device tensor"):
        m.dsa_indexer_scores(rows, _t(R * 32 * 128, bf), _t(R * 32), _t(128, bf), 1.0, _t(R * 100).view(R, 100))


def test_decode_step_workspace_follows_the_chunk_formula(lib):
    """dsa_decode_step_workspace_size as include/dsa.h spells it out: all rows'
    fp32 score rows while they fit the 1 GiB budget, else chunks of the
    largest multiple of 32 rows that fit (at least 32)."""
    budget = 1 << 30

    def a256(x):
        return (x + 255) // 256 * 256

    def formula(R, maxv, k):
        ld = (maxv + 3) // 4 * 4
        if R * ld * 4 <= budget:
            C = R
        else:
            fit = budget // (ld * 4)
            C = min(R, max(32, fit // 256 * 256 if fit >= 256 else fit // 32 * 32))
        return (a256(C * ld * 4) + a256(4 * C) + 256 + a256(m.dsa_topk_workspace_size(C, maxv, k))
                + a256(m.dsa_sparse_mla_workspace_size(R, k)))

    for R, maxv in [(64, 32768), (16, 202752), (16512, 131072), (8192, 8192), (1, 4096), (3, 1 << 24),
                    (40, 1 << 24), (70000, 9000), (2049, 131072)]:
        assert m.dsa_decode_step_workspace_size(R, maxv, 2048) == formula(R, maxv, 2048), (R, maxv)
    # the ragged batch (16,512 rows up to 131,072 positions) scores 2,048 rows at a time
    assert m.dsa_decode_step_workspace_size(16512, 131072, 2048) < 1.2 * budget
    # the paged step adds the translated index lists and zero row bases
    R, k = 100, 2048
    assert (m.dsa_decode_step_paged_workspace_size(R, 32768, k)
            == m.dsa_decode_step_workspace_size(R, 32768, k) + a256(R * k * 4) + a256(R * 8))
