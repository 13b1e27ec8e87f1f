"""GPU parity: libdsa (HIP, gfx950) against the fp64 CPU oracle on the same
seeded inputs.

Bars (from the method's requirements; tolerances are written here):
  - indexer scores: rel = |s_gpu - s_ref| / max(|s_ref|, 1e-3 * max_t |s_ref|) <= 5e-3
  - top-k fed the oracle's fp32 scores: bit-exact index arrays
  - attention given identical index lists: max |out_gpu - out_ref| <= 2e-2,
    |lse_gpu - lse_ref| <= 2e-2
  - fused path: mean recall >= 0.999, every miss inside the score-gap band
    |s_ref[j] - theta_r| <= 5e-3 * max(|theta_r|, tau_r)
  - rows seeing <= 2048 positions: indices = 0..n-1 and attention = dense
"""
import zlib

import numpy as np
import pytest
import torch

from sparse_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCORE_TOL = 5e-3
ATTN_TOL = 2e-2
DEV = "cuda"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def make_rows(dsa, vis, base, flags=0):
    return dsa.Rows(dev(vis.astype(np.int32)), dev(base.astype(np.int64)), int(vis.max()), flags=flags)


def ld_for(maxv):
    return (maxv + 3) // 4 * 4


def score_rel_err(gpu, ref, n):
    tau = 1e-3 * np.max(np.abs(ref[:n]))
    den = np.maximum(np.abs(ref[:n]), tau)
    diff = np.abs(gpu[:n].astype(np.float64) - ref[:n])
    diff[(gpu[:n] == 0) & (ref[:n] == 0)] = 0.0
    return float(np.max(diff / den)) if n else 0.0


_CACHE = {}


def inputs(name):
    """Generated arrays of a workload (cached for the session)."""
    if name not in _CACHE:
        w = wl.config(name)
        x = w.generate()
        _CACHE[name] = (w, x)
    return _CACHE[name]


def device_inputs(x):
    return dict(q_idx=dev_bf16(x["q_idx"]), w=dev(x["w"]), k_idx=dev_bf16(x["k_idx"]),
                q_abs=dev_bf16(x["q_abs"]), kv_latent=dev_bf16(x["kv_latent"]))


def run_indexer(dsa, x, d=None, flags=0):
    d = d or device_inputs(x)
    vis, base = x["visible_len"], x["row_cache_base"]
    rows = make_rows(dsa, vis, base, flags)
    ld = ld_for(int(vis.max()))
    scores = torch.empty((len(vis), ld), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(rows, d["q_idx"], d["w"], d["k_idx"], 1.0, scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def run_topk(dsa, vis, scores_f32, k):
    R = len(vis)
    ld = ld_for(int(vis.max()))
    s = np.zeros((R, ld), np.float32)
    s[:, : scores_f32.shape[1]] = scores_f32[:, :ld]
    rows = make_rows(dsa, vis, np.zeros(R, np.int64))
    idx = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.dsa_topk_workspace_size(R, int(vis.max()), k), DEV)
    dsa.dsa_topk_select(rows, dev(s), k, idx, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def run_attn(dsa, x, idx, k, rows_sel=None, d=None):
    d = d or device_inputs(x)
    vis, base = x["visible_len"], x["row_cache_base"]
    R = len(vis)
    rows = make_rows(dsa, vis, base)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    ws = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, k), DEV)
    dsa.dsa_sparse_mla_attn(rows, d["q_abs"], d["kv_latent"], dev(idx.astype(np.int32)), k, wl.SOFTMAX_SCALE, out,
                            lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_decode_step(dsa, x, k=2048, d=None):
    d = d or device_inputs(x)
    vis, base = x["visible_len"], x["row_cache_base"]
    R = len(vis)
    rows = make_rows(dsa, vis, base)
    idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
    dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv_latent"],
                        wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def sub(x, rows):
    """Per-row arrays restricted to `rows` (caches untouched)."""
    y = dict(x)
    for key in ("q_idx", "w", "q_abs", "visible_len", "row_cache_base"):
        y[key] = x[key][rows]
    return y


def oracle_scores(oracle, x, rows):
    y = sub(x, rows)
    return oracle.indexer_scores(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"], y["k_idx"])


def check_attention(out, lse, ref_out, ref_lse, label):
    err = float(np.max(np.abs(out - ref_out)))
    fin = np.isfinite(ref_lse)
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert np.array_equal(np.isfinite(lse), fin), label
    assert err <= ATTN_TOL and lerr <= ATTN_TOL, f"{label}: out err {err:.3e}, lse err {lerr:.3e}"
    return err


# ----------------------------------------------------------------------------- indexer

def test_indexer_c1_full(dsa, oracle_mod):
    w, x = inputs("c1")
    s = run_indexer(dsa, x)
    ref = oracle_scores(oracle_mod, x, [0])
    assert score_rel_err(s[0], ref[0], 4096) <= SCORE_TOL


def mixed_block_inputs():
    # 70 rows: rows 0..31 (one shared sequence, causal), rows 32..63 (one
    # block whose rows read two sequences: not shared), rows 64..69 (a
    # partial block).
    T1, T2 = 3000, 700
    vis = np.concatenate([np.arange(T1 - 31, T1 + 1), np.full(16, T2), np.full(16, 2 * T2 // 3),
                          [5, 77, 1024, 1025, 2049, 33]]).astype(np.int32)
    base = np.concatenate([np.zeros(32), np.full(16, T1), np.full(16, T1 + T2), np.full(6, T1 + 2 * T2)]).astype(np.int64)
    seq_len = np.array([T1, T2, T2, 2100], np.int64)
    w = wl.Workload(name="mix", seed=9, visible_len=vis, row_cache_base=base, seq_len=seq_len,
                    seq_base=np.concatenate([[0], np.cumsum(seq_len)[:-1]]).astype(np.int64),
                    row_seq=np.zeros(len(vis), np.int64))
    return w.generate()


def test_indexer_shared_blocks_mixed_with_rows(dsa, oracle_mod):
    # Every row must get its own scores exactly once.
    x = mixed_block_inputs()
    s = run_indexer(dsa, x)
    ref = oracle_mod.indexer_scores(x["visible_len"], x["row_cache_base"], x["q_idx"], x["w"], x["k_idx"])
    for r, n in enumerate(x["visible_len"]):
        assert score_rel_err(s[r], ref[r], n) <= SCORE_TOL, r


def test_indexer_distinct_sequences_hint_changes_nothing(dsa):
    # The hint only skips the shared-block pass; set on rows that do share a
    # sequence, it must still give the very same scores, bit for bit.
    x = mixed_block_inputs()
    d = device_inputs(x)
    a = run_indexer(dsa, x, d)
    b = run_indexer(dsa, x, d, flags=dsa.ROWS_DISTINCT_SEQUENCES)
    for r, n in enumerate(x["visible_len"]):
        assert np.array_equal(a[r, :n].view(np.uint32), b[r, :n].view(np.uint32)), r


def test_indexer_ragged_edge_lengths(dsa, oracle_mod):
    lens = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 9000]
    w = wl._decode("edges", 11, lens, "edge lengths")
    x = w.generate()
    s = run_indexer(dsa, x)
    ref = oracle_mod.indexer_scores(x["visible_len"], x["row_cache_base"], x["q_idx"], x["w"], x["k_idx"])
    for r, n in enumerate(lens):
        assert score_rel_err(s[r], ref[r], n) <= SCORE_TOL, n


@pytest.mark.parametrize("name, rows", [("c3", [0, 31, 63]), ("c4", [0, 15]), ("c2", [0, 1, 31, 32, 2047, 2048, 4095, 8191]),
                                        ("c5", [0, 57, 127, 128, 129, 159, 160, 8000, 16511])])
def test_indexer_sampled_rows(dsa, oracle_mod, name, rows):
    w, x = inputs(name)
    s = run_indexer(dsa, x)
    ref = oracle_scores(oracle_mod, x, rows)
    for i, r in enumerate(rows):
        n = int(x["visible_len"][r])
        assert score_rel_err(s[r], ref[i], n) <= SCORE_TOL, (name, r)


# ----------------------------------------------------------------------------- top-k

@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "signed_zeros", "coarse", "tiny"])
@pytest.mark.parametrize("k", [2048, 1, 7, 300])
def test_topk_bitexact_synthetic(dsa, oracle_mod, kind, k):
    lens = np.array([1, 5, 300, 2047, 2048, 2049, 4095, 4096, 4097, 9000, 20000], np.int32)
    s = wl.random_scores(zlib.crc32(f"{kind}/{k}".encode()) % 1000, len(lens), int(lens.max()), kind=kind)
    s[2, 7] = np.nan
    s[6, 100:110] = -np.inf
    s[7, 3] = np.inf
    got = run_topk(dsa, lens, s, k)
    ref = oracle_mod.topk(lens, s, k)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "signed_zeros", "coarse", "tiny"])
@pytest.mark.parametrize("k", [2048, 1, 7, 300])
def test_topk_bitexact_short_rows(dsa, oracle_mod, kind, k):
    """Calls whose rows all have at most 8,192 positions take the 256-thread
    kernel: every length class up to the limit, NaN, infinities, and a row
    with more NaN than the selection can avoid (NaN orders lowest, the lower
    positions first)."""
    lens = np.array([1, 5, 300, 2047, 2048, 2049, 4095, 4096, 4097, 5000, 8191, 8192, 3000], np.int32)
    s = wl.random_scores(zlib.crc32(f"short/{kind}/{k}".encode()) % 1000, len(lens), int(lens.max()), kind=kind)
    s[2, 7] = np.nan
    s[6, 100:110] = -np.inf
    s[7, 3] = np.inf
    s[12, 1000:2900] = np.nan
    got = run_topk(dsa, lens, s, k)
    ref = oracle_mod.topk(lens, s, k)
    assert np.array_equal(got, ref)


def test_topk_short_and_long_kernels_agree(dsa):
    """The same rows of at most 8,192 positions, once alone (256-thread
    kernel) and once beside a longer row (1024-thread kernel)."""
    lens = np.array([2049, 3000, 4097, 6000, 8192, 8000, 2500], np.int32)
    kinds = ["normal", "ties", "coarse", "tiny", "normal", "zeros", "signed_zeros"]
    s = np.concatenate([wl.random_scores(60 + i, 1, 9000, kind=kd) for i, kd in enumerate(kinds)])
    short = run_topk(dsa, lens, s[:, :8192], 2048)
    long_lens = np.concatenate([lens, [9000]]).astype(np.int32)
    long_s = np.concatenate([s, wl.random_scores(70, 1, 9000, kind="normal")])
    both = run_topk(dsa, long_lens, long_s, 2048)
    assert np.array_equal(short, both[: len(lens)])


def test_topk_bitexact_long_rows_and_overflow(dsa, oracle_mod):
    # 65,536-position rows (one workgroup per row): normal scores (sampled
    # fast path), 8-valued ties and all-equal rows (candidate overflow, exact
    # whole-row fallback), coarse values, fp32 denormals with signed zeros;
    # and 202,752-position rows (multi-workgroup path).
    for n in (65536, 202752):
        lens = np.array([n, n, n, n - 1000, n - 7], np.int32)
        s = np.concatenate([wl.random_scores(1, 1, n, kind="normal"), wl.random_scores(2, 1, n, kind="ties"),
                            wl.random_scores(3, 1, n, kind="zeros"), wl.random_scores(4, 1, n, kind="coarse"),
                            wl.random_scores(5, 1, n, kind="tiny")])
        got = run_topk(dsa, lens, s, 2048)
        ref = oracle_mod.topk(lens, s, 2048)
        assert np.array_equal(got, ref), n


def test_topk_bitexact_mixed_paths_in_one_call(dsa, oracle_mod):
    # One call whose rows straddle the per-row dispatch: rows of at most
    # 65,536 positions (one workgroup each, including rows with n <= k) and
    # longer rows (split over workgroups) must each be owned by exactly one path.
    lens = np.array([100, 5000, 65536, 65537, 131072, 2048, 70001, 2049], np.int32)
    kinds = ["normal", "ties", "normal", "ties", "normal", "coarse", "zeros", "normal"]
    s = np.concatenate([wl.random_scores(20 + i, 1, int(lens.max()), kind=kd) for i, kd in enumerate(kinds)])
    got = run_topk(dsa, lens, s, 2048)
    ref = oracle_mod.topk(lens, s, 2048)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros"])
def test_topk_bitexact_rows_beyond_one_workgroup(dsa, oracle_mod, kind):
    # Calls with rows longer than 65,536 positions take the multi-workgroup
    # path (for every row of the call): normal scores, 8-valued ties,
    # all-equal rows.
    lens = np.array([300000, 65537, 5000, 2049, 1], np.int32)
    s = wl.random_scores(zlib.crc32(kind.encode()) % 1000, len(lens), int(lens.max()), kind=kind)
    for k in (2048, 5):
        got = run_topk(dsa, lens, s, k)
        ref = oracle_mod.topk(lens, s, k)
        assert np.array_equal(got, ref), k


def test_topk_bitexact_many_rows_few_long(dsa, oracle_mod):
    """More than 256 rows, a few of them longer than 65,536 positions: the
    long rows are listed on the device and walked by fixed grids (the short
    ones stay with the one-workgroup-per-row kernel).  Long rows sit at the
    start, middle and end of the batch, and include ties and all-equal rows."""
    g = np.random.default_rng(77)
    R = 300
    lens = g.integers(1, 65537, size=R).astype(np.int32)
    lens[:4] = [2048, 1, 2049, 65536]
    long_at = [0, 5, 6, 71, 72, 100, 299]
    lens[long_at] = [65537, 150000, 99999, 70000, 131072, 66000, 120001]
    kinds = {5: "ties", 72: "zeros", 100: "coarse"}
    n = int(lens.max())
    s = wl.random_scores(31, R, n, kind="normal")
    for r, kd in kinds.items():
        s[r] = wl.random_scores(40 + r, 1, n, kind=kd)[0]
    got = run_topk(dsa, lens, s, 2048)
    ref = oracle_mod.topk(lens, s, 2048)
    bad = [r for r in range(R) if not np.array_equal(got[r], ref[r])]
    assert not bad, bad


def _stream_rows(R, seed, max_n):
    """R rows for the many-rows top-k kernel: every length class around its
    thresholds, normal scores in most rows and, in others, 8-valued ties,
    all-equal rows, coarse values, denormals with signed zeros, NaN runs, -inf
    blocks, +inf, an ascending row whose candidates all belong to the last
    wave (they share the pool), ties above every other score, and large
    scores hidden between the sample blocks (exact-bound pass)."""
    g = np.random.default_rng(seed)
    lens = g.integers(1, max_n + 1, size=R).astype(np.int32)
    edge = [1, 2047, 2048, 2049, 3071, 3072, 3073, 4096, 8192, 8193, 9000, 32768, 65535, 65536]
    lens[: len(edge)] = [min(e, max_n) for e in edge]
    n = int(lens.max())
    s = wl.random_scores(seed, R, n, kind="normal")
    kinds = ["ties", "zeros", "coarse", "tiny", "signed_zeros"]
    for i, r in enumerate(range(len(edge), len(edge) + 3 * len(kinds))):
        s[r] = wl.random_scores(seed + 1 + i, 1, n, kind=kinds[i % len(kinds)])[0]
        lens[r] = max(int(lens[r]), 9000)
    r0 = len(edge) + 3 * len(kinds)
    lens[r0:r0 + 5] = [60000, 60000, 40000, 20000, 65536]
    s[r0, 100:59000] = np.nan                        # fewer non-NaN scores than k: NaN kept, lowest positions first
    s[r0 + 1, :30000] = -np.inf
    s[r0 + 1, 40000] = np.inf
    s[r0 + 2, :40000] = np.arange(40000, dtype=np.float32)  # ascending: the last quarter holds every candidate
    s[r0 + 3] = s[r0 + 3] * np.float32(1 / 16)
    s[r0 + 3, ::20] = np.float32(5.0)                 # 1,000 ties above every other score: theta for k < 1,000
    # 2,400 large scores placed between the kernel's 64 sample blocks (64
    # positions at ((n - 64) b / 63) & ~3): the sampled bound misses them and
    # too many candidates pass it, so the row takes the exact-bound pass.
    n4 = 65536
    starts = [((n4 - 64) * b // 63) & ~3 for b in (10, 20, 30)]
    big = np.concatenate([np.arange(a + 200, a + 1000) for a in starts])
    s[r0 + 4, big] = np.float32(1e6) + np.arange(len(big), dtype=np.float32)
    return lens, s


@pytest.mark.parametrize("k", [2048, 1, 7, 300])
def test_topk_bitexact_stream_kernel_many_rows(dsa, oracle_mod, k):
    """Calls with at least 1,024 rows whose rows have at most 65,536 positions
    take the four-per-CU streaming kernel: sampled bound, per-wave ordered
    candidate lists in a shared chunk pool, radix rounds, and the exact-bound
    re-stream or whole-row fallback when the pool overflows or holds fewer
    than k (ties at the bound, NaN, all-equal rows)."""
    lens, s = _stream_rows(1030, 90 + k, 65536)
    got = run_topk(dsa, lens, s, k)
    ref = oracle_mod.topk(lens, s, k)
    bad = [r for r in range(len(lens)) if not np.array_equal(got[r], ref[r])]
    assert not bad, bad[:10]


def test_topk_bitexact_stream_kernel_beside_long_rows(dsa, oracle_mod):
    """Many rows with a few longer than 65,536 positions: the streaming kernel
    takes the short rows, the one-workgroup kernel only samples the long ones
    and the multi-workgroup path finishes them; each row has exactly one owner."""
    lens, s = _stream_rows(1040, 7, 65536)
    n_long = 90000
    s2 = np.zeros((len(lens), n_long), np.float32)
    s2[:, : s.shape[1]] = s
    del s
    long_at = [3, 200, 1039]
    for i, r in enumerate(long_at):
        lens[r] = [65537, n_long, 70001][i]
        s2[r] = wl.random_scores(500 + r, 1, n_long, kind=["normal", "ties", "normal"][i])[0]
    got = run_topk(dsa, lens, s2, 2048)
    ref = oracle_mod.topk(lens, s2, 2048)
    bad = [r for r in range(len(lens)) if not np.array_equal(got[r], ref[r])]
    assert not bad, bad[:10]


@pytest.mark.parametrize("k", [2048, 1, 300])
def test_topk_bitexact_chunked_path_for_few_rows(dsa, oracle_mod, k):
    """Calls with at most 256 rows whose longest row has 65,537..262,144
    positions split each row over 4,096-position chunks: a sampled bound per
    row, candidates per chunk in position order, one workgroup finishing each
    row.  Rows at and around the chunk and length limits; a row whose top sits
    in one chunk; 8-valued ties and all-equal rows (more candidates than the
    finishing workgroup holds: exact whole-row path); a row mostly NaN;
    normal rows."""
    lens = np.array([262144, 8193, 12288, 12289, 40000, 65536, 100000, 262143, 30000, 30000, 2048, 9000],
                    np.int32)
    R, n = len(lens), int(lens.max())
    kinds = ["normal", "normal", "ties", "normal", "zeros", "coarse", "normal", "tiny", "normal", "normal",
             "normal", "signed_zeros"]
    s = np.concatenate([wl.random_scores(90 + i, 1, n, kind=kd) for i, kd in enumerate(kinds)])
    s[8, 8192:12288] += 20.0  # the top of this row lies in one chunk
    s[9, 100:29000] = np.nan
    got = run_topk(dsa, lens, s, k)
    ref = oracle_mod.topk(lens, s, k)
    bad = [r for r in range(R) if not np.array_equal(got[r], ref[r])]
    assert not bad, bad


@pytest.mark.parametrize("name, rows", [("c1", [0]), ("c4", [3, 9]), ("c2", [0, 2047, 2048, 2049, 5000, 8191])])
def test_topk_bitexact_on_oracle_scores(dsa, oracle_mod, name, rows):
    w, x = inputs(name)
    ref_s = oracle_scores(oracle_mod, x, rows)
    s32 = oracle_mod.round_to_f32(np.nan_to_num(ref_s, nan=0.0))
    vis = x["visible_len"][rows]
    got = run_topk(dsa, vis, s32, 2048)
    ref = oracle_mod.topk(vis, s32, 2048)
    assert np.array_equal(got, ref)


def test_topk_tie_variant_on_gpu_scores(dsa, oracle_mod):
    """8-prototype index keys: equal keys give bitwise-equal GPU scores, so the
    top-k boundary falls inside a tie group and the lower positions must win."""
    w = wl.prefill(8192, seed=1, tie_keys=True)
    rows = [2048, 3000, 6000, 8191]
    x = w.generate(rows=rows)
    s = run_indexer(dsa, x)
    assert len(np.unique(s[3, :8192])) <= 8
    got = run_topk(dsa, x["visible_len"], s, 2048)
    ref = oracle_mod.topk(x["visible_len"], s, 2048)
    assert np.array_equal(got, ref)
    # and the GPU scores agree with the oracle's
    ref_s = oracle_mod.indexer_scores(x["visible_len"], x["row_cache_base"], x["q_idx"], x["w"], x["k_idx"])
    for i, r in enumerate(rows):
        assert score_rel_err(s[i], ref_s[i], r + 1) <= SCORE_TOL


def test_c2_tie_variant_topk_bitexact_on_oracle_scores(dsa, oracle_mod):
    """The 8-prototype variant of the 8,192-token prefill (every index key is
    one of 8 seeded rows, so each row has at most 8 distinct scores and the
    top-2048 boundary falls inside a tie group): the top-k fed the oracle's
    fp32 scores returns the oracle's lists bit for bit, which keep the lowest
    positions of the boundary group."""
    w, x = inputs("c2t")
    rows = [2048, 2049, 3000, 4095, 4096, 6000, 8191]
    ref_s = oracle_scores(oracle_mod, x, rows)
    s32 = oracle_mod.round_to_f32(np.nan_to_num(ref_s, nan=0.0))
    vis = x["visible_len"][rows]
    split = 0
    for i, n in enumerate(vis):
        vals = np.unique(s32[i, :n])
        assert len(vals) <= 8
        theta = np.sort(s32[i, :n])[::-1][2047]
        above = int(np.sum(s32[i, :n] > theta))
        ties = int(np.sum(s32[i, :n] == theta))
        split += above < 2048 < above + ties  # the boundary cuts a tie group
    assert split == len(rows)
    got = run_topk(dsa, vis, s32, 2048)
    ref = oracle_mod.topk(vis, s32, 2048)
    assert np.array_equal(got, ref)


def test_c2_tie_variant_fused_step(dsa, oracle_mod):
    """The whole step over all 8,192 rows of the tied-key prefill: rows seeing
    at most 2,048 positions select all of them; longer rows agree with the
    oracle's selection (recall with the gap rule), and attention agrees with
    the oracle on the lists the GPU chose."""
    w, x = inputs("c2t")
    idx, out, lse = run_decode_step(dsa, x)
    n = x["visible_len"]
    short = n <= 2048
    expect = np.where(np.arange(2048)[None, :] < n[short][:, None], np.arange(2048)[None, :], -1)
    assert np.array_equal(idx[short], expect)
    rows = [100, 2047, 2048, 2500, 4096, 7000, 8191]
    y = sub(x, rows)
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                   y["k_idx"], y["q_abs"], y["kv_latent"], 2048, 1.0,
                                                   wl.SOFTMAX_SCALE)
    assert recall_check(idx[rows], idx_ref, s64, y["visible_len"]) >= 0.999
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], idx[rows],
                                             wl.SOFTMAX_SCALE)
    check_attention(out[rows], lse[rows], ref_out, ref_lse, "c2 tie variant")


def test_c5_full_size_fused_step(dsa, oracle_mod):
    """The ragged mixed batch at full size: 128 decode rows of 517 to 129,329
    positions beside a 16,384-row causal chunk on a 49,152-position history
    (16,512 rows).  Their fp32 score rows exceed the step's 1 GiB budget, so
    the step scores and selects 2,048 rows at a time; its lists and outputs
    equal, bit for bit, the separate calls over all rows at once.  Sampled
    decode rows below 2,048, between 2,048 and 65,536 and above 65,536
    positions, and the chunk's first, middle and last rows, agree with the
    oracle (short rows take every position; recall with the gap rule;
    attention on the GPU's own lists)."""
    w, x = inputs("c5")
    d = device_inputs(x)
    vis, base = x["visible_len"], x["row_cache_base"]
    R, maxv, k = len(vis), int(vis.max()), 2048
    rows = make_rows(dsa, vis, base)
    ws_bytes = dsa.dsa_decode_step_workspace_size(R, maxv, k)
    assert ws_bytes < (5 << 28)  # 1 GiB of score rows plus the top-k's per-row state
    ws = dsa.workspace(ws_bytes, DEV)
    idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv_latent"],
                        wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
    del ws
    # the separate calls over every row at once (8.7 GB of scores)
    ld = ld_for(maxv)
    scores = torch.empty((R, ld), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, scores)
    idx_b = torch.empty_like(idx)
    dsa.dsa_topk_select(rows, scores, k, idx_b, dsa.workspace(dsa.dsa_topk_workspace_size(R, maxv, k), DEV))
    torch.cuda.synchronize()
    del scores
    assert torch.equal(idx, idx_b)
    out_b = torch.empty_like(out)
    lse_b = torch.empty_like(lse)
    dsa.dsa_sparse_mla_attn(rows, d["q_abs"], d["kv_latent"], idx_b, k, wl.SOFTMAX_SCALE, out_b, lse_b,
                            dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, k), DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out_b.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse_b.view(torch.int32))
    del out_b, lse_b
    idx_h = idx.cpu().numpy()
    dec = vis[:128]
    pick = []
    for lo, hi in [(1, 2047), (2048, 65536), (65537, 1 << 30)]:
        cand = np.nonzero((dec >= lo) & (dec <= hi))[0]
        pick += [int(cand[0]), int(cand[-1])]
    pick += [128, 128 + 8191, R - 1]
    # rows seeing fewer than 2,048 positions take all of them
    for r in range(128):
        if vis[r] <= k:
            assert np.array_equal(idx_h[r], np.where(np.arange(k) < vis[r], np.arange(k), -1)), r
    y = sub(x, pick)
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                   y["k_idx"], y["q_abs"], y["kv_latent"], k, 1.0,
                                                   wl.SOFTMAX_SCALE)
    assert recall_check(idx_h[pick], idx_ref, s64, y["visible_len"]) >= 0.999
    out_h = out[pick].cpu().numpy()
    lse_h = lse[pick].cpu().numpy()
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], idx_h[pick],
                                             wl.SOFTMAX_SCALE)
    check_attention(out_h, lse_h, ref_out, ref_lse, "c5")


# ----------------------------------------------------------------------------- attention

def test_attention_c1_oracle_indices(dsa, oracle_mod):
    w, x = inputs("c1")
    _, _, idx, ref_out, ref_lse = oracle_mod.decode_step(x["visible_len"], x["row_cache_base"], x["q_idx"], x["w"],
                                                         x["k_idx"], x["q_abs"], x["kv_latent"], 2048, 1.0,
                                                         wl.SOFTMAX_SCALE)
    out, lse = run_attn(dsa, x, idx, 2048)
    check_attention(out, lse, ref_out, ref_lse, "c1")


@pytest.mark.parametrize("k", [2048, 1, 100, 2047])
def test_attention_random_index_sets_with_padding(dsa, oracle_mod, k):
    lens = [4096, 3000, 700, 2048, 50, 1]
    w = wl._decode("attn", 21 + k, lens, "attention sets")
    x = w.generate()
    g = np.random.default_rng(k)
    idx = np.full((len(lens), k), -1, np.int32)
    for r, n in enumerate(lens):
        m = min(k, n)
        sel = np.sort(g.choice(n, size=m, replace=False))
        idx[r, :m] = sel
    if k >= 100:
        idx[1, 10:20] = -1          # padding inside the list
        idx[4, :] = -1              # a row with nothing selected -> out 0, lse -inf
    ref_out, ref_lse = oracle_mod.sparse_mla(x["row_cache_base"], x["q_abs"], x["kv_latent"], idx, wl.SOFTMAX_SCALE)
    out, lse = run_attn(dsa, x, idx, k)
    check_attention(out, lse, ref_out, ref_lse, f"k={k}")
    if k >= 100:
        assert np.all(out[4] == 0) and np.all(np.isneginf(lse[4]))


def _splits_of_call(dsa, R, k):
    """Splits per row of an attention call, read back from the workspace it asks
    for: R * s bf16 partials of 64 x 512 plus R * s (max, sum) pairs of 64."""
    ws = dsa.dsa_sparse_mla_workspace_size(R, k)
    al = lambda b: (b + 255) // 256 * 256
    found = [s for s in range(1, 17) if (0 if s == 1 else al(R * s * 64 * 512 * 2) + al(R * s * 64 * 8)) == ws]
    assert len(found) == 1, (R, k, ws)
    return found[0]


@pytest.mark.parametrize("R, k, splits", [(1, 2048, 16), (12, 2048, 13), (8, 1000, 11), (19, 2048, 8), (26, 2048, 7),
                                          (33, 2048, 5), (41, 2048, 4), (64, 2048, 3), (100, 2048, 2), (160, 2048, 1)])
def test_attention_each_split_count(dsa, oracle_mod, R, k, splits):
    """Attention against the oracle for calls whose rows are split 16, 13, 11,
    8, 7, 5, 4, 3, 2 ways or not at all (splits of equal whole tiles, the last
    one shorter where the tiles do not divide), with padding slots inside the
    lists and one row that selects nothing; sampled rows.  R rows read one
    4,096-position sequence through their own random index sets."""
    assert _splits_of_call(dsa, R, k) == splits
    T = 4096
    w = wl.Workload(name="splits", seed=40 + R, visible_len=np.full(R, T, np.int32),
                    row_cache_base=np.zeros(R, np.int64), seq_len=np.array([T], np.int64),
                    seq_base=np.zeros(1, np.int64), row_seq=np.zeros(R, np.int64))
    x = w.generate()
    g = np.random.default_rng(1000 * R + k)
    idx = np.stack([np.sort(g.choice(T, size=k, replace=False)) for _ in range(R)]).astype(np.int32)
    idx[0, 3:40] = -1                 # padding inside the first row's list
    if R > 2:
        idx[R // 2, :] = -1           # a row with nothing selected
    out, lse = run_attn(dsa, x, idx, k)
    rows = sorted({0, R // 2, R - 1})
    y = sub(x, rows)
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], x["kv_latent"], idx[rows],
                                             wl.SOFTMAX_SCALE)
    check_attention(out[rows], lse[rows], ref_out, ref_lse, f"R={R} k={k} splits={splits}")
    if R > 2:
        assert np.all(out[R // 2] == 0) and np.all(np.isneginf(lse[R // 2]))


def test_attention_many_rows_single_split(dsa, oracle_mod):
    # >= 512 rows: one split per row (no combine pass).
    w = wl.prefill(700, seed=5)
    x = w.generate()
    idx = np.where(np.arange(700)[None, :] <= np.arange(700)[:, None], np.arange(700)[None, :], -1).astype(np.int32)
    rows = [0, 1, 255, 699]
    ref_out, ref_lse = oracle_mod.sparse_mla(x["row_cache_base"][rows], x["q_abs"][rows], x["kv_latent"], idx[rows],
                                             wl.SOFTMAX_SCALE)
    out, lse = run_attn(dsa, x, idx, 700)
    check_attention(out[rows], lse[rows], ref_out, ref_lse, "single split")


# ----------------------------------------------------------------------------- fused path

def recall_check(idx_gpu, idx_ref, s_ref64, vis, k=2048):
    recalls = []
    for r in range(len(vis)):
        n = int(vis[r])
        kr = min(k, n)
        a = set(idx_gpu[r][idx_gpu[r] >= 0].tolist())
        b = set(idx_ref[r][idx_ref[r] >= 0].tolist())
        assert len(a) == kr
        recalls.append(len(a & b) / kr)
        if a != b:
            row = s_ref64[r, :n]
            theta = np.sort(row)[::-1][kr - 1]
            tau = 1e-3 * np.max(np.abs(row))
            band = 5e-3 * max(abs(theta), tau)
            for j in b - a:
                assert abs(row[j] - theta) <= band, (r, j, row[j], theta)
    return float(np.mean(recalls))


@pytest.mark.parametrize("name, rows", [("c1", [0]), ("c3", [0, 40, 63]), ("c4", [5])])
def test_decode_step_fused(dsa, oracle_mod, name, rows):
    w, x = inputs(name)
    idx, out, lse = run_decode_step(dsa, x)
    y = sub(x, rows)
    s64, s32, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                     y["k_idx"], y["q_abs"], y["kv_latent"], 2048, 1.0,
                                                     wl.SOFTMAX_SCALE)
    rec = recall_check(idx[rows], idx_ref, s64, y["visible_len"])
    assert rec >= 0.999, rec
    # attention against the oracle on the GPU's own index lists
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], idx[rows],
                                             wl.SOFTMAX_SCALE)
    check_attention(out[rows], lse[rows], ref_out, ref_lse, name)


def test_prefill_rows_up_to_k_equal_dense(dsa, oracle_mod):
    w, x = inputs("c2")
    idx, out, lse = run_decode_step(dsa, x)
    n = x["visible_len"]
    short = n <= 2048
    expect = np.where(np.arange(2048)[None, :] < n[short][:, None], np.arange(2048)[None, :], -1)
    assert np.array_equal(idx[short], expect)
    rows = [0, 1, 1000, 2047]
    y = sub(x, rows)
    dense = np.where(np.arange(2048)[None, :] < y["visible_len"][:, None], np.arange(2048)[None, :], -1).astype(np.int32)
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], dense, wl.SOFTMAX_SCALE)
    check_attention(out[rows], lse[rows], ref_out, ref_lse, "dense rows")
    # long rows: recall against the oracle
    rows = [2048, 6000, 8191]
    y = sub(x, rows)
    s64, s32, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                     y["k_idx"], y["q_abs"], y["kv_latent"], 2048, 1.0,
                                                     wl.SOFTMAX_SCALE)
    assert recall_check(idx[rows], idx_ref, s64, y["visible_len"]) >= 0.999


@pytest.mark.parametrize("R", [64, 128, 48, 16, 8])
def test_decode_step_attention_matches_standalone_call(dsa, R):
    """The attention inside dsa_decode_step equals dsa_sparse_mla_attn on the
    same index lists bit for bit, for 3, 2, 4, 11 and 16 splits per row, also when
    the workspace starts out full of garbage and is reused by a second call
    (the split partials and their merge leave nothing behind)."""
    w, x = inputs("c3")
    y = sub(x, [i % 64 for i in range(R)])
    d = device_inputs(y)
    vis, base = y["visible_len"], y["row_cache_base"]
    rows = make_rows(dsa, vis, base)
    k = 2048
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
    ws.fill_(255)
    for rep in range(2):
        idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
        out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
        lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
        dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv_latent"],
                            wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
        torch.cuda.synchronize()
        ref_out, ref_lse = run_attn(dsa, y, idx.cpu().numpy(), k, d=d)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref_out.view(np.uint32)), rep
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref_lse.view(np.uint32)), rep


@pytest.mark.parametrize("k, iscale", [(1, 0.25), (300, 3.0), (1000, 1.0)])
def test_decode_step_other_k_and_index_scale(dsa, oracle_mod, k, iscale):
    """The fused step at k below 2048 and index scales other than 1, over rows
    shorter than, equal to and longer than k: equal to the separate calls bit
    for bit; rows with n <= k select 0..n-1 and pad with -1; longer rows agree
    with the oracle's selection (recall, near-threshold swaps only); attention
    agrees with the oracle on the lists used."""
    lens = [5000, 700, 300, 1, 4096, 2049, k, k + 1]
    w = wl._decode("kvar", 13, lens, "k variants")
    x = w.generate()
    d = device_inputs(x)
    vis, base = x["visible_len"], x["row_cache_base"]
    R = len(vis)
    rows = make_rows(dsa, vis, base)
    idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
    dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], iscale, d["q_abs"], d["kv_latent"], wl.SOFTMAX_SCALE,
                        k, idx, out, lse, ws)
    torch.cuda.synchronize()
    idx_h, out_h, lse_h = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    # separate calls
    ld = ld_for(int(vis.max()))
    scores = torch.empty((R, ld), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(rows, d["q_idx"], d["w"], d["k_idx"], iscale, scores)
    idx_b = torch.empty((R, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk_select(rows, scores, k, idx_b, dsa.workspace(dsa.dsa_topk_workspace_size(R, int(vis.max()), k), DEV))
    torch.cuda.synchronize()
    assert np.array_equal(idx_h, idx_b.cpu().numpy())
    out_b, lse_b = run_attn(dsa, x, idx_h, k, d=d)
    assert np.array_equal(out_h.view(np.uint32), out_b.view(np.uint32))
    assert np.array_equal(lse_h.view(np.uint32), lse_b.view(np.uint32))
    for r in range(R):
        n = int(vis[r])
        if n <= k:
            assert np.array_equal(idx_h[r], np.where(np.arange(k) < n, np.arange(k), -1)), r
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(vis, base, x["q_idx"], x["w"], x["k_idx"], x["q_abs"],
                                                   x["kv_latent"], k, iscale, wl.SOFTMAX_SCALE)
    recalls = []
    for r in range(R):
        n, kr = int(vis[r]), min(k, int(vis[r]))
        a = set(idx_h[r][idx_h[r] >= 0].tolist())
        b = set(idx_ref[r][idx_ref[r] >= 0].tolist())
        assert len(a) == kr, r
        recalls.append(len(a & b) / kr)
        if a != b:
            row = s64[r, :n]
            theta = np.sort(row)[::-1][kr - 1]
            band = 5e-3 * max(abs(theta), 1e-3 * np.max(np.abs(row)))
            for j in b - a:
                assert abs(row[j] - theta) <= band, (r, j)
    assert np.mean(recalls) >= 0.999, recalls
    ref_out, ref_lse = oracle_mod.sparse_mla(base, x["q_abs"], x["kv_latent"], idx_h, wl.SOFTMAX_SCALE)
    check_attention(out_h, lse_h, ref_out, ref_lse, f"k={k}")


def test_decode_step_rows_beside_shared_blocks(dsa, oracle_mod):
    """A batch mixing a prefill chunk (two full 32-row blocks on one sequence,
    which the shared-block kernel scores) with decode rows of very different
    lengths: the decode step lists the other rows on the device and gives
    each many workgroups.  Its selection and output must equal, bit for bit,
    the separate calls (whose indexer scores every row directly), and the
    long rows must agree with the oracle."""
    T0 = 5000
    chunk_vis = np.arange(T0 - 63, T0 + 1)
    dec = [70000, 12000, 100, 3000, 2049, 1]
    vis = np.concatenate([chunk_vis, dec]).astype(np.int32)
    seq_len = np.array([T0] + dec, np.int64)
    seq_base = np.concatenate([[0], np.cumsum(seq_len)[:-1]]).astype(np.int64)
    base = np.concatenate([np.zeros(64), seq_base[1:]]).astype(np.int64)
    w = wl.Workload(name="mixdec", seed=23, visible_len=vis, row_cache_base=base, seq_len=seq_len,
                    seq_base=seq_base, row_seq=np.zeros(len(vis), np.int64))
    x = w.generate()
    d = device_inputs(x)
    idx_a, out_a, lse_a = run_decode_step(dsa, x, d=d)
    scores = run_indexer(dsa, x, d=d)
    idx_b = run_topk(dsa, vis, scores, 2048)
    out_b, lse_b = run_attn(dsa, x, idx_b, 2048, d=d)
    assert np.array_equal(idx_a, idx_b)
    assert np.array_equal(out_a.view(np.uint32), out_b.view(np.uint32))
    assert np.array_equal(lse_a.view(np.uint32), lse_b.view(np.uint32))
    rows = [0, 63, 64, 65, 67]
    y = sub(x, rows)
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                   y["k_idx"], y["q_abs"], y["kv_latent"], 2048, 1.0,
                                                   wl.SOFTMAX_SCALE)
    assert recall_check(idx_a[rows], idx_ref, s64, y["visible_len"]) >= 0.999


@pytest.mark.parametrize("distinct, span", [(False, 4096), (True, 9000)])
def test_decode_step_rows_past_grid_y_limit(dsa, oracle_mod, distinct, span):
    """70,000 decode rows, more than a launch grid's y dimension holds: every
    per-row kernel spills its rows into z.  Each row's per-row inputs are one
    of 509 drawn templates (row r uses r % 509), with its own length and cache
    base, so a row computed as another or not at all shows.  Every row is
    checked for whole selection counts and finite outputs; rows on both
    sides of the y limit are checked against the oracle.  Lengths up to 4,096
    without the distinct-sequence hint: listed row indexer, 256-thread top-k.
    Up to 9,000 with it: direct row-indexer grid, 1024-thread top-k."""
    R, NT = 70000, 509
    CACHE = 2048 + span
    r = np.arange(R, dtype=np.int64)
    vis = (1 + (r * 7919) % span).astype(np.int32)
    base = ((r * 97) % 2048).astype(np.int64)
    w = wl.Workload(name="manyrows", seed=31, visible_len=vis[:NT], row_cache_base=base[:NT],
                    seq_len=np.array([CACHE], np.int64), seq_base=np.zeros(1, np.int64), row_seq=np.zeros(NT, np.int64))
    x = w.generate()
    tmpl = torch.from_numpy(r % NT).to(DEV)
    q_idx = dev_bf16(x["q_idx"]).index_select(0, tmpl)
    wts = dev(x["w"]).index_select(0, tmpl)
    q_abs = dev_bf16(x["q_abs"]).index_select(0, tmpl)
    k = 2048
    rows = make_rows(dsa, vis, base, flags=dsa.ROWS_DISTINCT_SEQUENCES if distinct else 0)
    idx = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    out = torch.full((R, 64, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((R, 64), float("nan"), dtype=torch.float32, device=DEV)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
    dsa.dsa_decode_step(rows, q_idx, wts, dev_bf16(x["k_idx"]), wl.INDEX_SCALE, q_abs, dev_bf16(x["kv_latent"]),
                        wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
    torch.cuda.synchronize()
    vis_d = dev(vis).to(torch.int64)
    assert torch.equal((idx >= 0).sum(1), torch.clamp(vis_d, max=k))
    assert bool((idx < vis_d[:, None]).all()) and bool((idx >= -1).all())
    assert bool(torch.isfinite(lse).all()) and bool(torch.isfinite(out).all())
    pick = [0, 1, 2, 65534, 65535, 65536, 65537, 69998, 69999]
    pick += [int(v) for v in np.random.default_rng(31).integers(0, R, 4)]
    pick += [int(np.flatnonzero(vis[65535:] > k)[0]) + 65535, int(np.flatnonzero(vis[65535:] <= k)[0]) + 65535]
    sel = torch.tensor(pick, device=DEV)
    g_idx = idx.index_select(0, sel).cpu().numpy()
    g_out = out.index_select(0, sel).cpu().numpy()
    g_lse = lse.index_select(0, sel).cpu().numpy()
    t = np.asarray(pick) % NT
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(vis[pick], base[pick], x["q_idx"][t], x["w"][t], x["k_idx"],
                                                   x["q_abs"][t], x["kv_latent"], k, 1.0, wl.SOFTMAX_SCALE)
    assert recall_check(g_idx, idx_ref, s64, vis[pick]) >= 0.999
    ref_out, ref_lse = oracle_mod.sparse_mla(base[pick], x["q_abs"][t], x["kv_latent"], g_idx, wl.SOFTMAX_SCALE)
    check_attention(g_out, g_lse, ref_out, ref_lse, "rows past the y limit")


def test_decode_step_deterministic(dsa):
    w, x = inputs("c3")
    d = device_inputs(x)
    a = run_decode_step(dsa, x, d=d)
    b = run_decode_step(dsa, x, d=d)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


# ----------------------------------------------------------------------------- cache writers

SENTINEL = 0x7F7F  # a finite bf16 pattern no written row can be mistaken for in bulk


def run_cache_write(dsa, c, theta, eps=(1e-6, 1e-5)):
    N = c["hidden"].shape[0]
    kc = torch.full((c["cache_rows"], 128), SENTINEL, dtype=torch.int16, device=DEV)
    lc = torch.full((c["cache_rows"], 576), SENTINEL, dtype=torch.int16, device=DEV)
    ws = dsa.workspace(dsa.dsa_cache_write_workspace_size(N), DEV)
    ws.fill_(255)
    dsa.dsa_cache_write(dev_bf16(c["hidden"]), dev_bf16(c["wk"]), dev(c["k_norm_weight"]), dev(c["k_norm_bias"]), eps[0],
                        dev_bf16(c["kv_a"]), dev(c["kv_norm_weight"]), eps[1], dev(c["positions"]), dev(c["slots"]),
                        theta, kc, lc, ws)
    torch.cuda.synchronize()
    return kc.cpu().numpy().view(np.uint16), lc.cpu().numpy().view(np.uint16)


def check_cache_rows(got_bits, ref, label):
    """bf16 results against fp64 rows: within one bf16 rounding (2^-8 |ref|)
    plus the fp32 arithmetic before it (bounded by 1e-4 of the row's rms),
    and >= 99.5% of elements equal to bf16(ref)."""
    got = wl.bf16_bits_to_f32(got_bits).astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rms
    assert np.all(err <= bound), f"{label}: worst excess {np.max(err - bound):.3e}"
    same = got_bits == wl.f32_to_bf16_bits(ref.astype(np.float32))
    assert same.mean() >= 0.995, f"{label}: {same.mean():.4f} equal to bf16(ref)"


@pytest.mark.parametrize("N", [1, 5, 64, 300, 1000])
def test_cache_write_against_oracle(dsa, oracle_mod, N):
    """Both cache rows of N new tokens against the oracle, at positions up to
    2^20 (RoPE angles far from 0) and theta = 8e6: the rows named by slots
    hold the results, every other row (including those of tokens with slot
    -1) keeps its sentinel.  N = 1 and 64 split K 24 ways, 300 twelve, 1000
    three; 5, 300 and 1000 leave ragged token tiles."""
    c = wl.cache_write_inputs(N, seed=70 + N)
    theta = 8e6
    kc, lc = run_cache_write(dsa, c, theta)
    key, lat = oracle_mod.cache_rows(c["hidden"], c["wk"], c["k_norm_weight"], c["k_norm_bias"], 1e-6, c["kv_a"],
                                     c["kv_norm_weight"], 1e-5, c["positions"].astype(np.int64), theta)
    live = c["slots"] >= 0
    sl = c["slots"][live]
    check_cache_rows(kc[sl], key[live], f"key N={N}")
    check_cache_rows(lc[sl], lat[live], f"latent N={N}")
    untouched = np.setdiff1d(np.arange(c["cache_rows"]), sl)
    assert np.all(kc[untouched] == SENTINEL) and np.all(lc[untouched] == SENTINEL)


def test_cache_write_prefill_sized_sampled_and_deterministic(dsa, oracle_mod):
    """8192 tokens (no K split): 48 sampled tokens against the oracle, theta
    = 1e6; a second call gives the same bytes."""
    N = 8192
    c = wl.cache_write_inputs(N, seed=9, max_position=202752)
    theta = 1e6
    kc, lc = run_cache_write(dsa, c, theta)
    kc2, lc2 = run_cache_write(dsa, c, theta)
    assert np.array_equal(kc, kc2) and np.array_equal(lc, lc2)
    pick = np.unique(np.concatenate([[0, 1, N - 1], np.random.default_rng(0).choice(N, 45, replace=False)]))
    pick = pick[c["slots"][pick] >= 0]
    key, lat = oracle_mod.cache_rows(c["hidden"][pick], c["wk"], c["k_norm_weight"], c["k_norm_bias"], 1e-6,
                                     c["kv_a"], c["kv_norm_weight"], 1e-5, c["positions"][pick].astype(np.int64),
                                     theta)
    check_cache_rows(kc[c["slots"][pick]], key, "key prefill")
    check_cache_rows(lc[c["slots"][pick]], lat, "latent prefill")


def test_cache_write_feeds_the_path(dsa, oracle_mod):
    """Rows the writer produced are what the indexer and attention read: a
    decode step over a 3000-position cache written by dsa_cache_write (slots
    = positions) matches the oracle's step over the oracle's rows rounded to
    bf16 (recall, and attention on the GPU's own list)."""
    T = 3000
    c = wl.cache_write_inputs(T, seed=11, cache_rows=T)
    c["positions"] = np.arange(T, dtype=np.int32)
    c["slots"] = np.arange(T, dtype=np.int64)
    kc, lc = run_cache_write(dsa, c, 1e6)
    key, lat = oracle_mod.cache_rows(c["hidden"], c["wk"], c["k_norm_weight"], c["k_norm_bias"], 1e-6, c["kv_a"],
                                     c["kv_norm_weight"], 1e-5, c["positions"].astype(np.int64), 1e6)
    x = wl.decode(1, T, seed=12).generate(with_caches=False)
    x["k_idx"], x["kv_latent"] = kc, lc
    idx, out, lse = run_decode_step(dsa, x)
    kb = wl.f32_to_bf16_bits(key.astype(np.float32))
    lb = wl.f32_to_bf16_bits(lat.astype(np.float32))
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(x["visible_len"], x["row_cache_base"], x["q_idx"], x["w"], kb,
                                                   x["q_abs"], lb, 2048, 1.0, wl.SOFTMAX_SCALE)
    # The caches differ from bf16(oracle rows) in at most 0.5% of elements, by
    # one bf16 unit (test_cache_write_against_oracle); the scores move far
    # less than the gap band, so the usual recall rule applies, and the
    # oracle's attention runs on its own rows.
    assert recall_check(idx, idx_ref, s64, x["visible_len"]) >= 0.999
    ref_out, ref_lse = oracle_mod.sparse_mla(x["row_cache_base"], x["q_abs"], lb, idx, wl.SOFTMAX_SCALE)
    check_attention(out, lse, ref_out, ref_lse, "written caches")


# ----------------------------------------------------------------------------- paged caches

NAN_BF16 = 0x7FC0


def page_caches(x, seq_base, seq_len, B, seed):
    """Scatter the packed caches of x into pools of B-row blocks: every
    sequence gets a random set of pool blocks (spare blocks interleaved);
    rows no sequence owns hold NaN, so a wrong address poisons the result.
    Returns (key pool, latent pool, block table [S, max_blocks], block-table
    row of each query row)."""
    g = np.random.default_rng(seed)
    nb = [(int(T) + B - 1) // B for T in seq_len]
    total = sum(nb) + sum(nb) // 2 + 3
    perm = g.permutation(total).astype(np.int32)
    bt = np.zeros((len(seq_len), max(nb)), np.int32)
    kpool = np.full((total * B, 128), NAN_BF16, np.uint16)
    lpool = np.full((total * B, 576), NAN_BF16, np.uint16)
    o = 0
    for s_, (b0, T) in enumerate(zip(seq_base, seq_len)):
        blocks = perm[o:o + nb[s_]]
        o += nb[s_]
        bt[s_, :nb[s_]] = blocks
        pos = np.arange(int(T))
        rows = blocks[pos // B].astype(np.int64) * B + pos % B
        kpool[rows] = x["k_idx"][b0:b0 + T]
        lpool[rows] = x["kv_latent"][b0:b0 + T]
    seq_of_row = (np.searchsorted(seq_base, x["row_cache_base"], side="right") - 1).astype(np.int64)
    return kpool, lpool, bt, seq_of_row


def mixed_paged_inputs():
    x = mixed_block_inputs()
    seq_len = np.array([3000, 700, 700, 2100], np.int64)
    seq_base = np.concatenate([[0], np.cumsum(seq_len)[:-1]]).astype(np.int64)
    return x, seq_base, seq_len


@pytest.mark.parametrize("B", [16, 64, 256])
def test_paged_calls_equal_packed_calls(dsa, oracle_mod, B):
    """Indexer (row and shared-block paths), attention and the whole step over
    paged pools give bitwise the results of the packed calls on the same
    logical caches; the pools depage (oracle) back to the packed caches; the
    paged step agrees with the oracle on sampled rows."""
    x, seq_base, seq_len = mixed_paged_inputs()
    kpool, lpool, bt, seq_of_row = page_caches(x, seq_base, seq_len, B, seed=B)
    for s_ in range(len(seq_len)):
        b0, T = int(seq_base[s_]), int(seq_len[s_])
        assert np.array_equal(oracle_mod.depage(lpool, bt[s_], T, B), x["kv_latent"][b0:b0 + T])
        assert np.array_equal(oracle_mod.depage(kpool, bt[s_], T, B), x["k_idx"][b0:b0 + T])
    d = device_inputs(x)
    vis = x["visible_len"]
    R, k = len(vis), 2048
    rows = make_rows(dsa, vis, x["row_cache_base"])
    prow = make_rows(dsa, vis, seq_of_row)
    paged = dsa.Paged(dev(bt), B)
    kp, lp = dev_bf16(kpool), dev_bf16(lpool)
    ld = ld_for(int(vis.max()))
    s_packed = torch.zeros((R, ld), dtype=torch.float32, device=DEV)
    s_paged = torch.zeros((R, ld), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(rows, d["q_idx"], d["w"], d["k_idx"], 1.0, s_packed)
    dsa.dsa_indexer_scores_paged(prow, paged, d["q_idx"], d["w"], kp, 1.0, s_paged)
    torch.cuda.synchronize()
    a, b = s_packed.cpu().numpy(), s_paged.cpu().numpy()
    for r in range(R):
        n = int(vis[r])
        assert np.array_equal(a[r, :n].view(np.uint32), b[r, :n].view(np.uint32)), r
    # attention on one index list, packed vs paged
    idx = run_topk(dsa, vis, a, k)
    di = dev(idx.astype(np.int32))
    outs = []
    for paged_call in (False, True):
        out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
        lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
        if paged_call:
            ws = dsa.workspace(dsa.dsa_sparse_mla_paged_workspace_size(R, k), DEV)
            dsa.dsa_sparse_mla_attn_paged(prow, paged, d["q_abs"], lp, di, k, wl.SOFTMAX_SCALE, out, lse, ws)
        else:
            ws = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, k), DEV)
            dsa.dsa_sparse_mla_attn(rows, d["q_abs"], d["kv_latent"], di, k, wl.SOFTMAX_SCALE, out, lse, ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    # the whole step
    idx_a, out_a, lse_a = run_decode_step(dsa, x, d=d)
    ws = dsa.workspace(dsa.dsa_decode_step_paged_workspace_size(R, int(vis.max()), k), DEV)
    ws.fill_(255)
    idx_b = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out_b = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse_b = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    dsa.dsa_decode_step_paged(prow, paged, d["q_idx"], d["w"], kp, wl.INDEX_SCALE, d["q_abs"], lp, wl.SOFTMAX_SCALE,
                              k, idx_b, out_b, lse_b, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx_a, idx_b.cpu().numpy())
    assert np.array_equal(out_a.view(np.uint32), out_b.cpu().numpy().view(np.uint32))
    assert np.array_equal(lse_a.view(np.uint32), lse_b.cpu().numpy().view(np.uint32))
    # and against the oracle on sampled rows, from the depaged caches
    rs = [0, 31, 40, 64, 68]
    y = sub(x, rs)
    s64, _, idx_ref, out_ref, lse_ref = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"],
                                                               y["w"], y["k_idx"], y["q_abs"], y["kv_latent"], k, 1.0,
                                                               wl.SOFTMAX_SCALE)
    assert recall_check(idx_a[rs], idx_ref, s64, y["visible_len"]) >= 0.999
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], idx_a[rs],
                                             wl.SOFTMAX_SCALE)
    check_attention(out_b.cpu().numpy()[rs], lse_b.cpu().numpy()[rs], ref_out, ref_lse, f"paged B={B}")


def test_cache_writer_fills_paged_pools_for_the_paged_step(dsa, oracle_mod):
    """The next-row pieces together: dsa_cache_write scatters three sequences'
    new tokens into block-scattered pools (slots = pool rows from the block
    table), then dsa_decode_step_paged runs over those pools.  It must equal,
    bit for bit, the packed step over packed caches written by the same
    writer, and agree with the oracle's attention over the oracle's own cache
    rows."""
    B = 64
    lens = np.array([3000, 2048, 777], np.int64)
    S = len(lens)
    seq_base = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    T = int(lens.sum())
    c = wl.cache_write_inputs(T, seed=13, cache_rows=T)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    c["positions"] = pos
    nb = [(int(L) + B - 1) // B for L in lens]
    nblk = sum(nb) + 5
    perm = np.random.default_rng(3).permutation(nblk).astype(np.int32)
    bt = np.zeros((S, max(nb)), np.int32)
    o = 0
    for i in range(S):
        bt[i, :nb[i]] = perm[o:o + nb[i]]
        o += nb[i]
    seq_of_tok = np.repeat(np.arange(S), lens)
    pool_rows = bt[seq_of_tok, pos // B].astype(np.int64) * B + pos % B
    # packed caches and pools, both written by the cache writer
    c["slots"] = np.arange(T, dtype=np.int64)
    kc_packed, lc_packed = run_cache_write(dsa, c, 1e6)
    c["slots"] = pool_rows
    c["cache_rows"] = nblk * B
    kpool, lpool = run_cache_write(dsa, c, 1e6)
    # one decode row per sequence (sees the whole sequence)
    q = wl.decode(S, 1, seed=21).generate(with_caches=False)
    vis = lens.astype(np.int32)
    R, k = S, 2048
    x = dict(q_idx=q["q_idx"], w=q["w"], q_abs=q["q_abs"], visible_len=vis, row_cache_base=seq_base,
             k_idx=kc_packed, kv_latent=lc_packed)
    idx_a, out_a, lse_a = run_decode_step(dsa, x)
    d = device_inputs(x)
    prow = make_rows(dsa, vis, np.arange(S, dtype=np.int64))
    paged = dsa.Paged(dev(bt), B)
    ws = dsa.workspace(dsa.dsa_decode_step_paged_workspace_size(R, int(vis.max()), k), DEV)
    idx_b = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out_b = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse_b = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    dsa.dsa_decode_step_paged(prow, paged, d["q_idx"], d["w"], dev_bf16(kpool), wl.INDEX_SCALE, d["q_abs"],
                              dev_bf16(lpool), wl.SOFTMAX_SCALE, k, idx_b, out_b, lse_b, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx_a, idx_b.cpu().numpy())
    assert np.array_equal(out_a.view(np.uint32), out_b.cpu().numpy().view(np.uint32))
    assert np.array_equal(lse_a.view(np.uint32), lse_b.cpu().numpy().view(np.uint32))
    # every token's rows sit at its block-table slot of the pools
    assert np.array_equal(lpool[pool_rows], lc_packed) and np.array_equal(kpool[pool_rows], kc_packed)
    # the oracle attends over its own cache rows (bf16-rounded) on the GPU's lists
    _, lat = oracle_mod.cache_rows(c["hidden"], c["wk"], c["k_norm_weight"], c["k_norm_bias"], 1e-6, c["kv_a"],
                                   c["kv_norm_weight"], 1e-5, pos.astype(np.int64), 1e6)
    lb = wl.f32_to_bf16_bits(lat.astype(np.float32))
    ref_out, ref_lse = oracle_mod.sparse_mla(seq_base, q["q_abs"], lb, idx_a, wl.SOFTMAX_SCALE)
    check_attention(out_b.cpu().numpy(), lse_b.cpu().numpy(), ref_out, ref_lse, "written paged pools")


def test_paged_decode_step_full_size_equals_packed(dsa):
    """64 sequences x 32,768 positions in 64-row blocks scattered over the
    pool: the paged step gives bitwise the packed step's selection, output
    and LSE."""
    w, x = inputs("c3")
    B = 64
    kpool, lpool, bt, seq_of_row = page_caches(x, w.seq_base, w.seq_len, B, seed=3)
    d = device_inputs(x)
    vis = x["visible_len"]
    R, k = len(vis), 2048
    idx_a, out_a, lse_a = run_decode_step(dsa, x, d=d)
    prow = make_rows(dsa, vis, seq_of_row, flags=dsa.ROWS_DISTINCT_SEQUENCES)
    paged = dsa.Paged(dev(bt), B)
    ws = dsa.workspace(dsa.dsa_decode_step_paged_workspace_size(R, int(vis.max()), k), DEV)
    idx_b = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out_b = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse_b = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    dsa.dsa_decode_step_paged(prow, paged, d["q_idx"], d["w"], dev_bf16(kpool), wl.INDEX_SCALE, d["q_abs"],
                              dev_bf16(lpool), wl.SOFTMAX_SCALE, k, idx_b, out_b, lse_b, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx_a, idx_b.cpu().numpy())
    assert np.array_equal(out_a.view(np.uint32), out_b.cpu().numpy().view(np.uint32))
    assert np.array_equal(lse_a.view(np.uint32), lse_b.cpu().numpy().view(np.uint32))


def test_decode_step_chunk_boundaries_packed_and_paged(dsa, oracle_mod):
    """A host bound max_visible far above the rows' lengths (1,000,000) makes
    each fp32 score row 4 MB, so the fused step takes 256 rows at a time: 300
    rows split into chunks of 256 and 44.  Rows 0..255 are a prefill chunk on
    one sequence (shared 32-row blocks), rows 256..299 decode rows on their own
    sequences.  The packed and the paged step equal, bit for bit, the separate
    calls over all rows at once, and sampled rows on both sides of the chunk
    boundary agree with the oracle."""
    T0 = 4000
    dec = [2500, 1, 2049, 4097, 3333, 100, 2048, 5000] * 5 + [777, 3000, 4100, 1500]
    vis = np.concatenate([np.arange(T0 - 255, T0 + 1), dec]).astype(np.int32)
    seq_len = np.array([T0] + dec, np.int64)
    seq_base = np.concatenate([[0], np.cumsum(seq_len)[:-1]]).astype(np.int64)
    base = np.concatenate([np.zeros(256), seq_base[1:]]).astype(np.int64)
    row_seq = np.concatenate([np.zeros(256), np.arange(1, len(dec) + 1)]).astype(np.int64)
    w = wl.Workload(name="chunks", seed=29, visible_len=vis, row_cache_base=base, seq_len=seq_len,
                    seq_base=seq_base, row_seq=row_seq)
    x = w.generate()
    d = device_inputs(x)
    R, k, maxv = len(vis), 2048, 1_000_000
    rows = dsa.Rows(dev(vis), dev(base), maxv)
    ws_bytes = dsa.dsa_decode_step_workspace_size(R, maxv, k)
    assert 256 * 4 * maxv <= ws_bytes < 300 * 4 * maxv  # 256 score rows at a time
    idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
    ws = dsa.workspace(ws_bytes, DEV)
    ws.fill_(255)
    dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv_latent"],
                        wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
    # separate calls, all rows at once
    scores = torch.empty((R, maxv), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, scores)
    idx_b = torch.empty_like(idx)
    dsa.dsa_topk_select(rows, scores, k, idx_b, dsa.workspace(dsa.dsa_topk_workspace_size(R, maxv, k), DEV))
    out_b, lse_b = torch.empty_like(out), torch.empty_like(lse)
    dsa.dsa_sparse_mla_attn(rows, d["q_abs"], d["kv_latent"], idx_b, k, wl.SOFTMAX_SCALE, out_b, lse_b,
                            dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, k), DEV))
    torch.cuda.synchronize()
    del scores
    assert torch.equal(idx, idx_b)
    assert torch.equal(out.view(torch.int32), out_b.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse_b.view(torch.int32))
    # the paged step over 64-position blocks
    B = 64
    kpool, lpool, bt, seq_of_row = page_caches(x, seq_base, seq_len, B, seed=29)
    bt_wide = np.zeros((bt.shape[0], (maxv + B - 1) // B), np.int32)
    bt_wide[:, :bt.shape[1]] = bt
    prow = dsa.Rows(dev(vis), dev(seq_of_row), maxv)
    idx_p = torch.empty_like(idx)
    out_p, lse_p = torch.empty_like(out), torch.empty_like(lse)
    dsa.dsa_decode_step_paged(prow, dsa.Paged(dev(bt_wide), B), d["q_idx"], d["w"], dev_bf16(kpool), wl.INDEX_SCALE,
                              d["q_abs"], dev_bf16(lpool), wl.SOFTMAX_SCALE, k, idx_p, out_p, lse_p,
                              dsa.workspace(dsa.dsa_decode_step_paged_workspace_size(R, maxv, k), DEV))
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_p)
    assert torch.equal(out.view(torch.int32), out_p.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse_p.view(torch.int32))
    # oracle on rows around the boundary
    pick = [0, 254, 255, 256, 257, 259, 299]
    y = sub(x, pick)
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                   y["k_idx"], y["q_abs"], y["kv_latent"], k, 1.0, wl.SOFTMAX_SCALE)
    idx_h = idx.cpu().numpy()
    assert recall_check(idx_h[pick], idx_ref, s64, y["visible_len"]) >= 0.999
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], idx_h[pick],
                                             wl.SOFTMAX_SCALE)
    check_attention(out[pick].cpu().numpy(), lse[pick].cpu().numpy(), ref_out, ref_lse, "chunk boundary")


# ----------------------------------------------------------------------------- IndexShare

def _random_batch(seed):
    """A random decode batch: 1-39 decode rows with log-uniform lengths
    (1..12,000, each seeing its whole sequence) and, in most batches, a causal
    chunk of 1-89 rows on a 0-4,999-position history, inserted as one
    contiguous run at a random place (so shared 32-row blocks start at any
    offset).  Returns the workload and its per-row sequence index."""
    g = np.random.default_rng(1000 + seed)
    n_dec = int(g.integers(1, 40))
    dec = np.floor(np.exp(g.uniform(0.0, np.log(12000.0), size=n_dec))).astype(np.int64)
    chunk = int(g.integers(0, 90)) if seed % 3 else 0
    hist = int(g.integers(0, 5000))
    seq_len = np.array(list(dec) + ([hist + chunk] if chunk else []), np.int64)
    seq_base = np.concatenate([[0], np.cumsum(seq_len)[:-1]]).astype(np.int64)
    at = int(g.integers(0, n_dec + 1))
    vis = list(dec[:at]) + list(range(hist + 1, hist + chunk + 1)) + list(dec[at:])
    rseq = list(range(at)) + [n_dec] * chunk + list(range(at, n_dec))
    rseq = np.array(rseq, np.int64)
    w = wl.Workload(name=f"rand{seed}", seed=40 + seed, visible_len=np.array(vis, np.int32),
                    row_cache_base=seq_base[rseq], seq_len=seq_len, seq_base=seq_base, row_seq=rseq,
                    description="random batch")
    return w, seq_base, seq_len, chunk


@pytest.mark.parametrize("seed", list(range(6)))
def test_decode_step_random_batches(dsa, oracle_mod, seed):
    """Random batches through the fused step, packed and over a paged pool
    (random block size): the two agree bit for bit; rows with n <= k select
    0..n-1; sampled rows agree with the oracle (recall with near-threshold
    swaps only, attention on the GPU's own lists)."""
    w, seq_base, seq_len, chunk = _random_batch(seed)
    g = np.random.default_rng(2000 + seed)
    k = int(g.choice([1, 64, 300, 2048]))
    iscale = float(g.choice([1.0, 0.5]))
    B = int(g.choice([16, 64, 256]))
    x = w.generate()
    d = device_inputs(x)
    vis, base = x["visible_len"], x["row_cache_base"]
    R = len(vis)
    flags = 0 if chunk else dsa.ROWS_DISTINCT_SEQUENCES
    rows = make_rows(dsa, vis, base, flags)

    def outs():
        return (torch.empty((R, k), dtype=torch.int32, device=DEV),
                torch.empty((R, 64, 512), dtype=torch.float32, device=DEV),
                torch.empty((R, 64), dtype=torch.float32, device=DEV))

    idx_a, out_a, lse_a = outs()
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
    dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], iscale, d["q_abs"], d["kv_latent"],
                        wl.SOFTMAX_SCALE, k, idx_a, out_a, lse_a, ws)
    kpool, lpool, bt, seq_of_row = page_caches(x, seq_base, seq_len, B, seed=seed)
    prow = make_rows(dsa, vis, seq_of_row, flags)
    idx_b, out_b, lse_b = outs()
    ws = dsa.workspace(dsa.dsa_decode_step_paged_workspace_size(R, int(vis.max()), k), DEV)
    dsa.dsa_decode_step_paged(prow, dsa.Paged(dev(bt), B), d["q_idx"], d["w"], dev_bf16(kpool), iscale, d["q_abs"],
                              dev_bf16(lpool), wl.SOFTMAX_SCALE, k, idx_b, out_b, lse_b, ws)
    torch.cuda.synchronize()
    idx_h, out_h, lse_h = idx_a.cpu().numpy(), out_a.cpu().numpy(), lse_a.cpu().numpy()
    assert np.array_equal(idx_h, idx_b.cpu().numpy())
    assert np.array_equal(out_h.view(np.uint32), out_b.cpu().numpy().view(np.uint32))
    assert np.array_equal(lse_h.view(np.uint32), lse_b.cpu().numpy().view(np.uint32))
    for r in range(R):
        n = int(vis[r])
        if n <= k:
            assert np.array_equal(idx_h[r], np.where(np.arange(k) < n, np.arange(k), -1)), r
    rs = sorted(set(g.choice(R, size=min(R, 10), replace=False).tolist()) | {0, R - 1})
    y = sub(x, rs)
    s64, _, idx_ref, _, _ = oracle_mod.decode_step(y["visible_len"], y["row_cache_base"], y["q_idx"], y["w"],
                                                   y["k_idx"], y["q_abs"], y["kv_latent"], k, iscale,
                                                   wl.SOFTMAX_SCALE)
    assert recall_check(idx_h[rs], idx_ref, s64, y["visible_len"], k) >= 0.999
    ref_out, ref_lse = oracle_mod.sparse_mla(y["row_cache_base"], y["q_abs"], y["kv_latent"], idx_h[rs],
                                             wl.SOFTMAX_SCALE)
    check_attention(out_h[rs], lse_h[rs], ref_out, ref_lse, f"random batch {seed}")


def test_index_share_cold_start_block_and_first_period(dsa, oracle_mod):
    """Layers 0..9 of the GLM-5.2 pattern (3 full, 3 shared, 1 full, 3 shared;
    the schedule comes from dsa_index_share_source) over a decode batch with
    rows longer than, equal to and shorter than k.  Full layers run
    dsa_decode_step into one shared index buffer; shared layers run
    dsa_sparse_mla_attn on that buffer with their own queries and cache.
    Checks: the buffer is untouched by shared layers; each full layer's list
    against the oracle's selection (recall, near-threshold swaps only); every
    layer's attention against the oracle on the list it used, and against the
    oracle's whole IndexShare composition for rows whose lists agree."""
    lengths = [5000, 2048, 3001, 700]
    L = 10
    layers = wl.layer_stack(lengths, L, seed=6)
    vis, base = layers[0]["visible_len"], layers[0]["row_cache_base"]
    R, k = len(vis), 2048
    types = ["full" if dsa.dsa_index_share_source(l) == l else "shared" for l in range(L)]
    assert types == oracle_mod.GLM52_INDEXER_TYPES[:L]
    rows = make_rows(dsa, vis, base)
    idx = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
    ws_a = dsa.workspace(dsa.dsa_sparse_mla_workspace_size(R, k), DEV)
    got = []
    for l, x in enumerate(layers):
        d = device_inputs(x)
        out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
        lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)
        if types[l] == "full":
            dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv_latent"],
                                wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
            torch.cuda.synchronize()
            snap = idx.clone()
        else:
            dsa.dsa_sparse_mla_attn(rows, d["q_abs"], d["kv_latent"], idx, k, wl.SOFTMAX_SCALE, out, lse, ws_a)
            torch.cuda.synchronize()
            assert torch.equal(idx, snap), l
        got.append((snap.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()))
    ref = oracle_mod.index_share_layers(types, layers, vis, base, k, wl.INDEX_SCALE, wl.SOFTMAX_SCALE)
    for l in range(L):
        idx_g, out_g, lse_g = got[l]
        idx_r, out_r, lse_r = ref[l]
        x = layers[l]
        if types[l] == "full":
            s64 = oracle_mod.indexer_scores(vis, base, x["q_idx"], x["w"], x["k_idx"], wl.INDEX_SCALE)
            assert recall_check(idx_g, idx_r, s64, vis) >= 0.999, l
        on_own = oracle_mod.sparse_mla(base, x["q_abs"], x["kv_latent"], idx_g, wl.SOFTMAX_SCALE)
        check_attention(out_g, lse_g, on_own[0], on_own[1], f"layer {l} ({types[l]})")
        same = [r for r in range(R) if np.array_equal(idx_g[r], idx_r[r])]
        assert len(same) >= R - 1, (l, same)
        check_attention(out_g[same], lse_g[same], out_r[same], lse_r[same], f"layer {l} vs oracle composition")


# ----------------------------------------------------------------------------- projections

U32 = 2.0 ** -24  # fp32 unit roundoff


@pytest.mark.parametrize("R", [1, 5, 64, 130, 1000, 1024])
def test_absorb_queries_against_oracle(dsa, oracle_mod, R):
    """q_abs = [W_UK^T q_nope || q_pe]: the 512 absorbed columns within the
    error of fp32 accumulation over 192 products plus one bf16 rounding
    (at most 2^-8 |ref|: half an ulp of an 8-bit significand); the RoPE
    part copied bit for bit.  R = 5, 130 leave ragged row tiles; R = 1000 and
    1024 take the 256-column tiles (1000 with a ragged last row tile) and make
    each workgroup walk several row tiles."""
    x = wl.projection_inputs(R, seed=5 + R)
    qa = torch.empty((R, 64, 576), dtype=torch.bfloat16, device=DEV)
    dsa.dsa_absorb_queries(dev_bf16(x["q_nope"]), dev_bf16(x["q_pe"]), dev_bf16(x["kv_b"]), qa)
    torch.cuda.synchronize()
    got_bits = qa.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle_mod.absorb_queries(x["q_nope"], x["q_pe"], x["kv_b"])
    got = wl.bf16_bits_to_f32(got_bits).astype(np.float64)
    W = np.abs(wl.bf16_bits_to_f32(x["kv_b"][:, :192, :]).astype(np.float64))          # [64,192,512]
    qn = np.abs(wl.bf16_bits_to_f32(x["q_nope"]).astype(np.float64))                   # [R,64,192]
    mag = np.matmul(qn.transpose(1, 0, 2), W).transpose(1, 0, 2)                        # sum of |terms|
    bound = 2.0 ** -8 * np.abs(ref[:, :, :512]) + 192 * U32 * mag * 1.01
    assert np.all(np.abs(got[:, :, :512] - ref[:, :, :512]) <= bound)
    assert np.array_equal(got_bits[:, :, 512:], x["q_pe"])
    # and (up to accumulation-order flips at rounding ties) the bf16 rounding of the fp64 result
    same = got_bits[:, :, :512] == wl.f32_to_bf16_bits(ref[:, :, :512].astype(np.float32))
    assert same.mean() >= 0.999


@pytest.mark.parametrize("R", [1, 5, 64, 130, 1024])
def test_v_up_proj_against_oracle(dsa, oracle_mod, R):
    """out = W_UV bf16(o): within the fp32 accumulation bound over 512
    products, element by element (o rounded to bf16 the same way on both
    sides: round-to-nearest-even)."""
    x = wl.projection_inputs(R, seed=50 + R)
    out = torch.empty((R, 64, 256), dtype=torch.float32, device=DEV)
    dsa.dsa_v_up_proj(dev(x["o"]), dev_bf16(x["kv_b"]), out)
    torch.cuda.synchronize()
    ob = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x["o"])).astype(np.float64)
    ref = oracle_mod.v_up_proj(ob, x["kv_b"])
    W = np.abs(wl.bf16_bits_to_f32(x["kv_b"][:, 192:, :]).astype(np.float64))          # [64,256,512]
    mag = np.matmul(np.abs(ob).transpose(1, 0, 2), W.transpose(0, 2, 1)).transpose(1, 0, 2)
    assert np.all(np.abs(out.cpu().numpy() - ref) <= 512 * U32 * mag * 1.01 + 1e-30)
