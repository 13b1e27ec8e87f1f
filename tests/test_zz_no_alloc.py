"""dsa_decode_step_noalloc (the fused step over the library's own scratch
array, for callers that cannot allocate) against dsa_decode_step, through the
C ABI: bit-for-bit equal outputs on two calls in a row, the second smaller,
then a call whose score rows exceed the scratch and are taken in chunks; and
the call captured in a HIP graph (it allocates nothing, so it can be), whose
replays equal the eager call."""
import numpy as np
import pytest
import torch

from sparse_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _run(dsa, x, noalloc, k=2048):
    vis, base = x["visible_len"], x["row_cache_base"]
    R = len(vis)
    rows = dsa.Rows(torch.from_numpy(vis).to(DEV), torch.from_numpy(base).to(DEV), int(vis.max()))
    d = dict(q_idx=_dev_bf16(x["q_idx"]), w=torch.from_numpy(x["w"]).to(DEV), k_idx=_dev_bf16(x["k_idx"]),
             q_abs=_dev_bf16(x["q_abs"]), kv=_dev_bf16(x["kv_latent"]))
    # outputs start as garbage, so every element must be written
    idx = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    out = torch.full((R, 64, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((R, 64), float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        dsa.dsa_decode_step_noalloc(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv"],
                                    wl.SOFTMAX_SCALE, k, idx, out, lse)
    else:
        ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(R, int(vis.max()), k), DEV)
        dsa.dsa_decode_step(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv"],
                            wl.SOFTMAX_SCALE, k, idx, out, lse, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def _same(a, b):
    for u, v in zip(a, b):
        assert u.shape == v.shape
        assert np.array_equal(u.view(np.uint32) if u.dtype == np.float32 else u,
                              v.view(np.uint32) if v.dtype == np.float32 else v)


def test_noalloc_step_equals_decode_step(dsa):
    print("[noalloc] 64 x 32768 decode batch", flush=True)
    big = wl.config("c3").generate()
    _same(_run(dsa, big, True), _run(dsa, big, False))
    print("[noalloc] second, smaller call: ragged 5 rows", flush=True)
    small = wl._decode("na", 17, [3000, 1, 2048, 40000, 777], "noalloc small").generate()
    _same(_run(dsa, small, True), _run(dsa, small, False))
    print("[noalloc] prefill 8192 rows: 256 MiB of score rows, taken 32-row multiples at a time", flush=True)
    pre = wl.config("c2").generate()
    a = _run(dsa, pre, True)
    _same(a, _run(dsa, pre, False))
    # and the first call's inputs again, after the array held other contents
    _same(_run(dsa, big, True), _run(dsa, big, False))


def test_noalloc_rejects_rows_the_scratch_cannot_hold(dsa):
    # 32 score rows of 1,100,000 positions alone take 140.8 MB of the 128 MiB
    R, maxv = 64, 1100000
    vis = torch.full((R,), maxv, dtype=torch.int32, device=DEV)
    base = torch.zeros(R, dtype=torch.int64, device=DEV)
    rows = dsa.Rows(vis, base, maxv)
    t = lambda n, dt=torch.float32: torch.zeros(n, dtype=dt, device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_decode_step_noalloc(rows, t(R * 32 * 128, torch.bfloat16), t(R * 32), t(maxv * 128, torch.bfloat16),
                                    1.0, t(R * 64 * 576, torch.bfloat16), t(maxv * 576, torch.bfloat16), 0.0625,
                                    2048, t(R * 2048, torch.int32), t(R * 64 * 512), t(R * 64))
    assert e.value.status == 1 and "scratch" in e.value.detail


def test_noalloc_step_replays_from_a_graph(dsa):
    x = wl.decode(16, 5000, seed=11).generate()
    vis, base = x["visible_len"], x["row_cache_base"]
    R, k = len(vis), 2048
    rows = dsa.Rows(torch.from_numpy(vis).to(DEV), torch.from_numpy(base).to(DEV), int(vis.max()))
    d = dict(q_idx=_dev_bf16(x["q_idx"]), w=torch.from_numpy(x["w"]).to(DEV), k_idx=_dev_bf16(x["k_idx"]),
             q_abs=_dev_bf16(x["q_abs"]), kv=_dev_bf16(x["kv_latent"]))
    idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
    out = torch.empty((R, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((R, 64), dtype=torch.float32, device=DEV)

    def step():
        dsa.dsa_decode_step_noalloc(rows, d["q_idx"], d["w"], d["k_idx"], wl.INDEX_SCALE, d["q_abs"], d["kv"],
                                    wl.SOFTMAX_SCALE, k, idx, out, lse)

    step()
    torch.cuda.synchronize()
    ref = (idx.cpu().numpy(), out.cpu().numpy().view(np.uint32), lse.cpu().numpy().view(np.uint32))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: clobber the outputs
        idx.fill_(-5)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref[0]), rep
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref[1]), rep
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref[2]), rep
