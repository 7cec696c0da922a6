"""santa_decode_noalloc (the entry point for callers that cannot allocate) against
santa_decode with a caller workspace, through the C ABI: two calls in a row, the
second on a smaller problem, then a multinomial call (which uses the scratch
array's sorted-target region), each compared index for index and within the
parity bar on o, and each also checked against the oracle."""
import pytest
import torch

import sampling_sparse_attention_amd as santa
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    santa.library()


def _inputs(batch, G, kv_heads, n, lens, seed):
    w = W.Workload("noalloc", batch=batch, q_heads=G * kv_heads, kv_heads=kv_heads, head_dim=128, seq_len=n,
                   sinks=2, sink_scale=6.0)
    x = W.make_inputs(w, seed=seed)
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    return H.to_device(x)


def _compare(x, S, mode, seed):
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
    B, Hq, d = x["q"].shape
    o_n = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    i_n = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
    print(f"[case] noalloc B={B} Hq={Hq} n={x['workload'].seq_len} S={S} mode={mode}", flush=True)
    santa.santa_decode_noalloc(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, seed, o_n, i_n)
    o_w, i_w, ws, _ = H.run_hip(x, S, mode, seed)
    assert santa.santa_noalloc_status() == 0
    assert santa.santa_workspace_status(ws) == 0
    assert torch.equal(i_n.cpu(), i_w)
    err = float((o_n.cpu().double() - o_w.double()).norm() / o_w.double().norm())
    assert err <= H.O_REL_L2, err
    H.check_all(x, S, mode, seed, o_n.cpu(), i_n.cpu())


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    assert santa.santa_noalloc_scratch_bytes() == 64 << 20
    big = _inputs(batch=2, G=4, kv_heads=8, n=8192, lens=(8192, 5000), seed=1)
    _compare(big, 256, W.MODE_SYSTEMATIC, seed=3)
    small = _inputs(batch=1, G=4, kv_heads=2, n=1000, lens=(777,), seed=2)
    _compare(small, 64, W.MODE_STRATIFIED, seed=4)
    _compare(small, 96, W.MODE_MULTINOMIAL, seed=5)
    _compare(big, 128, W.MODE_MULTINOMIAL, seed=6)


def test_noalloc_refuses_a_problem_larger_than_its_scratch():
    w = W.WORKLOADS["paged"]
    shape = santa.Shape(w.batch, w.q_heads, w.kv_heads, w.head_dim, w.seq_len, 16, w.pages_per_seq,
                        w.num_pages, 0, 0, 16 * w.kv_heads * w.head_dim, w.kv_heads * w.head_dim, w.head_dim)
    assert santa.santa_workspace_size(shape, 256, 2) > santa.santa_noalloc_scratch_bytes()
    fake = torch.empty(0, device="cuda")
    lib = santa.library()
    import ctypes
    p = ctypes.c_void_p(fake.data_ptr() or 1 << 20)
    st = lib.santa_decode_noalloc(ctypes.byref(shape), p, p, p, p, p, 256, 2, ctypes.c_uint64(0), p, p, None)
    assert st == 3, lib.santa_last_error().decode()
    assert "scratch array holds" in lib.santa_last_error().decode()
