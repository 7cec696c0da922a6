"""santa_decode_flash (S^2ANTA-flash, section 3.3 of the SANTA page) against the
oracle's per-head flash sampling (sample_head_flash) and deferred-normalisation
merge (estimate_flash), both pinned on the CPU: small seeded inputs spanning several tiles and ragged
tails, every rule and shape the kernel is built for, budgets from one sample per
tile to several chunks of 256 per tile, and the workloads at full size (sampled
heads).  Every call goes through the C ABI."""
import random

import pytest
import torch

import sampling_sparse_attention_amd as santa
import workloads as W
from tests import gpu_helpers as H
from tests.test_gpu_parity import _inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    santa.library()


def _check(x, S, mode, seed=3, split=0, heads=None):
    o, idx, ws, tile = H.run_flash(x, S, mode, seed, split=split)
    rep = H.check_flash(x, S, mode, seed, tile, o, idx, heads=heads)
    print(f"  tile={tile} {rep}", flush=True)
    assert santa.workspace_error(ws) == 0
    assert torch.count_nonzero(ws) == 0
    return o, idx


@pytest.mark.parametrize("G", [4, 7])
@pytest.mark.parametrize("per_tile", [32, 33])
@pytest.mark.parametrize("mode", [W.MODE_STRATIFIED, W.MODE_SYSTEMATIC])
def test_flash_sampler_paths_at_the_few_target_limit(per_tile, mode, G):
    """Four 512-key tiles with S = 4 * per_tile: each tile samples per_tile
    targets, one per lane up to 32 and by per-key counts above; with 7 heads
    on four waves, up to 32 a wave samples its two heads before one gather of
    both, above that one head after the other."""
    _check(_inputs(G=G, lens=(2048,), q_scale=0.0, sinks=0), 4 * per_tile, mode, split=512)


@pytest.mark.parametrize("mode", [W.MODE_STRATIFIED, W.MODE_SYSTEMATIC])
@pytest.mark.parametrize("S", [32, 100, 300])
def test_flash_small_bf16_gqa4(mode, S):
    _check(_inputs(), S, mode)


@pytest.mark.parametrize("G,d,dtype,page", [(1, 64, "f32", 0), (2, 128, "bf16", 16), (7, 128, "bf16", 0),
                                            (8, 64, "bf16", 32), (4, 128, "f32", 16)])
def test_flash_shapes(G, d, dtype, page):
    x = _inputs(G=G, d=d, dtype=dtype, lens=(1000, 1537, 333), page_size=page)
    for mode in (W.MODE_STRATIFIED, W.MODE_SYSTEMATIC):
        _check(x, 128, mode, seed=17)


@pytest.mark.parametrize("split", [64, 128, 512, 1024])
def test_flash_split_sizes(split):
    x = _inputs(lens=(2049, 700, 1))
    T = -(-2049 // split)
    for S in (T, 3 * T + 1):             # one sample per tile, then a ragged budget
        _check(x, S, W.MODE_SYSTEMATIC, split=split)
        _check(x, S, W.MODE_STRATIFIED, split=split)


def test_flash_several_chunks_per_tile():
    """Budgets above 256 per tile are sampled in chunks of 256 targets."""
    x = _inputs(lens=(3000, 2500))
    for mode in (W.MODE_STRATIFIED, W.MODE_SYSTEMATIC):
        _check(x, 2000, mode, split=1024)


def test_flash_empty_and_tiny_sequences():
    x = _inputs(lens=(0, 1, 2, 513, 0))
    for mode in (W.MODE_STRATIFIED, W.MODE_SYSTEMATIC):
        _check(x, 64, mode)


def test_flash_dominant_sink():
    """A sink that holds almost all of its tile's mass takes all of that tile's samples."""
    x = _inputs(lens=(4096, 1500), q_scale=3.0, sinks=4)
    o, idx = _check(x, 128, W.MODE_SYSTEMATIC)


def test_flash_repeatable_and_seeded():
    x = _inputs(lens=(2000, 1777))
    _, a = _check(x, 96, W.MODE_SYSTEMATIC, seed=21)
    _, b = _check(x, 96, W.MODE_SYSTEMATIC, seed=21)
    _, c = _check(x, 96, W.MODE_SYSTEMATIC, seed=22)
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_flash_workspace_shared_with_santa_calls():
    """Flash and SANTA calls of different shapes in a row on one workspace."""
    xa = _inputs(lens=(2049, 700, 1))
    xb = _inputs(G=1, d=64, dtype="f32", lens=(300, 0, 1500))
    big = max(santa.santa_workspace_size(santa.make_shape(x["q"], x["k"], None,
                                                          max_seq_len=x["workload"].seq_len), 128, 2)
              for x in (xa, xb))
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    santa.santa_workspace_init(ws)
    for rep in range(2):
        for x in (xa, xb):
            o, idx, _, tile = H.run_flash(x, 128, W.MODE_SYSTEMATIC, 5 + rep, workspace=ws)
            H.check_flash(x, 128, W.MODE_SYSTEMATIC, 5 + rep, tile, o, idx)
            shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
            B, Hq, d = x["q"].shape
            o2 = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
            i2 = torch.empty((B, Hq, 128), dtype=torch.int32, device="cuda")
            santa.santa_decode(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, 128, W.MODE_SYSTEMATIC,
                               5 + rep, o2, i2, ws)
            torch.cuda.synchronize()
            H.check_all(x, 128, W.MODE_SYSTEMATIC, 5 + rep, o2.cpu(), i2.cpu())
    assert santa.workspace_error(ws) == 0
    assert torch.count_nonzero(ws) == 0


def _sample_heads(w, per_pair, seed):
    rng = random.Random(seed)
    return [(b, h) for b in range(w.batch) for g in range(w.kv_heads)
            for h in rng.sample(range(g * w.group, (g + 1) * w.group), per_pair)]


def _full(name, S, mode, heads=None):
    w = W.WORKLOADS[name]
    print(f"[case] flash {name} S={S} mode={W.MODE_NAMES[mode]}", flush=True)
    x = W.make_inputs(w, seed=0, device="cuda")
    o, idx, ws, tile = H.run_flash(x, S, mode, w.sample_seed)
    rep = H.check_flash(x, S, mode, w.sample_seed, tile, o, idx, heads=heads)
    print(f"  tile={tile} {rep} unique_v_rows={H.unique_v_rows(idx, w.group)}", flush=True)
    assert santa.workspace_error(ws) == 0
    del x
    torch.cuda.empty_cache()


def test_flash_llama32k():
    w = W.WORKLOADS["llama32k"]
    _full("llama32k", 256, W.MODE_SYSTEMATIC, heads=_sample_heads(w, 2, 1))
    _full("llama32k", 2048, W.MODE_SYSTEMATIC, heads=_sample_heads(w, 1, 2))


def test_flash_qwen128k_stratified():
    w = W.WORKLOADS["qwen128k"]
    _full("qwen128k", 1024, W.MODE_STRATIFIED, heads=_sample_heads(w, 1, 3))


def test_flash_paged():
    w = W.WORKLOADS["paged"]
    rng = random.Random(9)
    heads = [(b, rng.randrange(w.q_heads)) for b in rng.sample(range(w.batch), 16)]
    _full("paged", 256, W.MODE_SYSTEMATIC, heads=heads)
