"""HIP path vs the oracle on the five synthetic workloads at full size, in the
launch configuration the benchmark times (default split size, one decode call).
Where the oracle would be slow (the Qwen and paged workloads), a seeded sample of
query heads that covers every sequence and every KV head is checked one by one;
the Llama-shaped and batched workloads are checked on every head."""
import random

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


def _sample_heads(w, per_pair=1, seed=0):
    rng = random.Random(seed)
    heads = []
    for b in range(w.batch):
        for g in range(w.kv_heads):
            for h in rng.sample(range(g * w.group, (g + 1) * w.group), per_pair):
                heads.append((b, h))
    return heads


def _run(name, S, mode, heads=None, x=None):
    w = W.WORKLOADS[name]
    print(f"[case] {name} S={S} mode={W.MODE_NAMES[mode]}", flush=True)
    if x is None:
        x = W.make_inputs(w, seed=0, device="cuda")
    o, idx, _, shape = H.run_hip(x, S, mode, seed=w.sample_seed)
    rep = H.check_all(x, S, mode, w.sample_seed, o, idx, heads=heads)
    print(f"  {rep} unique_v_rows={H.unique_v_rows(idx, w.group)}", flush=True)
    return x


def test_llama32k_systematic():
    _run("llama32k", 256, W.MODE_SYSTEMATIC)


def test_batched_stratified():
    x = _run("batched", 128, W.MODE_STRATIFIED)
    _run("batched", 512, W.MODE_STRATIFIED, x=x)


@pytest.mark.parametrize("mode", [W.MODE_MULTINOMIAL, W.MODE_STRATIFIED, W.MODE_SYSTEMATIC])
def test_qwen128k_all_modes(mode):
    w = W.WORKLOADS["qwen128k"]
    _run("qwen128k", 1024, mode, heads=_sample_heads(w, per_pair=2, seed=mode))


def test_paged_systematic():
    """Every sequence and KV head of the paged workload, one seeded query head each."""
    w = W.WORKLOADS["paged"]
    _run("paged", 256, W.MODE_SYSTEMATIC, heads=_sample_heads(w, per_pair=1, seed=7))
    torch.cuda.empty_cache()
