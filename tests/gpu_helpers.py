"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle element by element."""
import math

import numpy as np
import torch

import sampling_sparse_attention_amd as santa
import workloads as W
from oracle import santa as O

BOUNDARY_WINDOW = 1e-6     # targets this close to a CDF edge may take either neighbour
O_REL_L2 = 1e-3            # o vs the fp64 gather of the same indices


def ensure_built():
    import os
    if not os.path.exists(santa.library_path):
        from sampling_sparse_attention_amd import build
        build.build()


def to_device(x: dict, device="cuda") -> dict:
    y = dict(x)
    for key in ("q", "k", "v", "seq_lens", "block_table"):
        if y[key] is not None:
            y[key] = y[key].to(device)
    return y


def run_hip(x: dict, S: int, mode: int, seed: int, split: int = 0, stages: str = "decode"):
    """Runs the HIP path on the tensors of ``x`` (already on the GPU)."""
    shape = santa.make_shape(x["q"], x["k"], x["block_table"], max_seq_len=x["workload"].seq_len,
                             split_size=split)
    B, Hq, d = x["q"].shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=x["q"].device)
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device=x["q"].device)
    ws = santa.allocate_workspace(shape, S, mode, x["q"].device)
    args = (shape, x["q"], x["k"], x["v"], x["seq_lens"], x["block_table"], S, mode, seed, o, idx, ws)
    if stages == "decode":
        santa.santa_decode(*args)
    else:
        santa.santa_score_pass(*args)
        santa.santa_sample_pass(*args)
    torch.cuda.synchronize()
    return o.cpu(), idx.cpu(), ws, shape


def head_rows(x: dict, b: int, g: int):
    """fp64 K and V rows ``[n_b, d]`` of sequence b, KV head g (exact widening)."""
    k = W.sequence_rows(x, "k", b)[:, g].double().cpu().numpy()
    v = W.sequence_rows(x, "v", b)[:, g].double().cpu().numpy()
    return k, v


def oracle_head(x: dict, b: int, h: int, S: int, mode: int, seed: int, rows=None):
    w = x["workload"]
    g = h // w.group
    k, v = rows if rows is not None else head_rows(x, b, g)
    q = x["q"][b, h].double().cpu().numpy()
    s = O.scores(q, k)
    idx, t, F, p = O.sample_head(s, S, mode, seed, b, h)
    return dict(idx=idx, t=t, F=F, p=p, s=s, v=v, delta=O.boundary_distance(F, idx, t))


# Parity reports of this test session by configuration; tests/conftest.py writes
# them to parity_report.json in the run's output folder when the session ends.
SESSION_REPORTS = {}


def record(label: str, rep: "ParityReport") -> None:
    """Adds a report's counts to the session record of configuration `label`."""
    r = SESSION_REPORTS.setdefault(label, dict(heads=0, targets=0, boundary_cases=0, boundary_mismatches=0,
                                                worst_rel_l2=0.0))
    r["heads"] += rep.heads
    r["targets"] += rep.targets
    r["boundary_cases"] += rep.boundary
    r["boundary_mismatches"] += rep.boundary_mismatch
    r["worst_rel_l2"] = max(r["worst_rel_l2"], rep.worst_rel_l2)


class ParityReport:
    def __init__(self):
        self.heads = 0
        self.targets = 0
        self.boundary = 0
        self.boundary_mismatch = 0
        self.worst_rel_l2 = 0.0

    def __repr__(self):
        return (f"heads={self.heads} targets={self.targets} boundary_cases={self.boundary} "
                f"boundary_mismatches={self.boundary_mismatch} worst_rel_l2={self.worst_rel_l2:.2e}")


def check_head(rep: ParityReport, ref: dict, idx_gpu: np.ndarray, o_gpu: np.ndarray, where: str,
               window: float = BOUNDARY_WINDOW):
    """idx exact outside the boundary window (``window`` in CDF units); o within
    O_REL_L2 of the fp64 gather of idx_gpu."""
    t, F, delta = ref["t"], ref["F"], ref["delta"]
    n = len(ref["p"])
    rep.heads += 1
    rep.targets += len(t)
    assert idx_gpu.min() >= 0 and idx_gpu.max() < n, f"{where}: index out of range"
    near = delta < window
    rep.boundary += int(near.sum())
    bad = idx_gpu != ref["idx"]
    far_bad = bad & ~near
    assert not far_bad.any(), (f"{where}: {int(far_bad.sum())} indices differ away from a boundary, "
                               f"first at m={int(np.nonzero(far_bad)[0][0])}: gpu "
                               f"{idx_gpu[far_bad][:4]} oracle {ref['idx'][far_bad][:4]}")
    if bad.any():
        gi = idx_gpu[bad]
        tb = t[bad]
        ok = (F[gi] - window <= tb) & (tb < F[gi + 1] + window)
        assert ok.all(), f"{where}: a boundary-case index is not adjacent to its target"
        rep.boundary_mismatch += int(bad.sum())
    own = O.estimate(ref["v"], idx_gpu)
    err = float(np.linalg.norm(o_gpu - own) / max(np.linalg.norm(own), 1e-30))
    rep.worst_rel_l2 = max(rep.worst_rel_l2, err)
    assert err <= O_REL_L2, f"{where}: o relative L2 error {err:.3e}"


def _label(x: dict, S: int, mode: int, kind: str) -> str:
    w = x["workload"]
    return (f"{kind} {w.name} B{w.batch} {w.q_heads}/{w.kv_heads} d{w.head_dim} n{w.seq_len} {w.dtype}"
            f"{' paged' + str(w.page_size) if w.page_size else ''} S{S} {W.MODE_NAMES[mode]}")


def check_all(x: dict, S: int, mode: int, seed: int, o: torch.Tensor, idx: torch.Tensor,
              heads=None, label=None) -> ParityReport:
    w = x["workload"]
    rep = ParityReport()
    lens = x["seq_lens"].cpu()
    B, Hq = w.batch, w.q_heads
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    rows_cache = {}
    for b, h in heads:
        n = int(lens[b])
        if n == 0:
            assert torch.all(idx[b, h] == -1) and torch.all(o[b, h] == 0), f"empty sequence {b}"
            continue
        g = h // w.group
        if (b, g) not in rows_cache:
            rows_cache.clear()
            rows_cache[(b, g)] = head_rows(x, b, g)
        ref = oracle_head(x, b, h, S, mode, seed, rows_cache[(b, g)])
        check_head(rep, ref, idx[b, h].numpy().astype(np.int64), o[b, h].double().numpy(),
                   f"(b={b}, h={h}, mode={mode}, S={S})")
    record(label or _label(x, S, mode, "santa"), rep)
    return rep


def run_flash(x: dict, S: int, mode: int, seed: int, split: int = 0, workspace=None):
    """Runs santa_decode_flash on the tensors of ``x``; returns o, idx, workspace, tile size."""
    shape = santa.make_shape(x["q"], x["k"], x["block_table"], max_seq_len=x["workload"].seq_len,
                             split_size=split)
    B, Hq, d = x["q"].shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=x["q"].device)
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device=x["q"].device)
    ws = workspace if workspace is not None else santa.allocate_workspace(shape, S, mode, x["q"].device)
    santa.santa_decode_flash(shape, x["q"], x["k"], x["v"], x["seq_lens"], x["block_table"], S, mode, seed,
                             o, idx, ws)
    torch.cuda.synchronize()
    tile = santa.santa_workspace_layout_query(shape, S, mode).split_size
    return o.cpu(), idx.cpu(), ws, tile


def check_flash(x: dict, S: int, mode: int, seed: int, tile: int, o: torch.Tensor, idx: torch.Tensor,
                heads=None, label=None) -> ParityReport:
    """S^2ANTA-flash parity: idx exact outside the boundary window of each tile's local CDF;
    o within O_REL_L2 of the oracle's fp64 merge of the GPU's own idx."""
    w = x["workload"]
    rep = ParityReport()
    lens = x["seq_lens"].cpu()
    if heads is None:
        heads = [(b, h) for b in range(w.batch) for h in range(w.q_heads)]
    rows_cache = {}
    for b, h in heads:
        n = int(lens[b])
        where = f"flash (b={b}, h={h}, mode={mode}, S={S}, tile={tile})"
        if n == 0:
            assert torch.all(idx[b, h] == -1) and torch.all(o[b, h] == 0), f"empty sequence {b}"
            continue
        g = h // w.group
        if (b, g) not in rows_cache:
            rows_cache.clear()
            rows_cache[(b, g)] = head_rows(x, b, g)
        k, v = rows_cache[(b, g)]
        s = O.scores(x["q"][b, h].double().cpu().numpy(), k)
        ref = O.sample_head_flash(s, S, mode, seed, b, h, tile)
        ig = idx[b, h].numpy().astype(np.int64)
        rep.heads += 1
        rep.targets += S
        assert ig.min() >= 0 and ig.max() < n, f"{where}: index out of range"
        assert np.all(ig // tile == ref["tile_of"]), f"{where}: a sample left its tile"
        near = ref["delta"] < BOUNDARY_WINDOW
        rep.boundary += int(near.sum())
        bad = ig != ref["idx"]
        far_bad = bad & ~near
        assert not far_bad.any(), (f"{where}: {int(far_bad.sum())} indices differ away from a boundary, "
                                   f"first at m={int(np.nonzero(far_bad)[0][0])}")
        for m in np.nonzero(bad)[0]:
            t = int(ref["tile_of"][m])
            F = ref["F"][t]
            lk = int(ig[m]) - t * tile
            assert F[lk] - BOUNDARY_WINDOW <= ref["t"][m] < F[lk + 1] + BOUNDARY_WINDOW, \
                f"{where}: a boundary-case index is not adjacent to its target"
            rep.boundary_mismatch += 1
        own = O.estimate_flash(v, ig, ref["tile_of"], ref["budget"], ref["weight"])
        err = float(np.linalg.norm(o[b, h].double().numpy() - own) / max(np.linalg.norm(own), 1e-30))
        rep.worst_rel_l2 = max(rep.worst_rel_l2, err)
        assert err <= O_REL_L2, f"{where}: o relative L2 error {err:.3e}"
    record(label or _label(x, S, mode, f"flash tile{tile}"), rep)
    return rep


unique_v_rows = W.unique_v_rows
