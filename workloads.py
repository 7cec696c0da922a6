"""Seeded synthetic inputs for SANTA decode-step attention.

This module only draws input tensors (queries and KV caches); it holds none of
the method's arithmetic.  Both the HIP path and the CPU oracle are fed from it,
and every byte either side sees comes from here (the oracle gets exact copies of
the tensors handed to the GPU).

The shapes follow the pages' model shapes ("Stochastic Sparse Attention for
Memory-Bound Inference", §1 and §3.4: Llama-3.1-8B with 32 query / 8 KV heads,
d=128, at a 32k context; the SANTA++ page, appendix on kernel evaluation:
Qwen2.5-7B with 28 query / 4 KV heads).  Real activations and the pages'
benchmark suites are not available, so seeded random tensors of those shapes
stand in for them.

Generation recipe (all draws from one ``torch.Generator`` seeded with ``seed``
on the device the tensors are created on, in this order):

1. ``seq_lens``: all equal to ``seq_len`` or, when ``seq_len_min`` is set,
   uniform integers in ``[seq_len_min, seq_len]``.
2. ``q`` ~ N(0, 1) in fp32, multiplied by ``q_scale``.
3. ``K`` ~ N(0, 1) in fp32, generated in chunks of whole sequences or pages.
4. ``V`` ~ N(0, 1) in fp32, same chunking.
5. Outlier channels: for every KV head ``outlier_channels`` channels from a
   random permutation of ``range(d)`` are multiplied by ``outlier_scale`` in both
   K and V (for every sequence and token).
6. Sinks: the first ``sinks`` tokens of every sequence and KV head have K
   multiplied by ``sink_scale``.
7. Needles: for every sequence ``b`` and query head ``h`` (KV head ``h // G``)
   ``needles`` positions uniform in ``[0, seq_lens[b])`` get
   ``k = 0.5 * |k_orig| * q_h / |q_h| + 0.1 * N(0, I)``.
8. Paging: ``block_table`` is a random permutation of all pages reshaped to
   ``[B, pages_per_seq]``; token ``i`` of sequence ``b`` lives in page
   ``block_table[b, i // page_size]`` at slot ``i % page_size``.
9. K and V are rounded to the storage dtype as they are drawn (bf16 uses round
   to nearest even, torch's conversion); the edits of steps 5-7 read the stored
   values and round their result to the storage dtype again.  ``q`` is rounded
   last, after the needles used its fp32 direction.
10. Query channel scales (``q_channel_sigma > 0`` only; drawn right after ``q``
   in step 2, so workloads without them draw the same bytes as before): per KV
   head g and channel i a log-normal factor ``exp(sigma * N(0, 1))`` multiplies
   channel i of every query head of group g, in every sequence.  Real queries
   have a few channels of large magnitude and many small ones; this spread is
   what lets the Bernoulli query sampler skip key features.  sigma = 0.8 gives
   about 72 % of the key features read at B = 8 draws with G = 4, d = 128, near
   the 72.8 % the pages report for Llama 8B at B = 8 (section 5.2, Table 8).

Layouts: ``q`` is ``[B, Hq, d]``; a contiguous cache is ``[B, n_max, Hkv, d]``
(token-major), a paged cache is ``[num_pages, page_size, Hkv, d]``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch

MODE_MULTINOMIAL = 0
MODE_STRATIFIED = 1
MODE_SYSTEMATIC = 2
MODE_NAMES = {MODE_MULTINOMIAL: "multinomial", MODE_STRATIFIED: "stratified",
              MODE_SYSTEMATIC: "systematic"}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    seq_len: int                      # n_max; every sequence has this length unless seq_len_min is set
    dtype: str = "bf16"               # "bf16" or "f32" for q, K and V
    seq_len_min: Optional[int] = None
    page_size: int = 0                # 0: contiguous cache
    samples: Tuple[int, ...] = (256,)
    modes: Tuple[int, ...] = (MODE_SYSTEMATIC,)
    sample_seed: int = 1
    q_scale: float = 1.0
    sinks: int = 0
    sink_scale: float = 1.0
    needles: int = 0
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    q_channel_sigma: float = 0.0
    bernoulli: int = 0                # draws B of the Bernoulli query sampler (0: not a Bernoulli workload)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def pages_per_seq(self) -> int:
        return -(-self.seq_len // self.page_size) if self.page_size else 0

    @property
    def num_pages(self) -> int:
        return self.batch * self.pages_per_seq

    def kv_cache_bytes(self) -> int:
        """Bytes of one of K or V as allocated."""
        tokens = self.num_pages * self.page_size if self.page_size else self.batch * self.seq_len
        return tokens * self.kv_heads * self.head_dim * self.elem_bytes

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the hot path.  Sizes are the pages' model shapes.
WORKLOADS = {
    "toy": Workload("toy", batch=1, q_heads=1, kv_heads=1, head_dim=64, seq_len=1024,
                    dtype="f32", samples=(64,), modes=(MODE_MULTINOMIAL, MODE_SYSTEMATIC),
                    q_scale=4.0, sample_seed=0),
    "llama32k": Workload("llama32k", batch=1, q_heads=32, kv_heads=8, head_dim=128,
                         seq_len=32768, samples=(256,), modes=(MODE_SYSTEMATIC,),
                         sinks=4, sink_scale=8.0),
    "batched": Workload("batched", batch=16, q_heads=32, kv_heads=8, head_dim=128,
                        seq_len=32768, seq_len_min=8192, samples=(128, 512),
                        modes=(MODE_STRATIFIED,), needles=16),
    "qwen128k": Workload("qwen128k", batch=4, q_heads=28, kv_heads=4, head_dim=128,
                         seq_len=131072, samples=(1024,),
                         modes=(MODE_MULTINOMIAL, MODE_STRATIFIED, MODE_SYSTEMATIC),
                         outlier_channels=8, outlier_scale=6.0),
    "paged": Workload("paged", batch=64, q_heads=32, kv_heads=8, head_dim=128,
                      seq_len=32768, page_size=16, samples=(256,),
                      modes=(MODE_SYSTEMATIC,)),
    # SANTA++ (its page, Appendix E): the Qwen-shaped 32K single-sequence layer,
    # nominal budget S = 124 with P = 16, R = 4 -> K = 31 teams per query head
    "qwen32k": Workload("qwen32k", batch=1, q_heads=28, kv_heads=4, head_dim=128, seq_len=32768,
                        samples=(124,), modes=(MODE_SYSTEMATIC,), outlier_channels=8, outlier_scale=6.0),
    # Bernoulli qK^T (section 5.2): the Llama-shaped step with B = 8 draws
    "bern32k": Workload("bern32k", batch=1, q_heads=32, kv_heads=8, head_dim=128,
                        seq_len=32768, samples=(256,), modes=(MODE_SYSTEMATIC,),
                        sinks=4, sink_scale=8.0, q_channel_sigma=0.8, bernoulli=8),
}


def _storage_dtype(w: Workload) -> torch.dtype:
    if w.dtype == "bf16":
        return torch.bfloat16
    if w.dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {w.dtype!r}")


def make_inputs(w: Workload, seed: int = 0, device="cpu", chunk_tokens: int = 1 << 18) -> dict:
    """Draw the inputs of workload ``w`` on ``device``.

    Returns a dict with ``q``, ``k``, ``v`` (storage dtype), ``seq_lens``
    (int32 ``[B]``) and ``block_table`` (int32 ``[B, pages_per_seq]`` or None).
    The same ``(w, seed, device type)`` always gives the same bytes.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, Hq, Hkv, d, n = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.seq_len
    G = w.group
    assert Hq % Hkv == 0
    sdt = _storage_dtype(w)

    if w.seq_len_min is not None:
        seq_lens = torch.randint(w.seq_len_min, n + 1, (B,), generator=gen, device=device,
                                 dtype=torch.int64).to(torch.int32)
    else:
        seq_lens = torch.full((B,), n, dtype=torch.int32, device=device)

    q32 = torch.randn((B, Hq, d), generator=gen, device=device, dtype=torch.float32)
    q32 *= w.q_scale
    if w.q_channel_sigma > 0:
        z = torch.randn((Hkv, d), generator=gen, device=device, dtype=torch.float32)
        q32 *= torch.exp(w.q_channel_sigma * z).repeat_interleave(G, dim=0)[None]

    if w.page_size:
        shape = (w.num_pages, w.page_size, Hkv, d)
    else:
        shape = (B, n, Hkv, d)
    k = _draw(shape, sdt, gen, device, chunk_tokens)
    v = _draw(shape, sdt, gen, device, chunk_tokens)

    if w.outlier_channels:
        for g in range(Hkv):
            ch = torch.randperm(d, generator=gen, device=device)[: w.outlier_channels]
            for cache in (k, v):
                sl = cache[:, :, g, :]
                sl[..., ch] = (sl[..., ch].float() * w.outlier_scale).to(sdt)

    block_table = None
    if w.page_size:
        perm = torch.randperm(w.num_pages, generator=gen, device=device)
        block_table = perm.view(B, w.pages_per_seq).to(torch.int32).contiguous()

    def token_view(b: int, i0: int, i1: int, g: int) -> torch.Tensor:
        """Writable view on tokens [i0, i1) of sequence b, KV head g (i0..i1 within one page if paged)."""
        if block_table is None:
            return k[b, i0:i1, g]
        ps = w.page_size
        page = int(block_table[b, i0 // ps])
        return k[page, i0 % ps: i0 % ps + (i1 - i0), g]

    if w.sinks:
        for b in range(B):
            for g in range(Hkv):
                i = 0
                while i < min(w.sinks, int(seq_lens[b])):
                    j = min(w.sinks, int(seq_lens[b]))
                    if w.page_size:
                        j = min(j, (i // w.page_size + 1) * w.page_size)
                    tv = token_view(b, i, j, g)
                    tv.copy_((tv.float() * w.sink_scale).to(sdt))
                    i = j

    if w.needles:
        for b in range(B):
            nb = int(seq_lens[b])
            for h in range(Hq):
                g = h // G
                qh = q32[b, h]
                qhat = qh / qh.norm()
                pos = torch.randint(0, nb, (w.needles,), generator=gen, device=device)
                noise = torch.randn((w.needles, d), generator=gen, device=device,
                                    dtype=torch.float32)
                for r in range(w.needles):
                    i = int(pos[r])
                    tv = token_view(b, i, i + 1, g)
                    korig = tv[0].float()
                    tv[0] = (0.5 * korig.norm() * qhat + 0.1 * noise[r]).to(sdt)

    q = q32.to(sdt).contiguous()
    return {"q": q, "k": k, "v": v, "seq_lens": seq_lens, "block_table": block_table,
            "workload": w, "seed": seed}


def keys_transposed(inputs: dict) -> torch.Tensor:
    """K of a contiguous cache in channel-major layout ``[B, Hkv, d, n_pad]`` (tokens
    contiguous; ``n_pad`` is ``n_max`` rounded up to a multiple of 16 bytes, the tail
    zero), the layout the Bernoulli query sampler reads feature rows from."""
    w: Workload = inputs["workload"]
    k = inputs["k"]
    assert inputs["block_table"] is None, "K^T is built from a contiguous cache"
    per16 = 16 // w.elem_bytes
    n_pad = -(-w.seq_len // per16) * per16
    kt = torch.zeros((w.batch, w.kv_heads, w.head_dim, n_pad), dtype=k.dtype, device=k.device)
    kt[..., : w.seq_len] = k[:, : w.seq_len].permute(0, 2, 3, 1)
    return kt


def _draw(shape, sdt, gen, device, chunk_tokens) -> torch.Tensor:
    out = torch.empty(shape, dtype=sdt, device=device)
    units_per_chunk = max(1, chunk_tokens // shape[1])
    for u0 in range(0, shape[0], units_per_chunk):
        u1 = min(shape[0], u0 + units_per_chunk)
        x = torch.randn((u1 - u0,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        out[u0:u1] = x.to(sdt)
    return out


def sequence_rows(inputs: dict, cache: str, b: int) -> torch.Tensor:
    """The logical rows ``[seq_lens[b], Hkv, d]`` of sequence ``b`` (a copy, through the block table)."""
    w: Workload = inputs["workload"]
    x = inputs[cache]
    n = int(inputs["seq_lens"][b])
    if inputs["block_table"] is None:
        return x[b, :n].clone()
    ps = w.page_size
    npg = -(-n // ps)
    pages = inputs["block_table"][b, :npg].long()
    return x[pages].reshape(npg * ps, w.kv_heads, w.head_dim)[:n].clone()


def traffic_bytes(w: Workload, seq_lens, unique_v_rows: int) -> int:
    """Algorithmic HBM bytes of one decode step: all K rows plus the distinct sampled V rows.

    ``unique_v_rows`` counts distinct (sequence, KV head, token) V rows read.
    """
    row = w.head_dim * w.elem_bytes
    k_rows = int(sum(int(n) for n in seq_lens)) * w.kv_heads
    return (k_rows + int(unique_v_rows)) * row


def dense_read_bytes(w: Workload, seq_lens) -> int:
    """Bytes a dense decode step reads: every K and every V row."""
    row = w.head_dim * w.elem_bytes
    return 2 * int(sum(int(n) for n in seq_lens)) * w.kv_heads * row


def unique_v_rows(idx: torch.Tensor, group: int) -> int:
    """Distinct (sequence, KV head, token) rows among sampled indices ``idx [B, Hq, S]``
    (negative entries mark empty sequences and are not rows)."""
    B, Hq, S = idx.shape
    per_group = idx.reshape(B, Hq // group, group * S)
    total = 0
    for b in range(B):
        for g in range(Hq // group):
            u = torch.unique(per_group[b, g])
            total += int((u >= 0).sum())
    return total
