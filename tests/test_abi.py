"""The C ABI on the host: libsanta.so loads, exports every symbol include/santa.h
declares, and validates arguments before touching any device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import sampling_sparse_attention_amd as santa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "santa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(santa.library_path):
        from sampling_sparse_attention_amd import build
        build.build()
    return santa.library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(santa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert len(declared) == 23
    out = subprocess.run(["nm", "-D", "--defined-only", santa.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (santa_\w+)", out))
    assert set(declared) <= exported
    assert set(declared) == set(santa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    version = int(re.search(r"#define SANTA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.santa_abi_version() == version
    names = [lib.santa_status_string(s).decode() for s in range(5)]
    assert names == ["ok", "invalid argument", "unsupported", "workspace too small", "HIP error"]
    assert lib.santa_status_string(99).decode() == "unknown status"


def _shape(**kw):
    d = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_seq_len=32768, page_size=0,
             pages_per_seq=0, num_pages=0, dtype=0, split_size=0,
             kv_stride_seq=32768 * 8 * 128, kv_stride_tok=8 * 128, kv_stride_head=128)
    d.update(kw)
    return santa.Shape(**d)


def _status_of_size(lib, shape, S=256, mode=2):
    n = ctypes.c_size_t()
    return lib.santa_workspace_size(ctypes.byref(shape) if shape is not None else None, S, mode,
                                    ctypes.byref(n)), n.value


def test_workspace_layout_llama_shape(lib):
    lay = santa.santa_workspace_layout_query(_shape(), 256, 2)
    T, split = lay.num_splits, lay.split_size
    assert split % 64 == 0 and T * split >= 32768 and (T - 1) * split < 32768
    assert lay.sync_offset == 0 and lay.records_offset >= 256
    assert lay.stash_offset >= lay.records_offset + 32 * T * 8
    assert lay.stash_row_bytes == T * split * 4
    assert lay.targets_offset >= lay.stash_offset + 32 * lay.stash_row_bytes
    assert lay.total_bytes >= lay.targets_offset and lay.total_bytes % 256 == 0
    for off in (lay.records_offset, lay.stash_offset, lay.targets_offset):
        assert off % 256 == 0
    assert santa.santa_workspace_size(_shape(), 256, 2) == lay.total_bytes
    # multinomial keeps S sorted targets per head
    lay0 = santa.santa_workspace_layout_query(_shape(), 256, 0)
    assert lay0.total_bytes >= lay0.targets_offset + 32 * 256 * 8
    lay_split = santa.santa_workspace_layout_query(_shape(split_size=128), 256, 2)
    assert lay_split.split_size == 128 and lay_split.num_splits == 256


def test_default_split_keeps_splits_per_sequence_bounded(lib):
    """A sequence has at most 512 splits (one merge wave holds 8 split records per lane);
    lengths that would need more, or more LDS than a workgroup has, are unsupported."""
    for n in (1, 1000, 32768, 131072, 200000, 262144, 524288):
        lay = santa.santa_workspace_layout_query(_shape(max_seq_len=n, kv_stride_seq=n * 8 * 128), 64, 2)
        assert lay.num_splits <= 512 and lay.num_splits * lay.split_size >= n
    with pytest.raises(santa.SantaError) as e:
        santa.santa_workspace_layout_query(_shape(max_seq_len=524289, kv_stride_seq=524289 * 8 * 128), 64, 2)
    assert e.value.status == UNSUPPORTED


@pytest.mark.parametrize("kw,S,mode,want", [
    (dict(num_q_heads=30), 256, 2, INVALID),
    (dict(num_q_heads=24), 256, 2, UNSUPPORTED),        # G = 3
    (dict(head_dim=96), 256, 2, UNSUPPORTED),
    (dict(dtype=7), 256, 2, INVALID),
    (dict(max_seq_len=0), 256, 2, INVALID),
    (dict(batch=0), 256, 2, INVALID),
    (dict(), 0, 2, INVALID),
    (dict(), 256, 3, INVALID),
    (dict(), 65536, 2, UNSUPPORTED),
    (dict(), 8193, 0, UNSUPPORTED),
    (dict(), 8192, 0, OK),
    (dict(), 65535, 1, OK),
    (dict(split_size=100), 256, 2, INVALID),
    (dict(split_size=192), 256, 2, INVALID),                # not a power of two
    (dict(split_size=2048), 256, 2, INVALID),
    (dict(page_size=8, pages_per_seq=4096, num_pages=4096), 256, 2, INVALID),
    (dict(page_size=24, pages_per_seq=4096, num_pages=4096), 256, 2, INVALID),
    (dict(page_size=16, pages_per_seq=100, num_pages=4096), 256, 2, INVALID),
    (dict(page_size=16, pages_per_seq=2048, num_pages=0), 256, 2, INVALID),
    (dict(page_size=16, pages_per_seq=2048, num_pages=2048), 256, 2, OK),
    (dict(kv_stride_tok=1001), 256, 2, INVALID),         # rows not 16-byte aligned
    (dict(kv_stride_tok=0), 256, 2, INVALID),
    (dict(num_q_heads=64, num_kv_heads=8, split_size=1024), 256, 2, OK),   # 133 KiB of LDS
    (dict(split_size=64), 256, 2, OK),                  # 512 splits
    (dict(max_seq_len=40000, split_size=64), 256, 2, UNSUPPORTED),   # 625 splits
    (dict(max_seq_len=524289), 256, 2, UNSUPPORTED),
])
def test_host_validation(lib, kw, S, mode, want):
    st, _ = _status_of_size(lib, _shape(**kw), S, mode)
    assert st == want, lib.santa_last_error().decode()
    if want != OK:
        assert lib.santa_last_error().decode() != ""


def test_null_shape_is_rejected(lib):
    st, _ = _status_of_size(lib, None)
    assert st == INVALID
    assert lib.santa_decode_path(None, 64, 2) == -INVALID


def test_decode_path_rejects_invalid_shapes_before_touching_hip(lib):
    assert lib.santa_decode_path(ctypes.byref(_shape(head_dim=96)), 64, 2) == -UNSUPPORTED
    assert lib.santa_decode_path(ctypes.byref(_shape()), 0, 2) == -INVALID


def test_workspace_init_validates_before_launch(lib):
    fake = ctypes.c_void_p(1 << 20)
    assert lib.santa_workspace_init(None, 4096, None) == INVALID
    assert lib.santa_workspace_init(ctypes.c_void_p((1 << 20) + 16), 4096, None) == INVALID
    assert lib.santa_workspace_init(fake, 255, None) == WS_SMALL


def test_decode_rejects_bad_pointers_before_launch(lib):
    """Every failing check returns before anything reaches a device (none exists here)."""
    shape = _shape(max_seq_len=1024, kv_stride_seq=1024 * 8 * 128)
    need = santa.santa_workspace_size(shape, 64, 2)
    fake = ctypes.c_void_p(1 << 20)                 # aligned, never dereferenced
    args = [fake] * 4 + [None]
    fn = lib.santa_decode

    def call(q=fake, k=fake, v=fake, lens=fake, bt=None, S=64, mode=2, o=fake, idx=fake, ws=fake,
             ws_bytes=need, shp=shape):
        return fn(ctypes.byref(shp), q, k, v, lens, bt, S, mode, ctypes.c_uint64(0), o, idx, ws,
                  ws_bytes, None)

    assert call(q=None) == INVALID
    assert call(o=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(bt=fake) == INVALID                 # table given for a contiguous cache
    assert call(q=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == INVALID
    assert call(ws_bytes=need - 1) == WS_SMALL
    assert "needs" in lib.santa_last_error().decode()
    paged = _shape(max_seq_len=1024, page_size=16, pages_per_seq=64, num_pages=64)
    assert call(shp=paged) == INVALID               # paged without a table
    assert call(S=0) == INVALID
    for name in ("santa_score_pass", "santa_sample_pass"):
        f = getattr(lib, name)
        assert f(ctypes.byref(shape), None, fake, fake, fake, None, 64, 2, ctypes.c_uint64(0),
                 fake, fake, fake, need, None) == INVALID
    del args


def test_flash_rejects_multinomial_and_too_few_samples_before_launch(lib):
    """santa_decode_flash samples by tiles: stratified or systematic only, and at
    least one sample per tile; both are checked on the host."""
    shape = _shape(max_seq_len=4096, kv_stride_seq=4096 * 8 * 128, split_size=256)    # 16 tiles
    fake = ctypes.c_void_p(1 << 20)

    def call(S, mode):
        need = santa.santa_workspace_size(shape, max(S, 1), mode)
        return lib.santa_decode_flash(ctypes.byref(shape), fake, fake, fake, fake, None, S, mode,
                                      ctypes.c_uint64(0), fake, fake, fake, need, None)

    assert call(64, 0) == UNSUPPORTED
    assert "stratified or systematic" in lib.santa_last_error().decode()
    assert call(15, 2) == UNSUPPORTED
    assert "a sample for every tile" in lib.santa_last_error().decode()
    assert call(0, 2) == INVALID
    lay = santa.santa_workspace_layout_query(shape, 64, 2)
    assert lay.accum_offset < lay.flash_offset < lay.records_offset
    assert lay.records_offset - lay.flash_offset >= 256 + 32 * 4 * 130 * 8   # refs, then 4 fp64 slots per head


def test_args_struct_matches_header_layout(lib):
    """The ctypes mirror of santa_args has the C layout (fields in header order, natural
    alignment), checked against offsets computed by the host compiler from santa.h."""
    import tempfile
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "santa.h"
#define F(x) printf("%s %zu\n", #x, offsetof(santa_args, x));
int main(void) {
    F(shape) F(q) F(k_cache) F(v_cache) F(seq_lens) F(block_table) F(num_samples) F(mode) F(seed)
    F(o) F(idx) F(workspace) F(workspace_bytes) F(algorithm) F(flags)
    printf("size %zu\n", sizeof(santa_args));
    return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "off.c")
        exe = os.path.join(d, "off")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    want = dict(line.split() for line in out.strip().splitlines())
    for name, _ in santa.Args._fields_:
        assert getattr(santa.Args, name).offset == int(want[name]), name
    assert ctypes.sizeof(santa.Args) == int(want["size"])


def test_decode_args_validates_before_launch(lib):
    shape = _shape(max_seq_len=1024, kv_stride_seq=1024 * 8 * 128)
    need = santa.santa_workspace_size(shape, 64, 2)
    fake = 1 << 20

    def call(**kw):
        a = santa.Args(shape, fake, fake, fake, fake, None, 64, 2, 0, fake, fake, fake, need, 0, 0)
        for k, v in kw.items():
            setattr(a, k, v)
        return lib.santa_decode_args(ctypes.byref(a), None)

    assert lib.santa_decode_args(None, None) == INVALID
    assert call(algorithm=2) == INVALID
    assert "algorithm" in lib.santa_last_error().decode()
    assert call(flags=2) == INVALID
    assert call(q=None) == INVALID
    assert call(workspace_bytes=need - 1) == WS_SMALL
    need0 = santa.santa_workspace_size(shape, 64, 0)
    assert call(algorithm=1, mode=0, workspace_bytes=need0) == UNSUPPORTED   # flash: stratified/systematic
    assert call(flags=1, num_samples=0) == INVALID


def test_bernoulli_validates_before_touching_the_device(lib):
    """santa_decode_bernoulli checks its K^T layout, B and the cache kind on the host."""
    shape = _shape(max_seq_len=1024, kv_stride_seq=1024 * 8 * 128)
    need = santa.santa_workspace_size(shape, 64, 2)
    fake = ctypes.c_void_p(1 << 20)
    good = santa.KtLayout(8 * 128 * 1024, 128 * 1024, 1024)

    def call(kt=good, B=8, counts=fake, shp=shape, k_t=fake):
        return lib.santa_decode_bernoulli(ctypes.byref(shp), fake, k_t, None if kt is None else ctypes.byref(kt),
                                          fake, fake, 64, 2, ctypes.c_uint64(0), B, fake, fake, counts, fake,
                                          need, None)

    assert call(kt=None) == INVALID
    assert call(counts=None) == INVALID
    assert call(k_t=ctypes.c_void_p((1 << 20) + 8)) == INVALID          # K^T not 16-byte aligned
    assert call(B=0) == UNSUPPORTED and call(B=65) == UNSUPPORTED
    assert "num_bernoulli" in lib.santa_last_error().decode()
    assert call(kt=santa.KtLayout(8 * 128 * 1024, 128 * 1024, 1000)) == INVALID     # rows shorter than n_max
    assert call(kt=santa.KtLayout(8 * 128 * 1028, 128 * 1028, 1028)) == INVALID     # rows not 16-byte aligned
    paged = _shape(max_seq_len=1024, page_size=16, pages_per_seq=64, num_pages=64)
    assert lib.santa_decode_bernoulli(ctypes.byref(paged), fake, fake, ctypes.byref(good), fake, fake, 64, 2,
                                      ctypes.c_uint64(0), 8, fake, fake, fake, fake, need, None) == INVALID


def test_santapp_team_count_and_validation_before_touching_the_device(lib):
    """santa_pp_num_teams is Algorithm 4's count; the SANTA++ entry points check their
    parameters, the cache kind and the workspace on the host."""
    assert santa.santa_pp_num_teams(32768, 16, 4) == 8192
    assert santa.santa_pp_num_teams(1000, 16, 4) == 62 * 4 + 4          # last parent of 8 tokens: 4 teams
    assert santa.santa_pp_num_teams(1001, 16, 4) == 62 * 4 + 4
    assert santa.santa_pp_num_teams(995, 16, 4) == 62 * 4 + 3           # last parent of 3 tokens
    assert santa.santa_pp_num_teams(10, 4, 4) == 10
    assert santa.santa_pp_num_teams(10, 16, 3) == -1 and santa.santa_pp_num_teams(10, 2, 4) == -1
    shape = _shape(max_seq_len=1024, kv_stride_seq=1024 * 8 * 128)
    fake = ctypes.c_void_p(1 << 20)
    tb = santa.PPTable(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    build = lib.santa_pp_build
    assert build(ctypes.byref(shape), fake, fake, 1000, 16, 3, ctypes.byref(tb), None) == INVALID
    assert build(ctypes.byref(shape), fake, fake, 1000, 128, 4, ctypes.byref(tb), None) == INVALID
    assert build(ctypes.byref(shape), fake, fake, 2000, 16, 4, ctypes.byref(tb), None) == INVALID     # N > n_max
    assert build(ctypes.byref(shape), fake, fake, 1000, 16, 4, None, None) == INVALID
    assert build(ctypes.byref(shape), None, fake, 1000, 16, 4, ctypes.byref(tb), None) == INVALID
    bad = santa.PPTable(1 << 20, (1 << 20) + 4, 1 << 20, 1 << 20, 1 << 20)
    assert build(ctypes.byref(shape), fake, fake, 1000, 16, 4, ctypes.byref(bad), None) == INVALID
    paged = _shape(max_seq_len=1024, page_size=16, pages_per_seq=64, num_pages=64)
    assert build(ctypes.byref(paged), fake, fake, 1000, 16, 4, ctypes.byref(tb), None) == UNSUPPORTED
    big = _shape(max_seq_len=262144, kv_stride_seq=262144 * 8 * 128, split_size=1024)
    assert build(ctypes.byref(big), fake, fake, 262144, 16, 16, ctypes.byref(tb), None) == UNSUPPORTED   # M > 131072
    need = santa.santa_pp_workspace_size(shape, 1000, 16, 4, 31)
    assert need > 0
    with pytest.raises(santa.SantaError):
        santa.santa_pp_workspace_size(shape, 1000, 16, 4, 0)

    def dec(K=31, ws_bytes=need, ws=fake, q=fake, N=1000):
        return lib.santa_pp_decode(ctypes.byref(shape), q, fake, fake, fake, N, 16, 4, ctypes.byref(tb), K,
                                   ctypes.c_uint64(0), fake, fake, fake, ws, ws_bytes, None)
    assert dec(K=0) == INVALID
    assert dec(ws_bytes=need - 1) == WS_SMALL
    assert dec(ws=ctypes.c_void_p((1 << 20) + 16)) == INVALID
    assert dec(q=None) == INVALID
    assert dec(N=0) == INVALID


def test_workspace_status_validates_before_touching_the_device(lib):
    word = ctypes.c_uint32(7)
    assert lib.santa_workspace_status(None, 4096, None, ctypes.byref(word)) == INVALID
    assert lib.santa_workspace_status(ctypes.c_void_p(1 << 20), 4096, None, None) == INVALID
    assert lib.santa_workspace_status(ctypes.c_void_p((1 << 20) + 4), 4096, None, ctypes.byref(word)) == INVALID
    assert lib.santa_workspace_status(ctypes.c_void_p(1 << 20), 16, None, ctypes.byref(word)) == WS_SMALL
    assert word.value == 7


def test_noalloc_refuses_oversized_problems_before_touching_the_device(lib):
    assert lib.santa_noalloc_scratch_bytes() == 64 << 20
    paged = _shape(batch=64, max_seq_len=32768, page_size=16, pages_per_seq=2048, num_pages=131072,
                   kv_stride_seq=16 * 8 * 128)
    fake = ctypes.c_void_p(1 << 20)
    st = lib.santa_decode_noalloc(ctypes.byref(paged), fake, fake, fake, fake, fake, 256, 2, ctypes.c_uint64(0),
                                  fake, fake, None)
    assert st == WS_SMALL
    assert "scratch array holds" in lib.santa_last_error().decode()
    assert lib.santa_decode_noalloc(ctypes.byref(_shape(head_dim=96)), fake, fake, fake, fake, None, 64, 2,
                                    ctypes.c_uint64(0), fake, fake, None) == UNSUPPORTED
