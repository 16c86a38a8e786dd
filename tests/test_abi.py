"""The C-ABI library on the CPU: it loads, exports every declared function, and
rejects bad arguments before touching the GPU (no kernel is launched here)."""
import os
import re

import pytest

import attention_attn_fwd_amd as af

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = af.load()
    declared = _declared_functions()
    assert set(af.EXPORTS) == set(declared), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_one_hip_runtime_in_the_process():
    """Loading the library (before anything imported torch) must leave a single
    libamdhip64 mapped: the one torch uses, which the library binds to."""
    import subprocess
    import sys
    code = ("import attention_attn_fwd_amd as af; af._binding.load(); import torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_strerror():
    for st in range(5):
        assert af.strerror(st)
    assert af.strerror(99) == "unknown status"


BAD = [
    # B, Hq, Hkv, Q, K, D, Dv, scale, expected
    (-1, 4, 2, 8, 8, 64, 64, 1.0, af.ATTN_ERR_INVALID_ARG),
    (1, 4, 3, 8, 8, 64, 64, 1.0, af.ATTN_ERR_INVALID_ARG),     # Hq % Hkv
    (1, 4, 0, 8, 8, 64, 64, 1.0, af.ATTN_ERR_INVALID_ARG),     # Hkv = 0 < Hq
    (1, 4, 2, 8, 8, 64, 64, float("nan"), af.ATTN_ERR_INVALID_ARG),
    (1, 4, 2, 8, 8, 64, 64, float("inf"), af.ATTN_ERR_INVALID_ARG),
    (1, 4, 2, 8, 8, 72, 64, 1.0, af.ATTN_ERR_UNSUPPORTED),     # D % 16
    (1, 4, 2, 8, 8, 64, 7, 1.0, af.ATTN_ERR_UNSUPPORTED),
    (1, 4, 2, 8, 8, 528, 64, 1.0, af.ATTN_ERR_UNSUPPORTED),    # beyond 512
    (1, 4, 2, 8, 8, 64, 528, 1.0, af.ATTN_ERR_UNSUPPORTED),
    (1, 4, 2, 8, 8, 504, 64, 1.0, af.ATTN_ERR_UNSUPPORTED),    # not a multiple of 16
    (1, 4, 2, 8, 8, 0, 64, 1.0, af.ATTN_ERR_UNSUPPORTED),
    (1, 4, 2, 8, 1 << 23, 128, 64, 1.0, af.ATTN_ERR_UNSUPPORTED),  # K*D = 2^30: a 2 GiB slice
    (1, 4, 2, 8, 1 << 23, 64, 128, 1.0, af.ATTN_ERR_UNSUPPORTED),  # K*Dv = 2^30
    (1, 4, 2, 1 << 23, 8, 128, 64, 1.0, af.ATTN_ERR_UNSUPPORTED),  # Q*D = 2^30
]


@pytest.mark.parametrize("case", BAD)
@pytest.mark.parametrize("fn", [af.attn_fwd, af.attn_fwd_f32], ids=["bf16", "f32"])
def test_bad_arguments_rejected_before_launch(fn, case):
    B, Hq, Hkv, Q, K, D, Dv, scale, want = case
    fake = 1 << 20  # never dereferenced: the checks come first
    assert fn(fake, fake, fake, fake, fake, B, Hq, Hkv, Q, K, D, Dv, None, 0, scale, None) == want


def test_wide_heads_only_on_the_16bit_path():
    fake = 1 << 20
    for D, Dv in [(256, 256), (144, 64), (64, 256), (512, 512), (512, 64), (400, 272)]:
        st = af.attn_fwd_f32(fake, fake, fake, fake, fake, 1, 4, 2, 8, 8, D, Dv, None, 0, 1.0, None)
        assert st == af.ATTN_ERR_UNSUPPORTED, (D, Dv)
        # 16 packed rows: the decode kernel up to 256 channels, else prefill.
        want = af.PATH_DECODE if max(D, Dv) <= 256 else af.PATH_PREFILL
        assert af.attn_fwd_plan(1, 4, 2, 8, 8, D, Dv)["path"] == want, (D, Dv)
    # Heads of 129..256 channels decode on the split-KV kernel up to 16 packed
    # rows; more rows, or heads above 256, take the prefill kernel.
    assert af.attn_fwd_plan(8, 8, 2, 1, 4096, 256, 256)["path"] == af.PATH_DECODE
    assert af.attn_fwd_plan(8, 32, 2, 1, 4096, 256, 256)["path"] == af.PATH_DECODE   # 16 rows
    assert af.attn_fwd_plan(8, 34, 2, 1, 4096, 256, 256)["path"] == af.PATH_PREFILL  # 17 rows
    assert af.attn_fwd_plan(8, 8, 2, 5, 4096, 256, 256)["path"] == af.PATH_PREFILL   # 20 rows
    assert af.attn_fwd_plan(8, 8, 2, 1, 4096, 512, 512)["path"] == af.PATH_PREFILL
    assert af.attn_fwd_plan(8, 8, 2, 1, 4096, 128, 128)["path"] == af.PATH_DECODE
    # Two 40 KiB ring stages of 256-channel K, V and Q: two workers per CU.
    assert af.attn_fwd_plan(64, 64, 8, 1, 32768, 256, 256)["split_workers"] == 512


def test_plans_follow_the_device_geometry(monkeypatch):
    """Worker counts and key-range pieces scale with the compute units the
    plan assumes (queried once per device; forced here)."""
    monkeypatch.delenv("ATTN_FWD_SPLIT_WORKERS", raising=False)
    monkeypatch.delenv("ATTN_FWD_PREFILL_SPLITS", raising=False)
    decode = (64, 64, 8, 1, 32768, 128, 128)   # batched long-context decode: 4 single-wave workers per CU
    chunk = (1, 32, 8, 512, 32768, 128, 128)  # 128 prefill tiles over 32768 keys
    monkeypatch.setenv("ATTN_FWD_CUS", "256")
    assert af.attn_fwd_plan(*decode)["split_workers"] == 4 * 256
    assert af.attn_fwd_plan(*chunk)["split_workers"] == 4   # 128 tiles x 4 pieces = 2 per CU
    monkeypatch.setenv("ATTN_FWD_CUS", "64")
    assert af.attn_fwd_plan(*decode)["split_workers"] == 4 * 64
    assert af.attn_fwd_plan(*chunk)["split_workers"] == 1   # the tiles alone fill 2 per CU
    monkeypatch.setenv("ATTN_FWD_CUS", "304")
    assert af.attn_fwd_plan(*decode)["split_workers"] == 4 * 304
    assert af.attn_fwd_plan(*chunk)["split_workers"] == 5   # ceil(608 / 128) pieces
    # A short problem never gets more workers than it has 4-sub-block shares.
    assert af.attn_fwd_plan(1, 8, 2, 1, 2053, 80, 96)["split_workers"] == (2 * 65 + 3) // 4


def test_wide_decode_ring_sizes_the_worker_count(monkeypatch):
    """Heads whose widths pad to 64 and 256 run on the kernel padded to 256 on
    both sides (two 40 KiB ring stages: two workers per CU), not three."""
    monkeypatch.delenv("ATTN_FWD_SPLIT_WORKERS", raising=False)
    monkeypatch.setenv("ATTN_FWD_CUS", "256")
    for D, Dv in [(64, 256), (256, 64), (256, 256), (144, 128)]:
        assert af.attn_fwd_plan(64, 64, 8, 1, 32768, D, Dv)["split_workers"] == 512, (D, Dv)
    assert af.attn_fwd_plan(64, 64, 8, 1, 32768, 64, 128)["split_workers"] == 1024


@pytest.mark.parametrize("fn", [af.attn_fwd, af.attn_fwd_f32], ids=["bf16", "f32"])
def test_null_and_misaligned_pointers(fn):
    fake = 1 << 20
    assert fn(None, fake, fake, fake, fake, 1, 4, 2, 8, 8, 64, 64, None, 0, 1.0, None) == af.ATTN_ERR_INVALID_ARG
    assert fn(fake, None, fake, fake, fake, 1, 4, 2, 8, 8, 64, 64, None, 0, 1.0, None) == af.ATTN_ERR_INVALID_ARG
    assert fn(fake, fake, fake, fake, None, 1, 4, 2, 8, 8, 64, 64, None, 0, 1.0, None) == af.ATTN_ERR_INVALID_ARG
    assert fn(fake + 2, fake, fake, fake, fake, 1, 4, 2, 8, 8, 64, 64, None, 0, 1.0, None) == af.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", [af.attn_fwd, af.attn_fwd_f32], ids=["bf16", "f32"])
def test_empty_problem_is_ok_without_launch(fn):
    for (B, Hq, Q) in [(0, 4, 8), (1, 0, 8), (2, 4, 0)]:
        Hkv = 2 if Hq else 0
        assert fn(None, None, None, None, None, B, Hq, Hkv, Q, 8, 64, 64, None, 0, 1.0, None) == af.ATTN_OK


def _ex(flags):
    def fn(q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, stream):
        return af.attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, flags, stream)
    return fn


@pytest.mark.parametrize("flags", [af.ATTN_FWD_FP16, af.ATTN_FWD_NONCAUSAL, af.ATTN_FWD_FP32 | af.ATTN_FWD_NONCAUSAL])
@pytest.mark.parametrize("case", BAD, ids=lambda c: "_".join(map(str, c[:8])))
def test_ex_bad_arguments_rejected_before_launch(flags, case):
    B, Hq, Hkv, Q, K, D, Dv, scale, want = case
    fake = 1 << 20
    assert _ex(flags)(fake, fake, fake, fake, fake, B, Hq, Hkv, Q, K, D, Dv, None, 0, scale, None) == want


def test_ex_flag_checks():
    fake = 1 << 20
    args = (fake, fake, fake, fake, fake, 1, 4, 2, 8, 8, 64, 64, None)
    bad = af.ATTN_ERR_INVALID_ARG
    assert af.attn_fwd_ex(*args, 0, 1.0, 8, None) == bad                       # unknown bit
    assert af.attn_fwd_ex(*args, 0, 1.0, -1, None) == bad
    assert af.attn_fwd_ex(*args, 0, 1.0, af.ATTN_FWD_FP16 | af.ATTN_FWD_FP32, None) == bad
    assert af.attn_fwd_ex(*args, 5, 1.0, af.ATTN_FWD_NONCAUSAL, None) == bad   # a window needs the causal limit
    assert af.attn_fwd_ex(*args, 5, 1.0, af.ATTN_FWD_NONCAUSAL | af.ATTN_FWD_FP16, None) == bad
    for flags in (0, af.ATTN_FWD_FP16, af.ATTN_FWD_FP32, af.ATTN_FWD_NONCAUSAL):
        assert af.attn_fwd_ex(None, None, None, None, None, 2, 4, 2, 0, 8, 64, 64, None, 0, 1.0, flags,
                              None) == af.ATTN_OK


def test_paged_argument_checks():
    fake = 1 << 20

    def paged(pps=4, page=64, npages=8, flags=0, window=0, table=fake, Q=8):
        return af.attn_fwd_paged(fake, fake, fake, fake, fake, 1, 4, 2, Q, 64, 64, table, pps, page, npages, None,
                                 window, 1.0, flags, None)
    assert paged(page=96) == af.ATTN_ERR_UNSUPPORTED            # not a power of two
    assert paged(page=32) == af.ATTN_ERR_UNSUPPORTED            # below 64
    assert paged(page=1 << 17) == af.ATTN_ERR_UNSUPPORTED
    assert paged(flags=af.ATTN_FWD_FP32) == af.ATTN_ERR_UNSUPPORTED
    assert paged(page=0) == af.ATTN_ERR_INVALID_ARG
    assert paged(pps=-1) == af.ATTN_ERR_INVALID_ARG
    assert paged(npages=-1) == af.ATTN_ERR_INVALID_ARG
    assert paged(npages=0) == af.ATTN_ERR_INVALID_ARG           # keys but no pages
    assert paged(table=None) == af.ATTN_ERR_INVALID_ARG
    assert paged(flags=af.ATTN_FWD_NONCAUSAL, window=3) == af.ATTN_ERR_INVALID_ARG
    assert paged(flags=16) == af.ATTN_ERR_INVALID_ARG
    assert paged(Q=0) == af.ATTN_OK                              # nothing to do
    assert paged(pps=1 << 25, page=128) == af.ATTN_ERR_UNSUPPORTED  # K*D over the 2 GiB slice bound


def test_slice_size_limit_boundary():
    # One row short of a 2 GiB (batch, head) slice is accepted by the plan.
    assert af.attn_fwd_plan(1, 4, 2, 64, (1 << 23) - 1, 128, 128)["path"] == af.PATH_PREFILL
    assert af.attn_fwd_plan(1, 4, 2, 8, (1 << 23) - 1, 128, 128)["path"] == af.PATH_DECODE
    with pytest.raises(af.AttnError) as e:
        af.attn_fwd_plan(1, 4, 2, 8, 1 << 23, 128, 128)
    assert e.value.status == af.ATTN_ERR_UNSUPPORTED


def test_plan_selects_paths():
    assert af.attn_fwd_plan(4, 32, 8, 4096, 4096, 128, 128)["path"] == af.PATH_PREFILL
    p = af.attn_fwd_plan(64, 64, 8, 1, 32768, 128, 128)
    assert p["path"] == af.PATH_DECODE and p["split_workers"] == 1024
    assert p["partial_slots"] == 64 * 8 + 1024
    assert p["workspace_bytes"] == p["partial_slots"] * 8 * (128 + 2) * 4
    # Small problems: at least 4 sub-blocks of 32 keys per worker.
    small = af.attn_fwd_plan(1, 8, 2, 1, 2053, 80, 96)
    assert small["split_workers"] == -(-(2 * -(-2053 // 32)) // 4)
    assert af.attn_fwd_plan(1, 8, 2, 1, 2053, 80, 96)["path"] == af.PATH_DECODE
    assert af.attn_fwd_plan(1, 8, 2, 4, 100, 64, 64)["path"] == af.PATH_DECODE      # 16 packed rows
    assert af.attn_fwd_plan(1, 64, 1, 1, 100, 64, 64)["path"] == af.PATH_PREFILL    # 64 rows: prefill kernel
    assert af.attn_fwd_plan(1, 8, 2, 5, 100, 64, 64)["path"] == af.PATH_DECODE      # 20 packed rows
    assert af.attn_fwd_plan(1, 2, 2, 32, 100, 64, 64)["path"] == af.PATH_DECODE     # Q = 32, MHA
    assert af.attn_fwd_plan(1, 8, 2, 9, 100, 64, 64)["path"] == af.PATH_PREFILL     # 36 rows
    assert af.attn_fwd_plan(0, 8, 2, 5, 100, 64, 64)["path"] == af.PATH_NONE
    assert af.attn_fwd_plan(1, 8, 2, 1, 0, 64, 64)["split_workers"] == 0
    with pytest.raises(af.AttnError):
        af.attn_fwd_plan(1, 8, 3, 1, 10, 64, 64)


def test_plan_prefill_splits(monkeypatch):
    monkeypatch.delenv("ATTN_FWD_PREFILL_SPLITS", raising=False)
    # 512 tiles fill the GPU: no split.
    p = af.attn_fwd_plan(4, 32, 8, 4096, 4096, 128, 128)
    assert (p["split_workers"], p["partial_slots"], p["workspace_bytes"]) == (1, 0, 0)
    # 32 packed tiles (16 rows of 8 heads each) over 16384 keys (256 blocks):
    # pieces of at least 32 blocks, so 8 of them (not the 16 that fill 512).
    p = af.attn_fwd_plan(4, 64, 8, 16, 16384, 128, 128)
    assert p["path"] == af.PATH_PREFILL and p["split_workers"] == 8
    assert p["partial_slots"] == 32 * 8 and p["workspace_bytes"] == 256 * 128 * 130 * 4
    # 128 per-head tiles: 4 pieces fill 512 workgroups.
    assert af.attn_fwd_plan(1, 32, 8, 512, 32768, 128, 128)["split_workers"] == 4
    # 4 tiles of 33 blocks: two pieces of at least 16.
    assert af.attn_fwd_plan(2, 8, 2, 9, 2053, 128, 128)["split_workers"] == 2
    assert af.attn_fwd_plan(2, 8, 2, 9, 1984, 128, 128)["split_workers"] == 1   # 31 blocks
    # 4 tiles: 32-block pieces leave most CUs idle, so 16-block ones (8).
    assert af.attn_fwd_plan(1, 8, 2, 48, 8192, 128, 128)["split_workers"] == 8
    assert af.attn_fwd_plan(2, 8, 2, 9, 4096, 128, 128)["split_workers"] == 4
    assert af.attn_fwd_plan(1, 8, 2, 256, 1024, 64, 64)["split_workers"] == 1
    assert af.attn_fwd_plan(1, 4, 2, 65, 511, 64, 64)["split_workers"] == 1
    assert af.attn_fwd_plan(1, 4, 2, 65, 0, 64, 64)["split_workers"] == 1
    # At most 32 pieces; the override is clamped the same way.
    assert af.attn_fwd_plan(1, 1, 1, 128, 1 << 20, 64, 64)["split_workers"] == 32
    # Lean tiles (decode with wide heads: 32 packed rows) over long keys:
    # pieces of 32 blocks whatever the tile count.
    assert af.attn_fwd_plan(128, 128, 4, 1, 32768, 256, 256)["split_workers"] == 16
    assert af.attn_fwd_plan(128, 128, 4, 1, 2047, 256, 256)["split_workers"] == 1
    # Pieces hold a fixed number of blocks: a count is rounded to what whole
    # pieces of ceil(blocks / count) blocks need.
    monkeypatch.setenv("ATTN_FWD_PREFILL_SPLITS", "7")
    p = af.attn_fwd_plan(1, 4, 2, 65, 1000, 64, 96)   # 16 blocks: pieces of 3, 6 of them
    # 130 packed rows per group: 2 tiles, 2 groups.
    assert p["split_workers"] == 6 and p["partial_slots"] == 4 * 6 and p["workspace_bytes"] == 24 * 128 * 98 * 4
    assert af.attn_fwd_plan(1, 4, 2, 65, 100, 64, 96)["split_workers"] == 2   # 2 blocks
    monkeypatch.setenv("ATTN_FWD_PREFILL_SPLITS", "1000")
    assert af.attn_fwd_plan(1, 4, 2, 65, 100000, 64, 64)["split_workers"] == 32
    # The fp32 path is never split (it has no plan of its own: D, Dv checks only).


def test_bwd_argument_checks():
    fake = 1 << 20

    def bwd(B=1, Hq=4, Hkv=2, Q=8, K=8, D=64, Dv=64, window=0, scale=1.0, flags=0, q=fake, dk=fake):
        return af.attn_bwd(q, fake, fake, fake, fake, fake, fake, dk, fake, B, Hq, Hkv, Q, K, D, Dv, None, window,
                           scale, flags, None)
    bad, uns = af.ATTN_ERR_INVALID_ARG, af.ATTN_ERR_UNSUPPORTED
    assert bwd(Hkv=3) == bad
    assert bwd(B=-1) == bad
    assert bwd(scale=float("nan")) == bad
    assert bwd(flags=8) == bad
    assert bwd(flags=af.ATTN_FWD_FP16 | af.ATTN_FWD_FP32) == bad
    assert bwd(flags=af.ATTN_FWD_NONCAUSAL, window=4) == bad
    assert bwd(q=None) == bad
    assert bwd(dk=None) == bad
    assert bwd(q=fake + 2) == bad
    assert bwd(flags=af.ATTN_FWD_FP32) == uns
    assert bwd(D=272) == uns
    assert bwd(Dv=512) == uns
    assert bwd(D=72) == uns
    assert bwd(K=1 << 23, D=128) == uns
    assert bwd(B=0) == af.ATTN_OK
    assert af.attn_bwd(None, None, None, None, None, None, None, None, None, 2, 4, 2, 0, 0, 64, 64, None, 0, 1.0, 0,
                       None) == af.ATTN_OK
