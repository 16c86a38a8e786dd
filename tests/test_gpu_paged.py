"""Paged K/V cache (attn_fwd_paged) against the fp64 oracle and the contiguous call.

Each case scatters the contiguous seeded K/V of a workload into pages in a
random order (pages of one sequence are not adjacent, a spare page is shared
by two sequences where lengths allow, and every page nobody's K_b reaches is
NaN), gives table entries past a sequence's length garbage values, and checks
that (a) the result matches the oracle on the contiguous K/V within the
tolerance, and (b) it is bitwise the result of attn_fwd_ex on the contiguous
K/V (same kernels, same order of arithmetic).
"""
import numpy as np
import pytest

import attention_attn_fwd_amd as af
from attention_attn_fwd_amd import inputs
from gpu_util import Outputs, call, compare, say, to_dev

pytestmark = pytest.mark.gpu


def _paginate(k, v, seqlens, page, rng, nan_pad):
    """Scatter [B,Hkv,K,*] into pages; returns (k_pages, v_pages, table, num_pages)."""
    B, Hkv, K, D = k.shape
    Dv = v.shape[-1]
    pps = K // page
    used = [(b, j) for b in range(B) for j in range(pps) if j * page < int(seqlens[b])]
    num_pages = len(used) + 3  # spare pages nobody references: NaN
    order = rng.permutation(num_pages)
    kp = np.empty((num_pages, Hkv, page, D), dtype=k.dtype)
    vp = np.empty((num_pages, Hkv, page, Dv), dtype=v.dtype)
    nan = np.array(0x7FC0, np.uint16) if k.dtype == np.uint16 else np.array(np.nan, k.dtype)
    kp[...] = nan
    vp[...] = nan
    table = rng.integers(-5, 1 << 20, size=(B, pps)).astype(np.int32)   # garbage past K_b
    for i, (b, j) in enumerate(used):
        pg = int(order[i])
        table[b, j] = pg
        kp[pg] = k[b, :, j * page:(j + 1) * page]
        vp[pg] = v[b, :, j * page:(j + 1) * page]
        if nan_pad:  # rows past K_b inside the last page: NaN, never read
            lim = int(seqlens[b]) - j * page
            if lim < page:
                kp[pg, :, lim:] = nan
                vp[pg, :, lim:] = nan
    return kp, vp, table, num_pages


def _flags(w):
    return (af.ATTN_FWD_FP16 if w.dtype == "f16" else 0) | (0 if w.causal else af.ATTN_FWD_NONCAUSAL)


def _run_paged(w, q, kp, vp, table, num_pages, page):
    import torch
    outs = Outputs(w, w.dtype)
    dseq = None if w.seqlens is None else to_dev(np.asarray(w.seqlens, np.int32))
    st = af.attn_fwd_paged(to_dev(q), to_dev(kp), to_dev(vp), outs.o, outs.l, w.B, w.Hq, w.Hkv, w.Q, w.D, w.Dv,
                           to_dev(table), table.shape[1], page, num_pages, dseq, w.window, w.scale, _flags(w),
                           torch.cuda.current_stream())
    assert st == af.ATTN_OK, af.strerror(st)
    torch.cuda.synchronize()
    assert outs.canaries_intact()
    return outs


CASES = [
    # B, Hq, Hkv, Q, K, D, Dv, page, window, dtype, causal, seqlens
    (4, 8, 2, 1, 1024, 128, 128, 64, 0, "bf16", True, [1024, 700, 0, 65]),
    (4, 8, 2, 3, 1024, 128, 128, 128, 0, "bf16", True, [1000, 64, 513, 1]),
    (3, 16, 2, 1, 4096, 64, 96, 256, 0, "f16", True, [4096, 2053, 300]),
    (2, 8, 2, 2, 2048, 128, 128, 1024, 100, "bf16", True, [2048, 1500]),
    (2, 8, 2, 1, 512, 128, 128, 64, 0, "bf16", False, [512, 130]),
    (2, 8, 4, 200, 512, 128, 128, 64, 0, "bf16", True, [512, 333]),
    (2, 4, 2, 300, 768, 64, 64, 256, 0, "f16", True, [768, 500]),
    (2, 8, 2, 256, 512, 128, 128, 128, 64, "bf16", True, [512, 400]),
    (2, 8, 2, 128, 256, 80, 96, 64, 0, "bf16", False, [256, 0]),
    (2, 16, 2, 60, 1024, 128, 128, 128, 0, "bf16", True, [1024, 317]),   # packed tiles across heads
    (3, 8, 2, 33, 512, 64, 64, 64, 31, "f16", True, [512, 0, 200]),
    (2, 32, 4, 100, 768, 128, 128, 256, 0, "bf16", False, [768, 129]),
    (2, 8, 2, 150, 1024, 256, 256, 128, 0, "bf16", True, [1024, 500]),    # wide heads
    (3, 8, 2, 1, 2048, 256, 256, 64, 0, "f16", True, [2048, 0, 999]),
    (2, 8, 2, 90, 512, 512, 512, 64, 0, "bf16", True, [512, 200]),        # 512 wide: 32-key blocks
    (2, 4, 2, 1, 1024, 384, 448, 128, 0, "f16", False, [1024, 3]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:8])) + f"_W{c[8]}_{c[9]}_{'c' if c[10] else 'nc'}")
def test_paged_matches_contiguous_and_oracle(orc, case):
    import torch
    B, Hq, Hkv, Q, K, D, Dv, page, window, dtype, causal, sl = case
    w = inputs.Workload("paged", B, Hq, Hkv, Q, K, D, Dv, dtype=dtype, window=window, causal=causal,
                        seqlens=np.array(sl, np.int32))
    say(f"[case] paged {case}")
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    rng = np.random.default_rng(B * 1000 + page)
    kp, vp, table, num_pages = _paginate(k, v, w.seqlens, page, rng, nan_pad=True)
    outs = _run_paged(w, q, kp, vp, table, num_pages, page)
    o, lse = outs.host()
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=window, causal=causal)
    compare(o, lse, ro, rl, dtype, f"paged {case}")
    ref = Outputs(w, w.dtype)
    dseq = to_dev(np.asarray(w.seqlens, np.int32))
    assert call(w, to_dev(q), to_dev(k), to_dev(v), dseq, ref) == af.ATTN_OK
    torch.cuda.synchronize()
    assert torch.equal(ref.o_raw, outs.o_raw), "paged O differs bitwise from the contiguous call"
    assert torch.equal(ref.l_raw, outs.l_raw), "paged LSE differs bitwise from the contiguous call"


def test_forward_paged_api(orc):
    import torch
    w = inputs.Workload("paged_fwd", 2, 8, 2, 1, 512, 64, 64, dtype="f16", seqlens=np.array([512, 77], np.int32))
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    kp, vp, table, _ = _paginate(k, v, w.seqlens, 128, np.random.default_rng(5), nan_pad=False)
    o, lse = af.forward_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(table), seqlens_k=to_dev(w.seqlens))
    torch.cuda.synchronize()
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens)
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, "f16",
            "forward_paged()")
