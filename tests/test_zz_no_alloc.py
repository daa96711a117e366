"""The allocation-free decode entry point (sparse_attn_decode_noalloc, for callers that
cannot allocate) against the workspace entry point it varies: bitwise-equal results on two
calls in a row, the second on a smaller input, and the oracle's bar on both."""
import sys

import pytest
import torch

from top_chunk_sparse_amd import configs, ops
from top_chunk_sparse_amd.configs import DecodeConfig
from top_chunk_sparse_amd.ops import DecodeCall
from top_chunk_sparse_amd.synth import make_decode
from harness import check_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = DecodeConfig("noalloc_small", B=2, Hq=8, Hkv=2, d=128, N=40 * 32 + 7, C=32, g=4, k=5,
                     gate=1, n_plant=6, paged=True)


def _pair(cfg, seed, **kw):
    print(f"[noalloc] {cfg.name} B={cfg.B} N={cfg.N} k={cfg.k} levels={cfg.levels} {kw}",
          flush=True)
    inp = make_decode(cfg, seed, device=DEV)
    ref = DecodeCall(inp, **kw)()
    na = DecodeCall(inp, **kw)
    for t in (na.out, na.lse, na.sel, na.chunk_scores):
        t.fill_(-7)
    na.noalloc()
    torch.cuda.synchronize()
    return inp, ref, na


@pytest.mark.parametrize("kw", [{}, {"gist_mode": 1}], ids=["all_gists", "selected_gists"])
def test_noalloc_matches_workspace_entry_point(kw):
    # the 128K-token workload, then a smaller one on the same (static) scratch
    for cfg, seed in ((configs.LLAMA8B, configs.seed_for(configs.LLAMA8B.name)), (SMALL, 901)):
        inp, ref, na = _pair(cfg, seed, **kw)
        for a, b in ((na.out, ref.out), (na.lse, ref.lse), (na.sel, ref.sel),
                     (na.chunk_scores, ref.chunk_scores)):
            assert torch.equal(a, b), cfg.name
        st = check_decode(inp, na)
        print("   ", st, flush=True)
        del inp, ref, na
        torch.cuda.empty_cache()


def test_noalloc_two_levels_then_smaller():
    cfg = configs.HSSA
    inp, ref, na = _pair(cfg, configs.seed_for(cfg.name))
    assert torch.equal(na.out, ref.out) and torch.equal(na.sel, ref.sel)
    assert torch.equal(na.sel_groups, ref.sel_groups)
    del inp, ref, na
    small = SMALL.with_(gate=0, levels=2, J=4, k2=3, k=6, n_plant=6, plant_groups=3)
    inp, ref, na = _pair(small, 902)
    assert torch.equal(na.out, ref.out) and torch.equal(na.sel_groups, ref.sel_groups)
    check_decode(inp, na)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    big = configs.LLAMA8B.with_(B=256)   # ~75 MB of workspace
    p = ops.decode_params(B=big.B, Hq=big.Hq, Hkv=big.Hkv, d=big.d, N=big.N, C_=big.C, g=big.g,
                          k=big.k, gate=big.gate, num_pages=big.B * big.M)
    assert ops.decode_workspace_size(p) > ops.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, device=DEV)
    with pytest.raises(ops.TcsError) as e:
        ops.sparse_attn_decode_noalloc(p, x, x, x, x, x, x, out=x)
    assert e.value.code == ops.TCS_ERR_TOO_LARGE
