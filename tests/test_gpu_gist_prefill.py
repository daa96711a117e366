"""GPU parity of the SSA gist-masked prefill (interleaved chunks of L raw tokens and g gist
tokens; a position sees its own chunk causally and every earlier chunk's gists) against the
fp64 oracle, through the C ABI: out and lse within 1e-2 max-abs (bf16 inputs, fp32
accumulation), every row on small shapes, sampled raw and gist rows at the 16K-token size."""
import sys

import numpy as np
import pytest
import torch

from top_chunk_sparse_amd import configs
from top_chunk_sparse_amd.configs import GistPrefillConfig
from top_chunk_sparse_amd.ops import GistPrefillCall
from top_chunk_sparse_amd.synth import make_gist_prefill
from harness import OUT_TOL, oracle_gist_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(cfg, seed, rows=None):
    say(f"[gist-prefill] {cfg.name} seed={seed} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} M={cfg.M} "
        f"L={cfg.L} g={cfg.g} rows={'all' if rows is None else len(rows)}")
    inp = make_gist_prefill(cfg, seed, device=DEV)
    call = GistPrefillCall(inp)()
    torch.cuda.synchronize()
    out, lse = oracle_gist_prefill(inp, rows=rows)
    go = call.out.cpu().double().numpy().reshape(-1, cfg.d)
    gl = call.lse.cpu().double().numpy().reshape(-1)
    idx = np.arange(go.shape[0]) if rows is None else np.asarray(rows)
    eo = float(np.abs(go[idx] - out.reshape(-1, cfg.d)[idx]).max())
    el = float(np.abs(gl[idx] - lse.reshape(-1)[idx]).max())
    say(f"    max-abs out {eo:.2e}  lse {el:.2e}")
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    assert eo <= OUT_TOL and el <= OUT_TOL
    return inp, call


SMALL = GistPrefillConfig("gist_small", B=1, Hq=8, Hkv=2, d=128, M=5, L=64, g=4)
CASES = [
    SMALL,
    SMALL.with_(L=128, g=1),
    SMALL.with_(g=8, M=9),
    SMALL.with_(g=64, M=3),                  # one full gist block per chunk
    SMALL.with_(Hq=2, Hkv=2),                # G = 1
    SMALL.with_(Hq=16),                      # G = 8: two head groups
    SMALL.with_(M=1),                        # a single chunk: causal attention
    SMALL.with_(B=2, M=3),
    SMALL.with_(M=40, g=4),                  # 160 gists: a prefix of 3 blocks, the last partial
    SMALL.with_(M=17, L=192, g=16),
    # 1,024 raw-row workgroups (B = 2, two head groups) behind the gist rows': more than the
    # GPU holds at once, every row compared
    SMALL.with_(B=2, Hq=16, M=64),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[f"gp{i}" for i in range(len(CASES))])
def test_gist_prefill_small(idx):
    run(CASES[idx], seed=1100 + idx)


def test_gist_prefill_full_size_sampled():
    cfg = configs.GIST_PREFILL
    rng = np.random.default_rng(11)
    rows = []
    for bh in rng.choice(cfg.B * cfg.Hq, size=6, replace=False):
        for c in (0, 1, cfg.M // 2, cfg.M - 1):
            base = int(bh) * cfg.Tp + c * cfg.W
            rows += [base, base + 63, base + 64, base + cfg.L - 1]          # raw rows
            rows += [base + cfg.L + t for t in range(cfg.g)]                # its gist rows
        rows += (int(bh) * cfg.Tp + rng.choice(cfg.Tp, size=40, replace=False)).tolist()
    run(cfg, configs.seed_for(cfg.name), rows=sorted(set(rows)))


# Two more shapes at full size (33,792 positions each): long chunks with many gists, and many
# short chunks, whose gist prefix spans 16 gathered blocks.
LARGE = [
    GistPrefillConfig("gist_prefill_long_chunks", B=2, Hq=32, Hkv=8, d=128, M=64, L=512, g=16),
    GistPrefillConfig("gist_prefill_many_chunks", B=1, Hq=32, Hkv=8, d=128, M=512, L=64, g=2),
]


@pytest.mark.parametrize("idx", range(len(LARGE)), ids=[c.name for c in LARGE])
def test_gist_prefill_large_shapes_sampled(idx):
    cfg = LARGE[idx]
    rng = np.random.default_rng(12 + idx)
    rows = []
    for bh in rng.choice(cfg.B * cfg.Hq, size=4, replace=False):
        for c in (0, 1, cfg.M // 2, cfg.M - 1):
            base = int(bh) * cfg.Tp + c * cfg.W
            rows += [base, base + 63, base + cfg.L - 64, base + cfg.L - 1]   # raw rows
            rows += [base + cfg.L, base + cfg.L + cfg.g - 1]                   # gist rows
        rows += (int(bh) * cfg.Tp + rng.choice(cfg.Tp, size=30, replace=False)).tolist()
    run(cfg, 6100 + idx, rows=sorted(set(rows)))


def test_gist_prefill_deterministic():
    cfg = SMALL.with_(M=12)
    inp = make_gist_prefill(cfg, 1200, device=DEV)
    a = GistPrefillCall(inp)()
    first = a.out.clone(), a.lse.clone()
    a()
    torch.cuda.synchronize()
    assert torch.equal(first[0], a.out) and torch.equal(first[1], a.lse)


def test_gist_prefill_workspace_garbage():
    """The gathered gist arrays (the padding rows included) are written before they are read: a
    workspace full of 0xFF bytes gives the same bits as a fresh one."""
    cfg = SMALL.with_(M=11, g=4)      # 44 gists: the gathered arrays end in 20 padding rows
    inp = make_gist_prefill(cfg, 1210, device=DEV)
    a = GistPrefillCall(inp)()
    torch.cuda.synchronize()
    out, lse = a.out.clone(), a.lse.clone()
    a.ws.fill_(255)
    a()
    torch.cuda.synchronize()
    assert torch.equal(out, a.out) and torch.equal(lse, a.lse)
