"""GPU parity of the chunk-sparse decode path against the fp64 oracle (calls go through the
C ABI via the ctypes binding).  Selected chunk ids must match exactly (near-ties at the k-th
boundary with a relative score gap < 1e-5 are excused, counted and re-checked against the
oracle run on the GPU's selection); out and lse within 1e-2 max-abs."""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from top_chunk_sparse_amd import configs
from top_chunk_sparse_amd.configs import DecodeConfig
from top_chunk_sparse_amd.ops import DecodeCall
from top_chunk_sparse_amd.synth import make_decode
from harness import check_decode, oracle_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(cfg, seed, units=None, gist_mode=0, top_p=0.0, head_select=0, adaptive_k=0, **kw):
    say(f"[decode] {cfg.name} seed={seed} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} "
        f"N={cfg.N} C={cfg.C} g={cfg.g} k={cfg.k} gate={cfg.gate} levels={cfg.levels} "
        f"gist_mode={gist_mode} top_p={top_p} head_select={head_select} "
        f"adaptive_k={adaptive_k} {kw}")
    inp = make_decode(cfg, seed, device=DEV, **kw)
    call = DecodeCall(inp, gist_mode=gist_mode, top_p=top_p, head_select=head_select,
                      adaptive_k=adaptive_k)()
    torch.cuda.synchronize()
    st = check_decode(inp, call, units=units)
    say("   ", st)
    return inp, call, st


@pytest.mark.parametrize("name", list(configs.DECODE_CONFIGS))
def test_named_config_full(name):
    cfg = configs.DECODE_CONFIGS[name]
    inp, call, st = run_case(cfg, configs.seed_for(name))
    assert st["excused"] <= max(1, st["units"] // 100)
    del inp, call
    torch.cuda.empty_cache()


SMALL = DecodeConfig("gpu_small", B=2, Hq=8, Hkv=2, d=128, N=40 * 32 + 7, C=32, g=4, k=5,
                     n_plant=6, paged=True)

VARIANTS = [
    SMALL,
    SMALL.with_(gate=1),
    SMALL.with_(d=64),
    SMALL.with_(d=64, gate=1, g=3, C=24, N=61 * 24 + 1),
    SMALL.with_(Hq=2, Hkv=2),                 # G = 1
    SMALL.with_(Hq=4, Hkv=2),                 # G = 2
    SMALL.with_(Hq=16, Hkv=2, gate=1),        # G = 8
    SMALL.with_(k=0),
    SMALL.with_(k=0, gate=1),
    SMALL.with_(k=10 ** 4, gate=1),           # every chunk
    SMALL.with_(N=20, C=32),                  # only the (partial) current chunk
    SMALL.with_(N=33, C=32, gate=1),          # one historical chunk
    SMALL.with_(g=1, C=64, N=300 * 64),       # many chunks, one gist each
    SMALL.with_(g=16, C=128, N=37 * 128 + 100, d=64),
    SMALL.with_(levels=2, J=4, k2=3, k=6, n_plant=6, plant_groups=3),
    SMALL.with_(levels=2, J=5, k2=100, k=7, n_plant=4, plant_groups=2, d=64),
    SMALL.with_(levels=2, J=3, k2=0, k=4, n_plant=0),
    SMALL.with_(levels=2, J=4, k2=2, k=0, n_plant=4, plant_groups=2),
    SMALL.with_(levels=2, J=8, k2=64, k=10 ** 4, n_plant=4, plant_groups=2, Hq=16),
    SMALL.with_(N=32, C=32, n_plant=0),            # exactly one full chunk: no history
    SMALL.with_(N=64, C=32, gate=1, n_plant=1),    # one full historical chunk + a full current
    SMALL.with_(levels=2, J=2, k2=1, k=1, N=3 * 32, n_plant=1, plant_groups=1),   # 2 chunks, 1 group
]


@pytest.mark.parametrize("cfg", VARIANTS, ids=[f"v{i}" for i in range(len(VARIANTS))])
def test_variants(cfg):
    run_case(cfg, seed=100 + VARIANTS.index(cfg), max_chunks=cfg.M + 5, extra_pages=3)


# Selected-gist token set (each selected chunk's gists next to its raw tokens; at two levels
# also the chosen groups' level-2 gists).
SEL_GISTS = [v for v in VARIANTS if v.C + v.g <= 1024] + [
    SMALL.with_(levels=2, J=4, k2=3, k=6, n_plant=6, plant_groups=3, g=1, Hq=2),   # G = 1
    SMALL.with_(levels=2, J=7, k2=5, k=9, n_plant=6, plant_groups=3, g=8, Hq=16),  # G = 8
    SMALL.with_(levels=2, J=6, k2=1, k=3, n_plant=3, plant_groups=1, d=64, C=64, g=64,
                N=30 * 64 + 63),                                                     # g = 64
]


@pytest.mark.parametrize("cfg", SEL_GISTS, ids=[f"sg{i}" for i in range(len(SEL_GISTS))])
def test_selected_gists_variants(cfg):
    run_case(cfg, seed=300 + SEL_GISTS.index(cfg), gist_mode=1, max_chunks=cfg.M + 2,
             extra_pages=1)


@pytest.mark.parametrize("name", ["llama32_1b_decode_32k", "llama31_8b_decode_128k",
                                  "hssa_decode_512k"])
def test_selected_gists_full(name):
    cfg = configs.DECODE_CONFIGS[name]
    inp, call, st = run_case(cfg, configs.seed_for(name), gist_mode=1)
    assert st["excused"] <= max(1, st["units"] // 100)
    del inp, call
    torch.cuda.empty_cache()


# Per-head selection with the union unfolded (one level, no gate), every gist or the selected
# chunks' gists in the softmax.
HEADS = [
    (SMALL, 0),
    (SMALL.with_(Hq=16), 0),                                          # G = 8
    (SMALL.with_(Hq=4), 1),                                           # G = 2, selected gists
    (SMALL.with_(Hq=2, Hkv=2), 0),                                    # G = 1
    (SMALL.with_(d=64, g=3, C=24, N=61 * 24 + 1), 1),
    (SMALL.with_(k=0), 0),
    (SMALL.with_(k=10 ** 4), 0),                                      # every chunk
    (SMALL.with_(N=20, C=32), 0),                                     # no historical chunk
    (SMALL.with_(N=33, C=32), 1),                                     # one historical chunk
    (SMALL.with_(g=1, C=64, N=300 * 64), 0),                          # 2 slices of 256 chunks
    # G = 8, 128 chunks per slice, 24 slices: 475 candidates per head reach the merge, which
    # then ranks them from global memory
    (SMALL.with_(g=1, C=16, N=16 * 3000 + 5, k=20, Hq=16, d=64), 0),
    (SMALL.with_(g=16, C=128, N=37 * 128 + 100, d=64), 1),
]


@pytest.mark.parametrize("idx", range(len(HEADS)), ids=[f"hs{i}" for i in range(len(HEADS))])
def test_head_select_variants(idx):
    cfg, gmode = HEADS[idx]
    run_case(cfg, seed=700 + idx, head_select=1, gist_mode=gmode, max_chunks=cfg.M + 2,
             extra_pages=1)


@pytest.mark.parametrize("name", ["llama32_1b_decode_32k", "llama31_8b_decode_128k"])
def test_head_select_full(name):
    cfg = configs.DECODE_CONFIGS[name].with_(gate=0)
    inp, call, st = run_case(cfg, configs.seed_for(name), head_select=1)
    assert st["excused"] <= max(1, st["units"] // 100)
    u = call.sel.cpu().numpy()
    n = (u >= 0).sum(-1)
    say(f"    union size: min {n.min()} mean {n.mean():.1f} max {n.max()} (k = {cfg.k}, G = {cfg.G})")
    assert (n >= min(cfg.k, cfg.H)).all() and (n <= min(cfg.G * cfg.k, cfg.H)).all()
    del inp, call
    torch.cuda.empty_cache()


# Top-p selection with a cap of k chunks (one level).
TOP_P = [
    (SMALL.with_(k=20), 0.3),
    (SMALL.with_(k=20, gate=1), 0.8),
    (SMALL.with_(k=20, gate=1, d=64, Hq=16), 0.95),
    (SMALL.with_(k=3), 0.9),                         # the cap decides
    (SMALL.with_(k=40, gate=1), 1.0),                # every chunk
    (SMALL.with_(k=20, g=1, C=64, N=300 * 64), 0.5),
    (SMALL.with_(k=20), 1e-6),                       # the best chunk only
]


@pytest.mark.parametrize("cfg,tp", TOP_P, ids=[f"tp{i}" for i in range(len(TOP_P))])
def test_top_p_variants(cfg, tp):
    run_case(cfg, seed=400 + [c for c, _ in TOP_P].index(cfg), top_p=tp)


# top-p at two levels: the cut runs over the chosen groups' member chunks (their shares of the
# softmax over the candidates' scores); the groups are still the top k2
TOP_P_L2 = [
    (SMALL.with_(levels=2, J=4, k2=3, k=10, n_plant=6, plant_groups=3), 0, 0.5),   # keeps 6
    (SMALL.with_(levels=2, J=5, k2=100, k=30, n_plant=4, plant_groups=2, d=64), 0, 0.9),  # cap
    (SMALL.with_(levels=2, J=4, k2=2, k=8, n_plant=4, plant_groups=2), 1, 0.7),    # keeps 6
    (SMALL.with_(levels=2, J=7, k2=5, k=9, n_plant=6, plant_groups=3, g=8, Hq=16), 0, 1.0),
    (SMALL.with_(levels=2, J=4, k2=3, k=10, n_plant=6, plant_groups=3), 1, 1e-6),  # keeps 1
    (SMALL.with_(levels=2, J=3, k2=0, k=4, n_plant=0), 0, 0.5),      # no group chosen
    (SMALL.with_(levels=2, J=4, k2=2, k=0, n_plant=4, plant_groups=2), 0, 0.5),   # k = 0
]


@pytest.mark.parametrize("idx", range(len(TOP_P_L2)), ids=[f"tpl2_{i}" for i in range(len(TOP_P_L2))])
def test_top_p_two_levels(idx):
    cfg, gmode, tp = TOP_P_L2[idx]
    run_case(cfg, seed=430 + idx, gist_mode=gmode, top_p=tp)


@pytest.mark.parametrize("name,tp", [("llama32_1b_decode_32k", 0.9), ("llama31_8b_decode_128k", 0.5),
                                     ("hssa_decode_512k", 0.5)])   # keeps 28-29 of 32
def test_top_p_full(name, tp):
    cfg = configs.DECODE_CONFIGS[name]
    inp, call, st = run_case(cfg, configs.seed_for(name), top_p=tp)
    assert st["excused"] <= max(1, st["units"] // 100)
    del inp, call
    torch.cuda.empty_cache()


# The largest documented shapes: C = 1024 rows per chunk with g = 64 gists; C + g = 1024 for the
# selected-gist set; k = 256 for top-p; J * g = 1024 and 64 chosen groups at two levels.
LIMITS = [
    (SMALL.with_(C=1024, g=64, d=64, N=9 * 1024 + 300, k=3, n_plant=2), 0, 0.0),
    (SMALL.with_(C=1024, g=8, N=5 * 1024 + 1, k=2, gate=1, n_plant=2), 0, 0.0),
    (SMALL.with_(C=960, g=64, d=64, N=7 * 960 + 5, k=2, n_plant=2), 1, 0.0),
    (SMALL.with_(C=16, g=1, d=64, N=300 * 16 + 3, k=256, n_plant=4, gate=1), 0, 0.95),
    # two levels, selected summaries: J * g = 1024 rows per group slice, all 64 groups chosen,
    # 64 level-2 gist rows in each group's partial
    (SMALL.with_(levels=2, J=16, k2=64, k=40, g=64, C=64, d=64, N=1024 * 64 + 10, n_plant=8,
                 plant_groups=4), 1, 0.0),
]
# per-head selection over the largest union bitmap: 65536 historical chunks
HEAD_LIMIT = SMALL.with_(B=1, Hkv=1, Hq=8, g=1, C=16, d=64, N=16 * 65536 + 7, k=50, n_plant=4)


@pytest.mark.parametrize("idx", range(len(LIMITS)), ids=[f"lim{i}" for i in range(len(LIMITS))])
def test_limit_shapes(idx):
    cfg, gmode, tp = LIMITS[idx]
    run_case(cfg, seed=500 + idx, gist_mode=gmode, top_p=tp)


def test_head_select_limit():
    run_case(HEAD_LIMIT, seed=520, head_select=1)


# One unit over many chunks: ~94 and ~141 gist slices, so the final merge takes its partials in
# several batches and (G * slots > 1024) its statistics from global memory, and the selection
# merge ranks more than 256 candidates with the radix path.
MANY_SLICES = [
    DecodeConfig("many_slices", B=1, Hq=8, Hkv=1, d=64, N=16 * 6000 + 5, C=16, g=1, k=8,
                 n_plant=4, paged=True),
    DecodeConfig("many_slices_big", B=1, Hq=8, Hkv=1, d=64, N=16 * 9000 + 3, C=16, g=1, k=8,
                 gate=1, n_plant=4, paged=True),
]


@pytest.mark.parametrize("idx", range(len(MANY_SLICES)), ids=["ms0", "ms1"])
def test_many_slices(idx):
    run_case(MANY_SLICES[idx], seed=700 + idx)


def test_radix_slice_selection():
    # 1024 units: one slice per unit holding all 400 chunks (g = 1), so each slice picks its
    # candidates with the radix select (more than 256 items); sampled units against the oracle
    cfg = DecodeConfig("radix_slices", B=128, Hq=16, Hkv=8, d=64, N=16 * 400 + 7, C=16, g=1,
                       k=8, gate=1, n_plant=4, paged=True)
    rng = np.random.default_rng(1)
    n = cfg.B * cfg.Hkv
    units = sorted(set(rng.choice(n, 96, replace=False).tolist()) | {0, n - 1})
    inp, call, st = run_case(cfg, seed=650, units=units)
    assert st["excused"] <= 1
    del inp, call
    torch.cuda.empty_cache()


def test_max_units():
    cfg = DecodeConfig("max_units", B=2048, Hq=16, Hkv=8, d=64, N=100, C=16, g=2, k=3,
                       n_plant=1, paged=True)
    rng = np.random.default_rng(0)
    n = cfg.B * cfg.Hkv   # 16384, the most one call takes
    units = sorted(set(rng.choice(n, 384, replace=False).tolist()) | {0, n - 1})
    inp, call, st = run_case(cfg, seed=600, units=units)
    assert st["units"] == len(units)
    del inp, call
    torch.cuda.empty_cache()


def test_deterministic_bitwise():
    cfg = configs.LLAMA1B
    inp = make_decode(cfg, 7, device=DEV)
    a = DecodeCall(inp)()
    b = DecodeCall(inp)()
    a()      # twice on the same workspace as well
    torch.cuda.synchronize()
    for x, y in ((a.out, b.out), (a.lse, b.lse), (a.sel, b.sel), (a.chunk_scores, b.chunk_scores)):
        assert torch.equal(x, y)


def test_permutation_invariance_gpu():
    cfg = SMALL.with_(gate=1)
    inp = make_decode(cfg, 55, device=DEV)
    a = DecodeCall(inp)()
    torch.cuda.synchronize()
    sel = a.sel.cpu().numpy()
    rng = np.random.default_rng(1)
    pt, gk, gv = inp.page_table.clone(), inp.gist_k.clone(), inp.gist_v.clone()
    for b in range(cfg.B):
        free = [c for c in range(cfg.H) if c not in set(sel[b].ravel().tolist())]
        perm = rng.permutation(free)
        pt[b, free] = inp.page_table[b, perm]
        gk[b, :, free] = inp.gist_k[b, :, perm]
        gv[b, :, free] = inp.gist_v[b, :, perm]
    b2 = DecodeCall(replace(inp, page_table=pt, gist_k=gk, gist_v=gv))()
    torch.cuda.synchronize()
    assert torch.equal(a.sel, b2.sel)
    assert (a.out - b2.out).abs().max().item() <= 1e-6
    assert (a.lse - b2.lse).abs().max().item() <= 1e-6


def test_bad_page_poisons_only_its_unit():
    cfg = SMALL
    inp = make_decode(cfg, 56, device=DEV)
    a = DecodeCall(inp)()
    torch.cuda.synchronize()
    c = int(a.sel[1, 0, 0])
    pt = inp.page_table.clone()
    pt[1, c] = inp.num_pages + 5
    b = DecodeCall(replace(inp, page_table=pt))()
    torch.cuda.synchronize()
    G = cfg.G
    heads_bad = [h for kv in range(cfg.Hkv) if c in a.sel[1, kv].tolist()
                 for h in range(kv * G, (kv + 1) * G)]
    assert torch.isnan(b.out[1, heads_bad]).all() and torch.isnan(b.lse[1, heads_bad]).all()
    good = [h for h in range(cfg.Hq) if h not in heads_bad]
    assert torch.equal(b.out[0], a.out[0]) and torch.equal(b.out[1, good], a.out[1, good])


def test_scale_override():
    cfg = SMALL.with_(gate=1)
    inp = make_decode(cfg, 57, device=DEV)
    call = DecodeCall(inp, scale=0.05)()
    torch.cuda.synchronize()
    check_decode(inp, call)


def test_workspace_reused_across_shapes():
    """One zero-initialised workspace serves calls of different shapes in turn: every call
    leaves its arrival counters at zero for the next."""
    from top_chunk_sparse_amd import ops
    cfgs = [SMALL.with_(levels=2, J=4, k2=3, k=6, n_plant=6, plant_groups=3),
            SMALL.with_(gate=1), SMALL.with_(d=64, k=3), SMALL.with_(gate=1, B=3)]
    calls = [DecodeCall(make_decode(c, 300 + i, device=DEV)) for i, c in enumerate(cfgs)]
    big = max(c.ws.numel() for c in calls)
    ws = ops.workspace(big, DEV)
    for rep in range(2):
        for call in calls:
            call.ws = ws
            call()
            torch.cuda.synchronize()
            check_decode(call.inp, call)


def test_repeated_calls_bitwise_identical_full_size():
    """40 back-to-back calls alternating two full-size (128K-token) instances: every result
    equals the first call's bit for bit (the cross-workgroup hand-off in the fused kernels
    sees complete data every time)."""
    cfg = configs.LLAMA8B
    insts = [make_decode(cfg, configs.seed_for(cfg.name, r), device=DEV) for r in range(2)]
    calls = [DecodeCall(i, with_scores=False) for i in insts]
    ref = []
    for c in calls:
        c()
        torch.cuda.synchronize()
        ref.append((c.out.clone(), c.lse.clone(), c.sel.clone()))
    for it in range(40):
        c = calls[it % 2]
        c()
        if it % 8 == 7:
            torch.cuda.synchronize()
            o, l, s = ref[it % 2]
            assert torch.equal(c.out, o) and torch.equal(c.lse, l) and torch.equal(c.sel, s), it
    torch.cuda.synchronize()
    del calls, insts
    torch.cuda.empty_cache()


# adaptive top-k: each level selects min(cap, floor(N / (L_eff G C)) + 1)
ADAPTIVE = [
    (SMALL.with_(N=300 * 32 + 5, k=6, gate=1), {}),                  # budget 3, under the cap
    (SMALL.with_(N=300 * 32 + 5, k=6, Hq=2, Hkv=2), {}),             # G = 1: budget 10, cap 6
    (SMALL.with_(N=300 * 32 + 5, k=6), dict(head_select=1)),         # per-head picks, union
    (SMALL.with_(N=300 * 32 + 5, k=6, gate=1), dict(gist_mode=1)),   # selected summaries
    (SMALL.with_(levels=2, J=4, k2=5, k=6, N=1250 * 32, n_plant=6, plant_groups=3), {}),
    (SMALL.with_(levels=2, J=4, k2=5, k=6, N=1250 * 32, n_plant=6, plant_groups=3),
     dict(gist_mode=1)),
    (SMALL.with_(N=100, k=3), {}),                                   # budget 1
]


def _adaptive_count(cfg):
    import oracle
    b = oracle.adaptive_k_budget(N=cfg.N, C_=cfg.C, Hq=cfg.Hq, Hkv=cfg.Hkv, levels=cfg.levels,
                                 J=cfg.J)
    return b, min(cfg.k, b), min(cfg.k2, b)


@pytest.mark.parametrize("idx", range(len(ADAPTIVE)), ids=[f"ak{i}" for i in range(len(ADAPTIVE))])
def test_adaptive_k_variants(idx):
    cfg, kw = ADAPTIVE[idx]
    inp, call, st = run_case(cfg, 800 + idx, adaptive_k=1, max_chunks=cfg.M + 2, **kw)
    b, k1, k2 = _adaptive_count(cfg)
    sel = call.sel.cpu().numpy()
    assert sel.shape[-1] == cfg.k * (cfg.G if kw.get("head_select") else 1)
    n = (sel >= 0).sum(-1)
    if cfg.levels == 2:
        assert ((call.sel_groups.cpu().numpy() >= 0).sum(-1) == min(k2, cfg.nG)).all()
        assert (n <= k1).all()
    elif kw.get("head_select"):
        assert ((n >= min(k1, cfg.H)) & (n <= min(cfg.G * k1, cfg.H))).all()
    else:
        assert (n == min(k1, cfg.H)).all()


@pytest.mark.parametrize("name", ["llama32_1b_decode_32k", "llama31_8b_decode_128k",
                                  "hssa_decode_512k"])
def test_adaptive_k_full(name):
    cfg = configs.DECODE_CONFIGS[name]
    inp, call, st = run_case(cfg, configs.seed_for(name), adaptive_k=1)
    assert st["excused"] <= max(1, st["units"] // 100)
    b, k1, k2 = _adaptive_count(cfg)
    n = (call.sel.cpu().numpy() >= 0).sum(-1)
    assert (n == (k1 if cfg.levels == 1 else min(k1, k2 * cfg.J))).all(), (b, k1, k2)
    del inp, call
    torch.cuda.empty_cache()
