"""GPU parity of the prefill backward (gradients of sum dout . out + sum dlse . lse with respect
to q, k, v and the selector scores S) against the fp64 oracle, through the C ABI.

The GPU rounds P and dS to bf16 as MFMA operands (relative error 2^-9 each) and accumulates
in fp32, so each gradient element carries an error of about 2^-9 times the root-sum-square of
its terms, well under 1% of the tensor's largest magnitude; dq, dk, dv and dS are compared by
max-abs error over the tensor's max-abs (REL_TOL).  At the full 16K-token size the gradients are
checked element by element on a prefix of query blocks (the rest of dout and dlse set to zero,
so the oracle only needs that prefix), and through identities that hold at any size."""
import sys

import numpy as np
import pytest
import torch

from top_chunk_sparse_amd import configs
from top_chunk_sparse_amd.configs import PrefillConfig
from top_chunk_sparse_amd.ops import PrefillBwdCall, PrefillCall
from top_chunk_sparse_amd.synth import make_prefill, make_prefill_grads
from harness import oracle_prefill_backward

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, want):
    scale = max(np.abs(want).max(), 1e-30)
    return float(np.abs(got - want).max() / scale)


def run_bwd(cfg, seed, with_dlse=True, with_dS=True):
    say(f"[prefill-bwd] {cfg.name} seed={seed} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} T={cfg.T} "
        f"k={cfg.k} gate={cfg.gate} dlse={with_dlse} dS={with_dS}")
    inp = make_prefill(cfg, seed, device=DEV)
    dout, dlse = make_prefill_grads(cfg, seed, device=DEV)
    dlse = dlse if with_dlse else None
    fwd = PrefillCall(inp)()
    bwd = PrefillBwdCall(inp, fwd, dout, dlse, with_dS=with_dS)()
    torch.cuda.synchronize()
    return inp, dout, dlse, fwd, bwd


def compare(inp, dout, dlse, bwd, with_dS=True):
    ref = oracle_prefill_backward(inp, dout, dlse)
    errs = {"dq": rel_err(bwd.dq.cpu().double().numpy(), ref.dq),
            "dk": rel_err(bwd.dk.cpu().double().numpy(), ref.dk),
            "dv": rel_err(bwd.dv.cpu().double().numpy(), ref.dv)}
    if with_dS:
        gS = bwd.dS.cpu().double().numpy()
        if np.abs(ref.dS).max() == 0:
            errs["dS"] = float(np.abs(gS).max())   # gate off or nothing chosen: exactly zero
        else:
            errs["dS"] = rel_err(gS, ref.dS)
    say("    rel max-abs errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= REL_TOL, (k, v)
    return errs


BASE = PrefillConfig("bwd_small", B=1, Hq=8, Hkv=2, d=128, T=64 * 6, blk=64, k=2, gate=1)
CASES = [
    (BASE, True),
    (BASE.with_(Hq=16, k=3), True),                 # G = 8: two head groups
    (BASE.with_(Hq=2, Hkv=2), True),                # G = 1
    (BASE.with_(Hq=4, T=64 * 9, k=4), True),        # G = 2
    (BASE.with_(gate=0), True),                     # no gate: dS = 0
    (BASE.with_(k=0), True),                        # diagonal blocks only
    (BASE.with_(k=100), True),                      # every earlier block
    (BASE, False),                                  # no dlse
    (BASE.with_(B=2, T=64 * 4), True),
    (BASE.with_(T=64), True),                       # one block
    # 128 dk / dv and 512 dq workgroups with two head groups: more than the GPU holds at
    # once, so the gradient grid's dq part starts as the dk / dv part drains
    (BASE.with_(Hq=16, T=64 * 64, k=4), True),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[f"bw{i}" for i in range(len(CASES))])
def test_prefill_backward_small(idx):
    cfg, with_dlse = CASES[idx]
    inp, dout, dlse, fwd, bwd = run_bwd(cfg, seed=900 + idx, with_dlse=with_dlse)
    errs = compare(inp, dout, dlse, bwd)
    if cfg.gate == 0 or cfg.k == 0:
        assert errs["dS"] == 0.0


def test_prefill_backward_without_dS():
    inp, dout, dlse, fwd, bwd = run_bwd(BASE.with_(k=3), seed=920, with_dS=False)
    compare(inp, dout, dlse, bwd, with_dS=False)


def test_prefill_backward_2k_workload_heads():
    """The 16K workload's head layout (32 query heads over 8 KV heads, k = 16) at 2K tokens,
    against the oracle on every element."""
    cfg = configs.PREFILL.with_(T=2048)
    inp, dout, dlse, fwd, bwd = run_bwd(cfg, seed=930)
    compare(inp, dout, dlse, bwd)


def test_prefill_backward_full_size_identities():
    """At 16K tokens: per KV head the dv rows add up to the group's dout rows and the dk rows to
    sigma sum dlse q (each query row's weights sum to one); every dS row sums to zero and dS is
    zero on and above the diagonal; repeated calls give the same bits."""
    cfg = configs.PREFILL
    inp, dout, dlse, fwd, bwd = run_bwd(cfg, seed=configs.seed_for(cfg.name))
    G, sig = cfg.G, 1.0 / np.sqrt(cfg.d)
    dv = bwd.dv.double().sum(2).cpu().numpy()          # [B][Hkv][d]
    dk = bwd.dk.double().sum(2).cpu().numpy()
    go = dout.double().sum(2).view(cfg.B, cfg.Hkv, G, cfg.d).sum(2).cpu().numpy()
    qd = (inp.q.double() * dlse.double()[..., None]).sum(2)
    want_dk = sig * qd.view(cfg.B, cfg.Hkv, G, cfg.d).sum(2).cpu().numpy()
    e_dv = float(np.abs(dv - go).max() / np.abs(go).max())
    e_dk = float(np.abs(dk - want_dk).max() / np.abs(want_dk).max())
    dS = bwd.dS.double()
    rows = dS.sum(-1).abs().max().item() / dS.abs().sum(-1).max().item()
    upper = torch.triu(dS, 0).abs().max().item()
    say(f"    identities: dv {e_dv:.2e}  dk {e_dk:.2e}  dS row sums {rows:.2e}  upper {upper}")
    assert e_dv < 1e-3 and e_dk < 2e-2 and rows < 1e-4 and upper == 0.0
    # every call gives the same bits (a hand-off through LDS that races shows up here first)
    names = ("dq", "dk", "dv", "dS")
    first = [t.clone() for t in (bwd.dq, bwd.dk, bwd.dv, bwd.dS)]
    for call in range(3):
        bwd()
        torch.cuda.synchronize()
        for n, a, b in zip(names, first, (bwd.dq, bwd.dk, bwd.dv, bwd.dS)):
            bad = (a != b).nonzero()
            assert bad.shape[0] == 0, (call, n, bad.shape[0], bad[:4].tolist())


def test_prefill_backward_workspace_garbage_and_reuse():
    """The backward reads only workspace it wrote in the same call: a workspace full of 0xFF
    bytes (NaN patterns), first used by a call of another shape, gives the same bits."""
    big = BASE.with_(T=64 * 9, k=4, Hq=16)
    inp, dout, dlse, fwd, bwd = run_bwd(BASE.with_(k=3), seed=940)
    ref = [t.clone() for t in (bwd.dq, bwd.dk, bwd.dv, bwd.dS)]
    inp2, dout2, dlse2, fwd2, bwd2 = run_bwd(big, seed=941)
    ws = torch.full((max(bwd.ws.numel(), bwd2.ws.numel()),), 255, dtype=torch.uint8, device=DEV)
    bwd2.ws = ws
    bwd2()                      # another shape first, on the shared workspace
    bwd.ws = ws
    bwd()
    torch.cuda.synchronize()
    for a, b in zip(ref, (bwd.dq, bwd.dk, bwd.dv, bwd.dS)):
        assert torch.equal(a, b)


def test_prefill_backward_full_size_elementwise_prefix():
    """The 16K workload in its full launch configuration, element by element: dout and dlse are
    zero outside the first NB query blocks, so every query row past them has dlambda = 0 and
    contributes nothing.  dk and dv (all rows) then equal the oracle's gradients of the first NB
    blocks; dq and dS equal them on those blocks' rows and are exactly zero past them."""
    NB = 32
    cfg = configs.PREFILL
    seed = configs.seed_for(cfg.name)
    say(f"[prefill-bwd] {cfg.name} seed={seed} full size, dout / dlse kept on {NB} blocks")
    inp = make_prefill(cfg, seed, device=DEV)
    dout, dlse = make_prefill_grads(cfg, seed, device=DEV)
    rows = NB * cfg.blk
    dout[:, :, rows:] = 0
    dlse[:, :, rows:] = 0
    fwd = PrefillCall(inp)()
    bwd = PrefillBwdCall(inp, fwd, dout, dlse, with_dS=True)()
    torch.cuda.synchronize()
    ref = oracle_prefill_backward(inp, dout, dlse, n_blocks=NB)
    gq = bwd.dq.cpu().double().numpy()
    gS = bwd.dS.cpu().double().numpy()
    errs = {"dq": rel_err(gq[:, :, :rows], ref.dq[:, :, :rows]),
            "dk": rel_err(bwd.dk.cpu().double().numpy(), ref.dk),
            "dv": rel_err(bwd.dv.cpu().double().numpy(), ref.dv),
            "dS": rel_err(gS[:, :, :NB], ref.dS[:, :, :NB])}
    say("    rel max-abs errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= REL_TOL, (k, v)
    assert (gq[:, :, rows:] == 0).all() and (gS[:, :, NB:] == 0).all()
    # the chosen key blocks of the first NB query blocks are earlier blocks: nothing past them
    assert (bwd.dk[:, :, rows:] == 0).all().item() and (bwd.dv[:, :, rows:] == 0).all().item()


def test_prefill_backward_multi_pass_inverse_lists():
    """More than 257 blocks (T = 272 x 64) with two KV heads: the chosen-by lists are compacted
    in several passes of the block scan; every element against the oracle."""
    cfg = PrefillConfig("bwd_long", B=1, Hq=4, Hkv=2, d=128, T=64 * 272, blk=64, k=4, gate=1)
    inp, dout, dlse, fwd, bwd = run_bwd(cfg, seed=950)
    compare(inp, dout, dlse, bwd)
