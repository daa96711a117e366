"""The byte and FLOP counts behind the bench's roofline figures, checked on the CPU against
numbers that do not come from the same formulas: the per-call totals of the workloads as the
hot-path scope table states them (decode at 128K tokens, the 16K SAS prefill), and brute-force
counts of attended pairs from the visibility rules themselves on small shapes."""
import numpy as np

import bench
from top_chunk_sparse_amd import configs


def test_decode_bytes_of_the_128k_workload():
    # 411,181,568 bytes per call: gist K+V 268,173,312; selected chunks 134,217,728; current
    # chunk 8,388,608; q 131,072; out 262,144; page-table entries 8,704
    total, parts = bench.decode_bytes(configs.LLAMA8B)
    assert total == 411_181_568
    assert parts["gists_kv"] == 268_173_312
    assert parts["selected_kv"] == 134_217_728
    assert parts["current_kv"] == 8_388_608
    assert parts["q"] == 131_072 and parts["out"] == 262_144 and parts["page_table"] == 8_704
    # the gist-scoring kernel: every historical gist row (K and V) of every unit, plus q
    assert bench.gist_kernel_bytes(configs.LLAMA8B) == 268_173_312 + 131_072


def test_decode_bytes_of_the_other_workloads():
    assert bench.decode_bytes(configs.LLAMA1B)[0] == 76_515_584
    assert bench.decode_bytes(configs.HSSA)[0] == 90_280_064
    assert bench.decode_bytes(configs.TINY)[0] == 99_604


def test_prefill_pairs_and_flops_of_the_16k_workload():
    # per head: sum_i min(16, i) = 3,960 whole 64 x 64 blocks and 256 diagonal blocks of 2,080
    # causal pairs; 32 heads
    assert bench.prefill_pairs(configs.PREFILL) == 536_084_480
    assert bench.prefill_flops(configs.PREFILL) == 274_475_253_760
    assert bench.prefill_bwd_flops(configs.PREFILL) == 686_188_134_400


def _brute_prefill_pairs(cfg):
    """Attended pairs from the block rule: a row of block i sees min(k, i) earlier blocks in
    full (which ones does not change the count) and the keys up to itself in its own block."""
    n = 0
    for i in range(cfg.nb):
        for r in range(cfg.blk):
            n += min(cfg.k, i) * cfg.blk + (r + 1)
    return cfg.B * cfg.Hq * n


def test_prefill_pairs_brute_force():
    for cfg in (configs.PREFILL.with_(T=64 * 7, k=3), configs.PREFILL.with_(T=64 * 5, k=0),
                configs.PREFILL.with_(B=2, Hq=8, Hkv=2, T=64 * 9, k=100)):
        assert bench.prefill_pairs(cfg) == _brute_prefill_pairs(cfg)


def _brute_gist_pairs(cfg):
    """Attended pairs from the gist mask: position x is visible to position p when x <= p and
    x lies in p's chunk or is a gist token.  Split into raw and gist query rows."""
    W = cfg.L + cfg.g
    p = np.arange(cfg.M * W)
    chunk = p // W
    is_gist = (p % W) >= cfg.L
    vis = (p[None, :] <= p[:, None]) & ((chunk[None, :] == chunk[:, None]) | is_gist[None, :])
    per_row = vis.sum(axis=1)
    heads = cfg.B * cfg.Hq
    return heads * int(per_row[~is_gist].sum()), heads * int(per_row[is_gist].sum())


def test_gist_prefill_pairs_brute_force():
    for kw in (dict(M=5, L=64, g=4), dict(M=3, L=128, g=1), dict(M=7, L=64, g=16),
               dict(M=1, L=64, g=2)):
        cfg = configs.GIST_PREFILL.with_(**kw)
        assert bench.gist_prefill_pairs(cfg) == _brute_gist_pairs(cfg), kw


def test_gist_prefill_row_bytes():
    cfg = configs.GIST_PREFILL   # 16K raw tokens: 128 chunks of 128 + 4 gists
    q = 32 * 16_896 * 128 * 2            # bf16 q, every position
    raw_kv = 8 * 128 * 128 * 128 * 2 * 2  # bf16 raw K and V rows
    gist_kv = 8 * 512 * 128 * 2 * 2       # gathered gists: 512 rows per KV head, K and V
    out_lse = 32 * 16_896 * (128 + 1) * 4
    assert bench.gist_prefill_row_bytes(cfg) == q + raw_kv + gist_kv + out_lse == 486_604_800
