"""GPU parity of msa_attn_fwd_blocksparse (attention over listed 64-key
blocks per 128-row query block) through the C ABI against the fp64 oracle:
every row on small random lists (out-of-range and repeated indices, empty
lists, causal and not), sampled rows on the 128K band pattern and on the
128K global + local pattern."""
import math

import numpy as np
import pytest
import torch

import msa_inputs as wl
from oracle import msa_oracle as orc
from tests.gpu_util import TOL_BF16, assert_close, bf16_rne, dev, host64

pytestmark = pytest.mark.gpu

msa = pytest.importorskip("long_context_sparse_msa_amd")
BQ, BK = 128, 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()  # a missing library is an error, not a skip
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def rand(shape, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev())


CASES = [
    # B, Hq, Hkv, n, d, max_blocks, causal
    (2, 4, 2, 700, 128, 6, True),
    (2, 4, 2, 700, 128, 6, False),
    (1, 8, 1, 1024, 64, 12, True),
    (1, 2, 2, 64, 128, 3, False),
    (1, 2, 1, 2048, 128, 0, True),     # every list empty
]


@pytest.mark.parametrize("B,Hq,Hkv,n,d,maxb,causal", CASES)
def test_blocksparse_small(B, Hq, Hkv, n, d, maxb, causal):
    print(f"[case] blocksparse B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} max_blocks={maxb} causal={causal}", flush=True)
    Q, K, V = rand((B, Hq, n, d), 1), rand((B, Hkv, n, d), 2), rand((B, Hkv, n, d), 3)
    counts, idx = wl.random_block_lists(B, Hq, n, maxb, seed=n + maxb)
    if maxb == 0:
        idx = np.zeros((B, Hq, counts.shape[2], 1), np.int32)
    cd, id_ = torch.from_numpy(counts).to(dev()), torch.from_numpy(idx).to(dev())
    scale = 1.0 / math.sqrt(d)
    O32, L32 = msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, causal, scale, out_dtype=torch.float32)
    O16, _ = msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn_blocksparse(host64(Q), host64(K), host64(V), counts, idx, BQ, BK, causal, scale)
    live = np.isfinite(l_ref)
    o, l = host64(O32), host64(L32)
    assert (np.isneginf(l) == ~live).all()
    assert (o[~live] == 0).all()
    if live.any():
        assert_close(o[live], l[live], o_ref[live], l_ref[live], TOL_BF16, "blocksparse")
    assert torch.equal(O16, bf16_rne(O32))


def test_blocksparse_band_128k():
    cfg = wl.GQA_128K
    print(f"[case] blocksparse band pattern on {cfg.name}", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    counts, idx = wl.band_block_lists(cfg.batch, cfg.heads_q, cfg.seq_len)
    cd, id_ = torch.from_numpy(counts).to(dev()), torch.from_numpy(idx).to(dev())
    O32, L32 = msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, False, cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    grp = cfg.heads_q // cfg.heads_kv
    for h in (0, 17, 63):
        g = h // grp
        rows = wl.sample_rows(cfg.seq_len, h, count=512)
        res = orc.attn_blocksparse_rows(host64(Q[:, h:h + 1]), host64(K[:, g:g + 1]), host64(V[:, g:g + 1]),
                                        counts[:, h:h + 1], idx[:, h:h + 1], BQ, BK, False, cfg.scale,
                                        rows={0: rows})
        r, o_ref, l_ref = res[0]
        ridx = torch.from_numpy(r).to(dev())
        assert_close(host64(O32[:, h].index_select(1, ridx)), host64(L32[:, h].index_select(1, ridx)), o_ref, l_ref,
                     TOL_BF16, f"band 128k head {h} ({len(r)} rows)")


def test_blocksparse_global_local_128k():
    """Global + local lists at the 128K GQA shapes (non-causal): the first two
    128-token blocks attend to every key and every block attends to them,
    the rest see a 16-block local band.  Lists of very unequal length (2048
    key blocks for the global rows, 20-36 for the others); rows of the
    global blocks are graded among the sampled ones."""
    cfg = wl.GQA_128K
    print(f"[case] blocksparse global + local pattern on {cfg.name}", flush=True)
    Q, K, V = wl.device_prefill_inputs(cfg, dev())
    counts, idx = wl.global_local_block_lists(cfg.batch, cfg.heads_q, cfg.seq_len)
    cd, id_ = torch.from_numpy(counts).to(dev()), torch.from_numpy(idx).to(dev())
    O32, L32 = msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, False, cfg.scale, out_dtype=torch.float32)
    O16, _ = msa.msa_attn_fwd_blocksparse(Q, K, V, cd, id_, False, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(O16, bf16_rne(O32))
    grp = cfg.heads_q // cfg.heads_kv
    for h in (0, 40, 63):
        g = h // grp
        rows = np.unique(np.concatenate([wl.sample_rows(cfg.seq_len, h, count=256),
                                         np.array([3, 127, 128, 200, 255, 256, 257, 1100])]))
        res = orc.attn_blocksparse_rows(host64(Q[:, h:h + 1]), host64(K[:, g:g + 1]), host64(V[:, g:g + 1]),
                                        counts[:, h:h + 1], idx[:, h:h + 1], BQ, BK, False, cfg.scale,
                                        rows={0: rows})
        r, o_ref, l_ref = res[0]
        ridx = torch.from_numpy(r).to(dev())
        assert_close(host64(O32[:, h].index_select(1, ridx)), host64(L32[:, h].index_select(1, ridx)), o_ref, l_ref,
                     TOL_BF16, f"global+local 128k head {h} ({len(r)} rows)")
    del Q, K, V, O32, L32, O16, cd, id_
