"""The allocation-free decode (msa_decode_fwd_noalloc) through the C ABI
against msa_decode_fwd with a caller workspace, on the same inputs: the same
kernels, so the results must be identical bit for bit.  Two calls in a row,
the second with a smaller problem (fewer partials than the array holds from
the first call), under the split schedule that uses the library's array,
then under the automatic choice."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

msa = pytest.importorskip("long_context_sparse_msa_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()  # a missing library is an error, not a skip
    yield
    torch.cuda.synchronize()


def inputs(B, Hq, Hkv, ctx, d, G, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    mk = lambda *s: torch.randn(s, generator=g, dtype=torch.float32).to(torch.bfloat16).cuda()  # noqa: E731
    q, Kc, Vc = mk(B, Hq, d), mk(B, Hkv, ctx, d), mk(B, Hkv, ctx, d)
    Kb, Vb = msa.msa_pool_landmarks(Kc, Vc, G) if G else (None, None)
    return q, Kc, Vc, Kb, Vb


CASES = [
    # B, Hq, Hkv, ctx, d, w, G, S -- the second smaller than the first
    (4, 16, 2, 8192, 128, 1024, 8, 32),
    (2, 8, 1, 2048, 64, 300, 16, 7),
]


@pytest.mark.parametrize("schedule", ["split", "auto"])
def test_noalloc_decode_equals_workspace_decode(schedule):
    for k, (B, Hq, Hkv, ctx, d, w, G, S) in enumerate(CASES):
        print(f"[case] noalloc decode {schedule} B={B} Hq={Hq} Hkv={Hkv} ctx={ctx} d={d} w={w} G={G} S={S}",
              flush=True)
        q, Kc, Vc, Kb, Vb = inputs(B, Hq, Hkv, ctx, d, G, seed=100 + k)
        scale = 1.0 / math.sqrt(d)
        sch = None if schedule == "auto" else schedule
        O_ref, L_ref = msa.msa_decode_fwd(q, Kc, Vc, Kb, Vb, w, G, S, scale, schedule=sch)
        O = torch.empty_like(O_ref)
        LSE = torch.empty_like(L_ref)
        msa.msa_decode_fwd_noalloc(q, Kc, Vc, Kb, Vb, w, G, S, scale, O=O, LSE=LSE, schedule=sch)
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref), (schedule, k)
        assert torch.equal(LSE, L_ref), (schedule, k)
