"""The Python binding refuses tensors that do not fit the call -- wrong
shape, dtype or device, landmarks pooled with another G, outputs of the
wrong type -- with a ValueError raised before the library launches
anything.  The library receives raw device pointers, so such a tensor would
otherwise become an out-of-bounds device access.  Runs on the CPU: the
library object is replaced by one that fails the test if a compute entry
point is reached."""
import pytest
import torch

msa = pytest.importorskip("long_context_sparse_msa_amd")
from long_context_sparse_msa_amd import binding  # noqa: E402

HOST_ONLY = {"msa_decode_workspace_size", "msa_attn_bwd_workspace_size", "msa_status_string", "msa_last_error",
             "msa_plan_rows", "msa_plan_tiles", "msa_plan_decode", "msa_plan_decode_varlen", "msa_abi_version"}


class NoLaunch:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name not in HOST_ONLY:
            raise AssertionError(f"{name} was called although validation should have failed first")
        return getattr(self._real, name)


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    real = binding.lib()
    monkeypatch.setattr(binding, "lib", lambda: NoLaunch(real))


bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
B, Hq, Hkv, n, d, w, G = 1, 4, 2, 256, 128, 64, 4


def t(*shape, dtype=bf, device="cpu"):
    return torch.zeros(shape, dtype=dtype, device=device)


def prefill_args(**over):
    a = dict(Q=t(B, Hq, n, d), K=t(B, Hkv, n, d), V=t(B, Hkv, n, d), Kbar=t(B, Hkv, G, d), Vbar=t(B, Hkv, G, d))
    a.update(over)
    return a


def run_fwd(**over):
    a = prefill_args(**over)
    O = over.get("O")
    LSE = over.get("LSE")
    return msa.msa_attn_fwd(a["Q"], a["K"], a["V"], a["Kbar"], a["Vbar"], w, G, O=O, LSE=LSE,
                            out_dtype=over.get("out_dtype"))


def test_prefill_on_host_memory_is_refused():
    with pytest.raises(ValueError, match="GPU memory"):
        run_fwd()


@pytest.mark.parametrize("over,msg", [
    (dict(Kbar=t(B, Hkv, 2 * G, d)), "Kbar has shape"),              # pooled with another G
    (dict(Vbar=t(B, Hkv, G, d, dtype=f32)), "Vbar has dtype"),
    (dict(Kbar=None), "Kbar is required"),
    (dict(O=t(B, Hq, n, d, dtype=f32)), "O has dtype"),               # bf16 output requested
    (dict(O=t(B, Hq, n, d), out_dtype=f32), "O has dtype"),
    (dict(O=t(B, Hq, n - 1, d)), "O has shape"),
    (dict(LSE=t(B, Hq, n, dtype=bf)), "LSE has dtype"),
    (dict(LSE=t(B, Hq, n + 1, dtype=f32)), "LSE has shape"),
])
def test_prefill_mismatch_is_refused(over, msg):
    with pytest.raises(ValueError, match=msg):
        run_fwd(**over)


def test_prefill_mixed_devices_is_refused():
    meta = t(B, Hkv, n, d, device="meta")
    with pytest.raises(ValueError, match="GPU memory"):
        run_fwd(K=meta)


def test_pool_refuses_wrong_landmark_buffers():
    K, V = t(B, Hkv, n, d), t(B, Hkv, n, d)
    with pytest.raises(ValueError, match="Kbar has shape"):
        msa.msa_pool_landmarks(K, V, G, t(B, Hkv, G + 1, d), t(B, Hkv, G, d))
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_pool_landmarks(K, V, G)


def test_blocksparse_refuses_host_lists():
    T = n // 128
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_attn_fwd_blocksparse(t(B, Hq, n, d), t(B, Hkv, n, d), t(B, Hkv, n, d), t(B, Hq, T, dtype=i32),
                                     t(B, Hq, T, 3, dtype=i32), True)


def test_backward_refuses_wrong_gradients():
    a = prefill_args()
    O, LSE, dO = t(B, Hq, n, d), t(B, Hq, n, dtype=f32), t(B, Hq, n, d)
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_attn_bwd(a["Q"], a["K"], a["V"], a["Kbar"], a["Vbar"], O, LSE, dO, w, G)
    with pytest.raises(ValueError, match="Kbar has shape"):
        msa.msa_attn_bwd(a["Q"], a["K"], a["V"], t(B, Hkv, 1, d), a["Vbar"], O, LSE, dO, w, G)


def dec_args():
    C = 512
    return dict(q=t(2, 8, d), Kc=t(2, 2, C, d), Vc=t(2, 2, C, d), Kbar=t(2, 2, 8, d), Vbar=t(2, 2, 8, d))


@pytest.mark.parametrize("over,msg", [
    (dict(), "GPU memory"),
    (dict(Kbar=t(2, 2, 16, d)), "Kbar has shape"),
    (dict(O=t(2, 8, d, dtype=f32)), "O has dtype"),
    (dict(LSE=t(2, 9, dtype=f32)), "LSE has shape"),
])
def test_decode_mismatch_is_refused(over, msg):
    a = dec_args()
    a.update({k: v for k, v in over.items() if k in a})
    with pytest.raises(ValueError, match=msg):
        msa.msa_decode_fwd(a["q"], a["Kc"], a["Vc"], a["Kbar"], a["Vbar"], 64, 8, 4, O=over.get("O"),
                           LSE=over.get("LSE"))


def test_varlen_decode_and_append_refuse_host_lengths():
    a = dec_args()
    lens = t(2, dtype=i32)
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_decode_fwd_varlen(a["q"], a["Kc"], a["Vc"], a["Kbar"], a["Vbar"], lens, 64, 8, 4)
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_append_kv(t(2, 2, d), t(2, 2, d), lens, a["Kc"], a["Vc"], a["Kbar"], a["Vbar"], 8)
    with pytest.raises(ValueError, match="Vbar has shape"):
        msa.msa_append_kv(t(2, 2, d), t(2, 2, d), lens, a["Kc"], a["Vc"], a["Kbar"], t(2, 2, 4, d), 8)


def test_paged_calls_refuse_host_tables():
    pool = t(16, 2, 64, d)
    table = t(2, 8, dtype=i32)
    lens = t(2, dtype=i32)
    a = dec_args()
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_decode_fwd_paged(a["q"], pool, pool, table, a["Kbar"], a["Vbar"], lens, 64, 8, 4)
    with pytest.raises(ValueError, match="GPU memory"):
        msa.msa_append_kv_paged(t(2, 2, d), t(2, 2, d), lens, pool, pool, table, a["Kbar"], a["Vbar"], 8)
