"""bench.py's measured references (libmsa_ref.so) run on the GPU and report
sane figures: a short launch of each stream completes and its FLOP count is
the one the stream's shape implies."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "long_context_sparse_msa_amd",
                    "libmsa_ref.so")


@pytest.mark.parametrize("mode", [0, 1], ids=["register", "chain"])
def test_reference_stream_runs(mode):
    assert os.path.exists(PATH), "libmsa_ref.so is not built"
    ref = ctypes.CDLL(PATH)
    f = ref.msa_ref_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                  ctypes.POINTER(ctypes.c_double)]
    ms, flops = ctypes.c_double(), ctypes.c_double()
    print(f"[case] msa_ref_mfma mode {mode}", flush=True)
    assert f(mode, 20, 2, ctypes.byref(ms), ctypes.byref(flops)) == 0
    assert flops.value == 32 * 32768.0 * 20 * 2048 * 4
    tflops = flops.value / (ms.value * 1e-3) / 1e12
    print(f"[info] mode {mode}: {ms.value:.3f} ms, {tflops:.0f} TFLOP/s", flush=True)
    assert 0 < ms.value < 1000 and 50 < tflops < 2600
