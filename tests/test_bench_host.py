"""Host-side pieces of bench.py that need no GPU."""

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class _Buf:
    """Stands in for a device tensor: the probe size depends only on its byte count."""
    def __init__(self, n):
        self.n = n

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,M", [("up", 1), ("gate_up", 8), ("down", 8), ("qkv", 4), ("o_proj", 1),
                                    ("qkv_tp4", 4), ("o_proj_tp4", 4), ("lm_head", 8), ("gate_up_swiglu", 8)])
def test_read_probe_stays_inside_the_weight_buffers(name, M):
    """The probe reads whole 9216-byte blocks of the buffers the GEMM reads, and
    never past their end: for FP8 the weight bytes include the block scales,
    which are not in the code buffers."""
    from fp8_quantized_skinny_amd import synth
    bench = _bench()
    fmt, _, K, N = synth.WORKLOADS[name]
    if fmt == "fp8":
        buf_bytes = K * N
        wbytes = K * N + (-(-N // 128)) * (-(-K // 128)) * 4
    else:
        Ncols = 16 * (-(-N // 8)) if fmt == "swiglu" else N
        buf_bytes = 256 + (-(-Ncols // 16)) * (-(-K // 1024)) * 9216
        wbytes = Ncols * K // 2 + Ncols * K // 16 + (8 if fmt == "swiglu" else 4)
    size = bench.probe_size(wbytes, [_Buf(buf_bytes), _Buf(buf_bytes)])
    assert size % 9216 == 0 and 9216 <= size <= buf_bytes
    assert buf_bytes - size < 2 * 9216 + (wbytes - min(wbytes, buf_bytes)) + 9216


def test_read_probe_size_rejects_tiny_buffers():
    bench = _bench()
    with pytest.raises(ValueError):
        bench.probe_size(10**6, [_Buf(100)])


def test_more_than_one_gpu_is_refused_before_any_device_use():
    """--gpus N > 1 ends with status 2 and says why; it touches no GPU first."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,M,weight_bytes", [("up", 1, 50135044), ("gate_up", 8, 100270084),
                                                 ("down", 8, 50135044)])
def test_recorded_traffic_is_plausible_when_current(name, M, weight_bytes):
    """The HBM traffic bench.py reports comes from a committed counter summary
    taken on the current kernel sources.  When one exists, it must lie near the
    weight bytes (every byte read once; 2% below for the copy calibration's
    own error) and at most 1.2 times them (x, partial sums, line rounding)."""
    traffic = _bench().recorded_traffic(name, M)
    if traffic is None:
        pytest.skip(f"no counter summary for {name} M={M} on the current kernel sources")
    assert 0.98 * weight_bytes <= traffic <= 1.2 * weight_bytes


def test_cpu_model_is_a_name():
    name = _bench().cpu_model()
    assert isinstance(name, str) and name.strip()
