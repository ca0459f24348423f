"""Host-side behaviour of bench.py's command line (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    """The library runs on one GPU: a request for several exits with status 2
    and a message, before anything touches a device."""
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and "--gpus 2" in p.stderr
    assert p.stdout == ""


def test_ceiling_library_host_side():
    """The measured-ceiling library that bench.py loads: it exports the three
    entry points bench.py calls, reports the int8 ops of one probe iteration
    (16 MFMAs of 32x32x32, or 32 of 16x16x64, per wave), and rejects an
    unknown instruction form or stream variant, or a size that the stream
    shape does not divide, before launching anything."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "int8_mixed_precision_amd", "libceiling.so"))
    for name in ("ceiling_mfma_i8", "ceiling_mfma_ops_per_iter", "ceiling_stream"):
        assert hasattr(lib, name), name
    assert lib.ceiling_mfma_ops_per_iter() == 16 * 32 * 32 * 32 * 2 == 32 * 16 * 16 * 64 * 2
    vp, ci, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.ceiling_mfma_i8.argtypes = [ci, ci, ci, vp, vp, vp]
    lib.ceiling_stream.argtypes = [vp, i64, ci, ci, vp, vp, vp]
    fake = vp(0x1000)
    assert lib.ceiling_mfma_i8(2, 1, 1, fake, fake, None) == 2
    assert lib.ceiling_mfma_i8(-1, 1, 1, fake, fake, None) == 2
    assert lib.ceiling_stream(fake, 1 << 20, 4, 4, fake, fake, None) == 2       # unknown variant
    assert lib.ceiling_stream(fake, 1 << 20, 0, 0, fake, fake, None) == 2       # no workgroups
    assert lib.ceiling_stream(fake, 16 * 4097, 1, 0, fake, fake, None) == 2     # not divisible
