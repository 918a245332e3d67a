"""Every fp32 pattern through the two hardware converts the kernels use,
compared on the device with integer rounding references (tests/hip/
convert_sweep.hip):

  * the bf16 pack-convert that rounds every combine output (v_cvt_pk_bf16_f32)
    must round to nearest even on all 2^32 patterns (NaN gives NaN);
  * the clamped FP8 pack-convert behind the FP8 and MXFP8 dispatch codes
    (v_cvt_pk_fp8_f32 after a clamp to +-448) and the software e4m3 rounding
    of the overflowing-multiplier path must give the e4m3fn code, rounded to
    nearest even and saturated at 448, of every non-NaN pattern.

The kernel counts mismatches and keeps the smallest mismatching pattern;
it always runs to completion."""

import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hip", "libconvert_sweep.so")


def test_converts_on_every_fp32_pattern():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libconvert_sweep.so is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.convert_sweep.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.convert_sweep.restype = ctypes.c_int
    res = torch.tensor([0, -1, 0, -1, 0, -1, 0, 0], dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.convert_sweep(ctypes.c_void_p(res.data_ptr()), ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    r = [int(v) & 0xFFFFFFFFFFFFFFFF for v in res.cpu().tolist()]
    print("bf16 mismatches %d, FP8 pack-convert mismatches %d, software e4m3 mismatches %d, "
          "non-NaN patterns %d" % (r[0], r[2], r[4], r[6]), flush=True)
    assert r[6] == (1 << 32) - 2 * ((1 << 23) - 1), "not every pattern was checked"
    assert r[0] == 0, "bf16 pack-convert differs first at fp32 pattern 0x%08x" % r[1]
    assert r[2] == 0, "FP8 pack-convert differs first at fp32 pattern 0x%08x" % r[3]
    assert r[4] == 0, "software e4m3 rounding differs first at fp32 pattern 0x%08x" % r[5]
