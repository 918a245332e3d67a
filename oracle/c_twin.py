"""Loader of the oracle's plain C twin (oracle_c.c): the FP8 block
quantisation and the fp32 slot-order combine, computed with C's own
arithmetic for parity checks at full workload sizes.

TEST INFRASTRUCTURE ONLY, like the rest of this folder. The library is
compiled with gcc into this folder (build(), also called by the package's
build step, or on first use when it is missing); it shares nothing with the
HIP library. The numpy oracle stays the definition: the CPU tests check these
functions against it bit for bit."""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_c.c")
LIB = os.path.join(HERE, "liboracle_c.so")

# -ffp-contract=off: every multiply and add rounds where the source says;
# fmaf() is the only fused operation. No fast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-Wall"]

_lib = None


def build() -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True,
                   capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        L.oc_quantize_fp8.argtypes = [i64, i64, p, p, p]
        L.oc_quantize_fp8.restype = None
        L.oc_combine.argtypes = [i64, i64, i64, i64, p, p, p, p, p]
        L.oc_combine.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize_fp8_blocks(x_bits: np.ndarray):
    """Same result as moe_oracle.quantize_fp8_blocks: codes [T, H] uint8 and
    scales [T, H/128] fp32."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    t, h = x.shape
    assert h % 128 == 0
    codes = np.empty((t, h), np.uint8)
    scales = np.empty((t, h // 128), np.float32)
    if t:
        lib().oc_quantize_fp8(t, h, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def combine(y_bits: np.ndarray, dst_row: np.ndarray, topk_w) -> np.ndarray:
    """Same bits as moe_oracle.combine(...)[0]; topk_w None means unit
    weights (moe_oracle.dispatch_backward)."""
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    d = np.ascontiguousarray(dst_row, dtype=np.int32)
    t, k = d.shape
    h = y.shape[1]
    out = np.empty((t, h), np.uint16)
    acc = np.empty(h, np.float32)
    w = None if topk_w is None else np.ascontiguousarray(topk_w, dtype=np.float32)
    if t:
        lib().oc_combine(t, h, k, y.shape[0], _ptr(y), _ptr(d),
                         None if w is None else _ptr(w), _ptr(out), _ptr(acc))
    return out
