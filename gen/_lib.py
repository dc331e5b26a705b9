"""ctypes loaders and the build step for the generator libraries."""
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_DIR, "libmoegen_host.so")
DEV_SO = os.path.join(_DIR, "libmoegen_dev.so")
HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-shared", "-fPIC"]


def build(verbose=False):
    """Compile the host generator with gcc and the device generator with hipcc."""
    cmds = [
        ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", HOST_SO, os.path.join(_DIR, "moegen_host.c")],
        ["hipcc", *HIP_FLAGS, "-o", DEV_SO, os.path.join(_DIR, "moegen_dev.hip")],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("generator build failed: %s\n%s" % (" ".join(c), r.stderr))
        if verbose and r.stderr:
            print(r.stderr)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            raise RuntimeError("generator host library missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(HOST_SO)
        u64, i64, u32, f64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
        lib.moegen_fill_f32.argtypes = [vp, u64, i64, u32, u32, f64]
        lib.moegen_fill_bf16.argtypes = [vp, u64, i64, u32, u32, f64]
        lib.moegen_fill_u32.argtypes = [vp, u64, i64, u32, u32]
        lib.moegen_philox.argtypes = [vp, u32, u32, vp]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_SO):
            raise RuntimeError("generator device library missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(DEV_SO)
        u64, i64, u32, f64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
        for f in (lib.moegen_dev_fill_f32, lib.moegen_dev_fill_bf16):
            f.argtypes = [vp, u64, i64, u32, u32, f64, vp]
            f.restype = ctypes.c_int
        _dev = lib
    return _dev


def host_philox(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    _host_lib().moegen_philox(c.ctypes.data, int(key[0]), int(key[1]), o.ctypes.data)
    return o


def host_u32(start, count, seed, stream):
    o = np.empty(count, dtype=np.uint32)
    _host_lib().moegen_fill_u32(o.ctypes.data, start, count, seed, stream)
    return o


def host_fill(start, count, seed, stream, scale, bf16):
    """Elements [start, start+count) of a stream: uint16 bf16 bits, or float32."""
    lib = _host_lib()
    if bf16:
        o = np.empty(count, dtype=np.uint16)
        lib.moegen_fill_bf16(o.ctypes.data, start, count, seed, stream, scale)
    else:
        o = np.empty(count, dtype=np.float32)
        lib.moegen_fill_f32(o.ctypes.data, start, count, seed, stream, scale)
    return o


def device_fill(ptr, start, count, seed, stream, scale, bf16, hip_stream=0):
    lib = _dev_lib()
    f = lib.moegen_dev_fill_bf16 if bf16 else lib.moegen_dev_fill_f32
    rc = f(ptr, start, count, seed, stream, scale, hip_stream)
    if rc != 0:
        raise RuntimeError("device generator launch failed (%d)" % rc)


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
