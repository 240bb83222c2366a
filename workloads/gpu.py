"""GPU side of the counter-based value generator (libpkvgen.so, built from gen.hip).

Test and benchmark infrastructure: fills device buffers with the same values as
`workloads.hash_values`, bit for bit, so large workloads need no host generation."""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import shutil

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gen.hip")
LIB = os.path.join(HERE, "libpkvgen.so")
_lib = None


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    arch = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={arch}", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"libpkvgen build failed\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built: run `python -m workloads.gpu`")
        L = C.CDLL(LIB)
        L.pkvgen_fill.restype = C.c_int
        L.pkvgen_fill.argtypes = [C.c_void_p, C.c_int, C.c_uint64, C.c_int64, C.c_int64, C.c_float, C.c_void_p]
        L.pkvgen_fill_segments.restype = C.c_int
        L.pkvgen_fill_segments.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_int64, C.c_float, C.c_void_p]
        L.pkvgen_read_probe.restype = C.c_int
        L.pkvgen_read_probe.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.pkvgen_read_probe_stream.restype = C.c_int
        L.pkvgen_read_probe_stream.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def fill(t, key: int, e0: int, sigma: float = 1.0) -> None:
    """Fill contiguous device tensor t (float32 or bfloat16) with elements e0.. of stream key."""
    import torch
    if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("contiguous float32/bfloat16 device tensor expected")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib().pkvgen_fill(C.c_void_p(t.data_ptr()), int(t.dtype == torch.bfloat16), C.c_uint64(key),
                           int(e0), t.numel(), float(sigma), C.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"pkvgen_fill failed ({rc})")


def fill_segments(t, seg_dev, nseg: int, total: int, sigma: float = 1.0) -> None:
    """Fill the first `total` elements of device tensor t from nseg segments described by
    seg_dev, a device int64 tensor [3 * nseg + 1]: keys (as int64 bits) [nseg], first
    element index [nseg], then the output offsets [nseg + 1] (starting at 0)."""
    import torch
    if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("contiguous float32/bfloat16 device tensor expected")
    if seg_dev.dtype != torch.int64 or seg_dev.numel() != 3 * nseg + 1 or t.numel() < total:
        raise ValueError("segment table mis-sized")
    st = torch.cuda.current_stream().cuda_stream
    base = seg_dev.data_ptr()
    rc = lib().pkvgen_fill_segments(C.c_void_p(t.data_ptr()), int(t.dtype == torch.bfloat16), int(nseg),
                                    C.c_void_p(base), C.c_void_p(base + 8 * nseg), C.c_void_p(base + 16 * nseg),
                                    int(total), float(sigma), C.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"pkvgen_fill_segments failed ({rc})")


def read_probe(buf, blocks: int, unroll: int, out) -> None:
    """Stream-read the whole of device tensor `buf` (out: int32 tensor of blocks*256)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    if out.numel() < blocks * 256 or nbytes % 16:
        raise ValueError("probe buffers mis-sized")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib().pkvgen_read_probe(C.c_void_p(buf.data_ptr()), nbytes // 16, blocks, unroll,
                                 C.c_void_p(out.data_ptr()), C.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"pkvgen_read_probe failed ({rc})")


def read_probe_stream(buf, blocks: int, out) -> None:
    """Stream-read device tensor `buf` with one contiguous share per workgroup and
    non-temporal loads (out: int32 tensor of blocks*512)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    if out.numel() < blocks * 512 or nbytes % 16:
        raise ValueError("probe buffers mis-sized")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib().pkvgen_read_probe_stream(C.c_void_p(buf.data_ptr()), nbytes // 16, blocks,
                                        C.c_void_p(out.data_ptr()), C.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"pkvgen_read_probe_stream failed ({rc})")


if __name__ == "__main__":
    print(build(verbose=True))
