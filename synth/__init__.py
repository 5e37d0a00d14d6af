"""Seeded synthetic inputs for the selective scan (test/bench infrastructure).

The generator is counter-based (SplitMix64 finaliser over (seed, stream, index),
Box-Muller normals, log-uniform step sizes); its definition is written out in
``synth.c``. It contains none of the scan's arithmetic. The GPU path and the
fp64 oracle both read the buffers produced here.

Input recipe (the workloads of the selective-scan pages: x, B, C, D standard
normal; step size Delta log-uniform on [1e-3, 1e-1]; A[e, n] = -(n + 1)):

  x     (Bs, L, ED)  N(0, 1)                   stream 1
  delta (Bs, L, ED)  exp(U(ln 1e-3, ln 1e-1))  stream 2
  B     (Bs, L, N)   N(0, 1)                   stream 3
  C     (Bs, L, N)   N(0, 1)                   stream 4
  D     (ED,)        N(0, 1)                   stream 5
  A     (ED, N)      -(n + 1), exact
  dy    (Bs, L, ED)  N(0, 1)                   stream 6 (output gradient, backward pass)

Multi-head (SSD) inputs, ``make_ssd_inputs``: x (Bs, L, H, P) N(0, 1) stream 11;
dt (Bs, L, H) log-uniform on [1e-3, 1e-1] stream 12; A (H) = -U(1, 16)
stream 13 (one decay rate per head); B, C (Bs, L, G, N) N(0, 1) streams 14,
15; D (H) N(0, 1) stream 16.

For bf16 workloads x, delta, B and C are rounded to bfloat16 (round to nearest
even) and handed over as uint16 bit patterns; A and D stay float32.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "libssm_synth.so")
_lib = None

STREAM_X, STREAM_DELTA, STREAM_B, STREAM_C, STREAM_D, STREAM_DY = 1, 2, 3, 4, 5, 6
DELTA_LO, DELTA_HI = 1e-3, 1e-1

# The five workloads of the selective-scan study, named by what they are.
WORKLOADS = {
    "fwd_f32_Bs2_L64_ED64_N16": dict(Bs=2, L=64, ED=64, N=16, dtype="f32", bidir=False, h_last=False),
    "fwd_f32_Bs8_L1024_ED1536_N16": dict(Bs=8, L=1024, ED=1536, N=16, dtype="f32", bidir=False, h_last=True),
    "fwd_bf16_Bs4_L8192_ED5120_N16": dict(Bs=4, L=8192, ED=5120, N=16, dtype="bf16", bidir=False, h_last=False),
    "fwd_f32_Bs1_L131072_ED2048_N16": dict(Bs=1, L=131072, ED=2048, N=16, dtype="f32", bidir=False, h_last=False),
    "bidir_f32_Bs8_L4096_ED1536_N16": dict(Bs=8, L=4096, ED=1536, N=16, dtype="f32", bidir=True, h_last=False),
    # the long sequence, bidirectional (split into chunks joined by a second kernel)
    "bidir_f32_Bs1_L131072_ED2048_N16": dict(Bs=1, L=131072, ED=2048, N=16, dtype="f32", bidir=True,
                                             h_last=True),
    # backward pass (all gradients, dy ~ N(0, 1)) at the forward training shape
    "bwd_f32_Bs8_L1024_ED1536_N16": dict(Bs=8, L=1024, ED=1536, N=16, dtype="f32", bidir=False, h_last=False,
                                         bwd=True),
    "bwd_bf16_Bs4_L8192_ED5120_N16": dict(Bs=4, L=8192, ED=5120, N=16, dtype="bf16", bidir=False, h_last=False,
                                          bwd=True),
    # backward pass of the long sequence (its sweep split into chunks)
    "bwd_f32_Bs1_L131072_ED2048_N16": dict(Bs=1, L=131072, ED=2048, N=16, dtype="f32", bidir=False,
                                           h_last=False, bwd=True),
    # backward pass of the bidirectional scan at its forward shape
    "bwd_bidir_f32_Bs8_L4096_ED1536_N16": dict(Bs=8, L=4096, ED=1536, N=16, dtype="f32", bidir=True,
                                               h_last=False, bwd=True),
    # a training step: the forward pass (y, and the state entering every
    # 32-step round kept for the backward) followed by the backward pass
    "train_f32_Bs8_L1024_ED1536_N16": dict(Bs=8, L=1024, ED=1536, N=16, dtype="f32", bidir=False, h_last=False,
                                           bwd=True, train=True),
    "train_bf16_Bs4_L8192_ED5120_N16": dict(Bs=4, L=8192, ED=5120, N=16, dtype="bf16", bidir=False,
                                            h_last=False, bwd=True, train=True),
    "train_f32_Bs1_L131072_ED2048_N16": dict(Bs=1, L=131072, ED=2048, N=16, dtype="f32", bidir=False,
                                             h_last=False, bwd=True, train=True),
    # the bidirectional scan's training step (the forward direction's round
    # states kept by the bidirectional forward)
    "train_bidir_f32_Bs8_L4096_ED1536_N16": dict(Bs=8, L=4096, ED=1536, N=16, dtype="f32", bidir=True,
                                                 h_last=False, bwd=True, train=True),
}

# Multi-head (SSD) workloads: batch 32, seqlen 400, 8 heads is the shape the
# Bi-Mamba2 page prints for its chunked scan; headdim 64, state 128 and one
# group are the usual Mamba-2 layer settings. The second is a longer,
# wider layer.
SSD_WORKLOADS = {
    "ssd_f32_Bs32_L400_H8_P64_N128": dict(Bs=32, L=400, H=8, P=64, G=1, N=128, dtype="f32"),
    "ssd_bf16_Bs8_L4096_H32_P64_N128": dict(Bs=8, L=4096, H=32, P=64, G=1, N=128, dtype="bf16"),
    "ssd_bidir_bf16_Bs8_L4096_H32_P64_N128": dict(Bs=8, L=4096, H=32, P=64, G=1, N=128, dtype="bf16", bidir=True),
}


def build():
    """Compile the generator library (gcc, no GPU needed)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, sz, fp = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
        L.synth_normal_f32.argtypes = [u64, u64, fp, sz, ctypes.c_int]
        L.synth_loguniform_f32.argtypes = [u64, u64, ctypes.c_double, ctypes.c_double, fp, sz, ctypes.c_int]
        L.synth_uniform_f32.argtypes = [u64, u64, ctypes.c_double, ctypes.c_double, fp, sz, ctypes.c_int]
        L.synth_word.argtypes = [u64, u64, u64]
        L.synth_word.restype = u64
        L.synth_f32_to_bf16.argtypes = [fp, fp, sz]
        L.synth_bf16_to_f32.argtypes = [fp, fp, sz]
        _lib = L
    return _lib


def _threads(nthreads):
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    return int(nthreads)


def normal(seed, stream, shape, nthreads=None):
    out = np.empty(shape, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, out.ctypes.data, out.size, _threads(nthreads))
    return out


def loguniform(seed, stream, shape, lo, hi, nthreads=None):
    out = np.empty(shape, dtype=np.float32)
    lib().synth_loguniform_f32(seed, stream, lo, hi, out.ctypes.data, out.size, _threads(nthreads))
    return out


def uniform(seed, stream, shape, lo, hi, nthreads=None):
    out = np.empty(shape, dtype=np.float32)
    lib().synth_uniform_f32(seed, stream, lo, hi, out.ctypes.data, out.size, _threads(nthreads))
    return out


def word(seed, stream, i):
    return int(lib().synth_word(seed, stream, i))


def to_bf16(a):
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def from_bf16(u):
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    out = np.empty(u.shape, dtype=np.float32)
    lib().synth_bf16_to_f32(u.ctypes.data, out.ctypes.data, u.size)
    return out


def a_matrix(ED, N):
    """A[e, n] = -(n + 1): the real diagonal initialisation used by the workloads."""
    return np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (ED, N)))


def make_inputs(Bs, L, ED, N, dtype="f32", seed=0, nthreads=None):
    """Inputs for one workload as numpy arrays (bf16 tensors as uint16 bit patterns)."""
    x = normal(seed, STREAM_X, (Bs, L, ED), nthreads)
    delta = loguniform(seed, STREAM_DELTA, (Bs, L, ED), DELTA_LO, DELTA_HI, nthreads)
    B = normal(seed, STREAM_B, (Bs, L, N), nthreads)
    C = normal(seed, STREAM_C, (Bs, L, N), nthreads)
    D = normal(seed, STREAM_D, (ED,), nthreads)
    A = a_matrix(ED, N)
    if dtype == "bf16":
        x, delta, B, C = to_bf16(x), to_bf16(delta), to_bf16(B), to_bf16(C)
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D)


def workload_inputs(name, seed=0, nthreads=None):
    w = WORKLOADS[name]
    return make_inputs(w["Bs"], w["L"], w["ED"], w["N"], w["dtype"], seed, nthreads)


def make_output_grad(Bs, L, ED, dtype="f32", seed=0, nthreads=None):
    """Gradient dL/dy for the backward pass, N(0, 1), of the workload's dtype."""
    dy = normal(seed, STREAM_DY, (Bs, L, ED), nthreads)
    return to_bf16(dy) if dtype == "bf16" else dy


STREAM_SSD_X, STREAM_SSD_DT, STREAM_SSD_A, STREAM_SSD_B, STREAM_SSD_C, STREAM_SSD_D = 11, 12, 13, 14, 15, 16


def make_ssd_inputs(Bs, L, H, P, G, N, dtype="f32", seed=0, nthreads=None):
    """Multi-head scan inputs as numpy arrays (bf16 tensors as uint16 bit patterns)."""
    x = normal(seed, STREAM_SSD_X, (Bs, L, H, P), nthreads)
    dt = loguniform(seed, STREAM_SSD_DT, (Bs, L, H), DELTA_LO, DELTA_HI, nthreads)
    A = -uniform(seed, STREAM_SSD_A, (H,), 1.0, 16.0, nthreads)
    B = normal(seed, STREAM_SSD_B, (Bs, L, G, N), nthreads)
    C = normal(seed, STREAM_SSD_C, (Bs, L, G, N), nthreads)
    D = normal(seed, STREAM_SSD_D, (H,), nthreads)
    if dtype == "bf16":
        x, dt, B, C = to_bf16(x), to_bf16(dt), to_bf16(B), to_bf16(C)
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D)
