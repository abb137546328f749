"""Thin ctypes binding of libhspeaks.so (C ABI: include/hs_peaks.h), the measurement kernels that
give the measured ceilings the attention kernels are compared with. Argument marshalling only."""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhspeaks.so")

HSP_MFMA_32X32X16, HSP_SMFMAC_32X32X32, HSP_MFMA_16X16X32, HSP_SMFMAC_16X16X64 = 0, 1, 2, 3
HSP_VALU_EXP2, HSP_VALU_FMA, HSP_VALU_MAX3, HSP_VALU_CVT, HSP_VALU_SOFTMAX = 0, 1, 2, 3, 4
HSP_VALU_DOT2 = 5

EXPORTS = ("hsp_matrix_loop", "hsp_matrix_chain", "hsp_valu_loop", "hsp_mix_wave", "hsp_mix_split", "hsp_mix_phase",
           "hsp_lds_read",
           "hsp_read")

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libhspeaks.so is not built ({LIB_PATH}); run "
                               "python -m sparse_kv_cache_magnitude_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.hsp_matrix_loop.argtypes = [I, I, I, I, P, P, P]
        L.hsp_matrix_chain.argtypes = [I, I, I, I, I, P, P, P]
        L.hsp_valu_loop.argtypes = [I, I, I, I, I, P, P, P]
        L.hsp_mix_wave.argtypes = [I, I, I, I, I, P, P, P]
        L.hsp_mix_split.argtypes = [I, I, I, I, P, P, P]
        L.hsp_mix_phase.argtypes = [I, I, I, I, I, P, P, P]
        L.hsp_lds_read.argtypes = [I, I, I, P, P, P]
        L.hsp_read.argtypes = [I, P, ctypes.c_size_t, I, P, P]
        for f in EXPORTS:
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def matrix_loop(kind, grid, waves, iters, out, clk=None):
    _check(lib().hsp_matrix_loop(kind, grid, waves, iters, _p(out), _p(clk), _s()), "matrix_loop")


def matrix_chain(kind, accumulators, grid, waves, iters, out, clk=None):
    _check(lib().hsp_matrix_chain(kind, accumulators, grid, waves, iters, _p(out), _p(clk), _s()),
           "matrix_chain")


def valu_loop(op, grid, waves, iters, out, clk=None, chains=8):
    _check(lib().hsp_valu_loop(op, chains, grid, waves, iters, _p(out), _p(clk), _s()),
           "valu_loop")


def mix_wave(op, nops, grid, waves, iters, out, clk=None):
    _check(lib().hsp_mix_wave(op, nops, grid, waves, iters, _p(out), _p(clk), _s()), "mix_wave")


def mix_split(op, mfma_iters, valu_iters, grid, out, clk=None):
    _check(lib().hsp_mix_split(op, mfma_iters, valu_iters, grid, _p(out), _p(clk), _s()),
           "mix_split")


def mix_phase(part, waves, iters, vrounds, grid, out, clk=None):
    _check(lib().hsp_mix_phase(part, waves, iters, vrounds, grid, _p(out), _p(clk), _s()),
           "mix_phase")


def lds_read(grid, waves, iters, out, clk=None):
    _check(lib().hsp_lds_read(grid, waves, iters, _p(out), _p(clk), _s()), "lds_read")


def read(mode, src, grid, out):
    nbytes = src.numel() * src.element_size()
    _check(lib().hsp_read(mode, _p(src), nbytes, grid, _p(out), _s()), "read")
