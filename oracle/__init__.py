"""fp64 CPU oracle for paged KV attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product.  It wraps ``pa_oracle.c`` (plain C, double precision, OpenMP over
(sequence, KV head)) through ctypes and takes numpy arrays:

* bf16 tensors are passed as ``numpy.uint16`` arrays of their bit patterns;
* index arrays are ``numpy.int32``;
* outputs are ``numpy.float64``.

Every function states the passage of the pages it follows in ``pa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

_P = ctypes.c_void_p
_I = ctypes.c_int32


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected C-contiguous numpy {np.dtype(dtype).name} array")
    return a


class Oracle:
    """One loaded copy of the oracle library (the tests also load planted mutants)."""

    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} missing: run `python oracle/build.py`")
        lib = ctypes.CDLL(path)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_slot_mapping.restype = ctypes.c_int
        lib.oracle_slot_mapping.argtypes = [_P, _P, _I, _P, _I, _I, _P]
        lib.oracle_store.restype = None
        lib.oracle_store.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _I,
                                         _I, _I, _I, ctypes.c_double, _P]
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def slot_mapping(self, cu_seqlens_q, seqlens_k, block_tables, block_size):
        """Slots of the new tokens (the last q_len positions of each sequence)."""
        cu = _need(cu_seqlens_q, np.int32, "cu_seqlens_q")
        sk = _need(seqlens_k, np.int32, "seqlens_k")
        bt = _need(block_tables, np.int32, "block_tables")
        num_seqs = cu.shape[0] - 1
        out = np.full(int(cu[-1]), -1, dtype=np.int32)
        rc = self.lib.oracle_slot_mapping(_ptr(cu), _ptr(sk), num_seqs, _ptr(bt),
                                          bt.shape[1], block_size, _ptr(out))
        if rc != 0:
            raise ValueError("block table does not cover a token position")
        return out

    def store(self, k, v, slot_mapping, k_cache, v_cache):
        """Write k/v rows [T, Hkv, d] into the pools [NB, bs, Hkv, d] in place."""
        _need(k, np.uint16, "k"), _need(v, np.uint16, "v")
        _need(k_cache, np.uint16, "k_cache"), _need(v_cache, np.uint16, "v_cache")
        sm = _need(slot_mapping, np.int32, "slot_mapping")
        T, Hkv, d = k.shape
        bs = k_cache.shape[1]
        assert v.shape == k.shape and k_cache.shape == v_cache.shape
        assert k_cache.shape[2:] == (Hkv, d) and sm.shape == (T,)
        self.lib.oracle_store(_ptr(k), _ptr(v), _ptr(sm), T, Hkv, d, bs,
                              _ptr(k_cache), _ptr(v_cache))

    def attention(self, q, cu_seqlens_q, *, k=None, v=None, cu_seqlens_k=None,
                  k_cache=None, v_cache=None, block_tables=None, seqlens_k=None,
                  num_kv_heads=None, scale):
        """Causal attention; keys from flat k/v (cu_seqlens_k) or from the pools."""
        _need(q, np.uint16, "q")
        cu = _need(cu_seqlens_q, np.int32, "cu_seqlens_q")
        Tq, Hq, d = q.shape
        num_seqs = cu.shape[0] - 1
        if k_cache is not None:
            _need(k_cache, np.uint16, "k_cache"), _need(v_cache, np.uint16, "v_cache")
            bt = _need(block_tables, np.int32, "block_tables")
            sk = _need(seqlens_k, np.int32, "seqlens_k")
            Hkv, bs = k_cache.shape[2], k_cache.shape[1]
            args = (None, None, _ptr(k_cache), _ptr(v_cache), _ptr(bt), bt.shape[1], bs,
                    _ptr(cu), None, _ptr(sk))
        else:
            _need(k, np.uint16, "k"), _need(v, np.uint16, "v")
            cuk = _need(cu_seqlens_k, np.int32, "cu_seqlens_k")
            Hkv = k.shape[1]
            args = (_ptr(k), _ptr(v), None, None, None, 0, 1, _ptr(cu), _ptr(cuk), None)
        if num_kv_heads is not None:
            assert num_kv_heads == Hkv
        out = np.zeros((Tq, Hq, d), dtype=np.float64)
        rc = self.lib.oracle_attention(_ptr(q), *args, num_seqs, Hq, Hkv, d, float(scale), _ptr(out))
        if rc != 0:
            raise ValueError("invalid attention problem (q_len > k_len or Hq % Hkv != 0)")
        return out

    def decode(self, q, k_cache, v_cache, block_tables, context_lens, scale):
        """One new query per sequence over context_lens[s] keys (the new one included)."""
        S = q.shape[0]
        cu = np.arange(S + 1, dtype=np.int32)
        return self.attention(q, cu, k_cache=k_cache, v_cache=v_cache,
                              block_tables=block_tables, seqlens_k=context_lens, scale=scale)


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
