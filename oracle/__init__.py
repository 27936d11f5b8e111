"""CPU oracle for paged KV cache decode — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library; the C part
(oracle.c) is written from the pool-layout definition and the pages:

  [P1] "LLM inference basics and vLLM internals" (ttlab.hopto.org), §2 KV
       cache size formula and GQA, §4 PagedAttention blocks / block table /
       null block.
  [P2] "vLLM internals (2): why PagedAttention pages the KV cache"
       (youngju.dev), "Block table", "Sharing".
  [P4] "vToken" (gotosocial.chinng-lab-srv.dev), "KV cache basics".

Every attention quantity is fp64.  Pins (tests/test_oracle_*.py) tie it to
the pages' printed numbers, the OCP E4M3 definition, torch's fp8 cast, the
contiguous brute force in oracle/brute.py, and closed forms.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16, FP16, FP8 = 0, 1, 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        i32, i64, f32, p = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        L.orc_bytes_per_token.restype = i64
        L.orc_bytes_per_token.argtypes = [i64, i64, i64, i64]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_fp16_value.restype = ctypes.c_double
        L.orc_fp16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_table.restype = None
        L.orc_e4m3_table.argtypes = [p]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [f32]
        L.orc_e4m3_encode_array.restype = None
        L.orc_e4m3_encode_array.argtypes = [p, i64, p]
        L.orc_k_sub_offset.restype = i64
        L.orc_k_sub_offset.argtypes = [i32, i32, i32]
        L.orc_v_sub_offset.restype = i64
        L.orc_v_sub_offset.argtypes = [i32, i32, i32]
        L.orc_pool_offset.restype = i64
        L.orc_pool_offset.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, i32]
        L.orc_slot_of_position.restype = i64
        L.orc_slot_of_position.argtypes = [p, i32, i32]
        L.orc_decode_slots.restype = None
        L.orc_decode_slots.argtypes = [p, i32, p, i32, i32, p]
        L.orc_reshape_and_cache.restype = None
        L.orc_reshape_and_cache.argtypes = [p, p, i32, p, p, p, i32, i32, i32, i32, i64,
                                            i32, f32, f32]
        L.orc_paged_decode_tokens.restype = None
        L.orc_paged_decode_tokens.argtypes = [p, p, i32, p, p, i32, p, i32, p, i32, i32, i32,
                                              i32, i32, f32, f32, f32]
        L.orc_move_tokens.restype = None
        L.orc_move_tokens.argtypes = [p, p, i32, p, i32, i32, i32, i32, i32]
        L.orc_paged_prefill.restype = None
        L.orc_paged_prefill.argtypes = [p, p, i32, p, p, i32, p, i32, p, p, i32, i32, i32, i32,
                                        i32, f32, f32, f32]
        L.orc_paged_decode.restype = None
        L.orc_paged_decode.argtypes = [p, p, i32, p, p, i32, p, i32, p, i32, i32, i32, i32,
                                       i32, f32, f32, f32]
        L.orc_max_threads.restype = i32
        L.orc_max_threads.argtypes = []
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def elem_bytes(dtype):
    return 1 if dtype == FP8 else 2


def bytes_per_token(layers, kv_heads, head_dim, elem_b):
    """[P1] §2 size formula 2*L*H_kv*d*b."""
    return int(lib().orc_bytes_per_token(layers, kv_heads, head_dim, elem_b))


def bf16_value(bits):
    return lib().orc_bf16_value(int(bits))


def fp16_value(bits):
    return lib().orc_fp16_value(int(bits))


def e4m3_value(code):
    return lib().orc_e4m3_value(int(code))


def e4m3_table():
    out = np.zeros(256, np.float64)
    lib().orc_e4m3_table(_ptr(out))
    return out


def e4m3_encode(x):
    """Encode an array of fp32 values to E4M3 codes (RNE, saturating)."""
    x = _c(x, np.float32)
    out = np.zeros(x.shape, np.uint8)
    lib().orc_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def decode_values(bits, dtype):
    """Exact fp64 values of raw element bits (uint16 for bf16/fp16, uint8 fp8)."""
    bits = np.asarray(bits)
    if dtype == FP8:
        return e4m3_table()[bits.astype(np.int64)]
    f = np.vectorize(bf16_value if dtype == BF16 else fp16_value, otypes=[np.float64])
    return f(bits.astype(np.uint16)) if bits.size else np.zeros(bits.shape)


def k_sub_offset(r, k, eb):
    return int(lib().orc_k_sub_offset(r, k, eb))


def v_sub_offset(r, k, eb):
    return int(lib().orc_v_sub_offset(r, k, eb))


def pool_offset(pb, g, t, k, is_value, kv_heads, head_dim, block_size, dtype):
    return int(lib().orc_pool_offset(pb, g, t, k, int(is_value), kv_heads, head_dim,
                                     block_size, dtype))


def layer_pool_bytes(num_blocks, kv_heads, head_dim, block_size, dtype):
    return num_blocks * kv_heads * block_size * head_dim * elem_bytes(dtype)


def slot_of_position(table_row, pos, block_size):
    row = _c(table_row, np.int32)
    return int(lib().orc_slot_of_position(_ptr(row), pos, block_size))


def decode_slots(block_tables, context_lens, block_size):
    """Slot of each sequence's newest token (position c-1); -1 when none."""
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    out = np.zeros(cl.shape[0], np.int64)
    lib().orc_decode_slots(_ptr(bt), bt.shape[1], _ptr(cl), cl.shape[0], block_size,
                           _ptr(out))
    return out


def reshape_and_cache(key_bits, value_bits, src_dtype, k_pool, v_pool, slots,
                      block_size, num_blocks, kv_dtype, k_scale=1.0, v_scale=1.0):
    """Return copies of the pools with the new tokens written.

    key_bits/value_bits: [T][H_kv][d] uint16 raw bits; pools: uint8 bytes.
    """
    key = _c(key_bits, np.uint16)
    val = _c(value_bits, np.uint16)
    kp = np.array(k_pool, dtype=np.uint8, copy=True)
    vp = np.array(v_pool, dtype=np.uint8, copy=True)
    sl = _c(slots, np.int64)
    T, H, D = key.shape
    lib().orc_reshape_and_cache(_ptr(key), _ptr(val), src_dtype, _ptr(kp), _ptr(vp),
                                _ptr(sl), T, H, D, block_size, num_blocks, kv_dtype,
                                float(k_scale), float(v_scale))
    return kp, vp


def paged_decode(q_bits, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens,
                 num_kv_heads, block_size, scale, k_scale=1.0, v_scale=1.0):
    """fp64 paged decode attention; q_bits [S][H][d] uint16 -> [S][H][d] fp64."""
    q = _c(q_bits, np.uint16)
    kp = _c(k_pool, np.uint8)
    vp = _c(v_pool, np.uint8)
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    S, H, D = q.shape
    out = np.zeros((S, H, D), np.float64)
    lib().orc_paged_decode(_ptr(out), _ptr(q), q_dtype, _ptr(kp), _ptr(vp), kv_dtype,
                           _ptr(bt), bt.shape[1], _ptr(cl), S, H, num_kv_heads, D,
                           block_size, float(np.float32(scale)), float(k_scale),
                           float(v_scale))
    return out


def paged_prefill(q_bits, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens,
                  query_start, num_kv_heads, block_size, scale, k_scale=1.0, v_scale=1.0):
    """fp64 multi-token causal attention over the paged cache; q_bits
    [T][H][d] uint16 (rows of sequence s at query_start[s] ..
    query_start[s+1]-1) -> [T][H][d] fp64."""
    q = _c(q_bits, np.uint16)
    kp = _c(k_pool, np.uint8)
    vp = _c(v_pool, np.uint8)
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    qs = _c(query_start, np.int32)
    T, H, D = q.shape
    S = cl.shape[0]
    assert qs.shape[0] == S + 1 and qs[0] == 0 and qs[-1] == T
    out = np.zeros((T, H, D), np.float64)
    lib().orc_paged_prefill(_ptr(out), _ptr(q), q_dtype, _ptr(kp), _ptr(vp), kv_dtype,
                            _ptr(bt), bt.shape[1], _ptr(cl), _ptr(qs), S, H, num_kv_heads, D,
                            block_size, float(np.float32(scale)), float(k_scale),
                            float(v_scale))
    return out


def paged_decode_tokens(q_bits, q_dtype, k_pool, v_pool, kv_dtype, token_slots, context_lens,
                        num_kv_heads, block_size, scale, k_scale=1.0, v_scale=1.0):
    """fp64 decode attention reading logical token t of sequence s from
    physical slot token_slots[s][t]; q_bits [S][H][d] -> [S][H][d]."""
    q = _c(q_bits, np.uint16)
    kp = _c(k_pool, np.uint8)
    vp = _c(v_pool, np.uint8)
    ts = _c(token_slots, np.int32)
    cl = _c(context_lens, np.int32)
    S, H, D = q.shape
    out = np.zeros((S, H, D), np.float64)
    lib().orc_paged_decode_tokens(_ptr(out), _ptr(q), q_dtype, _ptr(kp), _ptr(vp), kv_dtype,
                                  _ptr(ts), ts.shape[1], _ptr(cl), S, H, num_kv_heads, D,
                                  block_size, float(np.float32(scale)), float(k_scale),
                                  float(v_scale))
    return out


def move_tokens(k_pools, v_pools, moves, kv_heads, head_dim, block_size, kv_dtype):
    """Copies of the pools (lists of uint8 arrays, one per layer) with each
    token slot moves[i][0] copied to moves[i][1] (K and V, every kv head)."""
    ks = [np.array(p, np.uint8, copy=True) for p in k_pools]
    vs = [np.array(p, np.uint8, copy=True) for p in v_pools]
    mv = _c(np.asarray(moves, np.int32).reshape(-1, 2), np.int32)
    kp = (ctypes.c_void_p * max(len(ks), 1))(*[a.ctypes.data for a in ks])
    vp = (ctypes.c_void_p * max(len(vs), 1))(*[a.ctypes.data for a in vs])
    lib().orc_move_tokens(kp, vp, len(ks), _ptr(mv), mv.shape[0], kv_heads, head_dim, block_size,
                          kv_dtype)
    return ks, vs


def max_threads():
    return int(lib().orc_max_threads())


def set_threads(n):
    lib().orc_set_threads(int(n))
