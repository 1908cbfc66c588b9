"""Decode the bf16-io workspace of libkda_fwd back into natural-order arrays (test helper).

The layout is the one documented in include/kda_fwd.h's companion source (kda_internal.h,
WsBf16): per (value head, slot) chunk, fp16 fragments in the state kernel's lane order. This is
host-side test logic only; it does no KDA arithmetic.
"""
from __future__ import annotations

import numpy as np


def chunk_bytes(K, V):
    end = 32 * K * 3 + 32 * V + 512 + 4 * K
    return (end + 255) // 256 * 256


def decode_chunk(raw: np.ndarray, K: int, V: int):
    """raw: uint8 bytes of one chunk. Returns dict of float64 arrays w [16,K], qd [16,K],
    kr [16,K], u [16,V], Mqk [16,16], eg [K]."""
    off = 0
    h16 = lambda a, b: raw[a:b].view(np.float16).astype(np.float64)
    NS, NV = K // 32, V // 16
    lanes = np.arange(64)
    g, m = lanes // 16, lanes % 16
    out = {}
    for name in ("w", "qd"):
        frag = h16(off, off + 32 * K).reshape(NS, 64, 8)
        X = np.full((16, K), np.nan)
        for s in range(NS):
            for e in range(8):
                kd = 16 * (2 * s + e // 4) + 4 * g + e % 4
                X[m, kd] = frag[s, :, e]
        out[name] = X
        off += 32 * K
    frag = h16(off, off + 32 * K).reshape(NS, 64, 8)
    X = np.full((16, K), np.nan)
    for s in range(NS):
        for e in range(8):
            c, i = 2 * s + e // 4, e % 4
            X[4 * g + i, 16 * c + m] = frag[s, :, e]
    out["kr"] = X
    off += 32 * K
    frag = h16(off, off + 32 * V).reshape(NV, 64, 4)
    X = np.full((16, V), np.nan)
    for c in range(NV):
        for i in range(4):
            X[4 * g + i, 16 * c + m] = frag[c, :, i]
    out["u"] = X
    off += 32 * V
    frag = h16(off, off + 512).reshape(64, 4)
    X = np.full((16, 16), np.nan)
    for i in range(4):
        X[m, 4 * g + i] = frag[:, i]
    out["Mqk"] = X
    off += 512
    out["eg"] = raw[off:off + 4 * K].view(np.float32).astype(np.float64)
    return out


def chunk_bytes32(K, V):
    end = 64 * K * 3 + 64 * V + 512 + 1024 + 4 * K
    return (end + 255) // 256 * 256


def decode_chunk32(raw: np.ndarray, K: int, V: int):
    """Decode one 32-token chunk record (two 16-row blocks a, b). Returns float64 arrays
    w [32,K], qd [32,K], kr [32,K], u [32,V], Mqk [32,32] (upper-right block zero: never
    stored), eg [K]."""
    h16 = lambda a, b: raw[a:b].view(np.float16).astype(np.float64)
    NS, NK, NV = K // 32, K // 16, V // 16
    lanes = np.arange(64)
    g, m = lanes // 16, lanes % 16
    out, off = {}, 0
    for name in ("w", "qd"):
        frag = h16(off, off + 64 * K).reshape(2, NS, 64, 8)
        X = np.full((32, K), np.nan)
        for b in range(2):
            for s in range(NS):
                for e in range(8):
                    X[16 * b + m, 16 * (2 * s + e // 4) + 4 * g + e % 4] = frag[b, s, :, e]
        out[name] = X
        off += 64 * K
    frag = h16(off, off + 64 * K).reshape(NK, 64, 8)
    X = np.full((32, K), np.nan)
    for t in range(NK):
        for e in range(8):
            tokv = 4 * g + e if e < 4 else 16 + 4 * g + e - 4
            X[tokv, 16 * t + m] = frag[t, :, e]
    out["kr"] = X
    off += 64 * K
    frag = -h16(off, off + 64 * V).reshape(NV, 64, 8)
    X = np.full((32, V), np.nan)
    for b in range(2):
        for c in range(NV):
            for i in range(4):
                X[16 * b + 4 * g + i, 16 * c + m] = frag[c, :, 4 * b + i]
    out["u"] = X                       # stored negated
    off += 64 * V
    M = np.zeros((32, 32))
    fa = h16(off, off + 512).reshape(64, 4)
    for i in range(4):
        M[m, 4 * g + i] = fa[:, i]
    off += 512
    fb = h16(off, off + 1024).reshape(64, 8)
    for e in range(8):
        colv = 4 * g + e if e < 4 else 16 + 4 * g + e - 4
        M[16 + m, colv] = fb[:, e]
    out["Mqk"] = M
    off += 1024
    out["eg"] = raw[off:off + 4 * K].view(np.float32).astype(np.float64)
    return out


def pair_bytes(K, V):
    end = 64 * K * 3 + 64 * V + 512 + 1024 + 4 * K + 2048
    return (end + 255) // 256 * 256


def decode_pair(raw: np.ndarray, K: int, V: int):
    """Decode the two records of one 64-token pair (chunk-64 workspace): returns
    (first, second), each as decode_chunk32 returns it; second["P"] [32,32] is the product the
    second record carries in its PT field (rows: its tokens; columns: the first chunk's)."""
    rb = pair_bytes(K, V)
    first = decode_chunk32(raw[:rb], K, V)
    second = decode_chunk32(raw[rb:2 * rb], K, V)
    end32 = 64 * K * 3 + 64 * V + 512 + 1024 + 4 * K
    pt = raw[rb + end32:rb + end32 + 2048].view(np.float16).astype(np.float64).reshape(2, 64, 8)
    lanes = np.arange(64)
    g, n = lanes // 16, lanes % 16
    P = np.full((32, 32), np.nan)
    for x in range(2):
        for e in range(8):
            colv = 4 * g + e if e < 4 else 16 + 4 * g + e - 4
            P[16 * x + n, colv] = pt[x, :, e]
    second["P"] = P
    return first, second
