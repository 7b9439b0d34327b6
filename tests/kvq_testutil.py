"""Helpers shared by the GPU tests: allocation, a numpy decoder of the
documented pool layout (include/kvq.h), and the parity tolerance.

The decoder is written from the header's layout description only; it shares
no code with the HIP library.
"""
from __future__ import annotations

import numpy as np

import attention_quantized_kv_amd as kvq

# Output tolerance: elementwise |o - ref| <= ATOL + RTOL * |ref| (max-abs 2e-3,
# relative 1e-3); lse is a log-domain scalar whose fp32 rounding is ~1e-7
# relative, checked to LSE_ATOL + LSE_RTOL * |ref|.
ATOL, RTOL = 2e-3, 1e-3
LSE_ATOL, LSE_RTOL = 1e-4, 1e-5


def layout(n_kv, D, P, n_pages, codec=0) -> kvq.Layout:
    return kvq.Layout(n_kv, D, P, n_pages, codec)


def alloc_pool(L: kvq.Layout, device="cuda", fill=0):
    import torch
    nbytes = kvq.kvq_pool_bytes(L)
    pool = torch.full((nbytes,), fill, dtype=torch.uint8, device=device)
    return pool


def page_table_for(ctx: int, P: int, n_pages: int, perm_seed=None, device="cuda"):
    import torch
    n = (ctx + P - 1) // P
    assert n <= n_pages
    if perm_seed is None:
        pt = np.arange(n, dtype=np.int32)
    else:
        pt = np.random.default_rng(perm_seed).permutation(n_pages)[:n].astype(np.int32)
    return torch.from_numpy(pt).to(device), pt


def unit_bytes(D, P):
    return P * D * 26 // 16


def decode_unit(unit: np.ndarray, D: int, P: int):
    """One unit's bytes -> (k_codes int8 [P][D], k_scales u16 [P][nb],
    v_codes u8 [P][D], v_scales u16 [P][nb]) following include/kvq.h."""
    nb = D // 32
    o = 0
    kraw = unit[o:o + P * D].view(np.int8)
    o += P * D
    ks = unit[o:o + 2 * P * nb].view(np.uint16).reshape(P, nb)
    o += 2 * P * nb
    vraw = unit[o:o + P * D // 2]
    o += P * D // 2
    # V scales are block-major inside each 32-token chunk: [chunk][block][32]
    vs = unit[o:o + 2 * P * nb].view(np.uint16).reshape(P // 32, nb, 32).transpose(0, 2, 1).reshape(P, nb)
    # K: [tile][p][g][n][half][e] -> token 16t+n, dim 64p+32half+8g+e
    k6 = kraw.reshape(P // 16, D // 64, 4, 16, 2, 8)
    kc = k6.transpose(0, 3, 1, 4, 2, 5).reshape(P, D)
    # V: [chunk][u][g][n][w][byte] with nibble i of the dword = token 32c+8g+i
    v6 = vraw.reshape(P // 32, D // 64, 4, 16, 4, 4)
    nib = np.empty(v6.shape[:-1] + (8,), dtype=np.uint8)
    nib[..., 0::2] = v6 & 15
    nib[..., 1::2] = v6 >> 4
    # nib dims: c, u, g, n, w, i -> token (c, g, i), dim (u, w, n)
    vc = nib.transpose(0, 2, 5, 1, 4, 3).reshape(P, D)
    return kc, ks.copy(), vc, vs.copy()


def decode_pool(pool_np: np.ndarray, L: kvq.Layout, page_table: np.ndarray, ctx: int):
    """Logical [ctx][n_kv][...] arrays of the first ctx tokens."""
    D, P, n_kv = L.head_dim, L.page_size, L.n_kv_heads
    ub = unit_bytes(D, P)
    nb = D // 32
    kc = np.empty((ctx, n_kv, D), np.int8)
    ks = np.empty((ctx, n_kv, nb), np.uint16)
    vc = np.empty((ctx, n_kv, D), np.uint8)
    vs = np.empty((ctx, n_kv, nb), np.uint16)
    for lp in range((ctx + P - 1) // P):
        phys = int(page_table[lp])
        n = min(P, ctx - lp * P)
        for g in range(n_kv):
            u0 = (phys * n_kv + g) * ub
            a, b, c, d = decode_unit(pool_np[u0:u0 + ub], D, P)
            sl = slice(lp * P, lp * P + n)
            kc[sl, g], ks[sl, g], vc[sl, g], vs[sl, g] = a[:n], b[:n], c[:n], d[:n]
    return kc, ks, vc, vs


def assert_close(out, ref, lse=None, ref_lse=None, what=""):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at {idx}: "
                             f"got {out[idx]!r} want {ref[idx]!r} (max abs err {err.max():.3e})")
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        ref_lse = np.asarray(ref_lse, dtype=np.float64)
        e = np.abs(lse - ref_lse)
        b = LSE_ATOL + LSE_RTOL * np.abs(ref_lse)
        if not np.all(e <= b):
            i = np.unravel_index(np.argmax(e - b), e.shape)
            raise AssertionError(f"{what}: lse outside tolerance at {i}: got {lse[i]!r} want {ref_lse[i]!r}")
    return float(err.max())


def decode_pool_int2(pool_np: np.ndarray, L: kvq.Layout, page_table: np.ndarray, ctx: int):
    """INT2 pool -> per token and KV head: K codes, scales, zeros, V codes,
    scales, zeros ([ctx][n_kv][D] and [ctx][n_kv][D/128]), from the INT2 unit
    layout described in include/kvq.h."""
    D, P, n_kv = L.head_dim, L.page_size, L.n_kv_heads
    nb2 = D // 128
    ub = 9 * P * D // 16
    kc = np.empty((ctx, n_kv, D), np.uint8)
    vc = np.empty((ctx, n_kv, D), np.uint8)
    ks = np.empty((ctx, n_kv, nb2), np.uint16)
    kz = np.empty_like(ks)
    vs = np.empty_like(ks)
    vz = np.empty_like(ks)
    k_par, v_sc = P * D // 2, P * D // 2 + 4 * P * nb2
    v_ze = v_sc + 2 * P * nb2
    dims = np.arange(D)

    def code(u, word_off, word, e):
        """Code e of word `word` of a lane area starting at byte word_off: word
        2i+h lives in dword i, code e at bit 16 (e / 4) + 8 h + 2 (e % 4)."""
        off = word_off + (word // 2) * 4
        dw = (u[off].astype(np.uint32) | (u[off + 1].astype(np.uint32) << 8) |
              (u[off + 2].astype(np.uint32) << 16) | (u[off + 3].astype(np.uint32) << 24))
        return (dw >> (16 * (e // 4) + 8 * (word % 2) + 2 * (e % 4))) & 3

    for j in range(ctx):
        page, s = divmod(j, P)
        for h in range(n_kv):
            u = pool_np[(int(page_table[page]) * n_kv + h) * ub:][:ub]
            # K: tile s // 16, lane (g, n) with n = s % 16; word = 32-dim step, code e = dim % 8
            t, n = divmod(s, 16)
            step, grp, e = dims // 32, (dims % 32) // 8, dims % 8
            kc[j, h] = code(u, t * 16 * D // 4 + (grp * 16 + n) * (D // 16), step, e)
            # V: chunk s // 32, lane (g, n) with g = (s % 32) // 8, n = d % 16; word d // 16, code s % 8
            c, gi, ei = s // 32, (s % 32) // 8, s % 8
            vc[j, h] = code(u, P * D // 4 + c * 32 * D // 4 + (gi * 16 + dims % 16) * (D // 8), dims // 16, ei)
            kp = u[k_par + s * nb2 * 4:][:nb2 * 4].view(np.uint16).reshape(nb2, 2)
            ks[j, h], kz[j, h] = kp[:, 0], kp[:, 1]
            for b in range(nb2):
                i = (c * nb2 + b) * 32 + s % 32
                vs[j, h, b] = u[v_sc + 2 * i:v_sc + 2 * i + 2].view(np.uint16)[0]
                vz[j, h, b] = u[v_ze + 2 * i:v_ze + 2 * i + 2].view(np.uint16)[0]
    return kc, ks, kz, vc, vs, vz
