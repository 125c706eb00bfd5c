"""The KV4 page layout's code positions, written from its documented definition
(include/qoq.h, csrc/qoq_kv4.hip): used by the GPU tests to decode pages on the host
and pinned on the CPU by tests/test_kv4_layout.py."""
import numpy as np

D = 128
P = 64


def layout_index():
    """Byte offset (within a (page, head) section) and bit shift of the K and V code
    of every (slot t, dim d), from the documented page layout: 16-token block at
    blk * 1024 (+ 4096 for V), lane slot 16 qd + t (K) or 16 qt + dd (V) at 16 bytes
    each, word u, nibble k."""
    t = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    blk, tt = t // 16, t % 16
    # K: dim d = 16 (2u + (k >> 1 & 1)) + 4 qd + 2 (k & 1) + (k >> 2)
    j, r = d // 16, d % 16
    qd, rr = r // 4, r % 4
    u, kpar = j // 2, j % 2
    k = 4 * (rr % 2) + (rr // 2) + 2 * kpar
    kb = blk * 1024 + (16 * qd + tt) * 16 + 4 * u + k // 2
    ksh = 4 * (k % 2)
    # V: token 4 qt + 2 (k & 1) + (k >> 2) of dim 16 (2u + (k >> 1 & 1)) + dd
    qt, ti = tt // 4, tt % 4
    dd = d % 16
    k = 4 * (ti % 2) + (ti // 2) + 2 * kpar
    vb = 4096 + blk * 1024 + (16 * qt + dd) * 16 + 4 * u + k // 2
    vsh = 4 * (k % 2)
    return kb, np.broadcast_to(ksh, kb.shape), vb, np.broadcast_to(vsh, vb.shape)
