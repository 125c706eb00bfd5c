"""CPU pin of the host-side KV4 page decode (tests/kv4_layout.py): every (slot, dim)
maps to its own nibble, and each position agrees with the layout's definition read
directly (search over the nibble index k of the word)."""
import numpy as np

from tests.kv4_layout import layout_index


def test_layout_positions_match_definition():
    kb, ksh, vb, vsh = layout_index()
    assert len(np.unique(kb * 8 + ksh)) == 64 * 128 and kb.min() == 0 and kb.max() == 4095
    assert len(np.unique(vb * 8 + vsh)) == 64 * 128 and vb.min() == 4096 and vb.max() == 8191
    for t in range(64):
        blk, tt = t // 16, t % 16
        for d in range(128):
            qd, u = (d % 16) // 4, (d // 16) // 2
            ks = [k for k in range(8) if 16 * (2 * u + ((k >> 1) & 1)) + 4 * qd + 2 * (k & 1) + (k >> 2) == d]
            assert len(ks) == 1
            k = ks[0]
            assert kb[t, d] == blk * 1024 + (16 * qd + tt) * 16 + 4 * u + k // 2 and ksh[t, d] == 4 * (k % 2)
            qt, dd = tt // 4, d % 16
            ks = [k for k in range(8)
                  if 4 * qt + 2 * (k & 1) + (k >> 2) == tt and 16 * (2 * u + ((k >> 1) & 1)) + dd == d]
            assert len(ks) == 1
            k = ks[0]
            assert vb[t, d] == 4096 + blk * 1024 + (16 * qt + dd) * 16 + 4 * u + k // 2 and vsh[t, d] == 4 * (k % 2)
