"""Split a batch's contexts into shards of whole blocks (context parallelism), for tests."""
import numpy as np


def split_context(b, nshards: int, mode: str = "contiguous"):
    """Per shard: (block_tables_compact [B][W], block_tables_phys [B][W], lens [B]).

    Each logical block of each sequence goes to one shard, contiguous ranges or round
    robin; within a shard the blocks keep their logical order, so only a sequence's last
    (partly filled) block can be partial and it is last in its shard's table."""
    BS = b.BS
    out = []
    for s in range(nshards):
        rows_c, rows_p, lens = [], [], []
        for i in range(b.B):
            L = int(b.context_lens[i])
            nb = -(-L // BS)
            if mode == "contiguous":
                per = -(-nb // nshards)
                js = list(range(s * per, min(nb, (s + 1) * per)))
            else:
                js = list(range(s, nb, nshards))
            rows_c.append([int(b.block_tables_compact[i, j]) for j in js])
            rows_p.append([int(b.block_tables[i, j]) for j in js])
            lens.append(sum(min(BS, L - j * BS) for j in js))
        W = max(1, max(len(r) for r in rows_c))
        tc = np.full((b.B, W), -1, np.int32)
        tp = np.full((b.B, W), -1, np.int32)
        for i in range(b.B):
            tc[i, :len(rows_c[i])] = rows_c[i]
            tp[i, :len(rows_p[i])] = rows_p[i]
        out.append((tc, tp, np.array(lens, np.int32)))
    return out
