"""Helpers over a plan's blob sections, shared by host and GPU tests."""
def lists_by_item(lay):
    """Each work item's list, keyed by (tile, head); the chunks of a split
    dK/dV item are joined in list order."""
    f = {}
    for qt, h0, off, n in lay["fwd_items"]:
        f[(int(qt), int(h0))] = lay["fwd_list"][off:off + n].tolist()
    ch = {}
    for kt, kvh, off, n in lay["bwd_items"]:
        ch.setdefault((int(kt), int(kvh)), []).append((int(off), int(n)))
    b = {}
    for key, parts in ch.items():
        b[key] = [x for off, n in sorted(parts) for x in lay["bwd_list"][off:off + n].tolist()]
    return f, b



def bwd_as_shared(b, G):
    """dK/dV lists of (Q-tile, query head) stages (plans with
    stats["bwd_head_entries"]) in the form of lists shared by the G heads of
    a group, as dynamic plans build them: one entry per Q-tile that has a
    stage, partial unless all G heads have a full stage of it."""
    out = {}
    for key, ents in b.items():
        tiles, full = [], {}
        for e in ents:
            t = e & 0xFFFFFF
            if t not in full:
                tiles.append(t)
                full[t] = 0
            if not e >> 31:
                full[t] += 1
        out[key] = [t | (0 if full[t] == G else 0x80000000) for t in tiles]
    return out


def concat_lists(lay):
    """Numpy form of lists_by_item for large plans: per pass, the (tile, head)
    keys in sorted order, their list lengths, and all their entries joined in
    that order (the chunks of a split dK/dV item in list order)."""
    import numpy as np

    def one(items, lst):
        items = np.asarray(items, dtype=np.int64)
        order = np.lexsort((items[:, 2], items[:, 1], items[:, 0]))
        it = items[order]
        if len(it) == 0:
            return np.zeros((0, 2), np.int64), np.zeros(0, np.int64), np.zeros(0, np.uint32)
        ents = np.concatenate([lst[o:o + n] for _, _, o, n in it]) if it[:, 3].sum() else np.zeros(0, np.uint32)
        keys, first = np.unique(it[:, :2], axis=0, return_index=True)
        lens = np.add.reduceat(it[:, 3], first)
        return keys, lens, ents

    return one(lay["fwd_items"], lay["fwd_list"]), one(lay["bwd_items"], lay["bwd_list"])
