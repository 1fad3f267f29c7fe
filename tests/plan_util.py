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
