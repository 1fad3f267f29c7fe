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

