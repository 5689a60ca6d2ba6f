"""Memory-utilisation accounting, paged vs contiguous (oracle, test-only).

The pages measure the method by slots reserved versus slots holding a token:

* Contiguous reservation keeps ``max_len`` slots per request whatever its
  length; everything past the request's length is internal waste
  ([P1 "内存浪费的两种形式"], [P2 §1.2]).
* Paged allocation reserves ⌈L / bs⌉ blocks, so the only internal waste is the
  unfilled tail of each sequence's last block ([P1 "为什么 Paged Attention
  如此高效"], [P2 §3.3]).
* Blocks shared by refcount are stored once ([P2 §3.4]), so unique slots can
  be far fewer than the logical slots the sharers see.
"""


def contiguous_slots(lengths, max_len):
    """(reserved, used) slots when every request reserves ``max_len`` slots."""
    for n in lengths:
        if n > max_len:
            raise ValueError("a request is longer than its reservation")
    return len(lengths) * max_len, sum(lengths)


def paged_slots(lengths, block_size):
    """(reserved, used) slots when each request holds ⌈L/bs⌉ private blocks."""
    reserved = sum(-(-n // block_size) * block_size for n in lengths)
    return reserved, sum(lengths)


def utilisation(reserved, used):
    return 1.0 if reserved == 0 else used / reserved


def stats_utilisation(stats):
    """Fraction of slots in live blocks holding a token, from block-manager stats."""
    reserved = stats["used_blocks"] * stats["block_size"]
    return utilisation(reserved, stats["filled_slots"])


def sharing_ratio(stats):
    """Logical blocks seen by all sequences ÷ physical blocks actually held."""
    if stats["used_blocks"] == 0:
        return 1.0
    return stats["logical_blocks"] / stats["used_blocks"]
