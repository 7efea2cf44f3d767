"""Shard maps for the ring simulation (oracle side).

Follows the MTraining review, page 1, section 三.3 (balanced sparse ring
attention: striped vs. zigzag distribution) and the Ring Attention overview,
page 4, sections 2.1 (KV blocks rotate around the ring) and 3.1 (fine-grained
stripes dealt round-robin).

Readings where the pages leave the detail open:
  * stripe width = one 64-token tile (rank r owns global 64-blocks G = r mod P);
    the variant "striped1" deals single positions (rank r owns n = r mod P),
    the plainest reading of "fine-grained stripes dealt round-robin";
  * zigzag = 2P equal chunks, rank r owns chunks r and 2P-1-r;
  * at ring step s, rank r holds the KV shard of rank (r - s) mod P.
"""
import numpy as np

BLOCK = 64


def shard_positions(kind: str, n_global: int, P: int, rank: int) -> np.ndarray:
    """Global token positions held by ``rank``, listed in storage order."""
    pos = np.arange(n_global, dtype=np.int64)
    if kind == "contig":
        owner = pos // (n_global // P)
    elif kind == "striped":
        owner = (pos // BLOCK) % P
    elif kind == "striped1":
        owner = pos % P
    elif kind == "zigzag":
        chunk = pos // (n_global // (2 * P))
        owner = np.where(chunk < P, chunk, 2 * P - 1 - chunk)
    else:
        raise ValueError(kind)
    return pos[owner == rank]        # ascending global order is the storage order


def ring_source(rank: int, step: int, P: int) -> int:
    """KV shard visible to ``rank`` at ring step ``step`` (step 0 = own shard)."""
    return (rank - step) % P
