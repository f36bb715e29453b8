"""Per-chain compressed state and its refresh along the accepted path
(test infrastructure only: the library never imports this module).

[review] "How it works", steps 4 and 6, and "Secret weapon" (paper sections
4.1-4.2 as summarised there): in the verify preprocess the prefix's
compressed state is reused, but compression after the branch point is done
separately for every chain, because one compression over two chains would
mix histories that exclude each other; the chains' temporary compressed
tokens and intermediate buffers live in a scratch pad; once a path is
accepted only that chain's KV and C4 / C128 state reach the persistent cache
and the rest is dropped.

The pages name DeepSeek-V4's compression of every 4 / 128 tokens but give no
formula for it.  The stand-in used here is the plainest one with the same
shape: compressed entry j of a token sequence is the mean of the rows of
positions j*c .. j*c + c - 1, and the intermediate buffer is the sum of the
rows of the incomplete last block.  Because the pages fix no values, the
functions below are pinned by the mathematics of that definition (block
means of the whole sequence computed from scratch, the toy's accepted chain,
multi-round refresh) in tests/test_oracle_compress.py; against the pages'
own compression this is parity unpinned.

Arithmetic is fp64; the rows enter as given (bf16 or fp32 values are exact
in fp64).
"""

import numpy as np


def block_state(rows, c):
    """Compressed state of a whole token sequence, from its definition:
    (entries [L // c, E] block means, tail [E] sum of the rows of the
    incomplete last block)."""
    rows = np.asarray(rows, dtype=np.float64)
    L, E = rows.shape
    full = (L // c) * c
    entries = rows[:full].reshape(L // c, c, E).mean(axis=1) if full else np.zeros((0, E))
    tail = rows[full:].sum(axis=0) if L > full else np.zeros(E)
    return entries, tail


def chain_entries(tail, l, chain_rows, c):
    """The verify preprocess for one chain: the running buffer starts from
    the prefix's tail sum, each chain row (root side first) is added, and
    whenever the sequence length l + t + 1 reaches a multiple of c the block
    is closed: its mean is emitted and the buffer restarts from zero.
    Returns (entries [n, E], buffer after the last row)."""
    s = np.array(tail, dtype=np.float64)
    out = []
    for t, row in enumerate(chain_rows):
        s = s + np.asarray(row, dtype=np.float64)
        if (l + t + 1) % c == 0:
            out.append(s / c)
            s = np.zeros_like(s)
    E = s.shape[0]
    return (np.array(out) if out else np.zeros((0, E))), s


def compress_chains(rows, tail, prefix_len, n_chains, chain_len, chain_nodes, c, gamma):
    """Every chain's new compressed entries.

    rows [B, N_max, E] scratch rows; tail [B, E]; prefix_len [B];
    n_chains [B], chain_len [B, N_max], chain_nodes [B, N_max, gamma] as
    unfold_chains writes them.  Returns (entries [B, N_max, M, E] with
    M = (c - 1 + gamma) // c, zero where unwritten; n_entries [B, N_max]:
    entries written per chain, 0 past the last chain, -1 for a chain that
    cannot be read (negative prefix length, or a node index outside
    [0, N_max))).
    """
    rows = np.asarray(rows, dtype=np.float64)
    B, N, E = rows.shape
    M = (c - 1 + gamma) // c
    entries = np.zeros((B, N, M, E))
    n_entries = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        l = int(prefix_len[b])
        nc = min(max(int(n_chains[b]), 0), N)
        for q in range(nc):
            ln = min(max(int(chain_len[b, q]), 0), gamma)
            nodes = [int(x) for x in chain_nodes[b, q, :ln]]
            if l < 0 or any(x < 0 or x >= N for x in nodes):
                n_entries[b, q] = -1
                continue
            ent, _ = chain_entries(tail[b], l, [rows[b, x] for x in nodes], c)
            entries[b, q, :len(ent)] = ent
            n_entries[b, q] = len(ent)
    return entries, n_entries


def refresh_compressed(rows, prefix_len, accept_len, accept_nodes, n_chains, chain_len,
                       chain_nodes, entries, comp, tail, c, gamma):
    """Commit the accepted chain's compressed state (run before the prefix
    length is advanced).

    For request b with m = accept_len[b] accepted nodes: the chain is the
    lowest-numbered one whose node m - 1 is the last accepted node (its first
    m nodes are then the accepted path; every chain through that node gives
    the same blocks, which depend only on the accepted tokens, so the choice
    is a convention); the e = (l % c + m) // c blocks that
    the accepted tokens close are copied from its entries to comp[b, l // c
    ...]; the tail becomes the old tail plus the accepted rows when no block
    closes, else the sum of the accepted rows after the last closed block.
    Returns (comp, tail, status [B]): 0 done (m == 0 changes nothing); 1 the
    entries would pass comp's capacity (nothing written); 2 malformed input
    (m outside [0, gamma], negative prefix length, an accepted node outside
    [0, N_max), or no chain holding the path; nothing written).
    """
    rows = np.asarray(rows, dtype=np.float64)
    comp = np.array(comp, dtype=np.float64)
    tail = np.array(tail, dtype=np.float64)
    B, N, E = rows.shape
    cap = comp.shape[1]
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        m, l = int(accept_len[b]), int(prefix_len[b])
        if m < 0 or m > gamma or l < 0:
            status[b] = 2
            continue
        if m == 0:
            continue
        path = [int(x) for x in accept_nodes[b, :m]]
        if any(x < 0 or x >= N for x in path):
            status[b] = 2
            continue
        nc = min(max(int(n_chains[b]), 0), N)
        q = next((q for q in range(nc)
                  if int(chain_len[b, q]) >= m and int(chain_nodes[b, q, m - 1]) == path[-1]), None)
        if q is None:
            status[b] = 2
            continue
        e = (l % c + m) // c
        if l // c + e > cap:
            status[b] = 1
            continue
        comp[b, l // c: l // c + e] = entries[b, q, :e]
        if e == 0:
            s = tail[b].copy()
            first = 0
        else:
            s = np.zeros(E)
            first = m - (l + m) % c   # the first accepted row after the last closed block
        for t in range(first, m):
            s = s + rows[b, path[t]]
        tail[b] = s
    return comp, tail, status
