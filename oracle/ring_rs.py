"""Ring reduce-scatter simulator -- TEST INFRASTRUCTURE ONLY.

"MiniMind-tron: Sequence Parallelism", section 3.2.3: T ranks sit on a ring
R0 -> R1 -> ... -> R(T-1) -> R0, every rank holds its partial P_t cut into T
sequence blocks, and block letter j is destined for rank j.  At each of the
T-1 steps every rank forwards its one "active" cell to the next rank, which
adds it into its own cell of the same column; a forwarded cell is finished
with.  After T-1 steps rank j holds the fully summed block j -- the definition
of a reduce-scatter -- and every rank has sent (T-1) blocks of N/T elements.

The simulator runs on any block values that support "+": symbolic contributor
sets (to reproduce the pages' step tables) or numpy arrays (to check the
identity all-reduce = reduce-scatter + all-gather numerically).
"""


def active_block(rank, step, T):
    """Column that `rank` forwards at `step` (0-based): the cell it last
    received into (its own initial cell one column to the left at step 0)."""
    return (rank - 1 - step) % T


def simulate(blocks, record=None):
    """blocks[r][c]: rank r's initial block for column c (T x T).

    Runs the T-1 ring steps in place of a copy.  `record`, if given, receives
    after each step a T x T table whose finished (forwarded) cells are None.
    Returns (final table, elements sent per rank in block units).
    """
    T = len(blocks)
    table = [list(row) for row in blocks]
    sent = [0] * T
    for step in range(T - 1):
        outgoing = []
        for r in range(T):
            c = active_block(r, step, T)
            outgoing.append((r, c, table[r][c]))
        for r, c, val in outgoing:
            dst = (r + 1) % T
            table[dst][c] = table[dst][c] + val
            table[r][c] = None
            sent[r] += 1
        if record is not None:
            record.append([list(row) for row in table])
    return table, sent


def symbolic_blocks(T):
    """Initial cells as contributor sets: column letter + originating rank."""
    letters = "abcdefghijklmnopqrstuvwxyz"
    return [[frozenset({f"{letters[c]}{r}"}) for c in range(T)] for r in range(T)]


class _Sym:
    """A set of contributors, added by union (order-free, like exact sums)."""

    def __init__(self, names):
        self.names = frozenset(names)

    def __add__(self, other):
        return _Sym(self.names | other.names)

    def render(self):
        def key(n):
            return (n[0], int(n[1:]))
        return "+".join(sorted(self.names, key=key))


def symbolic_tables(T):
    """The per-step tables rendered as strings ('-' for a finished cell)."""
    init = [[_Sym(s) for s in row] for row in symbolic_blocks(T)]
    rec = []
    simulate(init, rec)
    return [[[("-" if cell is None else cell.render()) for cell in row] for row in tab]
            for tab in rec]
