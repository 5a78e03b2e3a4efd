"""Host block pool model in plain Python integers (test infrastructure only).

State: a double-ended free queue, one reference count per physical block,
and per sequence an append-only list of block ids plus its token count.

Sources
  * "PagedAttention: fragmentation, blocks, block tables":
      - 1. The block pool: construction (all ids in ascending order in the
        free queue), get_new_blocks (pop from the head, ref 0 -> 1, an
        error when more blocks are asked for than are free) and
        free_blocks (ref -= 1; a block reaching zero goes back to the
        *front* of the queue; the list is ordered by eviction priority,
        first evicted first, and a request frees its blocks in reverse so
        the tail of the sequence is reused first).
      - 2. The block table: position p lives in block table[p // B] at
        offset p % B.
      - 3. The slot mapping: slot = table[p // B] * B + p % B.
      - the copy-on-write section: a shared, partially filled tail is
        redirected in place to a private block and a (src, dst) copy is
        queued.
      - the CPU reference allocator: create / append / fork / release and
        the invariants its check() enforces.
  * "Memory management", Code: append with copy-on-write -- blocks needed =
    ceil((len + n) / B) - held; copy iff the tail is partial and its
    reference count exceeds one; the capacity test covers both before any
    state changes; otherwise nothing is modified.

Readings where the pages leave a step open
  * No null block: every block id is allocatable (the CPU reference
    allocator returns all three of its pages to the free list).
  * Freed blocks are put at the head of the free queue in the order they
    are released (tail block first), so the tail block is the next one
    handed out.
  * The copy block is taken from the queue before the appended blocks.
"""

from __future__ import annotations

from collections import deque


class PoolError(Exception):
    """Base class of pool errors."""


class InvalidArgument(PoolError):
    """Unknown or duplicate sequence, bad block id, bad size."""


class NoSpace(PoolError):
    """Not enough free blocks; the pool state is unchanged."""


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int, order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArgument("num_blocks and block_size must be positive")
        if order is None:
            order = range(num_blocks)
        order = [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("initial order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # -- sequences ---------------------------------------------------------
    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise InvalidArgument(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, src: int, dst: int) -> None:
        """dst shares every block of src; each shared block gains one ref."""
        if src not in self.tables:
            raise InvalidArgument(f"unknown sequence {src}")
        if dst in self.tables:
            raise InvalidArgument(f"sequence {dst} exists")
        self.tables[dst] = list(self.tables[src])
        self.lens[dst] = self.lens[src]
        for b in self.tables[dst]:
            self.ref[b] += 1

    def append(self, seq: int, n: int):
        """Append n >= 1 tokens to seq.

        Returns (slots, cow) where slots[i] is the flat slot of position
        len + i and cow is a (src, dst) pair or None.  Raises NoSpace with
        the state untouched when the blocks do not fit.
        """
        if seq not in self.tables:
            raise InvalidArgument(f"unknown sequence {seq}")
        if n <= 0:
            raise InvalidArgument("n must be positive")
        B = self.block_size
        table = self.tables[seq]
        cur = self.lens[seq]
        needed = -(-(cur + n) // B) - len(table)
        cow = (cur % B != 0) and self.ref[table[-1]] > 1
        if needed + (1 if cow else 0) > len(self.free):
            raise NoSpace(f"need {needed + int(cow)} blocks, {len(self.free)} free")
        pair = None
        if cow:
            src = table[-1]
            dst = self.free.popleft()
            self.ref[dst] = 1
            self.ref[src] -= 1
            table[-1] = dst
            pair = (src, dst)
        for _ in range(needed):
            b = self.free.popleft()
            self.ref[b] = 1
            table.append(b)
        slots = [table[p // B] * B + p % B for p in range(cur, cur + n)]
        self.lens[seq] = cur + n
        return slots, pair

    def free_seq(self, seq: int) -> None:
        """Release seq: walk its blocks tail first, ref -= 1, and put the
        blocks that reach zero at the head of the queue in that order."""
        if seq not in self.tables:
            raise InvalidArgument(f"unknown sequence {seq}")
        released = []
        for b in reversed(self.tables[seq]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                released.append(b)
        # released[0] (the sequence's tail block) becomes the new head
        self.free.extendleft(reversed(released))
        del self.tables[seq]
        del self.lens[seq]

    # -- queries -------------------------------------------------------------
    def block_table(self, seq: int) -> list[int]:
        if seq not in self.tables:
            raise InvalidArgument(f"unknown sequence {seq}")
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        if seq not in self.lens:
            raise InvalidArgument(f"unknown sequence {seq}")
        return self.lens[seq]

    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise InvalidArgument("block id out of range")
        return self.ref[block]

    def free_order(self) -> list[int]:
        return list(self.free)

    # -- invariants ----------------------------------------------------------
    def check(self) -> None:
        """Structural invariants of the CPU reference allocator section:
        free and allocated blocks are disjoint and cover every block once;
        every table entry exists and its count of owners is its refcount;
        every allocated block has an owner; no table repeats a block;
        every non-tail block is full and the tail holds 1..B tokens."""
        N, B = self.num_blocks, self.block_size
        free = list(self.free)
        if len(set(free)) != len(free):
            raise AssertionError("free queue holds a block twice")
        owners = [0] * N
        for seq, table in self.tables.items():
            if len(set(table)) != len(table):
                raise AssertionError(f"table of {seq} repeats a block")
            n = self.lens[seq]
            if len(table) != -(-n // B):
                raise AssertionError(f"table of {seq} has {len(table)} blocks for {n} tokens")
            for b in table:
                if not 0 <= b < N:
                    raise AssertionError(f"table of {seq} names block {b}")
                owners[b] += 1
        free_set = set(free)
        for b in range(N):
            if owners[b] != self.ref[b]:
                raise AssertionError(f"block {b}: {owners[b]} owners, ref {self.ref[b]}")
            if (b in free_set) != (self.ref[b] == 0):
                raise AssertionError(f"block {b}: free={b in free_set} ref={self.ref[b]}")
        if len(free) + sum(1 for r in self.ref if r > 0) != N:
            raise AssertionError("free and allocated blocks do not cover the pool")
