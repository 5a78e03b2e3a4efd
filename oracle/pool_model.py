"""Host block pool model in plain Python integers (test infrastructure only).

State: a double-ended free queue, one reference count per physical block,
and per sequence an append-only list of block ids plus its token count.

Sources
  * "PagedAttention: fragmentation, blocks, block tables":
      - 1. The block pool: construction (all ids in ascending order in the
        free queue), get_new_blocks (pop from the head, ref 0 -> 1, an
        error when more blocks are asked for than are free) and
        free_blocks (ref -= 1; a block reaching zero goes back to the
        *front* of the queue; the blocks handed in are ordered so that the
        one to be reused soonest comes first, and a request hands in its
        blocks tail first, so its tail block is the next one reused).
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

Prefix caching and retention (same page unless noted)
  * A full block carries a hash of its tokens and of the previous block's
    hash, so the hash captures position ("The pantry of pigeonholes", the
    prefix-sharing section); a global map from hash to block finds a cached
    prefix.  Matching a prefix "touches" each hit block: its reference
    count rises and, if it was waiting in the free queue as an eviction
    candidate, it leaves the queue (1. The block pool; the copy-on-write
    section on BlockPool.touch).
  * free_blocks: a block whose references reach zero keeps its hash; a
    hashed block goes to the tail of the queue (reused last, so it stays
    matchable), an unhashed one to the head (reused first).  Popping a
    hashed block for reuse evicts its hash entry (get_new_blocks).
  * Transfer pins (the CPU reference allocator's two kinds of references):
    a block is reusable only when it has neither owners nor pins; a pinned
    partial tail is copied before a write, like a shared one.
  * A copy-on-write keeps both endpoints retained until the copy has run
    (_apply_cow: the source keeps its reference, the destination takes an
    extra one); the caller reports the copies done.

Readings where the pages leave a step open
  * No null block: every block id is allocatable (the CPU reference
    allocator returns all three of its pages to the free list).
  * Freed blocks are put at the head of the free queue in the order they
    are released (tail block first), so the tail block is the next one
    handed out.  Hashed blocks go to the tail in release order.
  * The copy block is taken from the queue before the appended blocks.
  * The block hash is 64-bit FNV-1a over the previous block's hash (8 bytes,
    little-endian; 0 for the first block) followed by the block's token ids
    (4 bytes each, little-endian, two's complement).  The pages name no hash
    function; any 64-bit hash of that input fits their description.
  * Only full blocks are hashed and matched (prefix hits land on block
    boundaries; no partial hits).  When a hash is already mapped, the new
    block stays unhashed and the map keeps the first block.
  * A request's pins cover the blocks its table names when it is pinned;
    blocks released by an unpin, or by the completion of pending copies, are
    freed in reverse order of the pinned list, and for each copy the source
    before the destination.
"""

from __future__ import annotations

from collections import deque

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK64 = (1 << 64) - 1


def block_hash(parent: int, tokens) -> int:
    """64-bit FNV-1a over the parent hash (8 bytes LE) and the token ids
    (4 bytes LE each)."""
    h = FNV_OFFSET
    data = (int(parent) & MASK64).to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


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
        self.ref = [0] * num_blocks       # owners: tables that name the block
        self.pins = [0] * num_blocks      # transfer pins
        self.hold = [0] * num_blocks      # pending copy-on-write copies
        self.hash_of = [None] * num_blocks
        self.cached: dict[int, int] = {}  # block hash -> block
        self.transfers: dict = {}         # transfer id -> pinned blocks
        self.pending: list = []           # (src, dst) copies not yet run
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # -- retention -----------------------------------------------------------
    def _retained(self, b: int) -> bool:
        return self.ref[b] + self.pins[b] + self.hold[b] > 0

    def _release(self, blocks) -> None:
        """blocks (in eviction-priority order) have just lost their last
        reference: unhashed ones go to the head of the queue, hashed ones to
        the tail, each group in the given order."""
        first = [b for b in blocks if self.hash_of[b] is None]
        last = [b for b in blocks if self.hash_of[b] is not None]
        self.free.extendleft(reversed(first))
        self.free.extend(last)

    def _pop(self) -> int:
        """Head of the free queue, its cached hash (if any) evicted."""
        b = self.free.popleft()
        if self.hash_of[b] is not None:
            del self.cached[self.hash_of[b]]
            self.hash_of[b] = None
        return b

    def _touch(self, b: int) -> None:
        if not self._retained(b):
            self.free.remove(b)
        self.ref[b] += 1

    # -- sequences ---------------------------------------------------------
    def add_seq(self, seq: int, tokens=None) -> int:
        """New empty sequence; with ``tokens``, its longest prefix of cached
        full blocks is shared (each hit block touched) and the number of
        tokens covered is returned."""
        if seq in self.tables:
            raise InvalidArgument(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0
        if tokens is None:
            return 0
        B = self.block_size
        h = 0
        for j in range(len(tokens) // B):
            h = block_hash(h, tokens[j * B:(j + 1) * B])
            b = self.cached.get(h)
            if b is None:
                break
            self._touch(b)
            self.tables[seq].append(b)
            self.lens[seq] += B
        return self.lens[seq]

    def cache_blocks(self, seq: int, tokens) -> None:
        """Hash the full blocks of seq covered by ``tokens`` (its first
        len(tokens) token ids) and enter the unhashed ones into the map."""
        if seq not in self.tables:
            raise InvalidArgument(f"unknown sequence {seq}")
        if len(tokens) > self.lens[seq]:
            raise InvalidArgument("more tokens than the sequence holds")
        B = self.block_size
        chain, h = [], 0
        for j in range(len(tokens) // B):
            h = block_hash(h, tokens[j * B:(j + 1) * B])
            b = self.tables[seq][j]
            if self.hash_of[b] is not None and self.hash_of[b] != h:
                raise InvalidArgument(f"block {b} already holds other content")
            chain.append((b, h))
        for b, h in chain:                        # all checked: nothing changed on error
            if self.hash_of[b] is None and h not in self.cached:
                self.cached[h] = b
                self.hash_of[b] = h

    # -- transfer pins and pending copies -----------------------------------------
    def pin(self, seq: int, transfer) -> list:
        """Pin every block seq's table names under a new transfer id."""
        if seq not in self.tables:
            raise InvalidArgument(f"unknown sequence {seq}")
        if transfer in self.transfers:
            raise InvalidArgument(f"transfer {transfer} exists")
        blocks = list(self.tables[seq])
        for b in blocks:
            self.pins[b] += 1
        self.transfers[transfer] = blocks
        return list(blocks)

    def unpin(self, transfer) -> None:
        if transfer not in self.transfers:
            raise InvalidArgument(f"unknown transfer {transfer}")
        released = []
        for b in reversed(self.transfers.pop(transfer)):
            self.pins[b] -= 1
            if not self._retained(b):
                released.append(b)
        self._release(released)

    def copies_done(self) -> None:
        """The pending copy-on-write copies have run: their endpoints lose
        the retention held for them."""
        released = []
        for src, dst in self.pending:
            for b in (src, dst):
                self.hold[b] -= 1
                if not self._retained(b):
                    released.append(b)
        self.pending = []
        self._release(released)

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
        cow = (cur % B != 0) and (self.ref[table[-1]] > 1 or self.pins[table[-1]] > 0)
        if needed + (1 if cow else 0) > len(self.free):
            raise NoSpace(f"need {needed + int(cow)} blocks, {len(self.free)} free")
        pair = None
        if cow:
            src = table[-1]
            dst = self._pop()
            self.ref[dst] = 1
            self.ref[src] -= 1
            self.hold[src] += 1
            self.hold[dst] += 1
            self.pending.append((src, dst))
            table[-1] = dst
            pair = (src, dst)
        for _ in range(needed):
            b = self._pop()
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
            if not self._retained(b):
                released.append(b)
        # unhashed: released[0] (the sequence's tail block) becomes the new head
        self._release(released)
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

    def num_cached(self) -> int:
        return len(self.cached)

    # -- invariants ----------------------------------------------------------
    def check(self) -> None:
        """Structural invariants of the CPU reference allocator section:
        free and allocated blocks are disjoint and cover every block once;
        every table entry exists and its count of owners is its refcount;
        every retained block has an owner, a pin or a pending copy, and the
        pin and copy counts match their records; no table repeats a block;
        every non-tail block is full and the tail holds 1..B tokens; the
        hash map and the blocks' hashes agree one to one."""
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
        pins = [0] * N
        for blocks in self.transfers.values():
            for b in blocks:
                pins[b] += 1
        hold = [0] * N
        for src, dst in self.pending:
            hold[src] += 1
            hold[dst] += 1
        free_set = set(free)
        for b in range(N):
            if owners[b] != self.ref[b]:
                raise AssertionError(f"block {b}: {owners[b]} owners, ref {self.ref[b]}")
            if pins[b] != self.pins[b] or hold[b] != self.hold[b]:
                raise AssertionError(f"block {b}: pin or copy counts do not match their records")
            if (b in free_set) == self._retained(b):
                raise AssertionError(f"block {b}: free={b in free_set} but retained={self._retained(b)}")
        if len(free) + sum(1 for b in range(N) if self._retained(b)) != N:
            raise AssertionError("free and allocated blocks do not cover the pool")
        for h, b in self.cached.items():
            if self.hash_of[b] != h:
                raise AssertionError(f"hash map entry of block {b} does not match its hash")
        if sum(1 for h in self.hash_of if h is not None) != len(self.cached):
            raise AssertionError("a block holds a hash the map does not know")
