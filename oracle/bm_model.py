"""Reference model of the host block manager (TEST INFRASTRUCTURE).

A plain Python statement of the allocation rules the pages give, used to
check the product's C block manager bit for bit.  It shares no code with it.

Rules and where they come from:
  * "How PagedAttention Powers vLLM's KV Cache", section "PagedAttention:
    paging, borrowed from the operating system": the cache is cut into
    fixed-size blocks; when a sequence needs room the engine takes a free
    physical block from a shared pool and appends an entry to the sequence's
    block table; when the sequence finishes its blocks go back to the pool;
    the only waste is the last, partly filled block of each sequence.
  * same page, section "The bonus contiguous storage can't give you:
    sharing": sequences can point at the same physical block, which carries
    a reference count; a sequence that must write into a shared block copies
    it first (copy-on-write); parallel sampling reuses the prompt's blocks.
  * attention-lab "PagedAttention" page, widget "Share matching prefixes" and
    reference entry "Shared blocks and copy-on-write": appending beyond a
    full shared block only needs a new block.
  * same page, widget "Add pages as the request grows": a new page is taken
    only when the current one is full.

Choices the pages leave open (this build's specification, mirrored by the C
block manager):
  * Free pool order: start from the stack [N-1, ..., 1, 0] (top of stack is
    the last element, so the first pop yields block 0); if the seed is not 0,
    shuffle it with Fisher-Yates driven by SplitMix64(seed): for i from N-1
    down to 1, j = next() mod (i+1), swap a[i] and a[j].  Pop from the end.
  * Freed blocks are pushed on the end, walking the table from its last
    entry to its first.
  * Sequence ids are 0, 1, 2, ... in creation order and are never reused.
  * Copy-on-write: a block is shared while its refcount is above 1.  A
    sequence appending into a partly filled tail block whose refcount is
    above 1 takes a new block, emits the pair (old, new), decrements the old
    block's refcount and continues in the new block; the last holder writes
    in place.
  * An append is all or nothing: if the pool lacks the blocks it needs
    (new blocks plus a copy-on-write block) nothing changes and ENOMEM is
    returned.
  * Swap to host (vLLM post, "Where it bites": a full pool preempts sequences
    and swaps their blocks out to CPU memory; glossary entry, "Flexible
    Management": pages can be swapped out, spilling to CPU RAM).  A host
    pool of H blocks has the free stack [H-1, ..., 0], unshuffled.  Swapping
    a sequence out takes one host block per table entry in table order,
    pairing (device block, host block), then drops the sequence's device
    references from its last entry to its first, as freeing would; a block
    another sequence still holds stays resident, and the swapped sequence
    keeps its own copy.  Swapping in takes one device block per entry in
    table order, pairing (host block, device block), then returns the host
    blocks from the last entry to the first.  A swapped sequence cannot be
    appended to or forked until it is swapped in.  Both are all or nothing.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

MASK64 = (1 << 64) - 1

OK, EINVAL, ENOMEM = 0, 1, 2


def splitmix64_stream(seed: int):
    """SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): a Weyl sequence with
    increment 0x9E3779B97F4A7C15 passed through a 64-bit finaliser."""
    state = seed & MASK64
    while True:
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        yield z ^ (z >> 31)


def initial_free_stack(num_blocks: int, seed: int) -> List[int]:
    a = list(range(num_blocks - 1, -1, -1))
    if seed != 0:
        rng = splitmix64_stream(seed)
        for i in range(num_blocks - 1, 0, -1):
            j = next(rng) % (i + 1)
            a[i], a[j] = a[j], a[i]
    return a


@dataclass
class _Seq:
    table: List[int] = field(default_factory=list)
    n_tokens: int = 0
    alive: bool = True
    swapped: bool = False


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, seed: int = 0):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.B = block_size
        self.free = initial_free_stack(num_blocks, seed)
        self.refcount = [0] * num_blocks
        self.seqs: List[_Seq] = []
        self.cow_copies = 0
        self.enomem_events = 0
        self.num_host_blocks = 0
        self.host_free: List[int] = []
        self.swapped_out_blocks = 0
        self.swapped_in_blocks = 0

    # --- operations -------------------------------------------------------
    def add_seq(self) -> int:
        self.seqs.append(_Seq())
        return len(self.seqs) - 1

    def _live(self, s: int) -> bool:
        return 0 <= s < len(self.seqs) and self.seqs[s].alive

    def _resident(self, s: int) -> bool:
        return self._live(s) and not self.seqs[s].swapped

    def fork(self, parent: int) -> Tuple[int, int]:
        """Child shares every block of the parent (refcount + 1 each)."""
        if not self._resident(parent):
            return EINVAL, -1
        p = self.seqs[parent]
        child = _Seq(table=list(p.table), n_tokens=p.n_tokens)
        for b in child.table:
            self.refcount[b] += 1
        self.seqs.append(child)
        return OK, len(self.seqs) - 1

    def append(self, s: int, n: int):
        """Returns (status, slots, cow_pairs)."""
        if not self._resident(s) or n < 0:
            return EINVAL, [], []
        if n == 0:
            return OK, [], []
        seq, B = self.seqs[s], self.B
        p0, pend = seq.n_tokens, seq.n_tokens + n
        need_new = -(-pend // B) - len(seq.table)
        cow = p0 % B != 0 and self.refcount[seq.table[-1]] > 1
        if need_new + (1 if cow else 0) > len(self.free):
            self.enomem_events += 1
            return ENOMEM, [], []
        pairs = []
        if cow:
            src = seq.table[-1]
            dst = self.free.pop()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            seq.table[-1] = dst
            pairs.append((src, dst))
            self.cow_copies += 1
        slots = []
        for p in range(p0, pend):
            if p % B == 0:
                b = self.free.pop()
                self.refcount[b] = 1
                seq.table.append(b)
            slots.append(seq.table[p // B] * B + p % B)
        seq.n_tokens = pend
        return OK, slots, pairs

    def append_batch(self, seqs, ns):
        """Appends to several sequences as one all-or-nothing step: the
        appends run one after another in the order given; if any lacks
        blocks, nothing changes.  Returns (status, slots, cow_pairs)."""
        if len(set(seqs)) != len(seqs) or any(not self._resident(s) or n < 0
                                               for s, n in zip(seqs, ns)):
            return EINVAL, [], []
        snap = ([list(q.table) for q in self.seqs], [q.n_tokens for q in self.seqs],
                list(self.free), list(self.refcount), self.cow_copies)
        slots, pairs = [], []
        for s, n in zip(seqs, ns):
            st, sl, pr = self.append(s, n)
            if st != OK:
                for q, t, n_tok in zip(self.seqs, snap[0], snap[1]):
                    q.table, q.n_tokens = t, n_tok
                self.free, self.refcount, self.cow_copies = snap[2], snap[3], snap[4]
                return st, [], []
            slots += sl
            pairs += pr
        return OK, slots, pairs

    def prefix_groups(self, seqs, max_members: int):
        """Runs of consecutive batch entries that share leading full blocks:
        a run starting at sequence i may share its S full blocks; the next
        sequence joins (while the run has fewer than max_members) if its
        first c >= 1 entries among the first min(S, its full blocks) equal
        i's, and then S = c.  Returns (group_start, shared_blocks)."""
        B = self.B
        gs, sb = [], []
        i = 0
        while i < len(seqs):
            first = self.seqs[seqs[i]]
            shared = first.n_tokens // B
            j = i + 1
            while j < len(seqs) and j - i < max_members:
                q = self.seqs[seqs[j]]
                lim = min(shared, q.n_tokens // B)
                c = 0
                while c < lim and q.table[c] == first.table[c]:
                    c += 1
                if c == 0:
                    break
                shared = c
                j += 1
            gs.append(i)
            sb.append(shared if j - i > 1 else 0)
            i = j
        gs.append(len(seqs))
        return gs, sb

    def _drop_device_refs(self, seq: _Seq):
        for b in reversed(seq.table):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)

    def free_seq(self, s: int) -> int:
        if not self._live(s):
            return EINVAL
        seq = self.seqs[s]
        if seq.swapped:
            self.host_free.extend(reversed(seq.table))
        else:
            if any(self.refcount[b] <= 0 for b in seq.table):
                return EINVAL
            self._drop_device_refs(seq)
        seq.table = []
        seq.n_tokens = 0
        seq.alive = False
        seq.swapped = False
        return OK

    def set_host_blocks(self, n: int) -> int:
        if n < 0 or len(self.host_free) != self.num_host_blocks:
            return EINVAL
        self.num_host_blocks = n
        self.host_free = list(range(n - 1, -1, -1))
        return OK

    def swap_out(self, s: int):
        """Returns (status, [(device block, host block), ...])."""
        if not self._resident(s):
            return EINVAL, []
        seq = self.seqs[s]
        if len(seq.table) > len(self.host_free):
            return ENOMEM, []
        host = [self.host_free.pop() for _ in seq.table]
        pairs = list(zip(seq.table, host))
        self._drop_device_refs(seq)
        seq.table = host
        seq.swapped = True
        self.swapped_out_blocks += len(host)
        return OK, pairs

    def swap_in(self, s: int):
        """Returns (status, [(host block, device block), ...])."""
        if not self._live(s) or not self.seqs[s].swapped:
            return EINVAL, []
        seq = self.seqs[s]
        if len(seq.table) > len(self.free):
            return ENOMEM, []
        dev = []
        for _ in seq.table:
            d = self.free.pop()
            self.refcount[d] = 1
            dev.append(d)
        pairs = list(zip(seq.table, dev))
        self.host_free.extend(reversed(seq.table))
        seq.table = dev
        seq.swapped = False
        self.swapped_in_blocks += len(dev)
        return OK, pairs

    # --- queries ----------------------------------------------------------
    def block_table(self, s: int):
        if not self._live(s):
            return EINVAL, [], 0
        return OK, list(self.seqs[s].table), self.seqs[s].n_tokens

    def stats(self) -> dict:
        B = self.B
        used = sum(1 for r in self.refcount if r > 0)
        shared = sum(1 for r in self.refcount if r > 1)
        fill = [0] * self.num_blocks
        live = logical_tokens = logical_blocks = swapped = 0
        for seq in self.seqs:
            if not seq.alive:
                continue
            if seq.swapped:
                swapped += 1
                continue
            live += 1
            logical_tokens += seq.n_tokens
            logical_blocks += len(seq.table)
            for j, b in enumerate(seq.table):
                fill[b] = max(fill[b], min(B, seq.n_tokens - j * B))
        return {
            "num_blocks": self.num_blocks,
            "block_size": B,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": shared,
            "live_seqs": live,
            "logical_tokens": logical_tokens,
            "logical_blocks": logical_blocks,
            "stored_tokens": sum(fill),
            "allocated_slots": used * B,
            "cow_copies": self.cow_copies,
            "enomem_events": self.enomem_events,
            "swapped_seqs": swapped,
            "host_blocks": self.num_host_blocks,
            "host_free_blocks": len(self.host_free),
            "swapped_out_blocks": self.swapped_out_blocks,
            "swapped_in_blocks": self.swapped_in_blocks,
        }


def contiguous_reservation(lengths, reserve: int) -> dict:
    """Accounting of the baseline the pages contrast paging with: every
    request holds one contiguous region of ``reserve`` slots whatever its
    length ("Why contiguous storage wastes most of your memory" on the vLLM
    KV-cache page; widget "Reserved space can go unused" on the attention-lab
    page)."""
    used = sum(int(x) for x in lengths)
    reserved = reserve * len(lengths)
    return {"reserved": reserved, "used": used, "empty": reserved - used,
            "wasted_fraction": (reserved - used) / reserved if reserved else 0.0}


def paged_accounting(lengths, block_size: int) -> dict:
    """Slots a paged allocator holds for unshared requests: ceil(L/B) blocks
    each ("Block allocation" on the attention-lab page: only the last block of
    a sequence can have idle slots)."""
    blocks = sum(-(-int(x) // block_size) for x in lengths)
    stored = sum(int(x) for x in lengths)
    return {"blocks": blocks, "slots": blocks * block_size, "stored": stored,
            "empty": blocks * block_size - stored}
