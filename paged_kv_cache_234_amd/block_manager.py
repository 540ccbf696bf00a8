"""Host-side paged-KV block manager: the policy half of a paged cache.

The kernels hold no policy (include/pa.h: the library allocates nothing and
owns no blocks); this module is the owner.  That is the split InferX's
"Design" section draws: the scheduler side holds all the policy and no GPU
code, the executor side all the GPU code and no policy, so the paged KV
manager and the prefix cache are testable without a GPU.  In the shape the
pages describe for their engines:

* a fixed pool of 16-token blocks with a free list and a reference count per
  block (infer-lab, technique table, PagedAttention row: block allocator,
  block tables, reference counts, copy-on-write; InferX, introduction: KV
  blocks with scoped lifetimes and a single owner);
* prefix reuse: a full block is published under a hash of its tokens chained
  with its predecessor's, so a later sequence whose prompt starts with the
  same tokens maps the same physical blocks instead of recomputing them
  (infer-lab, RadixAttention row; llm-infer, "What It Does": prefix caching;
  InferX, "Status": radix prefix cache);
* copy-on-write: a sequence that must write into a block it shares gets a
  private copy first;
* liveness under KV pressure: cached blocks nobody references are evicted
  least recently used first; when none is left, the newest running sequence
  is preempted (its blocks are released and it is recomputed later), so the
  oldest request always makes progress.  Idle cached blocks count as
  available, not in use: infer-lab's ADR-0008 records the engine stalling
  with its pool full of cached blocks it counted as referenced (InferX,
  "Status": recompute preemption; infer-lab, KV accounting after draining:
  no leaked blocks).

Everything here is host bookkeeping over integers.  Moving K/V bytes (the
copy of copy-on-write) is done by the caller with the block-copy callback it
passes in, so this module touches no device memory itself.
"""

from collections import OrderedDict

BLOCK_SIZE = 16


class OutOfBlocks(RuntimeError):
    """No free block and nothing evictable."""


def block_hash(parent, tokens):
    """Hash of a full block's tokens chained with its predecessor's hash."""
    return hash((parent, tuple(tokens)))


class BlockPool:
    """Free list, reference counts and the prefix cache of one pool."""

    def __init__(self, num_blocks):
        self.num_blocks = int(num_blocks)
        self.ref = [0] * self.num_blocks
        self.free = list(range(self.num_blocks - 1, -1, -1))   # pop() hands out low ids first
        self.cached = {}                  # hash -> block id (full, published blocks)
        self.hash_of = {}                 # block id -> hash
        self.lru = OrderedDict()          # cached blocks with ref == 0, oldest first
        self.evictions = 0

    # ---- allocation -------------------------------------------------------
    def num_available(self):
        return len(self.free) + len(self.lru)

    def allocate(self):
        """A block with reference count 1; evicts the least recently used
        unreferenced cached block when the free list is empty."""
        if self.free:
            b = self.free.pop()
        elif self.lru:
            b, _ = self.lru.popitem(last=False)
            del self.cached[self.hash_of.pop(b)]
            self.evictions += 1
        else:
            raise OutOfBlocks("all %d blocks are referenced" % self.num_blocks)
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def incref(self, b):
        if self.ref[b] == 0:
            self.lru.pop(b, None)         # a cached block comes back into use
        self.ref[b] += 1

    def decref(self, b):
        assert self.ref[b] > 0, "double free of block %d" % b
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.hash_of:
                self.lru[b] = True        # keep the contents for reuse
            else:
                self.free.append(b)

    # ---- prefix cache -------------------------------------------------------
    def lookup(self, h):
        return self.cached.get(h)

    def publish(self, b, h):
        """Make full block b findable under hash h (first writer wins)."""
        if h in self.cached or b in self.hash_of:
            return
        self.cached[h] = b
        self.hash_of[b] = h


class Sequence:
    """A request: its tokens, how many of them have K/V in the pool, and its
    block table."""

    def __init__(self, seq_id, prompt):
        self.seq_id = seq_id
        self.tokens = list(prompt)
        self.num_cached = 0               # tokens whose K/V sit in the pool
        self.blocks = []
        self.hashes = []                  # chained hashes of the full blocks published

    @property
    def context_len(self):
        return len(self.tokens)


class BlockManager:
    """Block tables for a set of running sequences over one BlockPool.

    copy_block(src, dst) is called for copy-on-write; it must copy all K/V
    bytes of physical block src into dst (every layer and head).
    """

    def __init__(self, num_blocks, copy_block=None, enable_prefix_cache=True):
        self.pool = BlockPool(num_blocks)
        self.copy_block = copy_block
        self.enable_prefix_cache = enable_prefix_cache
        self.stats = {"prefix_hit_blocks": 0, "cow_copies": 0, "preemptions": 0}

    # ---- admission ------------------------------------------------------------
    def admit(self, seq):
        """Map seq's prompt: reuse cached full blocks of a matching prefix,
        allocate the rest.  Returns the number of leading tokens whose K/V are
        already in the pool (they need no recomputation).  Raises OutOfBlocks
        (with nothing held) when the pool cannot take the sequence."""
        n_tok = len(seq.tokens)
        need = -(-n_tok // BLOCK_SIZE)
        hits, parent = [], None
        if self.enable_prefix_cache:
            # a hit must leave at least one token to compute (the query of the step)
            for i in range((n_tok - 1) // BLOCK_SIZE):
                h = block_hash(parent, seq.tokens[i * BLOCK_SIZE:(i + 1) * BLOCK_SIZE])
                b = self.pool.lookup(h)
                if b is None:
                    break
                hits.append((b, h))
                parent = h
        if need - len(hits) > self.pool.num_available() - sum(
                1 for b, _ in hits if self.pool.ref[b] == 0):
            raise OutOfBlocks("cannot admit sequence %r" % (seq.seq_id,))
        for b, h in hits:
            self.pool.incref(b)
            seq.blocks.append(b)
            seq.hashes.append(h)
        self.stats["prefix_hit_blocks"] += len(hits)
        for _ in range(need - len(hits)):
            seq.blocks.append(self.pool.allocate())
        seq.num_cached = len(hits) * BLOCK_SIZE
        return seq.num_cached

    # ---- one step ---------------------------------------------------------------
    def slots_for_new_tokens(self, seq):
        """Slots of the tokens seq.tokens[num_cached:] (which the caller is about
        to append), after allocating blocks and copying shared ones on write.
        Publishes the blocks those tokens complete.  Raises OutOfBlocks when a
        needed block cannot be found (the caller preempts and retries)."""
        first, last = seq.num_cached, len(seq.tokens)
        need = -(-last // BLOCK_SIZE)
        while len(seq.blocks) < need:
            seq.blocks.append(self.pool.allocate())
        # copy-on-write: the block receiving the first new token may be shared
        bi = first // BLOCK_SIZE
        if first < last and bi < len(seq.blocks) and self.pool.ref[seq.blocks[bi]] > 1:
            src = seq.blocks[bi]
            dst = self.pool.allocate()
            if self.copy_block is not None:
                self.copy_block(src, dst)
            self.pool.decref(src)
            seq.blocks[bi] = dst
            self.stats["cow_copies"] += 1
        slots = [seq.blocks[p // BLOCK_SIZE] * BLOCK_SIZE + p % BLOCK_SIZE
                 for p in range(first, last)]
        seq.num_cached = last
        if self.enable_prefix_cache:
            full = last // BLOCK_SIZE
            parent = seq.hashes[-1] if seq.hashes else None
            for i in range(len(seq.hashes), full):
                h = block_hash(parent, seq.tokens[i * BLOCK_SIZE:(i + 1) * BLOCK_SIZE])
                self.pool.publish(seq.blocks[i], h)
                seq.hashes.append(h)
                parent = h
        return slots

    def fork(self, parent, seq_id):
        """A new sequence sharing all of parent's blocks, the partly filled
        last one included (parallel sampling): the first of the two to append
        into that block copies it."""
        child = Sequence(seq_id, parent.tokens)
        child.num_cached = parent.num_cached
        child.blocks = list(parent.blocks)
        child.hashes = list(parent.hashes)
        for b in child.blocks:
            self.pool.incref(b)
        return child

    def release(self, seq):
        """Drop seq's references (finished or preempted)."""
        for b in seq.blocks:
            self.pool.decref(b)
        seq.blocks = []
        seq.hashes = []
        seq.num_cached = 0

    def preempt(self, seq):
        self.release(seq)
        self.stats["preemptions"] += 1

    # ---- checks -------------------------------------------------------------------
    def check(self, running):
        """Every block's reference count equals the number of table entries
        naming it; free, cached-idle and referenced blocks partition the pool."""
        count = [0] * self.pool.num_blocks
        for s in running:
            for b in s.blocks:
                count[b] += 1
        assert count == self.pool.ref, "reference counts disagree with the block tables"
        free = set(self.pool.free)
        idle = set(self.pool.lru)
        used = {b for b in range(self.pool.num_blocks) if self.pool.ref[b] > 0}
        assert len(free) == len(self.pool.free), "a block is on the free list twice"
        assert not (free & idle) and not (free & used) and not (idle & used)
        assert len(free) + len(idle) + len(used) == self.pool.num_blocks, "a block leaked"
        for b in idle:
            assert b in self.pool.hash_of
