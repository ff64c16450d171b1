"""Plain reference model of the host block allocator with a radix prefix cache
(test infrastructure only; see the package docstring).

Sources (web pages; cited by title and section):
  [V3]    pyshine walkthrough of text-generation-inference v3 -- "The radix
          prefix cache": block 0 is reserved; a free list plus a trie; an
          allocation walks the trie with the request's token ids, takes a
          reference on the matched prefix before anything can evict it, then
          takes fresh blocks for the rest, evicting the least recently used
          unreferenced prefixes when the free list runs dry; freeing drops the
          reference and inserts the newly computed prefix into the trie,
          returning blocks that another request cached meanwhile to the free
          list; the trie is a compressed radix tree keyed by token ids at block
          granularity whose insert splits nodes where a new prompt diverges.
          "Inside the batching task": a forward pass over a fully cached prompt
          computes nothing, so at least one prompt token stays uncached.
  [TGI]   "Under the Hood: PagedAttention", "Prefix sharing" paragraph: sequences
          share physical blocks; a write into a shared block first copies it to a
          new block and updates the writer's table (copy-on-write).
  [SPEED] "The KV cache: ...": fixed-size blocks allocated on demand, mapped
          through a per-request block table, shared copy-on-write.

Readings where the pages are silent:
  * Only whole blocks are cached and matched; a match keeps at least one prompt
    token uncached, so it covers at most floor((n_prompt - 1) / bs) blocks.
  * Fresh blocks are taken lowest id first.
  * Recency: every operation advances a clock; an allocation touches the nodes
    of its matched path, an insert the nodes it walks or creates.  Eviction
    removes whole leaves whose subtree holds no reference, least recently used
    first (ties: the node created first), until enough blocks are free.
  * A block is shared by a count of holders (live allocations and the trie); it
    returns to the free list when the count reaches zero.
  * A reference taken at allocation stays with the deepest matched node: a node
    split keeps its identity for the lower part and gets a new parent.
  * fork(a, n) gives a new allocation the blocks of a's first n tokens
    (shared); prepare_write(a, pos) copies the block holding pos when it is
    shared, and returns (source, destination) for the caller's device copy.
"""
from __future__ import annotations

import heapq


class AllocError(RuntimeError):
    pass


class _Node:
    __slots__ = ("keys", "blocks", "children", "parent", "refs", "last", "nid")

    def __init__(self, keys, blocks, parent, nid, tick):
        self.keys = list(keys)        # one tuple of bs token ids per block on the edge
        self.blocks = list(blocks)    # physical block of each edge block
        self.children = {}            # first key of the child's edge -> child
        self.parent = parent
        self.refs = 0                 # allocations whose match ends at this node
        self.last = tick
        self.nid = nid


class RadixAllocator:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 2 or block_size < 1:
            raise ValueError("need block 0 plus at least one usable block")
        self.NB, self.bs = int(num_blocks), int(block_size)
        self.free_heap = list(range(1, self.NB))          # block 0 is never handed out
        heapq.heapify(self.free_heap)
        self.holders = [0] * self.NB                 # live allocations + trie, per block
        self.tick = 0
        self.next_nid = 1
        self.root = _Node([], [], None, 0, 0)
        self.allocs = {}                             # id -> dict(blocks, node, n_total)
        self.next_id = 1

    # -- trie helpers ------------------------------------------------------
    def _blocks_of(self, tokens, n_blocks):
        bs = self.bs
        return [tuple(int(t) for t in tokens[i * bs:(i + 1) * bs]) for i in range(n_blocks)]

    def _walk(self, keys):
        """Deepest match of the key list: (node, depth in its edge, matched count, path)."""
        node, matched, path = self.root, 0, [self.root]
        while matched < len(keys):
            child = node.children.get(keys[matched])
            if child is None:
                return node, len(node.keys), matched, path
            d = 0
            while d < len(child.keys) and matched < len(keys) and child.keys[d] == keys[matched]:
                d += 1
                matched += 1
            path.append(child)
            if d < len(child.keys):
                return child, d, matched, path
            node = child
        return node, len(node.keys), matched, path

    def _split(self, node, d):
        """Cut node's edge after d blocks: a new parent takes the first d, node keeps the rest."""
        if d == 0 or d == len(node.keys):
            return node
        top = _Node(node.keys[:d], node.blocks[:d], node.parent, self.next_nid, node.last)
        self.next_nid += 1
        parent = node.parent
        parent.children[node.keys[0]] = top
        node.keys, node.blocks = node.keys[d:], node.blocks[d:]
        node.parent = top
        top.children[node.keys[0]] = node
        return top

    def _release(self, b):
        self.holders[b] -= 1
        if self.holders[b] == 0:
            heapq.heappush(self.free_heap, b)

    def _subtree_refs(self, node):
        return node.refs + sum(self._subtree_refs(c) for c in node.children.values())

    def _evictable_leaves(self):
        out, stack = [], [self.root]
        while stack:
            n = stack.pop()
            for c in n.children.values():
                stack.append(c)
            if n is not self.root and not n.children and n.refs == 0:
                out.append(n)
        return out

    def _evict_until(self, need):
        while len(self.free_heap) < need:
            leaves = self._evictable_leaves()
            if not leaves:
                return False
            victim = min(leaves, key=lambda n: (n.last, n.nid))
            del victim.parent.children[victim.keys[0]]
            for b in victim.blocks:
                self._release(b)
        return True

    def _take(self, count):
        return [heapq.heappop(self.free_heap) for _ in range(count)]

    # -- operations --------------------------------------------------------
    def allocate(self, tokens, n_total: int):
        """Blocks for a request whose prompt is ``tokens`` and which will hold n_total tokens.
        Returns (alloc_id, block list, cached prefix length in tokens)."""
        n_prompt = len(tokens)
        if n_total < n_prompt or n_total < 1:
            raise ValueError("the allocation must hold its prompt and at least one token")
        self.tick += 1
        want = max(0, (n_prompt - 1) // self.bs)
        keys = self._blocks_of(tokens, want)
        node, d, matched, path = self._walk(keys)
        node = self._split(node, d) if d < len(node.keys) else node
        # the path now ends exactly at `node`, which covers `matched` blocks
        chain, n = [], node
        while n is not self.root:
            chain.append(n)
            n = n.parent
        chain.reverse()
        prefix_blocks = [b for c in chain for b in c.blocks]
        assert len(prefix_blocks) == matched
        if node is not self.root:
            node.refs += 1                                  # before anything can be evicted
        for c in chain:
            c.last = self.tick
        total_blocks = -(-n_total // self.bs)
        fresh = total_blocks - matched
        if not self._evict_until(fresh):
            if node is not self.root:
                node.refs -= 1
            raise AllocError("not enough free blocks")
        new = self._take(fresh)
        blocks = prefix_blocks + new
        for b in blocks:
            self.holders[b] += 1
        aid = self.next_id
        self.next_id += 1
        self.allocs[aid] = dict(blocks=blocks, node=node, n_total=n_total)
        return aid, list(blocks), matched * self.bs

    def free(self, aid: int, tokens):
        """End an allocation whose K/V now covers ``tokens``; cache its full blocks."""
        a = self.allocs.pop(aid)
        blocks, node = a["blocks"], a["node"]
        self.tick += 1
        n_full = min(len(tokens) // self.bs, len(blocks))
        keys = self._blocks_of(tokens, n_full)
        at, d, matched, path = self._walk(keys)
        for c in path[1:]:
            c.last = self.tick
        if matched < n_full:
            parent = self._split(at, d) if d < len(at.keys) else at
            leaf = _Node(keys[matched:], blocks[matched:n_full], parent, self.next_nid, self.tick)
            self.next_nid += 1
            parent.children[keys[matched]] = leaf
            for b in blocks[matched:n_full]:
                self.holders[b] += 1                        # the trie holds them now
        # blocks [0, matched) were already cached (ours, or another request's copies:
        # then ours go back); the rest beyond the cached prefix too
        if node is not self.root:
            node.refs -= 1
        for b in blocks:
            self._release(b)

    def fork(self, aid: int, n_tokens: int):
        """A new allocation sharing the blocks that hold a's first n_tokens tokens."""
        a = self.allocs[aid]
        k = -(-n_tokens // self.bs)
        if n_tokens < 1 or k > len(a["blocks"]):
            raise ValueError("fork beyond the allocation")
        blocks = list(a["blocks"][:k])
        for b in blocks:
            self.holders[b] += 1
        nid = self.next_id
        self.next_id += 1
        node = a["node"]
        if node is not self.root:
            node.refs += 1
        self.allocs[nid] = dict(blocks=blocks, node=node, n_total=k * self.bs)
        return nid, list(blocks)

    def extend(self, aid: int, n_total: int):
        """Grow an allocation to hold n_total tokens (fresh blocks at its end)."""
        a = self.allocs[aid]
        k = -(-n_total // self.bs)
        extra = k - len(a["blocks"])
        if extra > 0:
            self.tick += 1
            if not self._evict_until(extra):
                raise AllocError("not enough free blocks")
            new = self._take(extra)
            for b in new:
                self.holders[b] += 1
            a["blocks"] += new
        a["n_total"] = max(a["n_total"], n_total)
        return list(a["blocks"])

    def prepare_write(self, aid: int, pos: int):
        """Before writing token position pos: if its block is shared, give the allocation a
        private copy.  Returns (src, dst) for the device copy, or None."""
        a = self.allocs[aid]
        i = pos // self.bs
        b = a["blocks"][i]
        if self.holders[b] <= 1:
            return None
        self.tick += 1
        if not self._evict_until(1):
            raise AllocError("not enough free blocks")
        (nb,) = self._take(1)
        self.holders[nb] += 1
        a["blocks"][i] = nb
        self._release(b)
        return b, nb

    def table(self, aid: int):
        return list(self.allocs[aid]["blocks"])

    def slots(self, aid: int, start: int, count: int):
        a = self.allocs[aid]
        return [a["blocks"][p // self.bs] * self.bs + p % self.bs for p in range(start, start + count)]

    # -- inspection ----------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free_heap)

    def num_cached(self) -> int:
        out, stack = 0, [self.root]
        while stack:
            n = stack.pop()
            out += len(n.blocks)
            stack.extend(n.children.values())
        return out
