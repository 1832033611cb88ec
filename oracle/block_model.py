"""Reference model of KV block management: what a block manager must report.

TEST INFRASTRUCTURE ONLY: the test suite is its only caller; the product path
never imports it.

What is modelled (the contract of a paged KV block manager):

- The KV cache is a pool of fixed-size physical blocks handed to sequences
  like virtual-memory pages ("vLLM Project Update" talk, PagedAttention recap:
  the cache is managed like operating-system virtual memory, which lets
  requests share space).  A sequence of L tokens holds ceil(L / block_size)
  blocks; appending a token at a block boundary takes a new block.
- Sharing: a forked sequence shares all of its parent's blocks; a block is
  shared while more than one sequence maps it, and a sequence that writes into
  a shared block first gets a private copy (one copy per such write).
- Prefix caching (same talk, prefix-caching update: a new request reuses the
  cached KV of a common prefix, e.g. a system prompt, and computes only the
  rest): a full block whose KV has been written is registered under the exact
  token prefix it completes, unless that prefix is registered already.  A new
  sequence maps the registered blocks of its prompt's leading full blocks, in
  order, up to the first prefix that is not registered.  Registered blocks
  that no sequence maps stay registered until a block is needed and no
  never-registered free block is left; then the least recently released one
  is taken and its prefix is forgotten.  A sequence releases its blocks last
  block first.
- Swap ("[core] Multi Step Scheduling" pull request: the v2 block manager with
  a host swap space): swap-out moves every block of a sequence to its own host
  block and releases the device blocks; swap-in takes fresh device blocks and
  releases the host blocks.

The model keys the prefix cache by the full token prefix itself (a tuple), the
plainest exact definition, and keeps its own block numbering; it predicts
what any conforming manager reports -- cached-token counts, copy counts, free
device and host blocks, lengths and which calls fail for lack of blocks --
not which physical ids it picks.

Parity: pinned by hand-worked scenarios in tests/test_block_manager.py
(counts derived on paper from the rules above), not by the pages, which give
no numbers for block management.
"""
from __future__ import annotations

from collections import OrderedDict

CAPACITY = -7
SEQUENCE = -8
SHAPE = -2


class ModelError(Exception):
    def __init__(self, status: int):
        super().__init__(status)
        self.status = status


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0,
                 prefix_caching: bool = False):
        self.bs = block_size
        self.caching = prefix_caching
        self.free_ids = list(range(num_blocks))      # never-registered free blocks
        self.host_free = num_host_blocks
        self.refs: dict[int, int] = {}
        self.prefix_of: dict[int, tuple] = {}         # registered block -> its prefix
        self.block_of: dict[tuple, int] = {}          # registered prefix -> block
        self.released: OrderedDict[int, None] = OrderedDict()  # registered, unused; oldest first
        self.seqs: dict[int, dict] = {}

    # ---------------------------------------------------------------- blocks
    @property
    def num_free_blocks(self) -> int:
        return len(self.free_ids) + len(self.released)

    def _take(self) -> int:
        if self.free_ids:
            b = self.free_ids.pop()
        else:
            b, _ = self.released.popitem(last=False)
            del self.block_of[self.prefix_of.pop(b)]
        self.refs[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refs[b] -= 1
        if self.refs[b] == 0:
            if b in self.prefix_of:
                self.released[b] = None
            else:
                self.free_ids.append(b)

    def _seq(self, sid: int, resident: bool | None = True) -> dict:
        s = self.seqs.get(sid)
        if s is None or (resident is not None and s["resident"] != resident):
            raise ModelError(SEQUENCE)
        return s

    def _prefix(self, s: dict, i: int) -> tuple:
        return tuple(s["tokens"][: (i + 1) * self.bs])

    # ---------------------------------------------------------------- operations
    def add_sequence(self, sid: int, tokens: list[int]) -> int:
        if sid in self.seqs:
            raise ModelError(SEQUENCE)
        n = len(tokens)
        s = {"tokens": list(tokens), "len": n, "blocks": [], "resident": True, "host": 0,
             "marked": 0}
        hits = []
        if self.caching:
            for i in range(n // self.bs):
                b = self.block_of.get(self._prefix(s, i))
                if b is None:
                    break
                hits.append(b)
        need = -(-n // self.bs) - len(hits)
        revived = sum(1 for b in hits if self.refs.get(b, 0) == 0)
        if need > self.num_free_blocks - revived:
            raise ModelError(CAPACITY)
        for b in hits:
            if self.refs.get(b, 0) == 0:
                del self.released[b]
                self.refs[b] = 0
            self.refs[b] += 1
            s["blocks"].append(b)
        s["marked"] = len(hits)
        for _ in range(need):
            s["blocks"].append(self._take())
        self.seqs[sid] = s
        return len(hits) * self.bs

    def append(self, sids: list[int], tokens: list[int]) -> int:
        """Returns the number of copies (copy-on-write)."""
        if len(set(sids)) != len(sids):
            raise ModelError(SEQUENCE)
        ss = [self._seq(sid) for sid in sids]
        # blocks the batch takes: a boundary, or a last block still shared
        need, given_up = 0, {}
        for s in ss:
            if s["len"] % self.bs == 0:
                need += 1
            else:
                last = s["blocks"][-1]
                if self.refs[last] - given_up.get(last, 0) > 1:
                    need += 1
                    given_up[last] = given_up.get(last, 0) + 1
        if need > self.num_free_blocks:
            raise ModelError(CAPACITY)
        copies = 0
        for s, tok in zip(ss, tokens):
            if s["len"] % self.bs == 0:
                s["blocks"].append(self._take())
            elif self.refs[s["blocks"][-1]] > 1:
                src = s["blocks"][-1]
                s["blocks"][-1] = self._take()
                self._release(src)
                copies += 1
            s["tokens"].append(tok)
            s["len"] += 1
        return copies

    def fork(self, parent: int, child: int) -> None:
        p = self._seq(parent)
        if child in self.seqs:
            raise ModelError(SEQUENCE)
        c = {k: (list(v) if isinstance(v, list) else v) for k, v in p.items()}
        for b in c["blocks"]:
            self.refs[b] += 1
        self.seqs[child] = c

    def _release_all(self, s: dict) -> None:
        for b in reversed(s["blocks"]):
            self._release(b)
        s["blocks"] = []
        s["marked"] = 0

    def free(self, sid: int) -> None:
        s = self._seq(sid, resident=None)
        if s["resident"]:
            self._release_all(s)
        else:
            self.host_free += s["host"]
        del self.seqs[sid]

    def mark_computed(self, sid: int) -> None:
        s = self._seq(sid)
        if not self.caching:
            return
        for i in range(s["marked"], s["len"] // self.bs):
            pre = self._prefix(s, i)
            b = s["blocks"][i]
            if pre not in self.block_of and b not in self.prefix_of:
                self.block_of[pre] = b
                self.prefix_of[b] = pre
        s["marked"] = max(s["marked"], s["len"] // self.bs)

    def swap_out(self, sid: int) -> int:
        s = self._seq(sid)
        n = len(s["blocks"])
        if n > self.host_free:
            raise ModelError(CAPACITY)
        self.host_free -= n
        s["host"] = n
        self._release_all(s)
        s["resident"] = False
        return n

    def swap_in(self, sid: int) -> int:
        s = self._seq(sid, resident=False)
        n = s["host"]
        if n > self.num_free_blocks:
            raise ModelError(CAPACITY)
        s["blocks"] = [self._take() for _ in range(n)]
        self.host_free += n
        s["host"] = 0
        s["resident"] = True
        return n

    def length(self, sid: int) -> int:
        return self._seq(sid, resident=None)["len"]
