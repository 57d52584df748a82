"""Plain-Python model of the host block manager (test infrastructure, CPU only).

Follows the mini-llm-engine post: §3.1 (physical blocks with a ref count, an
O(1) free list taken from the front and refilled at the back, a per-sequence
table of physical blocks, a new block when the last one is full, every block
released at the end), §3.4 (full blocks found again by content are shared,
ref_count > 1; a shared block is copied before it is written) and §3.5
(swap-out to host slots, swap-in to new device blocks); and the Pico-vLLM
write-up, §3 (released cached blocks are evicted least recently used, lazily:
they keep their content until an allocation needs them).

The same policy as the C++ manager, written for clarity: a cached block is
keyed by the whole token prefix it ends (a tuple), so no hashing is involved;
reuse stops at the first miss and always leaves one prompt token to compute;
keys are registered by commit; allocation takes the never-cached free list
first, then the least recently released cached block.
"""

from collections import OrderedDict, deque

BLOCK = 16


class CapacityError(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks, num_host_blocks=0):
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks          # prefix tuple of a registered block
        self.free = deque(range(num_blocks))    # never-cached free blocks
        self.lru = OrderedDict()                # released registered blocks, oldest first
        self.prefix = {}                        # prefix tuple -> block
        self.seqs = {}                          # id -> dict(table, tokens, committed, swapped, host)
        self.host_free = deque(range(num_host_blocks))

    # ---- helpers ----------------------------------------------------------
    def available(self):
        return len(self.free) + len(self.lru)

    def _allocate(self):
        if self.free:
            b = self.free.popleft()
        elif self.lru:
            b, _ = self.lru.popitem(last=False)
            if self.prefix.get(self.key[b]) == b:
                del self.prefix[self.key[b]]
            self.key[b] = None
        else:
            raise CapacityError()
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] > 0:
            return
        if self.key[b] is not None:
            self.lru[b] = True
        else:
            self.free.append(b)

    # ---- operations (same meaning as the pa_bm_* calls) -------------------
    def add_sequence(self, sid, tokens):
        tokens = list(tokens)
        assert sid not in self.seqs and len(tokens) > 0
        nblk = -(-len(tokens) // BLOCK)
        reuse = []
        for i in range((len(tokens) - 1) // BLOCK):
            b = self.prefix.get(tuple(tokens[:(i + 1) * BLOCK]))
            if b is None:
                break
            reuse.append(b)
        in_lru = sum(1 for b in reuse if b in self.lru)
        if nblk - len(reuse) > self.available() - in_lru:
            raise CapacityError()
        for b in reuse:
            self.lru.pop(b, None)
            self.ref[b] += 1
        table = reuse + [self._allocate() for _ in range(nblk - len(reuse))]
        self.seqs[sid] = dict(table=table, tokens=tokens, committed=len(reuse), swapped=False, host=[])
        return len(reuse) * BLOCK

    def commit(self, sid, n_computed):
        s = self.seqs[sid]
        for i in range(s["committed"], n_computed // BLOCK):
            k = tuple(s["tokens"][:(i + 1) * BLOCK])
            b = s["table"][i]
            if self.key[b] is None and k not in self.prefix:
                self.key[b] = k
                self.prefix[k] = b
        s["committed"] = max(s["committed"], n_computed // BLOCK)

    def append_token(self, sid, token):
        s = self.seqs[sid]
        p = len(s["tokens"])
        cow = None
        if p % BLOCK == 0:
            s["table"].append(self._allocate())
        else:
            last = s["table"][-1]
            if self.ref[last] > 1:
                b = self._allocate()
                self._release(last)
                s["table"][-1] = b
                cow = (last, b)
        s["tokens"].append(token)
        return s["table"][p // BLOCK] * BLOCK + p % BLOCK, cow

    def fork(self, parent, child):
        s = self.seqs[parent]
        assert child not in self.seqs and not s["swapped"]
        for b in s["table"]:
            self.ref[b] += 1
        self.seqs[child] = dict(table=list(s["table"]), tokens=list(s["tokens"]),
                                committed=s["committed"], swapped=False, host=[])

    def free_sequence(self, sid):
        s = self.seqs.pop(sid)
        if s["swapped"]:
            self.host_free.extend(s["host"])
        else:
            for b in s["table"]:
                self._release(b)

    def block_table(self, sid):
        return list(self.seqs[sid]["table"])

    def slots(self, sid, start, n):
        t = self.seqs[sid]["table"]
        return [t[(start + i) // BLOCK] * BLOCK + (start + i) % BLOCK for i in range(n)]

    def swap_out(self, sid):
        s = self.seqs[sid]
        if len(s["table"]) > len(self.host_free):
            raise CapacityError()
        host = [self.host_free.popleft() for _ in s["table"]]
        dev = list(s["table"])
        for b in dev:
            self._release(b)
        s.update(table=[], host=host, swapped=True)
        return dev, host

    def swap_in(self, sid):
        s = self.seqs[sid]
        if len(s["host"]) > self.available():
            raise CapacityError()
        dev = [self._allocate() for _ in s["host"]]
        host = s["host"]
        self.host_free.extend(host)
        s.update(table=dev, host=[], swapped=False, committed=0)
        return host, dev
