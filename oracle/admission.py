"""Reference page allocator and admission control for the shared K/V pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference",
section *current scope* (the samir-vllm README):

* every request reserves credit for its largest processed prefix: prompt
  tokens plus allowed new tokens minus one (the last predicted token is
  returned without being processed), rounded up to 16-token pages, in each
  of the model's layers; the allowed output budget is capped by the context
  limit;
* credit and physical pages are separate: pages are taken lazily, when a
  sequence grows into a new page;
* a request whose credit does not fit beside the active ones waits, in FIFO
  order; one larger than the whole pool is rejected with an explicit error;
* finishing (early or not) returns the request's pages and its credit;
* continuous batching admits waiting requests whenever credit allows; static
  batching admits the next group only when the current group is done;
* ``--stats`` reports pool size, peak active requests, largest decode batch,
  peak allocated pages, admission waits and final free pages.

Readings where the page is silent: a new page is the lowest-numbered free
page (so block tables are reproducible); a request "waited" when it was not
admitted by the first admission pass after it was submitted; the largest
decode batch is the largest active set at a decode step; a prompt must leave
room for at least one new token (``1 <= prompt < context``, ``max_new >= 1``).
"""

from __future__ import annotations

import heapq
from collections import OrderedDict, deque

ADMIT, WAIT, REJECT = "admit", "wait", "reject"


class Request:
    def __init__(self, rid, prompt, max_new, allowed_new, credit_pages):
        self.rid = rid
        self.prompt = prompt
        self.max_new = max_new
        self.allowed_new = allowed_new
        self.credit = credit_pages            # pages reserved over all layers
        self.length = 0                       # tokens with K/V in the pool
        self.pages = None                     # per layer: list of physical pages
        self.waited = False


class PagePool:
    def __init__(self, num_pages, num_layers=16, page_tokens=16, context=2048, static=False):
        if num_pages < 1 or num_layers < 1 or page_tokens < 1 or context < 2:
            raise ValueError("bad pool geometry")
        self.num_pages = num_pages
        self.layers = num_layers
        self.page_tokens = page_tokens
        self.context = context
        self.static = static
        self.free = list(range(num_pages))    # min-heap of free page ids
        heapq.heapify(self.free)
        self.reserved = 0                     # credit pages held by active requests
        self.waiting = deque()
        self.active = OrderedDict()
        self.known = {}
        self.stats = dict(pool_pages=num_pages, peak_active=0, max_batch=0,
                          peak_allocated=0, admission_waits=0, free_pages=num_pages)

    # -- sizing -----------------------------------------------------------
    def pages_for(self, tokens):
        return -(-tokens // self.page_tokens)

    def credit_for(self, prompt, max_new):
        allowed_new = min(max_new, self.context - prompt)
        return allowed_new, self.layers * self.pages_for(prompt + allowed_new - 1)

    # -- requests ---------------------------------------------------------
    def submit(self, rid, prompt, max_new):
        """Queue a request; returns ``"wait"`` (queued) or ``"reject"``."""
        if rid in self.known:
            raise ValueError("request id reused")
        if not (1 <= prompt < self.context) or max_new < 1:
            return REJECT
        allowed_new, credit = self.credit_for(prompt, max_new)
        if credit > self.num_pages:
            return REJECT
        r = Request(rid, prompt, max_new, allowed_new, credit)
        self.known[rid] = r
        self.waiting.append(r)
        return WAIT

    def admit(self):
        """One admission pass; returns the ids admitted, in order."""
        out = []
        if not (self.static and self.active):
            while self.waiting:
                r = self.waiting[0]
                if self.reserved + r.credit > self.num_pages:
                    break
                self.waiting.popleft()
                self.reserved += r.credit
                r.pages = [[] for _ in range(self.layers)]
                self.active[r.rid] = r
                out.append(r.rid)
        for r in self.waiting:
            if not r.waited:
                r.waited = True
                self.stats["admission_waits"] += 1
        self.stats["peak_active"] = max(self.stats["peak_active"], len(self.active))
        return out

    def grow(self, rid, length):
        """Hold pages for tokens ``0 .. length-1`` of ``rid`` in every layer."""
        r = self.active[rid]
        if length < r.length or length > r.prompt + r.allowed_new - 1:
            raise ValueError("length outside the request's reserved prefix")
        need = self.pages_for(length)
        for layer in range(self.layers):
            while len(r.pages[layer]) < need:
                r.pages[layer].append(heapq.heappop(self.free))
        r.length = length
        used = self.num_pages - len(self.free)
        self.stats["peak_allocated"] = max(self.stats["peak_allocated"], used)
        self.stats["free_pages"] = len(self.free)

    def step(self):
        """A decode step over the active set (for the batch-size counter)."""
        self.stats["max_batch"] = max(self.stats["max_batch"], len(self.active))

    def finish(self, rid):
        r = self.active.pop(rid)
        for layer_pages in r.pages:
            for p in layer_pages:
                heapq.heappush(self.free, p)
        self.reserved -= r.credit
        self.stats["free_pages"] = len(self.free)

    def block_table(self, rid, layer):
        return list(self.active[rid].pages[layer])
