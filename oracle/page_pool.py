"""Page allocator of the paged cache: reference counts, prefix reuse at job
admission, prompt caching of released pages, and defragmentation (test
oracle, plain Python).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (ExLlamaV2 "Dynamic Generator" page):

* "Continuous Batching": a job queue starts as many jobs as fit in the cache;
  when a job finishes its pages are freed for the next job; the holes they
  leave are filled by the next jobs (block indices need not be contiguous).
  The cache can be defragmented; the generator does it only for unreferenced
  pages, and only when the queue is empty.
* "Deduplication": when a new job is activated, K/V already in the cache for
  the same prompt prefix is referenced and reused (saving prefill time and
  memory), also from pages of jobs still running.
* "Prompt caching": reuse is not limited to running jobs; the generator tries
  not to overwrite the most recently used pages, so a new job sharing a
  prefix with a recently finished one still finds it cached.

Readings taken (the page fixes no data structure):

* every page is in one of three states: FREE (holds nothing reusable),
  CACHED (unreferenced, holds a full prompt page that a later job may reuse)
  or USED (referenced ``ref > 0`` times: by block-table rows or free stacks
  the caller keeps);
* a page is reusable by its prefix key: every token id of the prompt up to
  the end of that page. Equal keys mean equal K/V, since the K/V of a token
  depends only on the tokens up to it (position included). Only full pages
  get a key; a prompt's partial last page is private;
* admission matches the prompt's full pages from the start and stops at the
  first miss; a page is matched only if at least one prompt token follows
  it, so the prefill always has a token to run and never writes into a
  shared page. The cached-token count returned is 256 x matched pages;
* new pages come from FREE pages first (lowest index first, which fills
  holes), then by evicting the CACHED page released longest ago (ties: lowest
  index), which forgets its key. Admission is all-or-nothing: with too few
  pages nothing changes;
* release drops one reference; at zero a keyed page becomes CACHED (stamped
  with a release counter), an unkeyed one FREE;
* defragmentation: ``n_occ`` = pages not FREE. Movable pages (CACHED ones; also
  USED ones when ``move_referenced``) at index >= n_occ move into the FREE
  pages below n_occ, both taken in ascending order. A move's target is always
  FREE and never the source of another move, so all moves can run at once.
  Returned: the page remap (identity except moved pages) and the move list;
  the caller copies the page contents and, for moved USED pages, rewrites its
  tables through the remap.
"""

PAGE = 256

FREE, CACHED, USED = 0, 1, 2


class PagePool:
    def __init__(self, num_pages):
        if num_pages < 1:
            raise ValueError("num_pages >= 1")
        self.P = int(num_pages)
        self.ref = [0] * self.P
        self.state = [FREE] * self.P
        self.key = [None] * self.P        # prefix key of a keyed page
        self.stamp = [0] * self.P         # release counter value when it became CACHED
        self.index = {}                   # prefix key -> page
        self.clock = 0

    # ------------------------------------------------------------- queries

    def stats(self):
        """(free, cached, used) page counts."""
        return (self.state.count(FREE), self.state.count(CACHED), self.state.count(USED))

    def allocatable(self):
        return self.P - self.state.count(USED)

    # ---------------------------------------------------------- allocation

    def _take(self):
        """One page for new content: the lowest FREE page, else the CACHED
        page released longest ago (lowest index on ties), forgetting its key."""
        for p in range(self.P):
            if self.state[p] == FREE:
                return p
        best = None
        for p in range(self.P):
            if self.state[p] == CACHED and (best is None or self.stamp[p] < self.stamp[best]):
                best = p
        if best is None:
            raise ValueError("no page left")
        del self.index[self.key[best]]
        self.key[best] = None
        self.state[best] = FREE
        return best

    def _use(self, p):
        self.ref[p] = 1
        self.state[p] = USED

    def alloc(self, n):
        """n private pages (reference count 1, no key), in allocation order."""
        if n < 0 or n > self.allocatable():
            raise ValueError("not enough pages")
        out = []
        for _ in range(n):
            p = self._take()
            self._use(p)
            out.append(p)
        return out

    def retain(self, pages):
        for p in pages:
            if self.state[p] != USED:
                raise ValueError(f"page {p} is not in use")
        for p in pages:
            self.ref[p] += 1

    def release(self, pages):
        """Drop one reference of each page (a page may appear several times)."""
        need = {}
        for p in pages:
            need[p] = need.get(p, 0) + 1
        for p, k in need.items():
            if not (0 <= p < self.P) or self.ref[p] < k:
                raise ValueError(f"page {p} released more often than referenced")
        for p in pages:
            self.ref[p] -= 1
            if self.ref[p] == 0:
                if self.key[p] is not None:
                    self.clock += 1
                    self.state[p] = CACHED
                    self.stamp[p] = self.clock
                else:
                    self.state[p] = FREE

    # ----------------------------------------------------------- admission

    def admit(self, tokens):
        """Pages for a prompt. Returns (pages in table order, cached tokens)."""
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        n_pages = -(-n // PAGE)
        # match full pages from the start while a prompt token follows them
        matched = []
        for j in range((n - 1) // PAGE if n > 0 else 0):
            p = self.index.get(tuple(tokens[:(j + 1) * PAGE]))
            if p is None:
                break
            matched.append(p)
        revived = sum(1 for p in matched if self.state[p] == CACHED)
        fresh = n_pages - len(matched)
        if fresh > self.allocatable() - revived:
            raise ValueError("not enough pages")
        pages = []
        for p in matched:
            if self.state[p] == CACHED:
                self._use(p)
            else:
                self.ref[p] += 1
            pages.append(p)
        for j in range(len(matched), n_pages):
            p = self._take()
            self._use(p)
            if (j + 1) * PAGE <= n:            # a full page gets its prefix key
                k = tuple(tokens[:(j + 1) * PAGE])
                if k not in self.index:
                    self.index[k] = p
                    self.key[p] = k
            pages.append(p)
        return pages, len(matched) * PAGE

    # ------------------------------------------------------ defragmentation

    def defrag(self, move_referenced=False):
        """Returns (remap list of P entries, [(src, dst), ...])."""
        n_occ = sum(1 for st in self.state if st != FREE)
        holes = [p for p in range(n_occ) if self.state[p] == FREE]
        movable = (CACHED, USED) if move_referenced else (CACHED,)
        sources = [p for p in range(n_occ, self.P) if self.state[p] in movable]
        moves = list(zip(sources, holes))
        remap = list(range(self.P))
        for src, dst in moves:
            remap[src] = dst
            self.ref[dst], self.state[dst], self.stamp[dst] = self.ref[src], self.state[src], self.stamp[src]
            self.key[dst] = self.key[src]
            if self.key[dst] is not None:
                self.index[self.key[dst]] = dst
            self.ref[src], self.state[src], self.stamp[src], self.key[src] = 0, FREE, 0, None
        return remap, moves


def copy_pages(k_pool, v_pool, moves):
    """Page contents after the moves: every head of page src copied to dst
    (numpy arrays [P, Hkv, 256, D]; returns copies)."""
    k, v = k_pool.copy(), v_pool.copy()
    for src, dst in moves:
        k[dst] = k_pool[src]
        v[dst] = v_pool[src]
    return k, v


def remap_table(block_table, remap):
    """Block table with every entry t >= 0 replaced by remap[t]."""
    out = block_table.copy()
    for b in range(out.shape[0]):
        for j in range(out.shape[1]):
            t = int(out[b, j])
            if t >= 0:
                out[b, j] = remap[t]
    return out
