"""Seeded input generators: draft trees, DFlash-style blocks, target-logit rows,
prompts.  Random draws only -- no step of the Graft method lives here.

Every draw comes from ``rng_for(cfg_id, request, step, stream)``, a PCG64
generator keyed by a ``SeedSequence`` of those four integers, so any
(request, step) can be regenerated on its own.

Target logits are materialised from a small pool of N(0,1) rows: row r of a
step is ``roll(pool[idx_r], -shift_r)`` with one entry raised by ``bump``
(6.0) at the token the synthetic target "intends" to emit next.  The row
descriptors (idx, shift, bump column, bump bit pattern) are computed once on
the host; materialising them is a pure bit copy, so the host (numpy) and
device (torch) copies are identical by construction.
"""
from __future__ import annotations

import numpy as np

from .configs import GraftConfig

STREAM_DRAFT = 1
STREAM_LOGITS = 2
STREAM_ROOT = 3
STREAM_INGEST = 4
STREAM_TABLES = 5
STREAM_PROMPT = 6
WARMUP_STREAM_OFFSET = 100     # warm-up steps draw from their own streams


def rng_for(cfg_id: int, request: int, step: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, request, step, stream])))


# --------------------------------------------------------------------------------------
# bf16 helpers (bit patterns held in uint16)
# --------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------
# static draft tree (EAGLE-style, depth 6, <= 8 children per expanded node, 60 nodes)
# --------------------------------------------------------------------------------------

def static_tree(layer_sizes=(8, 16, 12, 10, 8, 6), width=8):
    """Topology: each layer's nodes are the children of the previous layer's nodes
    in order, each parent taking up to ``width`` children (ranks 0..width-1) until
    the layer is full.  Returns (parent, layer, rank) as int32 arrays; parent -1 is
    the root (the last committed token)."""
    parent, layer, rank = [], [], []
    prev = [-1]
    for L, size in enumerate(layer_sizes):
        if size > width * len(prev):
            raise ValueError("layer %d too large for its parents" % L)
        cur, pi, r = [], 0, 0
        for _ in range(size):
            if r == width:
                pi, r = pi + 1, 0
            parent.append(prev[pi])
            layer.append(L)
            rank.append(r)
            cur.append(len(parent) - 1)
            r += 1
        prev = cur
    return (np.array(parent, np.int32), np.array(layer, np.int32), np.array(rank, np.int32))


def children_lists(parent: np.ndarray):
    kids = {-1: []}
    for i in range(len(parent)):
        kids.setdefault(i, [])
    for i, p in enumerate(parent):
        kids[int(p)].append(i)
    return kids


# --------------------------------------------------------------------------------------
# "intended next token" of the synthetic target / drafter, per workload
# --------------------------------------------------------------------------------------

class BigramIntent:
    """Next token = bigram[last token].  30 % of rows map into a fixed set of hot
    tokens, the rest are uniform over V (workloads 1, 3, 5)."""

    def __init__(self, cfg: GraftConfig):
        rng = rng_for(cfg.cfg_id, 0, 0, STREAM_TABLES)
        V = cfg.V
        hot = rng.choice(V, size=min(cfg.n_hot, V), replace=False)
        big = rng.integers(0, V, size=V)
        is_hot = rng.random(V) < cfg.hot_frac
        big[is_hot] = hot[rng.integers(0, len(hot), size=int(is_hot.sum()))]
        self.bigram = big.astype(np.int64)

    def next(self, prev: int, tok: int) -> int:
        return int(self.bigram[tok])

    def commit(self, tokens):
        pass

    def clone(self):
        return self  # stateless


class Order2Intent:
    """Order-2 successor with a Zipf(1.1) prior over a seeded permutation of V, plus
    copy-back: for 20 % of (a, b) pairs that occurred before in the committed
    stream, the successor repeats what followed that pair last time (workload 2)."""

    def __init__(self, cfg: GraftConfig, shared=None):
        if shared is None:
            rng = rng_for(cfg.cfg_id, 0, 0, STREAM_TABLES)
            perm = rng.permutation(cfg.V).astype(np.int64)
            ranks = np.arange(1, cfg.V + 1, dtype=np.float64)
            w = ranks ** (-cfg.zipf_s)
            cdf = np.cumsum(w)
            cdf /= cdf[-1]
            salt = int(rng.integers(1, 2**61))
            shared = (perm, cdf, salt, cfg.copy_frac)
        self.shared = shared
        self.pairs = {}
        self.hist = []

    @staticmethod
    def _mix(x: int) -> int:
        x &= (1 << 64) - 1
        x ^= x >> 33
        x = (x * 0xFF51AFD7ED558CCD) & ((1 << 64) - 1)
        x ^= x >> 33
        x = (x * 0xC4CEB9FE1A85EC53) & ((1 << 64) - 1)
        x ^= x >> 33
        return x

    def _h(self, a: int, b: int) -> int:
        return self._mix(self.shared[2] ^ (a * 1000003 + b * 7919 + 12345))

    def next(self, prev: int, tok: int) -> int:
        perm, cdf, _, copy_frac = self.shared
        a = -1 if prev is None else int(prev)
        h = self._h(a, int(tok))
        if (a, int(tok)) in self.pairs and (h & 0xFFFF) < int(copy_frac * 65536):
            return self.pairs[(a, int(tok))]
        u = ((h >> 11) & ((1 << 53) - 1)) / float(1 << 53)
        r = int(np.searchsorted(cdf, u, side="right"))
        return int(perm[min(r, len(perm) - 1)])

    def commit(self, tokens):
        for t in tokens:
            t = int(t)
            if len(self.hist) >= 2:
                self.pairs[(self.hist[-2], self.hist[-1])] = t
            self.hist.append(t)

    def clone(self):
        c = Order2Intent.__new__(Order2Intent)
        c.shared = self.shared
        c.pairs = dict(self.pairs)
        c.hist = list(self.hist)
        return c


class PromptCopyIntent:
    """Next token = what followed the most recent occurrence of the last token in
    the prompt + committed stream, else a seeded bigram (workload 4)."""

    def __init__(self, cfg: GraftConfig, prompt: np.ndarray | None = None, shared=None):
        if shared is None:
            shared = BigramIntent(cfg).bigram
        self.bigram = shared
        self.last_next = {}
        self.last = None
        if prompt is not None:
            self.commit(prompt)

    def next(self, prev: int, tok: int) -> int:
        t = int(tok)
        return self.last_next.get(t, int(self.bigram[t]))

    def commit(self, tokens):
        for t in tokens:
            t = int(t)
            if self.last is not None:
                self.last_next[self.last] = t
            self.last = t

    def clone(self):
        c = PromptCopyIntent.__new__(PromptCopyIntent)
        c.bigram = self.bigram
        c.last_next = dict(self.last_next)
        c.last = self.last
        return c


def make_intent(cfg: GraftConfig, prompt=None):
    if cfg.cfg_id == 2:
        return Order2Intent(cfg)
    if cfg.cfg_id == 4:
        return PromptCopyIntent(cfg, prompt)
    return BigramIntent(cfg)


# --------------------------------------------------------------------------------------
# draft inputs
# --------------------------------------------------------------------------------------

def _distinct_others(rng, V, n, exclude):
    out = []
    seen = set([exclude]) if exclude is not None else set()
    while len(out) < n:
        c = int(rng.integers(0, V))
        if c in seen:
            continue
        seen.add(c)
        out.append(c)
    return out


def draft_tree_inputs(cfg: GraftConfig, topo, rng, root_tok: int, prev_root, intent):
    """One request's static draft tree: per-node log-probs and tokens.

    Each expanded node draws 8 logits ~ N(0, sigma^2), log-softmaxes over those 8 and
    hands them in descending order to child ranks 0..7.  The target's intended next
    token is put at child rank J ~ Cat(p_0..p_7) with probability ``draft_hit``; every
    other child is a distinct random id."""
    parent, layer, rank = topo
    Nd = len(parent)
    kids = children_lists(parent)
    logp = np.zeros(Nd, np.float32)
    tok = np.full(Nd, -1, np.int64)
    order = [-1] + list(range(Nd))
    for u in order:
        ch = kids[u]
        if not ch:
            continue
        z = rng.normal(0.0, cfg.draft_sigma, 8)
        m = z.max()
        lsm = z - (m + np.log(np.exp(z - m).sum()))
        lsm = np.sort(lsm)[::-1]
        p = np.exp(lsm)
        p /= p.sum()
        J = int(rng.choice(8, p=p))
        hit = rng.random() < cfg.draft_hit
        ctx_prev = prev_root if u < 0 else (int(root_tok) if parent[u] < 0 else int(tok[parent[u]]))
        ctx_tok = int(root_tok) if u < 0 else int(tok[u])
        ystar = intent.next(ctx_prev, ctx_tok)
        place = J if (hit and J < len(ch)) else -1
        others = _distinct_others(rng, cfg.V, len(ch), ystar)
        oi = 0
        for c in ch:
            r = int(rank[c])
            logp[c] = np.float32(lsm[r])
            if r == place:
                tok[c] = ystar
            else:
                tok[c] = others[oi]
                oi += 1
    return logp, tok.astype(np.int32)


def tail_block_inputs(cfg: GraftConfig, rng, root_tok: int, prev_root, intent):
    """One request's 16-token block: confidences are Beta(4,2) draws sorted in
    descending order; token i is the intended next token with probability conf[i]."""
    L = cfg.tail_block
    conf = np.sort(rng.beta(4.0, 2.0, L))[::-1].astype(np.float32)
    tok = np.zeros(L, np.int32)
    a, b = prev_root, int(root_tok)
    for i in range(L):
        y = intent.next(a, b)
        if rng.random() < float(conf[i]):
            t = y
        else:
            t = _distinct_others(rng, cfg.V, 1, y)[0]
        tok[i] = t
        a, b = b, t
    return conf, tok


# --------------------------------------------------------------------------------------
# target logits
# --------------------------------------------------------------------------------------

class NoisePool:
    """``rows`` N(0,1) rows of length V, stored as bf16 or f32 bit patterns."""

    def __init__(self, cfg: GraftConfig):
        rng = rng_for(cfg.cfg_id, 0, 0, 0xF00D)
        z = rng.standard_normal((cfg.noise_pool_rows, cfg.V), dtype=np.float32)
        if cfg.dtype == "bf16":
            self.bits = f32_to_bf16_bits(z).reshape(z.shape)
        else:
            self.bits = z.view(np.uint32)
        self.dtype = cfg.dtype
        self.V = cfg.V
        self.bump = np.float32(cfg.bump)

    def bump_bits(self, idx, col, shift):
        src = self.bits[idx, (np.asarray(col, np.int64) + shift) % self.V]
        if self.dtype == "bf16":
            v = bf16_bits_to_f32(src) + self.bump
            return f32_to_bf16_bits(v)
        v = src.view(np.float32) + self.bump
        return v.astype(np.float32).view(np.uint32)


def row_descriptors(pool: NoisePool, rng, cols):
    """Descriptors for len(cols) rows: pool index, shift, bump column, bump bits."""
    n = len(cols)
    idx = rng.integers(0, pool.bits.shape[0], size=n)
    shift = rng.integers(0, pool.V, size=n)
    cols = np.asarray(cols, np.int64)
    return {"idx": idx, "shift": shift, "col": cols, "bits": pool.bump_bits(idx, cols, shift)}


def materialize_rows_np(pool: NoisePool, desc, out=None) -> np.ndarray:
    """Host copy: row r = roll(pool[idx_r], -shift_r) with the bump written in
    (into `out`, an array of at least n rows of V, when given)."""
    V = pool.V
    n = len(desc["idx"])
    if out is None or out.dtype != pool.bits.dtype or out.shape[0] < n or out.shape[1] != V:
        out = np.empty((n, V), pool.bits.dtype)
    else:
        out = out[:n]
    for r in range(n):
        src = pool.bits[desc["idx"][r]]
        s = int(desc["shift"][r])
        out[r, : V - s] = src[s:]
        out[r, V - s:] = src[:s]
    out[np.arange(n), desc["col"]] = desc["bits"]
    return out


def tree_row_cols(intent, tok_flat, parent_flat, prev_root):
    """Intended next token for every flattened row of one request."""
    cols = []
    for f in range(len(tok_flat)):
        if int(tok_flat[f]) < 0:      # an empty row (padding): its scores are never used
            cols.append(0)
            continue
        p = int(parent_flat[f])
        prev = prev_root if p < 0 else int(tok_flat[p])
        cols.append(intent.next(prev, int(tok_flat[f])))
    return cols


# --------------------------------------------------------------------------------------
# long prompt (workload 4)
# --------------------------------------------------------------------------------------

def long_prompt(cfg: GraftConfig) -> np.ndarray:
    """32768-token prompt: 35 % of it is repeated 64-token spans over a 4096-id
    identifier sub-vocabulary, the rest uniform filler over V."""
    rng = rng_for(cfg.cfg_id, 0, 0, STREAM_PROMPT)
    ident = rng.choice(cfg.V, size=cfg.ident_vocab, replace=False)
    spans = [rng.choice(ident, size=cfg.span_len) for _ in range(24)]
    out = []
    while len(out) < cfg.prompt_len:
        if rng.random() < cfg.span_frac:
            out.extend(spans[int(rng.integers(0, len(spans)))].tolist())
        else:
            out.extend(rng.integers(0, cfg.V, size=cfg.span_len).tolist())
    return np.array(out[: cfg.prompt_len], np.int32)


def prompt_row_cols(prompt: np.ndarray, intent_after_prompt) -> np.ndarray:
    """Intended next token at each prompt position: the actual next prompt token;
    for the last position, the target's intended continuation."""
    cols = np.empty(len(prompt), np.int64)
    cols[:-1] = prompt[1:]
    cols[-1] = intent_after_prompt.next(int(prompt[-2]), int(prompt[-1]))
    return cols


def initial_roots(cfg: GraftConfig):
    roots, prevs = [], []
    for b in range(cfg.B):
        rng = rng_for(cfg.cfg_id, b, 0, STREAM_ROOT)
        prevs.append(int(rng.integers(0, cfg.V)))
        roots.append(int(rng.integers(0, cfg.V)))
    return np.array(roots, np.int32), prevs
