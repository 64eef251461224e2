"""Seeded synthetic inputs for the speculative-decoding verification step.

This module only draws inputs: it holds none of the verification arithmetic
(no attention, no argmax, no acceptance walk, no compaction).  Both the CPU
oracle and the HIP path consume exactly the arrays produced here.

What is drawn, per case, in a fixed order so a seed fixes every byte:

1. per-request scalars: committed context length L_i, draft length gamma_i
   (chains) and, for ragged batches, a per-request draft-match probability;
2. draft-tree shapes (parent arrays, root = -1, parent[j] < j, BFS order);
3. the physical page permutation of the paged KV pool;
4. queries Q (bf16 bit patterns, [T, Hq, D], packed padding-free by cu_q);
5. the K/V pool (bf16 bit patterns, [num_pages, Hkv, page_size, D], the
   same token-major layout for K and V, on the host or drawn on the device;
   a caller of the library's *_vt calls transposes each V page block);
6. target logits (fp32, [T, V]);
7. the planted greedy target token of every logits row: a uniformly drawn id
   whose logit is raised strictly above the row's maximum, so the row's
   greedy token is known by construction without computing any argmax;
8. draft tokens: a draft copies its parent's planted target with the case's
   match probability, otherwise it is a uniformly drawn different id.

Geometry and distributions follow the workloads the pages evaluate (Llama-3
8B/70B and Qwen3-8B attention shapes; SwiftSpec-style batch-1 trees; FASER's
per-request draft lengths in continuous batches).  No dataset item is used:
seeded distributions stand in for the datasets' acceptance behaviour.

bf16 values are produced from fp32 samples with round-to-nearest-even on the
bit pattern, so the oracle and the GPU read identical bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PAGE_SIZE = 16
POISON_MAGNITUDE = 1.0e3


# --------------------------------------------------------------------------
# bf16 bit handling (pure data conversion)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Case container
# --------------------------------------------------------------------------
@dataclass
class VerifyCase:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    vocab: int
    context_lens: np.ndarray          # int32 [B]   committed L_i
    q_lens: np.ndarray                # int32 [B]   verify tokens q_i (chain: gamma_i+1)
    cu_q: np.ndarray                  # int32 [B+1] prefix sums of q_i
    tree_parent: Optional[np.ndarray]  # int32 [T] local parent (root -1) or None for chains
    block_tables: np.ndarray          # int32 [B, max_blocks] physical page ids, padded with poison
    num_pages: int
    poison_page: int
    q: np.ndarray                     # uint16 [T, Hq, D]
    k_cache: Optional[np.ndarray]     # uint16 [num_pages, Hkv, P, D]  (None when drawn on device)
    v_cache: Optional[np.ndarray]
    logits: Optional[np.ndarray]      # float32 [T, V] (None when drawn on device)
    draft_tokens: np.ndarray          # int32 [T]
    planted_target: np.ndarray        # int32 [T] greedy token planted in each logits row
    match_prob: np.ndarray            # float64 [T] probability each draft copies its parent's target
    qkv_scale: float = 1.0
    logit_sigma: float = 1.0
    kv_device: Optional[str] = None
    k_cache_dev: object = None        # torch tensors when the pool is drawn on device,
    v_cache_dev: object = None        # both in the layout of k_cache / v_cache
    logits_dev: object = None
    extra: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes_per_layer(self) -> int:
        """Algorithmic K+V bytes one verify-attention pass must stream."""
        keys = int(np.sum(self.context_lens.astype(np.int64) + self.q_lens))
        return keys * self.num_kv_heads * self.head_dim * 2 * 2

    def qo_bytes(self) -> int:
        return self.total_q * self.num_q_heads * self.head_dim * 2 * 2

    def attn_flops(self) -> int:
        s = np.sum(self.q_lens.astype(np.int64) * (self.context_lens.astype(np.int64) + self.q_lens))
        return int(4 * self.head_dim * self.num_q_heads * s)


# --------------------------------------------------------------------------
# Named workloads
# --------------------------------------------------------------------------
#   ctx:   ("fixed", L) | ("uniform", lo, hi) | ("loguniform", lo, hi)
#   gamma: int | ("uniform", lo, hi)
#   match: ("p", p) | ("beta", a, b) | ("tree", p_first_child, p_sibling)
CONFIGS = {
    # tiny correctness case (chain)
    "tiny_chain": dict(batch=1, gamma=4, tree=None, hq=8, hkv=2, d=64, ctx=("fixed", 256),
                       vocab=1024, logit_sigma=2.0, qkv_scale=1.0, match=("p", 0.7), seed=1),
    # Llama-3.1-8B attention geometry, batch-1 chain
    "llama31_8b_chain": dict(batch=1, gamma=5, tree=None, hq=32, hkv=8, d=128, ctx=("fixed", 4096),
                             vocab=128256, logit_sigma=3.0, qkv_scale=1 / math.sqrt(128),
                             match=("p", 0.8), seed=2),
    # Llama-3-70B geometry, SwiftSpec-style batch-1 draft tree (64 nodes, depth 6)
    "llama3_70b_tree": dict(batch=1, gamma=None, tree=dict(nodes=64, depth=6, root_fanout_max=4, fanout_max=4),
                            hq=64, hkv=8, d=128, ctx=("fixed", 8192), vocab=128256, logit_sigma=3.0,
                            qkv_scale=1 / math.sqrt(128), match=("tree", 0.6, 0.1), seed=3),
    # Qwen3-8B geometry, FASER-style ragged continuous batch
    "qwen3_8b_ragged": dict(batch=64, gamma=("uniform", 1, 8), tree=None, hq=32, hkv=8, d=128,
                            ctx=("loguniform", 512, 32768), vocab=151936, logit_sigma=3.0,
                            qkv_scale=1 / math.sqrt(128), match=("beta", 2.0, 2.0), seed=4),
    # Llama-3-70B geometry, large-batch chain verify over a shared interleaved page pool
    "llama3_70b_b256": dict(batch=256, gamma=3, tree=None, hq=64, hkv=8, d=128, ctx=("uniform", 2048, 8192),
                            vocab=128256, logit_sigma=3.0, qkv_scale=1 / math.sqrt(128),
                            match=("p", 0.75), seed=5),
}

# Transformer layer counts of the models whose attention geometry each workload
# uses (public model configurations); used to express per-step figures.
MODEL_LAYERS = {"tiny_chain": 1, "llama31_8b_chain": 32, "llama3_70b_tree": 80,
                "qwen3_8b_ragged": 36, "llama3_70b_b256": 80}


# --------------------------------------------------------------------------
# Drawing helpers
# --------------------------------------------------------------------------
def draw_tree(rng: np.random.Generator, nodes: int, depth: int, root_fanout_max: int,
              fanout_max: int) -> np.ndarray:
    """Random draft tree with exactly `nodes` nodes and maximum depth `depth`.

    A spine root->...->depth guarantees the depth; the root's fan-out cap is
    drawn from U{1..root_fanout_max}; every other node takes its parent
    uniformly among nodes of depth < `depth` whose fan-out is below the cap.
    Nodes are relabelled in BFS order (children in creation order), so
    parent[j] < j and parent[0] = -1.
    """
    assert nodes >= depth + 1
    root_cap = int(rng.integers(1, root_fanout_max + 1))
    par = [-1]
    dep = [0]
    kids = [0]
    for d in range(1, depth + 1):      # spine
        par.append(d - 1)
        dep.append(d)
        kids.append(0)
        kids[d - 1] += 1
    while len(par) < nodes:
        cand = [n for n in range(len(par))
                if dep[n] < depth and kids[n] < (root_cap if n == 0 else fanout_max)]
        if not cand:
            raise ValueError("tree caps too small for the requested node count")
        p = cand[int(rng.integers(0, len(cand)))]
        par.append(p)
        dep.append(dep[p] + 1)
        kids.append(0)
        kids[p] += 1
    # BFS relabel: children in creation order
    children = [[] for _ in par]
    for n in range(1, len(par)):
        children[par[n]].append(n)
    order = [0]
    head = 0
    while head < len(order):
        order.extend(children[order[head]])
        head += 1
    new_id = {old: new for new, old in enumerate(order)}
    out = np.empty(len(par), dtype=np.int32)
    for old in order:
        out[new_id[old]] = -1 if par[old] < 0 else new_id[par[old]]
    return out


def _first_child_flags(parent: np.ndarray) -> np.ndarray:
    """True for node j if it is the lowest-indexed child of its parent."""
    seen = set()
    flags = np.zeros(len(parent), dtype=bool)
    for j in range(1, len(parent)):
        if parent[j] not in seen:
            flags[j] = True
            seen.add(int(parent[j]))
    return flags


def _fill_poison(rng: np.random.Generator, shape) -> np.ndarray:
    signs = rng.integers(0, 2, size=shape).astype(np.float32) * 2.0 - 1.0
    return f32_to_bf16_bits(signs * POISON_MAGNITUDE)


def build_case(name: str, seed: int, *, batch: int, q_lens, context_lens, tree_parents,
               hq: int, hkv: int, d: int, vocab: int, logit_sigma: float, qkv_scale: float,
               match_prob_per_req=None, tree_match=None, page_size: int = PAGE_SIZE,
               rng: Optional[np.random.Generator] = None, kv_device: Optional[str] = None,
               logits_device: Optional[str] = None, permute_pages: bool = True,
               extra_pages: int = 0) -> VerifyCase:
    """Assemble a case from already-drawn per-request scalars and tree shapes.

    `rng` continues the case's draw sequence (pages, Q, K/V, logits, planted
    targets, drafts, in that order).  `tree_parents` is a list of per-request
    parent arrays or None (chains).  `match_prob_per_req` gives a chain
    request's per-position match probability; `tree_match` = (p_first, p_sib).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    q_lens = np.asarray(q_lens, dtype=np.int32)
    context_lens = np.asarray(context_lens, dtype=np.int32)
    assert q_lens.shape == (batch,) and context_lens.shape == (batch,)
    cu_q = np.zeros(batch + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    T = int(cu_q[-1])

    # ---- 3. page permutation ------------------------------------------------
    n_pages_req = (context_lens.astype(np.int64) + q_lens + page_size - 1) // page_size
    num_pages = int(n_pages_req.sum()) + 1 + extra_pages
    phys = rng.permutation(num_pages).astype(np.int32) if permute_pages else np.arange(num_pages, dtype=np.int32)
    poison_page = int(phys[-1])
    max_blocks = max(1, int(n_pages_req.max()) if batch else 1)
    block_tables = np.full((batch, max_blocks), poison_page, dtype=np.int32)
    off = 0
    for i in range(batch):
        n = int(n_pages_req[i])
        block_tables[i, :n] = phys[off:off + n]
        off += n

    # ---- 4. Q ---------------------------------------------------------------
    q = f32_to_bf16_bits(rng.standard_normal((T, hq, d), dtype=np.float32) * np.float32(qkv_scale))

    # ---- 5. K/V pool --------------------------------------------------------
    k_cache = v_cache = None
    k_dev = v_dev = None
    shape = (num_pages, hkv, page_size, d)
    if kv_device is None:
        k_cache = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(qkv_scale))
        v_cache = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(qkv_scale))
        k_cache[poison_page] = _fill_poison(rng, shape[1:])
        v_cache[poison_page] = _fill_poison(rng, shape[1:])
        for i in range(batch):
            used = int(context_lens[i] + q_lens[i])
            n = int(n_pages_req[i])
            if used < n * page_size:
                pg = int(block_tables[i, n - 1])
                s0 = used - (n - 1) * page_size
                k_cache[pg, :, s0:, :] = _fill_poison(rng, (hkv, page_size - s0, d))
                v_cache[pg, :, s0:, :] = _fill_poison(rng, (hkv, page_size - s0, d))
    else:
        k_dev, v_dev = _draw_kv_on_device(rng, shape, qkv_scale, kv_device, poison_page,
                                          block_tables, context_lens, q_lens, n_pages_req, page_size)

    # ---- 6. logits ----------------------------------------------------------
    logits = None
    logits_dev = None
    if logits_device is None:
        logits = rng.standard_normal((T, vocab), dtype=np.float32) * np.float32(logit_sigma)
    else:
        logits_dev = _draw_normal_on_device(rng, (T, vocab), logit_sigma, logits_device)

    # ---- 7. planted greedy targets -----------------------------------------
    planted = rng.integers(0, vocab, size=T).astype(np.int32)
    gaps = (rng.exponential(0.25, size=T) * logit_sigma).astype(np.float32)
    if T:
        if logits is not None:
            rowmax = logits.max(axis=1)
            newv = rowmax + gaps
            newv = np.maximum(newv, np.nextafter(rowmax, np.float32(np.inf)))
            logits[np.arange(T), planted] = newv
        else:
            import torch
            rowmax = logits_dev.max(dim=1).values.cpu().numpy()
            newv = rowmax + gaps
            newv = np.maximum(newv, np.nextafter(rowmax, np.float32(np.inf))).astype(np.float32)
            idx = torch.from_numpy(planted.astype(np.int64)).to(logits_dev.device)
            logits_dev[torch.arange(T, device=logits_dev.device), idx] = torch.from_numpy(newv).to(logits_dev.device)

    # ---- 8. draft tokens -----------------------------------------------------
    u = rng.random(T)
    other_off = rng.integers(1, max(vocab, 2), size=T)
    root_tok = rng.integers(0, vocab, size=T)
    draft = np.empty(T, dtype=np.int32)
    match_prob = np.zeros(T, dtype=np.float64)
    parent_all = None
    if tree_parents is not None:
        parent_all = np.concatenate([np.asarray(p, dtype=np.int32) for p in tree_parents]) if batch else np.zeros(0, np.int32)
        assert parent_all.shape == (T,)
    for i in range(batch):
        o = int(cu_q[i])
        qi = int(q_lens[i])
        if qi == 0:
            continue
        draft[o] = root_tok[o]
        if tree_parents is None:
            par = np.arange(-1, qi - 1, dtype=np.int32)
            probs = np.full(qi, float(match_prob_per_req[i]))
        else:
            par = parent_all[o:o + qi]
            first = _first_child_flags(par)
            probs = np.where(first, tree_match[0], tree_match[1]).astype(np.float64)
        for j in range(1, qi):
            target = int(planted[o + par[j]])
            match_prob[o + j] = probs[j]
            if u[o + j] < probs[j]:
                draft[o + j] = target
            else:
                draft[o + j] = (target + int(other_off[o + j])) % vocab
    case = VerifyCase(
        name=name, seed=seed, batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        page_size=page_size, vocab=vocab, context_lens=context_lens, q_lens=q_lens, cu_q=cu_q,
        tree_parent=parent_all, block_tables=block_tables, num_pages=num_pages,
        poison_page=poison_page, q=q, k_cache=k_cache, v_cache=v_cache, logits=logits,
        draft_tokens=draft, planted_target=planted, match_prob=match_prob, qkv_scale=qkv_scale,
        logit_sigma=logit_sigma, kv_device=kv_device, k_cache_dev=k_dev, v_cache_dev=v_dev,
        logits_dev=logits_dev)
    return case


def _draw_normal_on_device(rng, shape, scale, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(rng.integers(0, 2**62)))
    out = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    out.mul_(float(scale))
    return out


def _draw_kv_on_device(rng, shape, scale, device, poison_page, block_tables, context_lens,
                       q_lens, n_pages_req, page_size):
    """Large pools: draw N(0, scale) with torch's seeded device generator, round to bf16 (RNE)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(rng.integers(0, 2**62)))
    out = []
    per_page = int(np.prod(shape[1:]))
    chunk = max(1, (1 << 27) // per_page)
    for _ in range(2):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for p0 in range(0, shape[0], chunk):
            p1 = min(shape[0], p0 + chunk)
            tmp = torch.randn((p1 - p0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
            tmp.mul_(float(scale))
            t[p0:p1].copy_(tmp)
            del tmp
        sign = torch.randint(0, 2, tuple(shape[1:]), generator=g, device=device, dtype=torch.int32)
        t[poison_page] = (sign.to(torch.float32) * 2 - 1).mul_(POISON_MAGNITUDE).to(torch.bfloat16)
        # poison the unused tail slots of each request's last page
        for i in range(len(context_lens)):
            used = int(context_lens[i] + q_lens[i])
            n = int(n_pages_req[i])
            if used < n * page_size:
                pg = int(block_tables[i, n - 1])
                s0 = used - (n - 1) * page_size
                t[pg, :, s0:, :] = POISON_MAGNITUDE
        out.append(t)
    # both [pages, Hkv, P, D] (token-major pages, as the host-drawn pools)
    return out[0], out[1]


def make_case(name: str, seed: Optional[int] = None, *, unit_scale: bool = False,
              qkv_scale: Optional[float] = None, kv_device: Optional[str] = None,
              logits_device: Optional[str] = None, batch: Optional[int] = None) -> VerifyCase:
    """Draw one of the named workloads.  `unit_scale` replaces the Q/K/V scale by 1.

    `batch` overrides the request count (used for batch sweeps at a fixed shape).
    """
    cfg = CONFIGS[name]
    if seed is None:
        seed = cfg["seed"]
    rng = np.random.Generator(np.random.PCG64(seed))
    B = cfg["batch"] if batch is None else int(batch)
    # ---- 1. per-request scalars ---------------------------------------------
    ctx = cfg["ctx"]
    if ctx[0] == "fixed":
        L = np.full(B, ctx[1], dtype=np.int32)
    elif ctx[0] == "uniform":
        L = rng.integers(ctx[1], ctx[2] + 1, size=B).astype(np.int32)
    elif ctx[0] == "loguniform":
        L = np.floor(np.exp(rng.uniform(math.log(ctx[1]), math.log(ctx[2]), size=B))).astype(np.int32)
    else:
        raise ValueError(ctx)
    gamma = cfg["gamma"]
    match = cfg["match"]
    tree = cfg["tree"]
    if tree is None:
        if isinstance(gamma, tuple):
            g = rng.integers(gamma[1], gamma[2] + 1, size=B).astype(np.int32)
        else:
            g = np.full(B, gamma, dtype=np.int32)
        q_lens = g + 1
        if match[0] == "p":
            mp = np.full(B, match[1])
        elif match[0] == "beta":
            mp = rng.beta(match[1], match[2], size=B)
        else:
            raise ValueError(match)
        parents = None
        tree_match = None
    else:
        mp = None
        # ---- 2. tree shapes -------------------------------------------------
        parents = [draw_tree(rng, tree["nodes"], tree["depth"], tree["root_fanout_max"], tree["fanout_max"])
                   for _ in range(B)]
        q_lens = np.array([len(p) for p in parents], dtype=np.int32)
        tree_match = (match[1], match[2])
    scale = 1.0 if unit_scale else (cfg["qkv_scale"] if qkv_scale is None else qkv_scale)
    if qkv_scale is not None:
        scale = qkv_scale
    return build_case(name, seed, batch=B, q_lens=q_lens, context_lens=L, tree_parents=parents,
                      hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"], vocab=cfg["vocab"],
                      logit_sigma=cfg["logit_sigma"], qkv_scale=scale, match_prob_per_req=mp,
                      tree_match=tree_match, rng=rng, kv_device=kv_device,
                      logits_device=logits_device)


def make_custom(seed: int, *, context_lens, q_lens=None, tree_parents=None, hq=8, hkv=2, d=64,
                vocab=512, logit_sigma=2.0, qkv_scale=1.0, match_p=0.7, tree_match=(0.6, 0.2),
                page_size=PAGE_SIZE, permute_pages=True, extra_pages=0) -> VerifyCase:
    """A small hand-shaped case for edge tests (ragged lengths, L=0, q=1, trees)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = len(context_lens)
    if tree_parents is not None:
        q_lens = [len(p) for p in tree_parents]
    mp = np.full(B, match_p)
    return build_case(f"custom{seed}", seed, batch=B, q_lens=q_lens, context_lens=context_lens,
                      tree_parents=tree_parents, hq=hq, hkv=hkv, d=d, vocab=vocab,
                      logit_sigma=logit_sigma, qkv_scale=qkv_scale, match_prob_per_req=mp,
                      tree_match=tree_match, page_size=page_size, rng=rng,
                      permute_pages=permute_pages, extra_pages=extra_pages)


def expected_chain_accept_len(p: float, gamma: int) -> float:
    """Closed form E[accept_len] for a chain whose drafts match independently with prob p."""
    return float(sum(p ** k for k in range(gamma + 1)))
