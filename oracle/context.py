"""Decode driver of the oracle: batch intake, ubatches, KV cells, layer loop.

TEST INFRASTRUCTURE: imported only by tests, smoke() and bench.py's
cpu_baseline leg.

What one ``decode(batch)`` call does, in the pages' order:

1. Validate the batch and fill absent fields (llama.cpp walkthrough,
   "Step 10: forming the batch for one call"): every token id in
   [0, n_vocab); absent sequence ids mean sequence 0; absent positions
   continue each sequence from ``seq_pos_max(s) + 1`` in batch order; absent
   output flags select the last token only, or every token when
   ``output_all``.
2. Split the batch into consecutive ubatches of at most ``n_ubatch`` tokens,
   processed in order ("Steps 11-12: running the batch through the model").
3. Place each ubatch's tokens in KV cells and record (position, sequences)
   per cell (Ollama engine page, "KV Cache: memory for causal attention":
   find contiguous cache slots, store K/V, build the mask).
4. Run the forward pass over the ubatch (Ollama engine page, "Deep dive: the
   Llama forward pass in Go"): embedding, then per layer attention RMSNorm,
   Q/K/V, RoPE, attention over the cached cells, output projection and
   residual; in the last layer keep only the rows whose logits are wanted
   before the MLP; MLP RMSNorm, SwiGLU, down projection and residual; then
   output RMSNorm and the LM head.
5. Collect one logits row per flagged token in batch order ("Steps 14-15:
   logits in the buffer and choosing the next token"), and the greedy token
   (temperature 0 -> argmax; Ollama engine page, "Token sampling pipeline").

Readings where the pages are silent or inconsistent:
* Return codes: 0 success; 1 the batch could not be placed (fewer free cells
  than tokens), nothing changed; -1 invalid input, nothing changed.
* ``n_batch = min(n_ctx, n_batch)``, ``n_ubatch = min(n_batch, n_ubatch)``
  ("Step 7: creating the inference context"); a batch larger than n_batch is
  invalid.  At most 64 sequences (one bit each in a cell's sequence mask).
* Explicit positions must be >= 0 and greater than every earlier position of
  each of the token's sequences (cache and batch), so no two live cells share
  (sequence, position) and each sequence's cells are position-ordered.
* Cell placement: the first run of T consecutive free cells scanning from
  cell 0; if there is none, the T lowest-index free cells.  Token i of the
  ubatch goes to the i-th chosen cell.
* A token attends to the occupied cells whose sequence set holds the token's
  first sequence id and whose position is <= the token's position; this
  includes itself and earlier tokens of its own ubatch.  Cached K is stored
  after RoPE.
* Sliding-window attention (Ollama engine page, "KV Cache: memory for causal
  attention": a windowed layer's mask is limited to the window, each layer
  attending only to the most recent tokens): with ``n_swa = W > 0`` a
  windowed layer (``swa_layers[l]`` nonzero, or every layer when
  ``swa_layers`` is absent) lets a token at position p see only the cells
  above with position > p - W, i.e. the W most recent positions including
  its own.  Cells outside the window stay in the cache.
* The cache holds K and V in its element type (the Ollama cache carries a
  DType; the llama.cpp walkthrough's KV-cache section names the cache type
  as a storage setting): with ``kv_dtype`` set, each stored value is the
  float64 result rounded to nearest-even in that type (f32, f16 or bf16);
  without it the cache keeps float64.  ``q8_0`` (a quantized cache: the
  backend chapter and the walkthrough's KV-cache section name quantized
  cache types without defining them) stores each row of head_dim values as
  blocks of 32: the value is first rounded to float32 (the precision in
  which a float32 forward pass takes the decision), then
  d = fp16(max|x| / 127), q = round-half-even(x / d) clamped to [-127, 127]
  (q = 0 when d = 0), all in float32; the stored value is d * q.  Imported
  rows for such a cache are float32 values, quantized the same way.
* Logits: one row per flagged token, in batch order, accumulated over the
  ubatches of the call.  Greedy ties go to the lowest index.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .model import OracleModel, widen
from .ops import attend, rms_norm, rope, swiglu_mlp, window_visible

OK, NO_SLOT, INVALID = 0, 1, -1
MAX_SEQ = 64


@dataclass
class DecodeResult:
    status: int
    positions: List[int] = field(default_factory=list)
    seq_ids: List[List[int]] = field(default_factory=list)
    output_flags: List[bool] = field(default_factory=list)
    ubatches: List[range] = field(default_factory=list)
    slots: List[int] = field(default_factory=list)      # cell of each token, batch order
    out_index: List[int] = field(default_factory=list)  # batch indices that have logits
    logits: Optional[np.ndarray] = None                 # [n_out, n_vocab] float64
    tokens: Optional[np.ndarray] = None                 # greedy id per output row

    def logits_ith(self, i: int) -> Optional[np.ndarray]:
        if self.logits is None or i not in self.out_index:
            return None
        return self.logits[self.out_index.index(i)]


def _round_storage(a: np.ndarray, dtype: Optional[str]) -> np.ndarray:
    """Value of ``a`` once stored in the cache's element type (round to
    nearest, ties to even); float64 when no type is given."""
    if dtype is None or dtype == "f64":
        return a
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        f = a.astype(np.float32)
        u = f.view(np.uint32)
        u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
        return u.view(np.float32).astype(np.float64)
    if dtype == "q8_0":
        return quantize_q8_0_rows(a)
    raise ValueError(dtype)


def quantize_q8_0_rows(a: np.ndarray) -> np.ndarray:
    """Stored value of a Q8_0 cache row (last axis, a multiple of 32): per
    block of 32, d = fp16(max|x| / 127) and q = round-half-even(x / d)
    clamped to [-127, 127], with x rounded to float32 first and every step in
    float32; returns d * q (exact) in float64."""
    shape = a.shape
    f = np.asarray(a, dtype=np.float64).astype(np.float32).reshape(*shape[:-1], shape[-1] // 32, 32)
    amax = np.max(np.abs(f), axis=-1)
    d = (amax / np.float32(127)).astype(np.float16)
    d32 = d.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d32 > 0, np.rint(f / np.where(d32 > 0, d32, np.float32(1))), np.float32(0))
    q = np.clip(q, -127, 127)
    return (q.astype(np.float64) * d.astype(np.float64)[..., None]).reshape(shape)


class OracleContext:
    def __init__(self, model: Optional[OracleModel], n_ctx: int, n_batch: Optional[int] = None,
                 n_ubatch: int = 512, n_seq_max: int = 1, output_all: bool = False,
                 compute: bool = True, kv_dtype: Optional[str] = None):
        if n_ctx <= 0 or n_seq_max < 1 or n_seq_max > MAX_SEQ:
            raise ValueError("invalid context parameters")
        self.model = model
        self.hp = model.hp if model is not None else None
        self.n_ctx = int(n_ctx)
        nb = self.n_ctx if n_batch is None else int(n_batch)
        self.n_batch = min(self.n_ctx, nb)
        self.n_ubatch = min(self.n_batch, int(n_ubatch))
        if self.n_batch <= 0 or self.n_ubatch <= 0:
            raise ValueError("invalid batch sizes")
        self.n_seq_max = int(n_seq_max)
        self.output_all = bool(output_all)
        self.compute = compute and model is not None
        self.kv_dtype = kv_dtype
        self.cell_pos = np.full(self.n_ctx, -1, dtype=np.int64)   # -1 = free
        self.cell_seq = np.zeros(self.n_ctx, dtype=np.uint64)     # bit s = belongs to seq s
        self.k_cache: dict = {}
        self.v_cache: dict = {}

    # ---- bookkeeping ------------------------------------------------------

    def clear(self) -> None:
        self.cell_pos[:] = -1
        self.cell_seq[:] = 0
        self.k_cache.clear()
        self.v_cache.clear()

    def seq_pos_max(self, s: int) -> int:
        """Largest position held by sequence s, or -1 if it has no cell."""
        m = (self.cell_seq >> np.uint64(s)) & np.uint64(1)
        sel = self.cell_pos[m.astype(bool)]
        return int(sel.max()) if sel.size else -1

    def n_free(self) -> int:
        return int(np.count_nonzero(self.cell_pos < 0))

    def find_slots(self, n: int) -> Optional[np.ndarray]:
        """First run of n consecutive free cells from cell 0, else the n
        lowest-index free cells, else None."""
        free = np.flatnonzero(self.cell_pos < 0)
        if free.size < n:
            return None
        span = free[n - 1:] - free[: free.size - n + 1]
        hit = np.flatnonzero(span == n - 1)
        if hit.size:
            start = int(free[hit[0]])
            return np.arange(start, start + n, dtype=np.int64)
        return free[:n].astype(np.int64)

    def _intake(self, tokens, pos, seq_ids, logits):
        """Validation and defaults; returns (status, positions, seqs, flags)."""
        n = len(tokens) if tokens is not None else 0
        if n <= 0 or n > self.n_batch:
            return INVALID, None, None, None
        V = self.hp["n_vocab"] if self.hp is not None else None
        toks = [int(t) for t in tokens]
        if V is not None and any(t < 0 or t >= V for t in toks):
            return INVALID, None, None, None
        if seq_ids is None:
            seqs = [[0] for _ in range(n)]
        else:
            if len(seq_ids) != n:
                return INVALID, None, None, None
            seqs = [list(map(int, s)) for s in seq_ids]
            for s in seqs:
                if len(s) < 1 or len(set(s)) != len(s) or any(x < 0 or x >= self.n_seq_max for x in s):
                    return INVALID, None, None, None
        # running last position per sequence (cache, then this batch)
        last = {s: self.seq_pos_max(s) for s in range(self.n_seq_max)}
        out_pos = []
        for i in range(n):
            p = last[seqs[i][0]] + 1 if pos is None else int(pos[i])
            if p < 0 or any(p <= last[s] for s in seqs[i]):
                return INVALID, None, None, None
            for s in seqs[i]:
                last[s] = p
            out_pos.append(p)
        if logits is None:
            flags = [True] * n if self.output_all else [False] * (n - 1) + [True]
        else:
            if len(logits) != n:
                return INVALID, None, None, None
            flags = [bool(f) for f in logits]
        return OK, out_pos, seqs, flags

    # ---- decode -----------------------------------------------------------

    def decode(self, tokens: Sequence[int], pos: Optional[Sequence[int]] = None,
               seq_ids: Optional[Sequence[Sequence[int]]] = None,
               logits: Optional[Sequence[bool]] = None) -> DecodeResult:
        st, positions, seqs, flags = self._intake(tokens, pos, seq_ids, logits)
        if st != OK:
            return DecodeResult(status=st)
        n = len(tokens)
        if self.n_free() < n:
            return DecodeResult(status=NO_SLOT)
        res = DecodeResult(status=OK, positions=positions, seq_ids=seqs, output_flags=flags)
        toks = np.asarray(tokens, dtype=np.int64)
        rows = []
        for u0 in range(0, n, self.n_ubatch):
            ub = range(u0, min(n, u0 + self.n_ubatch))
            res.ubatches.append(ub)
            cells = self.find_slots(len(ub))
            assert cells is not None  # total free space was checked above
            for i, t in enumerate(ub):
                self.cell_pos[cells[i]] = positions[t]
                m = 0
                for s in seqs[t]:
                    m |= 1 << s
                self.cell_seq[cells[i]] = np.uint64(m)
            res.slots.extend(int(c) for c in cells)
            sel = [i for i, t in enumerate(ub) if flags[t]]
            res.out_index.extend(ub[i] for i in sel)
            if self.compute:
                out = self._forward(toks[ub.start:ub.stop], np.asarray([positions[t] for t in ub]),
                                    [seqs[t][0] for t in ub], cells, sel)
                if out is not None:
                    rows.append(out)
        if self.compute:
            V = self.hp["n_vocab"]
            res.logits = np.concatenate(rows, axis=0) if rows else np.zeros((0, V))
            res.tokens = np.argmax(res.logits, axis=1) if rows else np.zeros(0, dtype=np.int64)
        return res

    def kv_seq_rm(self, seq: int, p0: int, p1: int) -> int:
        """Remove sequence ``seq`` from its cells with position in [p0, p1)
        (p1 < 0: no upper end); a cell left with no sequence becomes free.
        This is the discarding half of sliding the context window forward
        (Ollama engine page, "KV Cache: memory for causal attention": when
        the cache is full the window slides instead of the whole context
        being dropped)."""
        if seq < 0 or seq >= self.n_seq_max or p0 < 0 or (p1 >= 0 and p1 < p0):
            return INVALID
        bit = np.uint64(1 << seq)
        hit = ((self.cell_seq & bit) != 0) & (self.cell_pos >= p0)
        if p1 >= 0:
            hit &= self.cell_pos < p1
        self.cell_seq[hit] &= ~bit
        self.cell_pos[hit & (self.cell_seq == 0)] = -1
        return OK

    def kv_seq_shift(self, seq: int, p0: int, p1: int, delta: int) -> int:
        """Add ``delta`` to the positions of sequence ``seq``'s cells with
        position in [p0, p1) (p1 < 0: no upper end) and rotate their cached
        keys by ``delta`` (Ollama engine page, "KV Cache: memory for causal
        attention": the model's shift function adjusts the RoPE position
        encoding of the cached keys).  Keys are stored after RoPE at position
        p; rotating them by delta gives the keys of position p + delta,
        because the rotations compose (R(a) R(b) = R(a + b)); the result is
        stored in the cache's element type again.  The cells must belong to
        ``seq`` alone, and ``seq``'s positions must keep their order and stay
        distinct and >= 0; otherwise nothing changes and -1 is returned."""
        if seq < 0 or seq >= self.n_seq_max or p0 < 0 or (p1 >= 0 and p1 < p0):
            return INVALID
        bit = np.uint64(1 << seq)
        mine = np.flatnonzero((self.cell_seq & bit) != 0)
        pos = self.cell_pos[mine]
        hit = pos >= p0
        if p1 >= 0:
            hit &= pos < p1
        if not hit.any() or delta == 0:
            return OK
        if np.any(self.cell_seq[mine[hit]] != bit):
            return INVALID
        new = pos + np.where(hit, delta, 0)
        order = np.argsort(pos, kind="stable")
        if np.any(new < 0) or np.any(np.diff(new[order]) <= 0):
            return INVALID
        cells = mine[hit]
        self.cell_pos[cells] += delta
        if self.compute:
            theta = self.hp["rope_theta"]
            for l in list(self.k_cache):
                kc = self.k_cache[l]
                kc[cells] = _round_storage(rope(kc[cells], np.full(cells.size, delta), theta), self.kv_dtype)
        return OK

    def kv_import(self, seq: int, pos0: int, pos1: int, k_layers, v_layers) -> int:
        """Place positions [pos0, pos1) of sequence ``seq`` in cells (one chunk,
        same placement rule as a ubatch) holding the given post-RoPE K and V.
        ``k_layers[l]`` / ``v_layers[l]`` are [pos1-pos0, n_head_kv, head_dim]
        stored values (float32 or bf16 bits), or callables l -> such arrays."""
        n = pos1 - pos0
        if n <= 0 or seq < 0 or seq >= self.n_seq_max or pos0 <= self.seq_pos_max(seq):
            return INVALID
        cells = self.find_slots(n)
        if cells is None:
            return NO_SLOT
        self.cell_pos[cells] = np.arange(pos0, pos1)
        self.cell_seq[cells] = np.uint64(1 << seq)
        if self.compute:
            for l in range(self.hp["n_layer"]):
                kl = k_layers(l) if callable(k_layers) else k_layers[l]
                vl = v_layers(l) if callable(v_layers) else v_layers[l]
                self._layer_cache(l)[0][cells] = _round_storage(widen(kl), self.kv_dtype)
                self._layer_cache(l)[1][cells] = _round_storage(widen(vl), self.kv_dtype)
        self.last_import_cells = cells
        return OK

    # ---- numerics ---------------------------------------------------------

    def _layer_cache(self, l: int):
        if l not in self.k_cache:
            shape = (self.n_ctx, self.hp["n_head_kv"], self.hp["head_dim"])
            self.k_cache[l] = np.zeros(shape, dtype=np.float64)
            self.v_cache[l] = np.zeros(shape, dtype=np.float64)
        return self.k_cache[l], self.v_cache[l]

    def _forward(self, toks, pos, seq0, cells, sel) -> Optional[np.ndarray]:
        hp, m = self.hp, self.model
        H, Hkv, hd = hp["n_head"], hp["n_head_kv"], hp["head_dim"]
        L, eps, theta = hp["n_layer"], hp["rms_eps"], hp["rope_theta"]
        T = len(toks)
        # visible cells per token: same (first) sequence, position <= own;
        # for windowed layers also position > own - W
        W = int(hp.get("n_swa") or 0)
        flags = hp.get("swa_layers")
        windowed = [W > 0 and (flags is None or bool(flags[l])) for l in range(L)]
        visible, visible_w = [], []
        for t in range(T):
            inseq = ((self.cell_seq >> np.uint64(seq0[t])) & np.uint64(1)).astype(bool)
            ok = inseq & (self.cell_pos >= 0) & (self.cell_pos <= pos[t])
            visible.append(np.flatnonzero(ok))
            visible_w.append(np.flatnonzero(ok & window_visible(self.cell_pos, pos[t], W)) if W > 0 else None)
        x = m.embed_rows(toks)
        for l in range(L):
            p = f"blk.{l}."
            h = rms_norm(x, m.w(p + "attn_norm.weight"), eps)
            q = (h @ m.w(p + "attn_q.weight").T).reshape(T, H, hd)
            k = (h @ m.w(p + "attn_k.weight").T).reshape(T, Hkv, hd)
            v = (h @ m.w(p + "attn_v.weight").T).reshape(T, Hkv, hd)
            q = rope(q, pos, theta)
            k = rope(k, pos, theta)
            kc, vc = self._layer_cache(l)
            kc[cells] = _round_storage(k, self.kv_dtype)
            vc[cells] = _round_storage(v, self.kv_dtype)
            vis = visible_w if windowed[l] else visible
            o = np.stack([attend(q[t], kc[vis[t]], vc[vis[t]]) for t in range(T)])
            x = x + o.reshape(T, H * hd) @ m.w(p + "attn_output.weight").T
            if l == L - 1:
                if not sel:
                    return None
                x = x[sel]
            h2 = rms_norm(x, m.w(p + "ffn_norm.weight"), eps)
            x = x + swiglu_mlp(h2, m.w(p + "ffn_gate.weight"), m.w(p + "ffn_up.weight"),
                               m.w(p + "ffn_down.weight"))
        if L == 0:
            if not sel:
                return None
            x = x[sel]
        return rms_norm(x, m.w("output_norm.weight"), eps) @ m.output_weight().T
