"""The five synthetic decode workloads (Qwen3-shaped), as seeded inputs.

Shapes, distributions and hyper-parameters follow the workload list of this
project (tiny / Qwen3-8B bs1 / bs64 ragged / 128K long context / Qwen3-32B
serving step).  Every array is drawn from a keyed numpy stream
``default_rng([seed, tag, ...])``, so any slice (one sequence, one range of
positions) can be regenerated on its own, on any machine, without drawing the
rest.  Values are drawn in fp32 and rounded once to bf16 (RNE) -- the same
bf16 bits go to the GPU and to the oracle.

Recipe (seed = 1000 + config index):
* R_K[h], R_V[h]: Q factor of a QR of a 128x128 standard normal matrix
  (stream [seed, 1 or 2, h]), columns sign-fixed so diag(R) > 0, then fp32.
* kappa: fixed per config, or one U[0.8, 1.0] draw per KV head (stream
  [seed, 3, 0 or 1]), fp32.
* outlier key channels (x20): an explicit list, or round(2% of 128) = 3
  channels per KV head from a seeded permutation (stream [seed, 4, h]).
* lengths (context after the step's append): fixed, or U{lo..hi} per sequence
  (stream [seed, 5]).
* K, V, Q: standard normal fp32, generated in blocks of 256 positions
  (streams [seed, 6 / 7 / 8, seq, block]); keys get the outlier channels x20
  and the first n_sink positions x sink_scale (low-norm attention sinks);
  values are multiplied by v_scale (1 in the five workloads; large-value
  test cases only).
* physical pages: a seeded permutation of the page pool (stream [seed, 9]),
  or the identity.
"""

from dataclasses import dataclass, field, replace

import numpy as np

D = 128
PAGE = 16
BLOCK = 256


def bf16_from_f32(x):
    """fp32 -> bf16 bits, round to nearest even on the 16 dropped bits (finite
    inputs; the same bits as torch's float -> bfloat16 cast)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (out >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n_seqs: int
    hq: int
    hkv: int
    group: int
    s_sink: int
    s_keep: int
    s_flush: int
    kappa: tuple            # (kappa_k, kappa_v) floats, or None for U[0.8, 1] per head
    lengths: tuple          # ("fixed", L) | ("uniform", lo, hi) | ("list", (L0, L1, ...))
    outliers: tuple         # explicit channel tuple, or () for 3 seeded channels per head
    n_sink_tokens: int = 4
    sink_scale: float = 0.05
    shuffled_pages: bool = True
    prefill_chunks: int = 0  # fresh sequences each appending one chunk in the step
    prefill_len: int = 0
    extra_pages: int = 0     # spare pages per sequence for appends after setup
    v_scale: float = 1.0     # values drawn from N(0, v_scale^2) (1 in the five workloads)
    description: str = ""
    meta: dict = field(default_factory=dict, compare=False)

    @property
    def seed(self):
        return 1000 + self.index

    @property
    def g(self):
        return self.hq // self.hkv

    def rng(self, *key):
        return np.random.default_rng([self.seed, *key])

    # ------------------------------------------------------------ parameters
    def rotations(self):
        out = []
        for tag in (1, 2):
            mats = np.empty((self.hkv, D, D), dtype=np.float32)
            for h in range(self.hkv):
                a = self.rng(tag, h).standard_normal((D, D))
                q, r = np.linalg.qr(a)
                q = q * np.sign(np.diag(r))[None, :]
                mats[h] = q.astype(np.float32)
            out.append(mats)
        return out[0], out[1]

    def kappas(self):
        if self.kappa is None:
            kk = self.rng(3, 0).uniform(0.8, 1.0, self.hkv).astype(np.float32)
            kv = self.rng(3, 1).uniform(0.8, 1.0, self.hkv).astype(np.float32)
            return kk, kv
        return (np.full(self.hkv, self.kappa[0], np.float32),
                np.full(self.hkv, self.kappa[1], np.float32))

    def outlier_channels(self):
        if self.outliers:
            return np.tile(np.array(self.outliers, np.int64), (self.hkv, 1))
        n = int(round(0.02 * D))
        return np.stack([self.rng(4, h).permutation(D)[:n] for h in range(self.hkv)])

    def lengths_after(self):
        kind = self.lengths[0]
        if kind == "fixed":
            return np.full(self.n_seqs, self.lengths[1], np.int64)
        if kind == "uniform":
            return self.rng(5).integers(self.lengths[1], self.lengths[2] + 1, self.n_seqs).astype(np.int64)
        if kind == "mix":
            # ("mix", base, n_long, long): n_long seeded sequences at ``long``.
            out = np.full(self.n_seqs, self.lengths[1], np.int64)
            out[self.rng(5, 1).permutation(self.n_seqs)[:self.lengths[2]]] = self.lengths[3]
            return out
        return np.array(self.lengths[1], np.int64)

    # ---------------------------------------------------------- token values
    def _blocks(self, tag, seq, p0, p1, heads):
        if p1 <= p0:
            return np.zeros((0, heads, D), np.float32)
        b0, b1 = p0 // BLOCK, (p1 - 1) // BLOCK
        parts = [self.rng(tag, seq, b).standard_normal((BLOCK, heads, D), dtype=np.float32)
                 for b in range(b0, b1 + 1)]
        x = np.concatenate(parts, axis=0)
        return x[p0 - b0 * BLOCK:p1 - b0 * BLOCK]

    def keys(self, seq, p0, p1):
        """Post-RoPE keys of positions [p0, p1) of sequence ``seq``: bf16 [n, Hkv, D]."""
        x = self._blocks(6, seq, p0, p1, self.hkv)
        ch = self.outlier_channels()
        for h in range(self.hkv):
            x[:, h, ch[h]] *= np.float32(20.0)
        n_s = max(0, min(p1, self.n_sink_tokens) - p0)
        if n_s > 0:
            x[:n_s] *= np.float32(self.sink_scale)
        return bf16_from_f32(x)

    def values(self, seq, p0, p1):
        x = self._blocks(7, seq, p0, p1, self.hkv)
        if self.v_scale != 1.0:
            x *= np.float32(self.v_scale)
        return bf16_from_f32(x)

    def queries(self, seq, p0, p1):
        return bf16_from_f32(self._blocks(8, seq, p0, p1, self.hq))

    # ----------------------------------------------------------------- pages
    def page_pool(self, pages_per_seq):
        """Block table int32 [n_seqs, max_pages] over a pool of sum(pages_per_seq) pages."""
        pages_per_seq = np.asarray(pages_per_seq, np.int64)
        total = int(pages_per_seq.sum())
        perm = self.rng(9).permutation(total) if self.shuffled_pages else np.arange(total)
        width = max(1, int(pages_per_seq.max()))
        bt = np.zeros((len(pages_per_seq), width), np.int32)
        off = 0
        for i, n in enumerate(pages_per_seq):
            bt[i, :n] = perm[off:off + n]
            off += n
        return bt, total

    def scaled(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "c1_tiny": Workload(
        "c1_tiny", 1, n_seqs=1, hq=4, hkv=1, group=128, s_sink=4, s_keep=128, s_flush=16,
        kappa=(0.9, 0.9), lengths=("fixed", 1024), outliers=(3, 17, 64, 100),
        shuffled_pages=False,
        description="bs1, 1 KV head, GQA 4, context 1024, G=128, clip 0.9, windows 4/128"),
    "c2_qwen3_8b_bs1": Workload(
        "c2_qwen3_8b_bs1", 2, n_seqs=1, hq=32, hkv=8, group=128, s_sink=64, s_keep=256, s_flush=16,
        kappa=None, lengths=("fixed", 32768), outliers=(),
        description="Qwen3-8B shape, bs1, context 32768, G=128, per-head clip U[0.8,1]"),
    "c3_bs64": Workload(
        "c3_bs64", 3, n_seqs=64, hq=32, hkv=8, group=64, s_sink=64, s_keep=256, s_flush=16,
        kappa=(0.96, 0.92), lengths=("uniform", 4096, 8192), outliers=(3, 17, 64, 100),
        description="bs64, context U[4096, 8192] per sequence, G=64"),
    "c4_long_bs1": Workload(
        "c4_long_bs1", 4, n_seqs=1, hq=32, hkv=8, group=32, s_sink=64, s_keep=256, s_flush=16,
        kappa=(0.96, 0.92), lengths=("fixed", 131072), outliers=(),
        n_sink_tokens=8, sink_scale=0.02,
        description="bs1, context 131072, G=32, 8 low-norm sinks x0.02"),
    "c5_qwen3_32b_step": Workload(
        "c5_qwen3_32b_step", 5, n_seqs=256, hq=64, hkv=8, group=128, s_sink=64, s_keep=256,
        s_flush=256, kappa=(0.96, 0.92), lengths=("mix", 4096, 8, 4160), outliers=(3, 17, 64, 100),
        prefill_chunks=16, prefill_len=2048,
        description="Qwen3-32B shape serving step: 256 decode tokens (8 sequences flush 256 "
                    "tokens), plus 16 fresh 2048-token prefill chunks"),
    # The OScaR key mode's workload (OScaR notes, efficiency benchmarks: batch
    # 48 at a 4K context, G = 32): keys with outlier channels go through the
    # token scale and per-channel blocks of 32; values keep the per-token
    # min-max quantizer (clip 1); no sink, no kept window, 128-token flushes.
    "ots_bs48": Workload(
        "ots_bs48", 6, n_seqs=48, hq=32, hkv=8, group=32, s_sink=0, s_keep=0, s_flush=128,
        kappa=(1.0, 1.0), lengths=("fixed", 4096), outliers=(),
        description="OScaR key mode: bs48, context 4096, G=32, flush 128, no windows"),
}


def get(name):
    return CONFIGS[name]
