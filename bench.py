"""Benchmark: INT2 paged decode attention (OSCAR-style cache) on one MI355X.

Headline (default): bs64 decode, 32 query / 8 KV heads, head_dim 128, context
lengths U[4096, 8192] per sequence, G = 64, windows 64 / 256 (flush 16),
clip 0.96 / 0.92, shuffled pages.  One step = one decode step of every
sequence through the whole hot path: oscar_rotate_quant_append with one new
token per sequence (rotate q/k/v, flush + quantize, window placement) and then
the decode (oscar_int2_decode_partials + oscar_int2_decode_merge) over the
whole cache.  The step cycles through ``--layers`` independent layer caches
(copies of the same populated cache), so each step reads a cache that is not
resident in the 256 MB MALL, as in a multi-layer model.

Prints one JSON line.  `value` = sequences decoded per second (tokens/s) from
exactly --steps steps after --warmup warm-up steps, timed with events only
at the ends of the run (an event record between launches adds a gap to the
stream) and queued behind a spin kernel long enough to cover the host's
queueing.  `roofline` is for the decode split kernel (all cache traffic):
algorithmic bytes per launch (INT2 token-heads x (64 + 1024/G) B + BF16
window token-heads x 512 B + block-table entries x 4 B + q' in) over its
average duration, measured with HIP events around each split launch, on the
stream it runs on, in a second timed pass of the same number of steps.

Legs reported beside the headline (--legs): bs1 (Qwen3-8B shape, 32K
context; eager and replayed from a HIP graph), c1 (tiny, MALL-resident), c4
(128K context), c5 (the Qwen3-32B serving step: one append carrying 256
decode tokens and 16 fresh 2048-token chunks, then the decode of the 256
sequences, timed together), ots (the OScaR key mode: bs48 at a 4K context,
G = 32, Hadamard rotation; with the BF16 decode at the same shape), probe
(a plain HBM read kernel: the measured
read ceiling), bf16 (the BF16 paged decode on the same shapes), prefill
(chunked-prefill attention), rotation (dense vs structured rotation in the
append).  Each leg times at least --leg-steps steps; every layer copy gets an
untimed step first.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "int2_decode_c3_bs64_traffic.json")


def decode_source_hash():
    h = hashlib.sha256()
    for f in ("k_decode.hip", "decode_common.h", "device_common.h", "oscar_internal.h", "api.cpp"):
        h.update(open(os.path.join(ROOT, "ultra_bit_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def int2_token_head_bytes(w, key_mode=0):
    """Cache bytes of one INT2 token-head: K and V codes (32 B each) and
    fp16 scale/zero per group of K and of V; in the OScaR key mode the V
    groups, the token's bf16 scale and its share of its key block's
    per-channel bf16 (Delta, z) (128 x 4 B per 32 tokens)."""
    if key_mode:
        return 64 + 512 // w.group + 2 + 128 * 4 // 32
    return 64 + 1024 // w.group


def algorithmic_bytes(w, lens, key_mode=0):
    """Bytes the split launch of one decode step must move, from the cache
    format: every INT2 token-head (int2_token_head_bytes), every BF16 window
    token-head (K and V rows), one block-table entry per INT2 page, and the
    rotated queries (bf16).  The flush boundary S_quant is the closed form of
    the placement rule."""
    per_int2 = int2_token_head_bytes(w, key_mode)
    total = 0
    for L in lens:
        L = int(L)
        s_quant = w.s_sink + w.s_flush * max(0, (L - w.s_sink - w.s_keep) // w.s_flush)
        n_int2 = max(0, s_quant - w.s_sink)
        n_bf16 = min(L, w.s_sink) + max(0, L - max(s_quant, w.s_sink))
        total += w.hkv * (n_int2 * per_int2 + n_bf16 * 512) + 4 * (-(-n_int2 // 16))
    total += len(lens) * w.hq * 128 * 2           # q' (bf16) in
    return total


def bf16_bytes(w, lens):
    """Bytes a BF16 paged decode must move: K and V rows of every
    token-head, one block-table entry per page, and the queries."""
    total = 0
    for L in lens:
        L = int(L)
        total += w.hkv * L * 512 + 4 * (-(-L // 16))
    total += len(lens) * w.hq * 128 * 2
    return total


def measure_bf16(w, n_layers, steps, hold):
    """Time `steps` BF16 paged decode calls over the lengths of workload w,
    cycling through n_layers caches of seeded random bf16 pages (hold: cycles
    of the spin kernel queued ahead of the timed calls)."""
    import torch
    from ultra_bit_kv_amd import BF16PagedCache, SeqBatch

    lens = [int(L) for L in w.lengths_after()]
    n = len(lens)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    layers = []
    for _ in range(n_layers):
        bt, total = w.page_pool([-(-L // 16) for L in lens])
        c = BF16PagedCache(num_q_heads=w.hq, num_kv_heads=w.hkv, max_seqs=n,
                           max_pages_per_seq=bt.shape[1], num_pages=total, block_table=bt)
        c.pages.normal_(generator=gen)
        c.workspace_for(n)
        layers.append(c)
    batch = SeqBatch(np.arange(n), lens)
    q = torch.randn((n, w.hq, 128), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((n, w.hq, 128), dtype=torch.float32, device="cuda")
    for s in range(2 * n_layers):
        layers[s % n_layers].decode(batch, q, out)
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    torch.cuda._sleep(int(hold))
    for j in range(steps):
        evs[j][0].record()
        layers[j % n_layers].decode(batch, q, out)
        evs[j][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    byts = bf16_bytes(w, lens)
    del layers
    torch.cuda.empty_cache()
    return {"decode_ms": ms, "bytes": byts, "GBs": byts / (ms * 1e-3) / 1e9,
            "layers_cycled": n_layers}


def read_traffic(src_hash):
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != src_hash:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, lens, seconds=12.0, n_sample=4):
    """The oracle's decode step (rotate the new q/k/v rows, fp64 attention over
    the decoded cache, un-rotate) on a sample of sequences, on the host cores."""
    from threadpoolctl import threadpool_info
    from oracle import rotate, attention
    from oracle.rounding import bf16_bits_to_f64
    from tests.oscar_testlib import oracle_head
    r_k, r_v = w.rotations()
    sample = list(range(n_sample))
    heads = {}
    for i in sample:
        for h in range(w.hkv):
            heads[(i, h)] = oracle_head(w, i, h, int(lens[i]), r_k, r_v)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for i in sample:
            L = int(lens[i])
            q = w.queries(i, L - 1, L)
            kq = w.keys(i, L - 1, L)
            vq = w.values(i, L - 1, L)
            qr = rotate.rotate_heads_to_bf16(q, r_k, g=w.g)[0]
            rotate.rotate_heads_to_bf16(kq, r_k)
            rotate.rotate_heads_to_bf16(vq, r_v)
            for h in range(w.hkv):
                hc = heads[(i, h)]
                attention.decode_head(bf16_bits_to_f64(qr[h * w.g:(h + 1) * w.g]), hc.k_dec,
                                      hc.v_dec, r_v[h])
            steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": steps / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 oracle decode step (rotate the new q/k/v rows, attention over the "
                       f"decoded cache for all {w.hkv} KV heads, un-rotate) for {n_sample} of the "
                       f"{len(lens)} sequences, repeated for {el:.1f} s ({steps} sequence-steps); "
                       f"decoded caches built beforehand, untimed")}


PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 matrix peak


def prefill_flops(hq, lbs, ns):
    """Algorithmic flops of chunked-prefill attention: each query head of the
    chunk row at position P multiplies against P + 1 keys and values
    (2 * 128 flops each for q.k and for p.v)."""
    return sum(hq * 512 * (n * lb + n * (n + 1) // 2) for lb, n in zip(lbs, ns))


def measure_prefill(w, lbs, ns, reps=10):
    """oscar_int2_prefill_attn after one append of a chunk per sequence (the
    prefixes are appended first through the library); median of `reps` timed
    calls (HIP events on the stream the kernel runs on)."""
    import torch
    from ultra_bit_kv_amd import SeqBatch
    lens = [lb + n for lb, n in zip(lbs, ns)]
    cache = make_layer(w, lens, len(lens))
    if max(lbs) > 0:
        populate(cache, w, lbs)
    idx = list(range(len(lbs)))
    k = np.concatenate([w.keys(i, lbs[i], lens[i]) for i in idx])
    v = np.concatenate([w.values(i, lbs[i], lens[i]) for i in idx])
    q = np.concatenate([w.queries(i, lbs[i], lens[i]) for i in idx])
    cache.workspace_for(len(idx), sum(ns))
    q_rot, k_rot, v_rot = cache.append_tokens(idx, lbs, ns, k, v, q, want_rot=True)
    b = SeqBatch(idx, lbs, ns)
    out = cache.prefill_attn(b, q_rot, k_rot, v_rot)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, c in evs:
        a.record()
        cache.prefill_attn(b, q_rot, k_rot, v_rot, out)
        c.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(c) for a, c in evs]))
    fl = prefill_flops(w.hq, lbs, ns)
    return {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "alg_tflop": fl / 1e12}


def append_bytes(w, ns):
    """Algorithmic bytes of one append of fresh chunks (positions 0 .. n - 1
    of each sequence) with their queries: the k, v and q rows in and q' out
    (bf16), and every row's cache image out -- an INT2 row-head is K and V
    codes plus fp16 scale/zero per group, a window row-head K and V bf16."""
    per_int2 = 64 + 1024 // w.group
    total = 0
    for n in ns:
        n = int(n)
        s_quant = w.s_sink + w.s_flush * max(0, (n - w.s_sink - w.s_keep) // w.s_flush)
        n_int2 = max(0, s_quant - w.s_sink)
        n_bf16 = min(n, w.s_sink) + max(0, n - max(s_quant, w.s_sink))
        total += n * (2 * w.hkv + 2 * w.hq) * 256
        total += w.hkv * (n_int2 * per_int2 + n_bf16 * 512)
    return total


def measure_append(w, ns, rotation, reps=10):
    """oscar_rotate_quant_append of one fresh chunk per sequence with queries
    (rotation, quantization of the rows that reach INT2, window placement);
    the chunk is re-appended at position 0, which rewrites the same rows.
    Median of `reps` calls (HIP events on the calls' stream)."""
    import torch
    from ultra_bit_kv_amd import SeqBatch, as_bf16
    cache = make_layer(w, ns, len(ns), rotation=rotation)
    idx = list(range(len(ns)))
    k = as_bf16(np.concatenate([w.keys(i, 0, ns[i]) for i in idx]))
    v = as_bf16(np.concatenate([w.values(i, 0, ns[i]) for i in idx]))
    q = as_bf16(np.concatenate([w.queries(i, 0, ns[i]) for i in idx]))
    q_rot = torch.empty_like(q)
    b = SeqBatch(idx, [0] * len(ns), ns)
    cache.workspace_for(len(ns), sum(ns))
    cache.append(b, k, v, q, q_rot)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, c in evs:
        a.record()
        cache.append(b, k, v, q, q_rot)
        c.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(c) for a, c in evs]))
    nb = append_bytes(w, ns)
    gbs = nb / (ms * 1e-3) / 1e9
    return {"ms": ms, "alg_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS}}


def cpu_prefill_baseline(w, lb, n, seconds=6.0, rows=16):
    """The oracle's chunked-prefill attention (O6) for a sample of chunk rows
    of one sequence and KV head, on the host cores: algorithmic TFLOP/s."""
    from threadpoolctl import threadpool_info
    from oracle import rotate, prefill
    from oracle.rounding import bf16_bits_to_f64
    from tests.oscar_testlib import oracle_head
    r_k, r_v = w.rotations()
    hc = oracle_head(w, 0, 0, lb + n, r_k, r_v)
    qr = bf16_bits_to_f64(rotate.rotate_heads_to_bf16(w.queries(0, lb, lb + n), r_k, g=w.g))
    qr = qr[:, :w.g]
    sample = list(range(n - rows, n))   # the longest rows
    done = 0
    fl = 0
    t0 = time.perf_counter()
    while True:
        prefill.prefill_head(qr, hc, lb, r_v=r_v[0], rows=sample)
        done += 1
        fl += sum(w.g * 512 * (lb + j + 1) for j in sample)
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 oracle prefill attention of the last {rows} chunk rows (all {w.g} "
                       f"query heads of KV head 0) of a {n}-token chunk after {lb} tokens, "
                       f"repeated {done} times in {el:.1f} s; cache built beforehand, untimed")}


def copy_calibration(nbytes):
    """A plain device copy of known size (for scaling FETCH_SIZE / WRITE_SIZE)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 5}))


def int2_pages(w, L):
    """INT2 pages of a row of L tokens (closed form of the flush rule)."""
    s_quant = w.s_sink + w.s_flush * max(0, (int(L) - w.s_sink - w.s_keep) // w.s_flush)
    return -(-max(0, s_quant - w.s_sink) // 16)


def make_layer(w, lens_max, n, rotation=0, key_mode=0):
    """An empty cache sized for rows growing to lens_max (seeded page pool);
    rotation 1 / 2: the structured R = H / sqrt(128) / H P_br / sqrt(128);
    key_mode 1: the OScaR keys."""
    from ultra_bit_kv_amd import OscarKVCache
    r_k, r_v = w.rotations() if rotation == 0 else (None, None)
    kk, kv = w.kappas()
    bt, total = w.page_pool([max(1, int2_pages(w, L)) for L in lens_max])
    return OscarKVCache(num_q_heads=w.hq, num_kv_heads=w.hkv, group_size=w.group,
                        s_sink=w.s_sink, s_keep=w.s_keep, s_flush=w.s_flush, max_seqs=n,
                        max_pages_per_seq=bt.shape[1], num_pages=total, clip_k=kk, clip_v=kv,
                        r_k=r_k, r_v=r_v, block_table=bt, rotation=rotation, key_mode=key_mode)


def populate(cache, w, lens, chunk=8192, max_tokens=1 << 18):
    """Append positions [0, L) of every row through the library's append path."""
    done = [0] * len(lens)
    while True:
        idx, n_new, budget = [], [], max_tokens
        for i, L in enumerate(lens):
            k = min(chunk, int(L) - done[i], budget)
            if k > 0:
                idx.append(i)
                n_new.append(k)
                budget -= k
            if budget == 0:
                break
        if not idx:
            return
        k = np.concatenate([w.keys(i, done[i], done[i] + m) for i, m in zip(idx, n_new)])
        v = np.concatenate([w.values(i, done[i], done[i] + m) for i, m in zip(idx, n_new)])
        cache.append_tokens(idx, [done[i] for i in idx], n_new, k, v)
        for i, m in zip(idx, n_new):
            done[i] += m


CLOCK_HZ = 2.4e9   # shader clock the spin kernel counts (MI355X peak engine clock)


def pct(xs):
    """Median, p10 and p90 of a list of durations."""
    a = np.asarray(xs, np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


def hold_for(host_s):
    """Spin-kernel length (cycles) that covers `host_s` seconds of host-side
    queueing three times over (at least 5 ms)."""
    return int(max(3.0 * host_s, 5e-3) * CLOCK_HZ)


def timed_region(enqueue, n, hold_cycles, retries=2):
    """GPU time of `n` calls of enqueue(j) queued behind a spin kernel, so the
    events time the GPU's execution of the queue, not the host's submission.
    When the host took longer to queue the calls than the spin kernel held
    the GPU (the GPU then waited on the host), the same calls are timed again
    behind a longer spin.  Returns (ms per call, host seconds spent queueing,
    whether the last attempt was still host-bound)."""
    import torch
    for attempt in range(retries + 1):
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(hold_cycles))
        t_start.record()
        h0 = time.perf_counter()
        for j in range(n):
            enqueue(j)
        host = time.perf_counter() - h0
        t_end.record()
        torch.cuda.synchronize()
        bound = host > hold_cycles / CLOCK_HZ
        if not bound:
            break
        hold_cycles = hold_for(host)
    return t_start.elapsed_time(t_end) / n, host, bound


def timed_regions(enqueue, n, region, hold_cycles):
    """timed_region over n calls cut into regions of at most `region` calls
    (the HIP runtime stops accepting launches once about 50 calls with the
    decode kernels' large argument tables are queued, so a long queue behind
    the spin kernel would time the host).  Returns (ms per call, host
    seconds, host-bound in any region)."""
    tot_ms = host = 0.0
    bound = False
    for r0 in range(0, n, region):
        m = min(region, n - r0)
        ms, h, b = timed_region(lambda j: enqueue(r0 + j), m, hold_cycles)
        tot_ms += ms * m
        host += h
        bound = bound or b
    return tot_ms / n, host, bound


def measure(w, n_layers, steps, warmup, rotation=0, graph_steps=0, graph_reps=0, region=0,
            key_mode=0, split_only=False):
    """Decode steps of every row of workload w, cycling through n_layers
    copies of the populated cache (``rotation``: the cache's rotation kind).

    Every layer copy gets at least one untimed step before timing (the first
    call on a cache pays one-off host and device costs).  Pass 1 times
    exactly `steps` steps with events only at its ends (``ms_step``); pass 2
    the same number with events around the append, split and merge launches
    of each step.  With graph_steps > 0 a further `graph_steps` steps are
    captured into one HIP graph and replayed `graph_reps` times (timed as a
    whole), which removes the host's launch path from the figure.  region > 0:
    both passes time their steps in regions of at most `region` steps.
    split_only: a third pass times `steps` split launches alone, back to
    back, each layer copy in turn at the length its last step of pass 2
    left it (its cache as that step decoded it), with events only at the
    ends of each region (``split_only_ms``, ``split_only_bytes``): the
    kernel's duration without the event records of pass 2 between launches."""
    import torch
    from ultra_bit_kv_amd import SeqBatch, as_bf16

    lens0 = w.lengths_after()                 # context of the first step, per layer
    n = len(lens0)
    warm = max(warmup, n_layers)
    total_steps = warm + 2 * steps + graph_steps
    per_layer = -(-total_steps // n_layers)
    grow = [int(L) + per_layer for L in lens0]
    t_setup = time.perf_counter()

    # layer 0 is populated through the library's own append path with L0 - 1
    # tokens; the other layers are copies.  Layer step k appends position
    # L0 - 1 + k, so the first step of every layer decodes a context of L0.
    base = make_layer(w, grow, n, rotation=rotation, key_mode=key_mode)
    populate(base, w, [int(L) - 1 for L in lens0])
    layers = [base]
    for _ in range(1, n_layers):
        c = make_layer(w, grow, n, rotation=rotation, key_mode=key_mode)
        c.pages.copy_(base.pages)
        c.win.copy_(base.win)
        layers.append(c)
    torch.cuda.synchronize()

    # per-step inputs (resident in HBM before timing) and per-sequence arrays
    slots = np.arange(n, dtype=np.int32)
    steps_in = []
    first = [int(L) - 1 for L in lens0]      # position appended at a layer's first step
    kseq = [w.keys(i, p, p + per_layer) for i, p in enumerate(first)]
    vseq = [w.values(i, p, p + per_layer) for i, p in enumerate(first)]
    qseq = [w.queries(i, p, p + per_layer) for i, p in enumerate(first)]
    for k in range(per_layer):
        pos = [p + k for p in first]
        steps_in.append({
            "app": SeqBatch(slots, pos, [1] * n),
            "dec": SeqBatch(slots, [p + 1 for p in pos]),
            "k": as_bf16(np.stack([x[k] for x in kseq])),
            "v": as_bf16(np.stack([x[k] for x in vseq])),
            "q": as_bf16(np.stack([x[k] for x in qseq])),
        })
    q_rot = torch.empty((n, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((n, w.hq, 128), dtype=torch.float32, device="cuda")
    for c in layers:
        c.workspace_for(n, n)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def step(s, ev=None):
        c = layers[s % n_layers]
        d = steps_in[s // n_layers]
        if ev is not None:
            ev[0].record()
        c.append(d["app"], d["k"], d["v"], d["q"], q_rot=q_rot)
        # the decode step as its two launches, timed apart when events are
        # given: the split kernel (all cache traffic) and the log-sum-exp
        # merge / un-rotation
        if ev is not None:
            ev[1].record()
        c.decode_partials(d["dec"], q_rot)
        if ev is not None:
            ev[2].record()
        c.decode_merge(d["dec"], out)
        if ev is not None:
            ev[3].record()

    for s in range(warm):
        step(s)
    torch.cuda.synchronize()
    # host queueing time of a step, measured on the warm-up path
    h0 = time.perf_counter()
    step(warm - 1)
    host_step = time.perf_counter() - h0
    torch.cuda.synchronize()
    hold = hold_for(host_step * steps * 4)   # pass 2 also records 4 events per step
    # pass 1: the whole step, no event records between its launches (each
    # record adds a gap to the stream)
    reg = region if region > 0 else steps
    ms_step, host1, bound1 = timed_regions(lambda j: step(warm + j), steps, reg, hold)
    # pass 2: the same number of steps with events around each launch
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(steps)]
    ms_step_ev, host2, _ = timed_regions(lambda j: step(warm + steps + j, evs[j]), steps, reg, hold)
    split_only_res = {}
    if split_only:
        last = {}
        for j in range(steps):
            last[(warm + steps + j) % n_layers] = warm + steps + j
        order = sorted(last)

        def split_step(j):
            li = order[j % len(order)]
            layers[li].decode_partials(steps_in[last[li] // n_layers]["dec"], q_rot)

        ms_so, _, _ = timed_regions(split_step, steps, reg, hold)
        so_bytes = [algorithmic_bytes(w, [int(L) + last[order[j % len(order)]] // n_layers for L in lens0],
                                      key_mode) for j in range(steps)]
        split_only_res = {"split_only_ms": ms_so, "split_only_bytes": float(np.mean(so_bytes))}
    app = [a.elapsed_time(b) for a, b, c, d in evs]
    split = [b.elapsed_time(c) for a, b, c, d in evs]
    merge = [c.elapsed_time(d) for a, b, c, d in evs]
    dec = [b.elapsed_time(d) for a, b, c, d in evs]
    whole = [a.elapsed_time(d) for a, b, c, d in evs]
    # algorithmic bytes of the average split launch (lengths grow during the run)
    byts = [algorithmic_bytes(w, [int(L) + (warm + steps + j) // n_layers for L in lens0], key_mode)
            for j in range(steps)]
    res = {"w": w, "lens0": lens0, "n": n, "ms_step": ms_step, "ms_step_ev": ms_step_ev,
           "dec_ms": float(np.mean(dec)), "split_ms": float(np.mean(split)),
           "merge_ms": float(np.mean(merge)), "append_ms": float(np.mean(app)),
           "split_pct": pct(split), "step_pct": pct(whole),
           "bytes": float(np.mean(byts)), "setup_s": setup_s, "warm": warm,
           "host_ms_per_step": 1e3 * host1 / steps, "hold_ms": 1e3 * hold / CLOCK_HZ,
           "steps_per_timed_region": reg, **split_only_res,
           # pass 1 waited on the host if the host took longer to queue the
           # steps than the spin kernel held the GPU (after retries)
           "host_bound": bound1}
    if graph_steps:
        g0 = warm + 2 * steps
        for j in range(graph_steps):      # the captured steps run once eagerly first
            step(g0 + j)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(graph_steps):
                step(g0 + j)
        g.replay()                        # replays re-run the same steps: same work
        torch.cuda.synchronize()
        ms_rep, _, _ = timed_region(lambda j: g.replay(), graph_reps, hold_for(1e-3 * graph_reps))
        res["graph"] = {"steps_per_graph": graph_steps, "replays": graph_reps,
                        "ms_per_step": ms_rep / graph_steps}
        del g
    return res


def leg_summary(m, peak_probe=None):
    """The per-leg record of a measure() result."""
    w = m["w"]
    gbs = m["bytes"] / (m["split_ms"] * 1e-3) / 1e9
    out = {
        "workload": f"{w.name}: {w.description}",
        "batch": m["n"], "context_min": int(m["lens0"].min()), "context_max": int(m["lens0"].max()),
        "warmup_steps": m["warm"],
        "ms_per_step": m["ms_step"], "tokens_per_s": m["n"] / (m["ms_step"] * 1e-3),
        "step_ms_events": m["step_pct"],
        "decode_ms": m["dec_ms"], "decode_split_ms": m["split_ms"],
        "decode_split_ms_pct": m["split_pct"], "decode_merge_ms": m["merge_ms"],
        "append_ms": m["append_ms"], "ms_per_step_with_kernel_events": m["ms_step_ev"],
        "algorithmic_bytes_per_launch": m["bytes"],
        "split_GBs": gbs, "split_frac_of_peak": gbs / PEAK_HBM_GBS,
        "decode_call_GBs": m["bytes"] / (m["dec_ms"] * 1e-3) / 1e9,
        "host_ms_per_step": m["host_ms_per_step"], "gpu_hold_ms": m["hold_ms"],
        "host_bound": m["host_bound"], "steps_per_timed_region": m["steps_per_timed_region"],
    }
    if peak_probe:
        out["split_frac_of_read_probe"] = gbs / peak_probe
    if "graph" in m:
        g = m["graph"]
        out["graph"] = dict(g, tokens_per_s=m["n"] / (g["ms_per_step"] * 1e-3))
    return out


def measure_probe(nbytes=1 << 30, reps=20, chunk_bytes=10240, chunk_total=325 << 20):
    """The read probe (oscar_read_probe): a sequential sweep of `nbytes` and a
    gather of shuffled `chunk_bytes` chunks (the size of one INT2 page of the
    bs64 workload across its 8 KV heads) adding up to `chunk_total` bytes, the
    bs64 decode step's traffic; median GB/s of `reps` calls each."""
    import ctypes
    import torch
    from ultra_bit_kv_amd import lib
    from ultra_bit_kv_amd._lib import check
    L = lib()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    grid = 2048
    sink = torch.empty(4 * grid, dtype=torch.int32, device="cuda")
    n_ch = nbytes // chunk_bytes
    pick = np.random.default_rng(77).permutation(n_ch)[:chunk_total // chunk_bytes].astype(np.int32)
    ids = torch.from_numpy(pick).to("cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run(chunks):
        if chunks:
            st = L.oscar_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                    ctypes.c_void_p(ids.data_ptr()), len(pick), chunk_bytes,
                                    ctypes.c_void_p(sink.data_ptr()), grid, 4 * grid, stream)
        else:
            st = L.oscar_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes, None, 0, 0,
                                    ctypes.c_void_p(sink.data_ptr()), grid, 4 * grid, stream)
        check(st, "oscar_read_probe")

    res = {}
    for name, chunks, nb in (("sequential", False, nbytes), ("shuffled_chunks", True,
                                                            len(pick) * chunk_bytes)):
        for _ in range(3):
            run(chunks)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(5e-3 * CLOCK_HZ))
        for a, b in evs:
            a.record()
            run(chunks)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        res[name] = {"bytes": nb, "ms": ms, "GBs": nb / (ms * 1e-3) / 1e9,
                     "frac_of_peak": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    res["shuffled_chunks"]["chunk_bytes"] = chunk_bytes
    res["kernel"] = "oscar_read_probe (16-byte loads, 2048 work-groups of 256 threads)"
    del buf
    torch.cuda.empty_cache()
    return res


def measure_c5_step(w, reps):
    """The Qwen3-32B-shaped serving step as one unit: one
    oscar_rotate_quant_append carrying every decode sequence's new token (the
    sequences at the longer length cross a 256-token flush) and the fresh
    2048-token prefill chunks, then oscar_int2_decode_attn over the decode
    sequences.  The same step is repeated (re-appending the same positions
    rewrites the same rows: the same work each time)."""
    import torch
    from ultra_bit_kv_amd import SeqBatch, as_bf16
    lens = [int(x) for x in w.lengths_after()]            # decode sequences, after the step
    n_dec, n_pre, plen = len(lens), w.prefill_chunks, w.prefill_len
    t0 = time.perf_counter()
    cache = make_layer(w, lens + [plen] * n_pre, n_dec + n_pre)
    populate(cache, w, [L - 1 for L in lens] + [0] * n_pre)
    slots = list(range(n_dec + n_pre))
    before = [L - 1 for L in lens] + [0] * n_pre
    n_new = [1] * n_dec + [plen] * n_pre
    k = as_bf16(np.concatenate([w.keys(i, b, b + m) for i, b, m in zip(slots, before, n_new)]))
    v = as_bf16(np.concatenate([w.values(i, b, b + m) for i, b, m in zip(slots, before, n_new)]))
    q = as_bf16(np.concatenate([w.queries(i, b, b + m) for i, b, m in zip(slots, before, n_new)]))
    q_rot = torch.empty_like(q)
    app = SeqBatch(slots, before, n_new)
    dec = SeqBatch(list(range(n_dec)), lens)
    out = torch.empty((n_dec, w.hq, 128), dtype=torch.float32, device="cuda")
    cache.workspace_for(n_dec + n_pre, int(sum(n_new)))
    qd = q_rot[:n_dec]
    setup_s = time.perf_counter() - t0

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        cache.append(app, k, v, q, q_rot)
        if ev is not None:
            ev[1].record()
        cache.decode_partials(dec, qd)
        if ev is not None:
            ev[2].record()
        cache.decode_merge(dec, out)
        if ev is not None:
            ev[3].record()

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    ms, host, _ = timed_region(lambda j: step(), reps, hold_for(4e-3 * reps))
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(reps)]
    timed_region(lambda j: step(evs[j]), reps, hold_for(4e-3 * reps))
    app_ms = [a.elapsed_time(b) for a, b, c, d in evs]
    split = [b.elapsed_time(c) for a, b, c, d in evs]
    merge = [c.elapsed_time(d) for a, b, c, d in evs]
    byts = algorithmic_bytes(w, lens)
    gbs = byts / (float(np.mean(split)) * 1e-3) / 1e9
    n_tok = int(sum(n_new))
    return {
        "workload": f"{w.name}: {w.description}",
        "step": "one rotate_quant_append (decode tokens + prefill chunks, dense rotation) + "
                "int2_decode_partials + int2_decode_merge",
        "decode_seqs": n_dec, "prefill_chunks": n_pre, "prefill_len": plen,
        "flushing_seqs": int(sum(1 for L in lens if w.lengths[0] == "mix" and L == w.lengths[3])),
        "reps": reps, "ms_per_step": ms,
        "decode_tokens_per_s": n_dec / (ms * 1e-3),
        "tokens_per_s_incl_prefill": n_tok / (ms * 1e-3),
        "append_ms": pct(app_ms), "decode_split_ms": pct(split), "decode_merge_ms": pct(merge),
        "decode_algorithmic_bytes": byts, "decode_split_GBs": gbs,
        "decode_split_frac_of_peak": gbs / PEAK_HBM_GBS,
        "host_ms_per_step": 1e3 * host / reps, "setup_s": setup_s,
    }


LEGS = ("bs1", "c1", "c4", "c5", "ots", "probe", "bf16", "prefill", "rotation")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--config", default="c3_bs64")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated legs reported next to the headline ('' for none): "
                         + ", ".join(LEGS))
    ap.add_argument("--leg-steps", type=int, default=100,
                    help="timed steps per leg (at least --steps)")
    ap.add_argument("--bs1-layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run a device copy of this many bytes (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (the decode path shards by "
              "sequence / KV head with no exchange; multi-GPU runs are not part of it)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    from synth import get

    legs = [x for x in args.legs.split(",") if x]
    for x in legs:
        if x not in LEGS:
            sys.exit(f"bench.py: unknown leg {x!r} (legs: {', '.join(LEGS)})")
    ls = max(args.steps, args.leg_steps)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    log(f"headline {args.config}: {args.steps} steps after {args.warmup} warm-up")
    # (regions of at most 32 steps behind the spin kernel: a longer queue of
    # these launches blocks the host, see timed_regions)
    m = measure(get(args.config), args.layers, args.steps, args.warmup, region=32, split_only=True)
    w, lens0, n = m["w"], m["lens0"], m["n"]
    # the split kernel's rate from the split-only pass (events at the ends of
    # back-to-back split launches); the per-launch events of pass 2 add their
    # own gaps to each launch (decode_split_ms below)
    achieved = m["split_only_bytes"] / (m["split_only_ms"] * 1e-3) / 1e9
    src_hash = decode_source_hash()
    res = {
        "metric": "INT2 paged decode-attn tokens/s + achieved HBM GB/s vs peak (bs1, bs64)",
        "value": n / (m["ms_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2",
        "data": "synthetic (seeded; Qwen3-8B-shaped heads, no weights needed)",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "batch": n, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": 128, "group": w.group,
            "windows": [w.s_sink, w.s_keep, w.s_flush], "context_min": int(lens0.min()),
            "context_max": int(lens0.max()), "layers_cycled": args.layers,
            "step": "rotate_quant_append(1 token/seq) + int2_decode_partials + int2_decode_merge",
            "decode_ms": m["dec_ms"], "decode_split_ms": m["split_ms"],
            "decode_split_ms_pct": m["split_pct"], "step_ms_events": m["step_pct"],
            "decode_split_only_ms": m["split_only_ms"],
            "decode_merge_ms": m["merge_ms"], "append_ms": m["append_ms"],
            "ms_per_step_with_kernel_events": m["ms_step_ev"],
            "decode_call_GBs": m["bytes"] / (m["dec_ms"] * 1e-3) / 1e9,
            "host_ms_per_step": m["host_ms_per_step"], "gpu_hold_ms": m["hold_ms"],
            "host_bound": m["host_bound"], "steps_per_timed_region": m["steps_per_timed_region"],
            "decode_kernel_source": src_hash,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": read_traffic(src_hash),
            "kernel": "int2_decode_kernel", "algorithmic_bytes_per_launch": m["split_only_bytes"],
            "duration": "split-only pass: back-to-back split launches over the layer copies, "
                        "events at the region ends",
        },
        "cpu_baseline": None,
        "setup_s": m["setup_s"],
    }
    probe = None
    if "probe" in legs:
        log("read probe")
        res["read_probe"] = measure_probe()
        probe = res["read_probe"]["shuffled_chunks"]["GBs"]
        res["roofline"]["frac_of_read_probe"] = achieved / probe
    if "bs1" in legs:
        # bs1 latency (C2, 32K context): enough layer copies that the cache is
        # not MALL-resident, every copy warmed, plus the same steps replayed
        # from a HIP graph (no host launch path)
        log(f"bs1 leg: {ls} steps, {args.bs1_layers} layers")
        b = measure(get("c2_qwen3_8b_bs1"), args.bs1_layers, ls, args.warmup,
                    graph_steps=args.bs1_layers, graph_reps=20, region=16)
        res["bs1"] = leg_summary(b, probe)
        res["bs1"]["layers_cycled"] = args.bs1_layers
    if "c1" in legs:
        log("c1 leg")
        c1 = measure(get("c1_tiny"), 8, ls, args.warmup, region=16)
        res["c1"] = leg_summary(c1, probe)
        res["c1"]["layers_cycled"] = 8
        res["c1"]["note"] = "0.14 MB per call: resident in the 256 MB MALL (launch-latency bound)"
    if "c4" in legs:
        log("c4 leg")
        c4 = measure(get("c4_long_bs1"), 4, ls, args.warmup, graph_steps=4, graph_reps=20, region=16)
        res["c4"] = leg_summary(c4, probe)
        res["c4"]["layers_cycled"] = 4
    if "c5" in legs:
        log("c5 serving step")
        res["c5_step"] = measure_c5_step(get("c5_qwen3_32b_step"), reps=20)
    if "ots" in legs:
        log("ots leg")
        wo = get("ots_bs48")
        mo = measure(wo, 4, ls, args.warmup, rotation=1, region=16, key_mode=1)
        res["ots"] = leg_summary(mo, probe)
        res["ots"]["layers_cycled"] = 4
        res["ots"]["rotation"] = "H / sqrt(128)"
        res["ots"]["int2_bytes_per_token_head"] = int2_token_head_bytes(wo, 1)
        bfo = measure_bf16(wo, 2, min(ls, 100), hold_for(2e-3 * min(ls, 100)))
        res["ots"]["bf16_decode_ms"] = bfo["decode_ms"]
        res["ots"]["bf16_GBs"] = bfo["GBs"]
        res["ots"]["int2_speedup_vs_bf16"] = bfo["decode_ms"] / res["ots"]["decode_ms"]
        res["ots"]["bytes_ratio_vs_bf16"] = bfo["bytes"] / mo["bytes"]
    if "bf16" in legs:
        log("bf16 comparison")
        # the uncompressed comparison point on the same shapes and lengths
        bf = measure_bf16(get(args.config), 2, min(ls, 100), hold_for(2e-3 * min(ls, 100)))
        res["bf16_compare"] = {
            "kernel": "oscar_bf16_paged_decode_attn (split + merge), same lengths",
            "bs64_decode_ms": bf["decode_ms"], "bs64_GBs": bf["GBs"],
            "bs64_bytes_per_call": bf["bytes"],
            "bs64_int2_speedup": bf["decode_ms"] / m["dec_ms"],
            "bs64_int2_bytes_ratio": bf["bytes"] / m["bytes"],
        }
        if "bs1" in res:
            bf1 = measure_bf16(get("c2_qwen3_8b_bs1"), 8, min(ls, 100),
                               hold_for(2e-3 * min(ls, 100)))
            res["bf16_compare"].update({
                "bs1_decode_ms": bf1["decode_ms"], "bs1_GBs": bf1["GBs"],
                "bs1_int2_speedup": bf1["decode_ms"] / res["bs1"]["decode_ms"],
            })
    if "prefill" in legs:
        log("prefill legs")
        # chunked-prefill attention: the Qwen3-32B step's 16 fresh 2048-token
        # chunks, and a 2048-token chunk after a 30720-token prefix (Qwen3-8B heads)
        w5 = get("c5_qwen3_32b_step")
        w5 = w5.scaled(n_seqs=w5.prefill_chunks,
                       lengths=("list", tuple([w5.prefill_len] * w5.prefill_chunks)))
        p5 = measure_prefill(w5, [0] * w5.prefill_chunks, [w5.prefill_len] * w5.prefill_chunks)
        w2 = get("c2_qwen3_8b_bs1").scaled(lengths=("list", (32768,)))
        p2 = measure_prefill(w2, [30720], [2048])
        res["prefill"] = {
            "kernel": "prefill_attn_kernel (oscar_int2_prefill_attn)",
            "c5_chunks": {"workload": "16 fresh 2048-token chunks, 64 / 8 heads, G=128, windows "
                                      "64/256/256", **p5,
                          "roofline": {"bound": "mfma", "achieved": p5["tflops"],
                                       "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                                       "frac": p5["tflops"] / PEAK_F16_MFMA_TFLOPS}},
            "chunk_after_prefix": {"workload": "2048-token chunk after 30720 tokens, 32 / 8 "
                                               "heads, G=128, windows 64/256/16", **p2,
                                   "roofline": {"bound": "mfma", "achieved": p2["tflops"],
                                                "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                                                "frac": p2["tflops"] / PEAK_F16_MFMA_TFLOPS}},
        }
        if not args.no_cpu_baseline:
            res["prefill"]["cpu_baseline"] = cpu_prefill_baseline(w5, 0, w5.prefill_len)
    if "rotation" in legs:
        log("append rotation modes")
        # the Qwen3-32B step's append (16 fresh 2048-token chunks, 64 / 8
        # heads) with the dense per-head rotation and the structured
        # R = H P_br / sqrt(128) (fast Walsh-Hadamard transform)
        w5 = get("c5_qwen3_32b_step")
        ns5 = [w5.prefill_len] * w5.prefill_chunks
        w5 = w5.scaled(n_seqs=len(ns5), lengths=("list", tuple(ns5)))
        res["append_rotation_modes"] = {
            "call": "oscar_rotate_quant_append (rotation + quantization + placement)",
            "workload": "16 fresh 2048-token chunks with queries, 64 / 8 heads, G=128, "
                        "windows 64/256/256",
            "dense": measure_append(w5, ns5, 0),
            "hadamard_bitrev": measure_append(w5, ns5, 2),
        }
        # the decode step of the headline workload with the structured rotation
        # (the merge generates R^T instead of reading R_V)
        hs = measure(w, args.layers, max(20, args.steps // 4), args.warmup, rotation=2)
        res["append_rotation_modes"]["decode_step_hadamard_bitrev"] = {
            "workload": w.name, "steps": max(20, args.steps // 4), "ms_per_step": hs["ms_step"],
            "decode_split_ms": hs["split_ms"], "decode_merge_ms": hs["merge_ms"],
            "append_ms": hs["append_ms"],
        }
    if not args.no_cpu_baseline:
        log("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(w, lens0, seconds=args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
