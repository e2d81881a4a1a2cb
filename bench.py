"""Benchmark of the quantized MoE expert FFN on one MI355X.

Step = one pass of the whole hot path over one batch: for each of the 43 MoE
layers of one GPU's share of the DS4.1 verify step (128 local experts of 256,
8 columns, half of the shared expert's intermediate axis): quantise x, shared
gate/up pair + SwiGLU, quantise, shared down (column-range slice), route
(select + weights + owner mask + grouping), grouped gate/up + SwiGLU,
quantise h, grouped down, combine.  Inputs are resident in HBM; the step is
captured once as a HIP graph and replayed.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value     effective HBM GB/s of the step (algorithmic bytes / step time)
  roofline  the dominant kernel (grouped gate/up + SwiGLU): algorithmic bytes
            per launch / mean launch time from HIP events, against 8 TB/s
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  sweep     the routed layer (256 experts, top-8) at 1, 2, 4, 5, 8 columns
  wide      the same layer at 32..1024 columns: grouped products on the int8
            matrix cores against the grouped MMVQ in passes of 8 columns
  q4_sweep  the routed layer of the sweep with 4-bit expert weights (18-byte
            blocks) at 1, 2, 4, 5, 8 columns
  codec     the 8-bit block exchange codec on prefill partials of 4096 values
            a row (a 1K-row band and an 8K-row one): encode, and the
            rank-order decode-sum of 2 and 8 ranks' blocks
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-wide", action="store_true",
                    help="skip the wide-batch (32..1024 columns) measurement")
    ap.add_argument("--no-codec", action="store_true",
                    help="skip the 8-bit exchange codec measurement")
    ap.add_argument("--no-q4", action="store_true",
                    help="skip the 4-bit expert-weight sweep")
    ap.add_argument("--sweep-cols", default="",
                    help="comma-separated column counts of the sweep (default 1,2,4,5,8)")
    ap.add_argument("--only-sweep", action="store_true",
                    help="run the column sweep alone (profiling runs); the JSON line then "
                         "carries the sweep only")
    ap.add_argument("--cpu-procs", type=int, default=min(16, os.cpu_count() or 1),
                    help="processes of the multi-process oracle leg (the host's CPU share; 1 = none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate budget of the oracle sample")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="after the step, copy 512 MiB device to device once: the known-size "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload construction
# ---------------------------------------------------------------------------

class Bank:
    """Routed experts of L layers x E local experts, plus optional shared
    expert (full matrices per layer), filled with synthetic Q8_0 blocks."""

    def __init__(self, moeq8, torch, layers, n_local, hidden, inter, seed, shared_inter=0, layer0=0):
        self.layers, self.n_local, self.hidden, self.inter = layers, n_local, hidden, inter
        rb_h = hidden // 32 * 34
        rb_i = inter // 32 * 34
        self.expert_gu = inter * rb_h
        self.expert_d = hidden * rb_i
        dev = "cuda"
        # a layer's gate, up and down banks are adjacent (one region for a
        # streaming read of any leading part)
        ng, nd = n_local * self.expert_gu, n_local * self.expert_d
        self.w = torch.empty((layers, 2 * ng + nd), dtype=torch.uint8, device=dev)
        self.gate = self.w[:, :ng]
        self.up = self.w[:, ng:2 * ng]
        self.down = self.w[:, 2 * ng:]
        for t, m, blocks in ((self.gate, 0, inter * hidden // 32), (self.up, 1, inter * hidden // 32),
                             (self.down, 2, hidden * inter // 32)):
            for l in range(layers):
                moeq8.synth_q8_0_fill(t[l], n_local, blocks, n_local, seed, layer0 + l, 0, m)
        self.shared_inter = shared_inter
        if shared_inter:
            self.sgate = torch.empty((layers, shared_inter * rb_h), dtype=torch.uint8, device=dev)
            self.sup = torch.empty_like(self.sgate)
            self.sdown = torch.empty((layers, hidden * (shared_inter // 32 * 34)), dtype=torch.uint8,
                                     device=dev)
            for t, m, blocks in ((self.sgate, 3, shared_inter * hidden // 32),
                                 (self.sup, 4, shared_inter * hidden // 32),
                                 (self.sdown, 5, hidden * shared_inter // 32)):
                moeq8.synth_q8_0_fill(t, layers, blocks, 1, seed, 0, 0, m)

    packed = False

    def pack_weights(self, moeq8, torch):
        """Repack every layer's weights into the packed layouts the fused
        launches read, in place through one layer-sized buffer: routed (and
        shared) gate and up in the 64-chunk layout, down in the round-major
        four-row one."""
        jobs = [((self.gate, self.up), moeq8.q8_0_pack64_rows, self.n_local * self.inter, self.hidden),
                ((self.down,), moeq8.q8_0_pack64_rounds, self.n_local * self.hidden, self.inter)]
        if self.shared_inter:
            jobs += [((self.sgate, self.sup), moeq8.q8_0_pack64_rows, self.shared_inter, self.hidden),
                     ((self.sdown,), moeq8.q8_0_pack64_rounds, self.hidden, self.shared_inter)]
        for banks, pack, rows, k in jobs:
            tmp = torch.empty_like(banks[0][0])
            for bank in banks:
                for l in range(self.layers):
                    pack(bank[l], rows, k, out=tmp)
                    bank[l].copy_(tmp)
            del tmp
        self.packed = True

    def experts(self, ml, l):
        return ml.RoutedExperts(self.gate[l], self.up[l], self.down[l], self.n_local, self.hidden,
                                self.inter, packed=self.packed)

    def shared(self, ml, l, share_rows, share_index=0):
        if not self.shared_inter:
            return None
        rb_h = self.hidden // 32 * 34
        return ml.SharedExpertShare(self.sgate[l].view(self.shared_inter, rb_h),
                                    self.sup[l].view(self.shared_inter, rb_h),
                                    self.sdown[l].view(self.hidden, self.shared_inter // 32 * 34),
                                    self.hidden, self.shared_inter, share_index * share_rows, share_rows,
                                    packed=self.packed)


def layer_inputs(torch, workloads, seed, layers, cols, hidden, n_expert):
    xs, lgs, bs = [], [], []
    for l in range(layers):
        xs.append(torch.from_numpy(workloads.activations(seed, cols, hidden, layer=l)).cuda())
        lgs.append(torch.from_numpy(workloads.router_logits(seed, cols, n_expert, layer=l)).cuda())
        bs.append(torch.from_numpy(workloads.router_bias(seed, n_expert, layer=l)).cuda())
    return xs, lgs, bs


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_grouped_gate_up_ep_share_l43_e128_c8.json")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs, or None when the kernel's sources changed since
    the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def capture(torch, fn):
    """Capture fn (already run once eagerly) as a graph on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph_each(torch, fn, per_graph, reps):
    """Mean ms of one call of fn, from a graph of per_graph calls replayed reps
    times (short launches: one graph replay per call would time the replay)."""
    def many():
        for _ in range(per_graph):
            fn()
    return time_graph(torch, many, reps) / per_graph


def time_graph(torch, fn, reps):
    """Mean ms of one replay of a graph of fn."""
    fn()
    torch.cuda.synchronize()
    g = capture(torch, fn)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# ---------------------------------------------------------------------------
# algorithmic bytes
# ---------------------------------------------------------------------------

def gate_up_launch_bytes(n_active, n_valid, cols, hidden, inter):
    """Per grouped gate/up launch: both matrices of every active expert once,
    the q8_1 x rows once, the h rows written."""
    return n_active * 2 * inter * (hidden // 32 * 34) + cols * (hidden // 32 * 36) + n_valid * inter * 4


def down_launch_bytes(n_active, n_valid, hidden, inter):
    """Per grouped down launch: every active expert's down matrix once, the fp32
    h rows once (quantised to q8_1 inside the launch), the y rows written."""
    return n_active * hidden * (inter // 32 * 34) + n_valid * inter * 4 + n_valid * hidden * 4


def shared_gate_up_bytes(cols, hidden, rows):
    """The shared expert's rows inside the gate/up launch: both matrices' rows,
    hs written (xq is already counted once for the launch)."""
    return 2 * rows * (hidden // 32 * 34) + cols * rows * 4


def shared_down_bytes(cols, hidden, rows):
    """The shared down slice inside the down launch: the slice of every row,
    the fp32 hs rows read, ys written."""
    return hidden * (rows // 32 * 34) + cols * rows * 4 + cols * hidden * 4


def layer_bytes(n_active, n_valid, cols, hidden, inter, topk, shared_rows):
    """Algorithmic bytes of one layer: every tensor written once by its producer
    and read once per consumer (weights of the active experts once)."""
    b = cols * hidden * 4 + cols * (hidden // 32 * 36)               # x read, xq written
    b += gate_up_launch_bytes(n_active, n_valid, cols, hidden, inter)
    b += down_launch_bytes(n_active, n_valid, hidden, inter)         # h read there (q8_1 in LDS)
    b += n_valid * hidden * 4 + 2 * cols * topk * 8 + cols * hidden * 4  # y read, ids/w, out
    b += cols * 256 * 4 * 2                                           # logits read (n_expert 256), bias
    if shared_rows:
        b += shared_gate_up_bytes(cols, hidden, shared_rows)         # pair weights, hs written
        b += shared_down_bytes(cols, hidden, shared_rows)            # slice, hs read, ys written
        b += cols * hidden * 4                                        # ys read by the combine
    return b


# ---------------------------------------------------------------------------
# CPU baseline (oracle, bounded sample)
# ---------------------------------------------------------------------------

def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_layer_work(oracle, workloads, cfg, share_rows, l, mats, shared_mats, own):
    """The oracle on layer l, as the single-thread leg runs it: the routed
    layer (q8_1 of x, routing, each route's expert FFN, the weighted combine)
    and the shared expert's share."""
    seed, hidden, topk, n_exp, cols = cfg["seed"], cfg["hidden"], cfg["topk"], cfg["experts"], cfg["cols"][0]
    x = workloads.activations(seed, cols, hidden, layer=l)
    lg = workloads.router_logits(seed, cols, n_exp, layer=l)
    bias = workloads.router_bias(seed, n_exp, layer=l)
    r = oracle.moe_layer(x, lg, bias, own, lambda e: mats[(l, e)], topk)
    sg, su, sd = shared_mats[l]
    h, _, _ = oracle.glu_pair(sg, su, r["xq"])
    hq = oracle.quantize_q8_1(h.astype(np.float32))
    oracle.mmvq(sd[:, :share_rows // 32], hq)


def _cpu_worker(rank, nproc, cfg, share_rows, root, start_evt, barrier, results):
    """One process of the multi-process oracle leg: waits until the GPU part
    is done, draws the inputs of its contiguous share of the layers, meets the
    others at a barrier, then runs the oracle on its layers."""
    import sys as _sys
    import time as _time
    if root not in _sys.path:
        _sys.path.insert(0, root)
    import oracle
    import workloads
    if not start_evt.wait(3600):
        return
    try:
        _cpu_worker_body(rank, nproc, cfg, share_rows, barrier, results, oracle, workloads, _time)
    except Exception as exc:                           # reported to the parent, never left hanging
        results.put((rank, None, None, f"{type(exc).__name__}: {exc}"))


def _cpu_worker_body(rank, nproc, cfg, share_rows, barrier, results, oracle, workloads, _time):
    seed, hidden, inter, topk = cfg["seed"], cfg["hidden"], cfg["inter"], cfg["topk"]
    cols, L, n_exp = cfg["cols"][0], cfg["layers"], cfg["experts"]
    own = workloads.owner_slots(n_exp, cfg["local_experts"])
    mine = list(range(rank * L // nproc, (rank + 1) * L // nproc))
    mats, shared_mats = {}, {}
    for l in mine:
        lg = workloads.router_logits(seed, cols, n_exp, layer=l)
        ids, _, _ = oracle.route_topk(lg, workloads.router_bias(seed, n_exp, layer=l), own, topk)
        for e in (int(v) for v in ids.reshape(-1) if v >= 0):
            if (l, e) not in mats:
                mats[(l, e)] = tuple(workloads.synth_q8_0_matrix(seed, l, e, m, r_, k_)
                                     for m, r_, k_ in ((0, inter, hidden), (1, inter, hidden), (2, hidden, inter)))
        if l not in shared_mats:
            shared_mats[l] = (workloads.synth_q8_0_matrix(seed, l, 0, 3, cfg["shared_inter"], hidden, 0, share_rows),
                              workloads.synth_q8_0_matrix(seed, l, 0, 4, cfg["shared_inter"], hidden, 0, share_rows),
                              workloads.synth_q8_0_matrix(seed, l, 0, 5, hidden, cfg["shared_inter"]))
    barrier.wait(600)
    t0 = _time.perf_counter()
    for l in mine:
        _cpu_layer_work(oracle, workloads, cfg, share_rows, l, mats, shared_mats, own)
    t1 = _time.perf_counter()
    results.put((rank, t0, t1, len(mine)))


class CpuPool:
    """The multi-process oracle leg's processes, started before the GPU is
    touched (spawned children of a process that has not initialised the GPU)
    and idle until run() releases them after the GPU part."""

    def __init__(self, nproc, cfg, share_rows):
        import multiprocessing as mp
        ctx = mp.get_context("spawn")
        self.nproc, self.cfg, self.share_rows = nproc, cfg, share_rows
        self.start_evt = ctx.Event()
        self.barrier = ctx.Barrier(nproc)
        self.results = ctx.Queue()
        self.procs = [ctx.Process(target=_cpu_worker, args=(r, nproc, cfg, share_rows, ROOT, self.start_evt,
                                                             self.barrier, self.results), daemon=True)
                      for r in range(nproc)]
        # one thread a process (the children read these when numpy loads)
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        os.environ.update({k: "1" for k in saved})
        try:
            for p in self.procs:
                p.start()
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def run(self, workloads):
        """All layers of the workload over the processes; throughput over the
        span from the first process's start to the last one's end."""
        self.start_evt.set()
        got = [self.results.get(timeout=900) for _ in range(self.nproc)]
        for p in self.procs:
            p.join(timeout=60)
        bad = [g for g in got if g[1] is None]
        if bad:
            raise RuntimeError(f"multi-process oracle leg failed: {bad[0][3]}")
        span = max(g[2] for g in got) - min(g[1] for g in got)
        return span

    def close(self):
        self.start_evt.set()
        for p in self.procs:
            if p.is_alive():
                p.terminate()


def cpu_baseline(workloads, cfg, budget_s, share_rows):
    import oracle
    seed, hidden, inter, topk = cfg["seed"], cfg["hidden"], cfg["inter"], cfg["topk"]
    cols = cfg["cols"][0]
    n_exp, n_local = cfg["experts"], cfg["local_experts"]
    own = workloads.owner_slots(n_exp, n_local)
    total_bytes, total_t, layers_done = 0, 0.0, 0
    for l in range(cfg["layers"]):
        x = workloads.activations(seed, cols, hidden, layer=l)
        lg = workloads.router_logits(seed, cols, n_exp, layer=l)
        bias = workloads.router_bias(seed, n_exp, layer=l)
        ids, _, _ = oracle.route_topk(lg, bias, own, topk)
        used = sorted(set(int(e) for e in ids.reshape(-1) if e >= 0))
        mats = {e: tuple(workloads.synth_q8_0_matrix(seed, l, e, m, r, k)
                         for m, r, k in ((0, inter, hidden), (1, inter, hidden), (2, hidden, inter)))
                for e in used}
        sg = workloads.synth_q8_0_matrix(seed, l, 0, 3, cfg["shared_inter"], hidden, 0, share_rows)
        su = workloads.synth_q8_0_matrix(seed, l, 0, 4, cfg["shared_inter"], hidden, 0, share_rows)
        sd = workloads.synth_q8_0_matrix(seed, l, 0, 5, hidden, cfg["shared_inter"])
        t0 = time.perf_counter()
        r = oracle.moe_layer(x, lg, bias, own, lambda e: mats[e], topk)
        h, _, _ = oracle.glu_pair(sg, su, r["xq"])
        hq = oracle.quantize_q8_1(h.astype(np.float32))
        oracle.mmvq(sd[:, :share_rows // 32], hq)
        total_t += time.perf_counter() - t0
        n_valid = int((ids >= 0).sum())
        total_bytes += layer_bytes(len(used), n_valid, cols, hidden, inter, topk, share_rows)
        layers_done += 1
        if total_t >= budget_s:
            break
    return {"value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": f"{layers_done} of {cfg['layers']} layers of {cfg['name']} (numpy oracle, "
                      f"unfused per-route loop, single thread); {layers_done / total_t:.3f} layers/s"}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU sharding of the "
                                   "expert FFN is not built (one process per GPU would each run this "
                                   "step on its own expert share)", "n_gpus": args.gpus}))
        sys.exit(2)
    import workloads
    pool = None
    if not args.no_cpu_baseline and not args.only_sweep and args.cpu_procs > 1:
        c5 = dict(workloads.CONFIGS["ep_share_l43_e128_c8"], name="ep_share_l43_e128_c8")
        # the processes start before anything touches the GPU
        pool = CpuPool(args.cpu_procs, c5, c5["shared_inter"] // c5["shared_share"])
    try:
        _main_gpu(args, workloads, pool)
    finally:
        if pool is not None:
            pool.close()


def _main_gpu(args, workloads, pool):
    import torch

    import quantized_moe_expert_q8_amd as moeq8
    from quantized_moe_expert_q8_amd import moe_layer as ml

    torch.cuda.init()
    if args.only_sweep:
        rec = sweep(torch, workloads, moeq8, ml, args)
        if args.pmc_copy:
            pmc_reference_copy(torch)
        print(json.dumps({"metric": "routed-expert MMVQ column sweep (profiling run)", "sweep": rec}),
              flush=True)
        return
    cfg = dict(workloads.CONFIGS["ep_share_l43_e128_c8"], name="ep_share_l43_e128_c8")
    L, n_local, n_exp = cfg["layers"], cfg["local_experts"], cfg["experts"]
    hidden, inter, topk, seed, cols = cfg["hidden"], cfg["inter"], cfg["topk"], cfg["seed"], cfg["cols"][0]
    share_rows = cfg["shared_inter"] // cfg["shared_share"]

    t0 = time.perf_counter()
    bank = Bank(moeq8, torch, L, n_local, hidden, inter, seed, cfg["shared_inter"])
    bank.pack_weights(moeq8, torch)
    xs, lgs, bs = layer_inputs(torch, workloads, seed, L, cols, hidden, n_exp)
    owner = torch.from_numpy(workloads.owner_slots(n_exp, n_local)).cuda()
    side = torch.cuda.Stream()
    wss = [ml.Workspace(cols, hidden, inter, topk, share_rows, "cuda", side_stream=side) for _ in range(L)]
    torch.cuda.synchronize()
    resident = sum(t.numel() for t in (bank.gate, bank.up, bank.down, bank.sgate, bank.sup, bank.sdown))
    log(f"setup {time.perf_counter() - t0:.1f}s, resident weights {resident / 1e9:.2f} GB")

    experts = [bank.experts(ml, l) for l in range(L)]
    shared = [bank.shared(ml, l, share_rows) for l in range(L)]

    def step():
        for l in range(L):
            ml.forward(xs[l], lgs[l], bs[l], owner, n_local, experts[l], shared[l], wss[l],
                       add_shared=True)

    # eager warm-up, then capture the step as one graph
    step()
    torch.cuda.synchronize()
    # routing statistics of every layer (measurement input: active experts)
    n_active, n_valid = [], []
    for l in range(L):
        words = wss[l].grouping.cpu().numpy().view(np.int32)
        n_active.append(int(words[0]))
        n_valid.append(int(words[1]))
    step_bytes = sum(layer_bytes(n_active[l], n_valid[l], cols, hidden, inter, topk, share_rows)
                     for l in range(L))
    weight_bytes = sum(n_active[l] * ml.expert_bytes(hidden, inter) + ml.shared_share_bytes(hidden, share_rows)
                       for l in range(L))
    log(f"active local experts per layer: mean {np.mean(n_active):.1f} (min {min(n_active)}, "
        f"max {max(n_active)}); step bytes {step_bytes / 1e9:.3f} GB (weights {weight_bytes / 1e9:.3f} GB)")

    g = capture(torch, step)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    # the spread of single steps (each replay bracketed by its own events;
    # not part of the timed region above)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b in step_ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"graph: {ms_per_step:.3f} ms/step ({wall / args.steps * 1e3:.3f} ms wall), "
        f"{value:.1f} GB/s, {L / ms_per_step * 1e3:.0f} layers/s")

    # eager step (host launch overhead included), for reference
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(3, args.steps // 5)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / reps

    # the dominant kernel: a graph of its 43 launches on this step's inputs,
    # timed with HIP events on the stream it runs on
    # the launches exactly as the step issues them (routed experts plus the
    # shared expert's rows as extra work items)
    rb_h = hidden // 32 * 34

    def gate_up_only():
        for l in range(L):
            w, sh = wss[l], shared[l]
            moeq8.moe_grouped_mmvq_ex(
                moeq8.GATE_UP_SWIGLU_P64, experts[l].gate, experts[l].up, w.xq, w.grouping, n=inter,
                k=hidden, n_local_expert=n_local, ncols=cols, topk=topk, out=w.h,
                shared={"a": sh.gate, "b": sh.up, "row_stride": rb_h, "n": sh.rows, "k": hidden,
                        "k_block_offset": 0, "offset_bytes": sh.gate_offset(), "out": w.hs})

    def down_only():
        for l in range(L):
            w, sh = wss[l], shared[l]
            kb = sh.down_block_offset()
            moeq8.moe_grouped_mmvq_ex(
                moeq8.DOWN_F32_ACT_P64, experts[l].down, None, w.h.view(cols * topk, inter), w.grouping,
                n=hidden, k=inter, n_local_expert=n_local, ncols=cols, topk=topk, out=w.y,
                shared={"a": sh.down, "row_stride": moeq8.ops.ROUND_BYTES, "n": hidden,
                        "k": sh.rows, "k_block_offset": 0,
                        "offset_bytes": kb // 32 * hidden * moeq8.ops.ROUND_BYTES,
                        "out": w.ys, "act": w.hs})

    # the two small launches of the layer, each alone in a graph of 43 (a
    # kernel trace lengthens such short kernels; the graphs time them as the
    # step issues them)
    def prologue_only():
        for l in range(L):
            w = wss[l]
            moeq8.moe_route_topk_quantize(xs[l], lgs[l], topk, bias=bs[l], owner_slot=owner,
                                          n_local_expert=n_local, xq=w.xq, ids=w.ids, weights=w.weights,
                                          grouping=w.grouping)

    def combine_only():
        for l in range(L):
            w = wss[l]
            moeq8.moe_combine(w.y, w.ids, w.weights, out=w.out, shared=w.ys)

    gu_us = time_graph(torch, gate_up_only, args.steps) / L * 1e3
    dn_us = time_graph(torch, down_only, args.steps) / L * 1e3
    pro_us = time_graph(torch, prologue_only, args.steps) / L * 1e3
    cmb_us = time_graph(torch, combine_only, args.steps) / L * 1e3
    gu_bytes = float(np.mean([gate_up_launch_bytes(n_active[l], n_valid[l], cols, hidden, inter)
                              for l in range(L)])) + shared_gate_up_bytes(cols, hidden, share_rows)
    dn_bytes = float(np.mean([down_launch_bytes(n_active[l], n_valid[l], hidden, inter)
                              for l in range(L)])) + shared_down_bytes(cols, hidden, share_rows)
    gu_gbps = gu_bytes / (gu_us * 1e-6) / 1e9
    dn_gbps = dn_bytes / (dn_us * 1e-6) / 1e9

    # the achievable ceiling: a plain coalesced streaming read of as many bytes
    # per launch from the same weight bank (layer l's gate matrices), 43
    # launches in a graph as the gate/up ones
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    read_bytes = [int(gate_up_launch_bytes(n_active[l], n_valid[l], cols, hidden, inter)
                      + shared_gate_up_bytes(cols, hidden, share_rows)) // 16 * 16 for l in range(L)]

    def stream_only():
        for l in range(L):
            moeq8.stream_read(bank.gate[l], read_bytes[l], sink)

    st_us = time_graph(torch, stream_only, args.steps) / L * 1e3
    st_gbps = float(np.mean(read_bytes)) / (st_us * 1e-6) / 1e9
    log(f"eager {eager_ms:.3f} ms/step; grouped gate/up {gu_us:.2f} us/launch {gu_gbps:.1f} GB/s; "
        f"grouped down {dn_us:.2f} us/launch {dn_gbps:.1f} GB/s; streaming-read ceiling "
        f"{st_us:.2f} us/launch {st_gbps:.1f} GB/s; step p10/p50/p90 "
        f"{np.percentile(step_ms, 10):.3f}/{np.median(step_ms):.3f}/{np.percentile(step_ms, 90):.3f} ms")

    result = {
        "metric": "Q8_0 MoE MMVQ effective HBM GB/s (% of peak) + MoE layers/s at 1-8 cols",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "layers": L, "experts": n_exp, "local_experts": n_local,
                   "cols": cols, "hidden": hidden, "inter": inter, "topk": topk,
                   "shared_rows": share_rows, "seed": seed, "graph": True},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "layers_per_s": round(L / ms_per_step * 1e3, 1),
        "eager_ms_per_step": round(eager_ms, 4),
        "step_bytes": step_bytes,
        "weight_bytes": weight_bytes,
        "active_experts_mean": round(float(np.mean(n_active)), 2),
        "roofline": {"bound": "hbm", "kernel": "k_mmvq grouped gate/up + SwiGLU on the 64-chunk packed layout (routed experts "
                               "and the shared expert's rows in one launch)",
                     "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "scaled by a 512 MiB copy)",
                     "mean_launch_us": round(gu_us, 2), "bytes_per_launch": int(gu_bytes),
                     "ceiling": {"what": "plain coalesced nontemporal streaming read of the same "
                                         "bytes per launch from the same weight bank, 43 launches "
                                         "in a graph",
                                 "gbps": round(st_gbps, 1), "mean_launch_us": round(st_us, 2),
                                 "frac_of_ceiling": round(gu_gbps / st_gbps, 4)}},
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, 10)), 4),
                                round(float(np.median(step_ms)), 4),
                                round(float(np.percentile(step_ms, 90)), 4)],
        "grouped_down": {"mean_launch_us": round(dn_us, 2), "gbps": round(dn_gbps, 1),
                         "bytes_per_launch": int(dn_bytes)},
        # per layer: each launch kind alone in a graph of 43, against the
        # step's time per layer (the rest is the dependent launches' gaps)
        "layer_breakdown_us": {"prologue": round(pro_us, 2), "gate_up": round(gu_us, 2),
                               "down": round(dn_us, 2), "combine": round(cmb_us, 2),
                               "sum": round(pro_us + gu_us + dn_us + cmb_us, 2),
                               "step_per_layer": round(ms_per_step / L * 1e3, 2)},
        # the routed-expert MMVQ as a whole: both grouped launches' bytes over
        # their summed times (the shared expert's rows ride in both launches)
        "gate_up_plus_down": {"gbps": round((gu_bytes + dn_bytes) / ((gu_us + dn_us) * 1e-6) / 1e9, 1),
                              "frac_of_peak": round((gu_bytes + dn_bytes) / ((gu_us + dn_us) * 1e-6) / 1e9
                                                    / HBM_PEAK_GBPS, 4)},
    }

    if args.pmc_copy:
        pmc_reference_copy(torch)

    # release the big bank before the sweep
    del g, bank, experts, shared, wss
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if not args.no_sweep:
        result["sweep"] = sweep(torch, workloads, moeq8, ml, args)
    if not args.no_wide:
        result["wide"] = wide_sweep(torch, workloads, moeq8, ml, args)
    if not args.no_codec:
        result["codec"] = codec_bench(torch, workloads, moeq8, args)
    if not args.no_q4:
        result["q4_sweep"] = q4_sweep(torch, workloads, moeq8, ml, args)

    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(workloads, cfg, args.cpu_seconds, share_rows)
        log(f"cpu baseline {time.perf_counter() - t0:.1f}s: {result['cpu_baseline']}")
        if pool is not None:
            t0 = time.perf_counter()
            span = pool.run(workloads)
            all_bytes = step_bytes                     # every layer of the step, as the GPU's value
            leg = {"value": round(all_bytes / span / 1e9, 4), "unit": "GB/s", "cores": pool.nproc,
                   "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
                   "sample": f"all {L} layers of {cfg['name']} in contiguous shares over {pool.nproc} "
                             f"processes (numpy oracle, one thread each; the span of the compute from the "
                             f"first start to the last end after a barrier); {L / span:.3f} layers/s"}
            result["cpu_baseline"] = {**result["cpu_baseline"], "single_thread": dict(result["cpu_baseline"]),
                                      "multi_process": leg}
            log(f"cpu baseline, {pool.nproc} processes, {time.perf_counter() - t0:.1f}s: {leg}")
    print(json.dumps(result), flush=True)


ROTATION_BYTES = 1.0e9      # bytes every timed sweep graph reads per replay, at least


def best_ceiling(torch, moeq8, regions, reps, sink):
    """The streaming-read ceiling of a graph of launches: regions is one
    (tensor, bytes) per launch; each shape of the plain read is timed as a
    graph of one read per region, and the fastest mean per launch (us) and its
    shape are returned."""
    best = None
    for wg in moeq8.STREAM_READ_SHAPES:
        def fn(wg=wg):
            for t, b in regions:
                moeq8.stream_read_shape(t, b, wg, sink)
        us = time_graph(torch, fn, reps) / len(regions) * 1e3
        if best is None or us < best[0]:
            best = (us, wg)
    return best


def sweep_replicas(torch, workloads, moeq8, cols, hidden, inter, topk, n_exp, seed, block_bytes=34):
    """Replica layers of the 256-expert routed layer at `cols` columns until
    the down launches of one rotation read at least ROTATION_BYTES.  Each
    replica draws its own x, logits and bias (seeded by its index) and is
    routed once here; its bank stores only the experts that routing selects,
    in slots 0..D-1, and its owner map sends those experts to their slots and
    every other expert to -1.  The top-k runs over all 256 experts whatever
    the owner map says, so the layer selects, weights and computes exactly as
    with all 256 experts stored, and its launches read the same bytes; the
    replicas only stop the 256 MB Infinity Cache from serving a rotation.
    block_bytes is the weight format's bytes per 32 values (34: Q8_0)."""
    dn_expert = hidden * (inter // 32 * block_bytes)
    reps, total = [], 0
    while total < ROTATION_BYTES:
        l = len(reps)
        x = torch.from_numpy(workloads.activations(seed, cols, hidden, layer=l)).cuda()
        lg = torch.from_numpy(workloads.router_logits(seed, cols, n_exp, layer=l)).cuda()
        bs = torch.from_numpy(workloads.router_bias(seed, n_exp, layer=l)).cuda()
        ids, _, _ = moeq8.moe_route_topk(lg, topk, bias=bs)
        sel = sorted(set(int(e) for e in ids.cpu().numpy().reshape(-1)))
        owner = np.full(n_exp, -1, np.int32)
        owner[sel] = np.arange(len(sel), dtype=np.int32)
        reps.append({"x": x, "logits": lg, "bias": bs, "owner": torch.from_numpy(owner).cuda(),
                     "n_local": len(sel)})
        total += len(sel) * dn_expert
    return reps


def pmc_reference_copy(torch):
    """A 512 MiB device-to-device copy of known size: what FETCH_SIZE and
    WRITE_SIZE read for it scales their readings of the other kernels."""
    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("pmc reference: copied 536870912 bytes device to device")
    del src, dst


def sweep(torch, workloads, moeq8, ml, args):
    """Routed layer, 256 experts, top-8, at 1..8 columns, on replica layers
    that rotate at least ROTATION_BYTES through every timed graph (the down
    launches, the smallest, included), so the 256 MB Infinity Cache cannot
    serve the reads.  Per column count: the layer (graph of the four-launch
    layers), the grouped gate/up launch and the grouped down launch alone
    (graphs of their launches, HIP events), the two together as the
    routed-expert MMVQ (their bytes over their summed times), and
    streaming-read ceilings of the same buffers at the gate/up's and the
    down's bytes per launch (best of the read shapes)."""
    cfg = workloads.CONFIGS["verify_e256_c5"]
    hidden, inter, topk, n_exp = cfg["hidden"], cfg["inter"], cfg["topk"], cfg["experts"]
    cols_list = [int(c) for c in args.sweep_cols.split(",")] if args.sweep_cols else (1, 2, 4, 5, 8)
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    rb_h, rb_i = hidden // 32 * 34, inter // 32 * 34
    out = []
    for cols in cols_list:
        reps = sweep_replicas(torch, workloads, moeq8, cols, hidden, inter, topk, n_exp, 4)
        R = len(reps)
        banks = []
        for l, rp in enumerate(reps):
            b = Bank(moeq8, torch, 1, rp["n_local"], hidden, inter, 4, layer0=l)
            b.pack_weights(moeq8, torch)
            banks.append(b)
        wss = [ml.Workspace(cols, hidden, inter, topk, 0, "cuda") for _ in range(R)]
        experts = [b.experts(ml, 0) for b in banks]

        def step():
            for l in range(R):
                rp = reps[l]
                ml.forward(rp["x"], rp["logits"], rp["bias"], rp["owner"], rp["n_local"], experts[l], None,
                           wss[l])

        step()
        torch.cuda.synchronize()
        n_active, n_valid = [], []
        for l in range(R):
            words = wss[l].grouping.cpu().numpy().view(np.int32)
            n_active.append(int(words[0]))
            n_valid.append(int(words[1]))
            assert n_active[l] == reps[l]["n_local"]
        n = max(20, args.steps)
        ms = time_graph(torch, step, n) / R
        lb = float(np.mean([layer_bytes(n_active[l], n_valid[l], cols, hidden, inter, topk, 0)
                            for l in range(R)]))

        def gate_up_only():
            for l in range(R):
                moeq8.moe_grouped_mmvq_ex(moeq8.GATE_UP_SWIGLU_P64, experts[l].gate, experts[l].up, wss[l].xq,
                                          wss[l].grouping, n=inter, k=hidden, n_local_expert=reps[l]["n_local"],
                                          ncols=cols, topk=topk, out=wss[l].h)

        def down_only():
            for l in range(R):
                moeq8.moe_grouped_mmvq_ex(moeq8.DOWN_F32_ACT_P64, experts[l].down, None,
                                          wss[l].h.view(cols * topk, inter), wss[l].grouping, n=hidden,
                                          k=inter, n_local_expert=reps[l]["n_local"], ncols=cols, topk=topk,
                                          out=wss[l].y)

        gu_b = [gate_up_launch_bytes(n_active[l], n_valid[l], cols, hidden, inter) for l in range(R)]
        dn_b = [down_launch_bytes(n_active[l], n_valid[l], hidden, inter) for l in range(R)]
        gu_us = time_graph(torch, gate_up_only, n) / R * 1e3
        dn_us = time_graph(torch, down_only, n) / R * 1e3
        # ceilings: one plain read per launch of the replica's own weights
        # (its gate and up banks, adjacent, in one read; its down bank)
        gu_w = [n_active[l] * inter * rb_h for l in range(R)]
        dn_w = [n_active[l] * hidden * rb_i for l in range(R)]
        st_gu_us, st_gu_wg = best_ceiling(
            torch, moeq8, [(banks[l].w[0], 2 * gu_w[l] // 16 * 16) for l in range(R)], n, sink)
        st_dn_us, st_dn_wg = best_ceiling(
            torch, moeq8, [(banks[l].down[0], dn_w[l] // 16 * 16) for l in range(R)], n, sink)
        st_all_us, st_all_wg = best_ceiling(
            torch, moeq8, [(banks[l].w[0], (2 * gu_w[l] + dn_w[l]) // 16 * 16) for l in range(R)], n, sink)
        gu_gbps = float(np.mean(gu_b)) / (gu_us * 1e-6) / 1e9
        dn_gbps = float(np.mean(dn_b)) / (dn_us * 1e-6) / 1e9
        both_gbps = float(np.mean(gu_b) + np.mean(dn_b)) / ((gu_us + dn_us) * 1e-6) / 1e9
        st_gu_gbps = 2 * float(np.mean(gu_w)) / (st_gu_us * 1e-6) / 1e9
        st_dn_gbps = float(np.mean(dn_w)) / (st_dn_us * 1e-6) / 1e9
        st_all_gbps = float(np.mean(gu_w) * 2 + np.mean(dn_w)) / (st_all_us * 1e-6) / 1e9
        st_pair_gbps = float(np.mean(gu_w) * 2 + np.mean(dn_w)) / ((st_gu_us + st_dn_us) * 1e-6) / 1e9
        rec = {"cols": cols, "active_experts": round(float(np.mean(n_active)), 2), "replicas": R,
               "rotation_bytes": {"layer": int(sum(n_active[l] * ml.expert_bytes(hidden, inter) for l in range(R))),
                                  "gate_up": int(sum(gu_b)), "down": int(sum(dn_b))},
               "layer_us": round(ms * 1e3, 2), "layers_per_s": round(1e3 / ms, 1),
               "effective_gbps": round(lb / (ms * 1e-3) / 1e9, 1),
               "gate_up_bytes_per_launch": round(float(np.mean(gu_b))),
               "down_bytes_per_launch": round(float(np.mean(dn_b))),
               "gate_up_us": round(gu_us, 2), "gate_up_gbps": round(gu_gbps, 1),
               "gate_up_frac_of_peak": round(gu_gbps / HBM_PEAK_GBPS, 4),
               "down_us": round(dn_us, 2), "down_gbps": round(dn_gbps, 1),
               "down_frac_of_peak": round(dn_gbps / HBM_PEAK_GBPS, 4),
               "routed_mmvq_gbps": round(both_gbps, 1),
               "routed_mmvq_frac_of_peak": round(both_gbps / HBM_PEAK_GBPS, 4),
               "gate_up_ceiling_gbps": round(st_gu_gbps, 1), "gate_up_ceiling_wg_bytes": st_gu_wg,
               "gate_up_frac_of_ceiling": round(gu_gbps / st_gu_gbps, 4),
               "down_ceiling_gbps": round(st_dn_gbps, 1), "down_ceiling_wg_bytes": st_dn_wg,
               "down_frac_of_ceiling": round(dn_gbps / st_dn_gbps, 4),
               # the two launches' ceilings together, and one read of all
               # three matrices' bytes in a single launch (what any split of
               # the work over launches is bounded by)
               "pair_ceiling_gbps": round(st_pair_gbps, 1),
               "routed_mmvq_frac_of_pair_ceiling": round(both_gbps / st_pair_gbps, 4),
               "one_read_ceiling_gbps": round(st_all_gbps, 1), "one_read_ceiling_wg_bytes": st_all_wg}
        log(f"sweep {rec}")
        out.append(rec)
        del banks, experts, wss, reps
        torch.cuda.empty_cache()
    return out


def wide_gate_up_bytes(n_active, n_valid, cols, hidden, inter):
    return gate_up_launch_bytes(n_active, n_valid, cols, hidden, inter)


def wide_down_bytes(n_active, n_valid, hidden, inter):
    """Per grouped down launch on q8_1 h: every active expert's down matrix
    once, the q8_1 h rows once, the y rows written."""
    return n_active * hidden * (inter // 32 * 34) + n_valid * (inter // 32 * 36) + n_valid * hidden * 4


def wide_sweep(torch, workloads, moeq8, ml, args):
    """The 256-expert layer at 32..1024 columns (one weight copy, 3.4 GB: a
    launch over all experts reads far more than the 256 MB Infinity Cache).
    Per column count: the seven-launch layer with the grouped products on the
    matrix cores and with the grouped MMVQ, and each grouped product alone
    (graphs, HIP events), against a plain streaming read of as many bytes;
    the layer, the gate/up and the down again on the GEMM's own layout
    (pack_gemm_experts: a second copy of the experts); then the MMVQ passes
    on the packed layouts."""
    cfg = workloads.CONFIGS["wide_e256"]
    hidden, inter, topk, n_exp, seed = cfg["hidden"], cfg["inter"], cfg["topk"], cfg["experts"], cfg["seed"]
    bank = Bank(moeq8, torch, 1, n_exp, hidden, inter, seed)
    experts = bank.experts(ml, 0)
    ge = ml.pack_gemm_experts(experts)
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    out = []
    for cols in cfg["cols"]:
        x = torch.from_numpy(workloads.activations(seed, cols, hidden)).cuda()
        lg = torch.from_numpy(workloads.router_logits(seed, cols, n_exp)).cuda()
        bs = torch.from_numpy(workloads.router_bias(seed, n_exp)).cuda()
        ws = ml.WideWorkspace(cols, hidden, inter, topk, "cuda")
        ml.forward_wide(x, lg, bs, None, n_exp, experts, ws)
        torch.cuda.synchronize()
        words = ws.grouping.cpu().numpy().view(np.int32)
        n_active, n_valid = int(words[0]), int(words[1])
        reps = 10 if cols >= 512 else 20
        rec = {"cols": cols, "active_experts": n_active,
               "routes_per_expert_mean": round(n_valid / max(1, n_active), 2)}
        gu_b = gate_up_launch_bytes(n_active, n_valid, cols, hidden, inter)
        dn_b = wide_down_bytes(n_active, n_valid, hidden, inter)
        for name, fn in (("gemm", moeq8.moe_grouped_gemm), ("mmvq", moeq8.moe_grouped_mmvq)):
            layer_ms = time_graph(torch, lambda: ml.forward_wide(x, lg, bs, None, n_exp, experts, ws,
                                                                 products=name), reps)
            gu_us = time_graph(torch, lambda: fn(moeq8.GATE_UP_SWIGLU, experts.gate, experts.up, ws.xq,
                                                 ws.grouping, n=inter, k=hidden, n_local_expert=n_exp,
                                                 ncols=cols, topk=topk, out=ws.h), reps) * 1e3
            dn_us = time_graph(torch, lambda: fn(moeq8.DOWN, experts.down, None, ws.hq, ws.grouping,
                                                 n=hidden, k=inter, n_local_expert=n_exp, ncols=cols,
                                                 topk=topk, out=ws.y), reps) * 1e3
            rec[name] = {"layer_us": round(layer_ms * 1e3, 1),
                         "cols_per_s": round(cols / (layer_ms * 1e-3), 1),
                         "gate_up_us": round(gu_us, 1),
                         "gate_up_gbps": round(gu_b / (gu_us * 1e-6) / 1e9, 1),
                         "down_us": round(dn_us, 1),
                         "down_gbps": round(dn_b / (dn_us * 1e-6) / 1e9, 1)}
        # gate/up in the GEMM's layout (the same bits)
        layer_ms = time_graph(torch, lambda: ml.forward_wide(x, lg, bs, None, n_exp, ge, ws, products="gemm"),
                              reps)
        gu_us = time_graph(torch, lambda: moeq8.moe_grouped_gemm(
            moeq8.GATE_UP_SWIGLU_G8, ge.gemm_gate, ge.gemm_up, ws.xq, ws.grouping, n=inter, k=hidden,
            n_local_expert=n_exp, ncols=cols, topk=topk, out=ws.h), reps) * 1e3
        dn_us = time_graph(torch, lambda: moeq8.moe_grouped_gemm(
            moeq8.DOWN_G8, ge.gemm_down, None, ws.hq, ws.grouping, n=hidden, k=inter, n_local_expert=n_exp,
            ncols=cols, topk=topk, out=ws.y), reps) * 1e3
        rec["gemm_layout"] = {"layer_us": round(layer_ms * 1e3, 1),
                              "cols_per_s": round(cols / (layer_ms * 1e-3), 1),
                              "gate_up_us": round(gu_us, 1),
                              "gate_up_gbps": round(gu_b / (gu_us * 1e-6) / 1e9, 1),
                              "gate_up_frac_of_peak": round(gu_b / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                              "down_us": round(dn_us, 1),
                              "down_gbps": round(dn_b / (dn_us * 1e-6) / 1e9, 1)}
        # the ceiling: as many bytes read from the gate and up banks
        half = min(int(gu_b) // 2, bank.gate[0].numel()) // 16 * 16

        def stream_only():
            moeq8.stream_read(bank.gate[0], half, sink)
            moeq8.stream_read(bank.up[0], half, sink)

        st_us = time_graph(torch, stream_only, reps) * 1e3
        st_bytes = 2 * half
        rec["gate_up_bytes"] = int(gu_b)
        rec["down_bytes"] = int(dn_b)
        rec["ceiling_gbps"] = round(st_bytes / (st_us * 1e-6) / 1e9, 1)
        rec["gemm"]["gate_up_frac_of_peak"] = round(rec["gemm"]["gate_up_gbps"] / HBM_PEAK_GBPS, 4)
        rec["gemm"]["gate_up_frac_of_ceiling"] = round(rec["gemm"]["gate_up_gbps"] / rec["ceiling_gbps"], 4)
        rec["gemm_layout"]["gate_up_frac_of_ceiling"] = round(rec["gemm_layout"]["gate_up_gbps"] / rec["ceiling_gbps"], 4)
        log(f"wide {rec}")
        out.append(rec)
        del ws, x, lg, bs
    del ge
    torch.cuda.empty_cache()
    # The MMVQ passes again on the packed layouts (the bank repacked in place):
    # the six-launch layer, the packed gate/up and the down that quantises h
    # in its launch, each alone.
    bank.pack_weights(moeq8, torch)
    experts = bank.experts(ml, 0)
    for rec in out:
        cols = rec["cols"]
        x = torch.from_numpy(workloads.activations(seed, cols, hidden)).cuda()
        lg = torch.from_numpy(workloads.router_logits(seed, cols, n_exp)).cuda()
        bs = torch.from_numpy(workloads.router_bias(seed, n_exp)).cuda()
        ws = ml.WideWorkspace(cols, hidden, inter, topk, "cuda")
        ml.forward_wide(x, lg, bs, None, n_exp, experts, ws, products="mmvq")
        torch.cuda.synchronize()
        reps = 10 if cols >= 512 else 20
        words = ws.grouping.cpu().numpy().view(np.int32)
        n_active, n_valid = int(words[0]), int(words[1])
        layer_ms = time_graph(torch, lambda: ml.forward_wide(x, lg, bs, None, n_exp, experts, ws,
                                                             products="mmvq"), reps)
        gu_us = time_graph(torch, lambda: moeq8.moe_grouped_mmvq_ex(
            moeq8.GATE_UP_SWIGLU_P64, experts.gate, experts.up, ws.xq, ws.grouping, n=inter, k=hidden,
            n_local_expert=n_exp, ncols=cols, topk=topk, out=ws.h), reps) * 1e3
        dn_us = time_graph(torch, lambda: moeq8.moe_grouped_mmvq_ex(
            moeq8.DOWN_F32_ACT_P64, experts.down, None, ws.h.view(cols * topk, inter), ws.grouping,
            n=hidden, k=inter, n_local_expert=n_exp, ncols=cols, topk=topk, out=ws.y), reps) * 1e3
        gu_b = rec["gate_up_bytes"]
        dn_b = down_launch_bytes(n_active, n_valid, hidden, inter)
        rec["mmvq_packed"] = {"layer_us": round(layer_ms * 1e3, 1),
                              "cols_per_s": round(cols / (layer_ms * 1e-3), 1),
                              "gate_up_us": round(gu_us, 1),
                              "gate_up_gbps": round(gu_b / (gu_us * 1e-6) / 1e9, 1),
                              "down_us": round(dn_us, 1),
                              "down_gbps": round(dn_b / (dn_us * 1e-6) / 1e9, 1)}
        log(f"wide packed mmvq {cols}: {rec['mmvq_packed']}")
        del ws, x, lg, bs
    del bank, experts
    torch.cuda.empty_cache()
    return out


def codec_bench(torch, workloads, moeq8, args):
    """The exchange codec on [rows, 4096] fp32 partials: encode (reads 4 B,
    writes 1.125 B a value) and decode-sum of R ranks (reads R * 1.125 B,
    writes 4 B a value), timed with HIP events over graphs of 20 launches."""
    n = 4096
    out = []
    for rows in (1024, 8192):
        x = torch.from_numpy(workloads.normal_f32(7, (rows, n), 1.0)).cuda()
        blocks = moeq8.q8_block_encode(x)
        per = blocks.numel()
        gathered = torch.empty((8, per), dtype=torch.uint8, device="cuda")
        for r in range(8):
            gathered[r].copy_(blocks.view(-1))
        res = torch.empty((rows, n), dtype=torch.float32, device="cuda")
        reps, per = 10, 20
        enc_us = time_graph_each(torch, lambda: moeq8.q8_block_encode(x, out=blocks), per, reps) * 1e3
        rec = {"rows": rows, "n": n, "encode_us": round(enc_us, 2),
               "encode_gbps": round(rows * n * 5.125 / (enc_us * 1e-6) / 1e9, 1)}
        for nr in (2, 8):
            g = gathered[:nr]
            us = time_graph_each(torch, lambda: moeq8.q8_block_decode_sum(g, rows, n, out=res), per, reps) * 1e3
            rec[f"decode_sum_{nr}_us"] = round(us, 2)
            rec[f"decode_sum_{nr}_gbps"] = round(rows * n * (nr * 1.125 + 4) / (us * 1e-6) / 1e9, 1)
        log(f"codec {rec}")
        out.append(rec)
        del x, blocks, gathered, res
    torch.cuda.empty_cache()
    return out


def q4_sweep(torch, workloads, moeq8, ml, args):
    """The sweep's routed layer (256 experts, top-8, no shared expert) with
    4-bit expert weights, on replica layers as in the sweep (each stores only
    the experts its routing selects; every rotation reads at least
    ROTATION_BYTES of 4-bit down weights, so the Infinity Cache cannot serve
    it).  Weights are N(0, 0.02^2) drawn on the GPU (torch, seeded) and
    quantised by q4_quantize_rows.  Per column count: the four-launch layer,
    the grouped gate/up alone, and the streaming-read ceiling of the same
    bytes per launch from the replicas' gate and up banks (best read shape);
    then the layer and the gate/up again on packed copies of the banks
    (pack_experts: the 64-chunk packed stages), after the plain banks are
    freed."""
    cfg = workloads.CONFIGS["verify_e256_c5"]
    hidden, inter, topk, n_exp = cfg["hidden"], cfg["inter"], cfg["topk"], cfg["experts"]
    q4b = 18
    gen = torch.Generator(device="cuda").manual_seed(44)
    row_gu = (hidden // 32) * q4b
    per_gu = inter * row_gu
    per_d = hidden * (inter // 32) * q4b
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    out = []
    for cols in (1, 2, 4, 5, 8):
        reps = sweep_replicas(torch, workloads, moeq8, cols, hidden, inter, topk, n_exp, 4, block_bytes=q4b)
        R = len(reps)
        banks = []
        for rp in reps:
            d = rp["n_local"]
            # gate then up in one buffer, so that one plain read covers both
            w = torch.empty(2 * d * per_gu, dtype=torch.uint8, device="cuda")
            down = torch.empty(d * per_d, dtype=torch.uint8, device="cuda")
            for buf, base, rows, k, per in ((w, 0, inter, hidden, per_gu), (w, d * per_gu, inter, hidden, per_gu),
                                            (down, 0, hidden, inter, per_d)):
                for e in range(d):
                    x = torch.randn((rows, k), generator=gen, device="cuda") * 0.02
                    moeq8.q4_quantize_rows(x, out=buf[base + e * per:base + (e + 1) * per].view(rows, -1))
            banks.append({"w": w, "gate": w[:d * per_gu], "up": w[d * per_gu:], "down": down})
        torch.cuda.synchronize()
        wss = [ml.Workspace(cols, hidden, inter, topk, 0, "cuda") for _ in range(R)]
        experts = [ml.RoutedExperts(b["gate"], b["up"], b["down"], reps[l]["n_local"], hidden, inter, fmt="q4")
                   for l, b in enumerate(banks)]

        def step():
            for l in range(R):
                rp = reps[l]
                ml.forward(rp["x"], rp["logits"], rp["bias"], rp["owner"], rp["n_local"], experts[l], None,
                           wss[l])

        step()
        torch.cuda.synchronize()
        n_active, n_valid = [], []
        for l in range(R):
            words = wss[l].grouping.cpu().numpy().view(np.int32)
            n_active.append(int(words[0]))
            n_valid.append(int(words[1]))
            assert n_active[l] == reps[l]["n_local"]
        n = max(20, args.steps)
        ms = time_graph(torch, step, n) / R

        def gate_up_only():
            for l in range(R):
                moeq8.moe_grouped_mmvq_q4(moeq8.GATE_UP_SWIGLU, banks[l]["gate"], banks[l]["up"], wss[l].xq,
                                          wss[l].grouping, n=inter, k=hidden, n_local_expert=reps[l]["n_local"],
                                          ncols=cols, topk=topk, out=wss[l].h)

        gu_b = [n_active[l] * 2 * inter * row_gu + cols * (hidden // 32 * 36) + n_valid[l] * inter * 4
                for l in range(R)]
        gu_us = time_graph(torch, gate_up_only, n) / R * 1e3
        gu_w = [n_active[l] * 2 * per_gu for l in range(R)]
        st_us, st_wg = best_ceiling(torch, moeq8, [(banks[l]["w"], gu_w[l] // 16 * 16) for l in range(R)], n, sink)
        gu_gbps = float(np.mean(gu_b)) / (gu_us * 1e-6) / 1e9
        st_gbps = float(np.mean(gu_w)) / (st_us * 1e-6) / 1e9
        weights = float(np.mean([n_active[l] * ml.expert_bytes_q4(hidden, inter) for l in range(R)]))
        rec = {"cols": cols, "active_experts": round(float(np.mean(n_active)), 2), "replicas": R,
               "rotation_bytes": int(sum(n_active[l] * ml.expert_bytes_q4(hidden, inter) for l in range(R))),
               "layer_us": round(ms * 1e3, 2), "layers_per_s": round(1e3 / ms, 1),
               "expert_weight_gbps": round(weights / (ms * 1e-3) / 1e9, 1),
               "gate_up_us": round(gu_us, 2), "gate_up_gbps": round(gu_gbps, 1),
               "gate_up_frac_of_peak": round(gu_gbps / HBM_PEAK_GBPS, 4),
               "ceiling_gbps": round(st_gbps, 1), "ceiling_wg_bytes": st_wg,
               "gate_up_frac_of_ceiling": round(gu_gbps / st_gbps, 4)}
        # the packed stages on packed copies (the plain banks freed first)
        packed = []
        for l in range(R):
            packed.append(ml.pack_experts(experts[l])[0])
            banks[l] = None
            experts[l] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

        def step_packed():
            for l in range(R):
                rp = reps[l]
                ml.forward(rp["x"], rp["logits"], rp["bias"], rp["owner"], rp["n_local"], packed[l], None,
                           wss[l])

        def gate_up_packed():
            for l in range(R):
                moeq8.moe_grouped_mmvq_q4(moeq8.GATE_UP_SWIGLU_P64, packed[l].gate, packed[l].up, wss[l].xq,
                                          wss[l].grouping, n=inter, k=hidden, n_local_expert=reps[l]["n_local"],
                                          ncols=cols, topk=topk, out=wss[l].h)

        pms = time_graph(torch, step_packed, n) / R
        pgu_us = time_graph(torch, gate_up_packed, n) / R * 1e3
        pgu_gbps = float(np.mean(gu_b)) / (pgu_us * 1e-6) / 1e9
        rec["packed"] = {"layer_us": round(pms * 1e3, 2), "expert_weight_gbps": round(weights / (pms * 1e-3) / 1e9, 1),
                         "gate_up_us": round(pgu_us, 2), "gate_up_gbps": round(pgu_gbps, 1),
                         "gate_up_frac_of_peak": round(pgu_gbps / HBM_PEAK_GBPS, 4),
                         "gate_up_frac_of_ceiling": round(pgu_gbps / st_gbps, 4)}
        log(f"q4 {rec}")
        out.append(rec)
        del banks, experts, wss, reps, packed
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
