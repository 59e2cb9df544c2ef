"""Verify-step benchmark on one MI355X.

One step is the whole hot path of a speculative-decoding verify pass over
synthetic Llama-shaped inputs already resident in HBM:

  1. the target's linear stack over M = B*(K+1) positions: per layer QKV,
     O, gate/up and down, each reading its bf16 weights once (bf16
     outputs): one spec_verify_gemm_chain launch for all of them up to
     M = 8, above that one spec_verify_gemm_ws per linear (the reduction
     split over workgroups where that is faster);
  2. the lm-head (spec_verify_gemm, fp32 logits over the vocabulary);
  3. the sampling stage (spec_verify on those logits): softmax statistics,
     accept test and first rejection, residual or bonus draw, emit.

Each phase is captured once in a HIP graph; a timed step replays the two
graphs back to back with HIP events between them on the same stream.
With --w8 every linear (stack and lm-head) holds FP8 E4M3 weights with a
per-row scale (weight-only 8-bit storage, bf16 activations and products):
one chain launch up to M = 16, per-linear MFMA tile launches
(spec_verify_gemm_w8_ws) above. Prints one JSON line: the throughput in verified positions per second, the
per-phase times, the roofline of the GEMM phase (algorithmic bytes over its
measured time, against the 8 TB/s HBM peak; MFMA peak where the FLOPs
dominate) and the fp64 oracle's rate on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload llama8b|llama70b]
                    [--batch B] [--no-graph] [--no-chain] [--no-split]
                    [--no-cpu-baseline] [--w8]
    python bench.py --attention [--batch B] [--context C]
                                         # the verify attention alone
    python bench.py --stress [--rounds R]  # the sampling-stress workload
    python bench.py --sweep [--w8]       # the batch sweep B = 1, 4, 16, 64, 256:
                                         # both roofline fractions per B and the
                                         # measured memory-to-compute crossover
    python bench.py --linear 4096x6144 --batch B
                                         # one linear per launch (for profiles)
    python bench.py --probe              # the achievable ceilings: HBM read
                                         # bandwidth and dense bf16 MFMA rate
    python bench.py --copy-calibration   # plain device copy of known size,
                                         # the scale for HBM traffic counters
"""

import argparse
import contextlib
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA
K_DRAFT = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=["llama8b", "llama70b"], default="llama8b")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-split", action="store_true",
                    help="per-linear launches: spec_verify_gemm / _w8 (no split "
                         "reduction) instead of spec_verify_gemm_ws / _w8_ws")
    ap.add_argument("--no-chain", action="store_true",
                    help="one spec_verify_gemm launch per linear instead of one chain launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--attention", action="store_true",
                    help="time spec_verify_attention alone: Llama-3.1-8B layer (32 query / 8 "
                         "key-value heads, head_dim 128), K+1 = 5 queries per sequence")
    ap.add_argument("--context", type=int, default=4096,
                    help="cached tokens before the verify positions (--attention)")
    ap.add_argument("--w8", action="store_true",
                    help="FP8 E4M3 weights with per-row scales for every linear")
    ap.add_argument("--lm-head", choices=["chain", "fused"], default="chain",
                    help="chain: the lm-head is the last linear of the chain launch and "
                         "spec_verify reads its logits; fused: the chain holds the stack only "
                         "and spec_verify runs the lm-head with the target rows' softmax "
                         "statistics fused into its epilogue (bf16 weights, M <= 8)")
    ap.add_argument("--t-target", type=float, default=1.0,
                    help="temperature of the target's distribution in the sampling stage "
                         "(0: greedy verification)")
    ap.add_argument("--t-draft", type=float, default=1.0,
                    help="temperature of the draft's distribution (0: greedy drafts); the draft "
                         "tokens are drawn from it")
    ap.add_argument("--stress", action="store_true",
                    help="sampling-stress workload: B=64, K=8, V=128256, target logits "
                         "N(0, 3^2), draft rows calibrated to alpha in {0.6, 0.81, 0.9}; "
                         "--rounds verification rounds per alpha")
    ap.add_argument("--rounds", type=int, default=100000,
                    help="rounds per alpha for --stress")
    ap.add_argument("--sweep", action="store_true",
                    help="batch sweep on the workload's shapes: B in --sweep-batches")
    ap.add_argument("--sweep-batches", default="1,4,16,64,256")
    ap.add_argument("--linear", default=None,
                    help="DINxDOUT: time spec_verify_gemm_ws (or _w8_ws; with --no-split the "
                         "calls without a split reduction) on one linear at M = 5 B, rotating "
                         "over weight copies that together exceed the 256 MB cache")
    ap.add_argument("--probe", action="store_true",
                    help="measure the achievable HBM read bandwidth and dense bf16 MFMA rate")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (the known-size "
                         "reference that scales FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def kernel_source_sha():
    """Hash of the streaming-GEMM sources; stored traffic counters are used
    only while this matches the hash recorded with them."""
    h = hashlib.sha256()
    for f in ("gemm_stream.hip", "common.h", "internal.h", "chain_sync.h"):
        with open(os.path.join(ROOT, "speculative_decoding_verification_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM traffic per launch measured with rocprofv3 counters, if it was
    taken on the current kernel source (profiles/<name>.txt)."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Workload:
    """Device-resident inputs of one verify step."""

    def __init__(self, stack, B, K, seed, dev, w8=False, fused_lm_head=False):
        import torch
        import synth
        from synth import device as sd

        self.stack, self.B, self.K, self.dev, self.w8 = stack, B, K, dev, w8
        self.fused_lm_head = fused_lm_head  # lm-head runs inside spec_verify
        self.split = True  # bf16 per-linear launches: spec_verify_gemm_ws
        self.t_target, self.t_draft = 1.0, 1.0  # sampling temperatures (0: greedy)
        self.M = B * (K + 1)
        self.linears = []  # (name, x, w, y)
        self.scales = []   # FP8 weights: per-row scales of each linear
        base = synth.WEIGHT_STD / synth.W8_CODE_STD

        def weights(d_out, d_in, wseed):
            if not w8:
                return sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, wseed, dev), None
            return (sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, wseed, dev),
                    sd.w8_row_scales(d_out, base, wseed + 977, dev))

        for i, (name, d_in, d_out) in enumerate(stack.all_linears()[:-1]):
            w, sc = weights(d_out, d_in, seed * 1000 + 2 * i)
            x = sd.normal_bf16((self.M, d_in), 1.0, seed * 1000 + 2 * i + 1, dev)
            y = torch.empty((self.M, d_out), dtype=torch.bfloat16, device=dev)
            self.linears.append((name, x, w, y))
            self.scales.append(sc)
        V, d = stack.vocab, stack.hidden
        self.V = V
        self.lm_head, self.lm_scale = weights(V, d, seed * 7 + 1)
        self.hidden = sd.normal_bf16((self.M, d), 1.0, seed * 7 + 2, dev)
        self.target_logits = torch.empty((B, K + 1, V), dtype=torch.float32, device=dev)
        self.out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        self.n_emitted = torch.empty(B, dtype=torch.int32, device=dev)
        self.u_accept = sd.uniform_f32((B, K), seed * 7 + 3, dev)
        self.u_sample = sd.uniform_f32((B, K + 1), seed * 7 + 4, dev)
        torch.cuda.synchronize()

    def make_drafts(self, sv, sigma, seed):
        """Draft logits = the lm-head's logits + sigma * N(0,1); draft tokens
        from the draft distributions (Gumbel-max)."""
        import torch
        from synth import device as sd
        self.lm_head_gemm(sv)
        tl = self.target_logits[:, :self.K, :]
        self.draft_logits = (tl + sd.normal_f32(tl.shape, sigma, seed * 7 + 5, self.dev)).contiguous()
        if self.t_draft == 0.0:
            self.draft_tokens = self.draft_logits.argmax(dim=-1).int()
        else:
            self.draft_tokens = sd.gumbel_max_tokens(
                (self.draft_logits / self.t_draft).contiguous(), seed * 7 + 6)
        self.workspace = sv.new_workspace(self.B, self.K, self.V, self.dev)
        torch.cuda.synchronize()

    def lm_head_gemm(self, sv):
        out = self.target_logits.view(self.M, self.V)
        if self.w8:
            sv.verify_gemm_w8(self.hidden, self.lm_head, self.lm_scale, out=out)
        else:
            sv.verify_gemm(self.hidden, self.lm_head, out=out)

    def make_chain(self, sv):
        """All stack linears and the lm-head as one chain (one launch)."""
        if self.w8:
            lin = [(x, w, sc, y) for (_, x, w, y), sc in zip(self.linears, self.scales)]
            lin.append((self.hidden, self.lm_head, self.lm_scale,
                        self.target_logits.view(self.M, self.V)))
        else:
            lin = [(x, w, y) for _, x, w, y in self.linears]
            if not self.fused_lm_head:
                lin.append((self.hidden, self.lm_head, self.target_logits.view(self.M, self.V)))
        self.chain = sv.Chain(lin, self.dev)

    def ws_bytes(self, sv, w):
        f = sv.gemm_w8_workspace_bytes if self.w8 else sv.gemm_workspace_bytes
        return f(self.M, w.shape[1], w.shape[0])

    def split_linears(self, sv):
        """Stack linears that spec_verify_gemm_ws (_w8_ws) runs with a split
        reduction."""
        if not self.split:
            return 0
        return sum(self.ws_bytes(sv, w) > 0 for _, _, w, _ in self.linears)

    def gemm_phase(self, sv):
        import torch
        if getattr(self, "chain", None) is not None:
            self.chain.run()
            return
        if self.split and getattr(self, "gemm_ws", None) is None:
            # one workspace for every linear: the calls run in stream order
            need = max(self.ws_bytes(sv, w) for _, _, w, _ in self.linears)
            self.gemm_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.dev)
        for (_, x, w, y), sc in zip(self.linears, self.scales):
            if self.w8 and self.split:
                sv.verify_gemm_w8_ws(x, w, sc, out=y, workspace=self.gemm_ws)
            elif self.w8:
                sv.verify_gemm_w8(x, w, sc, out=y)
            elif self.split:
                sv.verify_gemm_ws(x, w, out=y, workspace=self.gemm_ws)
            else:
                sv.verify_gemm(x, w, out=y)
        if not self.fused_lm_head:
            self.lm_head_gemm(sv)

    def sampling_phase(self, sv):
        lm = {"hidden": self.hidden, "lm_head": self.lm_head} if self.fused_lm_head else {}
        sv.verify(self.target_logits, self.draft_logits, self.draft_tokens, self.u_accept,
                  self.u_sample, workspace=self.workspace, out_tokens=self.out_tokens,
                  n_emitted=self.n_emitted, t_target=self.t_target, t_draft=self.t_draft, **lm)

    def gemm_bytes(self):
        """Algorithmic HBM bytes of the GEMM phase: every weight once, every
        activation once, every output once (bf16 stack outputs, fp32 logits)."""
        total = 0
        for (_, x, w, y), sc in zip(self.linears, self.scales):
            total += w.numel() * w.element_size() + 2 * x.numel() + 2 * y.numel()
            total += 0 if sc is None else 4 * sc.numel()
        if not self.fused_lm_head:
            total += self.lm_head_bytes()
        return total

    def lm_head_bytes(self):
        return (self.lm_head.numel() * self.lm_head.element_size() + 2 * self.hidden.numel()
                + 4 * self.target_logits.numel() + (0 if self.lm_scale is None else 4 * self.V))

    def gemm_flops(self):
        n = sum(2 * x.shape[0] * w.numel() for _, x, w, _ in self.linears)
        return n + (0 if self.fused_lm_head else 2 * self.M * self.lm_head.numel())

    def n_gemm_launches(self):
        if getattr(self, "chain", None) is not None:
            return 1
        return len(self.linears) + (0 if self.fused_lm_head else 1)


def time_steps(wl, sv, n, warmup, graph=True):
    """Times n steps (GEMM phase, then sampling phase) with HIP events on the
    stream both phases run on, after `warmup` untimed ones. With graph=True
    each phase is captured once and replayed. Returns sorted per-step
    (gemm ms, sampling ms, step ms) and the wall time of the timed loop."""
    import torch
    # eager pass (also initialises the library's per-device state)
    wl.gemm_phase(sv)
    wl.sampling_phase(sv)
    torch.cuda.synchronize()
    if not graph:
        run_gemm = lambda: wl.gemm_phase(sv)  # noqa: E731
        run_samp = lambda: wl.sampling_phase(sv)  # noqa: E731
    else:
        g_gemm, g_samp = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_gemm):
            wl.gemm_phase(sv)
        with torch.cuda.graph(g_samp):
            wl.sampling_phase(sv)
        torch.cuda.synchronize()
        run_gemm, run_samp = g_gemm.replay, g_samp.replay
    for _ in range(warmup):
        run_gemm()
        run_samp()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        ev[i][0].record()
        run_gemm()
        ev[i][1].record()
        run_samp()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_gemm = sorted(e[0].elapsed_time(e[1]) for e in ev)
    t_samp = sorted(e[1].elapsed_time(e[2]) for e in ev)
    t_step = sorted(e[0].elapsed_time(e[2]) for e in ev)
    return t_gemm, t_samp, t_step, wall


def measure_ceilings(sv, dev, read_bytes=4 << 30, reps=5, mfma_iters=2048):
    """The achievable ceilings beside the published peaks (the library's
    probe kernels): HBM read bandwidth streaming a buffer larger than the
    256 MB Infinity Cache, and the dense bf16 MFMA rate of independent
    16x16x32 and 32x32x16 chains. Each is the mean over `reps` launches."""
    import torch
    buf = torch.ones(read_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # bytes in flight per CU = 8 KB x loads per lane x workgroups per CU
    shapes = {}
    for wgs in (1, 2):
        for loads in (1, 2, 4, 8):
            sv.probe_read(buf, sink, loads, wgs)
            e0.record()
            for _ in range(reps):
                sv.probe_read(buf, sink, loads, wgs)
            e1.record()
            torch.cuda.synchronize()
            shapes[f"{8 * loads * wgs}KB_per_CU({wgs}wg,{loads}ld)"] = \
                read_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    best = max(shapes, key=shapes.get)
    out = {"read_gbs": shapes[best], "read_best_shape": best, "read_gbs_by_shape": shapes,
           "read_bytes": read_bytes}
    # the same read with the loads going straight to LDS (the tile kernels'
    # operand path), one workgroup per CU
    lds = {}
    for loads in (1, 2, 4, 8):
        sv.probe_read_lds(buf, sink, loads)
        e0.record()
        for _ in range(reps):
            sv.probe_read_lds(buf, sink, loads)
        e1.record()
        torch.cuda.synchronize()
        lds[f"{8 * loads}KB_per_CU(1wg,{loads}ld)"] = \
            read_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    out["read_lds_gbs"] = max(lds.values())
    out["read_lds_gbs_by_shape"] = lds
    del buf
    for shape in (16, 32):
        flops = sv.probe_mfma(shape, mfma_iters, sink)
        e0.record()
        for _ in range(reps):
            sv.probe_mfma(shape, mfma_iters, sink)
        e1.record()
        torch.cuda.synchronize()
        out[f"mfma_bf16_tflops_{shape}x{shape}"] = flops * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    out["mfma_bf16_tflops"] = max(out["mfma_bf16_tflops_16x16"], out["mfma_bf16_tflops_32x32"])
    return out


def cpu_baseline(wl, sample_layers=None):
    """The fp64 oracle on the host cores, on a bounded sample of the same
    step: the first layers' linears (whole layers until about 10 s of oracle
    time), the lm-head and the sampling stage on the GPU step's inputs; the
    remaining layers are scaled from the sampled ones."""
    import numpy as np
    import oracle
    from synth import device as sd
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    per_layer = len(wl.stack.linears)
    t_layer = 0.0
    def lin(x, w, sc):
        xb = sd.to_bits(x)
        if sc is None:
            wb = sd.to_bits(w)
            t0 = time.perf_counter()
            y = oracle.linear(xb, wb)
        else:
            wb, sb = w.cpu().numpy(), sc.cpu().numpy()
            t0 = time.perf_counter()
            y = oracle.linear_w8(xb, wb, sb)
        return y, time.perf_counter() - t0

    # whole layers until about 10 s of oracle time (or all of them)
    pairs = list(zip(wl.linears, wl.scales))
    done = 0
    while done < wl.stack.layers and (sample_layers is None and t_layer < 10.0
                                      or sample_layers is not None and done < sample_layers):
        for (name, x, w, _), sc in pairs[per_layer * done:per_layer * (done + 1)]:
            t_layer += lin(x, w, sc)[1]
        done += 1
    sample_layers = done
    t_layer /= sample_layers
    logits, t_lm = lin(wl.hidden, wl.lm_head, wl.lm_scale)
    logits = logits.astype(np.float32).reshape(wl.B, wl.K + 1, wl.V)
    dl = wl.draft_logits.cpu().numpy()
    toks = wl.draft_tokens.cpu().numpy()
    ua, us = wl.u_accept.cpu().numpy(), wl.u_sample.cpu().numpy()
    t0 = time.perf_counter()
    oracle.verify_batch(logits, dl, toks, ua, us)
    t_samp = time.perf_counter() - t0
    t_step = t_layer * wl.stack.layers + t_lm + t_samp
    return {
        "value": wl.M / t_step,
        "unit": "positions/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{sample_layers} of {wl.stack.layers} layers ({per_layer} linears each, "
                   f"{t_layer:.2f} s/layer, scaled x{wl.stack.layers}) + lm-head "
                   f"({t_lm:.2f} s) + sampling stage ({t_samp:.3f} s); fp64 numpy, "
                   f"BLAS threads={threads}, numpy conversion single-threaded"),
        "s_per_step": t_step,
    }


def attention_bench(args):
    """spec_verify_attention on the Llama-3.1-8B layer shape: B sequences,
    K+1 = 5 query positions each, a cache of context + 5 tokens, 32 query and
    8 key/value heads of 128. One step is one call (one layer). A graph holds
    32 calls, one per layer of the model, each on its own K/V cache while
    the caches together stay under 1 GiB (at B = 1, 32 caches of 16.8 MB: a
    single cache replayed would sit in the 256 MB last-level cache and read
    faster than HBM allows); the timed steps replay that graph. Bytes: the
    K/V cache read once, plus queries and outputs."""
    import math
    import numpy as np
    import torch
    import oracle
    import speculative_decoding_verification_gemm_amd as sv
    from synth import device as sd

    dev = torch.device("cuda:0")
    B, K, H, Hkv, D = args.batch, K_DRAFT, 32, 8, 128
    T = args.context + K + 1
    n_layers = 32
    kv_bytes = 2 * B * T * Hkv * D * 2
    n_caches = max(1, min(n_layers, -(-(1 << 30) // kv_bytes)))
    q = sd.normal_bf16((B, K + 1, H, D), 1.0, args.seed + 1, dev)
    caches = [(sd.normal_bf16((B, T, Hkv, D), 1.0, args.seed + 2 + 2 * i, dev),
               sd.normal_bf16((B, T, Hkv, D), 1.0, args.seed + 3 + 2 * i, dev))
              for i in range(n_caches)]
    k, v = caches[0]
    out = torch.empty((B, K + 1, H, D), dtype=torch.bfloat16, device=dev)
    nb = sv.lib.spec_verify_attention_workspace_bytes(B, K, T, H, Hkv, D)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

    def layers():
        for i in range(n_layers):
            kc, vc = caches[i % n_caches]
            sv.verify_attention(q, kc, vc, out=out, workspace=ws)

    layers()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layers()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    n = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (n * n_layers)
    io_bytes = 2 * q.numel() * 2
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    line = {
        "metric": "verify attention: K/V cache bytes read per second (Llama-3.1-8B layer)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": n * n_layers, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) queries, keys and values)",
        "config": {"workload": f"verify attention, {B} sequences x {K + 1} queries, cache of "
                               f"{T} tokens, {H}/{Hkv} heads of {D}",
                   "global_batch": B, "cache_tokens": T, "workspace_bytes": nb,
                   "calls_per_graph": n_layers, "distinct_caches": n_caches},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": kv_bytes + io_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # the oracle on the first cache's sequences, one at a time, until
        # about 10 s of oracle time or all B (a bounded sample); bytes/s of
        # the cache it read
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()
                           if p.get("user_api") == "blas"] or [1])
        except Exception:
            threads = 1
        dt, done = 0.0, 0
        while done < B and dt < 10.0:
            qb = sd.to_bits(q[done:done + 1])
            kb, vb = sd.to_bits(k[done:done + 1]), sd.to_bits(v[done:done + 1])
            t0 = time.perf_counter()
            oracle.verify_attention(qb, kb, vb, 1 / math.sqrt(D))
            dt += time.perf_counter() - t0
            done += 1
        line["cpu_baseline"] = {"value": done * 2 * T * Hkv * D * 2 / dt / 1e9, "unit": "GB/s",
                                "cores": int(threads), "kind": "oracle",
                                "sample": f"{done} of {B} sequences of one layer ({dt:.2f} s), "
                                          f"fp64 numpy, BLAS threads={threads}"}
    print(json.dumps(line), flush=True)


def stress_bench(args):
    """The sampling-stress workload: fixed target logits N(0, 3^2) for B = 64
    sequences of K = 8 drafts over V = 128256; each draft row's noise scale
    is bisected so that its acceptance rate sum_x min(p, q) equals alpha.
    Every round draws fresh drafts x_j ~ q_j and fresh uniforms, then runs
    spec_verify. Reports tokens per round against 1 + sum_i prod_{j<=i}
    alpha_j (which equals (1 - alpha^(K+1)) / (1 - alpha) here) and the
    verify call's time against the bytes it must read."""
    import math
    import torch
    import synth
    import speculative_decoding_verification_gemm_amd as sv

    dev = torch.device("cuda:0")
    B, K, V, seed = 64, 8, 128256, 2027
    tl = torch.from_numpy(synth.normals(seed, "stress.target", (B, K + 1, V), 3.0)).to(dev)
    z = torch.from_numpy(synth.normals(seed, "stress.noise", (B, K, V))).to(dev)
    p = torch.softmax(tl[:, :K].double(), dim=-1)
    ws = sv.new_workspace(B, K, V, dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    # bytes one call must move: every target and draft logit once for the
    # statistics, plus the one target and draft row of each sequence that the
    # residual or bonus draw re-reads
    call_bytes = 4 * V * B * (2 * K + 1) + 2 * 4 * V * B
    results, ms_total, rounds_total = [], 0.0, 0
    n_check = 0 if args.no_cpu_baseline else 8  # rounds per alpha given to the oracle leg
    checks = []
    for alpha in (0.6, 0.81, 0.9):
        lo = torch.zeros((B, K), dtype=torch.float64, device=dev)
        hi = torch.full((B, K), 8.0, dtype=torch.float64, device=dev)
        for _ in range(44):
            mid = 0.5 * (lo + hi)
            a = torch.minimum(p, torch.softmax((tl[:, :K] + mid.float()[..., None] * z).double(),
                                               dim=-1)).sum(-1)
            lo, hi = torch.where(a > alpha, mid, lo), torch.where(a > alpha, hi, mid)
        sigma = (0.5 * (lo + hi)).float()
        dl = (tl[:, :K] + sigma[..., None] * z).contiguous()
        q = torch.softmax(dl.double(), dim=-1)
        a = torch.minimum(p, q).sum(-1)
        expect = float((1.0 + torch.cumprod(a, dim=1).sum(1)).mean())
        cq = torch.cumsum(q, dim=-1).reshape(B * K, V)
        del q
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed + int(alpha * 100))
        tot = torch.zeros((), dtype=torch.float64, device=dev)
        tot2 = torch.zeros((), dtype=torch.float64, device=dev)
        ev = []
        for r in range(args.rounds):
            u_draft = torch.rand((B * K, 1), generator=gen, device=dev)
            tok = torch.searchsorted(cq, u_draft.double() * cq[:, -1:], right=True)
            tok = tok.clamp_(max=V - 1).reshape(B, K).int()
            u_acc = torch.rand((B, K), generator=gen, device=dev)
            u_smp = torch.rand((B, K + 1), generator=gen, device=dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sv.verify(tl, dl, tok, u_acc, u_smp, workspace=ws, out_tokens=out, n_emitted=n)
            e1.record()
            ev.append((e0, e1))
            if r < n_check:
                checks.append((alpha, dl, tok.cpu().numpy(), u_acc.cpu().numpy(),
                               u_smp.cpu().numpy(), out.cpu().numpy(), n.cpu().numpy()))
            nd = n.double()
            tot += nd.sum()
            tot2 += (nd * nd).sum()
            if len(ev) >= 2000:
                torch.cuda.synchronize()
                ms_total += sum(x.elapsed_time(y) for x, y in ev)
                rounds_total += len(ev)
                ev = []
            if r % 20000 == 0:
                print(f"alpha={alpha}: round {r}", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        ms_total += sum(x.elapsed_time(y) for x, y in ev)
        rounds_total += len(ev)
        cnt = args.rounds * B
        mean = float(tot) / cnt
        se = math.sqrt(max(float(tot2) / cnt - mean * mean, 0.0) / cnt)
        results.append({"alpha": alpha, "rounds": args.rounds, "sequence_rounds": cnt,
                        "tokens_per_round": mean, "expected": expect,
                        "closed_form": (1 - alpha ** (K + 1)) / (1 - alpha), "se": se,
                        "z": (mean - expect) / se if se > 0 else 0.0,
                        "max_row_alpha_error": float((a - alpha).abs().max())})
        del cq
    ms = ms_total / rounds_total
    gbs = call_bytes / (ms * 1e-3) / 1e9
    base = stress_cpu_baseline(tl, checks) if checks else None
    print(json.dumps({
        "metric": "sampling-stress verification rounds/s (B=64, K=8, V=128256)",
        "value": 1e3 / ms, "unit": "rounds/s", "n_gpus": 1, "steps": rounds_total, "warmup": 0,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 logits, f64 decisions", "data": "synthetic (seeded N(0,3^2) logits, "
        "per-row calibrated draft noise)",
        "config": {"workload": "sampling stress: spec_verify on fixed logits, fresh drafts "
                               "and uniforms every round", "global_batch": B, "draft_tokens_K": K,
                   "vocab": V},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_call": call_bytes},
        "alphas": results, "cpu_baseline": base}), flush=True)


def stress_cpu_baseline(tl, checks):
    """The fp64 oracle on a bounded sample of the stress run: the first
    rounds of each alpha, on the same logits, drafts and uniforms, timed on
    the host. As a by-product the oracle's decisions are compared with what
    the GPU emitted in those rounds (tests/parity.py: bit-exact outside the
    1e-5 tie band, inside it within the band's tokens) and the ties are
    counted."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare_rounds
    tl_h = tl.cpu().numpy()
    dl_h = {}
    t_total, seqs, prefix_ties, band_draws = 0.0, 0, 0, 0
    per_alpha = {}
    for alpha, dl, tok, ua, us, out, n in checks:
        if alpha not in dl_h:
            dl_h[alpha] = dl.cpu().numpy()
        t0 = time.perf_counter()
        ref = oracle.verify_batch(tl_h, dl_h[alpha], tok, ua, us)
        t_total += time.perf_counter() - t0
        with contextlib.redirect_stdout(sys.stderr):  # keep stdout to the one JSON line
            b, nt, nb = compare_rounds(out, n, ref, f"stress alpha={alpha}", us)
        seqs, prefix_ties, band_draws = seqs + b, prefix_ties + nt, band_draws + nb
        pa = per_alpha.setdefault(str(alpha), {"rounds": 0, "prefix_ties": 0,
                                               "draws_within_band": 0})
        pa["rounds"] += 1
        pa["prefix_ties"] += nt
        pa["draws_within_band"] += nb
    rounds = len(checks)
    return {"value": rounds / t_total, "unit": "rounds/s", "cores": 1, "kind": "oracle",
            "sample": (f"the first {rounds // max(1, len(dl_h))} rounds of each alpha "
                       f"({rounds} rounds, {seqs} sequences, {t_total:.1f} s): "
                       "oracle.verify_batch on the same fp32 logits, drafts and uniforms "
                       "(fp64 numpy, single-threaded elementwise work)"),
           "agreement": {"sequences": seqs, "prefix_ties": prefix_ties,
                         "tokens_exact": seqs - prefix_ties - band_draws,
                         "tokens_within_band": band_draws, "mismatches": 0,
                         "per_alpha": per_alpha}}


def sweep_bench(args):
    """The batch sweep on the workload's shapes at K = 4: for each B the
    whole step (GEMM phase, then sampling) as the default line times it
    (the chain where it runs, per-linear launches above), the GEMM phase's
    fraction of the HBM peak (algorithmic bytes / time) and of the dense
    MFMA peak (FLOPs / time), and the memory-to-compute crossover.

    The crossover is measured as where the two regimes of the measured GEMM
    time meet: a flat part t0 (the weight read, the smallest B) and a part
    that grows with the work, slope c per sequence (from the two largest B);
    B* = t0 / c. The roofline's own crossover is where the intensity
    B (K+1) FLOP per weight byte (2 B (K+1) with FP8 weights) reaches the
    ridge, peak FLOP/s / peak bytes/s ("Speculative Decoding: The Algebra
    and the Proof", Where it breaks; "Guess Several Tokens", Wasted work,
    and why batching changes the answer)."""
    import torch
    import synth
    import speculative_decoding_verification_gemm_amd as sv

    dev = torch.device("cuda:0")
    stack = {"llama8b": synth.LLAMA_8B, "llama70b": synth.LLAMA_70B_16L}[args.workload]
    key = {"llama8b": "llama8b_lm_head", "llama70b": "llama70b_lm_head"}[args.workload]
    K = K_DRAFT
    rows = []
    for B in [int(b) for b in args.sweep_batches.split(",")]:
        wl = Workload(stack, B, K, args.seed, dev, w8=args.w8)
        wl.split = not args.no_split
        wl.make_drafts(sv, synth.draft_noise_sigma(key, 0.8), args.seed)
        use_chain = wl.M <= (16 if args.w8 else 8)
        if use_chain:
            wl.make_chain(sv)
        steps = max(5, min(args.steps, int(200 / B)))
        t_gemm, t_samp, t_step, _ = time_steps(wl, sv, steps, max(2, args.warmup // 4))
        ms_gemm, ms_samp = sum(t_gemm) / steps, sum(t_samp) / steps
        by, fl = wl.gemm_bytes(), wl.gemm_flops()
        rows.append({"B": B, "M": wl.M, "steps": steps,
                     "gemm_launch": "chain" if use_chain else "per-linear",
                     "split_linears": 0 if use_chain else wl.split_linears(sv),
                     "ms_gemm_phase": ms_gemm, "ms_sampling_phase": ms_samp,
                     "positions_per_s": wl.M / ((ms_gemm + ms_samp) * 1e-3),
                     "gemm_bytes": by, "gemm_flops": fl,
                     "hbm_frac": by / (ms_gemm * 1e-3) / (HBM_PEAK_GBS * 1e9),
                     "mfma_frac": fl / (ms_gemm * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                     "floor_ms": 1e3 * max(by / (HBM_PEAK_GBS * 1e9),
                                           fl / (MFMA_BF16_PEAK_TFLOPS * 1e12))})
        rows[-1]["frac_of_floor"] = rows[-1]["floor_ms"] / ms_gemm
        if use_chain and wl.chain.error():
            print("chain reported a device error", file=sys.stderr)
            sys.exit(3)
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del wl
        torch.cuda.empty_cache()
    ceil = measure_ceilings(sv, dev)
    t0 = rows[0]["ms_gemm_phase"]
    big = sorted(rows, key=lambda r: r["B"])[-2:]
    slope = ((big[1]["ms_gemm_phase"] - big[0]["ms_gemm_phase"]) / (big[1]["B"] - big[0]["B"])
             if len(big) == 2 and big[1]["B"] != big[0]["B"] else None)
    bytes_per_weight = 1 if args.w8 else 2
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    print(json.dumps({
        "metric": f"batch sweep of the verify step ({stack.name} shapes, K={K})",
        "value": None if not slope else t0 / slope,
        "unit": "sequences (measured memory-to-compute crossover B*)",
        "n_gpus": 1, "higher_is_better": None, "vs_baseline": None,
        "dtype": "bf16 (fp8 e4m3 weights)" if args.w8 else "bf16", "data": "synthetic",
        "config": {"workload": f"{stack.name} verify step at B in {args.sweep_batches}",
                   "draft_tokens_K": K, "weights": "fp8_e4m3" if args.w8 else "bf16"},
        "crossover": {"measured_B": None if not slope else t0 / slope,
                      "flat_ms": t0, "slope_ms_per_sequence": slope,
                      "roofline_B": ridge * bytes_per_weight / (2 * (K + 1)),
                      "ridge_flop_per_byte": ridge},
        "ceilings": ceil, "rows": rows}), flush=True)


def linear_bench(args):
    """spec_verify_gemm_ws (spec_verify_gemm_w8_ws with --w8; the calls
    without a split reduction with --no-split) on one linear, one call per
    step, rotating over weight copies that together exceed the 256 MB
    Infinity Cache (so every launch reads its weights from HBM). Output
    bf16, or fp32 for a linear as wide as the vocabulary."""
    import torch
    import synth
    import speculative_decoding_verification_gemm_amd as sv
    from synth import device as sd

    dev = torch.device("cuda:0")
    d_in, d_out = (int(v) for v in args.linear.lower().split("x"))
    M = args.batch * (K_DRAFT + 1)
    esz = 1 if args.w8 else 2
    copies = max(1, min(8, -(-(768 << 20) // (d_in * d_out * esz))))
    ws, scs = [], []
    for c in range(copies):
        if args.w8:
            ws.append(sd.e4m3_normal_codes((d_out, d_in), synth.W8_CODE_STD, args.seed + c, dev))
            scs.append(sd.w8_row_scales(d_out, synth.WEIGHT_STD / synth.W8_CODE_STD,
                                        args.seed + 100 + c, dev))
        else:
            ws.append(sd.normal_bf16((d_out, d_in), synth.WEIGHT_STD, args.seed + c, dev))
    x = sd.normal_bf16((M, d_in), 1.0, args.seed + 999, dev)
    od = torch.float32 if d_out >= 100000 else torch.bfloat16
    y = torch.empty((M, d_out), dtype=od, device=dev)
    need = (sv.gemm_w8_workspace_bytes if args.w8 else sv.gemm_workspace_bytes)(M, d_in, d_out)
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    split = not args.no_split

    def call(i):
        if args.w8 and split:
            sv.verify_gemm_w8_ws(x, ws[i % copies], scs[i % copies], out=y, workspace=wsp)
        elif args.w8:
            sv.verify_gemm_w8(x, ws[i % copies], scs[i % copies], out=y)
        elif split:
            sv.verify_gemm_ws(x, ws[i % copies], out=y, workspace=wsp)
        else:
            sv.verify_gemm(x, ws[i % copies], out=y)
    for i in range(max(args.warmup, copies)):
        call(i)
    torch.cuda.synchronize()
    n = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    by = d_in * d_out * esz + 2 * M * d_in + y.element_size() * M * d_out + \
        (4 * d_out if args.w8 else 0)
    fl = 2 * M * d_in * d_out
    print(json.dumps({
        "metric": f"one verify linear {d_in}->{d_out} at M={M}", "value": ms * 1e3,
        "unit": "us per launch", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "higher_is_better": False, "vs_baseline": None,
        "dtype": "bf16 (fp8 e4m3 weights)" if args.w8 else "bf16", "data": "synthetic",
        "config": {"workload": f"linear {d_in}->{d_out}, M={M}, {copies} weight copies",
                   "split_reduction": need > 0 and split},
        "gbs": by / (ms * 1e-3) / 1e9, "tflops": fl / (ms * 1e-3) / 1e12,
        "hbm_frac": by / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "mfma_frac": fl / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)}), flush=True)


def probe_bench(args):
    import torch
    import speculative_decoding_verification_gemm_amd as sv
    ceil = measure_ceilings(sv, torch.device("cuda:0"), reps=max(5, min(args.steps, 50)))
    print(json.dumps({
        "metric": "achievable ceilings: HBM read bandwidth and dense bf16 MFMA rate",
        "value": ceil["read_gbs"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "probe kernels: read-only stream over 4 GiB; independent MFMA "
                               "chains (16x16x32 and 32x32x16 bf16)"},
        "read_frac_of_peak": ceil["read_gbs"] / HBM_PEAK_GBS,
        "mfma_frac_of_peak": ceil["mfma_bf16_tflops"] / MFMA_BF16_PEAK_TFLOPS,
        "ceilings": ceil}), flush=True)


def copy_calibration(reps=5):
    """Copy 1 GiB device to device `reps` times: each copy reads and writes
    exactly 2^30 bytes, so the counters of one copy dispatch give the ratio
    between counted and true bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps,
                      "ms_per_copy": ms, "gbs_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.attention:
        attention_bench(args)
        return
    if args.stress:
        stress_bench(args)
        return
    if args.sweep:
        sweep_bench(args)
        return
    if args.linear:
        linear_bench(args)
        return
    if args.probe:
        probe_bench(args)
        return
    import torch
    import synth
    import speculative_decoding_verification_gemm_amd as sv

    dev = torch.device("cuda:0")
    stack = {"llama8b": synth.LLAMA_8B, "llama70b": synth.LLAMA_70B_16L}[args.workload]
    key = {"llama8b": "llama8b_lm_head", "llama70b": "llama70b_lm_head"}[args.workload]
    B, K = args.batch, K_DRAFT
    fused = args.lm_head == "fused"
    if fused and (args.w8 or B * (K + 1) > 8):
        print("--lm-head fused covers bf16 weights at M <= 8", file=sys.stderr)
        sys.exit(2)
    if not (args.t_target >= 0.0 and args.t_draft >= 0.0):
        print("temperatures must be >= 0", file=sys.stderr)
        sys.exit(2)
    wl = Workload(stack, B, K, args.seed, dev, w8=args.w8, fused_lm_head=fused)
    wl.t_target, wl.t_draft = args.t_target, args.t_draft
    wl.split = not args.no_split
    wl.make_drafts(sv, synth.draft_noise_sigma(key, 0.8), args.seed)
    # the chain runs the streaming kernel: bf16 up to 8 positions (above, the
    # per-linear tile kernel is faster), FP8 weights up to 16 (its only kernel)
    use_chain = not args.no_chain and wl.M <= (16 if args.w8 else 8)
    if use_chain:
        wl.make_chain(sv)

    n = args.steps
    t_gemm, t_samp, t_step, wall = time_steps(wl, sv, n, args.warmup, not args.no_graph)
    emitted = wl.n_emitted.long()
    med = lambda a: a[len(a) // 2]  # noqa: E731
    ms_step = sum(t_step) / n
    ms_gemm = sum(t_gemm) / n
    ms_samp = sum(t_samp) / n
    ceil = measure_ceilings(sv, dev)

    gemm_bytes = wl.gemm_bytes()
    gemm_flops = wl.gemm_flops()
    launches = wl.n_gemm_launches()
    achieved = gemm_bytes / (ms_gemm * 1e-3) / 1e9
    traffic = load_traffic(f"traffic_gemm_stream_{'w8_' if args.w8 else ''}{args.workload}_b{B}"
                           + ("_stack" if fused else ""))
    # The GEMM phase is bound by whichever floor is higher: reading the
    # weights at the HBM peak, or the FLOPs at the dense bf16 MFMA peak.
    mfma_bound = gemm_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > gemm_bytes / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": gemm_flops / (ms_gemm * 1e-3) / 1e12,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "achievable": ceil["mfma_bf16_tflops"]}
    else:
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "achievable": ceil["read_gbs"]}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the same achieved rate against what the probe kernels reach on this part
    roof["frac_of_achievable"] = roof["achieved"] / roof["achievable"]
    # Expected tokens per round from each draft row's exact acceptance rate
    # alpha_j = sum_x min(p_j(x), q_j(x)): E[N] = 1 + sum_i prod_{j<=i} alpha_j.
    def warped(logits, t):
        if t == 0.0:  # one-hot at the first maximum
            return torch.nn.functional.one_hot(logits.argmax(dim=-1), logits.shape[-1]).double()
        return torch.softmax(logits.double() / t, dim=-1)
    p_rows = warped(wl.target_logits[:, :K, :], args.t_target)
    q_rows = warped(wl.draft_logits, args.t_draft)
    alpha = torch.minimum(p_rows, q_rows).sum(-1)  # [B][K]
    e_n = (1.0 + torch.cumprod(alpha, dim=1).sum(1)).mean().item()

    line = {
        "metric": f"verified positions/s at K={K} ({stack.name} shapes)",
        "value": wl.M / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (fp8 e4m3 weights)" if args.w8 else "bf16",
        "data": ("synthetic (seeded N(0,1) activations, "
                 + ("FP8 E4M3 weight codes N(0,64^2) with per-row scales ~0.02/64, "
                    if args.w8 else "N(0,0.02^2) bf16 weights, ")
                 + "draft logits = target logits + calibrated noise, alpha~0.8)"),
        "config": {
            "workload": (f"{stack.name} verify step: {stack.layers} layers x (QKV, O, gate/up, "
                         f"down) + lm-head {stack.hidden}->{stack.vocab} + sampling"),
            "global_batch": B,
            "draft_tokens_K": K,
            "positions_M": wl.M,
            "vocab": wl.V,
            "graph": not args.no_graph,
            "gemm_launch": "chain" if use_chain else "per-linear",
            "split_linears": 0 if use_chain else wl.split_linears(sv),
            "lm_head": ("in spec_verify, softmax statistics fused into its epilogue" if fused
                        else "last linear of the GEMM phase"),
            "weights": "fp8_e4m3 + fp32 row scale" if args.w8 else "bf16",
            "temperatures": {"target": args.t_target, "draft": args.t_draft},
        },
        "pct_hbm_peak_in_verify": 100.0 * achieved / HBM_PEAK_GBS,
        "achievable_gbs": ceil["read_gbs"],
        "pct_achievable_hbm_in_verify": 100.0 * achieved / ceil["read_gbs"],
        "ceilings": ceil,
        "ms_gemm_phase": ms_gemm,
        "ms_sampling_phase": ms_samp,  # with --lm-head fused: lm-head + sampling
        "sampling_share": ms_samp / ms_step,
        "ms_step_p10_p50_p90": [t_step[n // 10], med(t_step), t_step[(9 * n) // 10]],
        "wall_s": wall,
        "mean_emitted_per_sequence_last_step": float(emitted.float().mean()),
        "alpha_mean": alpha.mean().item(),
        "expected_tokens_per_round": e_n,
        "emitted_tokens_per_s": B * e_n / (ms_step * 1e-3),
        "roofline": {
            **roof,
            "kernel": (("gemm_stream FP8-weight chain" if args.w8 else "gemm_stream chain")
                       + (" (all stack linears in one launch)" if fused else
                          " (all stack linears + lm-head in one launch)") if use_chain
                       else "per-linear " + ("spec_verify_gemm_w8" if args.w8 else
                                             "spec_verify_gemm")
                       + ("_ws" if wl.split else "")
                       + " calls (stack linears" + ("" if fused else " + lm-head")
                       + "; a call with a split reduction runs two kernels)"),
            "traffic": traffic,
            "hbm_gbs": achieved,
            "hbm_frac": achieved / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": gemm_bytes / launches,
            "launches_per_step": launches,
            "avg_launch_ms": ms_gemm / launches,
            "gemm_tflops": gemm_flops / (ms_gemm * 1e-3) / 1e12,
        },
        "cpu_baseline": None,
    }
    if use_chain:
        err = wl.chain.error()
        if err:
            print(f"chain reported device error {err}", file=sys.stderr)
            sys.exit(3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
