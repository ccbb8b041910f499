"""Verify-round throughput on one MI355X: rounds/s and achieved HBM GB/s of the q8b32 head.

A step is one device-resident verify round through the C ABI entry point specverify_round:
  int8 per-block-32 head matmul of the S = K+1 window + fused argmax
  -> greedy accept (commits 1 + j tokens) -> n-gram drafter for the next round
The dense-stack workload runs 36 x [rmsnorm, gate/up + SiLU*mul, down + residual] and a final
rmsnorm in front of the head, through specverify_stack; the int4 workload swaps in the int4
per-block-32 head (specverify_round_q4b32); the sampling and tree workloads run
specverify_round_sample and specverify_round_tree; the generation-loop workload gathers each
window from a token-indexed stand-in model on the device (specverify_generate); the script
workload verifies windows of a stand-in target whose greedy continuation is a fixed script,
so that drafts are accepted at a rate strictly between 0 and 1; the decode workload times
plain S = 1 greedy steps.  The roofline
object times the dominant kernel: the head matmul, or the stack's gate/up projection.  Inputs are seeded
synthetic data resident in HBM before the timed region; hidden rows rotate over 64 sets and, for
heads that could sit in the 256 MB Infinity Cache, over several copies of the weights.

Beyond the K timed steps (the headline value), every run also times batches of rounds (64,
or 8 for the dense stack; median and interquartile range of rounds/s), the same batches on one
weight copy when the weights rotate over several, and the verify forward at the workload's S
against S = 1 (c_v(S) = t(S) / t(1)).  The oracle baseline runs on all host cores and on one
thread, plus a GEMM-only time with the fp64 dequantized weights cached.

Prints one JSON line.  --gpus N with N > 1 is refused: the library has no multi-GPU path.

Host-only helpers for the profile summaries (no GPU needed):
  bench.py summarize-trace DB OUT TITLE COMMAND [NOTE]
  bench.py summarize-counters WORKLOAD KERNEL_SUBSTRING PROFILE_DIR COMMAND...
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "verify rounds/s and achieved HBM GB/s (% of peak), int8 lm_head S=K+1"

# workloads: (config id for seeds, V, H, K, drafts, context length, copy rate, layers)
WORKLOADS = {
    "c1": dict(cid=0, V=8192, H=512, K=8, drafts="ngram", ctx=512, copy=None, layers=0, graph=64,
               name="tiny head H=512 V=8192 K=8 S=9, n-gram drafts over a 512-id context with a planted span"),
    "c2": dict(cid=1, V=151936, H=2560, K=8, drafts="ngram", ctx=4096, copy=0.30, layers=0,
               name="Qwen3-4B-shaped head H=2560 V=151936 K=8 S=9, n-gram drafts over 4096 Zipf(1.1) ids with 30% copied spans"),
    "c3": dict(cid=2, V=248320, H=2048, K=8, drafts="forced", ctx=4096, copy=0.30, layers=0,
               name="35B-A3B-shaped head H=2048 V=248320 K=8 S=9, drafts forced to match the first j~U{0..K} argmaxes"),
    "c3q4": dict(cid=2, V=248320, H=2048, K=8, drafts="forced", ctx=4096, copy=0.30, layers=0, fmt="q4",
                 name="35B-A3B-shaped int4 per-block-32 head H=2048 V=248320 K=8 S=9 (the same fp32 weights as c3), "
                      "drafts forced to match the first j~U{0..K} argmaxes"),
    "c3samp": dict(cid=2, V=248320, H=2048, K=8, drafts="forced", ctx=4096, copy=0.30, layers=0, temp=0.7,
                   name="sampling verify at T=0.7: 35B-A3B-shaped head H=2048 V=248320 K=8 S=9, drafts forced to "
                        "match the first j~U{0..K} argmaxes, kept with probability p(d) (speculative sampling)"),
    "c3tree": dict(cid=2, V=248320, H=2048, K=8, drafts="ngram", ctx=4096, copy=0.30, layers=0, tree=(3, 4),
                   name="tree verify: 35B-A3B-shaped head H=2048 V=248320, 8 tree nodes (S=9) from the 3 best "
                        "n-gram matches continued 4 deep over 4096 Zipf(1.1) ids with 30% copied spans, "
                        "greedy walk down the tree"),
    "c3s17": dict(cid=2, V=248320, H=2048, K=16, drafts="forced", ctx=4096, copy=0.30, layers=0,
                  name="35B-A3B-shaped head H=2048 V=248320 K=16 S=17, forced drafts"),
    "c4s1": dict(cid=3, V=248320, H=5120, K=0, drafts="none", ctx=16384, copy=0.20, layers=0,
                 name="decode step of the large-hidden head H=5120 V=248320 S=1 (plain greedy decoding: one-row "
                      "verify, the anchor committed), the c_v(S) denominator"),
    "c4s2": dict(cid=3, V=248320, H=5120, K=1, drafts="ngram", ctx=16384, copy=0.20, layers=0,
                 name="large-hidden head H=5120 V=248320 K=1 S=2, n-gram drafts over 16384 Zipf(1.1) ids with 20% copied spans"),
    "c4s9": dict(cid=3, V=248320, H=5120, K=8, drafts="ngram", ctx=16384, copy=0.20, layers=0,
                 name="large-hidden head H=5120 V=248320 K=8 S=9, n-gram drafts"),
    "c4s17": dict(cid=3, V=248320, H=5120, K=16, drafts="ngram", ctx=16384, copy=0.20, layers=0,
                  name="large-hidden head H=5120 V=248320 K=16 S=17, n-gram drafts"),
    "c3gen": dict(cid=2, V=248320, H=2048, K=8, drafts="ngram", ctx=4096, copy=0.30, layers=0, model="table",
                  name="generation loop: 35B-A3B-shaped head H=2048 V=248320 K=8 S=9 under a token-indexed stand-in "
                       "model (window rows gathered from a seeded fp16 N(0,1) table [V, H]), n-gram drafts, "
                       "device-resident rounds through specverify_generate"),
    "c3tied": dict(cid=2, V=248320, H=2048, K=8, drafts="ngram", ctx=4096, copy=0.30, layers=0, model="script",
                   name="generation loop with acceptance 0 < alpha < 1: 35B-A3B-shaped head H=2048 V=248320 K=8 S=9 "
                        "under a stand-in target whose greedy continuation is a fixed script (Zipf(1.1) ids with 30% "
                        "copied spans; window row at position p = sign of the head's code row of the scripted id), "
                        "n-gram drafts over the first 4096 script ids and the committed stream"),
    "c5": dict(cid=4, V=151936, H=4096, K=8, drafts="ngram", ctx=4096, copy=0.30, layers=36, F=12288,
               name="dense stack 36 x [4096->12288 gate/up, 12288->4096 down] + 4096x151936 head, K=8 S=9"),
}
R_SETS = 64
KERNEL_WARM = 1000         # most untimed calls before the launches of the roofline timing
SAMPLE_SEED = 0x5EED_0000_2026


def head_bytes(V, H, S, fmt="q8"):
    """Algorithmic HBM bytes of one head launch: int8 (or packed int4) codes, fp16 block
    scales, fp16 window."""
    codes = V * H // 2 if fmt == "q4" else V * H
    return codes + 2 * V * (H // 32) + 2 * S * H


def gateup_bytes(H, F, S):
    """Algorithmic HBM bytes of one gate/up launch of the dense stack: the int8 codes and fp16
    scales of both matrices, the fp16 window rows in, m = silu(g)*u out, the norm's fp32
    sum-of-squares partials in."""
    return 2 * (F * H + 2 * F * (H // 32)) + 2 * S * H + 2 * S * F + 4 * S * (H // 16)


def stack_bytes(layers, H, F, S):
    per = 3 * (F * H + 2 * F * (H // 32))
    return layers * (per + 2 * S * (H + 2 * F + H))


def kernel_fmt(workload):
    """Which kernel the roofline of a workload times: the stack's gate/up projection when the
    workload has a dense stack (its dominant kernel), else the head of its weight format."""
    wl = WORKLOADS[workload]
    return "stack" if wl["layers"] else wl.get("fmt", "q8")


def kernel_source_hash(fmt="q8"):
    """Hash of the code (comments and whitespace removed) of the sources the timed kernel of
    this format is built from: an edit of the code changes it, a comment edit does not."""
    h = hashlib.sha256()
    src = {"q4": "sv_q4.hip", "stack": "sv_chunked.hip"}.get(fmt, "sv_gemm.hip")
    for name in (src, "sv_device.h"):
        with open(os.path.join(ROOT, "weight_bound_verify_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counters_path(workload):
    fmt = kernel_fmt(workload)
    name = f"stack_gateup_q8b32_{workload}" if fmt == "stack" else f"verify_{fmt}b32_{workload}"
    return os.path.join(ROOT, "profiles", f"{name}_counters.json")


def load_traffic(workload):
    """HBM traffic per launch of the head kernel from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel_fmt(workload)):
        return None
    return rec.get("traffic_bytes_per_launch")


def summarize_trace(db_path, out, title, cmd, note=""):
    """Markdown per-kernel summary (calls, total, average duration) of a rocprofv3
    --kernel-trace database; runs on the host, no GPU needed."""
    import collections
    import sqlite3
    db = sqlite3.connect(db_path)
    st = collections.OrderedDict()
    for n, s, e in db.execute("select name, start, end from kernels order by start"):
        st.setdefault(n, []).append((e - s) / 1000.0)
    tot = sum(sum(v) for v in st.values())
    lines = [f"# {title}", "", "Command (from the repository root, TMPDIR=/tmp):", "", f"    {cmd}", ""]
    if note:
        lines += [note, ""]
    lines += ["| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for n, v in sorted(st.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{n[:110]}` | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.3f} | {100 * sum(v) / tot:.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(workload, kernel_sub, pdir, commands):
    """HBM traffic per head launch from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB per
    dispatch) and the same counters on a 1 GiB device copy (bench.py --calib-copy), which fix the
    factor from counter units to bytes.  Writes the counter summary that load_traffic reads."""
    import sqlite3
    import statistics

    def vals(path, sub):
        rows = sqlite3.connect(path).execute("select kernel_name, value from counters_collection").fetchall()
        return [v for n, v in rows if sub in n], sorted(set(n for n, v in rows if sub in n))

    f, names = vals(f"{pdir}/pmc_FETCH_SIZE/{workload}_results.db", kernel_sub)
    w, _ = vals(f"{pdir}/pmc_WRITE_SIZE/{workload}_results.db", kernel_sub)
    cf, _ = vals(f"{pdir}/calib_FETCH_SIZE/calib_results.db", "copyBuffer")
    cw, _ = vals(f"{pdir}/calib_WRITE_SIZE/calib_results.db", "copyBuffer")
    copy = 1 << 30
    ff = round(copy / 1024 / statistics.median(cf[1:]), 1)   # the first copy is the host upload
    fw = round(copy / 1024 / statistics.median(cw[1:]), 1)
    fm, wm = statistics.median(f), statistics.median(w)
    rec = {
        "workload": workload, "kernel": names[0] if len(names) == 1 else names,
        "kernel_source_hash": kernel_source_hash(kernel_fmt(workload)),
        "fetch_size_kib_per_dispatch_median": fm, "write_size_kib_per_dispatch_median": wm,
        "dispatches": len(f),
        "calibration": {"copy_bytes": copy, "fetch_factor": ff, "write_factor": fw,
                        "note": "a 1 GiB device copy reads and writes 1 GiB; the factors scale the counters to bytes"},
        "traffic_bytes_per_launch": int(round((fm * ff + wm * fw) * 1024)),
        "commands": commands,
    }
    with open(counters_path(workload), "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps(rec, indent=1))


def _streams(wl, synth):
    """The workload's seeded streams; a nonzero --seed moves every stream to another base (the
    config ids stay below 2^16 apart, so no two (seed, config) pairs share a base)."""
    return synth.streams(wl["cid"], synth.SEED_BASE + (wl["seed"] << 16))


def build_inputs(wl, args, torch, sv, synth):
    dev = torch.device("cuda:0")
    V, H, K = wl["V"], wl["H"], wl["K"]
    S = K + 1
    st = _streams(wl, synth)
    t0 = time.time()
    if wl.get("fmt") == "q4":
        q, s = synth.quantized_head_q4(st.weights, V, H)
    else:
        q, s = synth.quantized_head(st.weights, V, H)
    copies = args.rotate if args.rotate else (2 if V * H < 2 ** 31 else 1)
    wq = [torch.from_numpy(q).to(dev)]
    ws = [torch.from_numpy(s).to(dev)]
    for _ in range(copies - 1):
        wq.append(wq[0].clone())
        ws.append(ws[0].clone())
    rng_h = np.random.default_rng(st.hidden)
    hidden_np = synth.fp16_normal(rng_h, (R_SETS, S, wl["H"]))
    hidden = torch.from_numpy(hidden_np).to(dev)
    rng_c = np.random.default_rng(st.context)
    script = rows = None
    if wl.get("model") == "script":
        # the script: the context, then everything the target will commit (and a margin)
        n = wl["ctx"] + (args.warmup + args.steps + KERNEL_WARM + args.kernel_reps + 2 * args.batches * args.batch_rounds
                           + 64) * S
        script, frac = synth.zipf_context_with_copies(rng_c, n, V, wl["copy"])
        ctx = script[:wl["ctx"]].copy()
        rows = torch.from_numpy(synth.ScriptHidden(q, script).rows()).to(dev)
    elif wl["copy"] is None:
        ctx, _, _ = synth.uniform_context_with_span(rng_c, wl["ctx"], V, 12, 16)
        frac = None
    else:
        ctx, frac = synth.zipf_context_with_copies(rng_c, wl["ctx"], V, wl["copy"])
    layers = None
    if wl["layers"]:
        # stacked [L][rows][cols] tensors, one allocation per matrix kind
        F, L = wl["F"], wl["layers"]
        kids = st.weights.spawn(1)[0].spawn(3 * L)
        shapes = [(F, H), (F, H), (H, F)]
        layers = []
        for r, c in shapes:
            layers += [torch.empty((L, r, c), dtype=torch.int8, device=dev),
                       torch.empty((L, r, c // 32), dtype=torch.float16, device=dev)]
        for li in range(L):
            for m, (r, c) in enumerate(shapes):
                qq, ss = synth.quantized_head(kids[3 * li + m], r, c)
                layers[2 * m][li].copy_(torch.from_numpy(qq))
                layers[2 * m + 1][li].copy_(torch.from_numpy(ss))
    print(f"# inputs ready in {time.time() - t0:.1f} s (weight copies: {copies})", file=sys.stderr, flush=True)
    return dict(q=q, s=s, wq=wq, ws=ws, hidden=hidden, hidden_np=hidden_np, ctx=ctx, copy_frac=frac, layers=layers,
                copies=copies, script=script, rows=rows)


def _blas_threads():
    from threadpoolctl import threadpool_info
    n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    return n[0] if n else None


class _OracleRound:
    """One whole round of the oracle as it stands (propose, logits, argmax, accept) on the
    workload's inputs, on a host copy of the stream."""

    def __init__(self, wl, inp, table):
        import oracle
        from weight_bound_verify_amd import synth
        self.oracle, self.synth, self.wl, self.inp = oracle, synth, wl, inp
        self.table = table.cpu().numpy() if table is not None else None
        self.rows = inp["rows"].cpu().numpy() if inp["rows"] is not None else None
        self.rng = np.random.default_rng(12345)
        self.tokens = list(inp["ctx"])
        self.r = 0

    def window(self, drafts):
        K = self.wl["K"]
        if self.table is not None:
            return self.table[[self.tokens[-1]] + [d if d >= 0 else 0 for d in drafts]]
        if self.rows is not None:
            p = len(self.tokens) - 1
            return self.rows[p:p + K + 1]
        return self.inp["hidden_np"][self.r % 4]

    def logits(self, x):
        if self.wl.get("fmt") == "q4":
            return self.oracle.head_logits_q4b32(self.inp["q"], self.inp["s"], x)
        return self.oracle.head_logits(self.inp["q"], self.inp["s"], x)

    def __call__(self):
        oracle, wl, K = self.oracle, self.wl, self.wl["K"]
        if K == 0:                                          # a decode step: S = 1, commit the argmax
            x = self.inp["hidden_np"][self.r % 4][:1]
            self.tokens.append(int(oracle.argmax_lowest(self.logits(x))[0]))
            self.r += 1
            return
        if wl.get("tree"):
            parents, drafts, _, _ = oracle.propose_tree(self.tokens, wl["ngram"], K, *wl["tree"])
        else:
            drafts, _, _ = oracle.propose_scan(self.tokens, wl["ngram"], K)
        L = self.logits(self.window(drafts))
        a = oracle.argmax_lowest(L)
        if wl["drafts"] == "forced":
            drafts, _ = self.synth.forced_drafts(self.rng, a, K, wl["V"])
        if wl.get("temp"):
            app = oracle.sampling_verify(L, drafts, wl["temp"], wl["sample_seed"], len(self.tokens))["appended"]
        elif wl.get("tree"):
            _, app, _ = oracle.tree_accept(a, parents, drafts)
        else:
            _, app = oracle.accept(a, drafts)
        self.tokens += app
        self.r += 1


def _time_rounds(fn, max_rounds, budget):
    ts = []
    while len(ts) < max_rounds and sum(ts) < budget:
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return ts


def cpu_baseline(wl, inp, table=None, budget=15.0):
    """The oracle as it stands, timed on the host: whole rounds on all host cores (BLAS threads
    = cores), then on one thread, then the GEMM-only part (the window's fp64 logits against a
    cached fp64 dequantized head)."""
    import oracle
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    if wl["layers"]:
        return _cpu_baseline_stack(wl, inp, cores)
    S = wl["K"] + 1
    with threadpool_limits(limits=cores):
        blas = _blas_threads()
        t_all = _time_rounds(_OracleRound(wl, inp, table), 4, budget)
    with threadpool_limits(limits=1):
        t_one = _time_rounds(_OracleRound(wl, inp, table), 3, budget)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        wd = (oracle.dequantize_q4b32 if wl.get("fmt") == "q4" else oracle.dequantize)(inp["q"], inp["s"])
        t_deq = time.perf_counter() - t0
        xs = [inp["hidden_np"][i % 4][:S].astype(np.float64) for i in range(5)]
        t_g = []
        for x in xs:
            t0 = time.perf_counter()
            _ = x @ wd.T
            t_g.append(time.perf_counter() - t0)
        del wd
    med = float(np.median(t_all))
    kind = ("softmax, Philox noise, residual draws, sampling accept" if wl.get("temp") else
            "argmax, tree walk" if wl.get("tree") else "argmax, accept")
    return {"value": 1.0 / med, "unit": "rounds/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(t_all)} whole rounds of this workload, median {med:.2f} s per round (fp64 dequantize in "
                      f"8192-row chunks, fp64 logits for S={S}, {kind}, n-gram "
                      f"{'tree ' if wl.get('tree') else ''}propose over the {len(inp['ctx'])}-id context and what "
                      f"the rounds commit), on all {cores} host cores (BLAS threads {blas})",
            "blas_threads": blas,
            "single_thread": {"value": 1.0 / float(np.median(t_one)), "unit": "rounds/s", "rounds": len(t_one)},
            "gemm_only": {"value": 1.0 / float(np.median(t_g)), "unit": "rounds/s", "cores": cores,
                          "sample": f"median of {len(t_g)} fp64 [{S}, H] x [H, V] products against the fp64 head "
                                    f"dequantized once ({t_deq:.1f} s) and cached"}}


def _cpu_baseline_stack(wl, inp, cores, budget=8.0):
    """The dense-stack round is about a minute of oracle time, so the oracle runs a bounded
    sample: blocks in order (their exact weights, read back from the device) until the budget
    is spent, then one head round on their output, scaled to a whole round as L x mean block +
    head round; once on all host cores and once on one thread.  GEMM-only: the three
    projections of two blocks and the head's logits against cached fp64 dequantized weights."""
    import oracle
    from threadpoolctl import threadpool_limits

    K, L = wl["K"], wl["layers"]
    S = K + 1
    hid = inp["hidden_np"][0]

    def layer(li):
        return [(inp["layers"][2 * m][li].cpu().numpy(), inp["layers"][2 * m + 1][li].cpu().numpy())
                for m in range(3)]

    def sample():
        tb = []
        x = hid
        for li in range(L):
            lay = layer(li)
            t1 = time.perf_counter()
            x = oracle.mlp_block(x, lay)
            tb.append(time.perf_counter() - t1)
            if sum(tb) > budget:
                break
        t1 = time.perf_counter()
        drafts, _, _ = oracle.propose_scan(list(inp["ctx"]), wl["ngram"], K)
        Lg = oracle.head_logits(inp["q"], inp["s"], oracle.rmsnorm_fp16(x))
        oracle.accept(oracle.argmax_lowest(Lg), drafts)
        th = time.perf_counter() - t1
        return L * float(np.mean(tb)) + th, len(tb), float(np.mean(tb)), th

    with threadpool_limits(limits=cores):
        blas = _blas_threads()
        per_all, nb, tblock, thead = sample()
    with threadpool_limits(limits=1):
        per_one, nb1, _, _ = sample()
    with threadpool_limits(limits=cores):
        x = hid.astype(np.float64)
        tg = []
        for li in range(2):
            for qm, sm in layer(li):
                wd = oracle.dequantize(qm, sm)
                xin = np.ones((S, wd.shape[1]))
                t1 = time.perf_counter()
                _ = xin @ wd.T
                tg.append(time.perf_counter() - t1)
        wd = oracle.dequantize(inp["q"], inp["s"])
        t1 = time.perf_counter()
        _ = x @ wd.T
        th_g = time.perf_counter() - t1
        del wd
    per_gemm = L * 3 * float(np.mean(tg)) + th_g
    return {"value": 1.0 / per_all, "unit": "rounds/s", "cores": cores, "kind": "oracle",
            "sample": f"blocks 0..{nb - 1} of the {L} (fp64 dequantize and the three projections each, {tblock:.2f} s "
                      f"per block) and one head round on their output (final norm, fp64 logits, argmax, accept, "
                      f"n-gram propose: {thead:.2f} s), scaled to a whole round as {L} x block + head; on all {cores} "
                      f"host cores (BLAS threads {blas})",
            "blas_threads": blas,
            "single_thread": {"value": 1.0 / per_one, "unit": "rounds/s", "blocks_sampled": nb1},
            "gemm_only": {"value": 1.0 / per_gemm, "unit": "rounds/s", "cores": cores,
                          "sample": f"fp64 products of the 6 projections of blocks 0 and 1 (mean {np.mean(tg):.3f} s) "
                                    f"and the head ({th_g:.2f} s) against cached fp64 dequantized weights, scaled to "
                                    f"{L} x 3 projections + head"}}


def _batch_stats(ms_per_batch, rounds_per_batch):
    r = np.array([rounds_per_batch * 1000.0 / m for m in ms_per_batch])
    q1, med, q3 = np.percentile(r, [25, 50, 75])
    return {"rounds_per_batch": rounds_per_batch, "batches": len(r), "median_rounds_per_s": round(float(med), 2),
            "iqr_rounds_per_s": [round(float(q1), 2), round(float(q3), 2)],
            "median_us_per_round": round(1e6 / float(med), 3)}


def configure_workload(args):
    """The workload of --config with the --K, --ngram and --seed overrides applied (and --logits
    checked against it); raises SystemExit on a value the workload cannot take."""
    wl = dict(WORKLOADS[args.config])
    if getattr(args, "logits", False) and (wl.get("temp") or wl.get("model") or wl["K"] == 0):
        raise SystemExit(f"--logits: workload {args.config} has no round call that writes logits")
    if not 1 <= args.ngram <= 8:
        raise SystemExit(f"--ngram {args.ngram}: the drafter takes n-gram orders 1..8")
    if not 0 <= args.seed < 2 ** 15:
        raise SystemExit(f"--seed {args.seed}: use 0 .. {2 ** 15 - 1}")
    if args.K is not None and args.K != wl["K"]:
        # the sampling, tree, int4 and dense-stack paths take windows of at most 16 rows
        kmax = 15 if (wl.get("tree") or wl.get("temp") or wl.get("fmt") == "q4" or wl["layers"]) else 63
        if wl["K"] == 0 or not 1 <= args.K <= kmax:
            raise SystemExit(f"--K {args.K}: workload {args.config} takes K in 1..{kmax}"
                             if wl["K"] else f"--K: {args.config} is the one-row decode step (K = 0)")
        K = args.K
        name = re.sub(r"K=\d+ S=\d+", f"K={K} S={K + 1}", wl["name"])
        name = re.sub(r"\d+ tree nodes \(S=\d+\)", f"{K} tree nodes (S={K + 1})", name)
        wl["name"] = name if name != wl["name"] else f"{name}; K={K} S={K + 1}"
        wl["K"] = K
    wl["ngram"] = args.ngram
    wl["seed"] = args.seed
    wl["sample_seed"] = SAMPLE_SEED + args.seed
    return wl


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "summarize-trace":
        # bench.py summarize-trace DB OUT TITLE COMMAND [NOTE]
        summarize_trace(*sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "summarize-counters":
        # bench.py summarize-counters WORKLOAD KERNEL_SUBSTRING PROFILE_DIR COMMAND...
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0, help="weight copies to rotate (0 = automatic)")
    ap.add_argument("--batches", type=int, default=10, help="batches of rounds for the median and IQR")
    ap.add_argument("--batch-rounds", type=int, default=0, help="rounds per batch (0 = 64, 8 for the dense stack)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=50, help="isolated head launches timed for the roofline")
    ap.add_argument("--calib-copy", action="store_true", help="run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--graph-rounds", type=int, default=-1,
                    help="replay the timed rounds and the batches from one HIP graph of this many rounds "
                         "(0 = launch every round; -1 = the workload's default: a graph only where the round "
                         "is launch-bound)")
    ap.add_argument("--K", type=int, default=None,
                    help="drafts per round (S = K+1 window rows; default: the workload's K)")
    ap.add_argument("--ngram", type=int, default=3, help="largest n-gram order of the drafter (1..8)")
    ap.add_argument("--seed", type=int, default=0,
                    help="input seed: 0 = the workload's own streams, others move every seeded input")
    ap.add_argument("--logits", action="store_true",
                    help="every round also writes the full fp32 logits [S][V] (greedy workloads that verify "
                         "through a round call: not the sampling, generation or decode workloads)")
    ap.add_argument("--down-split", type=int, default=0,
                    help="dense stack: split the down projection's hidden axis this many ways (2..8; 0 = unsplit)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the vocab-sharded head "
              "and the tensor-parallel stack are a design, not code); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    wl = configure_workload(args)          # argument errors before anything touches the GPU

    import torch

    from weight_bound_verify_amd import specverify as sv
    from weight_bound_verify_amd import synth

    if args.down_split:
        sv.set_tuning(0, 0, 0, 0, args.down_split)
    if args.graph_rounds < 0:
        args.graph_rounds = WORKLOADS[args.config].get("graph", 0)
    if args.graph_rounds > 0:
        # whole graphs only: the timed rounds and every batch are replays of one graph
        G = args.graph_rounds
        args.steps = -(-args.steps // G) * G
        args.batch_rounds = G
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 3}))
        return

    V, H, K = wl["V"], wl["H"], wl["K"]
    S = K + 1
    if not args.batch_rounds:
        args.batch_rounds = 8 if wl["layers"] else 64
    inp = build_inputs(wl, args, torch, sv, synth)
    wq, ws, hidden = inp["wq"], inp["ws"], inp["hidden"]
    copies = inp["copies"]
    decode = K == 0

    # device-resident round state
    total_rounds = args.warmup + args.steps + KERNEL_WARM + args.kernel_reps + 2 * args.batches * args.batch_rounds + 8
    cap = len(inp["ctx"]) + total_rounds * S + 2 * S
    tokens = torch.zeros(cap, dtype=torch.int32, device=dev)
    tokens[:len(inp["ctx"])] = torch.from_numpy(inp["ctx"]).to(dev)
    state = sv.new_state(dev)
    state[sv.STATE_LEN] = len(inp["ctx"])
    drafts = torch.empty(max(K, 1), dtype=torch.int32, device=dev)
    argmax = torch.empty(S, dtype=torch.int32, device=dev)
    temp = wl.get("temp")
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S) if temp else sv.verify_workspace_bytes(V, H, S), dev)
    work1 = sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev)

    table = window = rows = None
    if wl.get("model") == "table":
        # token-indexed stand-in model: hidden row of a window position = table[token]
        gen = torch.Generator(device=dev)
        gen.manual_seed(20261202 + wl["cid"] + (wl["seed"] << 16))
        table = torch.randn((V, H), generator=gen, device=dev, dtype=torch.float32).half()
        window = torch.empty((S, H), dtype=torch.float16, device=dev)
        h_last = torch.empty((1, H), dtype=torch.float16, device=dev)
        sv.gather_window(tokens, state, drafts[:0], table, h_last)      # the context's last token
    elif wl.get("model") == "script":
        # position-indexed stand-in: the window at stream length n is rows[n-1 .. n-1+K], picked on
        # the device from the state word (specverify_gather_positions, no host synchronisation)
        rows = inp["rows"]
        window = torch.empty((S, H), dtype=torch.float16, device=dev)
        h_last = rows[len(inp["ctx"]) - 1:len(inp["ctx"])].clone()
    else:
        h_last = torch.from_numpy(synth.fp16_normal(_streams(wl, synth).h_last, (1, H))).to(dev)

    def gather_script(stream=None):
        sv.gather_positions(state, cap, rows, window, stream=stream)

    # anchor bootstrap: S = 1 verify of the last context row, then accept with K = 0 commits a0
    a0 = torch.empty(1, dtype=torch.int32, device=dev)
    head_verify = sv.verify_q4 if wl.get("fmt") == "q4" else sv.verify
    ngram = wl["ngram"]
    sample_seed = wl["sample_seed"]
    # --logits: every timed round also writes the window's full fp32 logits [S][V]
    logits_buf = torch.empty((S, V), dtype=torch.float32, device=dev) if args.logits else None
    head_round = functools.partial(sv.round_q4 if wl.get("fmt") == "q4" else sv.round, ngram_max=ngram,
                                   logits=logits_buf)
    if temp:
        # sampling: the anchor is a draw from the last context row, a one-row sampling round
        lse0, zd0 = (torch.empty(1, dtype=torch.float32, device=dev) for _ in range(2))
        sv.verify_sample(wq[0], ws[0], h_last, None, temp, sample_seed, state, a0, lse0, zd0,
                         sv.workspace(sv.sample_workspace_bytes(V, H, 1), dev))
        sv.accept_sample(a0, lse0, zd0, None, V, sample_seed, tokens, state)

        def head_round(w_, s_, x_, d_in_, tokens_, state_, drafts_, argmax_, work_, stream=None):
            sv.round_sample(w_, s_, x_, d_in_, temp, sample_seed, tokens_, state_, drafts_, work_, ngram, argmax_,
                            stream=stream)
    else:
        head_verify(wq[0], ws[0], h_last, a0, work1)
        sv.accept(a0, None, tokens, state)

    forced = None
    if wl["drafts"] == "forced":
        # drafts that match the first j ~ U{0..K} greedy ids of each hidden set (setup, untimed)
        rng_d = np.random.default_rng(_streams(wl, synth).drafts)
        fd = np.empty((R_SETS, K), dtype=np.int32)
        gwork = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev)
        for r in range(R_SETS):
            head_verify(wq[0], ws[0], hidden[r], argmax, gwork)
            torch.cuda.synchronize()
            fd[r], _ = synth.forced_drafts(rng_d, argmax.cpu().numpy(), K, V)
        forced = torch.from_numpy(fd).to(dev)

    F = wl.get("F", 0)
    if wl["layers"]:
        nbuf = torch.empty((S, H), dtype=torch.float16, device=dev)
        xl_buf = torch.empty((wl["layers"], S, H), dtype=torch.float16, device=dev)
        swork = sv.workspace(sv.stack_forward_workspace_bytes(H, F, S), dev)
        nbuf1 = torch.empty((1, H), dtype=torch.float16, device=dev)
        xl_buf1 = torch.empty((wl["layers"], 1, H), dtype=torch.float16, device=dev)
        swork1 = sv.workspace(sv.stack_forward_workspace_bytes(H, F, 1), dev)

    # A round is verify -> accept -> propose (the next round's drafts), through the fused
    # entry point: one launch when the hidden axis needs no split.  The first drafts come
    # from a plain propose after the anchor bootstrap.
    tree = wl.get("tree")
    if tree:
        parents = torch.empty(K, dtype=torch.int32, device=dev)
        sv.propose_tree(tokens, state, parents, drafts, ngram, tree[0], tree[1])

        def head_round(w_, s_, x_, d_in_, tokens_, state_, drafts_, argmax_, work_, stream=None):
            sv.round_tree(w_, s_, x_, parents, d_in_, tokens_, state_, parents, drafts_, argmax_, work_, ngram,
                          tree[0], tree[1], logits=logits_buf, stream=stream)
    elif not decode:
        sv.propose(tokens, state, drafts, ngram)

    def round_(r, single=False):
        c = 0 if single else r % copies
        if decode:
            # a plain greedy step: one-row verify, the argmax committed as the next anchor
            head_verify(wq[c], ws[c], hidden[r % R_SETS][:1], a0, work1)
            sv.accept(a0, None, tokens, state)
            return
        if table is not None:
            # gather the window [a0, drafts] from the stand-in model, verify, accept, draft
            sv.generate(wq[c], ws[c], table, tokens, state, drafts, window, argmax, work, 1, ngram)
            return
        if rows is not None:
            gather_script()
            head_round(wq[c], ws[c], window, drafts, tokens, state, drafts, argmax, work)
            return
        if wl["layers"]:
            # the whole stack in one call (2 launches per block); the round's input rows stay
            # unchanged, block outputs go to a scratch [L, S, H]
            sv.stack(*inp["layers"], hidden[r % R_SETS], nbuf, swork, 1e-6, x_layers=xl_buf)
            x = nbuf
        else:
            x = hidden[r % R_SETS]
        d_in = forced[r % R_SETS] if forced is not None else drafts
        head_round(wq[c], ws[c], x, d_in, tokens, state, drafts, argmax, work)

    def verify_forward(r, rows_):
        """The verify forward alone at `rows_` window rows (the stack in front for the dense
        stack): the numerator and denominator of c_v(S)."""
        c = r % copies
        x = hidden[r % R_SETS][:rows_]
        if wl["layers"]:
            if rows_ == 1:
                sv.stack(*inp["layers"], x, nbuf1, swork1, 1e-6, x_layers=xl_buf1)
                x = nbuf1
            else:
                sv.stack(*inp["layers"], x, nbuf, swork, 1e-6, x_layers=xl_buf)
                x = nbuf
        head_verify(wq[c], ws[c], x, argmax[:rows_], work if rows_ > 1 else work1)

    def time_batches(fn, n, per):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for b in range(n):
            for i in range(per):
                fn(b * per + i)
            evs[b + 1].record()
        torch.cuda.synchronize()
        return [evs[b].elapsed_time(evs[b + 1]) for b in range(n)]

    for r in range(args.warmup):
        round_(r)
    torch.cuda.synchronize()
    graph = None
    if args.graph_rounds > 0:
        # G rounds captured once (nothing runs during capture; the round state lives on the
        # device, so every replay advances it by G rounds).  Round i of the graph uses hidden
        # set, forced drafts and weight copy number i, as eager round i would.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.graph_rounds):
                round_(i)
        torch.cuda.synchronize()
    st0 = state.cpu().numpy().copy()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    if graph is not None:
        for _ in range(args.steps // args.graph_rounds):
            graph.replay()
    else:
        for r in range(args.steps):
            round_(args.warmup + r)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    st1 = state.cpu().numpy()
    if st1[sv.STATE_FLAGS]:
        raise RuntimeError(f"device state flags {st1[sv.STATE_FLAGS]}")
    if decode:
        assert st1[sv.STATE_LEN] - st0[sv.STATE_LEN] == args.steps
        hist, sum_j = [args.steps], 0
    else:
        rounds = int(st1[sv.STATE_ROUNDS] - st0[sv.STATE_ROUNDS])
        assert rounds == args.steps
        hist = (st1[sv.STATE_HIST:sv.STATE_HIST + K + 1] - st0[sv.STATE_HIST:sv.STATE_HIST + K + 1]).tolist()
        sum_j = int(st1[sv.STATE_SUMJ] - st0[sv.STATE_SUMJ])

    # batches of rounds (median, IQR), rotated weights and one copy; c_v(S)
    base = args.warmup + args.steps
    if graph is not None:
        replay = lambda i: graph.replay() if i % args.graph_rounds == 0 else None
        batches = _batch_stats(time_batches(replay, args.batches, args.batch_rounds), args.batch_rounds)
    else:
        batches = _batch_stats(time_batches(lambda i: round_(base + i), args.batches, args.batch_rounds),
                               args.batch_rounds)
    single = None
    if copies > 1 and graph is not None:
        # the same rounds on one weight copy, from a graph of their own
        graph1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph1):
            for i in range(args.graph_rounds):
                round_(i, single=True)
        replay1 = lambda i: graph1.replay() if i % args.graph_rounds == 0 else None
        single = _batch_stats(time_batches(replay1, args.batches, args.batch_rounds), args.batch_rounds)
    elif copies > 1:
        single = _batch_stats(time_batches(lambda i: round_(base + i, single=True), args.batches, args.batch_rounds),
                              args.batch_rounds)
    cv = None
    if not temp and not tree:
        t_s = time_batches(lambda i: verify_forward(i, S), args.batches, args.batch_rounds)
        t_1 = time_batches(lambda i: verify_forward(i, 1), args.batches, args.batch_rounds)
        us_s = 1000.0 * float(np.median(t_s)) / args.batch_rounds
        us_1 = 1000.0 * float(np.median(t_1)) / args.batch_rounds
        cv = {"S": S, "us_verify_S": round(us_s, 3), "us_verify_1": round(us_1, 3), "c_v": round(us_s / us_1, 4),
              "note": "median over batches of the verify forward alone (matmul and argmax"
                      + (", with the dense stack in front" if wl["layers"] else "") + ") at S rows and at one row"}
    st2 = state.cpu().numpy()
    if st2[sv.STATE_FLAGS]:
        raise RuntimeError(f"device state flags {st2[sv.STATE_FLAGS]}")

    # roofline of the dominant kernel: the head matmul with its fused argmax (or sampling)
    # stage 1, or for the dense stack its gate/up projection (block 0 of a whole-stack call;
    # every block's gate/up moves the same bytes).  Calls are launched one by one, with HIP
    # events recorded by the library on the launch stream right before and after the kernel.
    # About 60 ms of untimed calls (100 .. KERNEL_WARM) come first: the GPU clocks down
    # whenever it idles (the host synchronisation just before is enough), and a head launched
    # within the first milliseconds of load after that runs 4-15% slower than under sustained
    # load (measured: 84 and 221 us after 2 s idle against 81 and 191 us at H = 2048 and 5120).
    # The events are created beforehand so that the calls follow each other with no host-side
    # gap.
    warm = min(KERNEL_WARM, max(100, int(60.0 / ms)))
    stream = torch.cuda.current_stream()
    durs = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.kernel_reps)]
    for i in range(warm + args.kernel_reps):
        x, c = hidden[i % R_SETS], i % copies
        d_in = forced[i % R_SETS] if forced is not None else drafts
        if i >= warm:
            e0, e1 = evs[i - warm]
            sv.profile_next_matmul(e0, e1, stream=stream)
        if wl["layers"]:
            sv.stack(*inp["layers"], x, nbuf, swork, 1e-6, x_layers=xl_buf, stream=stream)
        elif decode:
            head_verify(wq[c], ws[c], x[:1], a0, work1, stream=stream)
        elif table is not None:
            sv.generate(wq[c], ws[c], table, tokens, state, drafts, window, argmax, work, 1, ngram, stream=stream)
        elif rows is not None:
            gather_script(stream)
            head_round(wq[c], ws[c], window, drafts, tokens, state, drafts, argmax, work, stream=stream)
        else:
            head_round(wq[c], ws[c], x, d_in, tokens, state, drafts, argmax, work, stream=stream)
        if i >= warm:
            durs.append((e0, e1))
    torch.cuda.synchronize()
    kern_all = np.array([a.elapsed_time(b) for a, b in durs])
    kern_ms = float(np.mean(kern_all))
    hb = head_bytes(V, H, S, wl.get("fmt", "q8"))
    kb = gateup_bytes(H, F, S) if wl["layers"] else hb
    achieved = kb / (kern_ms * 1e-3) / 1e9

    round_bytes = hb + (stack_bytes(wl["layers"], H, F, S) if wl["layers"] else 0)
    rps = 1000.0 / ms
    gbps = round_bytes * rps / 1e9
    out = {
        "metric": METRIC,
        "value": round(rps, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i4xf16->f32" if wl.get("fmt") == "q4" else "i8xf16->f32",
        "data": "synthetic",
        "config": {"workload": wl["name"], "V": V, "H": H, "S": S, "K": K, "layers": wl["layers"],
                   "drafts": wl["drafts"], "ngram_max": ngram, "seed": wl["seed"], "weight_copies": copies,
                   "hidden_sets": R_SETS},
        "achieved_GBps": round(gbps, 1),
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "bytes_per_round": round_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": load_traffic(args.config) if wl["K"] == WORKLOADS[args.config]["K"] else None,
                     "kernel": (f"q8b32 gate/up projection of the dense stack with the RMSNorm in its prologue "
                                f"and the SiLU-mul epilogue ({wl['layers']} launches per round, block 0 timed)"
                                if wl["layers"] else
                                ("q4b32" if wl.get("fmt") == "q4" else "q8b32")
                                + (" head matmul with the fused sampling epilogue (log-sum-exp, Gumbel-max "
                                   "draw) stage 1 (one launch per round)" if temp else
                                   " head matmul with the fused argmax stage 1 (one launch per round)")),
                     "kernel_ms": round(kern_ms, 5), "algorithmic_bytes_per_launch": kb,
                     "kernel_ms_median": round(float(np.median(kern_all)), 5),
                     "kernel_ms_p10_p90": [round(float(np.percentile(kern_all, 10)), 5),
                                           round(float(np.percentile(kern_all, 90)), 5)],
                     "launches_timed": int(kern_all.size), "untimed_calls_before": warm},
        "batches": dict(batches, weight_copies=copies,
                        pct_of_peak_hbm=round(100.0 * round_bytes * batches["median_rounds_per_s"] / 1e9
                                              / PEAK_HBM_GBPS, 2)),
        "accept_hist": hist,
        # the share of rounds that accepted at least one draft (the zero-accept rounds are what
        # the hit-rate gate counts)
        "draft_hit_rate": round(1.0 - hist[0] / max(1, sum(hist)), 4) if not decode else None,
        "tokens_per_round": round((args.steps + sum_j) / args.steps, 3),
    }
    if single is not None:
        out["batches_single_copy"] = dict(single, weight_copies=1, note="the same rounds on one weight copy, which "
                                          "the 256 MB Infinity Cache can partly serve across rounds")
    if cv is not None:
        out["c_v"] = cv
    if tree:
        out["config"]["tree"] = {"branches": tree[0], "depth": tree[1], "nodes": K}
    if args.logits:
        out["config"]["logits"] = "fp32 [S][V] written every round"
        out["bytes_per_round_with_logits"] = round_bytes + 4 * S * V
    if wl["layers"] and args.down_split:
        out["config"]["down_split"] = args.down_split
    if args.graph_rounds > 0:
        out["config"]["graph_rounds"] = args.graph_rounds
    if temp:
        out["config"]["temperature"] = temp
        out["config"]["sample_seed"] = sample_seed
    if inp["copy_frac"] is not None:
        out["config"]["context_copy_fraction"] = round(inp["copy_frac"], 3)
    if table is not None or rows is not None:
        # tokens/s accounting against the feasibility page's C-value model: with each draft
        # accepted independently with probability alpha, a round commits
        # E(alpha, K) = (1 - alpha^(K+1)) / (1 - alpha) tokens; alpha estimated from the
        # accept histogram (maximum likelihood: sum j / (sum j + rounds with j < K))
        stops = sum(hist[:K])
        alpha = sum_j / (sum_j + stops) if sum_j + stops else 0.0
        e_model = float(K + 1) if alpha >= 1.0 else (1.0 - alpha ** (K + 1)) / (1.0 - alpha)
        out["tokens_per_second"] = round(rps * (args.steps + sum_j) / args.steps, 1)
        out["alpha_hat"] = round(alpha, 4)
        out["expected_tokens_per_round"] = round(e_model, 3)
        out["gated_at_round"] = int(st1[sv.STATE_GATED])
    if rows is not None:
        n = int(st2[sv.STATE_LEN])
        out["script_reproduced"] = bool(np.array_equal(tokens[:n].cpu().numpy(), inp["script"][:n]))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, table)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
