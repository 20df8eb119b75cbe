#!/usr/bin/env python3
"""LoopVQ hot-path benchmark on one MI355X.

Headline: decode attention over the coded KV cache of an Ouro-1.4B-shaped
looped model (24 layers, 4 loop steps per token, 16 KV heads, d = 128, Tc = 4,
G = 32 -> 0.25 bit per element, 8 sequences of 32768 tokens, 4 sink + 64
recent tokens in bf16, shuffled 8-token pages).  One step = one decode token:
the 96 (loop step, layer) attention calls in model order (loop step outer,
layer inner), each layer with its own index pool, bf16 pool and codebooks, so
the 3.2 GB of coded pages stream from HBM (well beyond the 256 MB
Infinity Cache).  Metric: KV token-steps/s = 96 * sum_b L_b / step time.

Inputs are synthetic (seeded AR(1) loop-correlated keys/values, k-means
codebooks), generated on the GPU and prefill-encoded by the library's own
encoder before timing.  The JSON line also carries the roofline of the
attention call (float32 vector arithmetic binds it; its HBM fraction is reported
beside), the CPU oracle timed on a bounded sample, and the prefill
encoder's throughput (vectors/s, MFMA utilisation) on the 32768-token shape.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VQ decode attn: KV token-steps/s & % HBM peak at 32K; encode vectors/s"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3          # published; counts packed float32 (two lanes per op)
FP32_VECTOR_UNPACKED_TFLOPS = 78.6       # 256 CUs x 64 lanes x 2 flops (FMA) x 2.4 GHz

# Ouro-1.4B-shaped decode configuration
B, L, H, D, T, TC, G = 8, 32768, 16, 128, 4, 4, 32
N_SINK, N_RECENT = 4, 64
CONFIG_ID = 2
CALIB_BYTES = 1 << 30          # calibration copy for the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_ouro_b8_l32k_traffic.txt")
KSTATS_FILE = os.path.join(ROOT, "profiles", "decode_attn_ouro_b8_l32k_kernel_stats.txt")
ATTN_SOURCES = [os.path.join(ROOT, "sub_bit_loop_amd", "csrc", f)
                for f in ("lvq_attn.hip", "lvq_attn_common.h", "lvq_internal.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--splits", type=int, default=0, help="waves per query head of the decode call (the n_splits of its shape); 0 = automatic")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-encode", action="store_true", help="skip the encoder measurement")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the decode-attention measurement (for counter runs): no HBM probe, "
                         "multi-row, cache-manager or encoder legs")
    ap.add_argument("--encode-only", action="store_true",
                    help="only the encoder measurement (for counter runs): prints its JSON object")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="wall-time bound of the CPU oracle baseline")
    ap.add_argument("--pmc-instructions", metavar="DIR",
                    help="summarise a rocprofv3 --pmc run of the SQ instruction counters of this bench "
                         "into the instruction record the bench line reports")
    ap.add_argument("--kernel-stats-summary", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run of the headline measurement "
                         "into the kernel-time record the bench line reports")
    ap.add_argument("--cpu-worker", metavar="DIR", help=argparse.SUPPRESS)
    ap.add_argument("--cpu-cores", type=int, default=0,
                    help="worker processes of the CPU oracle baseline (0 = the host's cores, at most 16)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench "
                         "into the HBM-traffic record the bench line reports")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_inputs(args, torch, lvq, synth):
    import numpy as np
    dev = torch.device("cuda:0")
    c = G // TC
    nblk, ng = T // TC, D // c
    q_end = synth.prefill_q_end(L, N_RECENT)
    n_coded_pages = q_end // 8
    max_pages = L // 8
    # shuffled page table over the pool (the same placement for every layer; each layer owns a pool)
    rng = np.random.default_rng(synth.seed_for(CONFIG_ID, synth.STREAM_PAGES))
    pt_np, pool = synth.shuffled_page_table(rng, [n_coded_pages] * B, max_pages)
    pt = torch.from_numpy(pt_np).to(dev)
    # one spare coded page per sequence receives the decode-time re-encode of its oldest
    # recent page (the attention inputs stay those of the 32768-token state)
    spare = torch.arange(pool, pool + B, dtype=torch.int32, device=dev)
    pool += B
    # codebooks: built on the device (k-means++ and 10 Lloyd iterations on 4096 seeded
    # samples per book) for one layer, copied into every layer's buffer
    rk = np.random.default_rng(synth.seed_for(CONFIG_ID, synth.STREAM_K))
    rv = np.random.default_rng(synth.seed_for(CONFIG_ID, synth.STREAM_V))
    sc_k, sc_v = synth.channel_scales(rk, H, D), synth.channel_scales(rv, H, D)
    cb0, build_s = build_books(torch, lvq, synth, TC, G, sc_k, sc_v, synth.seed_for(CONFIG_ID, synth.STREAM_BOOKS))
    log(f"codebooks (2 x {H * (D // (G // TC)) * (T // TC)} books) built on the device in {build_s * 1e3:.1f} ms")
    # bf16 pool: per sequence the copy of page 0 and the recent pages
    n_recent_pages = (L - q_end + 7) // 8
    bf16_row = 1 + n_recent_pages
    n_bf16 = B * bf16_row
    bt = torch.arange(n_bf16, dtype=torch.int32, device=dev).view(B, bf16_row)
    gen = torch.Generator(device=dev)
    layers = []
    t0 = time.time()
    for layer in range(args.layers):
        ip = torch.zeros((pool, nblk, H, 2, 8, ng), dtype=torch.uint8, device=dev)
        bp = torch.zeros((n_bf16, T, H, 2, 8, D), dtype=torch.bfloat16, device=dev)
        for b in range(B):
            for kv in (0, 1):
                gen.manual_seed(synth.seed_for(CONFIG_ID, kv) * 1009 + 97 * layer + b)
                x = synth.gen_kv_torch(gen, T, L, H, D, sc_k if kv == 0 else sc_v, device=dev)
                chunk_page = pt[b, :n_coded_pages].contiguous()
                lvq.lvq_encode_pages(x[:, :q_end].contiguous(), cb0, kv, T, TC, G, chunk_page, ip)
                # page 0 copy (sink tokens) and recent pages [q_end, L)
                bp[b * bf16_row, :, :, kv] = x[:, 0:8].permute(0, 2, 1, 3)
                rec = x[:, q_end:L].reshape(T, n_recent_pages, 8, H, D).permute(1, 0, 3, 2, 4)
                bp[b * bf16_row + 1:(b + 1) * bf16_row, :, :, kv] = rec
                del x
        cb = cb0.clone()
        qs = []
        for t in range(T):
            gen.manual_seed(synth.seed_for(CONFIG_ID, synth.STREAM_Q) * 1009 + 97 * layer + t)
            qs.append(synth.gen_queries_torch(gen, B, H, D, device=dev))
        layers.append(dict(ip=ip, bp=bp.view(torch.int16), cb=cb, q=qs))
    torch.cuda.synchronize()
    log(f"{args.layers} layers generated and prefill-encoded in {time.time() - t0:.1f}s")
    pos = torch.full((B,), L, dtype=torch.int32, device=dev)
    seq_len = torch.full((B,), L, dtype=torch.int32, device=dev)
    qe = torch.full((B,), q_end, dtype=torch.int32, device=dev)
    rope = lvq.lvq_rope_tables(L + 1, D, 10000.0, device=dev)
    shp = lvq.make_shape(B, H, H, D, T, TC, G, N_SINK, max_pages, bf16_row, pool, n_bf16, L, L + 1,
                         args.splits)
    ws = torch.empty(lvq.lvq_decode_attn_workspace_bytes(shp), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    # a plain device copy of known size: the scale of the rocprofv3 byte counters
    calib = torch.empty(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    torch.empty_like(calib).copy_(calib)
    torch.cuda.synchronize()
    del calib
    return dict(pt=pt, pt_np=pt_np, layers=layers, pos=pos, seq_len=seq_len, qe=qe, rope=rope,
                shp=shp, ws=ws, out=out, lse=lse, bt=bt, pool=pool, q_end=q_end, bf16_row=bf16_row,
                cb0=cb0, build_s=build_s, spare=spare)


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _pmc_per_dispatch(directory, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 --pmc csv run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in vals.items():
        out.setdefault(name, []).append(v)
    return out


def pmc_summary(fetch_dir, write_dir):
    """HBM bytes per decode-attention call from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the counter reads for the bench's calibration copy of CALIB_BYTES."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")

    def calib(d):
        cands = [max(v) for k, v in d.items() if "copy" in k.lower()]
        return max(cands) * 1024.0 if cands else float("nan")

    def per_launch(d, key):
        v = [x for k, xs in d.items() if key in k for x in xs]
        return (sum(v) / len(v) * 1024.0, len(v)) if v else (float("nan"), 0)

    cf, cw = calib(fetch), calib(write)
    sf, sw = CALIB_BYTES / cf, CALIB_BYTES / cw
    af, na = per_launch(fetch, "attn_kernel<128, 8, false")
    aw, _ = per_launch(write, "attn_kernel<128, 8, false")
    mf, nm = per_launch(fetch, "merge_kernel")
    mw, _ = per_launch(write, "merge_kernel")
    traffic = (af + mf) * sf + (aw + mw) * sw
    algo = algorithmic_bytes_per_call(synth_q_end())
    print("# HBM traffic of one decode-attention call (attn_kernel<128, 8, false, false> + merge_kernel),")
    print("# Ouro-1.4B-shaped 32K decode bench\n")
    print("Commands (repository root $REPO on the GPU host):\n")
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        print(f"    cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv "
              f"-d {d} -o bench -- python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu --headline-only")
    print(f"    python3 $REPO/bench.py --pmc-summary {fetch_dir} {write_dir}\n")
    print(f"source_sha256: {attn_source_hash()}")
    print(f"calibration_copy_bytes: {CALIB_BYTES}")
    print(f"calibration_fetch_counter_bytes: {cf:.0f}  (scale {sf:.4f})")
    print(f"calibration_write_counter_bytes: {cw:.0f}  (scale {sw:.4f})")
    print(f"attn_kernel dispatches {na}: FETCH_SIZE {af / 1024:.1f} KiB, WRITE_SIZE {aw / 1024:.1f} KiB per dispatch")
    print(f"merge_kernel dispatches {nm}: FETCH_SIZE {mf / 1024:.1f} KiB, WRITE_SIZE {mw / 1024:.1f} KiB per dispatch")
    print(f"algorithmic_bytes_per_call: {algo}")
    print(f"traffic_bytes_per_call: {traffic:.0f}")
    print(f"traffic_over_algorithmic: {traffic / algo:.3f}")


INSTR_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                          "decode_attn_ouro_b8_l32k_instructions.txt")
INSTR_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_LDS_BANK_CONFLICT")
SIMDS, CLOCK_GHZ, VALU_CYCLES = 256 * 4, 2.4, 4   # a wave64 VALU instruction holds a 16-lane SIMD 4 cycles


def pmc_instructions(directory):
    """Instruction counts per decode-attention call (attn_kernel + merge_kernel) from a
    rocprofv3 --pmc run of SQ counters, and the VALU issue time they imply."""
    per = {}
    for c in INSTR_COUNTERS:
        d = _pmc_per_dispatch(directory, c)
        tot = 0.0
        for key in ("attn_kernel<128, 8, false", "merge_kernel"):
            v = [x for k, xs in d.items() if key in k for x in xs]
            tot += sum(v) / len(v) if v else float("nan")
        per[c] = tot
    valu = per["SQ_INSTS_VALU"] - per["SQ_INSTS_MFMA"]
    bound_us = valu * VALU_CYCLES / SIMDS / (CLOCK_GHZ * 1e3)
    print("# Instruction counts of one decode-attention call (attn_kernel<128, 8, false, false> + merge_kernel),")
    print("# Ouro-1.4B-shaped 32K decode bench\n")
    print("Command (repository root $REPO on the GPU host):\n")
    print(f"    cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {' '.join(INSTR_COUNTERS)} --output-format csv "
          f"-d {directory} -o bench -- python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu --headline-only")
    print(f"    python3 $REPO/bench.py --pmc-instructions {directory}\n")
    print(f"source_sha256: {attn_source_hash()}")
    for c in INSTR_COUNTERS:
        print(f"{c.lower()}_per_call: {per[c]:.0f}")
    print(f"valu_instructions_per_call: {valu:.0f}")
    print(f"valu_issue_bound_us: {bound_us:.2f}  ({SIMDS} SIMDs, {VALU_CYCLES} cycles per wave64 VALU "
          f"instruction, {CLOCK_GHZ} GHz)")


def recorded_instructions():
    """VALU issue bound per call (us) from the committed record, or None if stale."""
    try:
        text = open(INSTR_FILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith(" "))
    if fields.get("source_sha256", "").strip() != attn_source_hash():
        return None
    try:
        return float(fields["valu_issue_bound_us"].split()[0])
    except (KeyError, ValueError):
        return None


def recorded_traffic():
    """Traffic per call from the committed counter record, or None if the kernel changed since."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith(" "))
    if fields.get("source_sha256", "").strip() != attn_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_call"].split()[0])
    except (KeyError, ValueError):
        return None


def synth_q_end():
    return 8 * ((L - N_RECENT) // 8)


def algorithmic_bytes_per_call(q_end):
    """Bytes the method must move per (layer, step) call: index rows of coded tokens,
    bf16 sink/recent tokens, the step-t codebook slices once, query, output, page ids."""
    coded = q_end - N_SINK
    idx = B * coded * H * (2 * (D // (G // TC)))
    bf = B * (N_SINK + (L - q_end)) * H * 2 * D * 2
    books = H * 2 * 256 * D * 2
    small = B * H * D * 2 + B * H * D * 4 + B * H * 4 + B * (q_end // 8) * 4
    return idx + bf + books + small


def algorithmic_flops_per_call():
    """Float32 work the method must do per (layer, step) call: for every cached (token,
    head), the rotation of the key's d/2 channel pairs (4 products and 2 sums per pair),
    the scaled dot product with the rotated query (2 per channel) and the value sum
    (2 per channel): 7 d flops.  Coded and bf16 tokens cost the same."""
    return B * H * L * 7 * D


# Float32 lane operations that exact attention over the coded cache needs per cached
# (token, head): the rotated score takes 6 operations per channel pair (the key pair
# times the query-side phase coefficients) and the value sum one FMA per channel.
VALU_OPS_PER_TOKEN_HEAD = 6 * (D // 2) + D
LANE_OPS_PER_S = 256 * 64 * CLOCK_GHZ * 1e9    # non-packed float32: 64 lanes per CU per clock


def valu_floor_us():
    """Time of the essential float32 lane operations of one call at the non-packed rate."""
    return B * H * L * VALU_OPS_PER_TOKEN_HEAD / LANE_OPS_PER_S * 1e6


def recorded_kernel_us():
    """attn_kernel + merge_kernel average (us) from the committed rocprofv3 statistics
    record, or None if the attention sources changed since it was taken."""
    try:
        text = open(KSTATS_FILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith(" "))
    if fields.get("source_sha256", "").strip() != attn_source_hash():
        return None
    try:
        return float(fields["call_kernel_us"].split()[0])
    except (KeyError, ValueError):
        return None


def kernel_stats_summary(directory):
    """The library's kernels in a rocprofv3 --kernel-trace --stats csv run of the headline
    measurement, and the average kernel time of one decode call (attention + merge)."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    lib = ("attn_kernel", "attn_group_kernel", "merge_kernel", "encode_kernel", "seed_kernel", "update_kernel", "round_kernel",
           "rope_kernel", "rows_kernel", "cache_")
    out = []
    for r in rows:
        name = r["Name"]
        if not any(k in name for k in lib):
            continue
        short = name.replace("lvq::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        out.append((short, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3, float(r.get("StdDev", 0) or 0) / 1e3))
    out.sort(key=lambda x: -x[1] * x[2])
    attn = [x for x in out if x[0].startswith("attn_kernel<128, 8, false")]
    merge = [x for x in out if x[0].startswith("merge_kernel")]
    call_us = (sum(x[1] * x[2] for x in attn) / max(1, sum(x[1] for x in attn)) +
               sum(x[1] * x[2] for x in merge) / max(1, sum(x[1] for x in merge)))
    print("# Kernels of the Ouro-1.4B-shaped 32K decode bench (headline measurement only)\n")
    print("Command (repository root $REPO on the GPU host):\n")
    print(f"    cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
          f"-d {directory} -o bench -- python3 $REPO/bench.py --no-cpu --headline-only")
    print(f"    python3 $REPO/bench.py --kernel-stats-summary {directory}\n")
    print(f"source_sha256: {attn_source_hash()}")
    print(f"call_kernel_us: {call_us:.2f}  (attn_kernel + merge_kernel averages)")
    print(f"algorithmic_bytes_per_call: {algorithmic_bytes_per_call(synth_q_end())}\n")
    print(f"{'kernel':<62}{'calls':>7}{'avg_us':>10}{'min_us':>10}{'max_us':>10}{'stddev_us':>10}")
    for n, c, a, lo, hi, sd in out:
        print(f"{n[:61]:<62}{c:>7}{a:>10.2f}{lo:>10.2f}{hi:>10.2f}{sd:>10.2f}")


N_BOOK_SAMPLES, N_LLOYD = 4096, 10


def build_books(torch, lvq, synth, tc, g, sc_k, sc_v, seed):
    """K and V codebooks of one layer with lvq_build_codebooks: 4096 seeded sample tokens of
    the AR(1) generator, k-means++ draws from a seeded device generator, 10 Lloyd iterations.
    Returns (codebook bits as int16 [nblk][2][H][ng][Tc][256][c], seconds of the two builds)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    c = g // tc
    nblk, ng = T // tc, D // c
    cb = torch.zeros((nblk, 2, H, ng, tc, 256, c), dtype=torch.bfloat16, device=dev)
    samples, draws = [], []
    for kv, sc in ((0, sc_k), (1, sc_v)):
        gen.manual_seed(seed * 7 + kv)
        samples.append(synth.gen_kv_torch(gen, T, N_BOOK_SAMPLES, H, D, sc, device=dev))
        draws.append(torch.rand((nblk, H, ng, 256), generator=gen, dtype=torch.float64, device=dev))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for kv in (0, 1):
        lvq.lvq_build_codebooks(samples[kv], draws[kv], kv, T, tc, g, N_LLOYD, codebooks=cb)
    e1.record()
    torch.cuda.synchronize()
    return cb.view(torch.int16), e0.elapsed_time(e1) * 1e-3


def run_decode(args, torch, lvq, inp):
    layers = inp["layers"]
    common = dict(pos=inp["pos"], seq_len=inp["seq_len"], q_end=inp["qe"], rope_tab=inp["rope"],
                  shp=inp["shp"], out=inp["out"], lse=inp["lse"], ws=inp["ws"])

    def call(layer, t):
        Ly = layers[layer]
        lvq.lvq_decode_attn(Ly["q"][t], inp["pt"], Ly["ip"], Ly["bp"], inp["bt"], Ly["cb"], t,
                            common["pos"], common["seq_len"], common["q_end"], common["rope_tab"],
                            common["shp"], common["out"], common["lse"], common["ws"])

    # After a token's forward pass, every 8 tokens each sequence encodes its oldest recent
    # page (all loop steps, heads, K and V) in every layer; with 8 sequences that is one
    # sequence's page per step on average: step s re-encodes sequence s mod B.
    pools = [(Ly["bp"], Ly["cb"], Ly["ip"]) for Ly in layers]

    def reencode(s_idx):
        b = s_idx % B
        src = inp["bt"][b, 1:2].contiguous()
        dst = inp["spare"][b:b + 1].contiguous()
        lvq.lvq_reencode_pages_layers(pools, src, dst, T, TC, G)   # every layer, one launch

    # An event pair around a call costs about 5 us of queue time at each of its two ends, so
    # timing all 96 calls would add about 1 ms to a 10 ms step.  Each step times one call per
    # loop step instead: the call of layer (s mod layers) at every t, so the steps together
    # sample every (layer, loop step) position once per 24 steps.
    def sampled(s_idx):
        return {t * len(layers) + s_idx % len(layers) for t in range(T)}

    def step(s_idx, events=None):
        k = 0
        for t in range(T):
            for layer in range(len(layers)):
                ev = events.get(k) if events is not None else None
                if ev is not None:
                    ev[0].record()
                call(layer, t)
                if ev is not None:
                    ev[1].record()
                k += 1
        reencode(s_idx)

    for w in range(args.warmup):
        step(w)
    torch.cuda.synchronize()
    evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in sampled(s)}
           for s in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = [a.elapsed_time(b) * 1e-3 for e in evs for a, b in e.values()]
    return wall, per_call


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_cores(asked=0):
    """Worker processes for the CPU baseline: the cores this process may run on, at most 16
    (the host share of one GPU)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    n = min(n, 16)
    return max(1, min(asked, n) if asked > 0 else n)


def _oracle_pairs(job):
    """Worker: the oracle on a list of (b, head) pairs of the saved call; returns the count."""
    directory, pairs = job
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import lvq_oracle as orc
    z = {k: np.load(os.path.join(directory, k + ".npy"), mmap_mode="r") for k in
         ("ip", "bp", "cb", "q", "pt", "bt", "pos", "qe", "meta")}
    Bm, Hm, Dm, Tm, TCm, Gm, NS, t = (int(x) for x in z["meta"])
    shp = orc.AttnShape(Bm, Hm, Hm, Dm, Tm, TCm, Gm, NS)
    with threadpool_limits(limits=1):
        orc.decode_attn(shp, np.asarray(z["q"]), z["pt"], z["ip"], z["bp"], z["bt"], np.asarray(z["cb"]), t,
                        np.asarray(z["pos"]), np.asarray(z["pos"]), np.asarray(z["qe"]), pairs=pairs)
    return len(pairs)


def cpu_worker(directory, cores, seconds):
    """Runs in a child process that never touches the GPU: the oracle over every (b, head)
    pair of the saved call, one pair per task, on `cores` forked worker processes; pairs
    not started within `seconds` are skipped.  Returns the pairs done and the wall time."""
    import multiprocessing as mp
    import numpy as np
    meta = np.load(os.path.join(directory, "meta.npy"))
    Bm, Hm = int(meta[0]), int(meta[1])
    pairs = [(b, h) for h in range(Hm) for b in range(Bm)]
    n = host_cores(cores)
    done = 0
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        pending = [pool.apply_async(_oracle_pairs, ((directory, [p]),)) for p in pairs]
        for r in pending:
            left = seconds - (time.perf_counter() - t0)
            if left <= 0:
                break
            try:
                done += r.get(timeout=left)
            except mp.TimeoutError:
                break
        el = time.perf_counter() - t0
        pool.terminate()
    return {"pairs": done, "of": len(pairs), "seconds": el, "cores": n}


def cpu_baseline(args, torch, inp):
    """The float64 oracle on a bounded sample of the same workload: the (b, head) pairs of
    one (layer 0, loop step 1) call at full context, spread over the host's cores.  The
    oracle runs in a child process (and its forked workers) that never touches the GPU;
    the call's inputs reach it through .npy files."""
    import shutil
    import subprocess
    import tempfile
    import numpy as np
    Ly = inp["layers"][0]
    t = 1
    d = tempfile.mkdtemp(prefix="lvq_cpu_")
    try:
        arrays = dict(
            ip=Ly["ip"].cpu().numpy(), bp=Ly["bp"].cpu().numpy().view(np.uint16),
            cb=Ly["cb"].cpu().numpy().view(np.uint16),
            q=Ly["q"][t].cpu().view(torch.int16).numpy().view(np.uint16),
            pt=inp["pt_np"], bt=inp["bt"].cpu().numpy(), pos=np.full(B, L), qe=np.full(B, inp["q_end"]),
            meta=np.array([B, H, D, T, TC, G, N_SINK, t]))
        for k, v in arrays.items():
            np.save(os.path.join(d, k + ".npy"), np.ascontiguousarray(v))
        cmd = [sys.executable, os.path.abspath(__file__), "--cpu-worker", d, "--cpu-cores", str(args.cpu_cores),
               "--cpu-seconds", str(args.cpu_seconds)]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=args.cpu_seconds + 120)
        if r.returncode != 0:
            return {"error": r.stderr[-2000:]}
        w = json.loads(r.stdout.strip().splitlines()[-1])
    finally:
        shutil.rmtree(d, ignore_errors=True)
    # one (b, head) pair over L tokens is L/H token-steps of the all-head metric
    value = w["pairs"] * L / H / w["seconds"]
    return {"value": value, "unit": "KV token-steps/s", "cores": w["cores"], "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{w['pairs']} of the {w['of']} (sequence, head) pairs of one (layer, loop step) call "
                      f"at L={L} (float64 numpy oracle, one pair per task, {w['cores']} worker processes of "
                      f"one thread each, {w['seconds']:.1f}s wall); not extrapolated: the value is the "
                      f"sample's own rate"}


def manager_bench(torch, lvq, inp, n_tokens=64):
    """The paged cache manager through the decode loop of the same model shape: per token,
    begin_token, one append per (loop step, layer) of the new token's K/V, end_token, the
    re-encode of every due page in every layer, commit.  The sequences start at 32768
    tokens (pages allocated by the manager's prefill); attention is timed by the main loop
    and left out here.  Returns microseconds per token, whole and bookkeeping only."""
    dev = torch.device("cuda:0")
    c = G // TC
    nblk, ng = T // TC, D // c
    max_pages = (L + 4 * n_tokens) // 8 + 4          # three timed runs and their warm-up tokens
    n_index = B * max_pages
    cache = lvq.PagedCache(B, max_pages, N_SINK, N_RECENT, n_index, B * 12)
    cache.prefill(torch.full((B,), L, dtype=torch.int32, device=dev))
    nl = len(inp["layers"])
    ips = [torch.zeros((n_index, nblk, H, 2, 8, ng), dtype=torch.uint8, device=dev) for _ in range(nl)]
    bps = [torch.zeros((B * 12, T, H, 2, 8, D), dtype=torch.bfloat16, device=dev) for _ in range(nl)]
    pools = [(bps[layer], inp["layers"][layer]["cb"], ips[layer]) for layer in range(nl)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    kv = [torch.randn((2, 1, B, H, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(4)]

    def token(i, reencode=True):
        cache.begin_token()
        for t in range(T):
            for layer in range(nl):
                k = kv[(t + layer) % 4]
                cache.append(t, k[0], k[1], bps[layer])
        cache.end_token()
        if reencode:
            lvq.lvq_reencode_pages_layers(pools, cache.re_src, cache.re_dst, T, TC, G)
        cache.commit()

    res = {}
    for name, reenc in (("us_per_token", True), ("us_per_token_bookkeeping", False)):
        token(0, reenc)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_tokens):
            token(i, reenc)
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / n_tokens, 2)
    # the whole token holds no host decision, so it replays as one captured graph
    token(0)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        token(0)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_tokens):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    res["us_per_token_graph"] = round(e0.elapsed_time(e1) * 1e3 / n_tokens, 2)
    if cache.errors():
        raise RuntimeError(f"cache manager error bits {cache.errors()}")
    res["workload"] = (f"B={B} sequences from L={L}, {n_tokens} decode tokens, {nl} layers x {T} loop steps: "
                       f"begin, {nl * T} appends, end, re-encode of due pages in every layer, commit "
                       f"(8 pages x {nl} layers every 8 tokens)")
    return res


FP32_MFMA_PEAK_TFLOPS = 157.3
F16_MFMA_PEAK_TFLOPS = 2500.0   # dense float16 matrix peak


def _event_time(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def rows_bench(torch, lvq, inp, nq=512):
    """Multi-row attention at the model shape.
    prefill: nq new tokens of sequence 0 over its 32768-token coded prefix (layer 0, loop
      step 1, 16 heads), causal within the chunk; algorithmic flops 4 d per (query, visible
      key) per head at float32 precision, set against the fp32 matrix peak.  The coded
      tiles execute them as float16 hi/lo products (10 d per pair: three score and two
      value products), the bf16 tiles on fp32 matrix cores; those executed matrix flops are
      reported beside it.  Context: the same attention in bf16 with torch matmuls on dense
      K/V (not the path).
    gqa: decode over 8 x 32768 tokens with 16 query heads over 4, 2 and 1 KV heads:
      lvq_decode_attn (the grouped kernel at 4 heads per KV head, the multi-row kernel at 8
      and 16) and the multi-row kernel against the per-head kernel on the same cache."""
    dev = torch.device("cuda:0")
    Ly = inp["layers"][0]
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    res = {}
    # ---- prefill chunk
    rope = lvq.lvq_rope_tables(L + nq + 1, D, 10000.0, device=dev)
    q = torch.randn((1, nq, H, D), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((1, nq, H, D), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((1, nq, H, D), generator=gen, device=dev).to(torch.bfloat16)
    one = lambda v: torch.full((1,), v, dtype=torch.int32, device=dev)
    shp = lvq.make_rows_shape(1, nq, H, H, D, T, TC, G, N_SINK, inp["pt"].shape[1], inp["bf16_row"], inp["pool"],
                              inp["bf16_row"] * B, L, L + nq + 1)
    ws = torch.empty(lvq.lvq_rows_attn_workspace_bytes(shp), dtype=torch.uint8, device=dev)
    out = torch.empty((1, nq, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, nq, H), dtype=torch.float32, device=dev)
    pt0, bt0, pl, qe0 = inp["pt"][0:1].contiguous(), inp["bt"][0:1].contiguous(), one(L), one(inp["q_end"])
    run = lambda: lvq.lvq_rows_attn(q, pt0, Ly["ip"], Ly["bp"], bt0, Ly["cb"], 1, pl, pl, qe0, rope, shp,
                                    k_new=kn, v_new=vn, out=out, lse=lse, ws=ws)
    sec = _event_time(torch, run, 10)
    pairs = nq * L + nq * (nq + 1) // 2
    flops = 4.0 * D * pairs * H
    # context: dense bf16 attention over the same lengths with torch matmuls (contiguous operands)
    Kd = torch.randn((H, L + nq, D), generator=gen, device=dev).to(torch.bfloat16)
    KdT = Kd.transpose(1, 2).contiguous()
    Vd = torch.randn((H, L + nq, D), generator=gen, device=dev).to(torch.bfloat16)
    Qd = q[0].transpose(0, 1).contiguous()                  # [H][nq][D]
    mask = torch.ones((nq, L + nq), dtype=torch.bool, device=dev).tril(L)

    def dense():
        sc = torch.matmul(Qd, KdT).float() * (D ** -0.5)
        sc.masked_fill_(~mask, float("-inf"))
        return torch.matmul(torch.softmax(sc, dim=-1).to(torch.bfloat16), Vd)

    dsec = _event_time(torch, dense, 5)
    del Kd, KdT, Vd
    # matrix flops as executed: each row block of 16 queries runs every 16-key tile of the
    # coded prefix (10 d per pair on float16), the sink and recent tiles and the new-key
    # tiles its rows can see (4 d per pair on fp32)
    n_rb = nq // 16
    qe = inp["q_end"]
    coded_tiles = qe // 16
    bf_tiles = (1 if N_SINK else 0) + (L - 1) // 16 + 1 - max(qe, N_SINK) // 16
    new_tiles = sum(rb + 1 for rb in range(n_rb))
    exec_f16 = H * n_rb * coded_tiles * 256 * 10 * D
    exec_f32 = H * (n_rb * bf_tiles + new_tiles) * 256 * 4 * D
    res["prefill_chunk"] = {
        "workload": f"{nq} new tokens over a {L}-token coded prefix, 16 heads, d={D}, Tc={TC}, G={G}, one (layer, step)",
        "us": round(sec * 1e6, 1), "tokens_per_s": round(nq / sec, 1),
        "tflops": round(flops / sec / 1e12, 2), "fp32_mfma_peak": FP32_MFMA_PEAK_TFLOPS,
        "frac_fp32_mfma": round(flops / sec / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
        "executed_f16_mfma_tflops": round(exec_f16 / sec / 1e12, 2), "f16_mfma_peak": F16_MFMA_PEAK_TFLOPS,
        "frac_f16_mfma_executed": round(exec_f16 / sec / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
        "executed_f32_mfma_tflops": round(exec_f32 / sec / 1e12, 2),
        "dense_bf16_torch_us": round(dsec * 1e6, 1)}
    # ---- GQA decode: 16 query heads over 4, 2 or 1 KV heads
    c = G // TC
    ng = D // c
    n_coded = inp["q_end"] // 8
    pool = B * n_coded
    nbf = B * inp["bf16_row"]
    Hq = 16
    full = lambda v: torch.full((B,), v, dtype=torch.int32, device=dev)
    posg, qeg = full(L), full(inp["q_end"])
    pt = torch.full((B, L // 8), -1, dtype=torch.int32, device=dev)
    pt[:, :n_coded] = torch.randperm(pool, generator=gen, device=dev).to(torch.int32).view(B, n_coded)
    qg = torch.randn((B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    res["gqa_decode"] = {"workload": f"B={B}, L={L}, {Hq} query heads over Hk KV heads, d={D}, Tc={TC}, G={G}, "
                                     f"one (layer, step)"}
    # lvq_decode_attn runs the grouped kernel at 4 query heads per KV head and the
    # multi-row kernel at 8 and 16.  The per-head kernel is timed through lvq_decode_scores, which runs
    # it on the same call and also writes every score (B x 16 x L float32, 16.8 MB); its cost
    # does not depend on the grouping, so the 4-KV-head run is the per-head baseline for
    # every group size
    base_us = None
    sbuf = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    for Hk in (4, 2, 1):
        ip = torch.randint(0, 256, (pool, T // TC, Hk, 2, 8, ng), generator=gen, device=dev, dtype=torch.uint8)
        bp = torch.randn((nbf, T, Hk, 2, 8, D), generator=gen, device=dev).to(torch.bfloat16)
        cb = torch.randn((T // TC, 2, Hk, ng, TC, 256, c), generator=gen, device=dev).to(torch.bfloat16)
        dshp = lvq.make_shape(B, Hk, Hq, D, T, TC, G, N_SINK, L // 8, inp["bf16_row"], pool, nbf, L, L + 1)
        dws = torch.empty(lvq.lvq_decode_attn_workspace_bytes(dshp), dtype=torch.uint8, device=dev)
        o1 = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        l1 = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        dec = lambda: lvq.lvq_decode_attn(qg, pt, ip, bp, inp["bt"], cb, 2, posg, posg, qeg, inp["rope"], dshp,
                                          out=o1, lse=l1, ws=dws)
        rshp = lvq.make_rows_shape(B, 1, Hk, Hq, D, T, TC, G, N_SINK, L // 8, inp["bf16_row"], pool, nbf, L, L + 1)
        rws = torch.empty(lvq.lvq_rows_attn_workspace_bytes(rshp), dtype=torch.uint8, device=dev)
        o2 = torch.empty((B, 1, Hq, D), dtype=torch.float32, device=dev)
        l2 = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
        q4 = qg.view(B, 1, Hq, D)
        rows = lambda: lvq.lvq_rows_attn(q4, pt, ip, bp, inp["bt"], cb, 2, posg, posg, qeg, inp["rope"], rshp,
                                         out=o2, lse=l2, ws=rws)
        ds, rs = _event_time(torch, dec, 20), _event_time(torch, rows, 20)
        if base_us is None:
            o3 = torch.empty_like(o1)
            l3 = torch.empty_like(l1)
            per_head = lambda: lvq.lvq_decode_scores(qg, pt, ip, bp, inp["bt"], cb, 2, posg, posg, qeg, inp["rope"],
                                                     dshp, out=o3, lse=l3, ws=dws, scores=sbuf)
            base_us = _event_time(torch, per_head, 20)
            diff_ph = float((o1 - o3).abs().max())
        g = Hq // Hk
        res["gqa_decode"][f"g{g}"] = {
            "route": "grouped kernel" if g <= 4 else "multi-row kernel",
            "rows_us": round(rs * 1e6, 1), "lvq_decode_attn_us": round(ds * 1e6, 1),
            "per_head_kernel_us": round(base_us * 1e6, 1),
            "speedup_vs_per_head": round(base_us / ds, 2),
            "rows_speedup_vs_per_head": round(base_us / rs, 2),
            "max_abs_diff_decode_vs_rows": float((o1 - o2[:, 0]).abs().max())}
        if g == 4:
            res["gqa_decode"]["g4"]["max_abs_diff_grouped_vs_per_head"] = diff_ph
    del sbuf
    res["gqa_decode"]["per_head_note"] = ("per-head kernel timed through lvq_decode_scores on the 4-KV-head call "
                                          "(it also writes 16.8 MB of scores)")
    return res


def decode_loop_bench(torch, lvq, inp, n_tokens=24):
    """The whole decode loop as the product runs it, one token per replay of a captured HIP
    graph: the cache manager (begin, end, commit), the append of each (loop step, layer)'s
    new K/V, the 96 attention calls over the managed tables, and the re-encode of the pages
    that fall due, in all 24 layers, for B=8 sequences from 32768 tokens.  Page ids are
    handed out from a shuffled free list; codes and bf16 tokens are random."""
    dev = torch.device("cuda:0")
    nl = len(inp["layers"])
    c = G // TC
    nblk, ng = T // TC, D // c
    gen = torch.Generator(device=dev)
    gen.manual_seed(9001)
    max_pages = (L + 2 * n_tokens) // 8 + 4
    n_index = B * max_pages
    n_bf16 = B * 12
    cache = lvq.PagedCache(B, max_pages, N_SINK, N_RECENT, n_index, n_bf16)
    cache.index_free.copy_(cache.index_free[torch.randperm(n_index, generator=gen, device=dev)])
    cache.prefill(torch.full((B,), L, dtype=torch.int32, device=dev))
    ips = [torch.randint(0, 256, (n_index, nblk, H, 2, 8, ng), generator=gen, device=dev, dtype=torch.uint8)
           for _ in range(nl)]
    bps = [torch.randn((n_bf16, T, H, 2, 8, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(nl)]
    pools = [(bps[layer], inp["layers"][layer]["cb"], ips[layer]) for layer in range(nl)]
    kvs = [torch.randn((2, 1, B, H, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(4)]
    max_len = L + 2 * n_tokens + 8
    rope = lvq.lvq_rope_tables(max_len + 1, D, 10000.0, device=dev)
    shp = lvq.make_shape(B, H, H, D, T, TC, G, N_SINK, max_pages, cache.bf16_row, n_index, n_bf16, max_len,
                         max_len + 1)
    ws = torch.empty(lvq.lvq_decode_attn_workspace_bytes(shp), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    pos = torch.empty(B, dtype=torch.int32, device=dev)

    def token():
        cache.begin_token()
        torch.sub(cache.seq_len, 1, out=pos)
        for t in range(T):
            for layer in range(nl):
                kv = kvs[(t + layer) % 4]
                cache.append(t, kv[0], kv[1], bps[layer])
                Ly = inp["layers"][layer]
                lvq.lvq_decode_attn(Ly["q"][t], cache.page_table, ips[layer], bps[layer], cache.bf16_table,
                                    Ly["cb"], t, pos, cache.seq_len, cache.q_end, rope, shp, out=out, lse=lse,
                                    ws=ws)
        cache.end_token()
        lvq.lvq_reencode_pages_layers(pools, cache.re_src, cache.re_dst, T, TC, G)
        cache.commit()

    token()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        token()
    graph.replay()
    torch.cuda.synchronize()
    L0 = int(cache.seq_len.sum().item())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_tokens):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    if cache.errors():
        raise RuntimeError(f"cache manager error bits {cache.errors()}")
    # KV token-steps: every call attends over each sequence's current length
    steps = sum(nl * T * (L0 + B * (i + 1)) for i in range(n_tokens))
    return {"workload": f"B={B} sequences from about {L} tokens, {nl} layers x {T} loop steps per token, "
                        f"{n_tokens} tokens: manager + {nl * T} appends + {nl * T} attention calls + re-encodes, "
                        f"one HIP graph replay per token",
            "ms_per_token": round(sec * 1e3 / n_tokens, 3), "tokens_per_s": round(B * n_tokens / sec, 1),
            "kv_token_steps_per_s": steps / sec}


def encode_bench(torch, lvq, synth, inp):
    """Prefill encode of 32768 tokens x 16 heads x d=128 x 4 loop steps, K and V, for
    (Tc, G) = (4, 32) and (2, 16)."""
    import numpy as np
    dev = torch.device("cuda:0")
    N = 32768
    res = {}
    gen = torch.Generator(device=dev)
    rk = np.random.default_rng(synth.seed_for(4, synth.STREAM_K))
    sc = synth.channel_scales(rk, H, D)
    for (tc, g) in ((4, 32), (2, 16)):
        if (tc, g) == (TC, G) and inp.get("cb0") is not None:
            cb = inp["cb0"]
        else:
            cb, _ = build_books(torch, lvq, synth, tc, g, sc, sc, synth.seed_for(4, synth.STREAM_BOOKS))
        kvs = []
        for kv in (0, 1):
            gen.manual_seed(4000 + kv)
            kvs.append(synth.gen_kv_torch(gen, T, N, H, D, sc, device=dev))
        c = g // tc
        idx = [torch.empty((T // tc, N, H, D // c), dtype=torch.uint8, device=dev) for _ in range(2)]
        for _ in range(2):
            for kv in (0, 1):
                lvq.lvq_encode(kvs[kv], cb, kv, T, tc, g, idx[kv])
        torch.cuda.synchronize()
        reps = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for kv in (0, 1):
                lvq.lvq_encode(kvs[kv], cb, kv, T, tc, g, idx[kv])
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) * 1e-3 / reps        # K and V
        nvec = 2 * (T // tc) * N * H * (D // c)
        flops = nvec * 2 * g * 256
        hbm = 2 * (T * N * H * D * 2) + 2 * (T // tc) * N * H * (D // c) + cb.numel() * 2
        res[f"Tc{tc}_G{g}"] = {
            "vectors_per_s": nvec / dt, "us_per_KV_pair": dt * 1e6,
            "mfma_util": flops / dt / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "hbm_frac": hbm / dt / (HBM_PEAK_GBS * 1e9),
        }
        del kvs, idx
    return res


MIXED_B, MIXED_LO, MIXED_HI, MIXED_CONFIG = 64, 1024, 16384, 5
MIXED_LAYERS = ((8, 4, 32), (1, 1, 32))   # looped layer (two loop blocks), prelude layer (c = 32)


def mixed_bench(torch, lvq, synth, n_steps=64, warmup=3):
    """Mixed serving decode: 64 sequences with seeded lengths U[1024, 16384], H = 16, d = 128,
    4 sink + 64..71 recent bf16 tokens, shuffled pages.  One decode step = the looped
    layer's 8 loop-step calls (T = 8, Tc = 4, G = 32), the prelude layer's call (T = 1,
    Tc = 1, G = 32: c = 32, 4 groups) and the batched page re-encode of the 8 sequences
    whose recent window reaches 72 tokens at that step (round robin; both layers, K and V,
    one launch per layer shape).  Index pools hold uniform random codes (time does not depend on
    their values); the looped pool alone is larger than twice the 256 MB Infinity Cache."""
    import numpy as np
    dev = torch.device("cuda:0")
    Bm = MIXED_B
    rl = np.random.default_rng(synth.seed_for(MIXED_CONFIG, synth.STREAM_LENGTHS))
    lengths = synth.uniform_lengths(rl, Bm, MIXED_LO, MIXED_HI)
    Lmax = int(lengths.max())
    q_end = np.array([synth.prefill_q_end(int(x), N_RECENT) for x in lengths], dtype=np.int64)
    n_coded = (q_end // 8).tolist()
    max_pages = (Lmax + 7) // 8
    rp = np.random.default_rng(synth.seed_for(MIXED_CONFIG, synth.STREAM_PAGES))
    pool = int(sum(n_coded)) + Bm          # one spare page per sequence receives its re-encode
    pt_np, pool = synth.shuffled_page_table(rp, n_coded, max_pages, pool=pool)
    pt = torch.from_numpy(pt_np).to(dev)
    spare = torch.from_numpy(np.setdiff1d(np.arange(pool), pt_np[pt_np >= 0]).astype(np.int32)).to(dev)
    bf16_row = 1 + max((int(x) - int(e) + 7) // 8 for x, e in zip(lengths, q_end))
    n_bf16 = Bm * bf16_row
    bt = torch.arange(n_bf16, dtype=torch.int32, device=dev).view(Bm, bf16_row)
    pos = torch.from_numpy(lengths.astype(np.int32)).to(dev)
    seq_len = pos.clone()
    qe = torch.from_numpy(q_end.astype(np.int32)).to(dev)
    rope = lvq.lvq_rope_tables(Lmax + 1, D, 10000.0, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.seed_for(MIXED_CONFIG, synth.STREAM_K))
    layers = []
    for (T_, Tc_, G_) in MIXED_LAYERS:
        c = G_ // Tc_
        nblk, ng = T_ // Tc_, D // c
        ip = torch.randint(0, 256, (pool, nblk, H, 2, 8, ng), generator=gen, dtype=torch.uint8, device=dev)
        bp = torch.randn((n_bf16, T_, H, 2, 8, D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        cb = torch.randn((nblk, 2, H, ng, Tc_, 256, c), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        q = [synth.gen_queries_torch(gen, Bm, H, D, device=dev) for _ in range(T_)]
        shp = lvq.make_shape(Bm, H, H, D, T_, Tc_, G_, N_SINK, max_pages, bf16_row, pool, n_bf16, Lmax,
                             Lmax + 1, 0)
        ws = torch.empty(lvq.lvq_decode_attn_workspace_bytes(shp), dtype=torch.uint8, device=dev)
        layers.append(dict(T=T_, Tc=Tc_, G=G_, ng=ng, ip=ip, bp=bp, cb=cb, q=q, shp=shp, ws=ws))
    groups = {}
    for Ly in layers:
        groups.setdefault((Ly["T"], Ly["Tc"], Ly["G"]), []).append((Ly["bp"], Ly["cb"], Ly["ip"]))
    out = torch.empty((Bm, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((Bm, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(s, ev=None):
        for li, Ly in enumerate(layers):
            for t in range(Ly["T"]):
                if ev is not None:
                    ev[li][0].record()
                lvq.lvq_decode_attn(Ly["q"][t], pt, Ly["ip"], Ly["bp"], bt, Ly["cb"], t, pos, seq_len, qe,
                                    rope, Ly["shp"], out, lse, Ly["ws"])
                if ev is not None:
                    ev[li][1].record()
        b0 = (8 * s) % Bm
        src = bt[b0:b0 + 8, 1].contiguous()
        dst = spare[b0:b0 + 8].contiguous()
        for (T_, Tc_, G_), pools in groups.items():     # one launch per layer shape
            lvq.lvq_reencode_pages_layers(pools, src, dst, T_, Tc_, G_)

    for w in range(warmup):
        step(w)
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
           for _ in range(n_steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for s in range(n_steps):
        step(s, evs[s])
    s1.record()
    torch.cuda.synchronize()
    step_s = s0.elapsed_time(s1) * 1e-3 / n_steps
    last_call = [sum(evs[s][li][0].elapsed_time(evs[s][li][1]) for s in range(n_steps)) * 1e-3 / n_steps
                 for li in range(len(layers))]
    sum_l = int(lengths.sum())
    calls = sum(T_ for (T_, _, _) in MIXED_LAYERS)
    # algorithmic bytes of one step's attention calls: index rows of the call's loop
    # block, bf16 sink + recent tokens, the step's book slices, q/out/lse/page table
    coded = int(sum(max(int(e) - N_SINK, 0) for e in q_end))
    bf16_tok = int(sum(min(N_SINK, int(x)) + int(x) - int(e) for x, e in zip(lengths, q_end)))
    small = Bm * H * D * 2 + Bm * H * (D + 1) * 4 + Bm * max_pages * 4
    per_layer = []
    for Ly in layers:
        idx = coded * H * 2 * Ly["ng"]
        per_call = idx + bf16_tok * H * 2 * D * 2 + H * 2 * 256 * D * 2 + small
        per_layer.append(per_call)
    algo_step = sum(Ly["T"] * b for Ly, b in zip(layers, per_layer))
    gbs = algo_step / step_s / 1e9
    log(f"mixed B={Bm}: step {step_s * 1e3:.3f} ms, {sum_l * calls / step_s:.3e} KV token-steps/s, "
        f"{gbs:.0f} GB/s algorithmic ({gbs / HBM_PEAK_GBS * 100:.1f}% of peak)")
    del layers
    torch.cuda.empty_cache()
    # the looped layer's call with 16 query heads over 2 KV heads (GQA 8, the multi-row kernel)
    T_, Tc_, G_ = MIXED_LAYERS[0]
    Hk = 2
    c = G_ // Tc_
    nblk, ng = T_ // Tc_, D // c
    ipg = torch.randint(0, 256, (pool, nblk, Hk, 2, 8, ng), generator=gen, dtype=torch.uint8, device=dev)
    bpg = torch.randn((n_bf16, T_, Hk, 2, 8, D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    cbg = torch.randn((nblk, 2, Hk, ng, Tc_, 256, c), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    qg = synth.gen_queries_torch(gen, Bm, H, D, device=dev)
    shg = lvq.make_shape(Bm, Hk, H, D, T_, Tc_, G_, N_SINK, max_pages, bf16_row, pool, n_bf16, Lmax, Lmax + 1, 0)
    wsg = torch.empty(lvq.lvq_decode_attn_workspace_bytes(shg), dtype=torch.uint8, device=dev)

    def gqa_call():
        lvq.lvq_decode_attn(qg, pt, ipg, bpg, bt, cbg, 1, pos, seq_len, qe, rope, shg, out, lse, wsg)

    gqa_s = _event_time(torch, gqa_call, 20)
    gqa_bytes = coded * Hk * 2 * ng + bf16_tok * Hk * 2 * D * 2 + Hk * 2 * 256 * D * 2 + small
    log(f"mixed B={Bm} GQA 8 looped call: {gqa_s * 1e6:.1f} us")
    del ipg, bpg, cbg, wsg
    torch.cuda.empty_cache()
    return {"workload": f"mixed serving decode: B={Bm}, L~U[{MIXED_LO},{MIXED_HI}] (sum {sum_l}), H={H}, "
                        f"d={D}; per step 8 looped calls (T=8, Tc=4, G=32) + 1 prelude call (T=1, Tc=1, "
                        f"G=32) + re-encode of 8 sequences' oldest recent page in both layers",
            "steps": n_steps, "ms_per_step": round(step_s * 1e3, 4),
            "kv_token_steps_per_s": round(sum_l * calls / step_s),
            "algorithmic_bytes_per_step": algo_step, "achieved_gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "looped_call_us_last_t": round(last_call[0] * 1e6, 2),
            "prelude_call_us": round(last_call[1] * 1e6, 2),
            "looped_call_algorithmic_bytes": per_layer[0], "prelude_call_algorithmic_bytes": per_layer[1],
            "gqa8_looped_call_us": round(gqa_s * 1e6, 2), "gqa8_looped_call_algorithmic_bytes": gqa_bytes,
            "gqa8_note": "16 query heads over 2 KV heads, loop step 1 of the looped layer, same lengths"}


NEEDLE_L, NEEDLE_COPIES = 65536, 16


def needle_bench(torch, lvq, synth, reps=60):
    """One 65536-token sequence, H = 16, d = 128, T = 4, Tc = 2, G = 16, 4 sink + 64 recent:
    the call time of lvq_decode_attn (attention + merge) rotating over 16 copies of the
    index pool.  A call reads one loop block's rows, 33.5 MB, so a rotation reads 536 MB,
    beyond twice the 256 MB Infinity Cache.  Reported two ways: each call bracketed by
    its own events (p10/p50/p90; includes the event overhead), and back-to-back calls
    between one pair of events (the rate a decode loop sees)."""
    import numpy as np
    dev = torch.device("cuda:0")
    T_, Tc_, G_ = 4, 2, 16
    c = G_ // Tc_
    nblk, ng = T_ // Tc_, D // c
    q_end = synth.prefill_q_end(NEEDLE_L, N_RECENT)
    max_pages = NEEDLE_L // 8
    rp = np.random.default_rng(synth.seed_for(3, synth.STREAM_PAGES))
    pt_np, pool = synth.shuffled_page_table(rp, [q_end // 8], max_pages)
    pt = torch.from_numpy(pt_np).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.seed_for(3, synth.STREAM_K))
    ips = [torch.randint(0, 256, (pool, nblk, H, 2, 8, ng), generator=gen, dtype=torch.uint8, device=dev)
           for _ in range(NEEDLE_COPIES)]
    bf16_row = 1 + (NEEDLE_L - q_end + 7) // 8
    bp = torch.randn((bf16_row, T_, H, 2, 8, D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    bt = torch.arange(bf16_row, dtype=torch.int32, device=dev).view(1, bf16_row)
    cb = torch.randn((nblk, 2, H, ng, Tc_, 256, c), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    q = synth.gen_queries_torch(gen, 1, H, D, device=dev)
    one = torch.full((1,), NEEDLE_L, dtype=torch.int32, device=dev)
    qe = torch.full((1,), q_end, dtype=torch.int32, device=dev)
    rope = lvq.lvq_rope_tables(NEEDLE_L + 1, D, 10000.0, device=dev)
    shp = lvq.make_shape(1, H, H, D, T_, Tc_, G_, N_SINK, max_pages, bf16_row, pool, bf16_row, NEEDLE_L,
                         NEEDLE_L + 1, 0)
    ws = torch.empty(lvq.lvq_decode_attn_workspace_bytes(shp), dtype=torch.uint8, device=dev)
    out = torch.empty((1, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, H), dtype=torch.float32, device=dev)

    def call(i):
        lvq.lvq_decode_attn(q, pt, ips[i % NEEDLE_COPIES], bp, bt, cb, 1, one, one, qe, rope, shp, out, lse, ws)

    for i in range(5):
        call(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    med = ts[len(ts) // 2]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    b2b = e0.elapsed_time(e1) * 1e-3 / reps
    # The same call (same launch configuration) over an 8-token cache: its time is the
    # per-call overhead (two launches, the work-list scan, staging, the merge).
    eight = torch.full((1,), 8, dtype=torch.int32, device=dev)
    zero = torch.zeros((1,), dtype=torch.int32, device=dev)
    for _ in range(3):
        lvq.lvq_decode_attn(q, pt, ips[0], bp, bt, cb, 1, eight, eight, zero, rope, shp, out, lse, ws)
    evs0 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs0:
        a.record()
        lvq.lvq_decode_attn(q, pt, ips[0], bp, bt, cb, 1, eight, eight, zero, rope, shp, out, lse, ws)
        b.record()
    torch.cuda.synchronize()
    fixed = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs0)[reps // 2]
    e0.record()
    for _ in range(reps):
        lvq.lvq_decode_attn(q, pt, ips[0], bp, bt, cb, 1, eight, eight, zero, rope, shp, out, lse, ws)
    e1.record()
    torch.cuda.synchronize()
    fixed_b2b = e0.elapsed_time(e1) * 1e-3 / reps
    algo = (q_end - N_SINK) * H * 2 * ng + (N_SINK + NEEDLE_L - q_end) * H * 2 * D * 2 + H * 2 * 256 * D * 2 \
        + H * D * 2 + H * (D + 1) * 4 + max_pages * 4
    gbs = algo / med / 1e9
    log(f"needle 64K: call {med * 1e6:.1f} us median (own events), {b2b * 1e6:.1f} us back to back, "
        f"{gbs:.0f} GB/s algorithmic")
    del ips
    torch.cuda.empty_cache()
    return {"workload": f"one sequence of {NEEDLE_L} tokens, H={H}, d={D}, T=4, Tc=2, G=16 (0.5 bit), "
                        f"{N_SINK} sink + {N_RECENT} recent, shuffled pages, {NEEDLE_COPIES} pool copies "
                        f"rotated (536 MB read per rotation)",
            "call_us_p10": round(ts[len(ts) // 10] * 1e6, 2), "call_us_p50": round(med * 1e6, 2),
            "call_us_p90": round(ts[(9 * len(ts)) // 10] * 1e6, 2),
            "algorithmic_bytes_per_call": int(algo), "achieved_gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "kv_token_steps_per_s": round(NEEDLE_L / med),
            "call_us_back_to_back": round(b2b * 1e6, 2),
            "achieved_gbs_back_to_back": round(algo / b2b / 1e9, 1),
            "kv_token_steps_per_s_back_to_back": round(NEEDLE_L / b2b),
            "fixed_call_us": round(fixed * 1e6, 2),
            "fixed_call_us_back_to_back": round(fixed_b2b * 1e6, 2),
            "fixed_call_note": "the same call over an 8-token cache (same launch configuration): "
                               "launches, work-list scan, slice staging and merge; own events "
                               "and back to back"}


def hbm_probe(torch):
    """Attainable HBM rates on this GPU: row sums of a 2 GiB float32 matrix with 4096-wide
    rows (a streaming read; the fastest of torch's reductions here) and a 2 GiB copy (read +
    write), five timed repetitions each after a warm-up."""
    n = (2 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    out = {}
    for name, fn, nbytes in (("read_gbs", lambda: x.view(-1, 4096).sum(1), 4 * n),
                             ("copy_gbs", lambda: y.copy_(x), 8 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del x, y
    return out


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.pmc_instructions:
        pmc_instructions(args.pmc_instructions)
        return
    if args.kernel_stats_summary:
        kernel_stats_summary(args.kernel_stats_summary)
        return
    if args.cpu_worker:
        print(json.dumps(cpu_worker(args.cpu_worker, args.cpu_cores, args.cpu_seconds)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import sub_bit_loop_amd as lvq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.encode_only:
        print(json.dumps({"encode": encode_bench(torch, lvq, synth, {})}), flush=True)
        return
    inp = build_inputs(args, torch, lvq, synth)
    wall, per_call = run_decode(args, torch, lvq, inp)
    ncall = T * args.layers
    step_s = wall / args.steps
    token_steps = ncall * B * L
    value = token_steps / step_s
    call_avg = sum(per_call) / len(per_call)
    algo = algorithmic_bytes_per_call(inp["q_end"])
    achieved_gbs = algo / call_avg / 1e9
    log(f"step {step_s * 1e3:.3f} ms, call {call_avg * 1e6:.1f} us, {achieved_gbs:.0f} GB/s algorithmic")
    traffic = recorded_traffic()
    valu_bound = recorded_instructions()
    probe = None if args.headline_only else hbm_probe(torch)
    pc = sorted(per_call)
    pct = {f"p{q}": round(pc[min(len(pc) - 1, int(q / 100 * len(pc)))] * 1e6, 2) for q in (10, 50, 90)}
    # The metric names the HBM fraction, so the roofline reports the call against the HBM
    # peak (algorithmic bytes / event-timed call time / 8 TB/s).  The float32 vector work
    # of the per-token rotation after dequantisation is what actually binds the call; its
    # figures (VALU floor, issue bound, ALU fraction) sit beside it as flat fields.
    flops = algorithmic_flops_per_call()
    achieved_tflops = flops / call_avg / 1e12
    kern_us = recorded_kernel_us()
    floor_us = valu_floor_us()
    roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_call": algo,
            "traffic_over_algorithmic": None if traffic is None else round(traffic / algo, 3),
            "kernel": "lvq_decode_attn call: attn_kernel<128,8> + merge_kernel, one (layer, loop step)",
            "avg_call_us": round(call_avg * 1e6, 2), "call_us_percentiles": pct,
            "frac_event_timed": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "kernel_us_rocprof": kern_us,
            "frac_kernel_only": None if kern_us is None else round(algo / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "attainable_read_gbs": None if probe is None else probe["read_gbs"],
            "attainable_copy_gbs": None if probe is None else probe["copy_gbs"],
            "frac_of_attainable_read": None if probe is None else round(achieved_gbs / probe["read_gbs"], 4),
            "valu_floor_us": round(floor_us, 2),
            "frac_of_valu_floor": round(floor_us / (call_avg * 1e6), 4),
            "valu_issue_bound_us": valu_bound,
            "frac_of_valu_issue_bound": None if valu_bound is None else round(valu_bound / (call_avg * 1e6), 4),
            "alu_achieved_tflops": round(achieved_tflops, 2), "alu_peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
            "alu_frac": round(achieved_tflops / FP32_VECTOR_PEAK_TFLOPS, 4),
            "alu_peak_unpacked_tflops": FP32_VECTOR_UNPACKED_TFLOPS,
            "alu_frac_of_unpacked_peak": round(achieved_tflops / FP32_VECTOR_UNPACKED_TFLOPS, 4),
            "algorithmic_flops_per_call": flops}
    res = {
        "metric": METRIC, "value": value, "unit": "KV token-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"ouro-1.4b-shaped decode attention: {args.layers} layers x {T} loop steps "
                               f"per token, B={B}, L={L}, H={H}, d={D}, Tc={TC}, G={G} (0.25 bit), "
                               f"{N_SINK} sink + {N_RECENT} recent bf16, shuffled pages",
                   "global_batch": B, "seq_len": L, "parallelism": "single-gpu"},
        "roofline": roof,
    }
    n_books = 2 * H * (D // (G // TC)) * (T // TC)
    res["codebook_build"] = {
        "workload": f"one layer, K and V: {n_books} books of 256 codewords, {N_BOOK_SAMPLES} samples "
                    f"each, k-means++ + {N_LLOYD} Lloyd iterations (Tc={TC}, G={G})",
        "ms": round(inp["build_s"] * 1e3, 2), "books_per_s": round(n_books / inp["build_s"], 1)}
    if not args.headline_only:
        try:
            res.update(rows_bench(torch, lvq, inp))
        except Exception as e:  # report, never hide the headline
            res["prefill_chunk"] = {"error": repr(e)}
        try:
            res["cache_manager"] = manager_bench(torch, lvq, inp)
        except Exception as e:  # report, never hide the headline
            res["cache_manager"] = {"error": repr(e)}
        try:
            res["decode_loop"] = decode_loop_bench(torch, lvq, inp)
        except Exception as e:  # report, never hide the headline
            res["decode_loop"] = {"error": repr(e)}
        try:
            res["needle_64k"] = needle_bench(torch, lvq, synth)
        except Exception as e:  # report, never hide the headline
            res["needle_64k"] = {"error": repr(e)}
        try:
            res["mixed_serving"] = mixed_bench(torch, lvq, synth)
        except Exception as e:  # report, never hide the headline
            res["mixed_serving"] = {"error": repr(e)}
    if not args.no_encode and not args.headline_only:
        try:
            res["encode"] = encode_bench(torch, lvq, synth, inp)
        except Exception as e:  # report, never hide the headline
            res["encode"] = {"error": repr(e)}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(args, torch, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
