"""Throughput benchmark of the GDN hot path on one MI355X.

One step is one pass of the whole path over synthetic inputs of the layer's
shapes (Hk=16, Hv=32, Dk=Dv=128, K=4):
  * decode:  gdn_decode over 256 rows (one token each) against a 512-slot
             f32 state pool and a bf16 conv-history pool; the slot subset is
             re-drawn for every step so repeated steps do not hit the same
             rows in the last-level cache;
  * prefill: gdn_prepare + gdn_prefill_varlen over one 4096-token sequence,
             bf16 activations and q/k/v, f32 state from zero, chunk 64.
value = (256 + 4096) tokens / step time.  Per-kernel times come from HIP
events recorded on the stream the kernels run on.  A bounded sample of the
same work is also run through the f64 CPU oracle on the host cores
(cpu_baseline).  After the timed region the output epilogue and the
speculative multi-token decode (256 requests x 4 tokens) are timed on their
own and reported beside the step, and so are the two other prefill
workloads (16 varlen sequences with bf16 state carried in; 32768 tokens with
Hv=48 and f16 state, one call and 8 chained calls), the KDA variant's chunked
prefill (4096 tokens) and token-by-token decode (256 sequences).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 matrix peak, vendor figure
METRIC = "GDN prefill tokens/s + decode tokens/s; % of HBM/MFMA roofline, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--epilogue-only", action="store_true",
                    help="only run the output epilogue kernels (fused gated decode, standalone gated RMS norm)")
    ap.add_argument("--spec-only", action="store_true",
                    help="only run the speculative multi-token decode (gdn_decode_spec) workload")
    ap.add_argument("--kda-only", action="store_true",
                    help="only run the KDA workloads (chunked prefill, token-by-token decode)")
    ap.add_argument("--mamba2-only", action="store_true",
                    help="time only the Mamba2 prefill and decode workloads and print their record")
    ap.add_argument("--prefill-configs-only", action="store_true",
                    help="only time the varlen (16 sequences) and long (32768 tokens, Hv=48) prefill workloads")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the device-copy and cold-cache decode runs after the timed region (for profiling)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: min(16, cpu count))")
    ap.add_argument("--rmw-probe", action="store_true",
                    help="only time the decode's state stream alone (in-place update of 256 random 2 MB slots "
                         "of a 512-slot f32 pool, trivial arithmetic) under several launch shapes, beside gdn_decode")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference for HBM byte counters)")
    return ap.parse_args()


def decode_bytes(B, Hk, Hv, Dk, Dv, K, state_bytes=4, act_bytes=2):
    """Algorithmic HBM bytes of one gdn_decode call: every operand once."""
    Cc = 2 * Hk * Dk + Hv * Dv
    return (2 * B * Hv * Dv * Dk * state_bytes       # state read + write
            + 2 * B * Cc * (K - 1) * act_bytes       # conv history read + write
            + B * Cc * act_bytes                     # raw projections
            + 2 * B * Hv * act_bytes                 # a, b
            + B * Hv * Dv * act_bytes                # out
            + B * 4                                  # slot indices
            + Cc * K * act_bytes + 2 * Hv * 4)       # conv weight, A_log, dt_bias


def prefill_bytes(T, Hk, Hv, Dk, Dv, qkv_bytes=2, state_bytes=4, has_init=False):
    """Algorithmic HBM bytes of one gdn_prefill_varlen call (one sequence)."""
    return (T * (2 * Hk * Dk + Hv * Dv) * qkv_bytes  # q, k, v
            + 2 * T * Hv * 4                         # g, beta
            + T * Hv * Dv * qkv_bytes                # out
            + (2 if has_init else 1) * Hv * Dv * Dk * state_bytes)


def prefill_chunked_flops(T, Hk, Hv, Dk, Dv, c=64):
    """Algorithmic flops of the chunked (WY/UT) prefill on full chunks of c
    tokens, per token:
      per key head    K K^T and Q K^T over the chunk            4 c Dk
      per value head  (I + A)^-1 by substitution                2 c^2 / 3
                      W = T diag(beta gamma) K                  2 c Dk
                      U = T diag(beta) V,  P Delta              4 c Dv
                      W S^T, Q S^T, Delta^T K (state products)  6 Dk Dv
    Every product counts once; the f16 hi/lo split the kernels use to keep
    f32 accuracy issues two to three matrix instructions per product, which
    is not counted."""
    per_tok = Hk * 4 * c * Dk + Hv * (2 * c * c / 3 + 2 * c * Dk + 4 * c * Dv + 6 * Dk * Dv)
    return per_tok * T


def prepare_bytes(T, Hk, Hv, Dk, Dv, K, act_bytes=2, qkv_bytes=2):
    Cc = 2 * Hk * Dk + Hv * Dv
    return T * Cc * act_bytes + T * Cc * qkv_bytes + 2 * T * Hv * act_bytes + 2 * T * Hv * 4 + Cc * K * act_bytes


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_prepare_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_record(name, kernel, sources):
    """A kernel's record from a committed rocprofv3 counter summary, only if
    the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != source_sha(*sources):
        return None
    return rec


def stats_us(ms_list):
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"mean_us": float(a.mean()), "median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90))}


def measured_traffic(kernel, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != source_sha(*sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(dec, pre, threads):
    """The f64 oracle on a bounded sample of the same workload: all 256 decode
    rows and the first 2048 tokens of the prefill sequence (all heads)."""
    import oracle
    d_cfg, d_inp = dec
    p_cfg, p_inp = pre
    d = d_cfg.dims
    nrow = 256
    rows = np.arange(nrow)
    slots = d_inp["slots"][rows]
    conv = d_inp["conv_pool"][slots]
    ssm = d_inp["ssm_pool"][slots]
    t0 = time.perf_counter()
    oracle.decode(d, d_inp["x"][rows], d_inp["w"], d_inp["a"][rows], d_inp["b"][rows], d_inp["A_log"],
                  d_inp["dt_bias"], conv, ssm, np.arange(nrow, dtype=np.int32), d_cfg.scale, "f32", "bf16",
                  nthreads=threads)
    t_dec = (time.perf_counter() - t0) / nrow
    ntok = 2048
    cu = np.array([0, ntok], np.int32)
    t0 = time.perf_counter()
    prep = oracle.prepare(d, cu, p_inp["x"][:ntok], p_inp["w"], p_inp["a"][:ntok], p_inp["b"][:ntok],
                          p_inp["A_log"], p_inp["dt_bias"], p_inp["conv_pool"], p_inp["slots"], p_inp["has_init"],
                          True, "bf16", nthreads=threads)
    oracle.prefill(d, cu, prep["q"], prep["k"], prep["v"], prep["g"], prep["beta"], p_inp["ssm_pool"],
                   p_inp["slots"], p_inp["has_init"], p_cfg.scale, False, "f32", "bf16", nthreads=threads)
    t_pre = (time.perf_counter() - t0) / ntok
    step = d_cfg.batch * t_dec + p_cfg.T * t_pre
    # one thread on a smaller sample of the same work
    n1, nt1 = 16, 128
    t0 = time.perf_counter()
    oracle.decode(d, d_inp["x"][:n1], d_inp["w"], d_inp["a"][:n1], d_inp["b"][:n1], d_inp["A_log"],
                  d_inp["dt_bias"], conv[:n1], ssm[:n1], np.arange(n1, dtype=np.int32), d_cfg.scale, "f32", "bf16",
                  nthreads=1)
    t1_dec = (time.perf_counter() - t0) / n1
    cu1 = np.array([0, nt1], np.int32)
    t0 = time.perf_counter()
    prep1 = oracle.prepare(d, cu1, p_inp["x"][:nt1], p_inp["w"], p_inp["a"][:nt1], p_inp["b"][:nt1],
                           p_inp["A_log"], p_inp["dt_bias"], p_inp["conv_pool"], p_inp["slots"], p_inp["has_init"],
                           True, "bf16", nthreads=1)
    oracle.prefill(d, cu1, prep1["q"], prep1["k"], prep1["v"], prep1["g"], prep1["beta"], p_inp["ssm_pool"],
                   p_inp["slots"], p_inp["has_init"], p_cfg.scale, False, "f32", "bf16", nthreads=1)
    t1_pre = (time.perf_counter() - t0) / nt1
    step1 = d_cfg.batch * t1_dec + p_cfg.T * t1_pre
    return {"value": (d_cfg.batch + p_cfg.T) / step, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nrow} decode rows + first {ntok} prefill tokens (all heads), f64 oracle; "
                      f"scaled to the step's 256 decode + 4096 prefill tokens",
            "decode_tokens_per_s": 1.0 / t_dec, "prefill_tokens_per_s": 1.0 / t_pre,
            "host_cpus": os.cpu_count(),
            "single_thread": {"value": (d_cfg.batch + p_cfg.T) / step1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1} decode rows + first {nt1} prefill tokens, scaled likewise"}}


def extras(torch, gdn, gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets, slot_sets_h, dout, scale, stream, nsets):
    """After the timed region: a device-to-device copy of the decode call's
    size (read + write bytes / time), and decode with the 256 MB Infinity
    Cache flushed by a 512 MiB scratch write before each call."""
    dev = dx.device
    B = dx.shape[0]
    half = decode_bytes(B, gd.Hk, gd.Hv, gd.Dk, gd.Dv, gd.K) // 2 // 4
    csrc = torch.empty(half, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for i in range(6):
        if i:
            cev[i - 1][0].record(stream)
        cdst.copy_(csrc)
        if i:
            cev[i - 1][1].record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * half * 4 / (float(np.median([e[0].elapsed_time(e[1]) for e in cev])) * 1e-3) / 1e9
    del csrc, cdst
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for i in range(5):
        flush.fill_(float(i))
        cold_ev[i][0].record(stream)
        gdn.gdn_decode(gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets[i % nsets], dout, scale,
                       slot_idx_host=slot_sets_h[i % nsets], stream=stream)
        cold_ev[i][1].record(stream)
    torch.cuda.synchronize()
    cold_l = [e[0].elapsed_time(e[1]) for e in cold_ev]
    del flush
    return copy_gbs, cold_l


def prepare_copy_ref(torch, prep_b, dec_call, prep_call, stream, reps=10):
    """The prepare against a device copy of the same bytes (half read, half
    written) in the same cache state: each timed call follows a decode call,
    as in the step, whose state stream leaves the Infinity Cache cold and
    dirty.  HIP events on the kernels' stream, medians."""
    n = prep_b // 2 // 4
    csrc = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    cdst = torch.empty_like(csrc)
    res = {"copy": [], "prepare": []}
    for i in range(reps + 2):
        for name, fn in (("copy", lambda: cdst.copy_(csrc)), ("prepare", prep_call)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            dec_call(i)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                res[name].append(e0.elapsed_time(e1))
    del csrc, cdst
    cu, pu = (float(np.median(res[k])) * 1e3 for k in ("copy", "prepare"))
    return {"note": "each call after a decode call; copy of the prepare's bytes, half read and half written",
            "copy_us": cu, "copy_GBps": prep_b / (cu * 1e-6) / 1e9, "prepare_us": pu, "frac_of_copy": cu / pu}


def gated_decode_bytes(B, Hk, Hv, Dk, Dv, K, act_bytes=2):
    """gdn_decode bytes plus the gate (B*Hv*Dv) and the norm weight (Dv)."""
    return decode_bytes(B, Hk, Hv, Dk, Dv, K) + B * Hv * Dv * act_bytes + Dv * act_bytes


def gated_norm_bytes(T, Hv, Dv, io_bytes=2):
    """gdn_gated_rmsnorm bytes: x, z read, out written, the weight once."""
    return 3 * T * Hv * Dv * io_bytes + Dv * io_bytes


def epilogue(torch, gdn, gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets, slot_sets_h, scale, stream, T,
             reps=10):
    """The output epilogue (gated RMS norm) at the step's shapes: fused into
    decode over the 256 rows, and standalone over the 4096-token prefill
    output.  HIP events on the kernels' stream, median of ``reps`` calls."""
    dev = dx.device
    B = dx.shape[0]
    HvDv = gd.Hv * gd.Dv
    g = torch.Generator(device=dev)
    g.manual_seed(91)
    zd = torch.randn(B, HvDv, device=dev, generator=g).to(torch.bfloat16)
    wn = (torch.rand(gd.Dv, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    outd = torch.empty(B, gd.Hv, gd.Dv, device=dev, dtype=torch.bfloat16)
    xp = torch.randn(T, gd.Hv, gd.Dv, device=dev, generator=g).to(torch.bfloat16)
    zp = torch.randn(T, HvDv, device=dev, generator=g).to(torch.bfloat16)
    outp = torch.empty_like(xp)
    # plain and fused decode alternate on the same slot sets, so their times compare like for like
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(reps)]
    n = len(slot_sets)
    for i in range(reps + 2):
        e = ev[i - 2] if i >= 2 else None
        if e:
            e[0].record(stream)
        gdn.gdn_decode(gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets[i % n], outd, scale,
                       slot_idx_host=slot_sets_h[i % n], stream=stream)
        if e:
            e[1].record(stream)
            e[2].record(stream)
        gdn.gdn_decode_gated(gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets[(i + 1) % n], zd, wn, outd, scale,
                             1e-6, slot_idx_host=slot_sets_h[(i + 1) % n], stream=stream)
        if e:
            e[3].record(stream)
            e[4].record(stream)
        gdn.gdn_gated_rmsnorm(xp, zp, wn, outp, 1e-6, stream=stream)
        if e:
            e[5].record(stream)
    torch.cuda.synchronize()
    dp = [e[0].elapsed_time(e[1]) for e in ev]
    dg = [e[2].elapsed_time(e[3]) for e in ev]
    nm = [e[4].elapsed_time(e[5]) for e in ev]
    # the norm again, back to back with itself: its operands stay in the
    # Infinity Cache and no other kernel's dirty lines are written back
    nev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + 2)]
    for e in nev:
        e[0].record(stream)
        gdn.gdn_gated_rmsnorm(xp, zp, wn, outp, 1e-6, stream=stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    nm_loop = [e[0].elapsed_time(e[1]) for e in nev[2:]]
    db_ = gated_decode_bytes(B, gd.Hk, gd.Hv, gd.Dk, gd.Dv, gd.K)
    nb = gated_norm_bytes(T, gd.Hv, gd.Dv)
    gbs = lambda b, l: b / (float(np.median(l)) * 1e-3) / 1e9
    return {
        "decode_gated": {**stats_us(dg), "bytes_per_launch": db_,
                         "plain_decode_same_loop": stats_us(dp),
                         "roofline": {"bound": "hbm", "achieved": gbs(db_, dg), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": gbs(db_, dg) / HBM_PEAK_GBS}},
        "gated_rmsnorm_T4096": {**stats_us(nm), "bytes_per_launch": nb,
                                "note": "each call after the two decode calls; back_to_back: the norm alone in a loop",
                                "back_to_back": {**stats_us(nm_loop), "GBps": gbs(nb, nm_loop)},
                                "roofline": {"bound": "hbm", "achieved": gbs(nb, nm), "peak": HBM_PEAK_GBS,
                                             "unit": "GB/s", "frac": gbs(nb, nm) / HBM_PEAK_GBS}},
    }


def spec_bytes(N, L, Hk, Hv, Dk, Dv, K, W, state_bytes=4, act_bytes=2):
    """Algorithmic HBM bytes of one gdn_decode_spec call with N requests of L
    tokens: the initial state read once and L snapshots written per request,
    the widened conv row read and written, every other operand once."""
    Cc = 2 * Hk * Dk + Hv * Dv
    T = N * L
    return ((1 + L) * N * Hv * Dv * Dk * state_bytes   # state: one read, L snapshot writes
            + 2 * N * Cc * W * act_bytes               # conv rows read + write
            + T * Cc * act_bytes                       # raw projections
            + 2 * T * Hv * act_bytes                   # a, b
            + T * Hv * Dv * act_bytes                  # out
            + N * (L + 1 + 1) * 4                      # slot table, num_accepted, offsets
            + Cc * K * act_bytes + 2 * Hv * 4)         # conv weight, A_log, dt_bias


def speculative(torch, gdn, reps=20):
    """The speculative decode workload (gdn_inputs.spec_batch): HIP events on
    the kernel's stream, median of ``reps`` calls after 3 untimed ones.  Each
    call draws its own num_accepted (seeded), so successive calls start from
    different columns."""
    from gdn_inputs import spec_batch, spec_inputs
    sb = spec_batch()
    d = sb["dims"]
    N, C = sb["num_reqs"], sb["cols"]
    inp = spec_inputs(d, N, C, sb["num_slots"], sb["act_dtype"], sb["state_dtype"], sb["seed"])
    dev = torch.device("cuda:0")
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt=f32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    x, w, a, b = t(inp["x"], bf), t(inp["w"], bf), t(inp["a"], bf), t(inp["b"], bf)
    A, dt_ = t(inp["A_log"]), t(inp["dt_bias"])
    conv, ssm = t(inp["conv_pool"], bf), t(inp["ssm_pool"])
    del inp["ssm_pool"]
    cu_h, sidx_h = inp["cu"], inp["state_idx"]
    cu, sidx = torch.from_numpy(cu_h).to(dev), torch.from_numpy(sidx_h).to(dev)
    rng = np.random.default_rng(sb["seed"] + 1)
    nat_h = [rng.integers(1, C + 1, size=N).astype(np.int32) for _ in range(reps + 3)]
    nat = [torch.from_numpy(n).to(dev) for n in nat_h]
    out = torch.empty(N * C, d.Hv, d.Dv, device=dev, dtype=bf)
    gd = gdn.Dims(d.Hk, d.Hv, d.Dk, d.Dv, d.K)
    scale = 1.0 / math.sqrt(d.Dk)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps + 3):
        e = ev[i - 3] if i >= 3 else None
        if e:
            e[0].record(stream)
        gdn.gdn_decode_spec(gd, cu, x, a, b, w, A, dt_, conv, ssm, sidx, nat[i], out, scale, cu_seqlens_host=cu_h,
                            state_idx_host=sidx_h, num_accepted_host=nat_h[i], stream=stream)
        if e:
            e[1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    W = conv.shape[2]
    nb = spec_bytes(N, C, d.Hk, d.Hv, d.Dk, d.Dv, d.K, W)
    gbs = nb / (float(np.median(ms)) * 1e-3) / 1e9
    # reference for a write-dominated stream: torch's fill of a buffer the
    # size of one call's snapshot writes (HBM writes run well below 8 TB/s)
    del conv, ssm
    fill = torch.empty(N * C * d.Hv * d.Dv * d.Dk, dtype=f32, device=dev)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for i in range(6):
        if i:
            fev[i - 1][0].record(stream)
        fill.fill_(float(i))
        if i:
            fev[i - 1][1].record(stream)
    torch.cuda.synchronize()
    fill_gbs = fill.numel() * 4 / (float(np.median([e[0].elapsed_time(e[1]) for e in fev])) * 1e-3) / 1e9
    del fill
    return {"workload": f"{sb['name']}: {N} requests x {C} tokens, {sb['num_slots']}-slot f32 state pool, "
                        f"conv rows of {W} taps, bf16 activations",
            "tokens_per_s": N * C / (float(np.median(ms)) * 1e-3), **stats_us(ms), "bytes_per_launch": nb,
            "fill_GBps": fill_gbs, "frac_of_fill": gbs / fill_gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "kernel": "spec_decode_kernel",
                         "traffic": measured_traffic("spec_decode_kernel", ["gdn_spec.hip", "gdn_device.h"])}}


def kda_prefill_flops(T, Hk, Hv, Dk, Dv, c=64):
    """Algorithmic flops of the chunked KDA prefill on full chunks of c tokens,
    per token and value head (the decays are per value head and channel, so
    the chunk's K K^T and Q K^T products are per value head too):
      A and P with the per-pair decays           4 c Dk
      (I + A)^-1 by substitution                 2 c^2 / 3
      W = T diag(beta) (K e^G)                   2 c Dk
      U = T diag(beta) V,  P Delta               4 c Dv
      W S^T, (Q e^G) S^T, Delta^T (K e^(G_C-G))  6 Dk Dv
    Each product once; the f16 hi/lo split is not counted."""
    return T * Hv * (4 * c * Dk + 2 * c * c / 3 + 2 * c * Dk + 4 * c * Dv + 6 * Dk * Dv)


def kda_prefill_bytes(T, Hk, Hv, Dk, Dv, qkv_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one KDA prefill call from a zero state: q, k,
    v, the gate input g [T, Hv, Dk] f32 and beta read, out and the final state
    written."""
    return (T * (2 * Hk * Dk + Hv * Dv) * qkv_bytes + T * Hv * Dk * 4 + T * Hv * 4
            + T * Hv * Dv * qkv_bytes + Hv * Dv * Dk * state_bytes)


def kda_decode_bytes(B, Hk, Hv, Dk, Dv, qkv_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one KDA recurrent call over B one-token
    sequences: the state read and written, q, k, v, g, beta and out."""
    return (2 * B * Hv * Dv * Dk * state_bytes + B * (2 * Hk * Dk + Hv * Dv) * qkv_bytes + B * Hv * Dk * 4
            + B * Hv * 4 + B * Hv * Dv * qkv_bytes + B * 4 * 2)


def kda(torch, gdn, reps=20):
    """The KDA workloads (gdn_inputs.kda_prefill_workload, kda_decode_workload):
    HIP events on the kernels' stream, median of ``reps`` calls after 3
    untimed ones."""
    from gdn_inputs import kda_decode_workload, kda_inputs, kda_prefill_workload
    dev = torch.device("cuda:0")
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt=f32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    stream = torch.cuda.current_stream()
    res = {}
    for wl in (kda_prefill_workload(), kda_decode_workload()):
        d = wl["dims"]
        inp = kda_inputs(d, wl["seqlens"], wl["num_slots"], wl["qkv_dtype"], wl["state_dtype"], wl["seed"],
                         has_init=wl["has_init"])
        gd = gdn.Dims(d.Hk, d.Hv, d.Dk, d.Dv, d.K)
        q, k, v = t(inp["q"], bf), t(inp["k"], bf), t(inp["v"], bf)
        g, beta, A, dtb = t(inp["g"]), t(inp["beta"]), t(inp["A_log"]), t(inp["dt_bias"])
        pool = t(inp["ssm_pool"])
        cu_h, sl_h = inp["cu"], inp["slots"]
        cu, sl, hi = t(cu_h, torch.int32), t(sl_h, torch.int32), t(inp["has_init"], torch.uint8)
        T = int(cu_h[-1])
        out = torch.empty(T, d.Hv, d.Dv, device=dev, dtype=bf)
        scale = 1.0 / math.sqrt(d.Dk)
        chunked = wl["name"].startswith("kda_prefill")
        ws = None
        if chunked:
            ws = torch.empty(max(gdn.gdn_kda_prefill_workspace_size(gd, len(sl_h), T, gdn.GDN_BF16), 1),
                             dtype=torch.uint8, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps + 3):
            e = ev[i - 3] if i >= 3 else None
            if e:
                e[0].record(stream)
            if chunked:
                gdn.gdn_kda_prefill_varlen(gd, cu, q, k, v, g, beta, pool, out, scale, A_log=A, dt_bias=dtb,
                                           slot_idx=sl, has_initial_state=hi, use_qk_l2norm=True, workspace=ws,
                                           cu_seqlens_host=cu_h, slot_idx_host=sl_h, stream=stream)
            else:
                gdn.gdn_kda_recurrent(gd, cu, q, k, v, g, beta, pool, out, scale, A_log=A, dt_bias=dtb, slot_idx=sl,
                                      has_initial_state=hi, use_qk_l2norm=True, cu_seqlens_host=cu_h,
                                      slot_idx_host=sl_h, stream=stream)
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        sec = float(np.median(ms)) * 1e-3
        if chunked:
            fl = kda_prefill_flops(T, d.Hk, d.Hv, d.Dk, d.Dv)
            nb = kda_prefill_bytes(T, d.Hk, d.Hv, d.Dk, d.Dv)
            rl = {"bound": "mfma", "achieved": fl / sec / 1e12, "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": fl / sec / 1e12 / F16_MFMA_PEAK_TFLOPS, "flops_per_launch": fl, "bytes_per_launch": nb,
                  "hbm_frac": nb / sec / 1e9 / HBM_PEAK_GBS,
                  "kernels": "kda_prep_kernel + chunk_scan_kernel (KDA; one sequence: no chunk_table_kernel)"}
        else:
            nb = kda_decode_bytes(T, d.Hk, d.Hv, d.Dk, d.Dv)
            rl = {"bound": "hbm", "achieved": nb / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": nb / sec / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": nb, "kernel": "kda_recurrent_kernel"}
        res[wl["name"]] = {"tokens_per_s": T / sec, **stats_us(ms), "roofline": rl}
        del q, k, v, g, beta, pool, out, ws
    return res


def varlen_prefill_bytes(T, N, Hk, Hv, Dk, Dv, qkv_bytes=2, state_bytes=4, has_init=True):
    """Algorithmic HBM bytes of one gdn_prefill_varlen call over N sequences
    of T tokens in all: q, k, v, g, beta read and out written once, and each
    sequence's state read (when it continues its slot) and written once."""
    return (T * (2 * Hk * Dk + Hv * Dv) * qkv_bytes + 2 * T * Hv * 4 + T * Hv * Dv * qkv_bytes
            + N * (2 if has_init else 1) * Hv * Dv * Dk * state_bytes)


def varlen_prepare_bytes(T, N, Hk, Hv, Dk, Dv, K, act_bytes=2, qkv_bytes=2, has_init=True):
    """prepare_bytes plus each sequence's conv-history row read (when it
    continues its slot) and written."""
    Cc = 2 * Hk * Dk + Hv * Dv
    return (prepare_bytes(T, Hk, Hv, Dk, Dv, K, act_bytes, qkv_bytes)
            + N * (2 if has_init else 1) * Cc * (K - 1) * act_bytes)


def prefill_configs(torch, gdn, reps=10):
    """The two other prefill workloads, timed after the timed region, each as
    gdn_prepare + gdn_prefill_varlen per call (HIP events on the kernels'
    stream, median of ``reps`` calls after 2 untimed ones):
      * varlen: 16 sequences, lengths ~U[128, 8192] (73,145 tokens), bf16
        state pool and conv histories carried in (has_initial_state = 1): the
        general path, whose chunk table chunk_table_kernel builds;
      * long: one 32,768-token sequence, Hv = 48, f16 state from zero, as one
        call and as 8 chained 4096-token calls (conv history and state carried).
    The prefill is reported against the f16 MFMA peak (algorithmic flops of
    the chunked form) with its HBM fraction beside it, the prepare against the
    HBM peak."""
    from gdn_inputs import make_inputs, prefill_long, prefill_varlen
    dev = torch.device("cuda:0")
    bf, f32 = torch.bfloat16, torch.float32
    sdt = {"f32": f32, "bf16": bf, "f16": torch.float16}
    sbytes = {"f32": 4, "bf16": 2, "f16": 2}
    t = lambda a, dt=f32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    stream = torch.cuda.current_stream()
    res = {}
    for cfg in (prefill_varlen(), prefill_long()):
        d = cfg.dims
        gd = gdn.Dims(d.Hk, d.Hv, d.Dk, d.Dv, d.K)
        inp = make_inputs(cfg)
        x, w, a, b = t(inp["x"], bf), t(inp["w"], bf), t(inp["a"], bf), t(inp["b"], bf)
        A, dtb = t(inp["A_log"]), t(inp["dt_bias"])
        conv = t(inp["conv_pool"], bf)
        pool = t(inp["ssm_pool"], sdt[cfg.state_dtype])
        del inp["x"]
        T, N = cfg.T, cfg.N
        q = torch.empty(T, d.Hk, d.Dk, device=dev, dtype=bf)
        k = torch.empty_like(q)
        v = torch.empty(T, d.Hv, d.Dv, device=dev, dtype=bf)
        g = torch.empty(T, d.Hv, device=dev)
        beta = torch.empty_like(g)
        out = torch.empty(T, d.Hv, d.Dv, device=dev, dtype=bf)
        ws = torch.empty(max(gdn.gdn_prefill_workspace_size(gd, N, T, 64), 1), dtype=torch.uint8, device=dev)
        has_init = bool(inp["has_init"][0])
        # (first token, token count, cu host, has_init host) per call of one pass
        modes = {"one_call": [(0, T, inp["cu"], inp["has_init"])]}
        if cfg.name.startswith("long"):
            L = 4096
            modes["eight_calls"] = [(L * i, L, np.array([0, L], np.int32), np.array([1 if i else 0], np.uint8))
                                    for i in range(T // L)]
        rec = {"tokens": T, "sequences": N, "state_dtype": cfg.state_dtype, "Hv": d.Hv,
               "has_initial_state": has_init}
        for mode, calls in modes.items():
            dcalls = [(t0, n, cu_h, t(cu_h, torch.int32), hi_h, t(hi_h, torch.uint8)) for t0, n, cu_h, hi_h in calls]
            sl_h = inp["slots"]
            sl = t(sl_h, torch.int32)
            evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in dcalls] for _ in range(reps)]
            for it in range(reps + 2):
                for j, (t0, n, cu_h, cu_d, hi_h, hi_d) in enumerate(dcalls):
                    e = evs[it - 2][j] if it >= 2 else None
                    sl_ = slice(t0, t0 + n)
                    if e:
                        e[0].record(stream)
                    gdn.gdn_prepare(gd, cu_d, x[sl_], a[sl_], b[sl_], w, A, dtb, conv, q[sl_], k[sl_], v[sl_], g[sl_],
                                    beta[sl_], slot_idx=sl, has_initial_state=hi_d, cu_seqlens_host=cu_h,
                                    slot_idx_host=sl_h, stream=stream)
                    if e:
                        e[1].record(stream)
                    gdn.gdn_prefill_varlen(gd, cu_d, q[sl_], k[sl_], v[sl_], g[sl_], beta[sl_], pool, out[sl_],
                                           cfg.scale, slot_idx=sl, has_initial_state=hi_d, workspace=ws,
                                           cu_seqlens_host=cu_h, slot_idx_host=sl_h, stream=stream)
                    if e:
                        e[2].record(stream)
            torch.cuda.synchronize()
            prep_ms = [sum(e[0].elapsed_time(e[1]) for e in calls_e) for calls_e in evs]
            pre_ms = [sum(e[1].elapsed_time(e[2]) for e in calls_e) for calls_e in evs]
            sp, sq = float(np.median(prep_ms)) * 1e-3, float(np.median(pre_ms)) * 1e-3
            ncalls = len(dcalls)
            fl = prefill_chunked_flops(T, d.Hk, d.Hv, d.Dk, d.Dv)
            # state traffic per call: read when the call continues a slot, always written
            nb = varlen_prefill_bytes(T, N, d.Hk, d.Hv, d.Dk, d.Dv, 2, sbytes[cfg.state_dtype], has_init)
            nb += (ncalls - 1) * N * d.Hv * d.Dv * d.Dk * sbytes[cfg.state_dtype] * 2
            pb = varlen_prepare_bytes(T, N, d.Hk, d.Hv, d.Dk, d.Dv, d.K, has_init=has_init)
            pb += (ncalls - 1) * (2 * N * d.Cc * (d.K - 1) * 2 + d.Cc * d.K * 2)
            rec[mode] = {
                "calls": ncalls, "tokens_per_s": T / (sp + sq),
                "prepare": {**stats_us(prep_ms),
                            "roofline": {"bound": "hbm", "achieved": pb / sp / 1e9, "peak": HBM_PEAK_GBS,
                                         "unit": "GB/s", "frac": pb / sp / 1e9 / HBM_PEAK_GBS,
                                         "bytes_per_launch": pb}},
                "prefill": {**stats_us(pre_ms),
                            "kernels": "chunk_prep_kernel + chunk_scan_kernel" +
                                       (" + chunk_table_kernel" if N > 1 else " (one sequence: no chunk table)"),
                            "roofline": {"bound": "mfma", "achieved": fl / sq / 1e12, "peak": F16_MFMA_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": fl / sq / 1e12 / F16_MFMA_PEAK_TFLOPS,
                                         "flops_per_launch": fl, "bytes_per_launch": nb,
                                         "hbm_frac": nb / sq / 1e9 / HBM_PEAK_GBS}},
            }
        res[cfg.name] = rec
        del x, w, a, b, conv, pool, q, k, v, g, beta, out, ws
        torch.cuda.empty_cache()
    return res


def mamba2_prefill_flops(T, H, P, N, c=64):
    """Algorithmic flops of the chunked Mamba2 / SSD prefill on full chunks of
    c tokens, per token and head: C B^T (2 c N), the masked product with X
    (2 c P), the inter-chunk term C S^T (2 P N) and the chunk's state
    contribution X^T (w B) (2 P N).  Each product once, as dense c x c
    blocks; the f16 hi/lo split is not counted."""
    return T * H * (2 * c * N + 2 * c * P + 4 * P * N)


def mamba2_prefill_bytes(T, H, P, G, N, act_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one Mamba2 prefill call from a zero state: x, z
    and dt read, B and C read once per group, out and the final state written."""
    return T * (2 * H * P + H + 2 * G * N) * act_bytes + T * H * P * act_bytes + H * P * N * state_bytes


def mamba2_decode_bytes(Bn, H, P, G, N, act_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one Mamba2 single-step call over Bn rows: the
    state read and written, x, z, dt, B, C and out, the slot index."""
    return 2 * Bn * H * P * N * state_bytes + Bn * (3 * H * P + H + 2 * G * N) * act_bytes + Bn * 4


def mamba2(torch, gdn, reps=20):
    """The Mamba2 workloads (gdn_inputs.mamba2_prefill_workload,
    mamba2_decode_workload): HIP events on the kernels' stream, median of
    ``reps`` calls after 3 untimed ones."""
    from gdn_inputs import mamba2_decode_workload, mamba2_inputs, mamba2_prefill_workload
    dev = torch.device("cuda:0")
    bf, f32 = torch.bfloat16, torch.float32
    t = lambda a, dt=f32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    stream = torch.cuda.current_stream()
    res = {}
    for wl in (mamba2_prefill_workload(), mamba2_decode_workload()):
        H, P, G, N = wl["H"], wl["P"], wl["G"], wl["N"]
        inp = mamba2_inputs(H, P, G, N, wl["seqlens"], wl["num_slots"], wl["act"], wl["state"], wl["seed"],
                            has_init=wl["has_init"])
        x, z, dt, Bm, Cm = (t(inp[k], bf) for k in ("x", "z", "dt", "B", "C"))
        A, D, dtb = t(inp["A"]), t(inp["D"]), t(inp["dt_bias"])
        pool = t(inp["ssm_pool"])
        cu_h, sl_h = inp["cu"], inp["slots"]
        cu, sl, hi = t(cu_h, torch.int32), t(sl_h, torch.int32), t(inp["has_init"], torch.uint8)
        T = int(cu_h[-1])
        out = torch.empty(T, H, P, device=dev, dtype=bf)
        chunked = wl["name"].startswith("mamba2_prefill")
        ws = None
        if chunked:
            ws = torch.empty(max(gdn.gdn_mamba2_workspace_size(H, P, N, len(sl_h), T, G), 1), dtype=torch.uint8,
                             device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps + 3):
            e = ev[i - 3] if i >= 3 else None
            if e:
                e[0].record(stream)
            if chunked:
                gdn.gdn_mamba2_chunk_scan(cu, x, dt, A, Bm, Cm, pool, out, D=D, z=z, dt_bias=dtb, slot_idx=sl,
                                          has_initial_state=hi, workspace=ws, cu_seqlens_host=cu_h,
                                          slot_idx_host=sl_h, stream=stream)
            else:
                gdn.gdn_mamba2_state_update(x, dt, A, Bm, Cm, pool, sl, out, D=D, z=z, dt_bias=dtb,
                                            slot_idx_host=sl_h, stream=stream)
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        sec = float(np.median(ms)) * 1e-3
        if chunked:
            fl = mamba2_prefill_flops(T, H, P, N)
            nb = mamba2_prefill_bytes(T, H, P, G, N)
            # workspace traffic of one sequence: per (chunk pair, head) the
            # pair's f32 contribution written and read, the first chunk's f16
            # contribution written and read, the pair's f16 entering state
            # written and read twice, and each chunk's decay vector written
            # and read
            npairs = ((T + 127) // 128) * H
            ws_b = npairs * (2 * P * N * 4 + 2 * P * N * 2 + 3 * P * N * 2 + 2 * 2 * 1280)
            rl = {"bound": "hbm", "achieved": nb / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": nb / sec / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": nb,
                  "workspace_bytes_per_launch": ws_b, "flops_per_launch": fl,
                  "mfma_frac": fl / sec / 1e12 / F16_MFMA_PEAK_TFLOPS,
                  "kernels": "ssd_state_kernel + ssd_pass_kernel + ssd_out_kernel (one sequence: no ssd_table_kernel)"}
        else:
            nb = mamba2_decode_bytes(T, H, P, G, N)
            rl = {"bound": "hbm", "achieved": nb / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": nb / sec / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": nb, "kernel": "mamba2_update_kernel"}
        res[wl["name"]] = {"tokens_per_s": T / sec, **stats_us(ms), "roofline": rl}
        del x, z, dt, Bm, Cm, pool, out, ws
    return res


def rmw_probe(torch, gdn, reps=20):
    """The ceiling of the decode's memory access pattern: libgdn_probe.so's
    in-place read-modify-write of 256 random 2 MB slots out of a 512-slot f32
    pool (1 GiB; the slot subset re-drawn per call as in the decode bench),
    with a trivial update and none of the decode's other work, timed with HIP
    events (median of ``reps`` calls after 3), beside gdn_decode on the same
    slot sets.  Rates count the state bytes read and written (1 GiB per call)
    for the probe and the decode's algorithmic bytes for the decode."""
    import ctypes
    from gdn_inputs import decode_batch, decode_slot_sets, make_inputs
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_prepare_amd", "libgdn_probe.so"))
    lib.gdn_probe_slot_rmw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p]
    lib.gdn_probe_slot_rmw.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    cfg = decode_batch("f32")
    d = cfg.dims
    slot_floats = d.Hv * d.Dv * d.Dk
    pool = torch.zeros(cfg.num_slots * slot_floats, dtype=torch.float32, device=dev)
    n = reps + 3
    sets_h = decode_slot_sets(cfg, n, seed=4242)
    sets = torch.from_numpy(sets_h).to(dev)
    contiguous = torch.arange(cfg.batch, dtype=torch.int32, device=dev)
    state_bytes = 2 * cfg.batch * slot_floats * 4

    def timed(call):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            call(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in ev[3:]])) * 1e-3

    res = {"pool_slots": cfg.num_slots, "rows": cfg.batch, "slot_bytes": slot_floats * 4,
           "state_bytes_per_call": state_bytes}
    shapes = [("decode_shape_128KB_per_wg_nt_stores", 16, 0, False), ("128KB_per_wg_plain_stores", 16, 1, False),
              ("whole_2MB_slot_per_wg_1024_threads", 1, 2, False),
              ("decode_shape_contiguous_slots", 16, 0, True)]
    for name, regions, mode, contig in shapes:
        def call(i, regions=regions, mode=mode, contig=contig):
            sl = contiguous if contig else sets[i]
            rc = lib.gdn_probe_slot_rmw(ctypes.c_void_p(pool.data_ptr()), ctypes.c_void_p(sl.data_ptr()), cfg.batch,
                                        slot_floats, regions, mode, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
        sec = timed(call)
        res[name] = {"median_us": sec * 1e6, "GBps": state_bytes / sec / 1e9,
                     "frac_of_hbm_peak": state_bytes / sec / 1e9 / HBM_PEAK_GBS}
    del pool
    inp = make_inputs(cfg)
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    bf = torch.bfloat16
    gd = gdn.Dims(d.Hk, d.Hv, d.Dk, d.Dv, d.K)
    x, w, a, b = t(inp["x"], bf), t(inp["w"], bf), t(inp["a"], bf), t(inp["b"], bf)
    A, dtb, conv, ssm = t(inp["A_log"]), t(inp["dt_bias"]), t(inp["conv_pool"], bf), t(inp["ssm_pool"])
    out = torch.empty(cfg.batch, d.Hv, d.Dv, device=dev, dtype=bf)
    sec = timed(lambda i: gdn.gdn_decode(gd, x, a, b, w, A, dtb, conv, ssm, sets[i], out, cfg.scale,
                                         slot_idx_host=sets_h[i], stream=stream))
    nb = decode_bytes(cfg.batch, d.Hk, d.Hv, d.Dk, d.Dv, d.K)
    res["gdn_decode"] = {"median_us": sec * 1e6, "GBps": nb / sec / 1e9, "frac_of_hbm_peak": nb / sec / 1e9 / HBM_PEAK_GBS,
                         "frac_of_probe": (nb / sec) / (state_bytes / (res["decode_shape_128KB_per_wg_nt_stores"]["median_us"] * 1e-6))}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer shards "
              "without communication by batch or by key-head group, and one long sequence needs one exchange of "
              "per-segment state transitions)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read_per_launch": src.numel() * 4,
                          "copy_probe_bytes_written_per_launch": dst.numel() * 4}), flush=True)
        return

    import gated_delta_rule_prepare_amd as gdn
    from gdn_inputs import decode_batch, decode_slot_sets, make_inputs, prefill_single

    gdn.load_library()
    if args.spec_only:
        print(json.dumps({"decode_spec": speculative(torch, gdn, reps=args.steps)}), flush=True)
        return
    if args.kda_only:
        print(json.dumps({"kda": kda(torch, gdn, reps=args.steps)}), flush=True)
        return
    if args.mamba2_only:
        print(json.dumps({"mamba2": mamba2(torch, gdn, reps=args.steps)}), flush=True)
        return
    if args.rmw_probe:
        print(json.dumps({"rmw_probe": rmw_probe(torch, gdn, reps=args.steps)}), flush=True)
        return
    if args.prefill_configs_only:
        print(json.dumps({"prefill_configs": prefill_configs(torch, gdn, reps=args.steps)}), flush=True)
        return
    dev = torch.device("cuda:0")
    bf, f32 = torch.bfloat16, torch.float32

    # ---- decode inputs
    dcfg = decode_batch("f32")
    dinp = make_inputs(dcfg)
    d = dcfg.dims
    gd = gdn.Dims(d.Hk, d.Hv, d.Dk, d.Dv, d.K)
    B = dcfg.batch
    t = lambda a, dt=f32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    dx, dw, da, db = t(dinp["x"], bf), t(dinp["w"], bf), t(dinp["a"], bf), t(dinp["b"], bf)
    dA, ddt = t(dinp["A_log"]), t(dinp["dt_bias"])
    dconv = t(dinp["conv_pool"], bf)
    dssm = t(dinp["ssm_pool"])
    nsets = args.warmup + args.steps
    slot_sets_h = decode_slot_sets(dcfg, nsets, seed=4242)
    slot_sets = torch.from_numpy(slot_sets_h).to(dev)
    dout = torch.empty(B, d.Hv, d.Dv, device=dev, dtype=bf)

    # ---- prefill inputs
    pcfg = prefill_single("bf16")
    pinp = make_inputs(pcfg)
    T = pcfg.T
    px, pw, pa, pb = t(pinp["x"], bf), t(pinp["w"], bf), t(pinp["a"], bf), t(pinp["b"], bf)
    pA, pdt = t(pinp["A_log"]), t(pinp["dt_bias"])
    pconv = t(pinp["conv_pool"], bf)
    pssm = t(pinp["ssm_pool"])
    cu_h = pinp["cu"]
    cu = torch.from_numpy(cu_h).to(dev)
    sl_h = pinp["slots"]
    sl = torch.from_numpy(sl_h).to(dev)
    hi = torch.from_numpy(pinp["has_init"]).to(dev)
    q = torch.empty(T, d.Hk, d.Dk, device=dev, dtype=bf)
    k = torch.empty_like(q)
    v = torch.empty(T, d.Hv, d.Dv, device=dev, dtype=bf)
    g = torch.empty(T, d.Hv, device=dev)
    beta = torch.empty_like(g)
    pout = torch.empty(T, d.Hv, d.Dv, device=dev, dtype=bf)
    ws_bytes = gdn.gdn_prefill_workspace_size(gd, 1, T, 64)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    stream = torch.cuda.current_stream()
    nev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nev)]

    # Each event recorded between two kernels adds about 3.4 us to the step
    # (a marker the next dispatch waits for).  The timed steps record only
    # the decode's two events, which its roofline needs; the prepare and
    # prefill times come from a second pass over the same steps that also
    # records the events between them (rec_all).
    def step(i, rec=None, rec_all=False):
        if rec is not None:
            rec[0].record(stream)
        gdn.gdn_decode(gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets[i], dout, dcfg.scale,
                       slot_idx_host=slot_sets_h[i], stream=stream)
        if rec is not None:
            rec[1].record(stream)
        gdn.gdn_prepare(gd, cu, px, pa, pb, pw, pA, pdt, pconv, q, k, v, g, beta, slot_idx=sl, has_initial_state=hi,
                        cu_seqlens_host=cu_h, slot_idx_host=sl_h, stream=stream)
        if rec is not None and rec_all:
            rec[2].record(stream)
        gdn.gdn_prefill_varlen(gd, cu, q, k, v, g, beta, pssm, pout, pcfg.scale, slot_idx=sl, has_initial_state=hi,
                               workspace=ws, cu_seqlens_host=cu_h, slot_idx_host=sl_h, stream=stream)
        if rec is not None and rec_all:
            rec[3].record(stream)

    if args.epilogue_only:
        ep = epilogue(torch, gdn, gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets, slot_sets_h, dcfg.scale, stream,
                      T, reps=args.steps)
        print(json.dumps({"epilogue": ep}), flush=True)
        return
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dec_l = [e[0].elapsed_time(e[1]) for e in ev]
    # the same steps again, untimed, with every kernel boundary recorded
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nev)]
    for i in range(args.steps):
        step(args.warmup + i, ev2[i], rec_all=True)
    torch.cuda.synchronize()
    prep_l = [e[1].elapsed_time(e[2]) for e in ev2]
    pre_l = [e[2].elapsed_time(e[3]) for e in ev2]
    dec_ms, prep_ms, pre_ms = (float(np.mean(x)) for x in (dec_l, prep_l, pre_l))

    copy_gbs, cold_l, epi, spec, kda_r, m2, pcfgs, prep_ref = None, None, None, None, None, None, None, None
    if not args.no_extras:
        pcfgs = prefill_configs(torch, gdn)
        spec = speculative(torch, gdn)
        kda_r = kda(torch, gdn)
        m2 = mamba2(torch, gdn)
        epi = epilogue(torch, gdn, gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets, slot_sets_h, dcfg.scale,
                       stream, T)
        copy_gbs, cold_l = extras(torch, gdn, gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets, slot_sets_h, dout,
                                  dcfg.scale, stream, nsets)
        prep_ref = prepare_copy_ref(
            torch, prepare_bytes(T, d.Hk, d.Hv, d.Dk, d.Dv, d.K),
            lambda i: gdn.gdn_decode(gd, dx, da, db, dw, dA, ddt, dconv, dssm, slot_sets[i % nsets], dout, dcfg.scale,
                                     slot_idx_host=slot_sets_h[i % nsets], stream=stream),
            lambda: gdn.gdn_prepare(gd, cu, px, pa, pb, pw, pA, pdt, pconv, q, k, v, g, beta, slot_idx=sl,
                                    has_initial_state=hi, cu_seqlens_host=cu_h, slot_idx_host=sl_h, stream=stream),
            stream)


    dec_b = decode_bytes(B, d.Hk, d.Hv, d.Dk, d.Dv, d.K)
    dec_gbs = dec_b / (dec_ms * 1e-3) / 1e9
    pre_b = prefill_bytes(T, d.Hk, d.Hv, d.Dk, d.Dv)
    pre_flops = prefill_chunked_flops(T, d.Hk, d.Hv, d.Dk, d.Dv)
    prep_b = prepare_bytes(T, d.Hk, d.Hv, d.Dk, d.Dv, d.K)
    mfma = {k2: profile_record("mfma.json", k2, ["gdn_prefill.hip", "gdn_device.h"])
            for k2 in ("chunk_prep_kernel", "chunk_scan_kernel")}
    kernels = {
        "decode": {"avg_ms": dec_ms, "tokens_per_s": B / (dec_ms * 1e-3), **stats_us(dec_l),
                   "frac_of_copy": dec_gbs / copy_gbs if copy_gbs else None,
                   "cold_cache": {**stats_us(cold_l), "GBps": dec_b / (float(np.median(cold_l)) * 1e-3) / 1e9,
                                  "note": "512 MiB scratch write before each call"} if cold_l else None,
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_gbs / HBM_PEAK_GBS, "bytes_per_launch": dec_b,
                                "traffic": measured_traffic("decode_kernel", ["gdn_decode.hip", "gdn_device.h"])}},
        "note": "the timed steps record events around the decode only (each event between kernels adds about "
                "3.4 us); prepare and prefill come from a second pass over the same steps with an event at every "
                "kernel boundary",
        "prepare": {"avg_ms": prep_ms, "tokens_per_s": T / (prep_ms * 1e-3), **stats_us(prep_l),
                    "same_state_copy": prep_ref,
                    "roofline": {"bound": "hbm", "achieved": prep_b / (prep_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": prep_b / (prep_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "bytes_per_launch": prep_b}},
        "prefill": {"avg_ms": pre_ms, "tokens_per_s": T / (pre_ms * 1e-3), **stats_us(pre_l),
                    "mfma_counters": mfma,
                    "kernels": "chunk_prep_kernel + chunk_scan_kernel (one sequence: no chunk_table_kernel)",
                    "roofline": {"bound": "mfma", "achieved": pre_flops / (pre_ms * 1e-3) / 1e12,
                                 "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": pre_flops / (pre_ms * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS,
                                 "flops_per_launch": pre_flops, "bytes_per_launch": pre_b,
                                 "hbm_frac": pre_b / (pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}},
    }
    # decode_kernel is the longest single kernel of the step and the only
    # kernel of its entry point, so its event time is the kernel's own time
    rl = dict(kernels["decode"]["roofline"])
    rl["kernel"] = "decode_kernel"
    rl = {k2: rl[k2] for k2 in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel")}

    line = {
        "metric": METRIC, "value": (B + T) / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 vector arithmetic and state; matrix products on the f16 MFMA with f32 operands split into f16 "
                 "hi + lo (about 22 bits), hi only for Q S^T and P Delta into bf16 outputs; bf16 io",
        "data": "synthetic",
        "config": {"workload": "GDN step: decode 256 rows (512-slot f32 state pool) + prefill of one 4096-token "
                               "sequence; Hk=16 Hv=32 Dk=Dv=128 K=4; bf16 activations",
                   "decode_rows": B, "prefill_tokens": T, "chunk": 64, "state_dtype": "f32",
                   "activation_dtype": "bf16"},
        "decode_tokens_per_s": kernels["decode"]["tokens_per_s"],
        "prefill_tokens_per_s": T / ((prep_ms + pre_ms) * 1e-3),
        "roofline": rl,
        "copy_GBps": copy_gbs,
        "epilogue": epi,
        "prefill_configs": pcfgs,
        "decode_spec": spec,
        "kda": kda_r,
        "mamba2": m2,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        line["cpu_baseline"] = cpu_baseline((dcfg, dinp), (pcfg, pinp), threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
